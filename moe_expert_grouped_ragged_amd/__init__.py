"""Python binding of libgg, the MI355X (gfx950) grouped GEMM for frozen MoE experts.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind ``include/gg.h``.  PyTorch supplies device memory and the
current stream.  The functions carry the C names:

  gg_pack_weights(w1, w2)                        -> packed weight buffer
  gg_forward_fc1_swiglu(x, offsets, packed, ...) -> (h1, a)
  gg_forward_fc2(a, offsets, packed, ...)        -> y
  gg_dgrad(dy, h1, offsets, packed, ...)         -> dx  (dH1 left in the workspace)
  gg_forward_fc1_glu(x, offsets, packed, ..., activation, probs) -> (h1, a)
  gg_dgrad_glu(dy, h1, offsets, packed, ..., activation, probs)  -> (dx, dprobs)
  gg_dgrad_recompute(dy, x, offsets, packed, ...)                 -> (dx, dprobs)
        (no saved H1: FC1 is recomputed from x inside the call)
  gg_pack_frag(packed, E, H, F)                  -> opt-in fragment buffer
  gg_forward_fc2_frag(a, offsets, packed, frag, ...) -> y
        (the *_glu, recompute and fc2_frag calls take `frag`: fragment-ordered
        weight copies that speed up the GEMMs for H % 256 == 0 and
        F % 128 == 0, at 12*E*H*F more bytes)

The *_glu calls add the QuickGeGLU activation and the weighting of the
activation by each row's router probability (fp32 [M]), with dp of that
weight from the input gradient.  The probability can instead scale the FC1
input rows:

  gg_scale_rows(x, probs)                        -> x' = bf16(p_r * x_r)
  gg_scale_rows_backward(dxs, x, probs)          -> (dx, dprobs)
        (ScaleRows is the autograd form, to compose with FrozenExpertMLP)

Frozen, bias-free bf16 expert weights only: the Megatron-LM pull request
"perf(moe): add frozen grouped GEMM for adapter training" (section "Why
existing behavior remains safe") accepts only grouped, frozen, bias-free BF16
expert weights and fails during preparation otherwise; ``gg_pack_weights``
raises ValueError for other dtypes and for weights that require grad.

There is no fallback: if libgg.so is missing, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple, Union

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgg.so")

GG_OK = 0
GG_ERR_INVALID_ARGUMENT = 1
GG_ERR_MISALIGNED = 2
GG_ERR_UNSUPPORTED_DEVICE = 3
GG_ERR_WORKSPACE_TOO_SMALL = 4
GG_ERR_ALIASING = 5
GG_ERR_HIP = 6

GG_ACT_SWIGLU = 0
GG_ACT_QGEGLU = 1
ACTIVATIONS = {"swiglu": GG_ACT_SWIGLU, "qgeglu": GG_ACT_QGEGLU}

EXPORTED = ("gg_status_string", "gg_packed_bytes", "gg_dgrad_workspace_bytes", "gg_pack_weights",
            "gg_forward_fc1_swiglu", "gg_forward_fc2", "gg_dgrad", "gg_round_bf16",
            "gg_dgrad_glu_workspace_bytes", "gg_forward_fc1_glu", "gg_dgrad_glu", "gg_dgrad_recompute",
            "gg_frag_bytes", "gg_pack_frag", "gg_forward_fc2_frag", "gg_dgrad_noalloc",
            "gg_scale_rows", "gg_scale_rows_backward")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run "
                          "`python -m moe_expert_grouped_ragged_amd._build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    p, i64, sz, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    lib.gg_status_string.argtypes = [i32]
    lib.gg_status_string.restype = ctypes.c_char_p
    lib.gg_packed_bytes.argtypes = [i64, i64, i64]
    lib.gg_packed_bytes.restype = sz
    lib.gg_frag_bytes.argtypes = [i64, i64, i64]
    lib.gg_frag_bytes.restype = sz
    lib.gg_dgrad_workspace_bytes.argtypes = [i64, i64]
    lib.gg_dgrad_workspace_bytes.restype = sz
    lib.gg_pack_weights.argtypes = [i64, i64, i64, ctypes.POINTER(p), ctypes.POINTER(p), p, sz, p]
    lib.gg_pack_frag.argtypes = [i64, i64, i64, p, sz, p, sz, p]
    lib.gg_forward_fc1_swiglu.argtypes = [p, p, i64, p, i64, i64, i64, p, p, p]
    lib.gg_forward_fc2.argtypes = [p, p, i64, p, i64, i64, i64, p, p]
    lib.gg_forward_fc2_frag.argtypes = [p, p, i64, p, p, i64, i64, i64, p, p]
    lib.gg_dgrad.argtypes = [p, p, p, i64, p, i64, i64, i64, p, sz, p, p]
    lib.gg_round_bf16.argtypes = [p, p, i64, p]
    lib.gg_dgrad_noalloc.argtypes = [p, p, p, i64, p, i64, i64, i64, p, p]
    lib.gg_dgrad_glu_workspace_bytes.argtypes = [i64, i64, i32]
    lib.gg_dgrad_glu_workspace_bytes.restype = sz
    lib.gg_forward_fc1_glu.argtypes = [p, p, i64, p, p, i64, i64, i64, i32, p, p, p, p]
    lib.gg_dgrad_glu.argtypes = [p, p, p, i64, p, p, i64, i64, i64, i32, p, p, sz, p, p, p]
    lib.gg_dgrad_recompute.argtypes = [p, p, p, i64, p, p, i64, i64, i64, i32, p, p, sz, p, p, p]
    lib.gg_scale_rows.argtypes = [p, p, i64, i64, p, p]
    lib.gg_scale_rows_backward.argtypes = [p, p, p, i64, i64, p, p, p]
    for name in ("gg_pack_weights", "gg_pack_frag", "gg_forward_fc1_swiglu", "gg_forward_fc2",
                 "gg_forward_fc2_frag", "gg_dgrad", "gg_round_bf16", "gg_forward_fc1_glu", "gg_dgrad_glu",
                 "gg_dgrad_recompute", "gg_dgrad_noalloc", "gg_scale_rows", "gg_scale_rows_backward"):
        getattr(lib, name).restype = i32
    return lib


lib = _load()


class GGError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib.gg_status_string(status).decode()}")


def _check(status: int, what: str) -> None:
    if status != GG_OK:
        raise GGError(status, what)


def _stream_ptr(stream: Optional[torch.cuda.Stream], device: torch.device) -> int:
    """The given stream, or the current stream of the tensors' device; the
    library runs on the stream's device, so a stream of another device is
    refused."""
    if stream is None:
        return int(torch.cuda.current_stream(device).cuda_stream)
    if stream.device != device:
        raise ValueError(f"stream is on {stream.device}, the tensors on {device}")
    return int(stream.cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _bf16_cuda(t: torch.Tensor, name: str, shape=None, device=None) -> torch.Tensor:
    """A contiguous bf16 device tensor (of the given shape, on the given device)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    return t


def _offsets(offsets: torch.Tensor, E: int, device) -> torch.Tensor:
    """The split offsets as given (no copy: a strided tensor is refused)."""
    if (not isinstance(offsets, torch.Tensor) or offsets.dtype != torch.int64 or not offsets.is_cuda
            or offsets.shape != (E + 1,) or offsets.device != device or not offsets.is_contiguous()):
        raise ValueError(f"offsets must be a contiguous int64 tensor of shape [E+1] on {device}")
    return offsets


def _packed(packed: torch.Tensor, E: int, H: int, F: int, device) -> torch.Tensor:
    """The packed weights: a contiguous bf16 buffer of at least packed_bytes(E, H, F)."""
    _bf16_cuda(packed, "packed", device=device)
    need = packed_bytes(E, H, F)
    if need == 0 or packed.numel() * 2 < need:
        raise ValueError(f"packed holds {packed.numel() * 2} bytes; E={E}, H={H}, F={F} needs {need}")
    return packed


def _frag(frag: Optional[torch.Tensor], E: int, H: int, F: int, device) -> Optional[torch.Tensor]:
    """An optional fragment buffer of at least frag_bytes(E, H, F)."""
    if frag is None:
        return None
    _bf16_cuda(frag, "frag", device=device)
    need = frag_bytes(E, H, F)
    if need == 0:
        raise ValueError(f"H={H}, F={F} has no fragment-ordered copies (needs H % 256 == 0 and F % 128 == 0)")
    if frag.numel() * 2 < need:
        raise ValueError(f"frag holds {frag.numel() * 2} bytes; E={E}, H={H}, F={F} needs {need}")
    return frag


def _out(t: Optional[torch.Tensor], shape, name: str, device) -> torch.Tensor:
    """A caller-given output (checked) or a new one."""
    if t is None:
        return torch.empty(*shape, dtype=torch.bfloat16, device=device)
    return _bf16_cuda(t, name, shape=shape, device=device)


def _workspace(ws: Optional[torch.Tensor], nbytes: int, device) -> torch.Tensor:
    """A caller-given workspace (contiguous, on the device, any dtype, >= nbytes) or a new one."""
    if ws is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous() or ws.device != device:
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, {nbytes} needed")
    return ws


def packed_bytes(E: int, H: int, F: int) -> int:
    return int(lib.gg_packed_bytes(E, H, F))


def frag_bytes(E: int, H: int, F: int) -> int:
    """Bytes of the opt-in fragment-ordered copies (0 when the shape has none)."""
    return int(lib.gg_frag_bytes(E, H, F))


def has_frag(H: int, F: int) -> bool:
    return frag_bytes(1, H, F) > 0


def dgrad_workspace_bytes(M: int, F: int) -> int:
    return int(lib.gg_dgrad_workspace_bytes(M, F))


def gg_pack_weights(w1: Union[torch.Tensor, Sequence[torch.Tensor]],
                    w2: Union[torch.Tensor, Sequence[torch.Tensor]],
                    packed: Optional[torch.Tensor] = None,
                    stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Pack frozen expert weights (w1[e]: [2F, H], gate rows then up rows;
    w2[e]: [H, F]) into one expert-major bf16 buffer of exactly the weights'
    size.  Returns the packed buffer (1-D, packed_bytes(E, H, F) / 2
    elements).  Per-expert views into it: ``expert_views(packed, E, H, F)``."""
    w1s = list(w1.unbind(0)) if isinstance(w1, torch.Tensor) else list(w1)
    w2s = list(w2.unbind(0)) if isinstance(w2, torch.Tensor) else list(w2)
    if len(w1s) != len(w2s) or not w1s:
        raise ValueError("w1 and w2 need the same, nonzero number of experts")
    for t in w1s + w2s:
        if t.dtype != torch.bfloat16:
            raise ValueError(f"expert weights must be bfloat16 (got {t.dtype}); "
                             "fp8/fp4/fp32 expert weights are not supported")
        if t.requires_grad:
            raise ValueError("expert base weights must be frozen (requires_grad=False)")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("expert weights must be contiguous device tensors")
        if t.device != w1s[0].device:
            raise ValueError("expert weights must all be on one device")
    E = len(w1s)
    twoF, H = w1s[0].shape
    F = twoF // 2
    if twoF != 2 * F or any(t.shape != (2 * F, H) for t in w1s) or any(t.shape != (H, F) for t in w2s):
        raise ValueError("w1[e] must be [2F, H] and w2[e] must be [H, F] for every expert")
    nbytes = packed_bytes(E, H, F)
    if packed is None:
        packed = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=w1s[0].device)
    _packed(packed, E, H, F, w1s[0].device)
    arr1 = (ctypes.c_void_p * E)(*[t.data_ptr() for t in w1s])
    arr2 = (ctypes.c_void_p * E)(*[t.data_ptr() for t in w2s])
    _check(lib.gg_pack_weights(E, H, F, arr1, arr2, packed.data_ptr(), packed.numel() * 2,
                               _stream_ptr(stream, w1s[0].device)), "gg_pack_weights")
    return packed


def gg_pack_frag(packed: torch.Tensor, E: int, H: int, F: int, frag: Optional[torch.Tensor] = None,
                 stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Opt-in fragment-ordered copies of the packed weights (H % 256 == 0 and
    F % 128 == 0 only): returns the fragment buffer (frag_bytes(E, H, F) / 2
    bf16 elements) to pass as ``frag`` to the extended calls."""
    _packed(packed, E, H, F, packed.device)
    need = frag_bytes(E, H, F)
    if need == 0:
        raise ValueError(f"H={H}, F={F} has no fragment-ordered copies (needs H % 256 == 0 and F % 128 == 0)")
    if frag is None:
        frag = torch.empty(need // 2, dtype=torch.bfloat16, device=packed.device)
    _frag(frag, E, H, F, packed.device)
    _check(lib.gg_pack_frag(E, H, F, packed.data_ptr(), packed.numel() * 2, frag.data_ptr(), frag.numel() * 2,
                            _stream_ptr(stream, packed.device)), "gg_pack_frag")
    return frag


def expert_views(packed: torch.Tensor, E: int, H: int, F: int):
    """(w1_views, w2_views): per-expert views into the packed buffer.  A
    fragment buffer derived from it does not follow writes through them: call
    gg_pack_frag again."""
    per = packed_bytes(1, H, F) // 2
    w1 = [packed[e * per:e * per + 2 * F * H].view(2 * F, H) for e in range(E)]
    w2 = [packed[e * per + 2 * F * H:e * per + 3 * F * H].view(H, F) for e in range(E)]
    return w1, w2


def gg_forward_fc1_swiglu(x: torch.Tensor, offsets: torch.Tensor, packed: torch.Tensor,
                          E: int, H: int, F: int, save_h1: bool = True,
                          h1_out: Optional[torch.Tensor] = None, a_out: Optional[torch.Tensor] = None,
                          stream: Optional[torch.cuda.Stream] = None
                          ) -> Tuple[Optional[torch.Tensor], torch.Tensor]:
    """FC1 (x [M, H] -> H1 [M, 2F]) with the fused SwiGLU -> A [M, F]."""
    _bf16_cuda(x, "x")
    M, dev = x.shape[0], x.device
    _bf16_cuda(x, "x", shape=(M, H))
    _packed(packed, E, H, F, dev)
    off = _offsets(offsets, E, dev)
    if h1_out is not None:
        _bf16_cuda(h1_out, "h1_out", shape=(M, 2 * F), device=dev)
    a_out = _out(a_out, (M, F), "a_out", dev)
    if h1_out is None and save_h1:
        h1_out = _out(None, (M, 2 * F), "h1_out", dev)
    _check(lib.gg_forward_fc1_swiglu(x.data_ptr(), off.data_ptr(), M, packed.data_ptr(), E, H, F,
                                     _ptr(h1_out), a_out.data_ptr(), _stream_ptr(stream, dev)),
           "gg_forward_fc1_swiglu")
    return h1_out, a_out


def gg_forward_fc2(a: torch.Tensor, offsets: torch.Tensor, packed: torch.Tensor,
                   E: int, H: int, F: int, y: Optional[torch.Tensor] = None,
                   stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """FC2: a [M, F] -> y [M, H]."""
    return gg_forward_fc2_frag(a, offsets, packed, None, E, H, F, y=y, stream=stream)


def gg_forward_fc2_frag(a: torch.Tensor, offsets: torch.Tensor, packed: torch.Tensor,
                        frag: Optional[torch.Tensor], E: int, H: int, F: int, y: Optional[torch.Tensor] = None,
                        stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """FC2 with an optional fragment buffer (gg_pack_frag): a [M, F] -> y [M, H]."""
    _bf16_cuda(a, "a")
    M, dev = a.shape[0], a.device
    _bf16_cuda(a, "a", shape=(M, F))
    _packed(packed, E, H, F, dev)
    fr = _frag(frag, E, H, F, dev)
    off = _offsets(offsets, E, dev)
    y = _out(y, (M, H), "y", dev)
    if fr is None:
        st = lib.gg_forward_fc2(a.data_ptr(), off.data_ptr(), M, packed.data_ptr(), E, H, F, y.data_ptr(),
                                _stream_ptr(stream, dev))
        _check(st, "gg_forward_fc2")
    else:
        st = lib.gg_forward_fc2_frag(a.data_ptr(), off.data_ptr(), M, packed.data_ptr(), fr.data_ptr(), E, H, F,
                                     y.data_ptr(), _stream_ptr(stream, dev))
        _check(st, "gg_forward_fc2_frag")
    return y


def gg_dgrad(dy: torch.Tensor, h1: torch.Tensor, offsets: torch.Tensor, packed: torch.Tensor,
             E: int, H: int, F: int, workspace: Optional[torch.Tensor] = None,
             dx: Optional[torch.Tensor] = None,
             stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Input gradient: dy [M, H], saved h1 [M, 2F] -> dx [M, H].  The
    workspace (bf16 [M, 2F] or any buffer of dgrad_workspace_bytes) receives dH1."""
    _bf16_cuda(dy, "dy")
    M, dev = dy.shape[0], dy.device
    _bf16_cuda(dy, "dy", shape=(M, H))
    _bf16_cuda(h1, "h1", shape=(M, 2 * F), device=dev)
    _packed(packed, E, H, F, dev)
    off = _offsets(offsets, E, dev)
    if dx is not None:
        _bf16_cuda(dx, "dx", shape=(M, H), device=dev)
    if workspace is not None:
        _workspace(workspace, dgrad_workspace_bytes(M, F), dev)
    else:
        workspace = torch.empty(M, 2 * F, dtype=torch.bfloat16, device=dev)
    dx = _out(dx, (M, H), "dx", dev)
    _check(lib.gg_dgrad(dy.data_ptr(), h1.data_ptr(), off.data_ptr(), M, packed.data_ptr(), E, H, F,
                        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                        dx.data_ptr(), _stream_ptr(stream, dev)), "gg_dgrad")
    return dx


NOALLOC_SCRATCH_BYTES = 128 << 20    # GG_NOALLOC_SCRATCH_BYTES of include/gg.h


def gg_dgrad_noalloc(dy: torch.Tensor, h1: torch.Tensor, offsets: torch.Tensor, packed: torch.Tensor,
                     E: int, H: int, F: int, dx: Optional[torch.Tensor] = None,
                     stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """gg_dgrad with dH1 kept in the library's static per-GPU scratch (no
    workspace; 4*M*F <= NOALLOC_SCRATCH_BYTES).  Calls that overlap on one GPU
    race; with dx given, nothing is allocated."""
    _bf16_cuda(dy, "dy")
    M, dev = dy.shape[0], dy.device
    _bf16_cuda(dy, "dy", shape=(M, H))
    _bf16_cuda(h1, "h1", shape=(M, 2 * F), device=dev)
    _packed(packed, E, H, F, dev)
    off = _offsets(offsets, E, dev)
    dx = _out(dx, (M, H), "dx", dev)
    _check(lib.gg_dgrad_noalloc(dy.data_ptr(), h1.data_ptr(), off.data_ptr(), M, packed.data_ptr(), E, H, F,
                                dx.data_ptr(), _stream_ptr(stream, dev)), "gg_dgrad_noalloc")
    return dx


def _activation(activation) -> int:
    if isinstance(activation, str):
        if activation not in ACTIVATIONS:
            raise ValueError(f"activation must be one of {sorted(ACTIVATIONS)}")
        return ACTIVATIONS[activation]
    return int(activation)


def _probs_cuda(probs: Optional[torch.Tensor], M: int, device, name: str = "probs") -> Optional[torch.Tensor]:
    if probs is None:
        return None
    if (probs.dtype != torch.float32 or not probs.is_cuda or probs.shape != (M,) or not probs.is_contiguous()
            or probs.device != device):
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape [M] on {device}")
    return probs


def dgrad_glu_workspace_bytes(M: int, F: int, with_dprobs: bool) -> int:
    return int(lib.gg_dgrad_glu_workspace_bytes(M, F, int(bool(with_dprobs))))


def gg_forward_fc1_glu(x: torch.Tensor, offsets: torch.Tensor, packed: torch.Tensor,
                       E: int, H: int, F: int, activation="swiglu", probs: Optional[torch.Tensor] = None,
                       save_h1: bool = True, h1_out: Optional[torch.Tensor] = None,
                       a_out: Optional[torch.Tensor] = None, frag: Optional[torch.Tensor] = None,
                       stream: Optional[torch.cuda.Stream] = None
                       ) -> Tuple[Optional[torch.Tensor], torch.Tensor]:
    """FC1 with the fused activation ("swiglu" | "qgeglu"), optionally scaled
    per row by probs (float32 [M]) -> (H1 or None, A).  frag: optional
    fragment buffer (gg_pack_frag) of the same weights."""
    _bf16_cuda(x, "x")
    M, dev = x.shape[0], x.device
    _bf16_cuda(x, "x", shape=(M, H))
    _packed(packed, E, H, F, dev)
    fr = _frag(frag, E, H, F, dev)
    off = _offsets(offsets, E, dev)
    pr = _probs_cuda(probs, M, dev)
    if h1_out is not None:
        _bf16_cuda(h1_out, "h1_out", shape=(M, 2 * F), device=dev)
    a_out = _out(a_out, (M, F), "a_out", dev)
    if h1_out is None and save_h1:
        h1_out = _out(None, (M, 2 * F), "h1_out", dev)
    _check(lib.gg_forward_fc1_glu(x.data_ptr(), off.data_ptr(), M, packed.data_ptr(), _ptr(fr), E, H, F,
                                  _activation(activation), _ptr(pr), _ptr(h1_out), a_out.data_ptr(),
                                  _stream_ptr(stream, dev)), "gg_forward_fc1_glu")
    return h1_out, a_out


def gg_dgrad_glu(dy: torch.Tensor, h1: torch.Tensor, offsets: torch.Tensor, packed: torch.Tensor,
                 E: int, H: int, F: int, activation="swiglu", probs: Optional[torch.Tensor] = None,
                 want_dprobs: bool = True, workspace: Optional[torch.Tensor] = None,
                 dx: Optional[torch.Tensor] = None, dprobs: Optional[torch.Tensor] = None,
                 frag: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None
                 ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Input gradient of gg_forward_fc1_glu + FC2 -> (dx, dprobs or None).
    The workspace (a byte buffer of dgrad_glu_workspace_bytes) keeps dH1 [M, 2F]
    bf16 at its start.  frag: optional fragment buffer (gg_pack_frag)."""
    _bf16_cuda(dy, "dy")
    M, dev = dy.shape[0], dy.device
    _bf16_cuda(dy, "dy", shape=(M, H))
    _bf16_cuda(h1, "h1", shape=(M, 2 * F), device=dev)
    _packed(packed, E, H, F, dev)
    fr = _frag(frag, E, H, F, dev)
    off = _offsets(offsets, E, dev)
    pr = _probs_cuda(probs, M, dev)
    dprobs = _probs_cuda(dprobs, M, dev, "dprobs")
    if dx is not None:
        _bf16_cuda(dx, "dx", shape=(M, H), device=dev)
    with_dp = dprobs is not None or want_dprobs
    if workspace is not None:
        _workspace(workspace, dgrad_glu_workspace_bytes(M, F, with_dp), dev)
    if dprobs is None and want_dprobs:
        dprobs = torch.empty(M, dtype=torch.float32, device=dev)
    workspace = _workspace(workspace, dgrad_glu_workspace_bytes(M, F, with_dp), dev)
    dx = _out(dx, (M, H), "dx", dev)
    _check(lib.gg_dgrad_glu(dy.data_ptr(), h1.data_ptr(), off.data_ptr(), M, packed.data_ptr(), _ptr(fr), E, H, F,
                            _activation(activation), _ptr(pr), workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), dx.data_ptr(), _ptr(dprobs),
                            _stream_ptr(stream, dev)), "gg_dgrad_glu")
    return dx, dprobs


def gg_dgrad_recompute(dy: torch.Tensor, x: torch.Tensor, offsets: torch.Tensor, packed: torch.Tensor,
                       E: int, H: int, F: int, activation="swiglu", probs: Optional[torch.Tensor] = None,
                       want_dprobs: bool = False, workspace: Optional[torch.Tensor] = None,
                       dx: Optional[torch.Tensor] = None, dprobs: Optional[torch.Tensor] = None,
                       frag: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None
                       ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Input gradient without a saved H1: FC1 is recomputed from the forward
    input x [M, H] inside the call -> (dx, dprobs or None).  The workspace
    ends up holding dH1 [M, 2F] bf16 at its start."""
    _bf16_cuda(dy, "dy")
    M, dev = dy.shape[0], dy.device
    _bf16_cuda(dy, "dy", shape=(M, H))
    _bf16_cuda(x, "x", shape=(M, H), device=dev)
    _packed(packed, E, H, F, dev)
    fr = _frag(frag, E, H, F, dev)
    off = _offsets(offsets, E, dev)
    pr = _probs_cuda(probs, M, dev)
    dprobs = _probs_cuda(dprobs, M, dev, "dprobs")
    if dx is not None:
        _bf16_cuda(dx, "dx", shape=(M, H), device=dev)
    with_dp = dprobs is not None or want_dprobs
    if workspace is not None:
        _workspace(workspace, dgrad_glu_workspace_bytes(M, F, with_dp), dev)
    if dprobs is None and want_dprobs:
        dprobs = torch.empty(M, dtype=torch.float32, device=dev)
    workspace = _workspace(workspace, dgrad_glu_workspace_bytes(M, F, with_dp), dev)
    dx = _out(dx, (M, H), "dx", dev)
    _check(lib.gg_dgrad_recompute(dy.data_ptr(), x.data_ptr(), off.data_ptr(), M, packed.data_ptr(), _ptr(fr),
                                  E, H, F, _activation(activation), _ptr(pr), workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(), dx.data_ptr(), _ptr(dprobs),
                                  _stream_ptr(stream, dev)), "gg_dgrad_recompute")
    return dx, dprobs


def gg_round_bf16(x: torch.Tensor, stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Diagnostic: device fp32 -> bf16 rounding as used by the epilogues."""
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 device tensor")
    out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    _check(lib.gg_round_bf16(x.data_ptr(), out.data_ptr(), x.numel(), _stream_ptr(stream, x.device)),
           "gg_round_bf16")
    return out


def gg_scale_rows(x: torch.Tensor, probs: torch.Tensor, out: Optional[torch.Tensor] = None,
                  stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Router probability on the FC1 input: out [M, H] = bf16(probs[r] * x[r])
    for every row (out may be x).  x bf16 [M, H]; probs fp32 [M]."""
    x = _bf16_cuda(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be [M, H]")
    M, H = x.shape
    pr = _probs_cuda(probs, M, x.device)
    if pr is None:
        raise ValueError("probs is required")
    out = _out(out, (M, H), "out", x.device)
    _check(lib.gg_scale_rows(x.data_ptr(), pr.data_ptr(), M, H, out.data_ptr(), _stream_ptr(stream, x.device)),
           "gg_scale_rows")
    return out


def gg_scale_rows_backward(dxs: torch.Tensor, x: torch.Tensor, probs: torch.Tensor, want_dprobs: bool = True,
                           dx: Optional[torch.Tensor] = None, dprobs: Optional[torch.Tensor] = None,
                           stream: Optional[torch.cuda.Stream] = None):
    """Input gradient of gg_scale_rows given dxs = dL/dx' [M, H] and the
    unscaled x: (dx = bf16(probs[r] * dxs[r]), dprobs[r] = sum_h dxs*x in fp32
    or None).  dx may be dxs."""
    dxs = _bf16_cuda(dxs, "dxs")
    if dxs.dim() != 2:
        raise ValueError("dxs must be [M, H]")
    M, H = dxs.shape
    x = _bf16_cuda(x, "x", (M, H), dxs.device)
    pr = _probs_cuda(probs, M, dxs.device)
    if pr is None:
        raise ValueError("probs is required")
    dx = _out(dx, (M, H), "dx", dxs.device)
    dprobs = _probs_cuda(dprobs, M, dxs.device, "dprobs")
    if dprobs is None and want_dprobs:
        dprobs = torch.empty(M, dtype=torch.float32, device=dxs.device)
    _check(lib.gg_scale_rows_backward(dxs.data_ptr(), x.data_ptr(), pr.data_ptr(), M, H, dx.data_ptr(),
                                      _ptr(dprobs), _stream_ptr(stream, dxs.device)), "gg_scale_rows_backward")
    return dx, dprobs


class ScaleRows(torch.autograd.Function):
    """Autograd wrapper of gg_scale_rows: x' = bf16(probs[r] * x[r]); the
    backward gives dx and, when probs requires grad, dprobs."""

    @staticmethod
    def forward(ctx, x, probs):
        ctx.save_for_backward(x, probs)
        return gg_scale_rows(x, probs.detach())

    @staticmethod
    def backward(ctx, g):
        x, probs = ctx.saved_tensors
        dx, dprobs = gg_scale_rows_backward(g.contiguous(), x, probs.detach(),
                                            want_dprobs=ctx.needs_input_grad[1])
        return dx, dprobs


class FrozenExpertMLP(torch.autograd.Function):
    """Autograd wrapper: forward FC1 -> SwiGLU -> FC2, backward = input
    gradient only (the packed base weights are frozen)."""

    @staticmethod
    def forward(ctx, x, offsets, packed, E, H, F):
        h1, a = gg_forward_fc1_swiglu(x, offsets, packed, E, H, F, save_h1=True)
        y = gg_forward_fc2(a, offsets, packed, E, H, F)
        ctx.save_for_backward(h1, offsets, packed)
        ctx.shape = (E, H, F)
        return y

    @staticmethod
    def backward(ctx, dy):
        h1, offsets, packed = ctx.saved_tensors
        E, H, F = ctx.shape
        dx = gg_dgrad(dy.contiguous(), h1, offsets, packed, E, H, F)
        return dx, None, None, None, None, None
