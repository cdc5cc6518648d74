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

The *_glu calls add the QuickGeGLU activation and the weighting of the
activation by each row's router probability (fp32 [M]), with dp of that
weight from the input gradient.

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
            "gg_dgrad_glu_workspace_bytes", "gg_forward_fc1_glu", "gg_dgrad_glu", "gg_dgrad_recompute")


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
    lib.gg_dgrad_workspace_bytes.argtypes = [i64, i64]
    lib.gg_dgrad_workspace_bytes.restype = sz
    lib.gg_pack_weights.argtypes = [i64, i64, i64, ctypes.POINTER(p), ctypes.POINTER(p), p, sz, p]
    lib.gg_forward_fc1_swiglu.argtypes = [p, p, i64, p, i64, i64, i64, p, p, p]
    lib.gg_forward_fc2.argtypes = [p, p, i64, p, i64, i64, i64, p, p]
    lib.gg_dgrad.argtypes = [p, p, p, i64, p, i64, i64, i64, p, sz, p, p]
    lib.gg_round_bf16.argtypes = [p, p, i64, p]
    lib.gg_dgrad_glu_workspace_bytes.argtypes = [i64, i64, i32]
    lib.gg_dgrad_glu_workspace_bytes.restype = sz
    lib.gg_forward_fc1_glu.argtypes = [p, p, i64, p, i64, i64, i64, i32, p, p, p, p]
    lib.gg_dgrad_glu.argtypes = [p, p, p, i64, p, i64, i64, i64, i32, p, p, sz, p, p, p]
    lib.gg_dgrad_recompute.argtypes = [p, p, p, i64, p, i64, i64, i64, i32, p, p, sz, p, p, p]
    for name in ("gg_pack_weights", "gg_forward_fc1_swiglu", "gg_forward_fc2", "gg_dgrad",
                 "gg_round_bf16", "gg_forward_fc1_glu", "gg_dgrad_glu", "gg_dgrad_recompute"):
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


def _stream_ptr(stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _bf16_cuda(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _offsets(offsets: torch.Tensor, E: int) -> torch.Tensor:
    if offsets.dtype != torch.int64 or not offsets.is_cuda or offsets.shape != (E + 1,):
        raise ValueError("offsets must be an int64 device tensor of shape [E+1]")
    return offsets.contiguous()


def packed_bytes(E: int, H: int, F: int) -> int:
    return int(lib.gg_packed_bytes(E, H, F))


def dgrad_workspace_bytes(M: int, F: int) -> int:
    return int(lib.gg_dgrad_workspace_bytes(M, F))


def gg_pack_weights(w1: Union[torch.Tensor, Sequence[torch.Tensor]],
                    w2: Union[torch.Tensor, Sequence[torch.Tensor]],
                    packed: Optional[torch.Tensor] = None,
                    stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Pack frozen expert weights (w1[e]: [2F, H], gate rows then up rows;
    w2[e]: [H, F]) into one expert-major bf16 buffer.  Returns the packed
    buffer (1-D, packed_bytes(E, H, F) / 2 elements).  Per-expert views into it:
    ``expert_views(packed, E, H, F)``."""
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
    E = len(w1s)
    twoF, H = w1s[0].shape
    F = twoF // 2
    if twoF != 2 * F or any(t.shape != (2 * F, H) for t in w1s) or any(t.shape != (H, F) for t in w2s):
        raise ValueError("w1[e] must be [2F, H] and w2[e] must be [H, F] for every expert")
    nbytes = packed_bytes(E, H, F)
    if packed is None:
        packed = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=w1s[0].device)
    arr1 = (ctypes.c_void_p * E)(*[t.data_ptr() for t in w1s])
    arr2 = (ctypes.c_void_p * E)(*[t.data_ptr() for t in w2s])
    _check(lib.gg_pack_weights(E, H, F, arr1, arr2, packed.data_ptr(), packed.numel() * 2,
                               _stream_ptr(stream)), "gg_pack_weights")
    return packed


def expert_views(packed: torch.Tensor, E: int, H: int, F: int):
    """(w1_views, w2_views): per-expert views into the packed buffer.  After
    writing through them, call gg_pack_weights(w1_views, w2_views, packed=packed)
    so that the derived fragment-ordered copies follow."""
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
    _bf16_cuda(packed, "packed")
    M = x.shape[0]
    if x.shape != (M, H):
        raise ValueError("x must be [M, H]")
    off = _offsets(offsets, E)
    if a_out is None:
        a_out = torch.empty(M, F, dtype=torch.bfloat16, device=x.device)
    if h1_out is None and save_h1:
        h1_out = torch.empty(M, 2 * F, dtype=torch.bfloat16, device=x.device)
    _check(lib.gg_forward_fc1_swiglu(x.data_ptr(), off.data_ptr(), M, packed.data_ptr(), E, H, F,
                                     _ptr(h1_out), a_out.data_ptr(), _stream_ptr(stream)),
           "gg_forward_fc1_swiglu")
    return h1_out, a_out


def gg_forward_fc2(a: torch.Tensor, offsets: torch.Tensor, packed: torch.Tensor,
                   E: int, H: int, F: int, y: Optional[torch.Tensor] = None,
                   stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """FC2: a [M, F] -> y [M, H]."""
    _bf16_cuda(a, "a")
    _bf16_cuda(packed, "packed")
    M = a.shape[0]
    if a.shape != (M, F):
        raise ValueError("a must be [M, F]")
    off = _offsets(offsets, E)
    if y is None:
        y = torch.empty(M, H, dtype=torch.bfloat16, device=a.device)
    _check(lib.gg_forward_fc2(a.data_ptr(), off.data_ptr(), M, packed.data_ptr(), E, H, F,
                              y.data_ptr(), _stream_ptr(stream)), "gg_forward_fc2")
    return y


def gg_dgrad(dy: torch.Tensor, h1: torch.Tensor, offsets: torch.Tensor, packed: torch.Tensor,
             E: int, H: int, F: int, workspace: Optional[torch.Tensor] = None,
             dx: Optional[torch.Tensor] = None,
             stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Input gradient: dy [M, H], saved h1 [M, 2F] -> dx [M, H].  The
    workspace (bf16 [M, 2F] or larger) receives dH1."""
    _bf16_cuda(dy, "dy")
    _bf16_cuda(h1, "h1")
    _bf16_cuda(packed, "packed")
    M = dy.shape[0]
    if dy.shape != (M, H) or h1.shape != (M, 2 * F):
        raise ValueError("dy must be [M, H] and h1 [M, 2F]")
    off = _offsets(offsets, E)
    if workspace is None:
        workspace = torch.empty(M, 2 * F, dtype=torch.bfloat16, device=dy.device)
    if dx is None:
        dx = torch.empty(M, H, dtype=torch.bfloat16, device=dy.device)
    _check(lib.gg_dgrad(dy.data_ptr(), h1.data_ptr(), off.data_ptr(), M, packed.data_ptr(), E, H, F,
                        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                        dx.data_ptr(), _stream_ptr(stream)), "gg_dgrad")
    return dx


def _activation(activation) -> int:
    if isinstance(activation, str):
        if activation not in ACTIVATIONS:
            raise ValueError(f"activation must be one of {sorted(ACTIVATIONS)}")
        return ACTIVATIONS[activation]
    return int(activation)


def _probs_cuda(probs: Optional[torch.Tensor], M: int, name: str = "probs") -> Optional[torch.Tensor]:
    if probs is None:
        return None
    if probs.dtype != torch.float32 or not probs.is_cuda or probs.shape != (M,) or not probs.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 device tensor of shape [M]")
    return probs


def dgrad_glu_workspace_bytes(M: int, F: int, with_dprobs: bool) -> int:
    return int(lib.gg_dgrad_glu_workspace_bytes(M, F, int(bool(with_dprobs))))


def gg_forward_fc1_glu(x: torch.Tensor, offsets: torch.Tensor, packed: torch.Tensor,
                       E: int, H: int, F: int, activation="swiglu", probs: Optional[torch.Tensor] = None,
                       save_h1: bool = True, h1_out: Optional[torch.Tensor] = None,
                       a_out: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None
                       ) -> Tuple[Optional[torch.Tensor], torch.Tensor]:
    """FC1 with the fused activation ("swiglu" | "qgeglu"), optionally scaled
    per row by probs (float32 [M]) -> (H1 or None, A)."""
    _bf16_cuda(x, "x")
    _bf16_cuda(packed, "packed")
    M = x.shape[0]
    if x.shape != (M, H):
        raise ValueError("x must be [M, H]")
    off = _offsets(offsets, E)
    pr = _probs_cuda(probs, M)
    if a_out is None:
        a_out = torch.empty(M, F, dtype=torch.bfloat16, device=x.device)
    if h1_out is None and save_h1:
        h1_out = torch.empty(M, 2 * F, dtype=torch.bfloat16, device=x.device)
    _check(lib.gg_forward_fc1_glu(x.data_ptr(), off.data_ptr(), M, packed.data_ptr(), E, H, F,
                                  _activation(activation), _ptr(pr), _ptr(h1_out), a_out.data_ptr(),
                                  _stream_ptr(stream)), "gg_forward_fc1_glu")
    return h1_out, a_out


def gg_dgrad_glu(dy: torch.Tensor, h1: torch.Tensor, offsets: torch.Tensor, packed: torch.Tensor,
                 E: int, H: int, F: int, activation="swiglu", probs: Optional[torch.Tensor] = None,
                 want_dprobs: bool = True, workspace: Optional[torch.Tensor] = None,
                 dx: Optional[torch.Tensor] = None, dprobs: Optional[torch.Tensor] = None,
                 stream: Optional[torch.cuda.Stream] = None
                 ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Input gradient of gg_forward_fc1_glu + FC2 -> (dx, dprobs or None).
    The workspace (a byte buffer of dgrad_glu_workspace_bytes) keeps dH1 [M, 2F]
    bf16 at its start."""
    _bf16_cuda(dy, "dy")
    _bf16_cuda(h1, "h1")
    _bf16_cuda(packed, "packed")
    M = dy.shape[0]
    if dy.shape != (M, H) or h1.shape != (M, 2 * F):
        raise ValueError("dy must be [M, H] and h1 [M, 2F]")
    off = _offsets(offsets, E)
    pr = _probs_cuda(probs, M)
    if dprobs is None and want_dprobs:
        dprobs = torch.empty(M, dtype=torch.float32, device=dy.device)
    dprobs = _probs_cuda(dprobs, M, "dprobs")
    if workspace is None:
        workspace = torch.empty(dgrad_glu_workspace_bytes(M, F, dprobs is not None), dtype=torch.uint8,
                                device=dy.device)
    if dx is None:
        dx = torch.empty(M, H, dtype=torch.bfloat16, device=dy.device)
    _check(lib.gg_dgrad_glu(dy.data_ptr(), h1.data_ptr(), off.data_ptr(), M, packed.data_ptr(), E, H, F,
                            _activation(activation), _ptr(pr), workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), dx.data_ptr(), _ptr(dprobs),
                            _stream_ptr(stream)), "gg_dgrad_glu")
    return dx, dprobs


def gg_dgrad_recompute(dy: torch.Tensor, x: torch.Tensor, offsets: torch.Tensor, packed: torch.Tensor,
                       E: int, H: int, F: int, activation="swiglu", probs: Optional[torch.Tensor] = None,
                       want_dprobs: bool = False, workspace: Optional[torch.Tensor] = None,
                       dx: Optional[torch.Tensor] = None, dprobs: Optional[torch.Tensor] = None,
                       stream: Optional[torch.cuda.Stream] = None
                       ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Input gradient without a saved H1: FC1 is recomputed from the forward
    input x [M, H] inside the call -> (dx, dprobs or None).  The workspace
    ends up holding dH1 [M, 2F] bf16 at its start."""
    _bf16_cuda(dy, "dy")
    _bf16_cuda(x, "x")
    _bf16_cuda(packed, "packed")
    M = dy.shape[0]
    if dy.shape != (M, H) or x.shape != (M, H):
        raise ValueError("dy and x must be [M, H]")
    off = _offsets(offsets, E)
    pr = _probs_cuda(probs, M)
    if dprobs is None and want_dprobs:
        dprobs = torch.empty(M, dtype=torch.float32, device=dy.device)
    dprobs = _probs_cuda(dprobs, M, "dprobs")
    if workspace is None:
        workspace = torch.empty(dgrad_glu_workspace_bytes(M, F, dprobs is not None), dtype=torch.uint8,
                                device=dy.device)
    if dx is None:
        dx = torch.empty(M, H, dtype=torch.bfloat16, device=dy.device)
    _check(lib.gg_dgrad_recompute(dy.data_ptr(), x.data_ptr(), off.data_ptr(), M, packed.data_ptr(), E, H, F,
                                  _activation(activation), _ptr(pr), workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(), dx.data_ptr(), _ptr(dprobs),
                                  _stream_ptr(stream)), "gg_dgrad_recompute")
    return dx, dprobs


def gg_round_bf16(x: torch.Tensor, stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """Diagnostic: device fp32 -> bf16 rounding as used by the epilogues."""
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 device tensor")
    out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    _check(lib.gg_round_bf16(x.data_ptr(), out.data_ptr(), x.numel(), _stream_ptr(stream)),
           "gg_round_bf16")
    return out


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
