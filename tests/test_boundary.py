"""The C-ABI boundary on the CPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before any HIP call (no GPU
needed, no compute launched)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gg.h")


def _gg():
    import moe_expert_grouped_ragged_amd as gg
    return gg


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gg_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("gg_pack_weights", "gg_forward_fc1_swiglu", "gg_forward_fc2", "gg_dgrad"):
        assert n in names


def test_library_exports_every_declared_symbol():
    gg = _gg()
    lib = ctypes.CDLL(gg.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", gg.LIB_PATH], capture_output=True, text=True)
    exported = set(re.findall(r"\bT (gg_[a-z0-9_]+)", out.stdout))
    assert set(declared_functions()) <= exported
    # the binding gives every declared function its C signature
    assert set(gg.EXPORTED) == set(declared_functions())
    for n in gg.EXPORTED:
        assert getattr(gg.lib, n).argtypes is not None, n


def test_header_compiles_as_c():
    src = f'#include "{HEADER}"\nint main(void) {{ return (int)gg_packed_bytes(1, 8, 8) == 0; }}\n'
    proc = subprocess.run(["gcc", "-x", "c", "-std=c99", "-fsyntax-only", "-I/opt/rocm/include",
                           "-D__HIP_PLATFORM_AMD__", "-"], input=src, capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr


def test_size_helpers():
    """The packed buffer is exactly the weights, 6*E*H*F bytes, for every
    shape; the fragment-ordered copies are a separate, opt-in buffer of
    12*E*H*F bytes for shapes with H % 256 == 0 and F % 128 == 0 only."""
    gg = _gg()
    import workload
    assert gg.packed_bytes(4, 64, 128) == 6 * 4 * 64 * 128
    assert gg.dgrad_workspace_bytes(512, 128) == 4 * 512 * 128
    assert gg.packed_bytes(0, 64, 128) == 0
    for E, H, F in ((2, 256, 128), (2, 256, 64), (2, 384, 128), (7, 512, 1024)):
        assert gg.packed_bytes(E, H, F) == 6 * E * H * F
    for w in workload.WORKLOADS:
        assert gg.packed_bytes(w.E, w.H, w.F) == 6 * w.E * w.H * w.F
    # the largest workload's weights take 6.4 GB by default
    w = workload.by_name("padded_e128_h4096_f2048")
    assert gg.packed_bytes(w.E, w.H, w.F) == 6442450944
    assert gg.frag_bytes(2, 256, 128) == 12 * 2 * 256 * 128
    assert gg.frag_bytes(2, 256, 64) == 0 and gg.frag_bytes(2, 384, 128) == 0
    assert gg.frag_bytes(0, 256, 128) == 0
    assert gg.has_frag(4096, 2048) and not gg.has_frag(2688, 1856)
    assert gg.lib.gg_status_string(5) == b"GG_ERR_ALIASING"


def test_fragment_entry_points_validate_before_any_hip_call():
    gg = _gg()
    L = gg.lib
    INV, MIS, WS, ALI = (gg.GG_ERR_INVALID_ARGUMENT, gg.GG_ERR_MISALIGNED,
                         gg.GG_ERR_WORKSPACE_TOO_SMALL, gg.GG_ERR_ALIASING)
    base = 1 << 40
    E, H, F = 2, 256, 128
    pk, fr = base, base + 2 ** 30
    pb, fb = gg.packed_bytes(E, H, F), gg.frag_bytes(E, H, F)
    # a shape without copies, null or misaligned buffers, sizes, overlap
    assert L.gg_pack_frag(E, 264, F, pk, 1 << 30, fr, 1 << 30, None) == INV
    assert L.gg_pack_frag(E, H, 136, pk, 1 << 30, fr, 1 << 30, None) == INV
    assert L.gg_pack_frag(E, H, F, None, pb, fr, fb, None) == INV
    assert L.gg_pack_frag(E, H, F, pk, pb, fr + 8, fb, None) == MIS
    assert L.gg_pack_frag(E, H, F, pk, pb - 1, fr, fb, None) == WS
    assert L.gg_pack_frag(E, H, F, pk, pb, fr, fb - 1, None) == WS
    assert L.gg_pack_frag(E, H, F, pk, pb, pk + pb - 16, fb, None) == ALI
    # the extended calls: a frag for a shape without copies, misaligned, or overlapping an output
    M = 8
    x, off, a, y = base + 2 ** 31, base + 2 ** 32, base + 2 ** 33, base + 2 ** 34
    assert L.gg_forward_fc2_frag(a, off, M, pk, fr, E, 264, F, y, None) == INV
    assert L.gg_forward_fc2_frag(a, off, M, pk, fr + 8, E, H, F, y, None) == MIS
    assert L.gg_forward_fc2_frag(a, off, M, pk, fr, E, H, F, fr + 64, None) == ALI
    assert L.gg_forward_fc1_glu(x, off, M, pk, fr, E, H, 136, 0, None, None, a, None) == INV
    assert L.gg_forward_fc1_glu(x, off, M, pk, fr, E, H, F, 0, None, None, fr + fb - 16, None) == ALI
    ws, dx = base + 2 ** 35, base + 2 ** 36
    need = gg.dgrad_workspace_bytes(M, F)
    assert L.gg_dgrad_glu(x, a, off, M, pk, fr + 4, E, H, F, 0, None, ws, need, dx, None, None) == MIS
    assert L.gg_dgrad_glu(x, a, off, M, pk, fr, E, H, F, 0, None, ws, need, fr, None, None) == ALI
    assert L.gg_dgrad_recompute(x, a, off, M, pk, fr, E, 264, F, 0, None, ws, need, dx, None, None) == INV
    # empty batch: success without touching the pointers, a valid frag or not
    assert L.gg_forward_fc2_frag(None, None, 0, None, None, E, H, F, None, None) == 0
    assert L.gg_forward_fc2_frag(None, None, 0, None, fr, E, H, F, None, None) == 0


def test_python_binding_checks_buffers_before_any_call():
    """The binding refuses outputs, packed buffers, fragment buffers and
    offsets of the wrong dtype, shape, contiguity or size with ValueError,
    before any library call (the CPU tensors here would be refused for not
    being device tensors, so the checks are reached through fakes that pass
    the device test)."""
    gg = _gg()
    import torch

    class FakeCuda(torch.Tensor):
        """A CPU tensor that claims to be on the GPU (never reaches the library)."""
        @property
        def is_cuda(self):
            return True

        @property
        def device(self):
            return torch.device("cuda:0")

    def fake(shape, dtype=torch.bfloat16):
        return torch.zeros(*shape, dtype=dtype).as_subclass(FakeCuda)

    E, H, F, M = 2, 64, 64, 16
    x, off = fake((M, H)), fake((E + 1,), torch.int64)
    packed = fake((gg.packed_bytes(E, H, F) // 2,))
    with pytest.raises(ValueError, match="packed holds"):
        gg.gg_forward_fc1_swiglu(x, off, fake((gg.packed_bytes(E, H, F) // 2 - 1,)), E, H, F)
    with pytest.raises(ValueError, match="a_out must have shape"):
        gg.gg_forward_fc1_swiglu(x, off, packed, E, H, F, a_out=fake((M, F + 8)))
    with pytest.raises(ValueError, match="h1_out must be bfloat16"):
        gg.gg_forward_fc1_swiglu(x, off, packed, E, H, F, h1_out=fake((M, 2 * F), torch.float32))
    with pytest.raises(ValueError, match="y must be contiguous"):
        gg.gg_forward_fc2(fake((M, F)), off, packed, E, H, F, y=fake((H, M)).t())
    with pytest.raises(ValueError, match="dx must have shape"):
        gg.gg_dgrad(fake((M, H)), fake((M, 2 * F)), off, packed, E, H, F, dx=fake((M - 1, H)))
    with pytest.raises(ValueError, match="workspace holds"):
        gg.gg_dgrad(fake((M, H)), fake((M, 2 * F)), off, packed, E, H, F, workspace=fake((M, F)))
    with pytest.raises(ValueError, match="offsets must be"):
        gg.gg_forward_fc2(fake((M, F)), fake((E,), torch.int64), packed, E, H, F)
    with pytest.raises(ValueError, match="offsets must be a contiguous"):
        gg.gg_dgrad_noalloc(fake((M, H)), fake((M, 2 * F)), fake((2 * E + 2,), torch.int64)[::2], packed,
                            E, H, F)
    with pytest.raises(ValueError, match="no fragment-ordered copies"):
        gg.gg_forward_fc2_frag(fake((M, F)), off, packed, fake((1024,)), E, H, F)
    E2, H2, F2 = 2, 256, 128
    with pytest.raises(ValueError, match="frag holds"):
        gg.gg_forward_fc1_glu(fake((M, H2)), off, fake((gg.packed_bytes(E2, H2, F2) // 2,)), E2, H2, F2,
                              frag=fake((gg.frag_bytes(E2, H2, F2) // 2 - 8,)))


def test_validation_before_any_hip_call():
    gg = _gg()
    L = gg.lib
    INV, MIS, WS, ALI = (gg.GG_ERR_INVALID_ARGUMENT, gg.GG_ERR_MISALIGNED,
                         gg.GG_ERR_WORKSPACE_TOO_SMALL, gg.GG_ERR_ALIASING)
    # empty batch succeeds without touching pointers
    assert L.gg_forward_fc1_swiglu(None, None, 0, None, 4, 64, 128, None, None, None) == 0
    assert L.gg_forward_fc2(None, None, 0, None, 4, 64, 128, None, None) == 0
    assert L.gg_dgrad(None, None, None, 0, None, 4, 64, 128, None, 0, None, None) == 0
    # shapes
    assert L.gg_forward_fc2(16, 32, 8, 64, 0, 64, 128, 4096, None) == INV          # E < 1
    assert L.gg_forward_fc2(16, 32, 8, 64, 1025, 64, 128, 4096, None) == INV       # E too large
    assert L.gg_forward_fc2(16, 32, 8, 64, 4, 60, 128, 4096, None) == INV          # H % 8
    assert L.gg_forward_fc2(16, 32, 8, 64, 4, 64, 12, 4096, None) == INV           # F % 8
    assert L.gg_forward_fc2(16, 32, -1, 64, 4, 64, 128, 4096, None) == INV         # M < 0
    assert L.gg_forward_fc2(16, 32, 1 << 31, 64, 4, 64, 128, 4096, None) == INV    # M too large
    assert L.gg_forward_fc2(16, 32, 8, 64, 1, 1 << 22, 8, 4096, None) == INV        # H too large
    assert L.gg_forward_fc2(16, 32, 8, 64, 1, 64, 1 << 21, 4096, None) == INV       # 2F too large
    assert L.gg_forward_fc2(16, 32, 8, 64, 1, 1 << 15, 1 << 14, 4096, None) == INV  # W1_e >= 2 GiB
    # null pointers
    assert L.gg_forward_fc1_swiglu(None, 32, 8, 64, 4, 64, 128, None, 4096, None) == INV
    assert L.gg_forward_fc1_swiglu(16, 32, 8, 64, 4, 64, 128, None, None, None) == INV
    assert L.gg_dgrad(16, 4096, 32, 8, 1 << 20, 4, 64, 128, None, 1 << 20, 1 << 24, None) == INV
    # misalignment
    base = 1 << 40
    assert L.gg_forward_fc2(base + 2, base + 2 ** 30, 8, base + 2 ** 31, 4, 64, 128, base + 2 ** 32,
                            None) == MIS
    assert L.gg_forward_fc2(base, base + 2 ** 30 + 4, 8, base + 2 ** 31, 4, 64, 128, base + 2 ** 32,
                            None) == MIS
    # workspace too small
    M, H, F = 8, 64, 128
    need = gg.dgrad_workspace_bytes(M, F)
    assert L.gg_dgrad(base, base + 2 ** 30, base + 2 ** 31, M, base + 2 ** 32, 4, H, F,
                      base + 2 ** 33, need - 1, base + 2 ** 34, None) == WS
    # aliasing: output overlaps an input / another output
    assert L.gg_forward_fc2(base, base + 2 ** 30, M, base + 2 ** 31, 4, H, F, base + 64, None) == ALI
    assert L.gg_forward_fc1_swiglu(base, base + 2 ** 30, M, base + 2 ** 31, 4, H, F,
                                   base + 2 ** 32, base + 2 ** 32 + 16, None) == ALI
    assert L.gg_dgrad(base, base + 2 ** 30, base + 2 ** 31, M, base + 2 ** 32, 4, H, F,
                      base + 2 ** 33, need, base + 2 ** 33 + 32, None) == ALI
    # pack: bad sizes, too small a buffer, a source partially overlapping the buffer
    P = ctypes.c_void_p
    arr = (P * 2)(base, base + 2 ** 20)
    assert L.gg_pack_weights(2, 60, 8, arr, arr, base + 2 ** 32, 1 << 30, None) == INV
    assert L.gg_pack_weights(2, 64, 8, arr, arr, base + 2 ** 32, 10, None) == WS
    pk = base + 2 ** 32
    overl = (P * 2)(pk + 16, pk + 2 ** 16)
    assert L.gg_pack_weights(2, 64, 8, overl, overl, pk, gg.packed_bytes(2, 64, 8), None) == ALI
    # diagnostic rounding: negative n
    assert L.gg_round_bf16(base, base + 2 ** 30, -1, None) == INV


def test_glu_entry_points_validate_before_any_hip_call():
    gg = _gg()
    L = gg.lib
    INV, MIS, WS, ALI = (gg.GG_ERR_INVALID_ARGUMENT, gg.GG_ERR_MISALIGNED,
                         gg.GG_ERR_WORKSPACE_TOO_SMALL, gg.GG_ERR_ALIASING)
    base = 1 << 40
    M, H, F = 8, 64, 136
    x, off, pk, h1, a = base, base + 2 ** 30, base + 2 ** 31, base + 2 ** 32, base + 2 ** 33
    probs = base + 2 ** 34
    # the workspace sizes: dH1, then ceil(F/32) fp32 partial sums per row when dp is wanted
    assert gg.dgrad_glu_workspace_bytes(M, F, False) == 4 * M * F
    assert gg.dgrad_glu_workspace_bytes(M, F, True) == 4 * M * F + 4 * M * 5
    # empty batch and unknown activation (checked first)
    assert L.gg_forward_fc1_glu(None, None, 0, None, None, 4, H, F, 0, None, None, None, None) == 0
    assert L.gg_forward_fc1_glu(x, off, M, pk, None, 4, H, F, 2, None, h1, a, None) == INV
    assert L.gg_forward_fc1_glu(x, off, M, pk, None, 4, H, F, -1, None, h1, a, None) == INV
    assert L.gg_dgrad_glu(x, h1, off, M, pk, None, 4, H, F, 7, None, a, 1 << 20, base + 2 ** 35, None, None) == INV
    # probs / dprobs must be 4-byte aligned
    assert L.gg_forward_fc1_glu(x, off, M, pk, None, 4, H, F, 1, probs + 2, h1, a, None) == MIS
    ws, dx, dp = base + 2 ** 35, base + 2 ** 36, base + 2 ** 37
    need = gg.dgrad_glu_workspace_bytes(M, F, True)
    assert L.gg_dgrad_glu(x, h1, off, M, pk, None, 4, H, F, 1, probs, ws, need, dx, dp + 1, None) == MIS
    # the workspace must hold the partial sums when dprobs is given
    assert L.gg_dgrad_glu(x, h1, off, M, pk, None, 4, H, F, 1, probs, ws, need - 4, dx, dp, None) == WS
    # aliasing: probs is an input, dprobs an output
    assert L.gg_forward_fc1_glu(x, off, M, pk, None, 4, H, F, 0, a + 8, h1, a, None) == ALI
    assert L.gg_dgrad_glu(x, h1, off, M, pk, None, 4, H, F, 0, probs, ws, need, dx, ws + need - 4, None) == ALI
    assert L.gg_dgrad_glu(x, h1, off, M, pk, None, 4, H, F, 0, probs, ws, need, dx, probs, None) == ALI


def test_scale_rows_entry_points_validate_before_any_hip_call():
    """Router probability on the FC1 input: shapes, null pointers, alignment
    and overlaps are refused before any HIP call; in place (x_out == x,
    dx == dxs) is allowed and so not tried here (it would launch)."""
    gg = _gg()
    L = gg.lib
    INV, MIS, ALI = gg.GG_ERR_INVALID_ARGUMENT, gg.GG_ERR_MISALIGNED, gg.GG_ERR_ALIASING
    base = 1 << 40
    M, H = 8, 64                       # 1 KiB per [M][H] bf16 buffer
    x, pr, out = base, base + 2 ** 30, base + 2 ** 31
    g, dx, dp = base + 2 ** 32, base + 2 ** 33, base + 2 ** 34
    # empty batch: nothing to do, no pointers needed
    assert L.gg_scale_rows(None, None, 0, H, None, None) == 0
    assert L.gg_scale_rows_backward(None, None, None, 0, H, None, None, None) == 0
    # shapes
    assert L.gg_scale_rows(x, pr, M, 12, out, None) == INV
    assert L.gg_scale_rows(x, pr, M, 0, out, None) == INV
    assert L.gg_scale_rows(x, pr, -1, H, out, None) == INV
    assert L.gg_scale_rows_backward(g, x, pr, M, 4, dx, dp, None) == INV
    # null pointers (dprobs alone may be null)
    assert L.gg_scale_rows(None, pr, M, H, out, None) == INV
    assert L.gg_scale_rows(x, None, M, H, out, None) == INV
    assert L.gg_scale_rows_backward(g, x, None, M, H, dx, dp, None) == INV
    assert L.gg_scale_rows_backward(g, x, pr, M, H, None, dp, None) == INV
    # alignment: 16 bytes for the rows, 4 for probs and dprobs
    assert L.gg_scale_rows(x + 8, pr, M, H, out, None) == MIS
    assert L.gg_scale_rows(x, pr + 2, M, H, out, None) == MIS
    assert L.gg_scale_rows_backward(g, x, pr, M, H, dx + 8, dp, None) == MIS
    assert L.gg_scale_rows_backward(g, x, pr, M, H, dx, dp + 1, None) == MIS
    # overlaps other than exact in-place use
    assert L.gg_scale_rows(x, pr, M, H, x + 16, None) == ALI
    assert L.gg_scale_rows(x, out + 64, M, H, out, None) == ALI
    assert L.gg_scale_rows_backward(g, x, pr, M, H, g + 16, dp, None) == ALI
    assert L.gg_scale_rows_backward(g, x, pr, M, H, x, dp, None) == ALI
    assert L.gg_scale_rows_backward(g, x, pr, M, H, dx, dx + 64, None) == ALI
    assert L.gg_scale_rows_backward(g, x, pr, M, H, dx, pr, None) == ALI
    assert L.gg_scale_rows_backward(g, x, pr, M, H, dx, g + 32, None) == ALI


def test_scale_rows_binding_checks_before_any_call():
    gg = _gg()
    import torch
    x = torch.zeros(4, 16, dtype=torch.bfloat16)
    p = torch.ones(4, dtype=torch.float32)
    with pytest.raises(ValueError):
        gg.gg_scale_rows(x, p)                                   # host tensors
    with pytest.raises(ValueError):
        gg.gg_scale_rows(x.float(), p)                           # not bf16
    with pytest.raises(ValueError):
        gg.gg_scale_rows_backward(x, x, p)


def test_python_binding_refuses_unsupported_weights():
    gg = _gg()
    import torch
    w1 = torch.zeros(2, 16, 8, dtype=torch.float32)
    w2 = torch.zeros(2, 8, 8, dtype=torch.float32)
    with pytest.raises(ValueError, match="bfloat16"):
        gg.gg_pack_weights(w1, w2)
    w1 = torch.zeros(2, 16, 8, dtype=torch.bfloat16, requires_grad=True)
    w2 = torch.zeros(2, 8, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="frozen"):
        gg.gg_pack_weights(w1, w2)


def test_expert_views_slice_each_block():
    """expert_views: W1_e at e*3FH, W2_e right after it (host-side slicing
    only; a CPU tensor stands in for the packed buffer)."""
    import torch
    gg = _gg()
    for E, H, F in ((3, 64, 64), (3, 256, 128), (2, 512, 256)):
        n = gg.packed_bytes(E, H, F) // 2
        block = n // E
        assert block == 3 * F * H
        packed = torch.arange(n, dtype=torch.int64)
        w1, w2 = gg.expert_views(packed, E, H, F)
        for e in range(E):
            assert w1[e].shape == (2 * F, H) and w2[e].shape == (H, F)
            assert int(w1[e][0, 0]) == e * block and int(w1[e][-1, -1]) == e * block + 2 * F * H - 1
            assert int(w2[e][0, 0]) == e * block + 2 * F * H and int(w2[e][-1, -1]) == e * block + 3 * F * H - 1
