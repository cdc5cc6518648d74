"""GPU: gg_dgrad_noalloc, the input gradient for callers that cannot allocate
(dH1 in the library's static per-GPU scratch array instead of a caller
workspace), against gg_dgrad on the same inputs: two calls in a row, the
second on a smaller problem, each bit for bit equal to gg_dgrad (the same
kernels run), and sizes beyond the array refused before any launch."""
import numpy as np
import pytest
import torch

import workload
from gpu_harness import DeviceCase, log

pytestmark = pytest.mark.gpu


def _gpu_ok():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _compare(case):
    import moe_expert_grouped_ragged_amd as gg
    dc = DeviceCase(case)
    h1, a, y = dc.forward()
    ws = torch.empty(case.M, 2 * case.F, dtype=torch.bfloat16, device=dc.dev)
    dx_ref = gg.gg_dgrad(dc.dy, h1, dc.offsets, dc.packed, case.E, case.H, case.F, workspace=ws)
    dx = torch.full((case.M, case.H), float("nan"), dtype=torch.bfloat16, device=dc.dev)
    gg.gg_dgrad_noalloc(dc.dy, h1, dc.offsets, dc.packed, case.E, case.H, case.F, dx=dx)
    torch.cuda.synchronize()
    same = torch.equal(dx.view(torch.int16), dx_ref.view(torch.int16))
    log(f"[noalloc] {case.name} M={case.M} H={case.H} F={case.F}: bitwise equal to gg_dgrad: {same}")
    assert same


def test_noalloc_matches_dgrad_two_calls_second_smaller():
    _gpu_ok()
    # first the 32-expert workload (dH1 = 96 MiB of the 128 MiB array), then a
    # smaller problem: the array keeps the first call's contents, which the
    # second must not depend on
    _compare(workload.draw_case(workload.by_name("uniform_e32_h2048_f768")))
    _compare(workload.custom_case([300, 0, 257, 40, 1, 97], 256, 128, seed=71))


def test_noalloc_refuses_more_than_the_array():
    _gpu_ok()
    import moe_expert_grouped_ragged_amd as gg
    E, H, F = 2, 64, 256
    M = gg.NOALLOC_SCRATCH_BYTES // (4 * F) + 1          # dH1 one row too large
    dev = torch.device("cuda:0")
    dy = torch.zeros(M, H, dtype=torch.bfloat16, device=dev)
    h1 = torch.zeros(M, 2 * F, dtype=torch.bfloat16, device=dev)
    off = torch.tensor([0, M // 2, M], dtype=torch.int64, device=dev)
    packed = torch.zeros(gg.packed_bytes(E, H, F) // 2, dtype=torch.bfloat16, device=dev)
    dx = torch.full((M, H), 3.0, dtype=torch.bfloat16, device=dev)
    with pytest.raises(gg.GGError) as err:
        gg.gg_dgrad_noalloc(dy, h1, off, packed, E, H, F, dx=dx)
    assert err.value.status == gg.GG_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert bool((dx == 3.0).all())
