"""GPU parity of the router-probability-on-input calls through the C ABI
(gg_scale_rows, gg_scale_rows_backward) against the oracle's scale_rows and
scale_rows_backward: x' and dx bit for bit, dprobs within the fp32
summation bound; in-place use; a row count past the kernels' first pass over
the grid; and the whole probability-on-input path (the scale, the plain
forward and input gradient on the scaled rows, the scale's gradient) stage
by stage and through autograd."""
import numpy as np
import pytest
import torch

import oracle
import workload
from gpu_harness import log
from parity import stagewise, summary

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def _gpu_f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def _rows(M, H, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, H, generator=g).to(torch.bfloat16)
    rng = np.random.default_rng(seed)
    p = rng.uniform(0.0, 1.0, M).astype(np.float32)
    special = [0.0, 1.0, 0.5, 2.0 ** -20, 0.1, 1.0 - 2.0 ** -24]
    p[:min(M, len(special))] = special[:M]
    return x, p


def _dp_bound(g: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Two fp32 sums of the same exact products in different orders differ by
    at most 2 (H - 1) 2^-24 sum|g x|."""
    H = g.shape[1]
    return 2.0 * H * 2.0 ** -24 * np.sum(np.abs(g.astype(np.float64) * x.astype(np.float64)), axis=1) + 1e-38


@pytest.mark.parametrize("M,H", [(1, 8), (5, 64), (37, 136), (300, 2048), (1031, 4096)])
def test_scale_rows_matches_oracle(M, H):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_grouped_ragged_amd as gg
    log(f"[rows] scale M={M} H={H}")
    x, p = _rows(M, H, seed=M + H)
    g = torch.Generator().manual_seed(7 * M + H)
    dxs = torch.randn(M, H, generator=g).to(torch.bfloat16)
    xd, pd, gd = x.to(DEV), torch.from_numpy(p).to(DEV), dxs.to(DEV)
    xs = gg.gg_scale_rows(xd, pd)
    dx, dp = gg.gg_scale_rows_backward(gd, xd, pd)
    torch.cuda.synchronize()
    ref = oracle.scale_rows(x, p)
    assert np.array_equal(_bits(_gpu_f32(xs)), _bits(ref))
    rb = oracle.scale_rows_backward(dxs, x, p)
    assert np.array_equal(_bits(_gpu_f32(dx)), _bits(rb["dx"]))
    dpg = dp.cpu().numpy()
    xf, gf = x.float().numpy(), dxs.float().numpy()
    bound = _dp_bound(gf, xf)
    assert np.all(np.abs(dpg.astype(np.float64) - rb["dprobs"]) <= bound)
    exact = np.sum(gf.astype(np.float64) * xf.astype(np.float64), axis=1)
    assert np.all(np.abs(dpg - exact) <= bound / 2)
    log(f"[rows] dprobs worst / bound = {np.max(np.abs(dpg - rb['dprobs']) / bound):.3f}")


def test_scale_rows_in_place_and_without_dprobs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_grouped_ragged_amd as gg
    M, H = 129, 264
    x, p = _rows(M, H, seed=5)
    g = torch.Generator().manual_seed(6)
    dxs = torch.randn(M, H, generator=g).to(torch.bfloat16)
    pd = torch.from_numpy(p).to(DEV)
    xd = x.to(DEV)
    out = gg.gg_scale_rows(xd, pd, out=xd)
    gd = dxs.to(DEV)
    xd2 = x.to(DEV)
    dx, dp = gg.gg_scale_rows_backward(gd, xd2, pd, want_dprobs=False, dx=gd)
    torch.cuda.synchronize()
    assert out.data_ptr() == xd.data_ptr() and dx.data_ptr() == gd.data_ptr() and dp is None
    assert np.array_equal(_bits(_gpu_f32(out)), _bits(oracle.scale_rows(x, p)))
    assert np.array_equal(_bits(_gpu_f32(dx)), _bits(oracle.scale_rows_backward(dxs, x, p)["dx"]))


def test_scale_rows_past_one_grid_pass():
    """More rows than one pass of the grid (65536 workgroups x 4 rows), so
    the row loop strides; every row is compared."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_grouped_ragged_amd as gg
    M, H = 65536 * 4 + 4099, 64
    log(f"[rows] grid stride M={M} H={H}")
    x, p = _rows(M, H, seed=9)
    g = torch.Generator().manual_seed(10)
    dxs = torch.randn(M, H, generator=g).to(torch.bfloat16)
    xd, pd, gd = x.to(DEV), torch.from_numpy(p).to(DEV), dxs.to(DEV)
    xs = gg.gg_scale_rows(xd, pd)
    dx, dp = gg.gg_scale_rows_backward(gd, xd, pd)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(_gpu_f32(xs)), _bits(oracle.scale_rows(x, p)))
    rb = oracle.scale_rows_backward(dxs, x, p)
    assert np.array_equal(_bits(_gpu_f32(dx)), _bits(rb["dx"]))
    assert np.all(np.abs(dp.cpu().numpy().astype(np.float64) - rb["dprobs"]) <=
                  _dp_bound(dxs.float().numpy(), x.float().numpy()))


@pytest.mark.parametrize("counts,H,F", [([40, 0, 300, 7], 256, 128), ([5, 96, 0, 257, 33], 136, 200)])
def test_probs_on_input_path_stagewise(counts, H, F):
    """x' = scale(x, p), the plain forward and input gradient on x', then the
    scale's gradient: every stage against the oracle on the GPU's own input
    of that stage; and the autograd composition ScaleRows -> FrozenExpertMLP
    gives the same bits as the explicit calls."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_grouped_ragged_amd as gg
    c = workload.custom_case(counts, H, F, seed=23)
    log(f"[rows] probs on input counts={counts} H={H} F={F}")
    p = np.random.default_rng(3).uniform(0.02, 1.0, c.M).astype(np.float32)
    dev = torch.device(DEV)
    off = torch.from_numpy(np.ascontiguousarray(c.offsets)).to(dev)
    packed = gg.gg_pack_weights(c.w1.to(dev), c.w2.to(dev))
    x, dy, pd = c.x.to(dev), c.dy.to(dev), torch.from_numpy(p).to(dev)
    xs = gg.gg_scale_rows(x, pd)
    h1, a = gg.gg_forward_fc1_swiglu(xs, off, packed, c.E, c.H, c.F)
    y = gg.gg_forward_fc2(a, off, packed, c.E, c.H, c.F)
    ws = torch.empty(c.M, 2 * c.F, dtype=torch.bfloat16, device=dev)
    dxs = gg.gg_dgrad(dy, h1, off, packed, c.E, c.H, c.F, workspace=ws)
    dx, dp = gg.gg_scale_rows_backward(dxs, x, pd)
    torch.cuda.synchronize()
    xs_cpu = xs.cpu()
    assert np.array_equal(_bits(xs_cpu.float().numpy()), _bits(oracle.scale_rows(c.x, p)))
    infos = stagewise(xs_cpu, c.dy, c.offsets, c.w1, c.w2, h1, a, y, ws, dxs)
    log("[rows] " + summary(infos))
    rb = oracle.scale_rows_backward(dxs.cpu(), c.x, p)
    assert np.array_equal(_bits(_gpu_f32(dx)), _bits(rb["dx"]))
    assert np.all(np.abs(dp.cpu().numpy().astype(np.float64) - rb["dprobs"]) <=
                  _dp_bound(dxs.float().cpu().numpy(), c.x.float().numpy()))
    # the same path through autograd
    xa = c.x.to(dev).requires_grad_(True)
    pa = pd.clone().requires_grad_(True)
    ya = gg.FrozenExpertMLP.apply(gg.ScaleRows.apply(xa, pa), off, packed, c.E, c.H, c.F)
    ya.backward(dy)
    torch.cuda.synchronize()
    assert torch.equal(ya.detach().view(torch.int16), y.view(torch.int16))
    assert torch.equal(xa.grad.view(torch.int16), dx.view(torch.int16))
    assert torch.equal(pa.grad, dp)
