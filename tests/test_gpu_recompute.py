"""GPU: the input gradient without a saved H1 (gg_dgrad_recompute).

FC1 is recomputed inside the call with the same per-element K order as the
forward, so the recomputed H1 equals the saved one bit for bit, and with it
dH1, dX and dprobs.  Checked on shapes that exercise both kernel flavors,
K tails and zero-token experts, in the plain and the weighted QuickGeGLU
modes, at full workload sizes in the benchmark's launch configuration, and
end to end against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workload
from gpu_harness import log
from parity import check_chained, check

pytestmark = pytest.mark.gpu

CASES = [([5, 0, 7, 33], 64, 64), ([31, 32, 63, 64, 65, 0, 1], 136, 200), ([300, 0, 257, 40, 1], 128, 96),
         ([96, 95, 352, 0], 136, 200),
         # shapes with fragment copies (also run with them: four-wave forward tiles,
         # the recompute's H1 over W1's fragment copy, four-wave dX)
         ([300, 0, 257, 40, 1, 97], 256, 128),
         ([300, 0, 257, 40, 1, 97], 256, 256)]
MODES = [("swiglu", False), ("qgeglu", True)]


def _both(c, act, weighted, frag=False):
    import moe_expert_grouped_ragged_amd as gg
    dev = torch.device("cuda:0")
    x, dy = c.x.to(dev), c.dy.to(dev)
    off = torch.from_numpy(np.ascontiguousarray(c.offsets)).to(dev)
    packed = gg.gg_pack_weights(c.w1.to(dev), c.w2.to(dev))
    fr = gg.gg_pack_frag(packed, c.E, c.H, c.F) if frag else None
    probs = (torch.from_numpy(np.random.default_rng(3).uniform(0.05, 1, c.M).astype(np.float32)).to(dev)
             if weighted else None)
    nbytes = gg.dgrad_glu_workspace_bytes(c.M, c.F, weighted)
    # saved H1
    h1, a = gg.gg_forward_fc1_glu(x, off, packed, c.E, c.H, c.F, act, probs, frag=fr)
    ws_s = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dx_s, dp_s = gg.gg_dgrad_glu(dy, h1, off, packed, c.E, c.H, c.F, act, probs, want_dprobs=weighted,
                                 workspace=ws_s, frag=fr)
    # no saved H1
    none, a_r = gg.gg_forward_fc1_glu(x, off, packed, c.E, c.H, c.F, act, probs, save_h1=False, frag=fr)
    assert none is None
    ws_r = torch.full((nbytes,), 0x7f, dtype=torch.uint8, device=dev)
    dx_r, dp_r = gg.gg_dgrad_recompute(dy, x, off, packed, c.E, c.H, c.F, act, probs, want_dprobs=weighted,
                                       workspace=ws_r, frag=fr)
    torch.cuda.synchronize()
    n = 4 * c.M * c.F
    return dict(h1=h1, a=a, a_r=a_r, dx_s=dx_s, dx_r=dx_r, dp_s=dp_s, dp_r=dp_r,
                dh1_s=ws_s[:n], dh1_r=ws_r[:n])


def _bitwise(out, weighted, rows=None):
    sl = slice(None) if rows is None else rows
    assert torch.equal(out["a"].view(torch.int16), out["a_r"].view(torch.int16))
    assert torch.equal(out["dx_s"][sl].view(torch.int16), out["dx_r"][sl].view(torch.int16))
    assert torch.equal(out["dh1_s"], out["dh1_r"])
    if weighted:
        assert torch.equal(out["dp_s"][sl].view(torch.int32), out["dp_r"][sl].view(torch.int32))


@pytest.mark.parametrize("act,weighted", MODES)
@pytest.mark.parametrize("counts,H,F,frag", [case + (False,) for case in CASES] +
                         [case + (True,) for case in CASES if case[1] % 256 == 0 and case[2] % 128 == 0])
def test_recompute_is_bitwise_the_saved_h1_path(counts, H, F, frag, act, weighted):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = workload.custom_case(counts, H, F, seed=51)
    log(f"[recompute] {act} weighted={weighted} counts={counts} H={H} F={F} frag={frag}")
    out = _both(c, act, weighted, frag)
    _bitwise(out, weighted)
    # end to end against the oracle (dX from dY and X through the recomputed H1)
    pr = None if not weighted else out_probs(c)
    fw = oracle.forward_glu(c.x, c.offsets, c.w1, c.w2, act, pr)
    dg = oracle.dgrad_glu(c.dy, fw["h1"], c.offsets, c.w1, c.w2, act, pr)
    check_chained("dx_recompute", out["dx_r"], dg["dx"])
    if weighted:
        check("dprobs_recompute", out["dp_r"].cpu().numpy().astype(np.float64), dg["dprobs"])


def out_probs(c):
    return np.random.default_rng(3).uniform(0.05, 1, c.M).astype(np.float32)


@pytest.mark.parametrize("wl,frag", [("uniform_e32_h2048_f768", False), ("uniform_e32_h2048_f768", True),
                                     ("smallbatch_e128_h2688_f1856", False)])
def test_recompute_full_size_bitwise(wl, frag):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = workload.draw_case(workload.by_name(wl))
    log(f"[recompute] full size {wl} M={c.M} frag={frag}")
    out = _both(c, "swiglu", False, frag)
    _bitwise(out, False)
