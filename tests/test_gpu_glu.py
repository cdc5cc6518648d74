"""GPU parity of the weighted SwiGLU / QuickGeGLU entry points through the C ABI.

Every stage of gg_forward_fc1_glu + gg_forward_fc2 + gg_dgrad_glu is compared
with the oracle (forward_glu / dgrad_glu) on the same seeded inputs, including
dprobs, over shapes that exercise both flavors (streamed small experts and
tails, 256-row tiles), K tails and zero-token experts."""
import numpy as np
import pytest
import torch

import oracle
import workload
from gpu_harness import log
from parity import stagewise_glu

pytestmark = pytest.mark.gpu

CASES = [
    ([5, 0, 7, 33], 64, 64),
    ([31, 32, 63, 64, 65, 0, 1], 136, 200),
    ([300, 0, 257, 40, 1], 128, 96),
    ([0, 520, 0], 72, 264),
    ([96, 95, 352, 0], 136, 200),   # three full 32-row blocks in streaming items
    ([300, 0, 257, 40, 1, 97], 256, 128),
]


def _probs(M, seed):
    return np.random.default_rng(seed).uniform(0.02, 1.0, M).astype(np.float32)


def _run(c, act, probs_np, want_dprobs=True, frag=False):
    import moe_expert_grouped_ragged_amd as gg
    dev = torch.device("cuda:0")
    x, dy = c.x.to(dev), c.dy.to(dev)
    off = torch.from_numpy(np.ascontiguousarray(c.offsets)).to(dev)
    packed = gg.gg_pack_weights(c.w1.to(dev), c.w2.to(dev))
    fr = gg.gg_pack_frag(packed, c.E, c.H, c.F) if frag else None
    probs = None if probs_np is None else torch.from_numpy(probs_np).to(dev)
    h1, a = gg.gg_forward_fc1_glu(x, off, packed, c.E, c.H, c.F, act, probs, frag=fr)
    y = gg.gg_forward_fc2_frag(a, off, packed, fr, c.E, c.H, c.F)
    ws = torch.empty(gg.dgrad_glu_workspace_bytes(c.M, c.F, want_dprobs), dtype=torch.uint8, device=dev)
    dx, dprobs = gg.gg_dgrad_glu(dy, h1, off, packed, c.E, c.H, c.F, act, probs, want_dprobs=want_dprobs,
                                 workspace=ws, frag=fr)
    torch.cuda.synchronize()
    dh1 = ws[:4 * c.M * c.F].view(torch.bfloat16).view(c.M, 2 * c.F)
    return h1, a, y, dh1, dx, dprobs


@pytest.mark.parametrize("act", ["swiglu", "qgeglu"])
@pytest.mark.parametrize("counts,H,F,frag", [case + (False,) for case in CASES] +
                         [([300, 0, 257, 40, 1, 97], 256, 128, True),    # four-wave forward tiles and dX
                          ([300, 0, 257, 40, 1, 97], 256, 256, True)])   # and dA (F % 256 == 0)
def test_glu_stagewise_parity(act, counts, H, F, frag):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = workload.custom_case(counts, H, F, seed=41)
    probs = _probs(c.M, 7)
    log(f"[glu] act={act} counts={counts} H={H} F={F} frag={frag}")
    h1, a, y, dh1, dx, dprobs = _run(c, act, probs, frag=frag)
    infos = stagewise_glu(c.x, c.dy, c.offsets, c.w1, c.w2, act, probs, h1, a, y, dh1, dx, dprobs)
    log("  " + " ".join(f"{i['name']}:{i.get('rel_l2', 0):.1e}" for i in infos))


@pytest.mark.parametrize("act,weighted", [("qgeglu", True), ("swiglu", True), ("qgeglu", False)])
def test_fragment_buffer_gives_the_same_bits(act, weighted):
    """With F % 256 == 0 the four-wave kernel also runs dA with the
    activation options (slope, row probabilities, dp partial sums); every
    output, dprobs included, equals the run without the fragment buffer (the
    eight-wave kernel) bit for bit: thin items, partial and full tiles."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = workload.custom_case([300, 0, 257, 40, 1, 97, 512], 256, 256, seed=47)
    probs = _probs(c.M, 9) if weighted else None
    log(f"[glu] fragment buffer vs packed act={act} weighted={weighted}")
    ref = _run(c, act, probs, frag=False)
    got = _run(c, act, probs, frag=True)
    for name, g, r in zip(("h1", "a", "y", "dh1", "dx"), got[:5], ref[:5]):
        assert torch.equal(g.view(torch.int16), r.view(torch.int16)), name
    assert torch.equal(got[5], ref[5]), "dprobs"


def test_unit_probs_and_no_probs_are_bitwise_the_plain_path():
    """p = 1 multiplies exactly; SwiGLU with p = 1 or without p equals the
    plain entry points bit for bit, and dprobs is still produced."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_grouped_ragged_amd as gg
    c = workload.custom_case([31, 0, 300, 7], 136, 200, seed=43)
    dev = torch.device("cuda:0")
    x, dy = c.x.to(dev), c.dy.to(dev)
    off = torch.from_numpy(np.ascontiguousarray(c.offsets)).to(dev)
    packed = gg.gg_pack_weights(c.w1.to(dev), c.w2.to(dev))
    h1_ref, a_ref = gg.gg_forward_fc1_swiglu(x, off, packed, c.E, c.H, c.F)
    ws_ref = torch.empty(c.M, 2 * c.F, dtype=torch.bfloat16, device=dev)
    dx_ref = gg.gg_dgrad(dy, h1_ref, off, packed, c.E, c.H, c.F, workspace=ws_ref)
    for probs in (None, torch.ones(c.M, dtype=torch.float32, device=dev)):
        h1, a = gg.gg_forward_fc1_glu(x, off, packed, c.E, c.H, c.F, "swiglu", probs)
        ws = torch.empty(gg.dgrad_glu_workspace_bytes(c.M, c.F, True), dtype=torch.uint8, device=dev)
        dx, dprobs = gg.gg_dgrad_glu(dy, h1, off, packed, c.E, c.H, c.F, "swiglu", probs, workspace=ws)
        torch.cuda.synchronize()
        dh1 = ws[:4 * c.M * c.F].view(torch.bfloat16).view(c.M, 2 * c.F)
        for got, ref in ((h1, h1_ref), (a, a_ref), (dh1, ws_ref), (dx, dx_ref)):
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
        assert torch.isfinite(dprobs).all()


def test_dprobs_rows_outside_offsets_untouched_and_empty_batch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_grouped_ragged_amd as gg
    c = workload.custom_case([9, 0, 40], 64, 64, seed=44)
    dev = torch.device("cuda:0")
    pad = 13
    x = torch.cat([c.x, torch.ones(pad, c.H, dtype=torch.bfloat16)]).to(dev)
    dy = torch.cat([c.dy, torch.ones(pad, c.H, dtype=torch.bfloat16)]).to(dev)
    M = c.M + pad
    off = torch.from_numpy(np.ascontiguousarray(c.offsets)).to(dev)
    packed = gg.gg_pack_weights(c.w1.to(dev), c.w2.to(dev))
    probs = torch.from_numpy(_probs(M, 9)).to(dev)
    h1, a = gg.gg_forward_fc1_glu(x, off, packed, c.E, c.H, c.F, "qgeglu", probs)
    canary = torch.full((M,), 12345.0, dtype=torch.float32, device=dev)
    dx, dprobs = gg.gg_dgrad_glu(dy, h1, off, packed, c.E, c.H, c.F, "qgeglu", probs, dprobs=canary)
    torch.cuda.synchronize()
    assert (dprobs[c.M:] == 12345.0).all() and (dprobs[:c.M] != 12345.0).all()
    # empty batch: nothing launched, nothing written
    e = torch.empty(0, c.H, dtype=torch.bfloat16, device=dev)
    zero_off = torch.zeros(c.E + 1, dtype=torch.int64, device=dev)
    h1e, ae = gg.gg_forward_fc1_glu(e, zero_off, packed, c.E, c.H, c.F, "qgeglu",
                                    torch.empty(0, dtype=torch.float32, device=dev))
    assert ae.shape == (0, c.F)


@pytest.mark.parametrize("wl", ["zipf_e128_h2048_f768", "smallbatch_e128_h2688_f1856"])
def test_glu_workload_sampled_rows(wl):
    """Full-size workloads in the benchmark's launch configuration; the oracle
    checks a sample of rows from both flavors (every row depends only on its
    own inputs and its expert's weights).  Where the shape has fragment
    copies, the run with them (four-wave tiles for all four GEMMs, dA with
    the slope, the row weights and dp) equals the run without them bit for
    bit over every output, dprobs included."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_grouped_ragged_amd as gg
    c = workload.draw_case(workload.by_name(wl))
    probs = _probs(c.M, 11)
    log(f"[glu] workload {wl} M={c.M}")
    h1, a, y, dh1, dx, dprobs = _run(c, "qgeglu", probs)
    if gg.has_frag(c.H, c.F):
        got = _run(c, "qgeglu", probs, frag=True)
        for name, g, r in zip(("h1", "a", "y", "dh1", "dx", "dprobs"), got, (h1, a, y, dh1, dx, dprobs)):
            assert torch.equal(g.view(torch.int32) if g.dtype == torch.float32 else g.view(torch.int16),
                               r.view(torch.int32) if r.dtype == torch.float32 else r.view(torch.int16)), name
        log(f"[glu] workload {wl}: with fragment copies, bitwise equal")
        del got
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.choice(c.M, 96, replace=False),
                                     c.offsets[1:-1][np.diff(c.offsets)[1:] > 0][:16]]))
    rows = rows[rows < c.offsets[-1]]
    expert, compact = oracle.sample_rows(c.offsets, rows)
    sel = torch.from_numpy(rows)
    infos = stagewise_glu(c.x[sel], c.dy[sel], compact, c.w1, c.w2, "qgeglu", probs[rows],
                          h1[sel.to(h1.device)], a[sel.to(a.device)], y[sel.to(y.device)],
                          dh1[sel.to(dh1.device)], dx[sel.to(dx.device)], dprobs[sel.to(dprobs.device)])
    log("  " + " ".join(f"{i['name']}:{i.get('rel_l2', 0):.1e}" for i in infos))
