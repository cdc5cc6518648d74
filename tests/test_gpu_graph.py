"""HIP-graph capture of one forward + dgrad step, replayed with changing
expert offsets (same M, different splits).  Every replay is compared
bitwise with an eager run on the same offsets, with eager work and
synchronization between the replays.  The kernels read the offsets on the
device, so a captured step follows the new split without re-capture."""
import numpy as np
import pytest
import torch

import workload
from gpu_harness import DeviceCase, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("H,F,frag", [(128, 96, False), (256, 128, True)])
def test_graph_replays_follow_new_offsets(H, F, frag):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_grouped_ragged_amd as gg
    counts0 = [300, 0, 70, 20, 0, 513, 33, 1]
    case = workload.custom_case(counts0, H, F, seed=21)
    E, H, F, M = case.E, case.H, case.F, case.M
    dc = DeviceCase(case, frag=frag)
    dev = dc.dev
    off_dev = dc.offsets.clone()
    bufs = {"h1": torch.empty(M, 2 * F, dtype=torch.bfloat16, device=dev),
            "a": torch.empty(M, F, dtype=torch.bfloat16, device=dev),
            "y": torch.empty(M, H, dtype=torch.bfloat16, device=dev),
            "ws": torch.empty(M, 2 * F, dtype=torch.bfloat16, device=dev),
            "dx": torch.empty(M, H, dtype=torch.bfloat16, device=dev)}

    def step(off, b):
        gg.gg_forward_fc1_glu(dc.x, off, dc.packed, E, H, F, h1_out=b["h1"], a_out=b["a"], frag=dc.frag)
        gg.gg_forward_fc2_frag(b["a"], off, dc.packed, dc.frag, E, H, F, y=b["y"])
        gg.gg_dgrad_glu(dc.dy, b["h1"], off, dc.packed, E, H, F, want_dprobs=False, workspace=b["ws"],
                        dx=b["dx"], frag=dc.frag)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(off_dev, bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(off_dev, bufs)
    torch.cuda.synchronize()

    rng = np.random.default_rng(5)
    splits = [counts0, counts0[::-1], [M, 0, 0, 0, 0, 0, 0, 0], [0] * 7 + [M],
              list(rng.multinomial(M, np.ones(E) / E))]
    for i, counts in enumerate(splits):
        off = torch.from_numpy(workload.offsets_from_counts(np.asarray(counts))).to(dev)
        off_dev.copy_(off)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in bufs.items()}
        ref = {k: torch.full_like(v, 7.0) for k, v in bufs.items()}
        step(off, ref)                      # eager, fresh buffers
        torch.cuda.synchronize()
        for k in bufs:
            assert torch.equal(got[k].view(torch.int16), ref[k].view(torch.int16)), (i, counts, k)
        log(f"[graph] replay {i} counts {counts} matches eager")


def test_graph_replays_weighted_recompute_step():
    """The same with the weighted QuickGeGLU forward (no saved H1) and the
    recompute input gradient with dprobs: four kernels plus the dp reduction,
    all reading the offsets on the device."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_expert_grouped_ragged_amd as gg
    counts0 = [300, 0, 70, 20, 0, 513, 33, 1]
    case = workload.custom_case(counts0, 128, 96, seed=22)
    E, H, F, M = case.E, case.H, case.F, case.M
    dc = DeviceCase(case)
    dev = dc.dev
    off_dev = dc.offsets.clone()
    probs = torch.from_numpy(np.random.default_rng(6).uniform(0.05, 1, M).astype(np.float32)).to(dev)
    nws = gg.dgrad_glu_workspace_bytes(M, F, True)

    def bufs_like(fill):
        return {"a": torch.full((M, F), fill, dtype=torch.bfloat16, device=dev),
                "y": torch.full((M, H), fill, dtype=torch.bfloat16, device=dev),
                "ws": torch.zeros(nws, dtype=torch.uint8, device=dev),
                "dx": torch.full((M, H), fill, dtype=torch.bfloat16, device=dev),
                "dp": torch.full((M,), fill, dtype=torch.float32, device=dev)}

    def step(off, b):
        gg.gg_forward_fc1_glu(dc.x, off, dc.packed, E, H, F, "qgeglu", probs, save_h1=False, a_out=b["a"])
        gg.gg_forward_fc2(b["a"], off, dc.packed, E, H, F, y=b["y"])
        gg.gg_dgrad_recompute(dc.dy, dc.x, off, dc.packed, E, H, F, "qgeglu", probs, workspace=b["ws"],
                              dx=b["dx"], dprobs=b["dp"])

    bufs = bufs_like(0.0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(off_dev, bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(off_dev, bufs)
    torch.cuda.synchronize()
    n_dh1 = 4 * M * F
    for i, counts in enumerate([counts0, counts0[::-1], [0] * 7 + [M]]):
        off = torch.from_numpy(workload.offsets_from_counts(np.asarray(counts))).to(dev)
        off_dev.copy_(off)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in bufs.items()}
        ref = bufs_like(7.0)
        step(off, ref)
        torch.cuda.synchronize()
        for k in ("a", "y", "dx"):
            assert torch.equal(got[k].view(torch.int16), ref[k].view(torch.int16)), (i, counts, k)
        assert torch.equal(got["dp"].view(torch.int32), ref["dp"].view(torch.int32)), (i, counts, "dp")
        assert torch.equal(got["ws"][:n_dh1], ref["ws"][:n_dh1]), (i, counts, "dh1")
        log(f"[graph] weighted recompute replay {i} counts {counts} matches eager")
