"""Batch invariance: a token row's results do not depend on the rest of the batch.

One set of token rows routed to one expert's weights is computed inside many
different batches: alone (a small expert, weight-streaming flavor), as the
head of a large expert (256-row tiles), as the streamed tail of a large
expert, shifted by row counts that are not multiples of 32 (so the rows land
in other MFMA lanes), in another expert slot, and beside other experts.  As
the streamed tail of a 2048-row expert the grid is large next to the number
of streaming items, so each item is split into two halves of 96 weight rows;
alone, the items stay whole.  Both
flavors accumulate the same MFMA k-steps in the same order into fp32
accumulators that start at zero, and share the epilogue arithmetic, so H1, A,
Y, dH1 and dX of those rows must be bitwise equal in every batch.  The same holds for the weighted QuickGeGLU path, dprobs
included: its per-row sum is taken per 32-column group in the same lane order
by both flavors, then over the groups in order."""
import numpy as np
import pytest
import torch

import workload
from gpu_harness import DeviceCase, log

pytestmark = pytest.mark.gpu


def _layouts(R):
    """name -> per-slot list of segments; a segment is ("R", n) for the rows
    under test or ("o", n) for other rows.  The rows under test always use the
    test weights; every slot not holding them uses the other weights."""
    return {
        "alone": [[("R", R)]],
        "head_of_large": [[("R", R), ("o", 300)]],
        "streamed_tail": [[("o", 256), ("R", R)]],
        "shifted_in_small": [[("o", 7), ("R", R)]],
        "shifted_in_tile": [[("o", 13), ("R", R), ("o", 300)]],
        "shifted_tail": [[("o", 259), ("R", R)]],
        "other_slot": [[("o", 100)], [], [("o", 3), ("R", R)], [("o", 70)]],
        "beside_others": [[("R", R)], [("o", 300)], [("o", 256)], [("o", 70)]],
        "tail_of_wide": [[("o", 2048), ("R", R)]],
    }


def _run(layout, R, base, weighted=False, frag=False):
    xs, dys, counts, w1s, w2s, ps = [], [], [], [], [], []
    allp = torch.from_numpy(np.random.default_rng(77).uniform(0.05, 1.0, base.x.shape[0]).astype(np.float32))
    other = 0
    where = None
    for slot in layout:
        n_slot = 0
        has_r = any(kind == "R" for kind, _ in slot)
        for kind, n in slot:
            if kind == "R":
                where = sum(counts) + n_slot
                xs.append(base.x[:R]); dys.append(base.dy[:R]); ps.append(allp[:R])
            else:
                xs.append(base.x[R + other:R + other + n]); dys.append(base.dy[R + other:R + other + n])
                ps.append(allp[R + other:R + other + n])
                other += n
            n_slot += n
        counts.append(n_slot)
        w1s.append(base.w1[0 if has_r else 1]); w2s.append(base.w2[0 if has_r else 1])
    counts = np.asarray(counts, dtype=np.int64)
    off = workload.offsets_from_counts(counts)
    x = torch.cat(xs) if xs else base.x[:0]
    dy = torch.cat(dys) if dys else base.dy[:0]
    assert x.shape[0] == off[-1] and other <= base.x.shape[0] - R
    case = workload.Case("invariance", len(counts), base.H, base.F, int(counts.sum()), counts, off,
                         torch.stack(w1s), torch.stack(w2s), x, dy)
    dc = DeviceCase(case, frag=frag)
    sl = slice(where, where + R)
    if not weighted:
        h1, a, y = dc.forward()
        dh1, dx = dc.dgrad(h1)
        torch.cuda.synchronize()
        return {"h1": h1[sl].cpu(), "a": a[sl].cpu(), "y": y[sl].cpu(), "dh1": dh1[sl].cpu(),
                "dx": dx[sl].cpu()}
    gg = dc.gg
    probs = torch.cat(ps).to(dc.dev)
    h1, a = gg.gg_forward_fc1_glu(dc.x, dc.offsets, dc.packed, dc.E, dc.H, dc.F, "qgeglu", probs, frag=dc.frag)
    y = gg.gg_forward_fc2_frag(a, dc.offsets, dc.packed, dc.frag, dc.E, dc.H, dc.F)
    ws = torch.empty(gg.dgrad_glu_workspace_bytes(dc.M, dc.F, True), dtype=torch.uint8, device=dc.dev)
    dx, dprobs = gg.gg_dgrad_glu(dc.dy, h1, dc.offsets, dc.packed, dc.E, dc.H, dc.F, "qgeglu", probs,
                                 workspace=ws, frag=dc.frag)
    torch.cuda.synchronize()
    dh1 = ws[:4 * dc.M * dc.F].view(torch.bfloat16).view(dc.M, 2 * dc.F)
    return {"h1": h1[sl].cpu(), "a": a[sl].cpu(), "y": y[sl].cpu(), "dh1": dh1[sl].cpu(),
            "dx": dx[sl].cpu(), "dprobs": dprobs[sl].cpu()}


@pytest.mark.parametrize("weighted", [False, True], ids=["swiglu", "weighted_qgeglu"])
@pytest.mark.parametrize("H,F,R", [(256, 192, 40), (136, 200, 40), (256, 192, 64), (136, 200, 96),
                                   (256, 128, 40), (256, 128, 96), (256, 256, 64)])   # the last three: also with fragment copies
def test_rows_are_batch_invariant(H, F, R, weighted):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    base = workload.custom_case([R, 2400], H, F, seed=31)
    ref = None
    import moe_expert_grouped_ragged_amd as gg
    for i, (name, layout) in enumerate(_layouts(R).items()):
        # shapes with fragment-ordered copies alternate the weight layout, so
        # the eight-wave and the four-wave kernels are compared as well
        frag = gg.has_frag(H, F) and i % 2 == 1
        log(f"[invariance] H={H} F={F} R={R} {name} frag={frag}")
        got = _run(layout, R, base, weighted, frag)
        if ref is None:
            ref = got
            continue
        for k in ref:
            same = got[k].view(torch.int32 if k == "dprobs" else torch.int16) == \
                ref[k].view(torch.int32 if k == "dprobs" else torch.int16)
            assert bool(same.all()), (name, k, int((~same).sum()))
    log(f"[invariance] H={H} F={F} R={R}: every layout bitwise equal to 'alone'")
