"""GPU parity of the HIP path against the CPU oracle (MI355X only).

Same seeded inputs on both sides; forward (H1, A, Y) and input gradient
(dH1, dX) compared element by element at the tolerance in parity.py.  Shapes
with fragment-ordered copies run both weight layouts (the packed buffer
alone, and with the opt-in fragment buffer), which must agree bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workload
from gpu_harness import DeviceCase, bitwise_equal, layouts, log
from parity import DH1_ELEM_REL, check, check_chained, stagewise, summary

pytestmark = pytest.mark.gpu


def _gpu_ok():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_layouts(case, canary: bool = True):
    """Forward + dgrad in every layout the shape has; outputs pre-filled with
    NaN canaries (an element a kernel never writes stays NaN and fails the
    parity checks); the layouts must agree bit for bit.  Returns the first
    layout's DeviceCase and outputs (h1, a, y, dH1, dx)."""
    first = None
    for frag in layouts(case.H, case.F):
        log(f"[run] {case.name} E={case.E} H={case.H} F={case.F} M={case.M} frag={frag}")
        dc = DeviceCase(case, frag=frag)
        M, F, H = case.M, case.F, case.H
        nan = float("nan")
        fill = (lambda *shape: torch.full(shape, nan, dtype=torch.bfloat16, device=dc.dev)) if canary else \
            (lambda *shape: torch.empty(*shape, dtype=torch.bfloat16, device=dc.dev))
        h1, a, y = dc.forward(h1_out=fill(M, 2 * F), a_out=fill(M, F), y=fill(M, H))
        ws, dx = dc.dgrad(h1, workspace=fill(M, 2 * F), dx=fill(M, H))
        torch.cuda.synchronize()
        outs = (h1, a, y, ws, dx)
        if first is None:
            first = (dc, outs)
        else:
            for name, p, q in zip(("h1", "a", "y", "dh1", "dx"), first[1], outs):
                assert bitwise_equal(p, q), f"{case.name}: {name} differs between the weight layouts"
            log(f"[run] {case.name}: both weight layouts bitwise equal")
            del dc
    return first


def run_full_parity(case):
    """Whole-problem parity (every element), stage by stage, in every layout."""
    _gpu_ok()
    log(f"[parity] {case.name} E={case.E} H={case.H} F={case.F} M={case.M} counts={list(case.counts)[:16]}")
    dc, (h1, a, y, ws, dx) = run_layouts(case)
    rows = np.arange(int(case.offsets[0]), int(case.offsets[-1]))
    out = stagewise(case.x, case.dy, case.offsets, case.w1, case.w2, h1, a, y, ws, dx, rows)
    # dgrad from the oracle's H1 as well (same saved activation on both sides)
    ref = oracle.forward(case.x, case.offsets, case.w1, case.w2)
    h1_ref = torch.from_numpy(ref["h1"]).to(torch.bfloat16).to(dc.dev)
    ws_o, dx_o = dc.dgrad(h1_ref)
    torch.cuda.synchronize()
    dref = oracle.dgrad(case.dy, ref["h1"], case.offsets, case.w1, case.w2)
    out += [check("dh1_from_oracle_h1", ws_o, dref["dh1"], rows, elem_rel=DH1_ELEM_REL),
            check_chained("dx_from_oracle_h1", dx_o, dref["dx"], rows)]
    log(f"[parity] {case.name} ok: " + summary(out))
    return dc, (h1, a, y, dx)


def test_device_bf16_rounding_exhaustive():
    """The epilogue's fp32->bf16 conversion over all 2^32 fp32 patterns,
    against torch's device conversion (round to nearest even), plus a CPU
    check of a random subset against the oracle's rounding routine."""
    _gpu_ok()
    import moe_expert_grouped_ragged_amd as gg
    chunk = 1 << 28
    bad = 0
    for base in range(0, 1 << 32, chunk):
        bits = torch.arange(base, base + chunk, dtype=torch.int64, device="cuda").to(torch.int32)
        f = bits.view(torch.float32)
        got = gg.gg_round_bf16(f).view(torch.int16)
        want = f.to(torch.bfloat16).view(torch.int16)
        nan = torch.isnan(f)
        got_nan = torch.isnan(got.view(torch.bfloat16))
        mism = (got != want) & ~nan
        bad += int(mism.sum()) + int((nan & ~got_nan).sum())
    assert bad == 0
    rng = np.random.default_rng(0)
    sample = rng.integers(0, 1 << 32, 1 << 22, dtype=np.uint64).astype(np.uint32)
    fs = sample.view(np.float32)
    keep = np.isfinite(fs)
    fs = fs[keep]
    got = gg.gg_round_bf16(torch.from_numpy(fs.copy()).cuda()).cpu().view(torch.int16).numpy().view(np.uint16)
    want = oracle.f32_to_bf16_bits_exact(oracle.round_bf16(fs))
    np.testing.assert_array_equal(got, want)


def test_tiny_workload():
    run_full_parity(workload.draw_case(workload.by_name("tiny_e4_h64_f128")))


@pytest.mark.parametrize("counts,H,F", [
    ([1], 64, 64),
    ([17, 0, 255, 256, 257], 128, 96),
    ([0, 15, 16, 0, 33, 300, 0], 200, 136),
    ([513, 0, 0], 72, 264),
    ([0, 0, 40], 64, 8),
    ([300, 1, 0, 2, 130], 1024, 256),
    # one K stage (H = 64) with one- and two-block streaming items: the
    # accumulators are read right after the last MFMA
    ([5, 0, 7, 33], 64, 64),
    # one, two and three 32-row token blocks in streaming items, K tails
    ([31, 32, 63, 64, 65, 0, 1], 136, 200),
    # around the streaming threshold of 96 rows, for small experts and for the
    # rows a large expert leaves after its 256-row tiles (1 K stage, one block)
    ([96, 97, 352, 353, 0, 351, 95], 72, 136),
    ([95, 96, 97, 0, 609], 64, 64),
    # the maximum expert count: mostly 0..5 rows, one large expert in the middle
    ([300 if i == 500 else (i * 7919) % 6 for i in range(1024)], 64, 64),
    # four-wave forward tiles (H % 256 == 0, F % 128 == 0): full and partial
    # tiles, streamed tails on both sides of 96 rows, one- and two-iteration K
    # loops; its few thin items fit the grid twice over, so each runs as two
    # column halves
    ([17, 0, 255, 256, 257, 600, 97, 96], 256, 128),
    ([300, 1, 0, 2, 130, 513], 512, 256),
    ([0, 700, 129, 0, 256], 256, 512),
    ([130, 0, 513, 40], 256, 1024),   # FC2 on four-wave tiles from F = 1024
    # 279 small experts and 17 of 512 rows: taking the small ones as partial
    # tiles would add a round, so they stay streaming items beside the tiles
    # (four-wave: 279 thin items, more than half the grid, run whole)
    ([512 if i % 18 == 0 else 40 for i in range(296)], 256, 128),
    # the maximum expert count with fragment copies: the four-wave tiles find
    # their expert among 1024 beside the streaming launch
    ([300 if i == 500 else (i * 7919) % 6 for i in range(1024)], 256, 128),
    # only thin items in the four-wave kernel: small experts at a shape with
    # fragment copies (40 thin items on a grid of 92: column halves)
    ([24, 0, 19, 31, 27, 22, 0, 25, 30, 18, 26, 21, 0, 29, 23, 17, 28, 24, 20, 33, 96, 1], 512, 256),
    # many small experts, as in the small-batch workload
    ([24, 0, 19, 31, 27, 22, 0, 25, 30, 18, 26, 21, 0, 29, 23, 17, 28, 24, 20, 33,
      0, 26, 22, 19, 27, 25, 31, 16, 24, 0, 21, 28, 23, 26, 18, 29, 22, 25, 20, 24], 264, 328),
])
def test_shape_sweep(counts, H, F):
    run_full_parity(workload.custom_case(counts, H, F, seed=sum(counts) + H + F))


def test_padded_segments_zero_rows():
    case = workload.custom_case([100, 3, 0, 260], 256, 128, seed=7, pad_to=256)
    dc, (h1, a, y, dx) = run_full_parity(case)
    for e in range(case.E):
        pad = slice(int(case.offsets[e] + case.counts[e]), int(case.offsets[e + 1]))
        for t in (h1, a, y, dx):
            assert int((t[pad].float() != 0).sum()) == 0


def test_zero_experts_everywhere_and_canaries():
    """Empty experts at first, middle and last position; rows outside
    [offsets[0], offsets[E]) are canaries that must stay untouched; weights of
    empty experts are NaN and must not leak."""
    _gpu_ok()
    case = workload.custom_case([0, 37, 0, 0, 90, 0], 128, 64, seed=11)
    M = case.M
    lead, tail = 5, 7
    x = torch.cat([torch.ones(lead, case.H, dtype=torch.bfloat16), case.x,
                   torch.ones(tail, case.H, dtype=torch.bfloat16)])
    dy = torch.cat([torch.ones(lead, case.H, dtype=torch.bfloat16), case.dy,
                    torch.ones(tail, case.H, dtype=torch.bfloat16)])
    w1 = case.w1.clone()
    w2 = case.w2.clone()
    for e in (0, 2, 3, 5):
        w1[e] = float("nan")
        w2[e] = float("nan")
    big = workload.Case(case.name, case.E, case.H, case.F, case.T, case.counts, case.offsets + lead,
                        w1, w2, x, dy)
    dc = DeviceCase(big)
    canary = -7.0
    h1 = torch.full((M + lead + tail, 2 * case.F), canary, dtype=torch.bfloat16, device="cuda")
    a = torch.full((M + lead + tail, case.F), canary, dtype=torch.bfloat16, device="cuda")
    y = torch.full((M + lead + tail, case.H), canary, dtype=torch.bfloat16, device="cuda")
    dc.forward(h1_out=h1, a_out=a, y=y)
    ws = torch.full((M + lead + tail, 2 * case.F), canary, dtype=torch.bfloat16, device="cuda")
    dx = torch.full((M + lead + tail, case.H), canary, dtype=torch.bfloat16, device="cuda")
    dc.dgrad(h1, workspace=ws, dx=dx)
    torch.cuda.synchronize()
    for t in (h1, a, y, ws, dx):
        assert bool((t[:lead] == canary).all()) and bool((t[lead + M:] == canary).all())
        assert bool(torch.isfinite(t[lead:lead + M].float()).all())
    ref = oracle.forward(case.x, case.offsets, case.w1, case.w2)
    check("y", y[lead:lead + M], ref["y"])
    dref = oracle.dgrad(case.dy, h1[lead:lead + M].cpu(), case.offsets, case.w1, case.w2)
    check("dx", dx[lead:lead + M], dref["dx"])


def test_all_experts_empty_and_empty_batch():
    _gpu_ok()
    import moe_expert_grouped_ragged_amd as gg
    E, H, F, M = 4, 64, 64, 32
    off = torch.zeros(E + 1, dtype=torch.int64, device="cuda")
    packed = torch.zeros(3 * E * F * H, dtype=torch.bfloat16, device="cuda")
    x = torch.randn(M, H, device="cuda").to(torch.bfloat16)
    a = torch.full((M, F), 3.0, dtype=torch.bfloat16, device="cuda")
    h1 = torch.full((M, 2 * F), 3.0, dtype=torch.bfloat16, device="cuda")
    gg.gg_forward_fc1_swiglu(x, off, packed, E, H, F, h1_out=h1, a_out=a)
    y = torch.full((M, H), 3.0, dtype=torch.bfloat16, device="cuda")
    gg.gg_forward_fc2(a, off, packed, E, H, F, y=y)
    torch.cuda.synchronize()
    assert bool((a == 3.0).all()) and bool((h1 == 3.0).all()) and bool((y == 3.0).all())
    # M = 0: success, nothing launched
    x0 = torch.empty(0, H, dtype=torch.bfloat16, device="cuda")
    h, a0 = gg.gg_forward_fc1_swiglu(x0, off, packed, E, H, F)
    assert a0.shape == (0, F)


@pytest.mark.parametrize("H,F,frag", [(256, 192, False), (256, 128, False), (256, 128, True)])
def test_determinism_and_grouped_equals_per_expert(H, F, frag):
    """Two runs are bitwise equal; a grouped call equals per-expert calls
    (E = 1 views of the packed buffer, and of the fragment buffer) bitwise."""
    _gpu_ok()
    import moe_expert_grouped_ragged_amd as gg
    case = workload.custom_case([70, 0, 300, 5], H, F, seed=13)
    dc = DeviceCase(case, frag=frag)
    h1, a, y = dc.forward()
    ws, dx = dc.dgrad(h1)
    h1b, ab, yb = dc.forward()
    wsb, dxb = dc.dgrad(h1b)
    torch.cuda.synchronize()
    for p, q in ((h1, h1b), (a, ab), (y, yb), (ws, wsb), (dx, dxb)):
        assert torch.equal(p.view(torch.int16), q.view(torch.int16))
    per = gg.packed_bytes(1, case.H, case.F) // 2     # one expert block is an E = 1 packed buffer
    fper = gg.frag_bytes(1, case.H, case.F) // 2      # and one fragment block an E = 1 fragment buffer
    for e in range(case.E):
        s, t = int(case.offsets[e]), int(case.offsets[e + 1])
        if s == t:
            continue
        pk = dc.packed[e * per:(e + 1) * per]
        fr = dc.frag[e * fper:(e + 1) * fper] if frag else None
        off1 = torch.tensor([0, t - s], dtype=torch.int64, device="cuda")
        h1e, ae = gg.gg_forward_fc1_glu(dc.x[s:t].contiguous(), off1, pk, 1, case.H, case.F, frag=fr)
        ye = gg.gg_forward_fc2_frag(ae, off1, pk, fr, 1, case.H, case.F)
        dxe, _ = gg.gg_dgrad_glu(dc.dy[s:t].contiguous(), h1e, off1, pk, 1, case.H, case.F, want_dprobs=False,
                                 frag=fr)
        torch.cuda.synchronize()
        assert torch.equal(ye.view(torch.int16), y[s:t].view(torch.int16))
        assert torch.equal(dxe.view(torch.int16), dx[s:t].view(torch.int16))


@pytest.mark.parametrize("H,F,counts,frag", [(64, 64, [20, 30, 40], False),
                                              (256, 128, [120, 300, 40], False),
                                              # the fragment copies are re-derived after re-packing
                                              (256, 128, [120, 300, 40], True)])
def test_repack_after_middle_expert_replaced(H, F, counts, frag):
    _gpu_ok()
    import moe_expert_grouped_ragged_amd as gg
    case = workload.custom_case(counts, H, F, seed=17)
    dc = DeviceCase(case, frag=frag)
    w1v, w2v = gg.expert_views(dc.packed, case.E, case.H, case.F)
    # views into the packed buffer re-pack as a no-op
    gg.gg_pack_weights(w1v, w2v, packed=dc.packed)
    y0 = dc.forward()[2].clone()
    new_w1 = workload.custom_case([1], H, F, seed=99).w1[0].cuda()
    w1v = list(w1v)
    w1v[1] = new_w1                       # the middle expert is replaced by a new tensor
    gg.gg_pack_weights(w1v, w2v, packed=dc.packed)
    if frag:
        gg.gg_pack_frag(dc.packed, case.E, case.H, case.F, frag=dc.frag)
    y1 = dc.forward()[2]
    torch.cuda.synchronize()
    s1, t1 = int(case.offsets[1]), int(case.offsets[2])
    assert torch.equal(y1[:s1], y0[:s1]) and torch.equal(y1[t1:], y0[t1:])
    w1 = case.w1.clone()
    w1[1] = new_w1.cpu()
    ref = oracle.forward(case.x, case.offsets, w1, case.w2)
    check("y_repacked", y1, ref["y"])


def _tile_rows(case, n_random=512, seed=0):
    """Rows that touch every 256-row tile of every expert: the first and the
    last row of each tile, the first and last row of each expert and of its
    real (unpadded) rows, one padding row, and random rows."""
    rng = np.random.default_rng(seed)
    off = case.offsets
    rows = set()
    for e in range(case.E):
        s, t = int(off[e]), int(off[e + 1])
        if s == t:
            continue
        for r0 in range(s, t, 256):
            rows |= {r0, min(r0 + 255, t - 1)}
        real_end = s + int(case.counts[e])
        rows |= {s, t - 1, max(s, real_end - 1)}
        if real_end < t:
            rows.add(real_end)
    rows |= set(int(v) for v in rng.integers(int(off[0]), int(off[-1]), n_random))
    return np.array(sorted(rows), dtype=np.int64)


def _full_size_run(name, whole: bool):
    _gpu_ok()
    w = workload.by_name(name)
    log(f"[full] drawing {name}")
    case = workload.draw_case(w)
    log(f"[full] {name} M={case.M}; running the GPU in every layout")
    dc, (h1, a, y, ws, dx) = run_layouts(case, canary=True)
    if whole:
        rows = np.arange(int(case.offsets[0]), int(case.offsets[-1]))
        log(f"[full] {name}: oracle on every one of the {rows.size} rows")
        out = stagewise(case.x, case.dy, case.offsets, case.w1, case.w2, h1, a, y, ws, dx, rows)
    else:
        rows = _tile_rows(case)
        log(f"[full] {name}: oracle on {rows.size} rows (both ends of every 256-row tile of every expert)")
        _, compact = oracle.sample_rows(case.offsets, rows)
        rt = torch.from_numpy(rows)
        rd = rt.to(dc.dev)
        out = stagewise(case.x[rt], case.dy[rt], compact, case.w1, case.w2,
                        h1[rd], a[rd], y[rd], ws[rd], dx[rd])
    log(f"[full] {name} ok: " + summary(out))
    # padding rows (if any) are exact zeros everywhere
    for e in range(case.E):
        pad = slice(int(case.offsets[e] + case.counts[e]), int(case.offsets[e + 1]))
        if pad.stop > pad.start:
            for t in (h1, a, y, ws, dx):
                assert int((t[pad].float() != 0).sum()) == 0
    log(f"[full] {name} ok")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["uniform_e32_h2048_f768", "smallbatch_e128_h2688_f1856",
                                  "zipf_e128_h2048_f768"])
def test_workload_whole_output(name):
    """Full-size workloads in the benchmark's launch configuration: every
    element of H1, A, Y, dH1 and dX against the oracle, stage by stage and end
    to end, in every weight layout."""
    _full_size_run(name, whole=True)


@pytest.mark.timeout(900)
def test_padded_workload_every_tile():
    """The largest workload (278,272 rows, H = 4096): the oracle computes both
    ends of every 256-row tile of every expert, the padding boundaries and
    random rows; the GPU runs the whole problem in every weight layout."""
    _full_size_run("padded_e128_h4096_f2048", whole=False)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("H,F", [(256, 128), (16384, 32640)])
def test_largest_expert_matrix(H, F):
    """The largest expert matrices the boundary accepts: at H = 16384,
    F = 32640 one expert's W1 is 4FH = 2,139,095,040 bytes, just under the
    2^31-byte limit, so the kernels' 32-bit byte offsets inside a matrix and
    a token panel reach their largest values, and the second expert's
    weights start 3.2 GB into the packed buffer.  Expert 0 has 40 rows (a
    thin item only), expert 1 has 300 (a full tile and a thin remainder).
    Both weight layouts run the whole problem with NaN-filled outputs; the
    oracle computes the first and last rows of each expert and both sides of
    the tile boundary, every stage."""
    _gpu_ok()
    log(f"[max] drawing E=2 H={H} F={F}")
    case = workload.custom_case([40, 300], H, F, seed=31)
    dc, (h1, a, y, ws, dx) = run_layouts(case, canary=True)
    for name, t in (("h1", h1), ("a", a), ("y", y), ("dh1", ws), ("dx", dx)):
        assert bool(torch.isfinite(t).all()), f"{name}: an element was never written"
    rows = np.array([0, 39, 40, 41, 295, 296, 297, 339], dtype=np.int64)
    _, compact = oracle.sample_rows(case.offsets, rows)
    rt = torch.from_numpy(rows)
    rd = rt.to(dc.dev)
    log(f"[max] oracle on rows {rows.tolist()}")
    w1f, w2f = oracle._as_f32(case.w1), oracle._as_f32(case.w2)
    out = stagewise(case.x[rt], case.dy[rt], compact, w1f, w2f, h1[rd], a[rd], y[rd], ws[rd], dx[rd],
                    exact=False)
    log(f"[max] H={H} F={F} ok: " + summary(out))


def test_fragment_ordered_copies_layout():
    """The opt-in fragment buffer: per expert, W1 (rows in feature blocks of 64,
    gate rows then up rows), W2, W1^T and W2^T, each in blocks of 32 rows x 16 k
    where lane l holds rows 32b + (l & 31), k 16s + 8(l >> 5); the packed
    buffer keeps exactly the row-major weights."""
    _gpu_ok()
    import moe_expert_grouped_ragged_amd as gg
    E, H, F = 3, 256, 128
    case = workload.custom_case([1, 2, 3], H, F, seed=5)
    w1, w2 = case.w1.cuda(), case.w2.cuda()
    packed = gg.gg_pack_weights(w1, w2)
    frag = gg.gg_pack_frag(packed, E, H, F)
    torch.cuda.synchronize()
    assert packed.numel() == 3 * E * H * F and frag.numel() == 6 * E * H * F
    pblk = packed.view(E, 3 * H * F)
    fblk = frag.view(E, 6 * H * F)
    for e in range(E):
        assert torch.equal(pblk[e, :2 * F * H].view(2 * F, H), w1[e])
        assert torch.equal(pblk[e, 2 * F * H:].view(H, F), w2[e])
        w1i = torch.cat([w1[e][:F].view(F // 64, 64, H), w1[e][F:].view(F // 64, 64, H)], 1).reshape(2 * F, H)
        for got, w, K in ((fblk[e, :2 * F * H], w1i, H), (fblk[e, 2 * F * H:3 * F * H], w2[e], F),
                          (fblk[e, 3 * F * H:5 * F * H], w1[e].t().contiguous(), 2 * F),
                          (fblk[e, 5 * F * H:], w2[e].t().contiguous(), H)):
            n = w.shape[0]
            want = w.reshape(n // 32, 32, K // 16, 2, 8).permute(0, 2, 3, 1, 4).reshape(-1)
            assert torch.equal(got, want)
