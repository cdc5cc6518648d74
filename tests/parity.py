"""Parity helpers shared by the GPU tests (tests only).

The bar: relative L2 ||gpu - ref|| / ||ref|| <= 2e-3 and, per element,
|gpu - ref| <= 1e-2 * |ref| + 1e-3, both in float64 over every compared
element.  Any fp32 summation order is a correct result, so parity of the
floating-point outputs is tolerance-based; integer/index work (which rows are
written) is compared exactly.

Stage-wise reading of the per-element bar.  Every stage rounds to bf16, and
two correct summation orders can round an intermediate that lies within an
fp32 ulp of a bf16 rounding midpoint to neighbouring bf16 values (one bf16
ulp apart, both within half an ulp of the exact value).  Such a flip of an
H1 or A element of magnitude ~3 moves a downstream sum by ~1e-3 while that
sum may itself be ~1e-3 after cancellation, so the per-element bound on the
outputs Y and dX is applied given the SAME bf16 input of their last rounding
stage on both sides (A for Y, dH1 for dX), and the chained outputs (Y from X,
dX from dY and H1) are held to the relative-L2 bound, their per-element
statistics are reported, and check_not_less_accurate asserts that, against
a float64 evaluation with the same rounding points, the GPU has no more
elements over the per-element bound than the oracle itself.  The intermediates are
diagnostics: H1 from X and A from H1 are held to the per-element bound as
well; dH1 has two rounding points inside the dgrad call (dA, never stored,
then dH1), so its per-element bound is two bf16 ulps (2**-6 * |ref|) + 1e-3.
"""
from __future__ import annotations

import numpy as np
import torch

REL_L2 = 2e-3
ELEM_REL = 1e-2
ELEM_ABS = 1e-3
DH1_ELEM_REL = 2.0 ** -6     # two bf16 roundings (dA, then dH1) inside one call


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float32).numpy().astype(np.float64)


def check(name: str, got, ref, rows=None, elem_rel: float = ELEM_REL) -> dict:
    """got: torch bf16 (any device) or float array; ref: float array (oracle)."""
    g = bf16_to_f64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    if rows is not None:
        g, r = g[rows], r[rows]
    assert g.shape == r.shape, (name, g.shape, r.shape)
    if g.size == 0:
        return {"name": name, "n": 0}
    assert np.isfinite(g).all(), f"{name}: non-finite values in the GPU result"
    diff = np.abs(g - r)
    nref = np.linalg.norm(r)
    rel = np.linalg.norm(g - r) / nref if nref > 0 else np.linalg.norm(g - r)
    bound = elem_rel * np.abs(r) + ELEM_ABS
    ratio = diff / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    info = {"name": name, "n": int(g.size), "rel_l2": float(rel), "worst_ratio": float(ratio[worst]),
            "exact_frac": float(np.mean(diff == 0))}
    assert rel <= REL_L2, f"{name}: relative L2 {rel:.3e} > {REL_L2} ({info})"
    assert ratio[worst] <= 1.0, (f"{name}: element {worst} got {g[worst]} ref {r[worst]} "
                                 f"exceeds |d| <= {elem_rel:.3g}|ref| + {ELEM_ABS} ({info})")
    return info


def elem_stats(got, ref, rows=None) -> dict:
    """Relative L2 and the per-element statistics of |got - ref| against the
    bound 1e-2 |ref| + 1e-3 (float64, every compared element)."""
    g = bf16_to_f64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    if rows is not None:
        g, r = g[rows], r[rows]
    assert g.shape == r.shape, (g.shape, r.shape)
    if g.size == 0:
        return {"n": 0, "rel_l2": 0.0, "worst_ratio": 0.0, "over_bound": 0, "exact_frac": 1.0}
    d = np.abs(g - r)
    nref = np.linalg.norm(r)
    ratio = d / (ELEM_REL * np.abs(r) + ELEM_ABS)
    return {"n": int(g.size), "rel_l2": float(np.linalg.norm(g - r) / nref if nref > 0 else np.linalg.norm(g - r)),
            "worst_ratio": float(ratio.max()), "over_bound": int(np.count_nonzero(ratio > 1.0)),
            "exact_frac": float(np.mean(d == 0)), "finite": bool(np.isfinite(g).all())}


def check_chained(name: str, got, ref, rows=None) -> dict:
    """Outputs whose inputs came from an earlier stage on each side (Y from X,
    dX from dY through a separately computed H1 or dH1): the relative-L2 bound
    is asserted; the per-element statistics (worst ratio to the bound and the
    count of elements over it) are computed and returned for the log, and
    bounded by check_not_less_accurate against a float64 reference."""
    info = elem_stats(got, ref, rows)
    info["name"] = name
    if info["n"] == 0:
        return info
    assert info["finite"], f"{name}: non-finite values in the GPU result"
    assert info["rel_l2"] <= REL_L2, f"{name}: relative L2 {info['rel_l2']:.3e} > {REL_L2}"
    return info


# Margins of the accuracy comparison.  Elements over the per-element bound
# come from rare one-ulp rounding flips of an intermediate (H1, A, dA, dH1)
# that SwiGLU and the next GEMM amplify; the two implementations flip at
# different elements, so their counts and tails are samples of the same
# rare-event process.  Asserted: the count over the bound, the relative L2 and
# the 10th-largest ratio (a stable tail statistic) no worse than the oracle's
# within sampling margins (on small problems a single flip moves the relative
# L2 by several percent, hence its absolute slack); the single worst element,
# a maximum over a few dozen rare events, only within a looser factor.
ACC_COUNT_FACTOR, ACC_COUNT_ABS = 1.5, 16
# relative L2: one one-ulp flip of an element of typical size adds about
# 2**-8 / sqrt(n) to it, so the slack is 1e-4 (5% of the 2e-3 bar) plus a few
# such flips
ACC_REL_L2_FACTOR, ACC_REL_L2_ABS, ACC_REL_L2_FLIPS = 1.25, 1e-4, 2.0 ** -6
ACC_TAIL_K, ACC_TAIL_FACTOR = 10, 1.5
ACC_WORST_FACTOR = 3.0


def exact_reference(x, dy, offsets, w1, w2):
    """The most accurate evaluation of the method: float64 sums, rounded to
    bf16 at the same points as the oracle (H1, A, Y, dA, dH1, dX), dgrad from
    its own H1.  From tests/brute.py, which shares nothing with the oracle."""
    import brute
    import oracle
    xf, dyf = oracle._as_f32(x), oracle._as_f32(dy)
    w1f, w2f = oracle._as_f32(w1), oracle._as_f32(w2)
    h1, _, y = brute.dense_forward(xf, offsets, w1f, w2f, round_points=True)
    _, dx = brute.dense_dgrad(dyf, h1, offsets, w1f, w2f, round_points=True)
    return y, dx


def _kth_largest_ratio(got, ref, rows, k):
    g = bf16_to_f64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    if rows is not None:
        g, r = g[rows], r[rows]
    ratio = (np.abs(g - r) / (ELEM_REL * np.abs(r) + ELEM_ABS)).ravel()
    if ratio.size == 0:
        return 0.0
    k = min(k, ratio.size)
    return float(np.partition(ratio, ratio.size - k)[ratio.size - k])


def check_not_less_accurate(name: str, gpu, orac, exact, rows=None) -> dict:
    """The end-to-end per-element reading, checked: against the float64
    reference with the same rounding points, the GPU's chained result has no
    more elements over the per-element bound, no larger a relative L2 and no
    heavier a tail than the oracle's own chained result (margins above)."""
    sg = elem_stats(gpu, exact, rows)
    so = elem_stats(orac, exact, rows)
    tg = _kth_largest_ratio(gpu, exact, rows, ACC_TAIL_K)
    to = _kth_largest_ratio(orac, exact, rows, ACC_TAIL_K)
    info = {"name": name, "n": sg["n"], "gpu_over_bound": sg["over_bound"], "oracle_over_bound": so["over_bound"],
            "gpu_worst_ratio": sg["worst_ratio"], "oracle_worst_ratio": so["worst_ratio"],
            "gpu_tail10_ratio": tg, "oracle_tail10_ratio": to,
            "gpu_rel_l2": sg["rel_l2"], "oracle_rel_l2": so["rel_l2"]}
    assert sg["over_bound"] <= ACC_COUNT_FACTOR * so["over_bound"] + ACC_COUNT_ABS, \
        f"{name}: GPU has more elements over the bound than the oracle, against float64: {info}"
    slack = ACC_REL_L2_ABS + ACC_REL_L2_FLIPS / np.sqrt(max(sg["n"], 1))
    assert sg["rel_l2"] <= ACC_REL_L2_FACTOR * so["rel_l2"] + slack, \
        f"{name}: GPU relative L2 above the oracle's, against float64: {info}"
    assert tg <= ACC_TAIL_FACTOR * max(to, 1.0), \
        f"{name}: GPU tail (10th-largest ratio) above the oracle's, against float64: {info}"
    assert sg["worst_ratio"] <= ACC_WORST_FACTOR * max(so["worst_ratio"], 1.0), \
        f"{name}: GPU worst ratio far above the oracle's, against float64: {info}"
    return info


def stagewise(x, dy, offsets, w1, w2, h1, a, y, dh1, dx, rows=None, exact: bool = True) -> list:
    """Parity of every stage of one forward + dgrad pass.

    x, dy: CPU bf16 inputs over the compared rows (offsets index into them);
    h1, a, y, dh1, dx: the GPU outputs for the same rows (dgrad having been run
    from the GPU's own H1).  Each stage is compared per element against the
    oracle fed the GPU's bf16 input of that stage.  Y and dX are also compared
    end to end, each side from its own forward (relative L2 asserted,
    per-element statistics reported), and with exact=True both sides' end-to-end
    results are held against the float64 reference (check_not_less_accurate)."""
    import oracle
    h1c, ac, dh1c = h1.cpu(), a.cpu(), dh1.cpu()
    fw = oracle.forward(x, offsets, w1, w2)
    out = [check("h1", h1, fw["h1"], rows),
           check("a", a, oracle.swiglu(h1c, offsets), rows),
           check("y", y, oracle.fc2(ac, offsets, w2), rows),
           check_chained("a_chained", a, fw["a"], rows),
           check_chained("y_chained", y, fw["y"], rows)]
    dg = oracle.dgrad(dy, h1c, offsets, w1, w2)
    out += [check("dh1", dh1, dg["dh1"], rows, elem_rel=DH1_ELEM_REL),
            check("dx", dx, oracle.dgrad_fc1(dh1c, offsets, w1), rows),
            check_chained("dx_chained_from_gpu_h1", dx, dg["dx"], rows)]
    del dg
    dx_own = oracle.dgrad(dy, fw["h1"], offsets, w1, w2)["dx"]
    out.append(check_chained("dx_chained", dx, dx_own, rows))
    if exact:
        ye, dxe = exact_reference(x, dy, offsets, w1, w2)
        out += [check_not_less_accurate("y_vs_float64", y, fw["y"], ye, rows),
                check_not_less_accurate("dx_vs_float64", dx, dx_own, dxe, rows)]
    return out


def summary(out: list) -> str:
    """One log line per parity run: every check's relative L2, worst ratio and
    over-bound count, and the float64 comparisons."""
    parts = []
    for o in out:
        if "gpu_over_bound" in o:
            parts.append(f"{o['name']} over(gpu/oracle)={o['gpu_over_bound']}/{o['oracle_over_bound']} "
                         f"worst={o['gpu_worst_ratio']:.2f}/{o['oracle_worst_ratio']:.2f} "
                         f"tail10={o['gpu_tail10_ratio']:.2f}/{o['oracle_tail10_ratio']:.2f} "
                         f"rl2={o['gpu_rel_l2']:.2e}/{o['oracle_rel_l2']:.2e} n={o['n']}")
        else:
            parts.append(f"{o['name']} rl2={o.get('rel_l2', 0):.2e} wr={o.get('worst_ratio', 0):.2f}"
                         + (f" over={o['over_bound']}" if "over_bound" in o else ""))
    return ", ".join(parts)


def stagewise_glu(x, dy, offsets, w1, w2, act, probs, h1, a, y, dh1, dx, dprobs, rows=None) -> list:
    """stagewise() for the weighted SwiGLU / QuickGeGLU passes; probs is the
    fp32 [M] weight (numpy or None) and dprobs the GPU's fp32 [M] gradient of
    it, compared per element with the oracle fed the GPU's H1."""
    import oracle
    h1c, ac, dh1c = h1.cpu(), a.cpu(), dh1.cpu()
    fw = oracle.forward_glu(x, offsets, w1, w2, act, probs)
    out = [check("h1", h1, fw["h1"], rows),
           check("a", a, oracle.glu(h1c, offsets, act, probs), rows),
           check("y", y, oracle.fc2(ac, offsets, w2), rows),
           check_chained("a_chained", a, fw["a"], rows),
           check_chained("y_chained", y, fw["y"], rows)]
    dg = oracle.dgrad_glu(dy, h1c, offsets, w1, w2, act, probs)
    out += [check("dh1", dh1, dg["dh1"], rows, elem_rel=DH1_ELEM_REL),
            check("dx", dx, oracle.dgrad_fc1(dh1c, offsets, w1), rows),
            check_chained("dx_chained_from_gpu_h1", dx, dg["dx"], rows),
            check_chained("dx_chained", dx, oracle.dgrad_glu(dy, fw["h1"], offsets, w1, w2, act, probs)["dx"],
                          rows)]
    if dprobs is not None:
        out.append(check("dprobs", dprobs.detach().cpu().numpy().astype(np.float64), dg["dprobs"], rows))
    return out
