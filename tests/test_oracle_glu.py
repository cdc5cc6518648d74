"""Pins of the oracle's weighted SwiGLU / QuickGeGLU passes (CPU only).

The pages name the fused weighted SwiGLU and QuickGeGLU activations (paged-stash
pull request, "What does this PR do" and "Validation") without a formula; the
oracle reads them as A = p_r * act(gate) * up with act(g) = g * sigmoid(c g),
c = 1 or 1.702, and adds dp_r = sum_j dA act(gate) up to the input gradient.
Each test targets a plausible mistake: p applied to the wrong factor or at the
wrong rounding point, p missing from the gradient, a wrong slope or a dropped
term in the QuickGeGLU derivative, dp summing the wrong product.
"""
import math

import numpy as np
import pytest

import oracle
import workload
from brute import act64, bf16_ulp, dense_dgrad_glu, dense_forward_glu, rne_bf16


def f32(t):
    return oracle._as_f32(t)


def _case(counts, H, F, seed):
    c = workload.custom_case(counts, H, F, seed)
    rng = np.random.default_rng(seed + 100)
    probs = rng.uniform(0.05, 1.0, c.M).astype(np.float32)
    return c, f32(c.x), f32(c.w1), f32(c.w2), f32(c.dy), probs


def _gate_probe(g_vals, u_vals, act, probs=None):
    """H1 gate/up equal to the given bf16 values exactly (E=1, H=2, F=1)."""
    M = g_vals.shape[0]
    x = np.stack([g_vals, u_vals], axis=1).astype(np.float32)
    w1 = np.array([[[1.0, 0.0], [0.0, 1.0]]], np.float32)
    w2 = np.array([[[1.0], [0.0]]], np.float32)
    return oracle.forward_glu(x, np.array([0, M]), w1, w2, act, probs)


def _all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    return v[np.isfinite(v)]


@pytest.mark.parametrize("counts,H,F,seed", [([5, 0, 7, 2], 24, 16, 1), ([9], 40, 8, 2)])
def test_swiglu_without_or_with_unit_probs_is_the_unweighted_oracle(counts, H, F, seed):
    """p absent or p = 1 reproduces the (separately pinned) SwiGLU passes bit for bit."""
    c, x, w1, w2, dy, _ = _case(counts, H, F, seed)
    base_f = oracle.forward(x, c.offsets, w1, w2)
    base_d = oracle.dgrad(dy, base_f["h1"], c.offsets, w1, w2)
    for probs in (None, np.ones(c.M, np.float32)):
        f = oracle.forward_glu(x, c.offsets, w1, w2, "swiglu", probs)
        d = oracle.dgrad_glu(dy, f["h1"], c.offsets, w1, w2, "swiglu", probs)
        for k in ("h1", "a", "y"):
            np.testing.assert_array_equal(f[k], base_f[k])
        for k in ("dh1", "dx"):
            np.testing.assert_array_equal(d[k], base_d[k])


def test_qgeglu_exhaustive_over_bf16_gate():
    """A = act(g) for every finite bf16 gate with up = 1, against the float64
    closed form g / (1 + exp(-1.702 g)) rounded to bf16 (within one bf16 ulp)."""
    g = _all_finite_bf16()
    a = _gate_probe(g, np.ones_like(g), "qgeglu")["a"][:, 0].astype(np.float64)
    ref = rne_bf16(act64(g, "qgeglu"))
    ok = (np.abs(a - ref) <= bf16_ulp(ref) * 1.0000001) | (np.abs(a - ref) < 1e-30)
    assert ok.all(), g[~ok][:10]
    assert np.mean(a != ref) < 2e-3
    # spot values of the closed form
    a2 = _gate_probe(np.array([1.0, 0.0, 50.0], np.float32), np.ones(3, np.float32), "qgeglu")["a"][:, 0]
    assert a2[0] == pytest.approx(1.0 / (1.0 + math.exp(-1.702)), rel=4e-3)
    assert a2[1] == 0.0 and a2[2] == 50.0


def test_probs_scale_the_activation_after_it():
    """p multiplies act(g) * up, not the gate: with g = 2, up = 1, p = 0.25 the
    result is 0.25 * act(2), not act(0.5)."""
    for act in ("swiglu", "qgeglu"):
        a = _gate_probe(np.array([2.0], np.float32), np.array([1.0], np.float32), act,
                        np.array([0.25], np.float32))["a"][0, 0]
        assert a == pytest.approx(0.25 * float(act64(2.0, act)), rel=4e-3)


def test_derivatives_at_zero_and_large_gate():
    """act'(0) = 1/2 for both slopes; act'(g) -> 1 and act(g) -> g for large g;
    p scales both gradient halves; dp = dA act(g) up."""
    x = np.array([[1.0], [1.0]], np.float32)
    # row 0: g = 0, u = 1;  row 1: g = 40, u = 1 (W1 gate weight per row is the same, so use 2 experts)
    w1 = np.array([[[0.0], [1.0]], [[40.0], [1.0]]], np.float32)
    w2 = np.array([[[1.0]], [[1.0]]], np.float32)
    off = np.array([0, 1, 2])
    for act in ("swiglu", "qgeglu"):
        p = np.array([0.5, 0.25], np.float32)
        f = oracle.forward_glu(x, off, w1, w2, act, p)
        d = oracle.dgrad_glu(np.ones((2, 1), np.float32), f["h1"], off, w1, w2, act, p)
        assert d["dh1"][0, 0] == 0.5 * 0.5 and d["dh1"][0, 1] == 0.0
        assert d["dprobs"][0] == 0.0
        assert d["dh1"][1, 0] == 0.25 and d["dh1"][1, 1] == 0.25 * 40.0
        assert d["dprobs"][1] == 40.0


@pytest.mark.parametrize("act", ["swiglu", "qgeglu"])
@pytest.mark.parametrize("counts,H,F,seed", [([3, 0, 5, 1], 16, 8, 4), ([6, 2], 40, 24, 5)])
def test_float64_passes_equal_dense_float64(act, counts, H, F, seed):
    c, x, w1, w2, dy, probs = _case(counts, H, F, seed)
    f = oracle.forward_glu64(x, c.offsets, w1, w2, act, probs)
    h1, a, y = dense_forward_glu(x, c.offsets, w1, w2, act, probs, round_points=False)
    np.testing.assert_allclose(f["y"], y, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(f["a"], a, rtol=1e-12, atol=1e-15)
    d = oracle.dgrad_glu64(dy, f["h1"], c.offsets, w1, w2, act, probs)
    dh1, dx, dp = dense_dgrad_glu(dy, f["h1"], c.offsets, w1, w2, act, probs, round_points=False)
    np.testing.assert_allclose(d["dh1"], dh1, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(d["dx"], dx, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(d["dprobs"], dp, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("act", ["swiglu", "qgeglu"])
def test_fp32_passes_stagewise_vs_rounded_float64(act):
    """Each rounded stage of the fp32 passes, given the oracle's own previous
    stage, is within one bf16 ulp of the float64 value rounded once (A, dH1);
    dp agrees to fp32 accumulation accuracy."""
    c, x, w1, w2, dy, probs = _case([6, 0, 11, 3], 48, 40, 6)
    f = oracle.forward_glu(x, c.offsets, w1, w2, act, probs)
    _, a_ref, _ = dense_forward_glu(x, c.offsets, w1, w2, act, probs, round_points=True)
    rows = slice(0, c.M)
    # A from the oracle's own H1 (H1 itself is pinned by the unweighted tests)
    a_from_h1 = rne_bf16(probs[:, None].astype(np.float64) * act64(f["h1"][:, :40], act) * f["h1"][:, 40:])
    err = np.abs(f["a"][rows] - a_from_h1[rows])
    assert (err <= bf16_ulp(a_from_h1[rows]) * 1.0000001).all()
    assert np.isfinite(a_ref).all()
    d = oracle.dgrad_glu(dy, f["h1"], c.offsets, w1, w2, act, probs)
    dh1, _, dp = dense_dgrad_glu(dy, f["h1"], c.offsets, w1, w2, act, probs, round_points=True)
    err = np.abs(d["dh1"] - dh1)
    # dA itself may differ by one bf16 ulp (fp32 vs fp64 sums near a tie), hence two ulps
    assert (err <= 2 * bf16_ulp(dh1) * 1.0000001 + 1e-30).all()
    np.testing.assert_allclose(d["dprobs"], dp, rtol=2e-2, atol=2e-5)


def test_power_of_two_probs_scale_bitwise_and_dp_ignores_p():
    """A and dH1 are linear in p after rounding when p is a power of two
    (exact scaling); dX follows; dp does not depend on p at all."""
    c, x, w1, w2, dy, probs = _case([7, 0, 5], 32, 24, 7)
    for act in ("swiglu", "qgeglu"):
        f1 = oracle.forward_glu(x, c.offsets, w1, w2, act, probs)
        f2 = oracle.forward_glu(x, c.offsets, w1, w2, act, probs * np.float32(0.5))
        np.testing.assert_array_equal(f2["a"], f1["a"] * np.float32(0.5))
        d1 = oracle.dgrad_glu(dy, f1["h1"], c.offsets, w1, w2, act, probs)
        d2 = oracle.dgrad_glu(dy, f1["h1"], c.offsets, w1, w2, act, probs * np.float32(0.5))
        np.testing.assert_array_equal(d2["dh1"], d1["dh1"] * np.float32(0.5))
        np.testing.assert_array_equal(d2["dx"], d1["dx"] * np.float32(0.5))
        np.testing.assert_array_equal(d2["dprobs"], d1["dprobs"])


@pytest.mark.parametrize("act", ["swiglu", "qgeglu"])
def test_finite_difference_vjp_in_x_and_probs(act):
    """<dX, V> + <dp, v> = d/de <dY, Y(X + e V, p + e v)> (fp64 mode)."""
    rng = np.random.default_rng(8)
    counts = [5, 0, 7, 2]
    off = workload.offsets_from_counts(counts)
    E, H, F, M = 4, 16, 12, int(off[-1])
    x = rng.standard_normal((M, H))
    w1 = rng.standard_normal((E, 2 * F, H)) * 0.3
    w2 = rng.standard_normal((E, H, F)) * 0.3
    dy = rng.standard_normal((M, H))
    p = rng.uniform(0.1, 1.0, M)
    vx = rng.standard_normal((M, H))
    vp = rng.standard_normal(M)
    fw = oracle.forward_glu64(x, off, w1, w2, act, p)
    d = oracle.dgrad_glu64(dy, fw["h1"], off, w1, w2, act, p)
    eps = 1e-5
    yp = oracle.forward_glu64(x + eps * vx, off, w1, w2, act, p + eps * vp)["y"]
    ym = oracle.forward_glu64(x - eps * vx, off, w1, w2, act, p - eps * vp)["y"]
    fd = np.sum(dy * (yp - ym)) / (2 * eps)
    an = np.sum(d["dx"] * vx) + np.sum(d["dprobs"] * vp)
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))
    # the p part alone
    yp = oracle.forward_glu64(x, off, w1, w2, act, p + eps * vp)["y"]
    ym = oracle.forward_glu64(x, off, w1, w2, act, p - eps * vp)["y"]
    fd_p = np.sum(dy * (yp - ym)) / (2 * eps)
    assert abs(fd_p - np.sum(d["dprobs"] * vp)) <= 1e-7 * max(1.0, abs(fd_p))


def test_dprobs_written_only_for_routed_rows():
    c, x, w1, w2, dy, probs = _case([4, 0, 3], 16, 8, 9)
    M = c.M + 5
    xx = np.concatenate([x, np.ones((5, 16), np.float32)])
    dyy = np.concatenate([dy, np.ones((5, 16), np.float32)])
    pp = np.concatenate([probs, np.ones(5, np.float32)])
    f = oracle.forward_glu(xx, c.offsets, w1, w2, "qgeglu", pp)
    d = oracle.dgrad_glu(dyy, f["h1"], c.offsets, w1, w2, "qgeglu", pp)
    assert np.isfinite(d["dprobs"][:c.M]).all() and np.isnan(d["dprobs"][c.M:M]).all()
