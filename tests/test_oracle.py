"""Pins of the CPU oracle against things other than itself (CPU only).

Each test targets a plausible mistake: a wrong bf16 rounding, a swapped
gate/up half, a transposed weight, a dropped term in the SiLU derivative, a
wrong expert segment, a thread-count dependence.
"""
import json
import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import workload
from brute import bf16_ulp, dense_dgrad, dense_forward, rne_bf16, silu64, sigmoid64

HERE = os.path.dirname(os.path.abspath(__file__))


def f32(t):
    return oracle._as_f32(t)


def within_one_ulp(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.abs(got - ref) <= bf16_ulp(ref) * 1.0000001


# --------------------------------------------------------------------------- rounding

def test_round_bf16_exhaustive(tmp_path):
    """All 2^32 fp32 patterns against the round-to-nearest-even definition."""
    exe = str(tmp_path / "rne_exhaustive")
    subprocess.check_call(["gcc", "-O2", "-o", exe, os.path.join(HERE, "rne_exhaustive.c"),
                           "-ldl", "-lm"])
    oracle._load()
    out = subprocess.run([exe, oracle._LIB], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr


def test_round_bf16_matches_torch_and_float64_grid():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 200000),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 1.001953125, 3.3895314e38, 3.4e38,
                  1e-40, -1e-40, 2 ** -133, 2 ** -134], dtype=np.float32),
    ]).astype(np.float32)
    got = oracle.round_bf16(v)
    want_torch = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(got.view(np.uint32), want_torch.view(np.uint32))
    np.testing.assert_array_equal(got.astype(np.float64), rne_bf16(v.astype(np.float64)))


# --------------------------------------------------------------------------- SwiGLU

def _silu_probe(g_vals, u_vals):
    """A problem whose H1 gate/up equal the given bf16 values exactly:
    E=1, H=2, F=1, x=[g, u], W1 gate row [1, 0], up row [0, 1], W2 = [[1], [0]]."""
    M = g_vals.shape[0]
    x = np.stack([g_vals, u_vals], axis=1).astype(np.float32)
    w1 = np.array([[[1.0, 0.0], [0.0, 1.0]]], np.float32)
    w2 = np.array([[[1.0], [0.0]]], np.float32)
    return oracle.forward(x, np.array([0, M]), w1, w2)


def _all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    return v[np.isfinite(v)]


def test_swiglu_exhaustive_over_bf16_gate():
    g = _all_finite_bf16()
    out = _silu_probe(g, np.ones_like(g))
    np.testing.assert_array_equal(out["h1"][:, 0], g)          # gate passes through exactly
    np.testing.assert_array_equal(out["h1"][:, 1], 1.0)
    a = out["a"][:, 0].astype(np.float64)
    ref = rne_bf16(silu64(g))
    # below g = -88.7 fp32 exp(-g) overflows and silu becomes -0 instead of a
    # value under 2e-37: an absolute difference far below any tolerance.
    ok = within_one_ulp(a, ref) | (np.abs(a - ref) < 1e-30)
    assert ok.all(), g[~ok][:10]
    assert np.mean(a != ref) < 2e-3
    # FC2 with W2 = [[1],[0]] copies A into Y[:, 0] and gives exact zeros in Y[:, 1]
    np.testing.assert_array_equal(out["y"][:, 0], out["a"][:, 0])
    np.testing.assert_array_equal(out["y"][:, 1], 0.0)


def test_swiglu_special_values():
    g = np.array([0.0, 30.0, 100.0, -100.0, -30.0, 1.0], np.float32)
    u = np.array([5.0, 1.0, -2.0, 3.0, 1.0, 0.0], np.float32)
    a = _silu_probe(g, u)["a"][:, 0]
    assert a[0] == 0.0                                   # silu(0) = 0
    assert a[1] == 30.0                                  # silu(x) -> x as x -> +inf
    assert a[2] == -200.0
    assert abs(a[3]) < 1e-30 and abs(a[4]) < 1e-10       # silu(x) -> 0 as x -> -inf
    assert a[5] == 0.0                                   # up = 0
    # the gate half is the first F outputs, the up half the last F
    a2 = _silu_probe(np.array([2.0], np.float32), np.array([-1.0], np.float32))["a"][0, 0]
    assert a2 == pytest.approx(-2.0 / (1 + math.exp(-2.0)), rel=4e-3)


def test_dswiglu_derivative_special_values():
    """silu'(0) = 1/2: with g = 0, u = 1, dA = 1 the gate gradient is 1/2 and
    the up gradient is silu(0) = 0."""
    # E=1, H=1, F=1; W1 = [[0],[1]] gives g = 0, u = x; W2 = [[1]] gives dA = dy.
    x = np.array([[1.0]], np.float32)
    w1 = np.array([[[0.0], [1.0]]], np.float32)
    w2 = np.array([[[1.0]]], np.float32)
    fw = oracle.forward(x, np.array([0, 1]), w1, w2)
    dg = oracle.dgrad(np.array([[1.0]], np.float32), fw["h1"], np.array([0, 1]), w1, w2)
    assert dg["dh1"][0, 0] == 0.5 and dg["dh1"][0, 1] == 0.0
    assert dg["dx"][0, 0] == 0.0       # dX = 0.5 * W1[0] + 0 * W1[1] = 0


# --------------------------------------------------------------------------- brute force

def _random_problem(counts, H, F, seed, w_std=0.02):
    c = workload.custom_case(counts, H, F, seed, w_std=w_std)
    return c, f32(c.x), f32(c.w1), f32(c.w2), f32(c.dy)


@pytest.mark.parametrize("counts,H,F,seed", [
    ([3, 0, 5, 1], 16, 8, 1),
    ([7, 2], 40, 24, 2),
    ([1], 8, 8, 3),
    ([0, 9, 0, 4, 0], 24, 16, 4),
])
def test_forward_stagewise_vs_float64_brute_force(counts, H, F, seed):
    c, x, w1, w2, _ = _random_problem(counts, H, F, seed, w_std=0.3)
    out = oracle.forward(x, c.offsets, w1, w2)
    off = c.offsets
    rows = np.concatenate([np.arange(off[e], off[e + 1]) for e in range(c.E)]).astype(np.int64)
    ex = np.searchsorted(off, rows, side="right") - 1
    # FC1 per row against a float64 dot product of the right expert's weights
    ref_h1 = rne_bf16(np.einsum("rk,rjk->rj", x[rows].astype(np.float64), w1[ex].astype(np.float64)))
    assert within_one_ulp(out["h1"][rows], ref_h1).all()
    assert np.mean(out["h1"][rows] != ref_h1) < 0.02
    # SwiGLU from the oracle's own H1 (isolates the stage)
    h1 = out["h1"][rows].astype(np.float64)
    ref_a = rne_bf16(silu64(h1[:, :F]) * h1[:, F:])
    assert within_one_ulp(out["a"][rows], ref_a).all()
    assert np.mean(out["a"][rows] != ref_a) < 0.02
    # FC2 from the oracle's own A
    ref_y = rne_bf16(np.einsum("rj,rnj->rn", out["a"][rows].astype(np.float64), w2[ex].astype(np.float64)))
    assert within_one_ulp(out["y"][rows], ref_y).all()
    assert np.mean(out["y"][rows] != ref_y) < 0.02


@pytest.mark.parametrize("counts,H,F,seed", [
    ([3, 0, 5, 1], 16, 8, 5),
    ([6, 2], 40, 24, 6),
    ([0, 9, 0, 4, 0], 24, 16, 7),
])
def test_dgrad_stagewise_vs_float64_brute_force(counts, H, F, seed):
    c, x, w1, w2, dy = _random_problem(counts, H, F, seed, w_std=0.3)
    fw = oracle.forward(x, c.offsets, w1, w2)
    out = oracle.dgrad(dy, fw["h1"], c.offsets, w1, w2)
    off = c.offsets
    rows = np.concatenate([np.arange(off[e], off[e + 1]) for e in range(c.E)]).astype(np.int64)
    ex = np.searchsorted(off, rows, side="right") - 1
    h1 = fw["h1"][rows].astype(np.float64)
    g, u = h1[:, :F], h1[:, F:]
    da = rne_bf16(np.einsum("rn,rnj->rj", dy[rows].astype(np.float64), w2[ex].astype(np.float64)))
    sg = sigmoid64(g)
    ref_dg = rne_bf16(da * u * sg * (1 + g * (1 - sg)))
    ref_du = rne_bf16(da * g * sg)
    got = out["dh1"][rows]
    # dA can round differently by one ulp; the gradient then moves by about one ulp
    # of dA relative, so allow two ulps for dH1 and require most to be exact.
    for got_h, ref_h in ((got[:, :F], ref_dg), (got[:, F:], ref_du)):
        assert (np.abs(got_h - ref_h) <= 2.0000001 * bf16_ulp(ref_h) + 1e-30).all()
        assert np.mean(got_h != ref_h) < 0.05
    ref_dx = rne_bf16(np.einsum("rj,rjk->rk", got.astype(np.float64), w1[ex].astype(np.float64)))
    assert within_one_ulp(out["dx"][rows], ref_dx).all()
    assert np.mean(out["dx"][rows] != ref_dx) < 0.02


def test_tiny_workload_vs_float64_pipeline():
    """Whole forward + dgrad of the 4-expert workload against dense float64
    matmuls (rounded at the same points): bf16-level agreement."""
    c = workload.draw_case(workload.by_name("tiny_e4_h64_f128"))
    assert c.counts[2] == 0 and c.M == 512
    x, w1, w2, dy = f32(c.x), f32(c.w1), f32(c.w2), f32(c.dy)
    fw = oracle.forward(x, c.offsets, w1, w2)
    h1r, ar, yr = dense_forward(x, c.offsets, w1, w2, round_points=True)
    for got, ref in ((fw["h1"], h1r), (fw["a"], ar), (fw["y"], yr)):
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert rel < 2e-3
    dg = oracle.dgrad(dy, fw["h1"], c.offsets, w1, w2)
    dh1r, dxr = dense_dgrad(dy, fw["h1"], c.offsets, w1, w2, round_points=True)
    for got, ref in ((dg["dh1"], dh1r), (dg["dx"], dxr)):
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert rel < 2e-3


def test_float64_mode_equals_dense_float64():
    c, x, w1, w2, dy = _random_problem([4, 0, 6], 12, 10, 11, w_std=0.3)
    fw = oracle.forward64(x, c.offsets, w1, w2)
    h1r, ar, yr = dense_forward(x, c.offsets, w1, w2, round_points=False)
    np.testing.assert_allclose(fw["y"], yr, rtol=1e-12, atol=1e-14)
    dg = oracle.dgrad64(dy, fw["h1"], c.offsets, w1, w2)
    dh1r, dxr = dense_dgrad(dy, fw["h1"], c.offsets, w1, w2, round_points=False)
    np.testing.assert_allclose(dg["dx"], dxr, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------- closed forms

def test_closed_form_one_element():
    """E = M = H = F = 1: y = w2 silu(a x) (b x),
    dx = dy w2 (b silu(a x) + a (b x) silu'(a x)), silu'(z) = s (1 + z (1 - s))."""
    a, b, w2v, xv, dyv = 0.7, -1.3, 0.45, 1.9, -0.8
    z = a * xv
    s = 1 / (1 + math.exp(-z))
    y = w2v * z * s * (b * xv)
    dx = dyv * w2v * (b * xv * s * (1 + z * (1 - s)) * a + b * z * s)
    w1 = np.array([[[a], [b]]])
    w2 = np.array([[[w2v]]])
    fw = oracle.forward64(np.array([[xv]]), np.array([0, 1]), w1, w2)
    assert fw["y"][0, 0] == pytest.approx(y, rel=1e-14)
    dg = oracle.dgrad64(np.array([[dyv]]), fw["h1"], np.array([0, 1]), w1, w2)
    assert dg["dx"][0, 0] == pytest.approx(dx, rel=1e-14)


def test_single_expert_is_a_dense_gated_mlp():
    """E = 1 reduces to the textbook gated MLP written with torch float64 ops."""
    c, x, w1, w2, dy = _random_problem([9], 16, 12, 12, w_std=0.3)
    fw = oracle.forward64(x, c.offsets, w1, w2)
    X = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    W1 = torch.tensor(w1[0], dtype=torch.float64)
    W2 = torch.tensor(w2[0], dtype=torch.float64)
    gate, up = (X @ W1.T).chunk(2, dim=1)
    Y = (torch.nn.functional.silu(gate) * up) @ W2.T
    np.testing.assert_allclose(fw["y"], Y.detach().numpy(), rtol=1e-12)
    Y.backward(torch.tensor(dy, dtype=torch.float64))
    dg = oracle.dgrad64(dy, fw["h1"], c.offsets, w1, w2)
    np.testing.assert_allclose(dg["dx"], X.grad.numpy(), rtol=1e-11, atol=1e-13)


def test_finite_difference_vjp():
    """<dX, V> = d/de <dY, Y(X + e V)> at e = 0 (central differences, fp64 mode)."""
    rng = np.random.default_rng(3)
    counts = [5, 0, 7, 2]
    off = workload.offsets_from_counts(counts)
    E, H, F, M = 4, 16, 12, int(off[-1])
    x = rng.standard_normal((M, H))
    w1 = rng.standard_normal((E, 2 * F, H)) * 0.3
    w2 = rng.standard_normal((E, H, F)) * 0.3
    dy = rng.standard_normal((M, H))
    v = rng.standard_normal((M, H))
    fw = oracle.forward64(x, off, w1, w2)
    dx = oracle.dgrad64(dy, fw["h1"], off, w1, w2)["dx"]
    eps = 1e-5
    yp = oracle.forward64(x + eps * v, off, w1, w2)["y"]
    ym = oracle.forward64(x - eps * v, off, w1, w2)["y"]
    fd = np.sum(dy * (yp - ym)) / (2 * eps)
    an = np.sum(dx * v)
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an))


# --------------------------------------------------------------------------- invariants

def test_zero_token_experts_write_nothing_and_read_no_weights():
    c, x, w1, w2, dy = _random_problem([4, 0, 3, 0], 16, 8, 21)
    w1p, w2p = w1.copy(), w2.copy()
    w1p[1] = np.nan
    w2p[1] = np.nan
    w1p[3] = np.nan
    w2p[3] = np.nan
    fw = oracle.forward(x, c.offsets, w1p, w2p)
    assert np.isfinite(fw["y"]).all() and np.isfinite(fw["h1"]).all()
    dg = oracle.dgrad(dy, fw["h1"], c.offsets, w1p, w2p)
    assert np.isfinite(dg["dx"]).all()
    ref = oracle.forward(x, c.offsets, w1, w2)
    np.testing.assert_array_equal(fw["y"], ref["y"])


def test_rows_outside_offsets_are_untouched():
    c, x, w1, w2, dy = _random_problem([3, 2], 8, 8, 22)
    M = c.M
    xx = np.concatenate([np.zeros((2, 8), np.float32), x, np.zeros((3, 8), np.float32)])
    off = c.offsets + 2
    fw = oracle.forward(xx, off, w1, w2)
    assert np.isnan(fw["y"][:2]).all() and np.isnan(fw["y"][2 + M:]).all()
    assert np.isfinite(fw["y"][2:2 + M]).all()
    np.testing.assert_array_equal(fw["y"][2:2 + M], oracle.forward(x, c.offsets, w1, w2)["y"])


def test_empty_batch():
    w1 = np.zeros((3, 16, 8), np.float32)
    w2 = np.zeros((3, 8, 8), np.float32)
    fw = oracle.forward(np.zeros((0, 8), np.float32), np.zeros(4, np.int64), w1, w2)
    assert fw["y"].shape == (0, 8)


def test_grouped_equals_per_expert_concatenation():
    c, x, w1, w2, dy = _random_problem([5, 0, 7, 3], 24, 16, 23)
    fw = oracle.forward(x, c.offsets, w1, w2)
    dg = oracle.dgrad(dy, fw["h1"], c.offsets, w1, w2)
    for e in range(c.E):
        s, t = int(c.offsets[e]), int(c.offsets[e + 1])
        if s == t:
            continue
        one = oracle.forward(x[s:t], np.array([0, t - s]), w1[e:e + 1], w2[e:e + 1])
        np.testing.assert_array_equal(one["y"], fw["y"][s:t])
        d1 = oracle.dgrad(dy[s:t], one["h1"], np.array([0, t - s]), w1[e:e + 1], w2[e:e + 1])
        np.testing.assert_array_equal(d1["dx"], dg["dx"][s:t])


def test_power_of_two_homogeneity_bitwise():
    c, x, w1, w2, dy = _random_problem([6, 4], 32, 16, 24)
    fw = oracle.forward(x, c.offsets, w1, w2)
    fw2 = oracle.forward(2 * x, c.offsets, w1, w2)
    np.testing.assert_array_equal(fw2["h1"], 2 * fw["h1"])          # FC1 is linear in X
    dg = oracle.dgrad(dy, fw["h1"], c.offsets, w1, w2)
    dg2 = oracle.dgrad(2 * dy, fw["h1"], c.offsets, w1, w2)
    np.testing.assert_array_equal(dg2["dh1"], 2 * dg["dh1"])        # dgrad is linear in dY
    np.testing.assert_array_equal(dg2["dx"], 2 * dg["dx"])


def test_dgrad_additivity_fp64():
    rng = np.random.default_rng(5)
    off = workload.offsets_from_counts([4, 3])
    M, H, F = 7, 10, 6
    x = rng.standard_normal((M, H))
    w1 = rng.standard_normal((2, 2 * F, H))
    w2 = rng.standard_normal((2, H, F))
    d1, d2 = rng.standard_normal((M, H)), rng.standard_normal((M, H))
    h1 = oracle.forward64(x, off, w1, w2)["h1"]
    s = oracle.dgrad64(d1 + d2, h1, off, w1, w2)["dx"]
    p = oracle.dgrad64(d1, h1, off, w1, w2)["dx"] + oracle.dgrad64(d2, h1, off, w1, w2)["dx"]
    np.testing.assert_allclose(s, p, rtol=1e-12, atol=1e-12)


def test_zero_padding_rows_give_exact_zeros():
    c = workload.custom_case([5, 3, 1], 16, 8, 25, pad_to=8)
    x, w1, w2, dy = f32(c.x), f32(c.w1), f32(c.w2), f32(c.dy)
    fw = oracle.forward(x, c.offsets, w1, w2)
    dg = oracle.dgrad(dy, fw["h1"], c.offsets, w1, w2)
    for e in range(3):
        pad = slice(int(c.offsets[e] + c.counts[e]), int(c.offsets[e + 1]))
        for arr in (fw["h1"], fw["a"], fw["y"], dg["dh1"], dg["dx"]):
            assert (arr[pad] == 0).all()


def test_expert_permutation_permutes_results():
    c, x, w1, w2, dy = _random_problem([3, 5, 2], 16, 8, 26)
    perm = [2, 0, 1]
    segs = [(int(c.offsets[e]), int(c.offsets[e + 1])) for e in range(3)]
    xp = np.concatenate([x[s:t] for s, t in (segs[p] for p in perm)])
    offp = workload.offsets_from_counts([c.counts[p] for p in perm])
    fw = oracle.forward(x, c.offsets, w1, w2)
    fwp = oracle.forward(xp, offp, w1[perm], w2[perm])
    np.testing.assert_array_equal(fwp["y"], np.concatenate([fw["y"][s:t] for s, t in (segs[p] for p in perm)]))


def test_thread_count_does_not_change_bits():
    c, x, w1, w2, dy = _random_problem([40, 0, 33], 64, 32, 27)
    oracle.set_threads(1)
    a = oracle.forward(x, c.offsets, w1, w2)
    oracle.set_threads(4)
    b = oracle.forward(x, c.offsets, w1, w2)
    oracle.set_threads(os.cpu_count() or 1)
    np.testing.assert_array_equal(a["y"], b["y"])


def test_sample_rows_equals_full_problem():
    c, x, w1, w2, dy = _random_problem([5, 0, 7, 3], 16, 8, 28)
    fw = oracle.forward(x, c.offsets, w1, w2)
    rows = np.array([0, 4, 5, 11, 14])
    expert, compact = oracle.sample_rows(c.offsets, rows)
    np.testing.assert_array_equal(expert, [0, 0, 2, 2, 3])
    sub = oracle.forward(x[rows], compact, w1, w2)
    np.testing.assert_array_equal(sub["y"], fw["y"][rows])


# --------------------------------------------------------------------------- golden

def test_tiny_workload_golden():
    """Regression fixture written by tests/golden/make_golden.py (oracle only)."""
    path = os.path.join(HERE, "golden", "tiny_e4_h64_f128.json")
    with open(path) as fh:
        gold = json.load(fh)
    from golden.make_golden import summarize
    now = summarize()
    assert now == gold


def test_stage_entry_points_compose_to_the_whole_passes():
    """swiglu(H1), fc2(A) and dgrad_fc1(dH1) are the later steps of forward / dgrad (bitwise)."""
    c, x, w1, w2, dy = _random_problem([5, 0, 7, 3], 24, 16, 29, w_std=0.3)
    fw = oracle.forward(x, c.offsets, w1, w2)
    np.testing.assert_array_equal(oracle.swiglu(fw["h1"], c.offsets), fw["a"])
    np.testing.assert_array_equal(oracle.fc2(fw["a"], c.offsets, w2), fw["y"])
    dg = oracle.dgrad(dy, fw["h1"], c.offsets, w1, w2)
    np.testing.assert_array_equal(oracle.dgrad_fc1(dg["dh1"], c.offsets, w1), dg["dx"])
