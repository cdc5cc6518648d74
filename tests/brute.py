"""Independent float64 references used to pin the oracle (tests only).

Nothing here is shared with the oracle or the HIP library: bf16 rounding is
done with ``np.rint`` on a power-of-two grid (round half to even) instead of
bit manipulation, products are dense ``numpy`` matmuls in float64, and SiLU
uses float64 ``np.exp``.
"""
from __future__ import annotations

import numpy as np

BF16_MAX = float.fromhex("0x1.fep127")


def rne_bf16(v) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even."""
    v = np.asarray(v, dtype=np.float64)
    out = np.array(v, copy=True)
    fin = np.isfinite(v) & (v != 0)
    a = np.abs(v[fin])
    e = np.floor(np.log2(a))
    # log2 can be off by one at exact powers of two / near them: fix it.
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > a, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= a, e + 1, e)
    e = np.maximum(e, -126.0)                       # subnormal bf16 share 2^-133 spacing
    ulp_exp = (e - 7).astype(np.int64)
    q = np.rint(np.ldexp(np.sign(v[fin]) * a, -ulp_exp))   # half to even
    r = np.ldexp(q, ulp_exp)
    r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, r), r)
    out[fin] = r
    return out


def bf16_ulp(v) -> np.ndarray:
    """Spacing of bf16 values at |v| (for tolerance statements)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def silu64(g):
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def sigmoid64(g):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(g, dtype=np.float64)))


def dense_forward(x, offsets, w1, w2, round_points: bool):
    """Per-expert dense float64 forward via numpy matmul; optionally rounds to
    bf16 at H1, A and Y (the oracle's points)."""
    x = np.asarray(x, np.float64)
    w1 = np.asarray(w1, np.float64)
    w2 = np.asarray(w2, np.float64)
    E, twoF, H = w1.shape
    F = twoF // 2
    M = x.shape[0]
    R = rne_bf16 if round_points else (lambda t: t)
    h1 = np.full((M, 2 * F), np.nan)
    a = np.full((M, F), np.nan)
    y = np.full((M, H), np.nan)
    for e in range(E):
        s, t = int(offsets[e]), int(offsets[e + 1])
        if s == t:
            continue
        he = R(x[s:t] @ w1[e].T)
        ae = R(silu64(he[:, :F]) * he[:, F:])
        h1[s:t], a[s:t], y[s:t] = he, ae, R(ae @ w2[e].T)
    return h1, a, y


def dense_dgrad(dy, h1, offsets, w1, w2, round_points: bool):
    """Per-expert dense float64 input gradient; optionally rounds at dA, dH1, dX."""
    dy = np.asarray(dy, np.float64)
    h1 = np.asarray(h1, np.float64)
    w1 = np.asarray(w1, np.float64)
    w2 = np.asarray(w2, np.float64)
    E, twoF, H = w1.shape
    F = twoF // 2
    M = dy.shape[0]
    R = rne_bf16 if round_points else (lambda t: t)
    dh1 = np.full((M, 2 * F), np.nan)
    dx = np.full((M, H), np.nan)
    for e in range(E):
        s, t = int(offsets[e]), int(offsets[e + 1])
        if s == t:
            continue
        da = R(dy[s:t] @ w2[e])
        g, u = h1[s:t, :F], h1[s:t, F:]
        sg = sigmoid64(g)
        dg = R(da * u * sg * (1.0 + g * (1.0 - sg)))
        du = R(da * g * sg)
        dh = np.concatenate([dg, du], axis=1)
        dh1[s:t] = dh
        dx[s:t] = R(dh @ w1[e])
    return dh1, dx


GATE_SLOPE = {"swiglu": 1.0, "qgeglu": 1.702}


def act64(g, act: str):
    """Gate activation g * sigmoid(c g) in float64 (c from GATE_SLOPE)."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-GATE_SLOPE[act] * g))


def dense_forward_glu(x, offsets, w1, w2, act: str, probs, round_points: bool):
    """dense_forward with the activation chosen by act and the result of the
    activation scaled per row by probs (None: no scaling)."""
    x = np.asarray(x, np.float64)
    w1 = np.asarray(w1, np.float64)
    w2 = np.asarray(w2, np.float64)
    E, twoF, H = w1.shape
    F = twoF // 2
    M = x.shape[0]
    p = np.ones(M) if probs is None else np.asarray(probs, np.float64)
    R = rne_bf16 if round_points else (lambda t: t)
    h1 = np.full((M, 2 * F), np.nan)
    a = np.full((M, F), np.nan)
    y = np.full((M, H), np.nan)
    for e in range(E):
        s, t = int(offsets[e]), int(offsets[e + 1])
        if s == t:
            continue
        he = R(x[s:t] @ w1[e].T)
        ae = R(p[s:t, None] * act64(he[:, :F], act) * he[:, F:])
        h1[s:t], a[s:t], y[s:t] = he, ae, R(ae @ w2[e].T)
    return h1, a, y


def dense_dgrad_glu(dy, h1, offsets, w1, w2, act: str, probs, round_points: bool):
    """Input gradient of dense_forward_glu plus the gradient of the per-row
    scale: returns dH1, dX and dp (dp unrounded)."""
    dy = np.asarray(dy, np.float64)
    h1 = np.asarray(h1, np.float64)
    w1 = np.asarray(w1, np.float64)
    w2 = np.asarray(w2, np.float64)
    E, twoF, H = w1.shape
    F = twoF // 2
    M = dy.shape[0]
    c = GATE_SLOPE[act]
    p = np.ones(M) if probs is None else np.asarray(probs, np.float64)
    R = rne_bf16 if round_points else (lambda t: t)
    dh1 = np.full((M, 2 * F), np.nan)
    dx = np.full((M, H), np.nan)
    dp = np.full(M, np.nan)
    for e in range(E):
        s, t = int(offsets[e]), int(offsets[e + 1])
        if s == t:
            continue
        da = R(dy[s:t] @ w2[e])
        g, u = h1[s:t, :F], h1[s:t, F:]
        sg = sigmoid64(c * g)
        pe = p[s:t, None]
        dg = R(pe * da * u * sg * (1.0 + c * g * (1.0 - sg)))
        du = R(pe * da * g * sg)
        dh = np.concatenate([dg, du], axis=1)
        dh1[s:t] = dh
        dx[s:t] = R(dh @ w1[e])
        dp[s:t] = np.sum(da * act64(g, act) * u, axis=1)
    return dh1, dx, dp
