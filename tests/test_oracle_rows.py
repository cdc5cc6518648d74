"""CPU pins of the oracle's router-probability-on-input functions
(scale_rows, scale_rows_backward): the FC1 input row scaled by its router
probability, the optional multiply before FC1 that the paged-stash pull
request ("[Main] Support paged stash with device-initiated GroupedLinear",
"What does this PR do") names beside the activation boundary.

Reading pinned here: x'_r = bf16(fp32(p_r * x_r)) (fp32 product, then one
rounding to bf16), dx_r = bf16(fp32(p_r * g_r)), dp_r = sum_h g*x.

Pins, none of which retypes the oracle's formula:
* exact rational arithmetic (fractions.Fraction) with an independent
  round-to-nearest-even to a binary format, on random values and on pairs
  where rounding the exact product once would give another bf16 value;
* p = 1 is the identity, bit for bit;
* per-row powers of two scale exactly, which also pins the row indexing;
* finite differences of L = <G, p x> in p and in x (fp64).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _round_rational(q: Fraction, bits: int, emin: int = -126) -> Fraction:
    """Nearest value with `bits` significant bits (subnormal below 2^emin),
    ties to even.  Overflow is not handled (the inputs stay far from it)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, emin) - (bits - 1))
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def _expected_scale(p: np.float32, x: np.float32) -> float:
    exact = Fraction(float(p)) * Fraction(float(x))
    return float(_round_rational(_round_rational(exact, 24), 8))


def _bf16_values(rng, shape):
    return oracle.round_bf16(rng.standard_normal(shape).astype(np.float32))


def _double_rounding_pairs(rng, want=12):
    """(p, x) pairs whose fp32 product sits exactly halfway between two bf16
    values while the exact product does not: there the fp32-then-bf16
    reading and a single rounding of the exact product differ."""
    found = []
    while len(found) < want:
        p = rng.random(1 << 16).astype(np.float32)
        x = _bf16_values(rng, 1 << 16)
        prod32 = p * x
        bits = prod32.view(np.uint32)
        tie = (bits & 0xFFFF) == 0x8000
        exact_differs = p.astype(np.float64) * x.astype(np.float64) != prod32.astype(np.float64)
        for i in np.flatnonzero(tie & exact_differs):
            found.append((p[i], x[i]))
    return found[:want]


def test_scale_rows_exact_rational():
    rng = np.random.default_rng(11)
    M, H = 7, 24
    x = _bf16_values(rng, (M, H))
    p = rng.random(M).astype(np.float32)
    p[0], p[1] = 0.0, 1.0
    got = oracle.scale_rows(x, p)
    for r in range(M):
        for h in range(H):
            assert got[r, h] == _expected_scale(p[r], x[r, h]), (r, h)


def test_scale_rows_double_rounding_reading():
    rng = np.random.default_rng(12)
    pairs = _double_rounding_pairs(rng)
    p = np.array([q for q, _ in pairs], np.float32)
    x = np.array([[v] for _, v in pairs], np.float32)
    got = oracle.scale_rows(x, p)[:, 0]
    single = [float(_round_rational(Fraction(float(q)) * Fraction(float(v)), 8)) for q, v in pairs]
    want = [_expected_scale(q, v) for q, v in pairs]
    assert list(got) == want
    assert any(a != b for a, b in zip(want, single)), "the pairs do not separate the readings"
    # the backward's dx uses the same product and rounding
    dx = oracle.scale_rows_backward(x, np.zeros_like(x), p)["dx"][:, 0]
    assert list(dx) == want


def test_scale_rows_identity_and_zero():
    rng = np.random.default_rng(13)
    x = _bf16_values(rng, (9, 40))
    ones = np.ones(9, np.float32)
    assert np.array_equal(oracle.scale_rows(x, ones).view(np.uint32), x.view(np.uint32))
    b = oracle.scale_rows_backward(x, x, ones)
    assert np.array_equal(b["dx"].view(np.uint32), x.view(np.uint32))
    z = oracle.scale_rows(x, np.zeros(9, np.float32))
    assert np.all(z == 0)


def test_scale_rows_per_row_powers_of_two():
    rng = np.random.default_rng(14)
    M, H = 6, 33          # H != M, so a transposed index scales by the wrong power
    x = _bf16_values(rng, (M, H))
    k = np.array([-3, -1, 0, 1, 2, 5])
    p = np.ldexp(np.ones(M), k).astype(np.float32)
    want = np.ldexp(x.astype(np.float64), k[:, None])
    assert np.array_equal(oracle.scale_rows(x, p).astype(np.float64), want)
    g = _bf16_values(rng, (M, H))
    b = oracle.scale_rows_backward(g, x, p)
    assert np.array_equal(b["dx"].astype(np.float64), np.ldexp(g.astype(np.float64), k[:, None]))


def test_scale_rows_backward_finite_differences():
    rng = np.random.default_rng(15)
    M, H = 5, 20
    x = _bf16_values(rng, (M, H)).astype(np.float64)
    G = _bf16_values(rng, (M, H)).astype(np.float64)
    p = rng.random(M)

    def loss(pp, xx):
        return float(np.sum(G * oracle.scale_rows64(xx, pp)))

    b64 = oracle.scale_rows_backward64(G, x, p)
    eps = 1e-3
    for r in range(M):
        e = np.zeros(M)
        e[r] = eps
        fd = (loss(p + e, x) - loss(p - e, x)) / (2 * eps)
        assert abs(fd - b64["dprobs"][r]) <= 1e-9 * (1 + abs(fd))
    for r, h in [(0, 0), (2, 7), (4, 19)]:
        e = np.zeros((M, H))
        e[r, h] = eps
        fd = (loss(p, x + e) - loss(p, x - e)) / (2 * eps)
        assert abs(fd - b64["dx"][r, h]) <= 1e-9 * (1 + abs(fd))
    # the fp32 parity reference: dp within the fp32 summation bound of fp64
    b32 = oracle.scale_rows_backward(G.astype(np.float32), x.astype(np.float32), p.astype(np.float32))
    bound = H * 2.0 ** -23 * np.sum(np.abs(G * x), axis=1)
    assert np.all(np.abs(b32["dprobs"] - b64["dprobs"]) <= bound)


def test_scale_rows_empty():
    x = np.zeros((0, 16), np.float32)
    assert oracle.scale_rows(x, np.zeros(0, np.float32)).shape == (0, 16)
    b = oracle.scale_rows_backward(x, x, np.zeros(0, np.float32))
    assert b["dx"].shape == (0, 16) and b["dprobs"].shape == (0,)
