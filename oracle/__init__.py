"""CPU oracle for the frozen MoE expert grouped GEMM -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its
Python binding) never does, and shares no code with it.

The arithmetic lives in ``oracle.cpp`` (plain C++, OpenMP over rows, built
with g++ without fast-math); this module only converts bf16 bit patterns to
and from fp32 and calls it.  See ``oracle.cpp`` for what is computed and the
passages it follows.

Parity pins: brute force in float64 (numpy matmul) on small inputs, the
closed-form one-element case, exhaustive bf16 rounding and SiLU checks,
a finite-difference check of the gradient, and invariants -- all in
``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with g++ (no fast-math, no FMA contraction)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + f".tmp{os.getpid()}"
    cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-Wall", "-Werror", _SRC, "-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build()
            lib = ctypes.CDLL(_LIB)
            i64, p = ctypes.c_int64, ctypes.c_void_p
            lib.oracle_round_bf16.argtypes = [p, p, i64]
            for name in ("oracle_forward_f32", "oracle_forward_f64"):
                getattr(lib, name).argtypes = [i64, i64, i64, p, p, p, p, p, p, p]
            for name in ("oracle_dgrad_f32", "oracle_dgrad_f64"):
                getattr(lib, name).argtypes = [i64, i64, i64, p, p, p, p, p, p, p]
            lib.oracle_swiglu_f32.argtypes = [i64, i64, p, p, p]
            lib.oracle_fc2_f32.argtypes = [i64, i64, i64, p, p, p, p]
            lib.oracle_dgrad_fc1_f32.argtypes = [i64, i64, i64, p, p, p, p]
            i32 = ctypes.c_int
            lib.oracle_glu_f32.argtypes = [i64, i64, p, i32, p, p, p]
            for name in ("oracle_forward_glu_f32", "oracle_forward_glu_f64"):
                getattr(lib, name).argtypes = [i64, i64, i64, p, i32, p, p, p, p, p, p, p]
            for name in ("oracle_dgrad_glu_f32", "oracle_dgrad_glu_f64"):
                getattr(lib, name).argtypes = [i64, i64, i64, p, i32, p, p, p, p, p, p, p, p]
            for name in ("oracle_scale_rows_f32", "oracle_scale_rows_f64"):
                getattr(lib, name).argtypes = [i64, i64, p, p, p]
            for name in ("oracle_scale_rows_bwd_f32", "oracle_scale_rows_bwd_f64"):
                getattr(lib, name).argtypes = [i64, i64, p, p, p, p, p]
            for name in ("oracle_round_bf16", "oracle_forward_f32", "oracle_forward_f64",
                         "oracle_dgrad_f32", "oracle_dgrad_f64", "oracle_swiglu_f32", "oracle_fc2_f32",
                         "oracle_dgrad_fc1_f32", "oracle_glu_f32", "oracle_forward_glu_f32",
                         "oracle_forward_glu_f64", "oracle_dgrad_glu_f32", "oracle_dgrad_glu_f64",
                         "oracle_scale_rows_f32", "oracle_scale_rows_f64", "oracle_scale_rows_bwd_f32",
                         "oracle_scale_rows_bwd_f64"):
                getattr(lib, name).restype = None
            _lib = lib
    return _lib


def set_threads(n: int) -> None:
    """Threads used by the OpenMP loops of later calls (process-wide)."""
    os.environ["OMP_NUM_THREADS"] = str(int(n))
    try:
        ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))
    except OSError:
        pass


# ---- bf16 bit patterns <-> fp32 values (exact in both directions for bf16 values) ----

def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits).view(np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits_exact(v: np.ndarray) -> np.ndarray:
    """fp32 arrays whose values are already bf16 values -> uint16 bit patterns."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("value not representable in bf16")
    return (u >> 16).astype(np.uint16)


def round_bf16(v: np.ndarray) -> np.ndarray:
    """The oracle's bf16 rounding (RNE), applied to fp32 values; returns fp32."""
    src = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty_like(src)
    _load().oracle_round_bf16(src.ctypes.data, out.ctypes.data, src.size)
    return out


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _as_f32(t) -> np.ndarray:
    """torch bf16 tensor / uint16 array / fp32 array -> contiguous fp32 ndarray."""
    if hasattr(t, "dtype") and str(getattr(t, "dtype", "")) == "torch.bfloat16":
        t = t.contiguous().view(dtype=__import__("torch").int16).numpy().view(np.uint16)
    a = np.asarray(t)
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a)
    return np.ascontiguousarray(a, dtype=np.float32)


def _check_offsets(offsets, E: int, M: int) -> np.ndarray:
    off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    if off.shape != (E + 1,) or off[0] < 0 or off[-1] > M or np.any(np.diff(off) < 0):
        raise ValueError("offsets must be int64 [E+1], non-decreasing, within [0, M]")
    return off


def forward(x, offsets, w1, w2):
    """fp32-accumulating forward. Inputs as bf16 (torch bf16, uint16 bits or fp32
    holding bf16 values).  x [M,H], w1 [E,2F,H], w2 [E,H,F].  Returns dict of
    fp32 arrays holding bf16 values: h1 [M,2F], a [M,F], y [M,H].  Rows outside
    [offsets[0], offsets[E]) are NaN (never written)."""
    x32, w132, w232 = _as_f32(x), _as_f32(w1), _as_f32(w2)
    E, twoF, H = w132.shape
    F = twoF // 2
    M = x32.shape[0]
    assert w232.shape == (E, H, F) and x32.shape == (M, H)
    off = _check_offsets(offsets, E, M)
    h1 = np.full((M, 2 * F), np.nan, np.float32)
    a = np.full((M, F), np.nan, np.float32)
    y = np.full((M, H), np.nan, np.float32)
    _load().oracle_forward_f32(E, H, F, _ptr(off), _ptr(x32), _ptr(w132), _ptr(w232),
                               _ptr(h1), _ptr(a), _ptr(y))
    return {"h1": h1, "a": a, "y": y}


def dgrad(dy, h1, offsets, w1, w2):
    """fp32-accumulating input gradient.  dy [M,H], h1 [M,2F] (bf16 values).
    Returns dict: dh1 [M,2F], dx [M,H] (fp32 arrays holding bf16 values)."""
    dy32, h132, w132, w232 = _as_f32(dy), _as_f32(h1), _as_f32(w1), _as_f32(w2)
    E, twoF, H = w132.shape
    F = twoF // 2
    M = dy32.shape[0]
    assert h132.shape == (M, 2 * F) and w232.shape == (E, H, F)
    off = _check_offsets(offsets, E, M)
    dh1 = np.full((M, 2 * F), np.nan, np.float32)
    dx = np.full((M, H), np.nan, np.float32)
    _load().oracle_dgrad_f32(E, H, F, _ptr(off), _ptr(dy32), _ptr(h132), _ptr(w132),
                             _ptr(w232), _ptr(dh1), _ptr(dx))
    return {"dh1": dh1, "dx": dx}


def swiglu(h1, offsets):
    """SwiGLU alone from a given H1 [M,2F] (bf16 values): a [M,F]."""
    h132 = _as_f32(h1)
    M, twoF = h132.shape
    F = twoF // 2
    off = _check_offsets(offsets, np.asarray(offsets).shape[0] - 1, M)
    a = np.full((M, F), np.nan, np.float32)
    _load().oracle_swiglu_f32(off.shape[0] - 1, F, _ptr(off), _ptr(h132), _ptr(a))
    return a


def fc2(a, offsets, w2):
    """FC2 alone from a given A [M,F] (bf16 values): y [M,H] (fp32 holding bf16)."""
    a32, w232 = _as_f32(a), _as_f32(w2)
    E, H, F = w232.shape
    M = a32.shape[0]
    assert a32.shape == (M, F)
    off = _check_offsets(offsets, E, M)
    y = np.full((M, H), np.nan, np.float32)
    _load().oracle_fc2_f32(E, H, F, _ptr(off), _ptr(a32), _ptr(w232), _ptr(y))
    return y


def dgrad_fc1(dh1, offsets, w1):
    """Last step of the input gradient alone, from a given dH1 [M,2F]: dx [M,H]."""
    dh132, w132 = _as_f32(dh1), _as_f32(w1)
    E, twoF, H = w132.shape
    F = twoF // 2
    M = dh132.shape[0]
    assert dh132.shape == (M, 2 * F)
    off = _check_offsets(offsets, E, M)
    dx = np.full((M, H), np.nan, np.float32)
    _load().oracle_dgrad_fc1_f32(E, H, F, _ptr(off), _ptr(dh132), _ptr(w132), _ptr(dx))
    return dx


def forward64(x, offsets, w1, w2):
    """fp64 forward without rounding (same code, double instantiation)."""
    x, w1, w2 = (np.ascontiguousarray(v, dtype=np.float64) for v in (x, w1, w2))
    E, twoF, H = w1.shape
    F = twoF // 2
    M = x.shape[0]
    off = _check_offsets(offsets, E, M)
    h1 = np.full((M, 2 * F), np.nan)
    a = np.full((M, F), np.nan)
    y = np.full((M, H), np.nan)
    _load().oracle_forward_f64(E, H, F, _ptr(off), _ptr(x), _ptr(w1), _ptr(w2),
                               _ptr(h1), _ptr(a), _ptr(y))
    return {"h1": h1, "a": a, "y": y}


def dgrad64(dy, h1, offsets, w1, w2):
    """fp64 input gradient without rounding."""
    dy, h1, w1, w2 = (np.ascontiguousarray(v, dtype=np.float64) for v in (dy, h1, w1, w2))
    E, twoF, H = w1.shape
    F = twoF // 2
    M = dy.shape[0]
    off = _check_offsets(offsets, E, M)
    dh1 = np.full((M, 2 * F), np.nan)
    dx = np.full((M, H), np.nan)
    _load().oracle_dgrad_f64(E, H, F, _ptr(off), _ptr(dy), _ptr(h1), _ptr(w1), _ptr(w2),
                             _ptr(dh1), _ptr(dx))
    return {"dh1": dh1, "dx": dx}


ACTIVATIONS = {"swiglu": 0, "qgeglu": 1}


def _act(act) -> int:
    if isinstance(act, str):
        return ACTIVATIONS[act]
    if int(act) not in ACTIVATIONS.values():
        raise ValueError(f"unknown activation {act}")
    return int(act)


def _probs(probs, M: int, dtype=np.float32):
    """Optional per-row probabilities [M] -> contiguous array (or None)."""
    if probs is None:
        return None
    if hasattr(probs, "detach"):
        probs = probs.detach().cpu().numpy()
    a = np.ascontiguousarray(np.asarray(probs, dtype=dtype))
    if a.shape != (M,):
        raise ValueError("probs must be [M]")
    return a


def _optr(a):
    return None if a is None else a.ctypes.data


def glu(h1, offsets, act="swiglu", probs=None):
    """Activation alone from a given H1 [M,2F]: a [M,F] = bf16(p * act(gate) * up)."""
    h132 = _as_f32(h1)
    M, twoF = h132.shape
    F = twoF // 2
    off = _check_offsets(offsets, np.asarray(offsets).shape[0] - 1, M)
    pr = _probs(probs, M)
    a = np.full((M, F), np.nan, np.float32)
    _load().oracle_glu_f32(off.shape[0] - 1, F, _ptr(off), _act(act), _optr(pr), _ptr(h132), _ptr(a))
    return a


def forward_glu(x, offsets, w1, w2, act="swiglu", probs=None):
    """forward() with the activation chosen by act ("swiglu" | "qgeglu") and
    optional fp32 per-row router probabilities probs [M] weighting it."""
    x32, w132, w232 = _as_f32(x), _as_f32(w1), _as_f32(w2)
    E, twoF, H = w132.shape
    F = twoF // 2
    M = x32.shape[0]
    assert w232.shape == (E, H, F) and x32.shape == (M, H)
    off = _check_offsets(offsets, E, M)
    pr = _probs(probs, M)
    h1 = np.full((M, 2 * F), np.nan, np.float32)
    a = np.full((M, F), np.nan, np.float32)
    y = np.full((M, H), np.nan, np.float32)
    _load().oracle_forward_glu_f32(E, H, F, _ptr(off), _act(act), _optr(pr), _ptr(x32), _ptr(w132),
                                   _ptr(w232), _ptr(h1), _ptr(a), _ptr(y))
    return {"h1": h1, "a": a, "y": y}


def dgrad_glu(dy, h1, offsets, w1, w2, act="swiglu", probs=None):
    """dgrad() for forward_glu: returns dh1, dx and dprobs [M] (fp32, NaN
    outside the routed rows)."""
    dy32, h132, w132, w232 = _as_f32(dy), _as_f32(h1), _as_f32(w1), _as_f32(w2)
    E, twoF, H = w132.shape
    F = twoF // 2
    M = dy32.shape[0]
    assert h132.shape == (M, 2 * F) and w232.shape == (E, H, F)
    off = _check_offsets(offsets, E, M)
    pr = _probs(probs, M)
    dh1 = np.full((M, 2 * F), np.nan, np.float32)
    dx = np.full((M, H), np.nan, np.float32)
    dp = np.full(M, np.nan, np.float32)
    _load().oracle_dgrad_glu_f32(E, H, F, _ptr(off), _act(act), _optr(pr), _ptr(dy32), _ptr(h132),
                                 _ptr(w132), _ptr(w232), _ptr(dh1), _ptr(dx), _ptr(dp))
    return {"dh1": dh1, "dx": dx, "dprobs": dp}


def forward_glu64(x, offsets, w1, w2, act="swiglu", probs=None):
    """fp64 forward_glu without rounding."""
    x, w1, w2 = (np.ascontiguousarray(v, dtype=np.float64) for v in (x, w1, w2))
    E, twoF, H = w1.shape
    F = twoF // 2
    M = x.shape[0]
    off = _check_offsets(offsets, E, M)
    pr = _probs(probs, M, np.float64)
    h1 = np.full((M, 2 * F), np.nan)
    a = np.full((M, F), np.nan)
    y = np.full((M, H), np.nan)
    _load().oracle_forward_glu_f64(E, H, F, _ptr(off), _act(act), _optr(pr), _ptr(x), _ptr(w1), _ptr(w2),
                                   _ptr(h1), _ptr(a), _ptr(y))
    return {"h1": h1, "a": a, "y": y}


def dgrad_glu64(dy, h1, offsets, w1, w2, act="swiglu", probs=None):
    """fp64 dgrad_glu without rounding."""
    dy, h1, w1, w2 = (np.ascontiguousarray(v, dtype=np.float64) for v in (dy, h1, w1, w2))
    E, twoF, H = w1.shape
    F = twoF // 2
    M = dy.shape[0]
    off = _check_offsets(offsets, E, M)
    pr = _probs(probs, M, np.float64)
    dh1 = np.full((M, 2 * F), np.nan)
    dx = np.full((M, H), np.nan)
    dp = np.full(M, np.nan)
    _load().oracle_dgrad_glu_f64(E, H, F, _ptr(off), _act(act), _optr(pr), _ptr(dy), _ptr(h1), _ptr(w1),
                                 _ptr(w2), _ptr(dh1), _ptr(dx), _ptr(dp))
    return {"dh1": dh1, "dx": dx, "dprobs": dp}


def scale_rows(x, probs):
    """Router probability on the FC1 input: x [M,H] -> bf16(p_r * x_r) [M,H]
    (fp32 product rounded once), every row."""
    x32 = _as_f32(x)
    M, H = x32.shape
    pr = _probs(probs, M)
    out = np.full((M, H), np.nan, np.float32)
    _load().oracle_scale_rows_f32(M, H, _ptr(pr), _ptr(x32), _ptr(out))
    return out


def scale_rows_backward(g, x, probs):
    """Input gradient of scale_rows given g = dL/dx' [M,H] and the unscaled
    x [M,H]: dx = bf16(p_r * g_r), dprobs [M] = sum_h g*x (fp32)."""
    g32, x32 = _as_f32(g), _as_f32(x)
    M, H = x32.shape
    assert g32.shape == (M, H)
    pr = _probs(probs, M)
    dx = np.full((M, H), np.nan, np.float32)
    dp = np.full(M, np.nan, np.float32)
    _load().oracle_scale_rows_bwd_f32(M, H, _ptr(pr), _ptr(g32), _ptr(x32), _ptr(dx), _ptr(dp))
    return {"dx": dx, "dprobs": dp}


def scale_rows64(x, probs):
    """fp64 scale_rows without rounding."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    M, H = x.shape
    pr = _probs(probs, M, np.float64)
    out = np.full((M, H), np.nan)
    _load().oracle_scale_rows_f64(M, H, _ptr(pr), _ptr(x), _ptr(out))
    return out


def scale_rows_backward64(g, x, probs):
    """fp64 scale_rows_backward without rounding."""
    g, x = (np.ascontiguousarray(v, dtype=np.float64) for v in (g, x))
    M, H = x.shape
    pr = _probs(probs, M, np.float64)
    dx = np.full((M, H), np.nan)
    dp = np.full(M, np.nan)
    _load().oracle_scale_rows_bwd_f64(M, H, _ptr(pr), _ptr(g), _ptr(x), _ptr(dx), _ptr(dp))
    return {"dx": dx, "dprobs": dp}


def sample_rows(offsets, rows):
    """Restrict a problem to a sorted subset of its rows: returns (expert of each
    row, compact offsets over the subset) so the oracle can compute just those
    rows (every row depends only on its own inputs and its expert's weights)."""
    off = np.asarray(offsets, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    if np.any(np.diff(rows) < 0):
        raise ValueError("rows must be sorted")
    E = off.shape[0] - 1
    expert = np.searchsorted(off, rows, side="right") - 1
    if np.any(expert < 0) or np.any(expert >= E) or np.any(rows >= off[-1]):
        raise ValueError("row outside the routed range")
    compact = np.zeros(E + 1, dtype=np.int64)
    np.cumsum(np.bincount(expert, minlength=E), out=compact[1:])
    return expert, compact
