"""Parity helpers shared by the GPU tests (tests only).

The bar: relative L2 ||gpu - ref|| / ||ref|| <= 2e-3 and, per element,
|gpu - ref| <= 1e-2 * |ref| + 1e-3, both in float64 over every compared
element.  Any fp32 summation order is a correct result, so parity of the
floating-point outputs is tolerance-based; integer/index work (which rows are
written) is compared exactly.
"""
from __future__ import annotations

import numpy as np
import torch

REL_L2 = 2e-3
ELEM_REL = 1e-2
ELEM_ABS = 1e-3


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float32).numpy().astype(np.float64)


def check(name: str, got, ref, rows=None) -> dict:
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
    bound = ELEM_REL * np.abs(r) + ELEM_ABS
    ratio = diff / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    info = {"name": name, "n": int(g.size), "rel_l2": float(rel), "worst_ratio": float(ratio[worst]),
            "exact_frac": float(np.mean(diff == 0))}
    assert rel <= REL_L2, f"{name}: relative L2 {rel:.3e} > {REL_L2} ({info})"
    assert ratio[worst] <= 1.0, (f"{name}: element {worst} got {g[worst]} ref {r[worst]} "
                                 f"exceeds |d| <= 1e-2|ref| + 1e-3 ({info})")
    return info
