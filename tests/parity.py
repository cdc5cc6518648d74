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
dX from dY and H1) are held to the relative-L2 bound.  The intermediates are
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


def check_chained(name: str, got, ref, rows=None) -> dict:
    """Relative-L2 bound only: for outputs whose inputs came from an earlier
    stage on each side (the per-element bound is checked stage by stage)."""
    g = bf16_to_f64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    if rows is not None:
        g, r = g[rows], r[rows]
    assert g.shape == r.shape, (name, g.shape, r.shape)
    if g.size == 0:
        return {"name": name, "n": 0}
    assert np.isfinite(g).all(), f"{name}: non-finite values in the GPU result"
    nref = np.linalg.norm(r)
    rel = np.linalg.norm(g - r) / nref if nref > 0 else np.linalg.norm(g - r)
    assert rel <= REL_L2, f"{name}: relative L2 {rel:.3e} > {REL_L2}"
    return {"name": name, "n": int(g.size), "rel_l2": float(rel), "worst_ratio": 0.0}


def stagewise(x, dy, offsets, w1, w2, h1, a, y, dh1, dx, rows=None) -> list:
    """Parity of every stage of one forward + dgrad pass.

    x, dy: CPU bf16 inputs over the compared rows (offsets index into them);
    h1, a, y, dh1, dx: the GPU outputs for the same rows (dgrad having been run
    from the GPU's own H1).  Each stage is compared per element against the
    oracle fed the GPU's bf16 input of that stage; Y and dX are also compared
    end to end (relative L2)."""
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
            check_chained("dx_chained", dx, dg["dx"], rows)]
    return out


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
            check_chained("dx_chained", dx, dg["dx"], rows)]
    if dprobs is not None:
        out.append(check("dprobs", dprobs.detach().cpu().numpy().astype(np.float64), dg["dprobs"], rows))
    return out
