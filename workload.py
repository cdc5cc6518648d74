"""Seeded synthetic workloads for the frozen MoE expert grouped GEMM.

This module draws inputs and nothing else: per-expert routed-row counts, the
int64 offsets array, frozen bf16 expert weights and bf16 activations.  It
holds none of the method's arithmetic, so both the CPU oracle and the HIP
path may take their inputs from here.

Shapes and distributions follow the workloads the method is used on (the
Megatron-LM pull request "perf(moe): add frozen grouped GEMM for adapter
training", section "Why this change": 128 local frozen experts, bias-free
BF16 weights; section "B200 throughput evidence": a 32k dynamic token cap;
the TE device-metadata pull request, section "Summary": 256-row per-expert
padding).  All draws are synthetic: the production token batch and the
trained checkpoint those pages measure on are stood in for by normals of the
stated scale.

Layouts (row-major):
  W1[e]  [2F, H]   rows 0..F-1 gate, F..2F-1 up (non-interleaved)
  W2[e]  [H, F]
  X, dY  [M, H]    rows sorted by expert, expert e owns [off[e], off[e+1])
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "by_name", "draw_counts", "offsets_from_counts",
           "draw_case", "custom_case", "Case"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    E: int            # local experts
    T: int            # tokens
    topk: int         # experts per token
    H: int            # hidden size (FC1 in, FC2 out)
    F: int            # FFN width per expert (FC1 out = 2F gated)
    routing: str      # multinomial | uniform | zipf | poisson
    seed: int
    forced_zero: Sequence[int] = ()   # experts forced to 0 rows (explicit ids)
    n_forced_zero: int = 0            # number of experts forced to 0 (seeded choice)
    zipf_s: float = 1.2
    poisson_mean: float = 24.0
    pad_to: int = 1                   # pad each expert's rows up to a multiple of this
    w_std: float = 0.02


WORKLOADS = [
    Workload("tiny_e4_h64_f128", E=4, T=256, topk=2, H=64, F=128,
             routing="multinomial", seed=1000, forced_zero=(2,)),
    Workload("uniform_e32_h2048_f768", E=32, T=4096, topk=8, H=2048, F=768,
             routing="uniform", seed=1001),
    Workload("zipf_e128_h2048_f768", E=128, T=16384, topk=8, H=2048, F=768,
             routing="zipf", seed=1002, n_forced_zero=10, zipf_s=1.2),
    Workload("padded_e128_h4096_f2048", E=128, T=32768, topk=8, H=4096, F=2048,
             routing="uniform", seed=1003, pad_to=256),
    Workload("smallbatch_e128_h2688_f1856", E=128, T=512, topk=6, H=2688, F=1856,
             routing="poisson", seed=1004, n_forced_zero=8, poisson_mean=24.0),
]


def by_name(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def _gen(seed: int, stream: int) -> torch.Generator:
    return torch.Generator().manual_seed(seed * 1009 + stream)


def _gumbel_topk_counts(logp: np.ndarray, T: int, k: int, g: torch.Generator,
                        chunk: int = 4096) -> np.ndarray:
    """Each of T tokens picks k distinct experts (Gumbel-top-k over log-weights)."""
    E = logp.shape[0]
    counts = np.zeros(E, dtype=np.int64)
    lp = torch.from_numpy(logp.astype(np.float64))
    for t0 in range(0, T, chunk):
        n = min(chunk, T - t0)
        u = torch.rand(n, E, generator=g, dtype=torch.float64).clamp_(1e-300, 1.0)
        keys = lp.unsqueeze(0) - torch.log(-torch.log(u))
        top = torch.topk(keys, k, dim=1).indices.reshape(-1).numpy()
        counts += np.bincount(top, minlength=E)
    return counts


def draw_counts(w: Workload) -> np.ndarray:
    """Real (unpadded) routed rows per expert, int64 [E]."""
    g = _gen(w.seed, 0)
    E = w.E
    zero = np.zeros(E, dtype=bool)
    zero[list(w.forced_zero)] = True
    if w.n_forced_zero:
        perm = torch.randperm(E, generator=g).numpy()
        if w.routing == "zipf":
            pass  # the lowest-ranked experts are zeroed below
        else:
            zero[perm[:w.n_forced_zero]] = True
    if w.routing == "multinomial":
        live = np.flatnonzero(~zero)
        p = torch.zeros(E, dtype=torch.float64)
        p[torch.from_numpy(live)] = 1.0
        picks = torch.multinomial(p, w.T * w.topk, replacement=True, generator=g).numpy()
        return np.bincount(picks, minlength=E).astype(np.int64)
    if w.routing == "uniform":
        logp = np.zeros(E)
        logp[zero] = -np.inf
        return _gumbel_topk_counts(logp, w.T, w.topk, g)
    if w.routing == "zipf":
        rank_of = torch.randperm(E, generator=g).numpy()        # expert -> rank 0..E-1
        logp = -w.zipf_s * np.log(rank_of + 1.0)
        logp[rank_of >= E - w.n_forced_zero] = -np.inf           # lowest-ranked forced to 0
        logp[zero] = -np.inf
        return _gumbel_topk_counts(logp, w.T, w.topk, g)
    if w.routing == "poisson":
        lam = torch.full((E,), float(w.poisson_mean), dtype=torch.float64)
        c = torch.poisson(lam, generator=g).numpy().astype(np.int64)
        c[zero] = 0
        return c
    raise ValueError(w.routing)


def offsets_from_counts(counts: np.ndarray, pad_to: int = 1) -> np.ndarray:
    c = np.asarray(counts, dtype=np.int64)
    if pad_to > 1:
        c = (c + pad_to - 1) // pad_to * pad_to
    off = np.zeros(c.shape[0] + 1, dtype=np.int64)
    np.cumsum(c, out=off[1:])
    return off


def _normal_bf16(shape, std: float, g: torch.Generator, chunk_elems: int = 1 << 26) -> torch.Tensor:
    """N(0, std^2) drawn in fp32, rounded to bf16 (round-to-nearest-even)."""
    out = torch.empty(shape, dtype=torch.bfloat16)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        v = torch.randn(e - s, generator=g, dtype=torch.float32)
        if std != 1.0:
            v.mul_(std)
        flat[s:e] = v.to(torch.bfloat16)
    return out


@dataclasses.dataclass
class Case:
    """One drawn problem; all tensors on the CPU, bf16 unless stated."""
    name: str
    E: int
    H: int
    F: int
    T: int
    counts: np.ndarray      # real rows per expert (int64 [E])
    offsets: np.ndarray     # int64 [E+1], padded segments
    w1: torch.Tensor        # [E, 2F, H]
    w2: torch.Tensor        # [E, H, F]
    x: torch.Tensor         # [M, H]   zero rows in padding
    dy: torch.Tensor        # [M, H]   zero rows in padding

    @property
    def M(self) -> int:
        return int(self.offsets[-1])


def _rows_with_padding(M: int, H: int, counts, offsets, std: float, g) -> torch.Tensor:
    x = _normal_bf16((M, H), std, g)
    padded = np.diff(offsets) != np.asarray(counts)
    for e in np.flatnonzero(padded):
        x[int(offsets[e]) + int(counts[e]):int(offsets[e + 1])] = 0
    return x


def draw_case(w: Workload, with_dy: bool = True) -> Case:
    counts = draw_counts(w)
    off = offsets_from_counts(counts, w.pad_to)
    M = int(off[-1])
    w1 = _normal_bf16((w.E, 2 * w.F, w.H), w.w_std, _gen(w.seed, 1))
    w2 = _normal_bf16((w.E, w.H, w.F), w.w_std, _gen(w.seed, 2))
    x = _rows_with_padding(M, w.H, counts, off, 1.0, _gen(w.seed, 3))
    dy = (_rows_with_padding(M, w.H, counts, off, 1.0, _gen(w.seed, 4)) if with_dy
          else torch.empty(0, w.H, dtype=torch.bfloat16))
    return Case(w.name, w.E, w.H, w.F, w.T, counts, off, w1, w2, x, dy)


def custom_case(counts: Sequence[int], H: int, F: int, seed: int, pad_to: int = 1,
                w_std: float = 0.02, x_std: float = 1.0, name: Optional[str] = None) -> Case:
    """A case with explicit per-expert counts (edge-case and sweep tests)."""
    counts = np.asarray(counts, dtype=np.int64)
    E = counts.shape[0]
    off = offsets_from_counts(counts, pad_to)
    M = int(off[-1])
    w1 = _normal_bf16((E, 2 * F, H), w_std, _gen(seed, 1))
    w2 = _normal_bf16((E, H, F), w_std, _gen(seed, 2))
    x = _rows_with_padding(M, H, counts, off, x_std, _gen(seed, 3))
    dy = _rows_with_padding(M, H, counts, off, 1.0, _gen(seed, 4))
    return Case(name or f"custom_e{E}_h{H}_f{F}_s{seed}", E, H, F, int(counts.sum()),
                counts, off, w1, w2, x, dy)


def flops_fwd_dgrad(M: int, H: int, F: int) -> float:
    """Dense multiply-add work of forward (FC1 + FC2) plus dgrad, 2 flops per MAC."""
    return 12.0 * M * H * F


if __name__ == "__main__":
    for w in WORKLOADS:
        c = draw_counts(w)
        off = offsets_from_counts(c, w.pad_to)
        nz = int((c == 0).sum())
        print(f"{w.name}: M={int(off[-1])} real={int(c.sum())} empty={nz} "
              f"max={int(c.max())} min_nonzero={int(c[c > 0].min())}")
