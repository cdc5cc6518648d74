"""Benchmark of the frozen MoE expert grouped GEMM (forward FC1 -> SwiGLU -> FC2
plus the input gradient) on one MI355X.

One step = gg_forward_fc1_swiglu (saving H1) + gg_forward_fc2 + gg_dgrad
over one synthetic batch that is already resident in HBM.  Before every step
(warm-up and timed) a 1 GiB scratch buffer is written and another 1 GiB read,
outside the timed events, so that no operand is left in the 256 MiB MALL or
the L2 from the step before and no dirty line of the write is left for the
step to write back.  Each call is timed with HIP events on the launch stream; the step
time is the median over the timed steps (the minimum is reported beside it).

Prints ONE JSON line: grouped-GEMM TFLOP/s (12*M*H*F per step), routed
rows/s, tokens/s, the roofline record of the dominant kernel (the FC1 grouped
GEMM), the device, its clocks and the ROCm version, the parity of the run's
GPU outputs against the CPU oracle on a sample of rows, and the CPU oracle
timed on that sample.  The default workload is the largest one that fits one
GPU: 128 experts, 32768 tokens x top-8 (each expert's rows padded up to a
multiple of 256), hidden 4096, FFN 2048.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--layout auto|frag|packed]
                    [--activation swiglu|qgeglu] [--weighted | --probs-on-input] [--recompute]

Weights: the packed buffer alone (6*E*H*F bytes, the library's default) and,
for shapes with H % 256 == 0 and F % 128 == 0, also with the opt-in
fragment-ordered copies (gg_pack_frag, 12*E*H*F more bytes), which the
extended calls take to run the GEMMs in the four-wave kernel.  With
--layout auto both are timed, the same steps each; the line's headline is
the copies' arm (the faster), and "layouts" gives both.

--activation / --weighted time the QuickGeGLU and router-probability-weighted
variants (gg_forward_fc1_glu + gg_forward_fc2 + gg_dgrad_glu, dprobs
included); --recompute keeps no H1 and recomputes FC1 inside the dgrad call
(gg_dgrad_recompute; the step's counted work stays 12*M*H*F).
--probs-on-input scales the FC1 input rows by the router probabilities
instead (gg_scale_rows before FC1 and gg_scale_rows_backward after the
input gradient, both timed in the step; their HBM rooflines are in
roofline.row_scaling).  The default line is plain SwiGLU with a saved H1.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "grouped-GEMM TFLOP/s + routed tokens/s (fwd+dgrad), % of MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
DEFAULT_WORKLOAD = "padded_e128_h4096_f2048"
FLUSH_BYTES = 1 << 30          # > MALL (256 MiB) + all L2s: written before every step
KERNEL_SOURCES = ["moe_expert_grouped_ragged_amd/csrc/gg_kernels.hip",
                  "moe_expert_grouped_ragged_amd/csrc/gg_kernels.h",
                  "moe_expert_grouped_ragged_amd/csrc/gg_api.cpp"]   # which kernels a call launches


def kernel_source_hash() -> str:
    """sha256 (16 hex digits) of the kernel and launch sources with their
    comments removed and whitespace collapsed, so that a measurement keyed by
    it goes stale when the code changes but not when only a comment or the
    layout does (the sources hold no string literal with a comment marker)."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(M, H, F, n_live):
    """Forward and dgrad algorithmic HBM bytes (weights of non-empty experts
    read once per pass; activations read/written once)."""
    w_act = 6 * H * F * n_live
    fwd = w_act + 4 * M * H + 8 * M * F
    dgrad = w_act + 4 * M * H + 12 * M * F
    return fwd, dgrad


def load_traffic(workload_name: str, kernel: str):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE,
    stored in profiles/traffic.json; null when the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload_name, {}).get(kernel)
    if not ent or ent.get("kernel_source_sha") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(case, target_s: float, act: str = "swiglu", probs=None, probs_in=None):
    """The CPU oracle, as it stands, on the first k rows of every non-empty
    expert (k calibrated to about target_s seconds of work).  probs weights
    the activation; probs_in instead scales the FC1 input rows (the scale and
    its gradient then run around the plain path)."""
    import numpy as np
    import torch

    import oracle
    threads = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        threads = min(threads, int(os.environ["OMP_NUM_THREADS"]))
    oracle.set_threads(threads)
    w1 = oracle._as_f32(case.w1)
    w2 = oracle._as_f32(case.w2)
    off = case.offsets
    live = [e for e in range(case.E) if off[e + 1] > off[e]]

    result = {}

    def run(k):
        rows = np.concatenate([np.arange(off[e], min(off[e] + k, off[e + 1])) for e in live]).astype(np.int64)
        _, comp = oracle.sample_rows(off, rows)
        xs = case.x[torch.from_numpy(rows)]
        dys = case.dy[torch.from_numpy(rows)]
        t0 = time.perf_counter()
        if probs_in is not None:
            pin = probs_in[rows]
            fw = oracle.forward(oracle.scale_rows(xs, pin), comp, w1, w2)
            dg = oracle.dgrad(dys, fw["h1"], comp, w1, w2)
            dg = {"dx": oracle.scale_rows_backward(dg["dx"], xs, pin)["dx"]}
        elif act == "swiglu" and probs is None:
            fw = oracle.forward(xs, comp, w1, w2)
            dg = oracle.dgrad(dys, fw["h1"], comp, w1, w2)
        else:
            pr = None if probs is None else probs[rows]
            fw = oracle.forward_glu(xs, comp, w1, w2, act, pr)
            dg = oracle.dgrad_glu(dys, fw["h1"], comp, w1, w2, act, pr)
        t = time.perf_counter() - t0
        result.update(rows=rows, y=fw["y"], dx=dg["dx"])
        return rows.size, t

    # grow the sample until one run takes about target_s (small samples
    # under-use the threads, so a single extrapolation undershoots)
    cap = int(np.max(np.diff(off)))
    k = 4
    while True:
        n, t = run(k)
        if t >= 0.6 * target_s or k >= cap:
            break
        k = min(cap, max(k + 1, int(k * min(8.0, 0.9 * target_s / max(t, 1e-3)))))
    flops = 12.0 * n * case.H * case.F
    rec = {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"first {k} rows of each of the {len(live)} non-empty experts ({n} routed rows "
                     f"of {case.M}), forward + dgrad, {t:.1f} s",
           "rows_per_s": n / t, "seconds": t}
    return rec, result


def parity_of_sample(sample, y_gpu, dx_gpu):
    """End-to-end parity of the run's GPU outputs on the oracle's sample rows:
    Y from X and dX from dY (each side from its own forward), per element
    against |d| <= 1e-2 |ref| + 1e-3 and in relative L2, in float64."""
    import numpy as np
    import torch
    rows = torch.from_numpy(sample["rows"])
    out = {}
    for name, got, ref in (("y", y_gpu, sample["y"]), ("dx", dx_gpu, sample["dx"])):
        g = got[rows.to(got.device)].float().cpu().numpy().astype(np.float64)
        r = np.asarray(ref, np.float64)
        d = np.abs(g - r)
        ratio = d / (1e-2 * np.abs(r) + 1e-3)
        out[name] = {"rel_l2": float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)),
                     "worst_ratio": float(ratio.max()), "over_bound": int((ratio > 1.0).sum()),
                     "elements": int(r.size), "exact_frac": float(np.mean(d == 0))}
    out["rows"] = int(rows.numel())
    out["bar"] = ("end to end, each side from its own forward: rel_l2 <= 2e-3; the per-element bound "
                  "|d| <= 1e-2|ref| + 1e-3 holds stage by stage (given the same bf16 input of the last "
                  "rounding) and is counted here, where one-ulp flips of intermediate bf16 values on "
                  "either side can exceed it")
    return out


def query_clocks():
    """The device clocks as rocm-smi reports them.  Called before this process
    initialises the GPU (a process that has must not start other programs);
    skipped under a profiler, whose preloaded library initialises the GPU in
    every child process."""
    import subprocess
    if any(k.startswith(("ROCPROF", "ROCP_")) for k in os.environ):
        return "not queried (running under a profiler)"
    try:
        proc = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=30)
        card = next(iter(json.loads(proc.stdout).values()))
        return {k: v for k, v in card.items()
                if "clock" in k.lower() or k.lower().startswith(("sclk", "mclk", "fclk", "socclk"))}
    except Exception as exc:   # a missing or silent rocm-smi must not fail the benchmark
        return f"unavailable ({type(exc).__name__})"


def device_record(dev, clocks):
    """Device name, architecture, clocks (queried before the run) and the
    ROCm / HIP versions."""
    import torch
    prop = torch.cuda.get_device_properties(dev)
    rec = {"name": prop.name, "arch": getattr(prop, "gcnArchName", None),
           "compute_units": prop.multi_processor_count, "hip_runtime": torch.version.hip, "clocks": clocks}
    try:
        with open("/opt/rocm/.info/version") as fh:
            rec["rocm"] = fh.read().strip()
    except OSError:
        rec["rocm"] = None
    return rec


def launch_ab(gg, case, x, dy, off, packed, h1, a, y, ws, dx, stream, args):
    """Step time (forward + dgrad) on the same data: one persistent launch per
    GEMM (the library as shipped) against one launch per expert and GEMM (E = 1
    calls on each expert's rows and packed weights, the split known on the
    host), each issued from Python and as a HIP-graph replay (the replay
    removes the host launch cost and leaves the kernels' own)."""
    import numpy as np
    import torch
    E, H, F = case.E, case.H, case.F
    off_h = case.offsets
    per = gg.packed_bytes(1, H, F) // 2     # elements of one expert block
    live = [e for e in range(E) if off_h[e + 1] > off_h[e]]
    one = {e: torch.tensor([0, int(off_h[e + 1] - off_h[e])], dtype=torch.int64, device=x.device) for e in live}

    def grouped():
        gg.gg_forward_fc1_swiglu(x, off, packed, E, H, F, h1_out=h1, a_out=a)
        gg.gg_forward_fc2(a, off, packed, E, H, F, y=y)
        gg.gg_dgrad(dy, h1, off, packed, E, H, F, workspace=ws, dx=dx)

    def per_expert():
        for e in live:
            s0, s1 = int(off_h[e]), int(off_h[e + 1])
            pk = packed[e * per:(e + 1) * per]
            gg.gg_forward_fc1_swiglu(x[s0:s1], one[e], pk, 1, H, F, h1_out=h1[s0:s1], a_out=a[s0:s1])
            gg.gg_forward_fc2(a[s0:s1], one[e], pk, 1, H, F, y=y[s0:s1])
            gg.gg_dgrad(dy[s0:s1], h1[s0:s1], one[e], pk, 1, H, F, workspace=ws[s0:s1], dx=dx[s0:s1])

    def timed(fn, n):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n

    ms_grouped = timed(grouped, args.steps)
    ms_per_expert = timed(per_expert, args.steps)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        grouped()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        grouped()
    ms_graph = timed(graph.replay, args.steps)
    # the per-expert loop captured as well: no host launch cost left, only the
    # per-expert kernels themselves
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        per_expert()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph_pe = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_pe):
        per_expert()
    ms_graph_pe = timed(graph_pe.replay, args.steps)
    M = case.M
    return {"launch_ab": {"workload": args.workload, "experts_with_rows": len(live),
                          "launches_per_step": {"grouped": 4, "per_expert": 4 * len(live)},
                          "ms_per_step": {"grouped": ms_grouped, "per_expert": ms_per_expert,
                                          "grouped_graph_replay": ms_graph,
                                          "per_expert_graph_replay": ms_graph_pe},
                          "tokens_per_s": {"grouped": case.T / (ms_grouped * 1e-3),
                                           "per_expert": case.T / (ms_per_expert * 1e-3),
                                           "grouped_graph_replay": case.T / (ms_graph * 1e-3),
                                           "per_expert_graph_replay": case.T / (ms_graph_pe * 1e-3)},
                          "speedup_grouped_vs_per_expert": ms_per_expert / ms_grouped,
                          "speedup_grouped_vs_per_expert_both_replayed": ms_graph_pe / ms_graph,
                          "routed_rows": M, "steps": args.steps, "warmup": args.warmup}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--launch-ab", action="store_true",
                    help="instead of the benchmark line, compare one grouped launch per GEMM with one "
                         "launch per expert (the same library, E=1 calls) and with a HIP-graph replay "
                         "of the grouped step; prints one JSON line")
    ap.add_argument("--activation", choices=("swiglu", "qgeglu"), default="swiglu",
                    help="gated activation of the FC1 epilogue (gg_forward_fc1_glu / gg_dgrad_glu "
                         "for anything but plain SwiGLU)")
    ap.add_argument("--weighted", action="store_true",
                    help="weight the activation by a per-row router probability (fp32, seeded "
                         "uniform in [0.05, 1)) and return its gradient dprobs from the dgrad")
    ap.add_argument("--probs-on-input", action="store_true",
                    help="router probabilities scale the FC1 input rows (gg_scale_rows before FC1, "
                         "gg_scale_rows_backward after the input gradient, both in the step) instead of "
                         "weighting the activation")
    ap.add_argument("--recompute", action="store_true",
                    help="forward without saving H1 and input gradient through gg_dgrad_recompute "
                         "(FC1 recomputed from X inside the dgrad call)")
    ap.add_argument("--layout", choices=("auto", "frag", "packed"), default="auto",
                    help="weights: 'packed' = the packed buffer alone (the library's default); 'frag' = with "
                         "the opt-in fragment-ordered copies (gg_pack_frag); 'auto' = both where the shape "
                         "has copies, the line's headline being 'frag'")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB five times "
                         "(calibrates the FETCH_SIZE / WRITE_SIZE counters), then exit")
    args = ap.parse_args()

    if args.weighted and args.probs_on_input:
        print("bench.py: --weighted and --probs-on-input are alternatives", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this path runs on one GPU only (no sharding or collectives are part of it); "
              "use --gpus 1", file=sys.stderr)
        sys.exit(2)

    clocks = query_clocks() if not args.copy_probe_mib else None   # before the GPU is initialised

    import numpy as np
    import torch

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)
        return

    import workload
    import moe_expert_grouped_ragged_amd as gg

    w = workload.by_name(args.workload)
    case = workload.draw_case(w)
    E, H, F, M = case.E, case.H, case.F, case.M
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x, dy = case.x.to(dev), case.dy.to(dev)
    off = torch.from_numpy(case.offsets).to(dev)
    packed = gg.gg_pack_weights(case.w1.to(dev), case.w2.to(dev))
    # weight layouts timed: the packed buffer alone (the default), and with the
    # opt-in fragment-ordered copies where the shape has them; the headline is
    # the first of them
    if args.layout == "auto":
        arms = ["frag", "packed"] if gg.has_frag(H, F) else ["packed"]
    else:
        arms = [args.layout]
    if "frag" in arms and not gg.has_frag(H, F):
        print(f"bench.py: H={H}, F={F} has no fragment-ordered copies", file=sys.stderr)
        sys.exit(2)
    frag = gg.gg_pack_frag(packed, E, H, F) if "frag" in arms else None
    h1 = torch.empty(M, 2 * F, dtype=torch.bfloat16, device=dev)
    a = torch.empty(M, F, dtype=torch.bfloat16, device=dev)
    y = torch.empty(M, H, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(M, 2 * F, dtype=torch.bfloat16, device=dev)
    dx = torch.empty(M, H, dtype=torch.bfloat16, device=dev)
    glu = args.activation != "swiglu" or args.weighted or args.recompute
    with_probs = args.weighted or args.probs_on_input
    probs_np = (np.random.default_rng(w.seed + 17).uniform(0.05, 1.0, M).astype(np.float32)
                if with_probs else None)
    probs_all = torch.from_numpy(probs_np).to(dev) if with_probs else None
    probs = probs_all if args.weighted else None          # at the activation
    dprobs = torch.empty(M, dtype=torch.float32, device=dev) if with_probs else None
    # probabilities on the input: the scaled rows and the gradient at them
    xs = torch.empty(M, H, dtype=torch.bfloat16, device=dev) if args.probs_on_input else None
    dxs = torch.empty(M, H, dtype=torch.bfloat16, device=dev) if args.probs_on_input else None
    x_in = xs if args.probs_on_input else x
    dx_mlp = dxs if args.probs_on_input else dx
    ws_glu = torch.empty(gg.dgrad_glu_workspace_bytes(M, F, args.weighted), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step(arm, ev):
        fr = frag if arm == "frag" else None
        if args.probs_on_input:
            if ev is not None:
                s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s0.record(stream)
            gg.gg_scale_rows(x, probs_all, out=xs)
            if ev is not None:
                s1.record(stream)
                ev["scale_rows"].append((s0, s1))
        if ev is not None:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e2 = torch.cuda.Event(enable_timing=True)
            e3 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        if args.recompute:
            gg.gg_forward_fc1_glu(x_in, off, packed, E, H, F, args.activation, probs, save_h1=False, a_out=a,
                                  frag=fr)
        elif glu or fr is not None:
            gg.gg_forward_fc1_glu(x_in, off, packed, E, H, F, args.activation, probs, h1_out=h1, a_out=a, frag=fr)
        else:
            gg.gg_forward_fc1_swiglu(x_in, off, packed, E, H, F, h1_out=h1, a_out=a)
        if ev is not None:
            e1.record(stream)
        if fr is None:
            gg.gg_forward_fc2(a, off, packed, E, H, F, y=y)
        else:
            gg.gg_forward_fc2_frag(a, off, packed, fr, E, H, F, y=y)
        if ev is not None:
            e2.record(stream)
        if args.recompute:
            gg.gg_dgrad_recompute(dy, x_in, off, packed, E, H, F, args.activation, probs,
                                  want_dprobs=args.weighted, workspace=ws_glu, dx=dx_mlp,
                                  dprobs=dprobs if args.weighted else None, frag=fr)
        elif glu or fr is not None:
            gg.gg_dgrad_glu(dy, h1, off, packed, E, H, F, args.activation, probs,
                            want_dprobs=args.weighted, workspace=ws_glu, dx=dx_mlp,
                            dprobs=dprobs if args.weighted else None, frag=fr)
        else:
            gg.gg_dgrad(dy, h1, off, packed, E, H, F, workspace=ws, dx=dx_mlp)
        if ev is not None:
            e3.record(stream)
            ev["fc1"].append((e0, e1))
            ev["fc2"].append((e1, e2))
            ev["dgrad"].append((e2, e3))
        if args.probs_on_input:
            if ev is not None:
                b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                b0.record(stream)
            gg.gg_scale_rows_backward(dxs, x, probs_all, dx=dx, dprobs=dprobs)
            if ev is not None:
                b1.record(stream)
                ev["scale_rows_bwd"].append((b0, b1))

    if args.launch_ab:
        print(json.dumps(launch_ab(gg, case, x, dy, off, packed, h1, a, y, ws, dx, stream, args)), flush=True)
        return

    # a scratch buffer larger than the MALL and all L2s, written before every
    # step outside the timed events, so that each step starts cold; a read of a
    # second one follows, so that the write's dirty lines are written back
    # before the step (else the first kernel pays for that write-back)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    flush_rd = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    sink = torch.empty((), dtype=torch.int64, device=dev)

    def evict(i):
        flush.fill_(i & 0xFF)
        torch.sum(flush_rd, dim=0, dtype=torch.int64, out=sink)

    def timed_arm(arm):
        ev = {k: [] for k in ("fc1", "fc2", "dgrad") + (("scale_rows", "scale_rows_bwd") if args.probs_on_input
                                                         else ())}
        for i in range(args.warmup):
            evict(i)
            step(arm, None)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            evict(i)
            step(arm, ev)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps          # includes the evictions
        per_step = {k: np.array([s.elapsed_time(e) for s, e in v]) for k, v in ev.items()}
        steps_ms = sum(per_step.values())
        return {"ms_per_step": float(np.median(steps_ms)), "ms_per_step_min": float(np.min(steps_ms)),
                "wall_ms_per_step_incl_eviction": wall_ms,
                "per_call_ms": {k: float(np.median(v)) for k, v in per_step.items()},
                "per_call_min_ms": {k: float(np.min(v)) for k, v in per_step.items()}}

    # the headline arm last, so that the outputs left in y and dx are its own
    results = {arm: timed_arm(arm) for arm in reversed(arms)}
    head = results[arms[0]]
    ms, wall_ms = head["ms_per_step"], head["wall_ms_per_step_incl_eviction"]
    call_ms, call_min_ms = head["per_call_ms"], head["per_call_min_ms"]
    steps_min = head["ms_per_step_min"]

    flops = workload.flops_fwd_dgrad(M, H, F)
    tflops = flops / (ms * 1e-3) / 1e12
    n_live = int(np.count_nonzero(np.diff(case.offsets)))
    bfwd, bdg = algorithmic_bytes(M, H, F, n_live)
    # dominant kernel: the FC1 grouped GEMM with the SwiGLU epilogue (the
    # largest share of the step), one launch per FC1 call: the four-wave
    # kernel with the fragment-ordered weight copies, else the eight-wave
    # kernel.
    # Algorithmic work per launch: 4*M*H*F FLOPs; HBM bytes = X read (2MH) +
    # W1 of the experts with rows (4HF each) + H1 and A written (4MF + 2MF).
    # The bound is whichever of MFMA time and HBM time is larger.
    fc1_flops = 4.0 * M * H * F
    fc1_bytes = 2.0 * M * H + 4.0 * H * F * n_live + 6.0 * M * F
    fc1_ms = call_ms["fc1"]
    kname = "tile4_kernel<SwiGLU>" if arms[0] == "frag" else "grouped_gemm_kernel<FC1+SwiGLU>"
    mfma_bound = fc1_flops / (PEAK_BF16_TFLOPS * 1e12) >= fc1_bytes / (PEAK_HBM_GBS * 1e9)
    if mfma_bound:
        achieved = fc1_flops / (fc1_ms * 1e-3) / 1e12
        roof = {"kernel": kname, "bound": "mfma", "achieved": achieved,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS}
    else:
        achieved = fc1_bytes / (fc1_ms * 1e-3) / 1e9
        roof = {"kernel": kname, "bound": "hbm", "achieved": achieved,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS}
    roof.update({"traffic": None if glu else load_traffic(args.workload, f"fc1_{arms[0]}"),
                 "median_launch_ms": fc1_ms, "min_launch_ms": call_min_ms["fc1"],
                 "flops_per_launch": fc1_flops, "algorithmic_bytes_per_launch": fc1_bytes})
    if args.probs_on_input:
        # the two row-scaling kernels are bound by HBM: the scale reads x and
        # probs and writes x' (4MH + 4M bytes); its gradient reads dx' and x
        # and probs and writes dx and dprobs (6MH + 8M bytes)
        rows_bytes = {"scale_rows": 4.0 * M * H + 4.0 * M, "scale_rows_bwd": 6.0 * M * H + 8.0 * M}
        roof["row_scaling"] = {
            k: {"bound": "hbm", "algorithmic_bytes_per_launch": b, "median_launch_ms": call_ms[k],
                "achieved": b / (call_ms[k] * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": b / (call_ms[k] * 1e-3) / 1e9 / PEAK_HBM_GBS}
            for k, b in rows_bytes.items()}
    out = {
        "metric": METRIC, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "experts": E, "tokens": case.T, "topk": w.topk,
                   "routed_rows": M, "real_rows": int(case.counts.sum()), "hidden": H, "ffn": F,
                   "routing": w.routing, "pad_to": w.pad_to,
                   "parallelism": "single-gpu", "activation": args.activation,
                   "weighted": bool(args.weighted), "probs_on_input": bool(args.probs_on_input),
                   "recompute_fc1_in_dgrad": bool(args.recompute),
                   "weights": ("packed buffer (6*E*H*F bytes) + opt-in fragment-ordered copies (12*E*H*F bytes)"
                               if arms[0] == "frag" else "packed buffer (6*E*H*F bytes)")},
        "timing": "median over the timed steps of HIP-event step times on the launch stream; a 1 GiB "
                  "scratch write and a 1 GiB read before every step (outside the events) evict the MALL and L2",
        "ms_per_step_min": steps_min,
        "wall_ms_per_step_incl_eviction": wall_ms,
        "routed_rows_per_s": M / (ms * 1e-3), "tokens_per_s": case.T / (ms * 1e-3),
        "real_rows_tflops": 12.0 * int(case.counts.sum()) * H * F / (ms * 1e-3) / 1e12,
        "mfma_frac": tflops / PEAK_BF16_TFLOPS,
        "hbm_GBps_algorithmic": (bfwd + bdg) / (ms * 1e-3) / 1e9,
        "hbm_frac": (bfwd + bdg) / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "per_call_ms": call_ms,
        "per_call_min_ms": call_min_ms,
        "layouts": {arm: dict(r, tflops=flops / (r["ms_per_step"] * 1e-3) / 1e12) for arm, r in results.items()},
        "roofline": roof,
        "kernel_source_sha": kernel_source_hash(),
        "device": device_record(dev, clocks),
    }
    if not args.no_cpu_baseline:
        rec, sample = cpu_baseline(case, args.cpu_seconds, args.activation,
                                   probs_np if args.weighted else None,
                                   probs_np if args.probs_on_input else None)
        out["cpu_baseline"] = rec
        out["parity"] = parity_of_sample(sample, y, dx)
    else:
        out["cpu_baseline"] = None
        out["parity"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
