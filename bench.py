#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE layer at Kimi-K2 shapes on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--gpus 1]

One step is one pass of the whole layer over one batch already resident in HBM:
moe_dispatch -> moe_grouped_swiglu (activation quantisation, grouped FP8 gate|up
GEMM with the fused silu*up requantisation, grouped FP8 down GEMM) -> moe_combine,
plus the shared expert when the workload has one. W untimed warm-up steps, then K
timed steps between two device synchronisations. Prints one JSON line.

The dominant kernel (the grouped gate|up GEMM: two thirds of the weight bytes and
flops) is timed live with HIP events the library records on its launch stream;
its algorithmic bytes per launch are the gate and up weights and block scales of
every expert the batch touches, plus the quantised activations it reads and the
quantised product it writes.

The CPU baseline is the plain oracle (test infrastructure) on a bounded sample of
the same batch, on this host's cores.

The default run measures the 256-token decode batch (the headline: tokens/s, and the gate|up
kernel against the HBM roofline) and then, in the same process and on the same resident expert
weights, the 8192-token prefill batch, reported under the key "k2_prefill_8192" with its own
step time, tokens/s, roofline record and the layer's fractions of the HBM and FP8 matrix peaks
(the metric's other half). --secondary picks another workload or none.

For the dense workload (the dense block's SwiGLU MLP) a step is that MLP over the batch, run
through the same kernels as one expert that every token visits (dense_swiglu).

With --graph the step is also captured once in a HIP graph and replayed; its time is
reported under "graph" (the headline value and the kernel timings stay eager).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 matrix peak (no sparsity)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="k2_decode_256")
    ap.add_argument("--secondary", default=None,
                    help="a second workload measured in the same process and reported under its own key "
                         "(default: k2_prefill_8192 when --config is k2_decode_256, the other half of the "
                         "metric; 'none' to skip). It reuses the resident expert weights when they are the same")
    ap.add_argument("--cpu-tokens", type=int, default=None,
                    help="rows of x in the oracle's CPU-baseline sample (default: whole batch up to "
                         "2048 * 2048 / (top_k * d_ff))")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tile", choices=["auto", "16", "128", "192", "224", "256"], default="auto",
                    help="force the grouped GEMMs' tile height (default: chosen from rows per expert)")
    ap.add_argument("--block", action="store_true",
                    help="time the FFN half of a block around the layer instead: hidden + layer(RMSNorm(hidden)), "
                         "with the RMSNorm fused into the activation quantisation and the residual addition "
                         "into the combine")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph (replays; reported under \"graph\")")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of the layer, run a plain device-to-device copy of this many bytes "
                         "(5 launches): the reference for scaling rocprofv3's HBM byte counters")
    return ap.parse_args()


def source_sha256(names) -> str:
    """sha256 over the named kernel sources (files under the package's csrc/, in order)."""
    import hashlib
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "mixture_experts_ffn_ids_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(workload: str):
    """HBM bytes per gate|up launch from the committed rocprofv3 counter summary of this
    workload (FETCH_SIZE and WRITE_SIZE, scaled by the copy calibration), or None when
    there is none or the kernel's sources (listed in the record) have changed since the
    counters were taken."""
    path = os.path.join(ROOT, "profiles", f"gate_up_{workload}.md")
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith("traffic-record:"):
                rec = dict(kv.split("=", 1) for kv in line.split()[1:])
    if not rec or "sources" not in rec:
        return None
    if rec.get("source_sha256") != source_sha256(rec["sources"].split(",")):
        return None
    kib = float(rec["fetch_kib"]) * float(rec["fetch_scale"]) + float(rec["write_kib"]) * float(rec["write_scale"])
    return int(kib * 1024)


def copy_calibration(nbytes: int):
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": 5}), flush=True)


def measure(cfg, args, dev, graph: bool):
    """Time `args.steps` steps of one workload after `args.warmup` warm-up steps. Returns the
    result fields of that workload and the host inputs the CPU baseline needs."""
    import numpy as np
    import torch

    import mixture_experts_ffn_ids_amd as moe
    from workloads import make_routing, make_x_bits
    from workloads.gen import make_experts_device, make_shared_device

    # ---- inputs, resident in HBM before timing
    x_bits = make_x_bits(cfg)
    ids, w = make_routing(cfg)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    t_ids = torch.from_numpy(ids).to(dev)
    t_w = torch.from_numpy(w).to(dev)
    experts = make_experts_device(cfg, dev)
    shared = make_shared_device(cfg, dev) if cfg.shared else None
    torch.cuda.synchronize()

    flags = {"auto": 0, "16": moe.FLAG_TILE_16, "128": moe.FLAG_TILE_128, "192": moe.FLAG_TILE_192,
             "224": moe.FLAG_TILE_224, "256": moe.FLAG_TILE_256}[args.tile]

    if args.block:
        from workloads.gen import make_block_inputs
        h_bits, g_bits = make_block_inputs(cfg)
        hidden = torch.from_numpy(h_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        gain = torch.from_numpy(g_bits.view(np.int16)).view(torch.bfloat16).to(dev)

        if cfg.dense:
            def step():
                return moe.dense_block_ffn(hidden, gain, 1e-6, experts, flags=flags)
        else:
            def step():
                return moe.moe_block_ffn(hidden, gain, 1e-6, t_ids, t_w, experts, shared, flags=flags)
    elif cfg.dense:
        def step():
            return moe.dense_swiglu(x, experts, flags=flags)
    else:
        def step():
            return moe.moe_layer(x, t_ids, t_w, experts, shared, flags=flags)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # inside the timed region only the dominant kernel's launches carry HIP events (each timed
    # launch adds two event records to the stream); the other kernels are timed afterwards
    moe.profile_reset()
    moe.profile_enable(True, kinds=[moe.KERNEL_GATE_UP])
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # an event after every step (recording one does not synchronise) gives per-step times too
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    start.record()
    for i in range(args.steps):
        out = step()
        marks[i].record()
    end.record()
    torch.cuda.synchronize()
    moe.profile_enable(False)
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    per_step = sorted([start.elapsed_time(marks[0])] +
                      [marks[i - 1].elapsed_time(marks[i]) for i in range(1, args.steps)])

    graph_result = None
    if graph:
        # the same step captured once in a HIP graph (the eager runs above sized the workspaces),
        # replayed W times untimed and K times timed
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.steps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        g_ms = g0.elapsed_time(g1) / args.steps
        graph_result = {"ms_per_step": round(g_ms, 4), "tokens_per_s": round(cfg.layer_tokens / (g_ms / 1e3), 2)}
        del graph

    def read_kernels():
        res = {}
        for name, kind in (("quant", moe.KERNEL_QUANT), ("dispatch", moe.KERNEL_DISPATCH),
                           ("gate_up", moe.KERNEL_GATE_UP), ("down", moe.KERNEL_DOWN),
                           ("combine", moe.KERNEL_COMBINE)):
            ms, n = moe.profile_read(kind)
            res[name] = {"total_ms": round(ms, 4), "launches": n, "avg_ms": round(ms / n, 5) if n else None}
        return res

    gu = read_kernels()["gate_up"]     # the dominant kernel, timed inside the timed region
    # every kernel kind, from K more steps with every launch timed (outside the timed region)
    moe.profile_reset()
    moe.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    moe.profile_enable(False)
    per_kernel = read_kernels()

    # ---- algorithmic work
    N, d, d_ff, E, K = cfg.N, cfg.d, cfg.d_ff, cfg.E, cfg.K
    touched = int((np.bincount(ids.ravel(), minlength=E) > 0).sum())
    n_sh = 1 if cfg.shared else 0
    w_proj = d * d_ff                                   # bytes of one fp8 projection
    s_proj = (d // 128) * (d_ff // 128) * 4             # its block scales
    # gate|up launches: one for the routed experts (+ one for the shared expert, which runs on a
    # second stream alongside the routed launches, so that its launch times include the overlap)
    gu_bytes_routed = touched * 2 * (w_proj + s_proj) + N * d + N * (d // 128) * 4 + N * K * d_ff + N * K * (d_ff // 128) * 4
    gu_bytes_shared = n_sh * (2 * (w_proj + s_proj) + N * d + N * (d // 128) * 4 + N * d_ff + N * (d_ff // 128) * 4)
    gu_launches_per_step = 1 + n_sh
    gu_bytes_per_launch = (gu_bytes_routed + gu_bytes_shared) / gu_launches_per_step
    gu_flops_per_launch = 2.0 * 2 * d * d_ff * (N * K + n_sh * N) / gu_launches_per_step
    gu_avg_s = gu["avg_ms"] / 1e3
    achieved_gbs = gu_bytes_per_launch / gu_avg_s / 1e9
    achieved_tflops = gu_flops_per_launch / gu_avg_s / 1e12
    layer_bytes = (touched + n_sh) * 3 * (w_proj + s_proj) + 4 * N * d + 8 * N * K + (2 * d if args.block else 0)
    layer_flops = 2.0 * 3 * d * d_ff * (N * K + n_sh * N)

    # the kernel's bound: HBM unless its arithmetic intensity is above the machine's ridge point
    mfma_bound = gu_flops_per_launch / gu_bytes_per_launch > FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(achieved_tflops, 1), "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved_tflops / FP8_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved_gbs / HBM_PEAK_GBS, 4)}
    tokens_per_s = cfg.layer_tokens / (ms_per_step / 1e3)
    result = {
        "metric": "MoE-layer tokens/s at K2 shapes; % HBM roofline (decode), % FP8 MFMA (prefill)",
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms": {"median": round(per_step[len(per_step) // 2], 4), "min": round(per_step[0], 4),
                    "max": round(per_step[-1], 4)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 x fp8-e4m3 -> fp32 (gate|up block sums on bf16 matrix ops, exact for e4m3 codes; down on fp8 ones; bf16 in/out)",
        "data": "synthetic (seeded; random-init fp8 expert weights, 128x128 block scales)",
        "config": {"workload": cfg.name, "tile": args.tile, "tokens": cfg.layer_tokens, "rows": N * K, "d": d,
                   "d_ff": d_ff, "experts": E, "top_k": K, "shared_expert": bool(cfg.shared),
                   "experts_touched": touched},
        "roofline": {**roof, "traffic": stored_traffic(cfg.name),
                     "kernel": "grouped gate|up GEMM (+silu*up requant)",
                     "algorithmic_bytes_per_launch": int(gu_bytes_per_launch),
                     "algorithmic_flops_per_launch": gu_flops_per_launch,
                     "achieved_gbs": round(achieved_gbs, 1), "achieved_tflops": round(achieved_tflops, 1),
                     "avg_launch_ms": gu["avg_ms"]},
        "layer": {"hbm_frac": round(layer_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                  "fp8_mfma_frac": round(layer_flops / (ms_per_step / 1e3) / 1e12 / FP8_PEAK_TFLOPS, 4),
                  "algorithmic_bytes": int(layer_bytes), "algorithmic_flops": layer_flops,
                  "gate_up_fp8_mfma_frac": round(achieved_tflops / FP8_PEAK_TFLOPS, 4)},
        "kernels": per_kernel,
        "kernel_timing": "roofline: HIP events around the gate|up launches inside the timed region (the only "
                         "instrumented launches there); kernels: K further steps with every launch timed",
    }

    if graph_result is not None:
        result["graph"] = graph_result
    if args.block:
        result["config"]["block"] = ("hidden + layer(RMSNorm(hidden)): the block's RMSNorm fused into the "
                                     "activation quantisation (kernel 'quant'), its residual addition into "
                                     "the combine")
    if cfg.dense:
        result["config"]["dense"] = (f"the dense block's SwiGLU MLP (intermediate size {d_ff}, an assumption: the "
                                     f"pages print none) run as one expert that every token visits; no routing "
                                     f"weights, no combine" + ("" if not args.block else " beyond the residual "
                                                               "addition"))
    if cfg.shard_topk:
        result["config"]["shard"] = (f"one GPU's part of an expert-parallel layer: {N} received rows (token "
                                     f"choices of a top-{cfg.shard_topk} router) over its {E} local experts, "
                                     f"sorted, run and put back in arrival order; tokens = rows / "
                                     f"{cfg.shard_topk}; the exchanges between GPUs are not part of the step")
    ctx = {"x_bits": x_bits, "ids": ids, "w": w, "experts": experts, "shared": shared}
    if args.block:
        ctx.update(h_bits=h_bits, g_bits=g_bits)
    del out
    return result, ctx


def cpu_baseline(cfg, args, ctx) -> dict:
    """The oracle as it stands, on a bounded sample of the same batch, on this host's cores."""
    import numpy as np

    import oracle
    from workloads.gen import experts_to_host
    x_bits, ids, w, experts, shared = (ctx[k] for k in ("x_bits", "ids", "w", "experts", "shared"))
    N, K, d_ff = cfg.N, cfg.K, cfg.d_ff
    # about 2048 evaluations of a 2048-wide expert per pass
    n_cpu = args.cpu_tokens or max(1, min(N, 2048 * 2048 // (K * d_ff)))
    tok = np.arange(n_cpu, dtype=np.int64)
    exh = experts_to_host(experts, np.unique(ids[tok]))
    shh = experts_to_host(shared) if shared is not None else None
    # every core of the affinity mask, unless OMP_NUM_THREADS asks for fewer: a host that runs
    # several GPUs' jobs gives each its share of the cores that way (16 per GPU on the MI355X
    # hosts this was measured on)
    threads = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and 0 < int(omp) < threads:
        threads = int(omp)
    used = oracle.threads_used(threads)
    # repeat the sample until about 10 s of CPU work has been timed (at most 32 passes)
    passes = 0
    t0 = time.perf_counter()
    while True:
        if args.block:
            xn = oracle.rmsnorm_rows(ctx["h_bits"][tok], ctx["g_bits"], 1e-6)
            oracle.moe_forward(xn, ids[tok], w[tok], exh, shh, threads=threads, residual=ctx["h_bits"][tok])
        else:
            oracle.moe_forward(x_bits, ids, w, exh, shh, tokens=tok, threads=threads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or passes >= 32:
            break
    per_row = cfg.layer_tokens / N                # layer tokens per row of x
    return {"value": round(passes * n_cpu * per_row / dt, 3), "unit": "tokens/s", "cores": used,
            "kind": "oracle",
            "sample": f"{passes} passes over the first {n_cpu} of the {N} rows of x in the same batch, {dt:.1f} s"}


# fields of a secondary workload's record
_SECONDARY_KEYS = ("value", "unit", "ms_per_step", "step_ms", "config", "roofline", "layer", "kernels")


def main():
    args = parse()
    if args.copy_bytes:
        copy_calibration(args.copy_bytes)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer is built and measured on a single MI355X "
              "(no sharding or collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from workloads import config_by_name

    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = config_by_name(args.config)
    result, ctx = measure(cfg, args, dev, args.graph)
    print(f"[bench] {cfg.name}: {result['ms_per_step']} ms/step", file=sys.stderr, flush=True)

    secondary = args.secondary or ("k2_prefill_8192" if cfg.name == "k2_decode_256" else "none")
    if secondary != "none":
        scfg = config_by_name(secondary)
        sres, _ = measure(scfg, args, dev, False)
        result[scfg.name] = {k: sres[k] for k in _SECONDARY_KEYS}
        result[scfg.name]["measured"] = ("in the same process after the headline workload, with the same "
                                         "warm-up and step counts and the same timing")
        print(f"[bench] {scfg.name}: {sres['ms_per_step']} ms/step", file=sys.stderr, flush=True)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, args, ctx)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
