#!/usr/bin/env python3
"""Benchmark of the dropless MoE layer (route + forward + backward) on one MI355X.

One step = moe_route + moe_forward + moe_backward over one batch of seeded synthetic inputs
already resident in HBM.  Prints one JSON line (the benchmark contract) with useful TFLOPS
(18 * routed_pairs * d * f flop per step), tokens/s, the fraction of the dense bf16 MFMA peak,
a roofline entry for the dominant kernel (average duration from HIP stream events recorded
around every kernel launch during the timed steps), and the fp64 CPU oracle timed on a bounded
sample of the same workload on the host cores.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config qwen3] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "MoE layer fwd+bwd useful TFLOPS and tokens/s on 1 MI355X; % MFMA peak"
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

WORKLOADS = {
    "qwen3": "Qwen3-30B-A3B-shaped MoE layer fwd+bwd: T=16384, d=2048, f=768, E=128, top-8, bf16",
    "skewed": "Qwen3-30B-A3B-shaped MoE layer fwd+bwd with Zipf-skewed routing (bias 3*ln(1/rank)), bf16",
    "mixtral": "Mixtral-8x7B-shaped MoE layer fwd+bwd: T=8192, d=4096, f=14336, E=8, top-2, bf16",
    "tiny": "tiny MoE layer: T=64, d=128, f=256, E=8, top-2, bf16",
}

# stage -> (flop per routed pair as a multiple of d*f) for the grouped GEMMs
GEMM_FLOP_PER_PAIR = {"gemm_up": 4, "gemm_down": 2, "gemm_dact": 2, "gemm_dx": 4, "gemm_dw2": 2, "gemm_dw1": 4}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stage_bytes(stage, T, d, f, E, k, A):
    """Algorithmic HBM bytes of one launch of a bandwidth-bound stage."""
    if stage in ("combine", "combine_dx"):
        return A * d * 2 + T * d * 2 + T * k * 4
    if stage == "router":
        return T * E * 4 + T * k * 8
    if stage == "plan":
        return A * 4 * 3
    if stage == "dlogits":
        return T * k * 4 * 3 + T * E * 4
    return None


def cpu_baseline(inp, n_tokens: int):
    """The fp64 oracle (route, plan, forward, backward) on the first n_tokens tokens."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    import oracle
    try:
        ncores = len(os.sched_getaffinity(0))
    except AttributeError:
        ncores = os.cpu_count() or 1
    ncores = max(1, min(16, ncores))
    n = min(n_tokens, inp.T)
    x = oracle.bf16_to_f64(inp.x[:n])
    dy = oracle.bf16_to_f64(inp.dy[:n])
    W1 = oracle.bf16_to_f64(inp.W1)
    W2 = oracle.bf16_to_f64(inp.W2)
    L = inp.logits[:n]
    with threadpool_limits(limits=ncores):
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        t0 = time.perf_counter()
        ids, w = oracle.route(L, inp.k)
        oracle.forward(x, W1, W2, ids, w)
        oracle.backward(x, W1, W2, ids, w, dy)
        dt = time.perf_counter() - t0
    A = n * inp.k
    return {"value": 18.0 * A * inp.d * inp.f / dt / 1e12, "unit": "TFLOPS", "cores": int(threads),
            "kind": "oracle", "tokens_per_s": n / dt, "seconds": dt,
            "sample": f"first {n} of {inp.T} tokens of the same workload (all {inp.E} experts), "
                      f"route+plan+forward+backward in fp64 numpy, {threads} BLAS threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="qwen3", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=2048)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this layer is one GPU's share of an expert-parallel "
              f"layer and the build has no multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import grouped_gemm_expert_router_amd as moe
    from workloads import make_config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    moe.load_library()
    t_gen = time.perf_counter()
    inp = make_config(args.config)
    log(f"[bench] generated {args.config} inputs in {time.perf_counter() - t_gen:.1f}s")
    T, d, f, E, k = inp.T, inp.d, inp.f, inp.E, inp.k
    dm = moe.dims(T, d, f, E, k)
    dev = "cuda"

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    x, W1, W2, dy = bf16(inp.x), bf16(inp.W1), bf16(inp.W2), bf16(inp.dy)
    logits = torch.from_numpy(inp.logits).to(dev)
    b = moe.alloc_layer_buffers(dm, dev, backward=True)
    torch.cuda.synchronize()

    def step():
        moe.moe_route(dm, logits, b["topk_ids"], b["topk_w"], b["counts"], b["offsets"], b["perm"], b["inv_perm"],
                      b["ws_route"])
        moe.moe_forward(dm, x, None, W1, None, W2, None, b["topk_w"], b["offsets"], b["perm"], b["inv_perm"], b["y"],
                        b["saved"], b["ws_fwd"])
        moe.moe_backward(dm, dy, x, None, W1, None, W2, None, b["topk_ids"], b["topk_w"], b["offsets"], b["perm"],
                         b["inv_perm"], b["saved"], b["dx"], b["dW1"], b["dW2"], b["d_topk_w"], b["d_logits"],
                         b["ws_bwd"])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")

    # per-kernel stream events around every launch inside the timed steps
    events = []
    open_ev = {}

    def hook(stage, begin, stream_ptr):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record()
        if begin:
            open_ev[stage] = ev
        else:
            events.append((stage, open_ev.pop(stage), ev))

    moe.moe_set_stage_hook(hook)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    moe.moe_set_stage_hook(None)
    ms = start.elapsed_time(stop) / args.steps
    log(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step")

    A = int(b["offsets"][-1].item())
    useful = 18.0 * A * d * f
    tflops = useful / (ms * 1e-3) / 1e12
    per = {}
    for stage, e0, e1 in events:
        per.setdefault(stage, []).append(e0.elapsed_time(e1))
    stages = {}
    for stage, ts in per.items():
        avg = sum(ts) / len(ts)
        ent = {"launches": len(ts), "avg_ms": avg, "ms_per_step": sum(ts) / args.steps}
        if stage in GEMM_FLOP_PER_PAIR:
            fl = GEMM_FLOP_PER_PAIR[stage] * A * d * f
            ent["tflops"] = fl / (avg * 1e-3) / 1e12
            ent["frac_mfma_peak"] = ent["tflops"] / PEAK_BF16_TFLOPS
        else:
            by = stage_bytes(stage, T, d, f, E, k, A)
            if by:
                ent["gbs"] = by / (avg * 1e-3) / 1e9
        stages[stage] = ent
    log("[bench] per-kernel: " + ", ".join(f"{s}={v['avg_ms']:.3f}ms" for s, v in
                                           sorted(stages.items(), key=lambda kv: -kv[1]["ms_per_step"])))
    dom = max(stages, key=lambda s: stages[s]["ms_per_step"])
    dom_e = stages[dom]
    if dom in GEMM_FLOP_PER_PAIR:
        fl = GEMM_FLOP_PER_PAIR[dom] * A * d * f
        achieved = fl / (dom_e["avg_ms"] * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None, "algorithmic_flop_per_launch": fl,
                "avg_launch_ms": dom_e["avg_ms"]}
    else:
        by = stage_bytes(dom, T, d, f, E, k, A)
        achieved = by / (dom_e["avg_ms"] * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": None, "algorithmic_bytes_per_launch": by,
                "avg_launch_ms": dom_e["avg_ms"]}

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle on {min(args.cpu_tokens, T)} tokens ...")
        cpu = cpu_baseline(inp, args.cpu_tokens)
        log(f"[bench] CPU oracle: {cpu['seconds']:.1f}s, {cpu['value'] * 1e3:.2f} GFLOPS, {cpu['cores']} threads")

    out = {
        "metric": METRIC, "value": tflops, "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": WORKLOADS[args.config], "T": T, "d": d, "f": f, "E": E, "k": k,
                   "routed_pairs": A, "seed_config": args.config},
        "tokens_per_s": T / (ms * 1e-3), "frac_of_bf16_peak": tflops / PEAK_BF16_TFLOPS,
        "useful_flop_per_step": useful, "stages": stages, "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
