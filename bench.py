#!/usr/bin/env python3
"""Benchmark of the dropless MoE layer (route or plan + forward + backward) on one MI355X.

One step = moe_route (moe_plan for pre-routed input) + moe_forward + moe_backward over one
batch of seeded synthetic inputs already resident in HBM.  Prints one JSON line with useful
TFLOPS (18 * routed_pairs * d * f flop per step), tokens/s, the fraction of the dense MFMA
peak, a roofline entry for the dominant kernel (average duration from HIP events recorded on
the launch stream around every kernel during the timed steps; HBM traffic from committed
rocprofv3 counter summaries when they match the current kernel sources) and the fp64 CPU
oracle timed on a bounded sample of the same workload on the host cores.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config qwen3] [--no-cpu-baseline]

Helpers that read rocprofv3 CSV output (CPU only, print a text summary):

    python bench.py --summarize-stats DIR --config C --command "..."
    python bench.py --summarize-counters FETCH_DIR WRITE_DIR --config C --command "..."
    python bench.py --summarize-mfma DIR --config C --command "..."
    python bench.py --summarize-memory DIR --config C --command "..."
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "MoE layer fwd+bwd useful TFLOPS and tokens/s on 1 MI355X; % MFMA peak"
# MI355X dense MFMA peaks: 256 CU x 2.4 GHz x (4096 bf16 | 8192 fp8) flop per CU-clock
PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2}
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
CALIB_MIB = 1024              # size of the copy kernel that calibrates the HBM byte counters

WORKLOADS = {
    "qwen3": "Qwen3-30B-A3B-shaped MoE layer fwd+bwd: T=16384, d=2048, f=768, E=128, top-8, bf16",
    "skewed": "Qwen3-30B-A3B-shaped MoE layer fwd+bwd with Zipf-skewed routing (bias 3*ln(1/rank)), bf16",
    "mixtral": "Mixtral-8x7B-shaped MoE layer fwd+bwd: T=8192, d=4096, f=14336, E=8, top-2, bf16",
    "dsv3_fp8": ("DeepSeek-V3-shaped single-GPU expert share fwd+bwd: 32 of 256 experts, 8x4096 tokens "
                 "pre-routed top-8, d=7168, f=2048, e4m3 with fp32 block scales, bf16 outputs"),
    "tiny": "tiny MoE layer: T=64, d=128, f=256, E=8, top-2, bf16",
}

# stage -> flop per routed pair as a multiple of d*f, for the grouped GEMMs
GEMM_FLOP_PER_PAIR = {"gemm_up": 4, "gemm_down": 2, "gemm_dact": 2, "gemm_dx": 4, "gemm_dw2": 2, "gemm_dw1": 4}
# stage -> (kernel symbol prefix) as it appears in rocprofv3 output
STAGE_KERNEL_BF16 = {"gemm_up": "moe::grouped_gemm_kernel<0,", "gemm_down": "moe::grouped_gemm_kernel<1,",
                     "gemm_dact": "moe::grouped_gemm_kernel<2,", "gemm_dx": "moe::grouped_gemm_kernel<3,",
                     "gemm_dw2": "moe::grouped_gemm_kernel<4,", "gemm_dw1": "moe::grouped_gemm_kernel<5,",
                     "combine": "moe::combine_kernel", "router": "moe::router_topk_kernel",
                     "dlogits": "moe::dlogits_kernel", "wg_reduce": "moe::wg_reduce_kernel",
                     "plan": "moe::plan_", "tile_map": "moe::tile_map_kernel", "wg_split": "moe::wg_split_kernel",
                     "tokrow": "moe::tokrow_kernel", "permute": "moe::permute_kernel",
                     "gemm_fused": "moe::fused_forward_kernel", "fwd_queue": "moe::fwd_queue_kernel",
                     "ksort": "moe::kstep_sort_kernel"}
# blockwise fp8: the four data GEMMs in e4m3, the weight gradients in bf16 on x dequantised to bf16
STAGE_KERNEL_FP8 = dict(STAGE_KERNEL_BF16, gemm_up="moe::grouped_gemm_fp8_kernel<0>",
                        gemm_down="moe::grouped_gemm_fp8_kernel<1>", gemm_dact="moe::grouped_gemm_fp8_kernel<2>",
                        gemm_dx="moe::grouped_gemm_fp8_kernel<3>", quant_dy="moe::quant_rows_kernel",
                        dequant_x="moe::dequant_rows_kernel")
FP8_STAGES = ("gemm_up", "gemm_down", "gemm_dact", "gemm_dx")


def workload_name(run_name):
    base, _, dt = run_name.partition(":")
    return WORKLOADS[base] + (", run as MXFP8 (quantised per call)" if dt == "mxfp8" else "")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


STAGE_KERNEL_MX = dict(STAGE_KERNEL_BF16, gemm_up="moe::grouped_gemm_mx_kernel<0>",
                       gemm_down="moe::grouped_gemm_mx_kernel<1>", gemm_dact="moe::grouped_gemm_mx_kernel<2>",
                       gemm_dx="moe::grouped_gemm_mx_kernel<3>", gemm_dw2="moe::grouped_gemm_mx_wg_kernel<0>",
                       gemm_dw1="moe::grouped_gemm_mx_wg_kernel<1>", mx_quant_t="moe::mx_quant_tokens",
                       mx_pad="moe::mx_pad_offsets", mx_quant="moe::mx_quant_")
MX_FP8_STAGES = FP8_STAGES + ("gemm_dw2", "gemm_dw1")


def is_fp8(config):
    """True for the fp8 runs: the blockwise-fp8 workload or any workload run as MXFP8."""
    return config.endswith("fp8") or config.endswith(":mxfp8")


def stage_dtype(config, stage):
    # MXFP8 runs every GEMM in fp8 (the weight gradients too); blockwise fp8 runs the four data
    # GEMMs in fp8 and the weight gradients in bf16
    if config.endswith(":mxfp8"):
        return "fp8" if stage in MX_FP8_STAGES else "bf16"
    return "fp8" if (is_fp8(config) and stage in FP8_STAGES) else "bf16"


def stage_kernels(config):
    if config.endswith(":mxfp8"):
        return STAGE_KERNEL_MX
    return STAGE_KERNEL_FP8 if is_fp8(config) else STAGE_KERNEL_BF16


def stage_bytes(stage, T, d, f, E, k, A):
    """Algorithmic HBM bytes of one launch of a bandwidth-bound stage (each byte the stage
    must read or write once; A = routed pairs)."""
    if stage in ("combine", "combine_dx"):
        return A * d * 2 + T * d * 2 + T * k * 4
    if stage == "router":
        return T * E * 4 + T * k * 8
    if stage == "plan":
        return A * 4 * 3
    if stage == "dlogits":
        return T * k * 4 * 3 + T * E * 4
    if stage == "quant_dy":
        return T * d * 2 + T * d + T * (d // 128) * 4
    if stage == "dequant_x":                                 # e4m3 + 1x128 scales in, bf16 out
        return T * d + T * (d // 128) * 4 + T * d * 2
    if stage in ("mx_quant_x", "mx_quant_dy"):
        return T * d * 2 + T * d + T * d // 32
    if stage == "mx_quant_as_t":                            # sorted rows in, token-axis blocks out
        return A * f * 2 + A * f + A * f // 32
    if stage == "mx_quant_dh_t":
        return A * 2 * f * 2 + A * 2 * f + A * 2 * f // 32
    if stage in ("mx_quant_x_t", "mx_quant_dy_t"):           # each token row read once, A rows out
        return T * d * 2 + A * d + A * d // 32
    if stage in ("ksort_x", "ksort_dy"):    # token-major words (d/32 bytes a row) in, sorted by k step out
        return T * d // 32 + A * 4 + A * d // 32
    if stage in ("mx_quant_w1", "mx_quant_w2"):   # bf16 in, both orientations' codes and exponents out
        n = E * d * f * (2 if stage == "mx_quant_w1" else 1)
        return n * 2 + 2 * n + 2 * (n // 32)
    return None


SOURCE_DIR = os.path.join(ROOT, "grouped_gemm_expert_router_amd", "csrc")


def kernel_source_hash(src_dir=None):
    """Hash of every kernel and ABI source; a stored counter summary is only used while it matches."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(src_dir or SOURCE_DIR, "*"))):
        with open(p, "rb") as fh:
            h.update(os.path.basename(p).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_file(config):
    return os.path.join(ROOT, "profiles", f"hbm_traffic_{config.replace(':', '_')}.txt")


def stored_traffic(config, stage):
    """HBM bytes per launch of `stage` (FETCH_SIZE + WRITE_SIZE scaled by the copy-kernel
    calibration) from the committed counter summary, or None if absent or stale."""
    path = traffic_file(config)
    if not os.path.exists(path):
        return None
    rec, src = {}, None
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if line.startswith("source_hash:"):
                src = line.split(":", 1)[1].strip()
            elif line.startswith("stage "):
                parts = dict(kv.split("=", 1) for kv in line.split()[2:])
                rec[line.split()[1]] = float(parts["traffic_bytes"])
    if src != kernel_source_hash():
        return None
    return rec.get(stage)


# ------------------------------------------------------------------ CPU oracle baseline
def _host_cores():
    """Host cores this process may run on (its CPU affinity), all of which the oracle's BLAS uses."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, n)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp, target_s: float):
    """The fp64 oracle (route or plan, forward, backward) on the first n tokens, with n grown
    from 256 until one timed run takes at least half of target_s (the last run is reported)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    import oracle
    ncores = _host_cores()
    fp8 = inp.dtype == "fp8"
    if fp8:
        x_all = oracle.dequant_rows_1x128(inp.x, inp.x_scale)
        W1 = np.empty(inp.W1.shape, np.float64)
        W2 = np.empty(inp.W2.shape, np.float64)
        for e in range(inp.E):      # one expert at a time bounds the temporaries
            W1[e] = oracle.dequant_blocks_128x128(inp.W1[e], inp.W1_scale[e])
            W2[e] = oracle.dequant_blocks_128x128(inp.W2[e], inp.W2_scale[e])
    else:
        x_all = None
        W1 = oracle.bf16_to_f64(inp.W1)
        W2 = oracle.bf16_to_f64(inp.W2)

    def run(n):
        x = x_all[:n] if fp8 else oracle.bf16_to_f64(inp.x[:n])
        dy = oracle.bf16_to_f64(inp.dy[:n])
        t0 = time.perf_counter()
        if fp8:
            ids, w = inp.topk_ids[:n], inp.topk_w[:n].astype(np.float64)
            oracle.plan(ids, inp.E)
        else:
            ids, w = oracle.route(inp.logits[:n], inp.k)
            oracle.plan(ids, inp.E)
        oracle.forward(x, W1, W2, ids, w, E=inp.E)
        oracle.backward(x, W1, W2, ids, w, dy, logits_routed=not fp8)
        dt = time.perf_counter() - t0
        pairs = int((ids >= 0).sum())
        return dt, pairs

    with threadpool_limits(limits=ncores):
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        # the oracle's per-expert loop has a fixed cost, so grow the sample until it is long enough
        n = min(inp.T, 256)
        for _ in range(5):
            dt, pairs = run(n)
            if dt >= 0.5 * target_s or n >= inp.T:
                break
            n = int(min(inp.T, max(2 * n, n * target_s / max(dt, 1e-3))))
    return {"value": 18.0 * pairs * inp.d * inp.f / dt / 1e12, "unit": "TFLOPS", "cores": int(threads),
            "affinity_cores": ncores, "blas_threads": int(threads),
            "kind": "oracle", "tokens_per_s": n / dt, "seconds": dt, "cpu_model": _cpu_model(),
            "sample": f"first {n} of {inp.T} tokens of the same workload ({pairs} routed pairs, all {inp.E} "
                      f"experts), {'plan' if fp8 else 'route+plan'}+forward+backward in fp64 numpy on "
                      f"{'exactly dequantised fp8 inputs' if fp8 else 'bf16 inputs'}, {threads} BLAS threads"}


# ------------------------------------------------------------------ rocprofv3 summaries
def _csv_rows(d, suffix):
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    rows = []
    for p in files:
        with open(p, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _stage_of(name, config):
    for st, pre in stage_kernels(config).items():
        if pre in name:
            return st
    return None


def summarize_stats(d, config, command):
    rows = _csv_rows(d, "kernel_stats.csv")
    print(f"# rocprofv3 kernel statistics: {workload_name(config)}")
    print(f"command: {command}")
    print(f"source_hash: {kernel_source_hash(SOURCE_DIR)}")
    print(f"{'stage':<12} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'share%':>7}  kernel")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        st = _stage_of(r["Name"], config) or "-"
        print(f"{st:<12} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.1f} {float(r['MinNs']) / 1e3:>10.1f} "
              f"{float(r['MaxNs']) / 1e3:>10.1f} {float(r['Percentage']):>7.2f}  {r['Name'][:110]}")


def summarize_counters(fetch_dir, write_dir, config, command):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) per kernel, scaled by what the same counters
    read for the calibration copy (torch.neg over CALIB_MIB MiB of fp32: that many bytes read
    and written)."""
    def per_kernel(d, counter):
        acc = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return acc
    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    copy_bytes = CALIB_MIB * 2 ** 20

    def calib(acc, what):
        ks = [k for k in acc if "neg_kernel" in k]
        if not ks:
            raise SystemExit(f"calibration copy kernel not found among {what} dispatches")
        v = sorted(acc[ks[0]])[len(acc[ks[0]]) // 2] * 1024.0
        return copy_bytes / v
    ff, fw = calib(fetch, "FETCH_SIZE"), calib(write, "WRITE_SIZE")
    print(f"# rocprofv3 HBM byte counters per dispatch: {workload_name(config)}")
    print(f"command: {command}")
    print(f"source_hash: {kernel_source_hash(SOURCE_DIR)}")
    print(f"calibration: torch.neg over {CALIB_MIB} MiB fp32 -> fetch_factor={ff:.4f} write_factor={fw:.4f}")
    print("# stage <name> kernel=<symbol> fetch_kib=<median raw> write_kib=<median raw> traffic_bytes=<scaled sum>")
    for name in sorted(set(fetch) & set(write)):
        st = _stage_of(name, config)
        if st is None:
            continue
        fk = sorted(fetch[name])[len(fetch[name]) // 2]
        wk = sorted(write[name])[len(write[name]) // 2]
        tb = fk * 1024.0 * ff + wk * 1024.0 * fw
        print(f"stage {st} fetch_kib={fk:.1f} write_kib={wk:.1f} traffic_bytes={tb:.0f} "
              f"kernel={name.split('(')[0].replace(' ', '')}")


def summarize_mfma(d, config, command):
    """MFMA pipe utilisation per kernel: SQ_VALU_MFMA_BUSY_CYCLES (summed over the 1024 SIMDs)
    over 1024 x the kernel's cycles per XCD (GRBM_GUI_ACTIVE is summed over the 8 XCDs).  The
    kernel's average clock is those cycles over the dispatch's duration, and busy x clock x
    1024 SIMDs x 1024 flop per SIMD cycle (dense bf16; 2048 for fp8) is the rate the counters
    imply."""
    acc = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        acc.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
            acc[r["Kernel_Name"]].setdefault("_clock", []).append(float(r["Counter_Value"]) / 8.0 / dur)
    print(f"# rocprofv3 MFMA utilisation per dispatch: {workload_name(config)}")
    print(f"command: {command}")
    print(f"source_hash: {kernel_source_hash(SOURCE_DIR)}")
    print("# mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs); clock = GRBM_GUI_ACTIVE / 8 "
          "/ dispatch duration; implied = busy x clock x 1024 SIMDs x flop per SIMD cycle; medians over dispatches")
    print(f"{'stage':<12} {'mfma_busy':>9} {'clock_GHz':>9} {'implied_TF':>10} {'mfma_insts':>12} "
          f"{'lds_bank_conf/cu_cyc':>21}  kernel")
    med = lambda v: sorted(v)[len(v) // 2]
    for name, c in sorted(acc.items()):
        st = _stage_of(name, config)
        if st is None or not st.startswith("gemm") or "SQ_VALU_MFMA_BUSY_CYCLES" not in c:
            continue
        cyc = med(c["GRBM_GUI_ACTIVE"]) / 8.0
        busy = med(c["SQ_VALU_MFMA_BUSY_CYCLES"]) / (1024.0 * cyc)
        bc = med(c["SQ_LDS_BANK_CONFLICT"]) / (256.0 * cyc) if "SQ_LDS_BANK_CONFLICT" in c else float("nan")
        ins = med(c["SQ_INSTS_MFMA"]) if "SQ_INSTS_MFMA" in c else float("nan")
        clk = med(c["_clock"])
        fpc = 2048.0 if ("fp8" in name or "_mx_" in name) else 1024.0  # dense flop per SIMD cycle
        implied = busy * clk * 1024.0 * fpc / 1e12
        print(f"{st:<12} {busy:>9.3f} {clk / 1e9:>9.3f} {implied:>10.0f} {ins:>12.4g} {bc:>21.4f}  "
              f"{name.split('(')[0].replace('void ', '')}")


MEMORY_COUNTERS = ("TCC_HIT_sum", "TCC_MISS_sum", "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum", "TCC_TAG_STALL_sum",
                   "TA_ADDR_STALLED_BY_TC_CYCLES_sum", "TA_DATA_STALLED_BY_TC_CYCLES_sum",
                   "TCP_PENDING_STALL_CYCLES_sum", "GRBM_GUI_ACTIVE")


def summarize_memory(d, config, command):
    """Memory-side counters per GEMM: the L2 hit rate by request (TCC_HIT / (TCC_HIT + TCC_MISS)),
    and per compute unit the fraction of the kernel's cycles its vector L1 was stalled on data
    pending from L2 (TCP_PENDING_STALL_CYCLES, summed over the 256 units), its texture addresser
    was stalled by the L1 (address and data paths), and per L2 channel the cycles read requests
    waited for DRAM credits (summed over 8 XCDs x 16 channels).  GRBM_GUI_ACTIVE is summed over
    the 8 XCDs."""
    acc = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        acc.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    print(f"# rocprofv3 memory-side counters per dispatch: {workload_name(config)}")
    print(f"command: {command}")
    print(f"source_hash: {kernel_source_hash(SOURCE_DIR)}")
    print("# l2_hit = TCC_HIT / (TCC_HIT + TCC_MISS); l1_pending, ta_addr, ta_data = TCP_PENDING_STALL_CYCLES, "
          "TA_ADDR/DATA_STALLED_BY_TC_CYCLES over (256 CUs x GRBM_GUI_ACTIVE / 8); dram_credit = "
          "TCC_EA0_RDREQ_DRAM_CREDIT_STALL over (128 channels x GRBM_GUI_ACTIVE / 8); medians over dispatches")
    print(f"{'stage':<12} {'l2_hit':>7} {'l1_pending':>10} {'ta_addr':>8} {'ta_data':>8} {'dram_credit':>11}  kernel")
    med = lambda v: sorted(v)[len(v) // 2]
    for name, c in sorted(acc.items()):
        st = _stage_of(name, config)
        if st is None or not st.startswith("gemm") or not all(k in c for k in MEMORY_COUNTERS):
            continue
        cyc = med(c["GRBM_GUI_ACTIVE"]) / 8.0
        hit, miss = med(c["TCC_HIT_sum"]), med(c["TCC_MISS_sum"])
        print(f"{st:<12} {hit / (hit + miss):>7.3f} {med(c['TCP_PENDING_STALL_CYCLES_sum']) / (256 * cyc):>10.3f} "
              f"{med(c['TA_ADDR_STALLED_BY_TC_CYCLES_sum']) / (256 * cyc):>8.3f} "
              f"{med(c['TA_DATA_STALLED_BY_TC_CYCLES_sum']) / (256 * cyc):>8.3f} "
              f"{med(c['TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum']) / (128 * cyc):>11.4f}  "
              f"{name.split('(')[0].replace('void ', '')}")


# ------------------------------------------------------------------ benchmark
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="steps timed one by one after a 512 MiB cache-flushing write (0: skip)")
    ap.add_argument("--config", default="qwen3", choices=sorted(WORKLOADS))
    ap.add_argument("--dtype", default="auto", choices=["auto", "mxfp8"],
                    help="auto: the workload's own format; mxfp8: run a bf16 workload as MXFP8 (quantised inside)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target duration of the CPU oracle sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help=f"run a {CALIB_MIB} MiB copy kernel first (calibrates profiler byte counters)")
    ap.add_argument("--summarize-stats", metavar="DIR")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-mfma", metavar="DIR")
    ap.add_argument("--summarize-memory", metavar="DIR")
    ap.add_argument("--command", default="", help="profiler command recorded in a summary")
    ap.add_argument("--source-dir", default=None, help="kernel sources the profiled run used (for the hash)")
    args = ap.parse_args()
    global SOURCE_DIR
    if args.source_dir:
        SOURCE_DIR = args.source_dir
    run_name = args.config + (":mxfp8" if args.dtype == "mxfp8" else "")
    if args.summarize_stats:
        return summarize_stats(args.summarize_stats, run_name, args.command)
    if args.summarize_counters:
        return summarize_counters(*args.summarize_counters, run_name, args.command)
    if args.summarize_memory:
        return summarize_memory(args.summarize_memory, run_name, args.command)
    if args.summarize_mfma:
        return summarize_mfma(args.summarize_mfma, run_name, args.command)
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
    # the tiny workload is defined forward-only; a step here is forward + backward, so it gets an
    # upstream gradient too (a smoke-sized run of the bench itself)
    inp = make_config(args.config, fwd_only=False) if args.config == "tiny" else make_config(args.config)
    log(f"[bench] generated {args.config} inputs in {time.perf_counter() - t_gen:.1f}s; kernel sources "
        f"{kernel_source_hash()}")
    fp8 = inp.dtype == "fp8"
    mx = args.dtype == "mxfp8"
    assert not (mx and fp8), "the blockwise-fp8 workload has its own format"
    T, d, f, E, k = inp.T, inp.d, inp.f, inp.E, inp.k
    dm = moe.dims(T, d, f, E, k, moe.MOE_FP8_E4M3 if fp8 else (moe.MOE_MXFP8 if mx else moe.MOE_BF16))
    dev = "cuda"

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def raw(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    if fp8:
        x, W1, W2 = raw(inp.x), raw(inp.W1), raw(inp.W2)
        xs, W1s, W2s = raw(inp.x_scale), raw(inp.W1_scale), raw(inp.W2_scale)
        logits = None
    else:
        x, W1, W2 = bf16(inp.x), bf16(inp.W1), bf16(inp.W2)
        xs = W1s = W2s = None
        logits = torch.from_numpy(inp.logits).to(dev)
    dy = bf16(inp.dy)
    b = moe.alloc_layer_buffers(dm, dev, backward=True)
    if fp8:
        b["topk_ids"].copy_(torch.from_numpy(inp.topk_ids))
        b["topk_w"].copy_(torch.from_numpy(inp.topk_w))
    torch.cuda.synchronize()

    if args.calibrate_copy:
        src = torch.ones(CALIB_MIB * 2 ** 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    def step():
        if fp8:
            moe.moe_plan(dm, b["topk_ids"], b["counts"], b["offsets"], b["perm"], b["inv_perm"], b["ws_route"])
        else:
            moe.moe_route(dm, logits, b["topk_ids"], b["topk_w"], b["counts"], b["offsets"], b["perm"],
                          b["inv_perm"], b["ws_route"])
        moe.moe_forward(dm, x, xs, W1, W1s, W2, W2s, b["topk_w"], b["offsets"], b["perm"], b["inv_perm"], b["y"],
                        b["saved"], b["ws_fwd"])
        moe.moe_backward(dm, dy, x, xs, W1, W1s, W2, W2s, b["topk_ids"], b["topk_w"], b["offsets"], b["perm"],
                         b["inv_perm"], b["saved"], b["dx"], b["dW1"], b["dW2"], b["d_topk_w"],
                         None if fp8 else b["d_logits"], b["ws_bwd"])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")

    # The step time comes from K steps with nothing between the kernels; the per-stage times from
    # the same K steps run again right after with a HIP event recorded on the launch stream around
    # every kernel (the events themselves add gaps between kernels, about 2.5 % of a qwen3 step).
    cur = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(cur)
    for _ in range(args.steps):
        step()
    stop.record(cur)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    log(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step")

    # The same K steps replayed from a HIP graph captured once (every entry point only enqueues
    # kernels on the caller's stream): the step without host launch overhead.
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        step()
    cur.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()
    start.record(cur)
    for _ in range(args.steps):
        graph.replay()
    stop.record(cur)
    torch.cuda.synchronize()
    ms_graph = start.elapsed_time(stop) / args.steps
    del graph
    log(f"[bench] timed {args.steps} graph replays: {ms_graph:.3f} ms/step")

    events, open_ev, streams = [], {}, {}

    def hook(stage, begin, stream_ptr):
        sp = stream_ptr or 0
        if sp not in streams:
            streams[sp] = cur if sp == (cur.cuda_stream or 0) else torch.cuda.ExternalStream(sp)
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(streams[sp])
        if begin:
            open_ev[(stage, sp)] = ev
        else:
            events.append((stage, open_ev.pop((stage, sp)), ev))

    moe.moe_set_stage_hook(hook)
    start.record(cur)
    for _ in range(args.steps):
        step()
    stop.record(cur)
    torch.cuda.synchronize()
    moe.moe_set_stage_hook(None)
    ms_ev = start.elapsed_time(stop) / args.steps
    log(f"[bench] timed {args.steps} steps with stage events: {ms_ev:.3f} ms/step")

    A = int(b["offsets"][-1].item())
    useful = 18.0 * A * d * f
    tflops = useful / (ms * 1e-3) / 1e12
    per = {}
    for stage, e0, e1 in events:
        per.setdefault(stage, []).append(e0.elapsed_time(e1))
    stages = {}
    ideal_ms = 0.0   # time of the GEMMs at their dtype's MFMA peak
    for stage, ts in per.items():
        avg = sum(ts) / len(ts)
        ent = {"launches": len(ts), "avg_ms": avg, "ms_per_step": sum(ts) / args.steps}
        if stage in GEMM_FLOP_PER_PAIR:
            fl = GEMM_FLOP_PER_PAIR[stage] * A * d * f
            pk = PEAK_TFLOPS[stage_dtype(run_name, stage)]
            ent.update(dtype=stage_dtype(run_name, stage), tflops=fl / (avg * 1e-3) / 1e12)
            ent["frac_mfma_peak"] = ent["tflops"] / pk
            ideal_ms += fl / (pk * 1e12) * 1e3
        else:
            by = stage_bytes(stage, T, d, f, E, k, A)
            if by:
                ent["gbs"] = by / (avg * 1e-3) / 1e9
        stages[stage] = ent
    log("[bench] per-kernel: " + ", ".join(f"{s}={v['avg_ms']:.3f}ms" for s, v in
                                           sorted(stages.items(), key=lambda kv: -kv[1]["ms_per_step"])))
    dom = max(stages, key=lambda s: stages[s]["ms_per_step"])
    dom_e = stages[dom]
    traffic = stored_traffic(run_name, dom)
    if dom in GEMM_FLOP_PER_PAIR:
        fl = GEMM_FLOP_PER_PAIR[dom] * A * d * f
        pk = PEAK_TFLOPS[stage_dtype(run_name, dom)]
        achieved = fl / (dom_e["avg_ms"] * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": pk, "unit": "TFLOP/s",
                "frac": achieved / pk, "traffic": traffic, "dtype": stage_dtype(run_name, dom),
                "algorithmic_flop_per_launch": fl, "avg_launch_ms": dom_e["avg_ms"]}
    else:
        by = stage_bytes(dom, T, d, f, E, k, A)
        achieved = by / (dom_e["avg_ms"] * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": traffic, "algorithmic_bytes_per_launch": by,
                "avg_launch_ms": dom_e["avg_ms"]}

    # dispatch on its own (the step fuses it into the first GEMM's loads): HBM bandwidth of the
    # standalone permute kernel, outside the timed region
    permute = None
    if not fp8:
        xp = torch.empty((T * k, d), dtype=torch.bfloat16, device=dev)
        pdm = moe.dims(T, d, f, E, k)  # the permute moves bf16 rows
        moe.moe_permute(pdm, x, b["inv_perm"], xp)
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p0.record(cur)
        for _ in range(10):
            moe.moe_permute(pdm, x, b["inv_perm"], xp)
        p1.record(cur)
        torch.cuda.synchronize()
        pms = p0.elapsed_time(p1) / 10
        pby = T * d * 2 + A * d * 2
        permute = {"avg_ms": pms, "algorithmic_bytes": pby, "gbs": pby / (pms * 1e-3) / 1e9,
                   "frac_hbm_peak": pby / (pms * 1e-3) / 1e9 / PEAK_HBM_GBS}
        del xp

    # the single-launch forward (moe_forward_fused: gather, both grouped GEMMs and the SwiGLU in
    # one persistent launch, then the combine) against the forward of the timed step, on the same
    # routing, outside the timed region; its output must equal the step's bit for bit
    fused = None
    if not fp8 and not mx:
        y2 = torch.empty_like(b["y"])
        s2 = torch.empty_like(b["saved"])
        fwd = lambda: moe.moe_forward(dm, x, None, W1, None, W2, None, b["topk_w"], b["offsets"], b["perm"],
                                      b["inv_perm"], b["y"], b["saved"], b["ws_fwd"])
        fus = lambda: moe.moe_forward_fused(dm, x, W1, W2, b["topk_w"], b["offsets"], b["perm"], b["inv_perm"], y2,
                                            s2, b["ws_fwd"])
        fwd()
        fus()
        torch.cuda.synchronize()
        same = bool(torch.equal(b["y"].view(torch.int16), y2.view(torch.int16)))
        f0, f1, f2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        reps = 10
        f0.record(cur)
        for _ in range(reps):
            fwd()
        f1.record(cur)
        for _ in range(reps):
            fus()
        f2.record(cur)
        torch.cuda.synchronize()
        tms, fms = f0.elapsed_time(f1) / reps, f1.elapsed_time(f2) / reps
        ffl = 6.0 * A * d * f
        fused = {"fused_ms": fms, "two_launch_ms": tms, "fused_tflops": ffl / (fms * 1e-3) / 1e12,
                 "two_launch_tflops": ffl / (tms * 1e-3) / 1e12, "y_bitwise_equal": same,
                 "note": "forward only (queue or tile table, GEMMs, combine); outside the timed step"}
        log(f"[bench] forward: single launch {fms:.3f} ms, two launches {tms:.3f} ms, equal={same}")
        del y2, s2

    # router front end (the gate in front of the layer; its logits are the step's input, so it is
    # timed here on its own): logits = x Wg, then the backward through it (dWg and dx += dl Wg^T)
    router = None
    if not fp8 and inp.Wg is not None:
        Wg = bf16(inp.Wg)
        lg = torch.empty((T, E), dtype=torch.float32, device=dev)
        dWg = torch.empty((d, E), dtype=torch.bfloat16, device=dev)
        rws = torch.empty((max(moe.moe_workspace_bytes(dm, moe.MOE_WS_ROUTER), 256),), dtype=torch.uint8,
                          device=dev)
        dxr = b["dx"].clone()
        moe.moe_router_logits(dm, x, Wg, lg)
        moe.moe_router_backward(dm, x, Wg, b["d_logits"], dxr, dWg, rws)
        r0, r1, r2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        reps = 10
        r0.record(cur)
        for _ in range(reps):
            moe.moe_router_logits(dm, x, Wg, lg)
        r1.record(cur)
        for _ in range(reps):
            moe.moe_router_backward(dm, x, Wg, b["d_logits"], dxr, dWg, rws)
        r2.record(cur)
        torch.cuda.synchronize()
        lms, bms = r0.elapsed_time(r1) / reps, r1.elapsed_time(r2) / reps
        fl = 2.0 * T * d * E
        router = {"logits_ms": lms, "backward_ms": bms, "logits_tflops": fl / (lms * 1e-3) / 1e12,
                  "backward_tflops": 2 * fl / (bms * 1e-3) / 1e12,
                  "note": "x.Wg and its backward (dWg, dx += d_logits.Wg^T), bf16 MFMA; outside the timed step"}
        log(f"[bench] router front end: logits {lms:.3f} ms, backward {bms:.3f} ms")
        del lg, dWg, rws, dxr

    # LLC-cold steps: a 512 MiB scratch write before each one (outside its timing) evicts the
    # step's operands from the 256 MB last-level cache and the L2s; the median step is reported
    cold = None
    if args.cold_steps > 0:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cts = []
        for i in range(args.cold_steps):
            scratch.fill_(i & 0xFF)
            c0.record(cur)
            step()
            c1.record(cur)
            torch.cuda.synchronize()
            cts.append(c0.elapsed_time(c1))
        cms = sorted(cts)[len(cts) // 2]
        cold = {"ms_per_step": cms, "value": useful / (cms * 1e-3) / 1e12, "unit": "TFLOPS",
                "steps": args.cold_steps, "statistic": "median", "flush_bytes_between_steps": 512 << 20}
        log(f"[bench] LLC-cold: {cms:.3f} ms/step (median of {args.cold_steps})")
        del scratch

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle (~{args.cpu_seconds:.0f}s sample) ...")
        cpu = cpu_baseline(inp, args.cpu_seconds)
        log(f"[bench] CPU oracle: {cpu['seconds']:.1f}s, {cpu['value'] * 1e3:.2f} GFLOPS, {cpu['cores']} threads")

    out = {
        "metric": METRIC, "value": tflops, "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3+bf16" if fp8 else ("mxfp8+bf16" if mx else "bf16"),
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.config] + (", run as MXFP8 (quantised per call)" if mx else ""),
                   "T": T, "d": d, "f": f, "E": E, "k": k, "routed_pairs": A, "seed_config": run_name},
        "tokens_per_s": T / (ms * 1e-3),
        "frac_of_bf16_peak": tflops / PEAK_TFLOPS["bf16"],
        "frac_of_mfma_peak": ideal_ms / ms,
        "useful_flop_per_step": useful, "ms_per_step_with_stage_events": ms_ev,
        "ms_per_step_graph_replay": ms_graph, "stages": stages,
        "permute_standalone": permute, "router_front_end": router, "single_launch_forward": fused,
        "roofline": roof,
        "llc_cold": cold, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
