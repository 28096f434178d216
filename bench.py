"""Benchmark of the LLM.int8() mixed int8 linear layer on one MI355X.

Default workload: OPT-6.7B-shaped FFN up-projection at prefill, X fp16
[2048 x 4096] ~ N(0, 1) with 6 outlier hidden dims at +-U(15, 25) on 25% of
the tokens each, W [16384 x 4096] ~ N(0, 0.02^2) quantized once to int8,
threshold 6.0. One step = one whole layer call (outlier detection, row
quantization and outlier gather, int8 GEMM with the fused dequantize + fp16
outlier product + fp16 store). Inputs are resident in HBM before the timed
region; a pool of input/output sets larger than the 256 MB Infinity Cache is
rotated so successive steps do not reuse cached data.

Prints ONE JSON line (rank 0, N=1):
  value        effective TOPS = 2*M*N*K / step time (whole layer, all kernels)
  roofline     the int8 GEMM kernel alone vs the int8 MFMA peak (5.0 POP/s),
               its average duration measured with HIP events on the launch stream
  quantize     the X row-quantize kernel (HBM GB/s vs 8 TB/s) and the one-time
               weight quantization (GB/s)
  cpu_baseline the CPU oracle timed on this host on a bounded row sample

  python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload opt6.7b_ffn_up]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, TOP/s
PEAK_HBM_GBPS = 8000.0       # MI355X HBM3E, GB/s
MALL_BYTES = 256 << 20

WORKLOADS = {
    "opt6.7b_ffn_up": dict(M=2048, K=4096, N=16384),
    "ffn175b": dict(M=4096, K=12288, N=49152),
    "decode1": dict(M=1, K=4096, N=4096),
    "decode4": dict(M=4, K=4096, N=4096),
    "decode16": dict(M=16, K=4096, N=4096),
}

GEMM_SRC = os.path.join(ROOT, "int8_quantized_matmul_absmax_amd", "csrc", "gemm_kernel.hip")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "gemm_i8_opt6.7b_ffn_up_counters.json")


def _make(workload):
    from int8_quantized_matmul_absmax_amd import synth
    if workload == "opt6.7b_ffn_up":
        return synth.opt_ffn_up()
    if workload == "ffn175b":
        return synth.ffn_175b()
    if workload.startswith("decode"):
        return synth.decode(int(workload[6:]))
    raise ValueError(workload)


def _event_time_ms(fn, iters, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(iters):
        fn(i)
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters


def _traffic_from_counters():
    """HBM bytes per GEMM launch from committed rocprofv3 counter runs, or None
    when absent or taken on a different version of the kernel source."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
        src_hash = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
        if c.get("kernel_source_sha256") != src_hash:
            return None
        return float(c["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def _cpu_baseline(d, Wq_ref, sw_ref, M, N, K, target_s):
    """The oracle as it stands, on a bounded sample of rows: outlier detection
    over all rows, then quantization, int32 GEMM, outlier product and
    dequantization for S sampled rows x all N outputs. Scaled to TOPS by the
    dense-equivalent 2*S*N*K."""
    import numpy as np
    from oracle import llm_int8 as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    rng = np.random.default_rng(0)
    S = 64
    while True:
        rows = np.sort(rng.choice(M, size=min(S, M), replace=False))
        t0 = time.perf_counter()
        O.linear_int8_mixed(d["X"], Wq_ref, sw_ref, 6.0, rows=rows)
        dt = time.perf_counter() - t0
        if dt >= target_s or S >= M:
            break
        S = min(M, max(S * 2, int(S * target_s / max(dt, 1e-3) * 1.1)))
    tops = 2.0 * rows.size * N * K / dt / 1e12
    return {"value": round(tops, 6), "unit": "TOPS", "cores": int(threads), "kind": "oracle",
            "sample": "%d of %d token rows x all %d outputs (outlier detection over all rows), "
                      "%.1f s" % (rows.size, M, N, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="opt6.7b_ffn_up", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import int8_quantized_matmul_absmax_amd as i8
    from oracle import llm_int8 as O

    i8.ensure_built()
    ops = i8.ops
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    shp = WORKLOADS[args.workload]
    M, K, N = shp["M"], shp["K"], shp["N"]

    d = _make(args.workload)
    X_h, W_h = d["X"], d["W"]

    # ---- one-time weight quantization (a4), timed on its own
    W_dev = [torch.from_numpy(W_h).cuda()]
    w_bytes = W_h.nbytes
    n_wcopies = max(1, min(4, (2 * MALL_BYTES) // w_bytes + 1))
    for _ in range(n_wcopies - 1):
        W_dev.append(W_dev[0].clone())
    Wq0, sw0 = ops.int8_quantize_colwise_weight(W_dev[0])
    torch.cuda.synchronize()
    Wq_bufs = [torch.empty_like(Wq0) for _ in W_dev]
    sw_bufs = [torch.empty_like(sw0) for _ in W_dev]
    wq_iters = 10
    t_wq = _event_time_ms(
        lambda i: ops.int8_quantize_colwise_weight(W_dev[i % len(W_dev)], Wq_bufs[i % len(W_dev)],
                                                   sw_bufs[i % len(W_dev)]), wq_iters, stream)
    wq_gbps = (3.0 * N * K + 4.0 * N) / (t_wq * 1e-3) / 1e9
    del W_dev, Wq_bufs, sw_bufs

    # ---- rotation pool of (X, Wq, sw, Y, workspace) sets beyond the MALL
    set_bytes = X_h.nbytes + Wq0.numel() + 2 * M * N + ops.workspace_bytes(M, K)
    n_sets = int(max(2, min(8, (2 * MALL_BYTES) // max(set_bytes, 1) + 1)))
    X0 = torch.from_numpy(X_h).cuda()
    pool = []
    for s in range(n_sets):
        pool.append(dict(
            X=X0 if s == 0 else X0.clone(),
            Wq=Wq0 if s == 0 else Wq0.clone(),
            sw=sw0 if s == 0 else sw0.clone(),
            Y=torch.empty((M, N), dtype=torch.float16, device="cuda"),
            ws=torch.empty((ops.workspace_bytes(M, K),), dtype=torch.uint8, device="cuda")))
    torch.cuda.synchronize()

    def step(i):
        p = pool[i % n_sets]
        ops.linear_int8_mixed(p["X"], p["Wq"], p["sw"], None, 6.0, p["ws"], p["Y"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_step = _event_time_ms(step, args.steps, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eff_tops = 2.0 * M * N * K / (ms_step * 1e-3) / 1e12

    # ---- the dominant kernel alone: int8 GEMM + fused epilogue, same launch
    # configuration as inside the layer (intermediates from the last step)
    views = [ops.workspace_views(p["ws"], M, K) for p in pool]
    n_out = int(views[0]["n"].cpu().numpy()[0])

    def gemm(i):
        p, v = pool[i % n_sets], views[i % n_sets]
        ops.int8_mm_dequant(v["Xq"], p["Wq"], v["sx"], p["sw"], v["Xo"], v["cols"], v["n"],
                            None)

    for i in range(max(2, args.warmup // 2)):
        gemm(i)
    ms_gemm = _event_time_ms(gemm, args.steps, stream)
    gemm_tops = 2.0 * M * N * K / (ms_gemm * 1e-3) / 1e12

    # ---- the X row-quantize kernel alone (a3 + gather), same launch shape
    def rowq(i):
        p, v = pool[i % n_sets], views[i % n_sets]
        ops.int8_quantize_rowwise(p["X"], v["bitmap"], v["Xq"], v["sx"])

    for i in range(4):
        rowq(i)
    ms_rowq = _event_time_ms(rowq, args.steps, stream)
    rowq_gbps = (3.0 * M * K + 4.0 * M) / (ms_rowq * 1e-3) / 1e9

    # ---- parity spot check of the timed output (sampled rows vs the oracle)
    Wq_ref, sw_ref = O.quantize_weight_rows(W_h)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(1).choice(M, 8)]))
    ref = O.linear_int8_mixed(X_h, Wq_ref, sw_ref, 6.0, rows=rows)
    Y_last = pool[(args.steps - 1) % n_sets]["Y"]
    err = O.max_abs_rel_error(Y_last[torch.from_numpy(rows).cuda()].cpu().numpy(), ref["Y"])
    codes_ok = bool(np.array_equal(Wq0.cpu().numpy(), Wq_ref))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = _cpu_baseline(d, Wq_ref, sw_ref, M, N, K, args.cpu_seconds)

    traffic = _traffic_from_counters() if args.workload == "opt6.7b_ffn_up" else None
    out = {
        "metric": "effective int8-mixed linear TOPS",
        "value": round(eff_tops, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "%s_prefill" % args.workload if not args.workload.startswith("decode")
                   else args.workload, "M": M, "K": K, "N": N, "threshold": 6.0,
                   "n_outliers": n_out, "parallelism": "single_gpu"},
        "roofline": {"bound": "mfma", "kernel": "k_gemm_i8 (int8 GEMM + fused dequant/outlier epilogue)",
                     "achieved": round(gemm_tops, 3), "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
                     "traffic": traffic, "ms_per_launch": round(ms_gemm, 6),
                     "ops_per_launch": 2 * M * N * K},
        "int8_mfma_peak_frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
        "quantize": {"x_rowwise_gbps": round(rowq_gbps, 1),
                     "x_rowwise_hbm_frac": round(rowq_gbps / PEAK_HBM_GBPS, 4),
                     "x_rowwise_ms": round(ms_rowq, 6),
                     "weight_once_gbps": round(wq_gbps, 1),
                     "weight_once_hbm_frac": round(wq_gbps / PEAK_HBM_GBPS, 4),
                     "weight_once_ms": round(t_wq, 6)},
        "parity": {"y_max_abs_rel_err_sampled_rows": err, "weight_codes_bitexact": codes_ok},
        "cpu_baseline": cpu,
        "rotation_sets": n_sets,
        "timed_wall_s": round(wall, 4),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
