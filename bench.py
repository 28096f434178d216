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
import re
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


def _kernel_code_sha256():
    """SHA-256 of the GEMM kernel's code: its source with comments removed and
    whitespace collapsed, so that only a change of code (not of its comments)
    invalidates counters taken on it."""
    text = open(GEMM_SRC).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


def _traffic_from_counters():
    """HBM bytes per GEMM launch from committed rocprofv3 counter runs, or None
    when absent or taken on a different version of the kernel code."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
        if c.get("kernel_code_sha256") != _kernel_code_sha256():
            return None
        return float(c["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def _cpu_baseline(d, M, N, K, target_s, Wq_gpu, Y_rows, rows_y):
    """The oracle as it stands, on a bounded sample of rows: outlier detection
    over all rows, then quantization, int32 GEMM, outlier product and
    dequantization for S sampled rows x all N outputs. Scaled to TOPS by the
    dense-equivalent 2*S*N*K. The same leg checks the timed GPU output against
    the oracle on the rows rows_y (Y_rows, host copy) and the GPU weight codes
    (Wq_gpu, host copy) bit for bit."""
    import numpy as np
    from oracle import llm_int8 as O
    Wq_ref, sw_ref = O.quantize_weight_rows(d["W"])
    ref = O.linear_int8_mixed(d["X"], Wq_ref, sw_ref, 6.0, rows=rows_y)
    Yr = np.asarray(ref["Y"], np.float64)
    dY = np.abs(np.asarray(Y_rows, np.float64) - Yr)
    floor = 1e-2 * np.abs(Yr).max()
    parity = {"y_max_abs_rel_err_sampled_rows": O.max_abs_rel_error(Y_rows, ref["Y"]),
              # per element, relative to max(|Y_ref|, 1e-2 max |Y_ref|)
              "y_elem_rel_err_floor_1e-2_sampled_rows":
                  float((dY / np.maximum(np.abs(Yr), floor)).max()) if Yr.size else 0.0,
              "weight_codes_bitexact": bool(np.array_equal(Wq_gpu, Wq_ref))}
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
    # When the whole workload finishes well inside the window, repeat whole
    # calls until the window is filled and report the mean.
    calls, total = 1, dt
    while total < target_s:
        t0 = time.perf_counter()
        O.linear_int8_mixed(d["X"], Wq_ref, sw_ref, 6.0, rows=rows)
        total += time.perf_counter() - t0
        calls += 1
    dt = total / calls
    tops = 2.0 * rows.size * N * K / dt / 1e12
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                         None)
    except OSError:
        pass
    return ({"value": round(tops, 6), "unit": "TOPS", "cores": int(threads), "kind": "oracle",
             "sample": "%d of %d token rows x all %d outputs (outlier detection over all rows), "
                       "%d call(s), %.2f s each" % (rows.size, M, N, calls, dt),
             "host": {"cpu_model": model, "logical_cpus": os.cpu_count(),
                      "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}}, parity)


COPY_PROBE_BYTES = 512 << 20


def _copy_probe():
    """A plain device copy of known size (uint8 -> int8 elementwise copy kernel,
    COPY_PROBE_BYTES read and written per launch): the calibration run for the
    FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.empty((COPY_PROBE_BYTES,), dtype=torch.uint8, device="cuda")
    dst = torch.empty((COPY_PROBE_BYTES,), dtype=torch.int8, device="cuda")
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "launches": 4}), flush=True)


def _counter_means(csv_path, name_part):
    """Mean per-dispatch value of each counter over the dispatches whose kernel
    name contains name_part, from a rocprofv3 counter_collection.csv."""
    import csv
    per_dispatch = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if name_part not in r["Kernel_Name"]:
                continue
            key = (r["Dispatch_Id"], r["Counter_Name"])
            per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (_, c), v in per_dispatch.items():
        out.setdefault(c, []).append(v)
    return {c: (sum(v) / len(v), len(v)) for c, v in out.items()}


def _write_counters(pmc_dir):
    """Turns four rocprofv3 --pmc runs into the stored HBM-traffic figure of the
    GEMM kernel: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of k_gemm_i8 over
    the default workload, each scaled by known bytes / counter reading of the
    copy probe. Expects <pmc_dir>/{fetch,write,copy_fetch,copy_write}/
    run_counter_collection.csv."""
    def one(sub, kern, counter):
        path = os.path.join(pmc_dir, sub, "run_counter_collection.csv")
        m = _counter_means(path, kern)
        if counter not in m:
            raise SystemExit("%s: no %s dispatches of %s" % (path, counter, kern))
        return m[counter]
    gf, ngf = one("fetch", "k_gemm_i8", "FETCH_SIZE")
    gw, ngw = one("write", "k_gemm_i8", "WRITE_SIZE")
    cf, ncf = one("copy_fetch", "copy", "FETCH_SIZE")
    cw, ncw = one("copy_write", "copy", "WRITE_SIZE")
    known_kib = COPY_PROBE_BYTES / 1024.0
    f_fetch, f_write = known_kib / cf, known_kib / cw
    fetch_b = gf * f_fetch * 1024.0
    write_b = gw * f_write * 1024.0
    M, K, N = 2048, 4096, 16384
    algo = M * K + N * K + 4 * (M + N) + 2 * M * N
    rec = {
        "kernel": "k_gemm_i8", "workload": "opt6.7b_ffn_up M=2048 K=4096 N=16384",
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d %s/fetch -o run -- "
            "python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline" % pmc_dir,
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d %s/write -o run -- "
            "python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline" % pmc_dir,
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d %s/copy_fetch -o run -- "
            "python3 bench.py --copy-probe" % pmc_dir,
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d %s/copy_write -o run -- "
            "python3 bench.py --copy-probe" % pmc_dir,
            "python3 bench.py --write-counters %s" % pmc_dir],
        "counter_note": "FETCH_SIZE and WRITE_SIZE count L2-to-fabric traffic (KiB per dispatch); "
                        "each is scaled by the copy probe's known bytes / its reading",
        "kernel_code_sha256": _kernel_code_sha256(),
        "fetch_kib_per_dispatch": round(gf, 1), "write_kib_per_dispatch": round(gw, 1),
        "dispatches": [ngf, ngw],
        "copy_probe": {"bytes": COPY_PROBE_BYTES, "fetch_kib": round(cf, 1),
                       "write_kib": round(cw, 1), "dispatches": [ncf, ncw],
                       "fetch_scale": round(f_fetch, 5), "write_scale": round(f_write, 5)},
        "hbm_fetch_bytes_per_launch": round(fetch_b), "hbm_write_bytes_per_launch": round(write_b),
        "hbm_bytes_per_launch": round(fetch_b + write_b),
        "algorithmic_bytes_per_launch": algo,
        "traffic_over_algorithmic": round((fetch_b + write_b) / algo, 4),
    }
    with open(COUNTERS_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


TRACE_FILE = os.path.join(ROOT, "profiles", "k_gemm_i8_opt6.7b_ffn_up_kernel_trace.md")


def _summarize_trace(trace_dir):
    """Writes the committed kernel-trace summary from a rocprofv3 run of
    `bench.py --steps S --warmup W --no-cpu-baseline` (kernel trace + stats,
    csv output, -o bench): the per-kernel statistics, and the GEMM average over
    the launches of the timed GEMM-alone loop next to the HIP-event figure the
    bench printed."""
    import csv
    log = open(os.path.join(trace_dir, "bench.log")).read().splitlines()
    line = [x for x in log if x.startswith("{")][-1]
    b = json.loads(line)
    steps = b["steps"]
    tr = list(csv.DictReader(open(os.path.join(trace_dir, "bench_kernel_trace.csv"))))
    tr.sort(key=lambda r: int(r["Start_Timestamp"]))
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
    g = [r for r in tr if "k_gemm_i8" in r["Kernel_Name"]]
    alone = g[-steps:]
    in_step = g[b["warmup"]:b["warmup"] + steps]
    avg = lambda rs: sum(dur(r) for r in rs) / max(len(rs), 1)
    def short(n):
        n = n.replace("(anonymous namespace)::", "").replace("void ", "")
        return n.split("(")[0][:100]
    out = ["# Kernel trace: k_gemm_i8 and the layer's kernels, OPT-6.7B FFN up (2048 x 4096 -> 16384)",
           "",
           "Command (from the repository root):",
           "",
           "    rocprofv3 --kernel-trace --stats --output-format csv -d %s -o bench -- "
           "python3 bench.py --steps %d --warmup %d --no-cpu-baseline" % (trace_dir, steps, b["warmup"]),
           "    python3 bench.py --summarize-trace %s" % trace_dir,
           "",
           "k_gemm_i8 (%s, grid %s threads, %s VGPR + %s AGPR, LDS %s B, scratch %s B):" % (
               short(g[0]["Kernel_Name"]), g[0]["Grid_Size_X"],
               g[0]["VGPR_Count"], g[0]["Accum_VGPR_Count"], g[0]["LDS_Block_Size"],
               g[0]["Scratch_Size"]),
           "",
           "| measurement | launches | average (us) |",
           "|---|---|---|",
           "| rocprofv3, timed GEMM-alone loop | %d | %.2f |" % (len(alone), avg(alone)),
           "| HIP events on the launch stream, same loop (bench `roofline.ms_per_launch`) | %d | %.2f |"
           % (steps, 1000.0 * b["roofline"]["ms_per_launch"]),
           "| rocprofv3, inside the timed layer steps | %d | %.2f |" % (len(in_step), avg(in_step)),
           "",
           "Bench line printed under the profiler (whole layer step %.2f us):" % (1000.0 * b["ms_per_step"]),
           "",
           "    " + line,
           "",
           "rocprofv3 --stats (all launches of the run, warm-up and weight quantization included):",
           "",
           "| kernel | calls | average (us) | min (us) | max (us) | % of GPU time |",
           "|---|---|---|---|---|---|"]
    for r in csv.DictReader(open(os.path.join(trace_dir, "bench_kernel_stats.csv"))):
        out.append("| %s | %s | %.2f | %.2f | %.2f | %.2f |" % (
            short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1000, float(r["MinNs"]) / 1000,
            float(r["MaxNs"]) / 1000, float(r["Percentage"])))
    with open(TRACE_FILE, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


SWEEP_FILE = os.path.join(ROOT, "profiles", "layer_all_configs_sweep.md")


def _graph_time_us(call, reps, replays=20):
    """Per-call GPU time of `call` (a no-argument function that launches on
    torch's current stream): `reps` calls captured in one HIP graph, the graph
    replayed `replays` times between HIP events, so host launch overhead is
    out of the figure. Returns (us per call, outputs identical on every
    replay)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ref = call()
        torch.cuda.synchronize()
        ref = ref.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            outs = [call() for _ in range(reps)]
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    same = True
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    g.replay()
    torch.cuda.synchronize()
    same &= bool(torch.equal(outs[-1], ref))
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    end.synchronize()
    same &= bool(torch.equal(outs[-1], ref))
    return start.elapsed_time(end) * 1e3 / (replays * reps), same


def _sweep():
    """Every workload through linear_int8_mixed on one GPU; one JSON line per
    case and a markdown summary under profiles/."""
    import numpy as np
    import torch
    import int8_quantized_matmul_absmax_amd as i8
    from int8_quantized_matmul_absmax_amd import synth
    i8.ensure_built()
    ops = i8.ops
    torch.cuda.set_device(0)
    rows = []

    def emit(rec):
        rows.append(rec)
        print(json.dumps(rec), flush=True)

    def quantize(W):
        return ops.int8_quantize_colwise_weight(torch.from_numpy(W).cuda())

    # tiny layer and decode: graph-captured calls (host launch cost excluded),
    # the weight rotated over copies beyond 2 x MALL for the decode shapes
    for name, d in [("tiny 16x256->256", synth.tiny())] + [
            ("decode M=%d 4096->4096" % m, synth.decode(m)) for m in (1, 4, 16)]:
        X = torch.from_numpy(d["X"]).cuda()
        M, K = d["X"].shape
        Wq, sw = quantize(d["W"])
        N = Wq.shape[0]
        copies = max(1, min(40, (2 * MALL_BYTES) // max(Wq.numel(), 1) + 1))
        Wqs = [Wq] + [Wq.clone() for _ in range(copies - 1)]
        ws = torch.empty((ops.workspace_bytes(M, K, N),), dtype=torch.uint8, device="cuda")
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        state = {"i": 0}

        def call():
            state["i"] += 1
            return ops.linear_int8_mixed(X, Wqs[state["i"] % copies], sw, None, 6.0, ws, Y)
        us, same = _graph_time_us(call, reps=copies)
        # warm: the same weight copy every call, so it stays in the MALL
        us_w, same_w = _graph_time_us(
            lambda: ops.linear_int8_mixed(X, Wq, sw, None, 6.0, ws, Y), reps=copies)
        bytes_w = N * K + 4 * N
        emit({"case": name, "M": M, "K": K, "N": N, "us_per_layer": round(us, 3),
              "weight_stream_gbps": round(bytes_w / (us * 1e-6) / 1e9, 1),
              "eff_tops": round(2.0 * M * N * K / (us * 1e-6) / 1e12, 4),
              "us_per_layer_warm_mall_resident": round(us_w, 3),
              "timing": "hip graph of %d calls (weight rotated over %d copies; warm: one copy)"
                        % (copies, copies), "replays_identical": bool(same and same_w)})
        del Wqs, ws, Y, X

    def ev_us(fn, iters):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) * 1e3 / iters

    # two-layer MLP block, per outlier density
    for n_in in (0, 6, 32, 128, 512):
        d = synth.mlp_sweep(n_in)
        X = torch.from_numpy(d["X"]).cuda()
        M, H = d["X"].shape
        F = d["W1"].shape[0]
        Wq1, sw1 = quantize(d["W1"])
        Wq2, sw2 = quantize(d["W2"])
        ws1 = torch.empty((ops.workspace_bytes(M, H, F),), dtype=torch.uint8, device="cuda")
        ws2 = torch.empty((ops.workspace_bytes(M, F, H),), dtype=torch.uint8, device="cuda")
        Y1 = torch.empty((M, F), dtype=torch.float16, device="cuda")
        G = torch.empty_like(Y1)
        Y2 = torch.empty((M, H), dtype=torch.float16, device="cuda")
        ops.linear_int8_mixed(X, Wq1, sw1, None, 6.0, ws1, Y1)
        ops.gelu_f16(Y1, G)
        ops.linear_int8_mixed(G, Wq2, sw2, None, 6.0, ws2, Y2)
        torch.cuda.synchronize()
        n1 = int(ops.workspace_views(ws1, M, H)["n"].cpu()[0])
        n2 = int(ops.workspace_views(ws2, M, F)["n"].cpu()[0])
        t1 = ev_us(lambda: ops.linear_int8_mixed(X, Wq1, sw1, None, 6.0, ws1, Y1), 20)
        tg = ev_us(lambda: ops.gelu_f16(Y1, G), 20)
        t2 = ev_us(lambda: ops.linear_int8_mixed(G, Wq2, sw2, None, 6.0, ws2, Y2), 10)
        fl = 2.0 * M * F * H
        emit({"case": "mlp n_in=%d" % n_in, "M": M, "H": H, "F": F, "n_layer1": n1,
              "n_layer2": n2, "us_layer1": round(t1, 2), "us_gelu": round(tg, 2),
              "us_layer2": round(t2, 2), "eff_tops_layer1": round(fl / (t1 * 1e-6) / 1e12, 1),
              "eff_tops_layer2": round(fl / (t2 * 1e-6) / 1e12, 1), "timing": "hip events"})
        del Wq1, Wq2, ws1, ws2, Y1, G, Y2, X

    # the weight kept in fp16 (has_fp16_weights=True), OPT-6.7B FFN up shape:
    # W quantized at every call, and with the codes of an unchanged W given
    d = synth.opt_ffn_up()
    X = torch.from_numpy(d["X"]).cuda()
    W = torch.from_numpy(d["W"]).cuda()
    M, K = d["X"].shape
    N = W.shape[0]
    del d
    Wq = torch.empty((N, K), dtype=torch.int8, device="cuda")
    sw = torch.empty((N,), dtype=torch.float32, device="cuda")
    ws = torch.empty((ops.workspace_bytes(M, K, N),), dtype=torch.uint8, device="cuda")
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    tq = ev_us(lambda: ops.linear_int8_mixed_fp16_weights(X, W, Wq, sw, True, None, 6.0, ws, Y), 20)
    tc = ev_us(lambda: ops.linear_int8_mixed_fp16_weights(X, W, Wq, sw, False, None, 6.0, ws, Y), 20)
    fl = 2.0 * M * N * K
    emit({"case": "fp16 weights, OPT FFN up", "M": M, "K": K, "N": N,
          "us_weight_quantized_at_call": round(tq, 1), "us_codes_given": round(tc, 1),
          "eff_tops_quantized_at_call": round(fl / (tq * 1e-6) / 1e12, 1),
          "eff_tops_codes_given": round(fl / (tc * 1e-6) / 1e12, 1),
          "timing": "hip events, same buffers each call"})
    del X, W, Wq, sw, ws, Y

    # 175B-scale FFN layer
    d = synth.ffn_175b()
    X = torch.from_numpy(d["X"]).cuda()
    M, K = d["X"].shape
    W = torch.from_numpy(d["W"]).cuda()
    N = W.shape[0]
    del d
    Wq, sw = ops.int8_quantize_colwise_weight(W)
    tq = ev_us(lambda: ops.int8_quantize_colwise_weight(W, Wq, sw), 5)
    del W
    ws = torch.empty((ops.workspace_bytes(M, K, N),), dtype=torch.uint8, device="cuda")
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    t = ev_us(lambda: ops.linear_int8_mixed(X, Wq, sw, None, 6.0, ws, Y), 5)
    emit({"case": "ffn 175B-scale", "M": M, "K": K, "N": N, "us_per_layer": round(t, 1),
          "eff_tops": round(2.0 * M * N * K / (t * 1e-6) / 1e12, 1),
          "int8_peak_frac": round(2.0 * M * N * K / (t * 1e-6) / 1e12 / PEAK_INT8_TOPS, 4),
          "weight_quant_us": round(tq, 1),
          "weight_quant_gbps": round((3.0 * N * K + 4.0 * N) / (tq * 1e-6) / 1e9, 1),
          "timing": "hip events"})

    out = ["# linear_int8_mixed on every workload (one MI355X)", "",
           "Command (from the repository root):", "", "    python3 bench.py --sweep", "",
           "Decode and tiny layers: one HIP graph of many calls (weight rotated over copies "
           "beyond 2 x the 256 MB MALL), replayed; others: HIP events around back-to-back "
           "calls. Times are per whole layer call (all kernels).", ""]
    for r in rows:
        out.append("- `" + json.dumps(r) + "`")
    with open(SWEEP_FILE, "w") as f:
        f.write("\n".join(out) + "\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # The chip's clocks take on the order of 100 ms of load to settle after
    # idle; 1500 untimed steps (about 0.2 s) put the timed steps past that.
    ap.add_argument("--warmup", type=int, default=1500)
    ap.add_argument("--workload", default="opt6.7b_ffn_up", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run the copy kernel used to calibrate HBM byte counters")
    ap.add_argument("--write-counters", metavar="PMC_DIR",
                    help="write the stored GEMM traffic figure from rocprofv3 counter runs "
                         "(no GPU needed) and exit")
    ap.add_argument("--sweep", action="store_true",
                    help="time the layer on every workload and write the summary under profiles/")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="write the committed kernel-trace summary from a rocprofv3 run "
                         "(no GPU needed) and exit")
    args = ap.parse_args()
    if args.summarize_trace:
        _summarize_trace(args.summarize_trace)
        return
    if args.write_counters:
        _write_counters(args.write_counters)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        _copy_probe()
        return
    if args.sweep:
        _sweep()
        return

    import numpy as np
    import torch

    import int8_quantized_matmul_absmax_amd as i8

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

    # ---- per-step spread, from a separate pass with an event between steps
    nsp = min(args.steps, 100)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nsp + 1)]
    evs[0].record(stream)
    for i in range(nsp):
        step(i)
        evs[i + 1].record(stream)
    evs[-1].synchronize()
    step_us = np.sort([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(nsp)])
    spread = {q: round(float(np.percentile(step_us, v)), 2)
              for q, v in (("p10", 10), ("p50", 50), ("p90", 90))}

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

    # ---- CPU baseline (the oracle timed on the host), which also checks the
    # timed output on sampled rows and the weight codes against the oracle
    cpu, parity = None, None
    if not args.no_cpu_baseline:
        rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(1).choice(M, 8)]))
        Y_last = pool[(args.steps - 1) % n_sets]["Y"]
        cpu, parity = _cpu_baseline(d, M, N, K, args.cpu_seconds, Wq0.cpu().numpy(),
                                    Y_last[torch.from_numpy(rows).cuda()].cpu().numpy(), rows)

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
        "step_us_spread": spread,
        # the dense-equivalent count above split by arithmetic: int8 ops on the
        # K - n normal columns, fp16 flops on the n outlier columns
        "ops_split": {"int8_ops": 2 * M * N * (K - n_out), "fp16_flops": 2 * M * N * n_out},
        "quantize": {"x_rowwise_gbps": round(rowq_gbps, 1),
                     "x_rowwise_hbm_frac": round(rowq_gbps / PEAK_HBM_GBPS, 4),
                     "x_rowwise_ms": round(ms_rowq, 6),
                     "weight_once_gbps": round(wq_gbps, 1),
                     "weight_once_hbm_frac": round(wq_gbps / PEAK_HBM_GBPS, 4),
                     "weight_once_ms": round(t_wq, 6)},
        "parity": parity,
        "cpu_baseline": cpu,
        "rotation_sets": n_sets,
        "timed_wall_s": round(wall, 4),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
