"""Benchmark of the LLM.int8() mixed int8 linear layer on one MI355X.

Headline workload: the 175B-scale FFN layer at prefill, X fp16 [4096 x 12288]
~ N(0, 1) with 12 outlier hidden dims at +-U(10, 60), each on its own token
fraction from U(0.2, 0.6), W [49152 x 12288] ~ N(0, 0.01^2) quantized once to
int8, threshold 6.0. One step = one whole layer call (outlier detection, row
quantization and outlier gather, int8 GEMM with the fused dequantize + fp16
outlier product + fp16 store). Inputs are resident in HBM before the timed
region; every step streams more than 1 GB, four times the 256 MB Infinity
Cache (MALL), and two input/output sets are rotated.

Before each timed loop an untimed, time-based pre-warm runs the same work for
at least --prewarm-ms (the chip's clocks take on the order of 100 ms of load
to settle after idle), then --warmup untimed steps.

Prints ONE JSON line (N=1):
  value         effective TOPS = 2*M*N*K / step time (whole layer, all kernels)
  roofline      the int8 GEMM kernel alone (k_gemm_i8, the dominant kernel)
                against the MFMA roofline: its algorithmic work, 2*M*N*(K-n)
                int8 ops at the int8 peak (5.0 POP/s) plus 2*M*N*n fp16 flops
                at the fp16 peak (2.5 PFLOP/s), over its average duration from
                HIP events on the launch stream
  cpu_baseline  the CPU oracle timed on this host on a bounded row sample
  extras        the OPT-6.7B FFN-up layer; decode M = 1, 4, 16 (weight rotated
                beyond 2 x MALL, HIP-graph timed); the tiny 16 x 256 -> 256
                layer's per-call cost, eager and HIP-graph; the activation side and the
                one-time weight quantization against HBM (inputs rotated
                beyond 2 x MALL); the two-layer MLP outlier-density sweep; a
                plain device copy's bandwidth (the measured HBM ceiling)

  python bench.py [--gpus 1] [--steps 100] [--warmup 20] [--prewarm-ms 500]
  python bench.py --profile-kernels      # eager runs of every kernel for rocprofv3
  python bench.py --write-counters DIR   # stored counter figures (no GPU)
  python bench.py --summarize-trace DIR  # stored kernel-trace summary (no GPU)
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
PEAK_FP16_TFLOPS = 2500.0    # MI355X dense fp16 MFMA, TFLOP/s
PEAK_HBM_GBPS = 8000.0       # MI355X HBM3E, GB/s
MALL_BYTES = 256 << 20       # Infinity Cache

WORKLOADS = {
    "ffn175b": dict(M=4096, K=12288, N=49152),
    "opt6.7b_ffn_up": dict(M=2048, K=4096, N=16384),
}
HEADLINE = "ffn175b"
DESCRIPTION = {
    "ffn175b": "175B-scale FFN layer at prefill: X fp16 [4096 x 12288], W [49152 x 12288] "
               "quantized once to int8, 12 outlier dims on 20-60% of tokens, threshold 6",
    "opt6.7b_ffn_up": "OPT-6.7B FFN up-projection at prefill: X fp16 [2048 x 4096], "
                      "W [16384 x 4096] quantized once to int8, 6 outlier dims on 25% of "
                      "tokens, threshold 6",
}

CSRC = os.path.join(ROOT, "int8_quantized_matmul_absmax_amd", "csrc")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "pmc_counters.json")
COUNTERS_MD = os.path.join(ROOT, "profiles", "pmc_counters_all_kernels.md")
TRACE_FILE = os.path.join(ROOT, "profiles", "k_gemm_i8_ffn175b_kernel_trace.md")
COPY_PROBE_BYTES = 512 << 20


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def _make(workload):
    from int8_quantized_matmul_absmax_amd import synth
    if workload == "opt6.7b_ffn_up":
        return synth.opt_ffn_up()
    if workload == "ffn175b":
        return synth.ffn_175b()
    raise ValueError(workload)


def _kernel_code_sha256(paths=None):
    """SHA-256 of the HIP sources' code (comments removed, whitespace
    collapsed, files in name order), so that only a change of code, not of its
    comments, invalidates counters taken on it."""
    if paths is None:
        paths = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                       if f.endswith((".hip", ".h")))
    h = hashlib.sha256()
    for p in paths:
        text = open(p).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(os.path.basename(p).encode() + b"\0" + " ".join(text.split()).encode() + b"\0")
    return h.hexdigest()


# ---------------------------------------------------------------- timing

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


def _prewarm(fn, ms):
    """Untimed calls of fn(i) until at least `ms` of wall time has passed
    (synchronizing every few calls, so the time is the GPU's). Returns
    (elapsed ms, calls)."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(8):
            fn(i)
            i += 1
        torch.cuda.synchronize()
        el = (time.perf_counter() - t0) * 1e3
        if el >= ms:
            return el, i


def _timed(fn, steps, warmup, prewarm_ms, stream):
    """Pre-warm, warm-up, then the mean time (ms) of `steps` calls between two
    HIP events on `stream`."""
    import torch
    pw = _prewarm(fn, prewarm_ms) if prewarm_ms > 0 else (0.0, 0)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    return _event_time_ms(fn, steps, stream), pw


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
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.3:   # settle the clocks
        g.replay()
        torch.cuda.synchronize()
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    end.synchronize()
    same &= bool(torch.equal(outs[-1], ref))
    return start.elapsed_time(end) * 1e3 / (replays * reps), same


def _mfma_roofline(M, N, K, n, ms):
    """The GEMM's algorithmic work at its two peaks: 2MN(K-n) int8 ops and
    2MNn fp16 flops. Returns (achieved TOP/s, peak TOP/s, frac, ops)."""
    i8 = 2.0 * M * N * (K - n)
    f16 = 2.0 * M * N * n
    t_ideal_s = i8 / (PEAK_INT8_TOPS * 1e12) + f16 / (PEAK_FP16_TFLOPS * 1e12)
    t_s = ms * 1e-3
    ops = i8 + f16
    return ops / t_s / 1e12, ops / t_ideal_s / 1e12, t_ideal_s / t_s, ops


# ---------------------------------------------------------------- measurements

def _measure_layer(ops, d, steps, warmup, prewarm_ms, stream, keep_pool=False):
    """The whole layer on one workload: one-time weight quantization (cold),
    then the layer step over rotated sets, its per-step spread, and the GEMM
    alone on the last step's intermediates (same launch configuration)."""
    import numpy as np
    import torch
    X_h, W_h = d["X"], d["W"]
    M, K = X_h.shape
    N = W_h.shape[0]

    # one-time weight quantization (a4): W copies beyond 2 x MALL, so each
    # call reads its W from HBM
    W_dev = [torch.from_numpy(W_h).cuda()]
    n_wc = max(1, min(4, (2 * MALL_BYTES) // W_h.nbytes + 1))
    for _ in range(n_wc - 1):
        W_dev.append(W_dev[0].clone())
    Wq0, sw0 = ops.int8_quantize_colwise_weight(W_dev[0])
    Wq_b = [torch.empty_like(Wq0) for _ in W_dev]
    sw_b = [torch.empty_like(sw0) for _ in W_dev]

    def wquant(i):
        j = i % len(W_dev)
        ops.int8_quantize_colwise_weight(W_dev[j], Wq_b[j], sw_b[j])
    t_wq, _ = _timed(wquant, max(4, n_wc), 1, min(prewarm_ms, 200), stream)
    wq_bytes = 3.0 * N * K + 4.0 * N
    del W_dev, Wq_b, sw_b

    # rotation pool of (X, Wq, sw, Y, workspace) sets beyond 2 x MALL
    ws_bytes = ops.workspace_bytes(M, K)
    set_bytes = X_h.nbytes + N * K + 2 * M * N + ws_bytes
    n_sets = int(max(2, min(8, (2 * MALL_BYTES) // max(set_bytes, 1) + 1)))
    X0 = torch.from_numpy(X_h).cuda()
    pool = []
    for s in range(n_sets):
        pool.append(dict(X=X0 if s == 0 else X0.clone(), Wq=Wq0 if s == 0 else Wq0.clone(),
                         sw=sw0 if s == 0 else sw0.clone(),
                         Y=torch.empty((M, N), dtype=torch.float16, device="cuda"),
                         ws=torch.empty((ws_bytes,), dtype=torch.uint8, device="cuda")))
    torch.cuda.synchronize()

    def step(i):
        p = pool[i % n_sets]
        ops.linear_int8_mixed(p["X"], p["Wq"], p["sw"], None, 6.0, p["ws"], p["Y"])

    t0 = time.perf_counter()
    ms_step, pw = _timed(step, steps, warmup, prewarm_ms, stream)
    wall = time.perf_counter() - t0
    last_set = (steps - 1) % n_sets

    # per-step spread: a separate pass with an event between steps
    nsp = min(steps, 100)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nsp + 1)]
    evs[0].record(stream)
    for i in range(nsp):
        step(i)
        evs[i + 1].record(stream)
    evs[-1].synchronize()
    step_us = np.sort([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(nsp)])
    spread = {q: round(float(np.percentile(step_us, v)), 2)
              for q, v in (("p10", 10), ("p50", 50), ("p90", 90))}

    # the dominant kernel alone: int8 GEMM + fused epilogue, from the
    # intermediates the layer left in each set's workspace
    views = [ops.workspace_views(p["ws"], M, K) for p in pool]
    n_out = int(views[0]["n"].cpu().numpy()[0])
    Yg = [torch.empty((M, N), dtype=torch.float16, device="cuda") for _ in pool]

    def gemm(i):
        p, v = pool[i % n_sets], views[i % n_sets]
        ops.int8_mm_dequant(v["Xq"], p["Wq"], v["sx"], p["sw"], v["Xo"], v["cols"], v["n"],
                            None, out=Yg[i % n_sets])
    ms_gemm, pw_g = _timed(gemm, steps, warmup, prewarm_ms, stream)
    ach, peak, frac, ops_launch = _mfma_roofline(M, N, K, n_out, ms_gemm)
    out = {"M": M, "K": K, "N": N, "n_outliers": n_out, "ms_per_step": ms_step,
           "eff_tops": 2.0 * M * N * K / (ms_step * 1e-3) / 1e12, "spread": spread,
           "prewarm": {"ms": round(pw[0], 1), "steps": pw[1]}, "wall_s": wall,
           "gemm_ms": ms_gemm, "gemm_achieved": ach, "gemm_peak": peak, "gemm_frac": frac,
           "gemm_ops": ops_launch, "rotation_sets": n_sets,
           "weight_once_ms": t_wq, "weight_once_gbps": wq_bytes / (t_wq * 1e-3) / 1e9}
    if keep_pool:
        out["_pool"], out["_last_set"], out["_Wq"] = pool, last_set, Wq0
    else:
        del pool, views, Yg
    return out


def _measure_x_side(ops, X_h, prewarm_ms, stream, iters=50):
    """The layer's activation side alone (outlier_detect_quantize: detection,
    then the row pass that gathers and quantizes), X rotated over copies
    beyond 2 x MALL. Algorithmic bytes: the detection reads X (2MK), the row
    pass reads X (2MK) and writes Xq (MK), sx (4M) and Xo (2 M LD(n))."""
    import torch
    M, K = X_h.shape
    ws_bytes = ops.workspace_bytes(M, K)
    touched = 3 * M * K
    n_sets = int(max(2, min(32, (2 * MALL_BYTES) // max(touched, 1) + 1)))
    X0 = torch.from_numpy(X_h).cuda()
    Xs = [X0] + [X0.clone() for _ in range(n_sets - 1)]
    wss = [torch.empty((ws_bytes,), dtype=torch.uint8, device="cuda") for _ in range(n_sets)]

    def xs(i):
        ops.outlier_detect_quantize(Xs[i % n_sets], 6.0, wss[i % n_sets])
    ms, _ = _timed(xs, iters, 4, prewarm_ms, stream)
    n = int(ops.workspace_views(wss[0], M, K)["n"].cpu().numpy()[0])
    algo = 5.0 * M * K + 4.0 * M + 2.0 * M * ops.outlier_ld(n)
    del Xs, wss
    return {"M": M, "K": K, "n_outliers": n, "us": round(ms * 1e3, 2),
            "algorithmic_bytes": int(algo), "gbps": round(algo / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(algo / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "rotation_sets": n_sets,
            "timing": "hip events, X and workspace rotated over %d sets (%.0f MB touched)"
                      % (n_sets, n_sets * touched / 1e6)}


def _measure_decode(ops):
    """Decode-shaped layers (M = 1, 4, 16 tokens, 4096 -> 4096): one HIP graph
    of many calls, the int8 weight rotated over copies beyond 2 x MALL (each
    call streams its weight from HBM); also the warm (MALL-resident) time."""
    import torch
    from int8_quantized_matmul_absmax_amd import synth
    res = {}
    for m in (1, 4, 16):
        d = synth.decode(m)
        X = torch.from_numpy(d["X"]).cuda()
        M, K = d["X"].shape
        Wq, sw = ops.int8_quantize_colwise_weight(torch.from_numpy(d["W"]).cuda())
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
        us_w, same_w = _graph_time_us(
            lambda: ops.linear_int8_mixed(X, Wq, sw, None, 6.0, ws, Y), reps=copies)
        algo = N * K + 4 * N + 2 * M * K + 2 * M * N
        res["M%d" % m] = {"M": M, "K": K, "N": N, "us": round(us, 3),
                          "gbps": round(algo / (us * 1e-6) / 1e9, 1),
                          "hbm_frac": round(algo / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                          "us_warm_mall": round(us_w, 3), "algorithmic_bytes": algo,
                          "replays_identical": bool(same and same_w)}
        del Wqs, ws, Y, X
    res["timing"] = ("hip graph of many calls, replayed; weight rotated over copies beyond "
                     "2 x MALL; warm: one weight copy")
    return res


def _measure_tiny(ops):
    """The tiny layer (16 x 256 -> 256, one launch of the few-token kernel):
    what a call costs when there is almost no work. Timed eagerly (HIP events
    around 200 calls on the current stream, host launch overhead included)
    and from a HIP graph of 50 calls (GPU time only)."""
    import torch
    from int8_quantized_matmul_absmax_amd import synth
    d = synth.tiny()
    X = torch.from_numpy(d["X"]).cuda()
    Wq, sw = ops.int8_quantize_colwise_weight(torch.from_numpy(d["W"]).cuda())
    M, K = X.shape
    N = Wq.shape[0]
    ws = torch.empty((ops.workspace_bytes(M, K, N),), dtype=torch.uint8, device="cuda")
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")

    def call():
        return ops.linear_int8_mixed(X, Wq, sw, None, 6.0, ws, Y)
    for _ in range(50):
        call()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(200):
        call()
    end.record()
    end.synchronize()
    eager = start.elapsed_time(end) * 1e3 / 200
    us_g, same = _graph_time_us(call, reps=50)
    return {"M": M, "K": K, "N": N, "us_eager_per_call": round(eager, 3),
            "us_graph_per_call": round(us_g, 3), "replays_identical": bool(same),
            "timing": "eager: hip events around 200 calls (launch overhead included); "
                      "graph: 50 calls per graph, replayed"}


def _measure_mlp(ops, prewarm_ms, stream):
    """The two-layer MLP block (1024 x 4096 -> 16384 -> GELU -> 4096) per
    planted outlier density: layer times, layer 2's emergent outlier count,
    and each layer's GEMM roofline fraction (int8 and fp16 work at their own
    peaks). Layer 2 is timed with the default workspace (room for 512 outlier
    weight columns) and with one that has room for every count. Same buffers
    every call (the 67 MB weights may sit in the MALL)."""
    import torch
    from int8_quantized_matmul_absmax_amd import synth
    rows = []
    for n_in in (0, 6, 32, 128, 512):
        d = synth.mlp_sweep(n_in)
        X = torch.from_numpy(d["X"]).cuda()
        M, H = d["X"].shape
        F = d["W1"].shape[0]
        Wq1, sw1 = ops.int8_quantize_colwise_weight(torch.from_numpy(d["W1"]).cuda())
        Wq2, sw2 = ops.int8_quantize_colwise_weight(torch.from_numpy(d["W2"]).cuda())
        del d
        ws1 = torch.empty((ops.workspace_bytes(M, H, F),), dtype=torch.uint8, device="cuda")
        ws2 = torch.empty((ops.workspace_bytes(M, F, H),), dtype=torch.uint8, device="cuda")
        ws2_all = torch.empty((ops.workspace_bytes_all_outliers(M, F, H),), dtype=torch.uint8,
                              device="cuda")
        Y1 = torch.empty((M, F), dtype=torch.float16, device="cuda")
        G = torch.empty_like(Y1)
        Y2 = torch.empty((M, H), dtype=torch.float16, device="cuda")
        ops.linear_int8_mixed(X, Wq1, sw1, None, 6.0, ws1, Y1)
        ops.gelu_f16(Y1, G)
        ops.linear_int8_mixed(G, Wq2, sw2, None, 6.0, ws2, Y2)
        torch.cuda.synchronize()
        n1 = int(ops.workspace_views(ws1, M, H)["n"].cpu()[0])
        n2 = int(ops.workspace_views(ws2, M, F)["n"].cpu()[0])
        pw = prewarm_ms if n_in == 0 else min(prewarm_ms, 150)
        t1, _ = _timed(lambda i: ops.linear_int8_mixed(X, Wq1, sw1, None, 6.0, ws1, Y1), 20, 2,
                       pw, stream)
        tg, _ = _timed(lambda i: ops.gelu_f16(Y1, G), 20, 2, 0, stream)
        t2, _ = _timed(lambda i: ops.linear_int8_mixed(G, Wq2, sw2, None, 6.0, ws2, Y2), 20, 2,
                       min(prewarm_ms, 150), stream)
        t2a, _ = _timed(lambda i: ops.linear_int8_mixed(G, Wq2, sw2, None, 6.0, ws2_all, Y2), 20,
                        2, min(prewarm_ms, 150), stream)
        _, _, f1, _ = _mfma_roofline(M, F, H, n1, t1)
        _, _, f2, _ = _mfma_roofline(M, H, F, n2, t2)
        _, _, f2a, _ = _mfma_roofline(M, H, F, n2, t2a)
        rows.append({"n_in": n_in, "n_layer1": n1, "n_layer2": n2,
                     "us_layer1": round(t1 * 1e3, 2), "us_gelu": round(tg * 1e3, 2),
                     "us_layer2": round(t2 * 1e3, 2),
                     "us_layer2_room_all": round(t2a * 1e3, 2),
                     "layer1_mfma_frac": round(f1, 4), "layer2_mfma_frac": round(f2, 4),
                     "layer2_room_all_mfma_frac": round(f2a, 4),
                     "layer2_fp16_flops": 2 * M * H * n2})
        del X, Wq1, Wq2, ws1, ws2, ws2_all, Y1, G, Y2
    base = rows[0]
    for r in rows:
        r["overhead_us_vs_n0"] = round(r["us_layer1"] + r["us_layer2"]
                                       - base["us_layer1"] - base["us_layer2"], 2)
    return {"rows": rows, "shape": "1024 x 4096 -> 16384 -> GELU -> 4096",
            "timing": "hip events, whole layer calls, same buffers each call"}


def _measure_copy(prewarm_ms, stream):
    """A plain device-to-device copy of 1 GiB (2 GiB moved per call): the
    bandwidth this chip reaches on a streaming kernel, beside the 8 TB/s
    published peak."""
    import torch
    nbytes = 1 << 30
    src = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    ms, _ = _timed(lambda i: dst.copy_(src), 10, 2, min(prewarm_ms, 200), stream)
    del src, dst
    return {"bytes_moved": 2 * nbytes, "us": round(ms * 1e3, 1),
            "gbps": round(2.0 * nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_8tbps": round(2.0 * nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}


def _cpu_baseline(d, M, N, K, target_s, Wq_gpu, Y_rows, rows_y, label):
    """The oracle as it stands, on a bounded sample of rows: outlier detection
    over all rows, then quantization, int32 GEMM, outlier product and
    dequantization for S sampled rows x all N outputs. Scaled to TOPS by the
    dense-equivalent 2*S*N*K. The same leg checks the timed GPU output against
    the oracle on the rows rows_y (Y_rows, host copy) and the GPU weight codes
    (Wq_gpu, host copy) bit for bit."""
    import numpy as np
    from oracle import llm_int8 as O
    t0 = time.perf_counter()
    Wq_ref, sw_ref = O.quantize_weight_rows(d["W"])
    t_wquant = time.perf_counter() - t0
    ref = O.linear_int8_mixed(d["X"], Wq_ref, sw_ref, 6.0, rows=rows_y)
    Yr = np.asarray(ref["Y"], np.float64)
    dY = np.abs(np.asarray(Y_rows, np.float64) - Yr)
    floor = 1e-2 * np.abs(Yr).max()
    parity = {"y_max_abs_rel_err_sampled_rows": O.max_abs_rel_error(Y_rows, ref["Y"]),
              # per element, relative to max(|Y_ref|, 1e-2 max |Y_ref|)
              "y_elem_rel_err_floor_1e-2_sampled_rows":
                  float((dY / np.maximum(np.abs(Yr), floor)).max()) if Yr.size else 0.0,
              "rows_checked": int(np.asarray(rows_y).size), "features_checked": int(N),
              "weight_codes_bitexact": bool(np.array_equal(Wq_gpu, Wq_ref))}
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    rng = np.random.default_rng(0)
    S = 16
    while True:
        rows = np.sort(rng.choice(M, size=min(S, M), replace=False))
        t0 = time.perf_counter()
        O.linear_int8_mixed(d["X"], Wq_ref, sw_ref, 6.0, rows=rows)
        dt = time.perf_counter() - t0
        if dt >= target_s or S >= M:
            break
        S = min(M, max(S * 2, int(S * target_s / max(dt, 1e-3) * 1.1)))
    calls, total = 1, dt
    while total < target_s:
        t0 = time.perf_counter()
        O.linear_int8_mixed(d["X"], Wq_ref, sw_ref, 6.0, rows=rows)
        total += time.perf_counter() - t0
        calls += 1
    dt = total / calls
    tops = 2.0 * rows.size * N * K / dt / 1e12
    # the tiny config (16 x 256 -> 256) on one thread: the whole layer call,
    # weight quantization included, best of 20
    tiny_ms = None
    try:
        from threadpoolctl import threadpool_limits
        from int8_quantized_matmul_absmax_amd import synth
        t = synth.tiny()
        with threadpool_limits(limits=1):
            best = float("inf")
            for _ in range(20):
                t0 = time.perf_counter()
                Wq_t, sw_t = O.quantize_weight_rows(t["W"])
                O.linear_int8_mixed(t["X"], Wq_t, sw_t, 6.0)
                best = min(best, time.perf_counter() - t0)
        tiny_ms = round(best * 1e3, 3)
    except ImportError:
        pass
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                         None)
    except OSError:
        pass
    return ({"value": round(tops, 6), "unit": "TOPS", "cores": int(threads), "kind": "oracle",
             "sample": "%d of %d token rows x all %d outputs of the %s layer (outlier "
                       "detection over all rows; weight quantization outside the timing), "
                       "%d call(s), %.2f s each" % (rows.size, M, N, label, calls, dt),
             "weight_quant_s": round(t_wquant, 3),
             "weight_quant_note": "the oracle's per-row weight quantization of the whole "
                                  "[%d x %d] weight, once, same threads" % (N, K),
             "tiny_16x256x256_single_thread_ms": tiny_ms,
             "host": {"cpu_model": model, "logical_cpus": os.cpu_count(),
                      "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}}, parity)


def _traffic_from_counters(section):
    """HBM bytes per launch of the GEMM on `section` from the stored counter
    runs (FETCH_SIZE + WRITE_SIZE, each scaled by the copy probe), or None when
    absent or taken on a different version of the kernel code."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
        if c.get("kernel_code_sha256") != _kernel_code_sha256():
            return None
        return float(c["sections"][section]["kernels"]["k_gemm_i8"]["fetch_write_bytes"])
    except (OSError, KeyError, ValueError, TypeError):
        return None


# ---------------------------------------------------------------- profiling mode

PROFILE_SECTIONS = ("copy_probe", "ffn175b_weight_quant", "ffn175b_layer", "opt6.7b_layer",
                    "decode_m1", "decode_m4", "decode_m16", "mlp_n32_layer2",
                    "mlp_n32_layer2_room_all")


def _profile_kernels():
    """Eager runs of every kernel of the path on the benchmark's workloads, for
    rocprofv3 counter and trace runs. Sections are separated by a marker
    dispatch (a float64 fill of one element) and listed on stdout as JSON, so
    the counter summary can assign each dispatch to its section."""
    import torch
    import int8_quantized_matmul_absmax_amd as i8
    from int8_quantized_matmul_absmax_amd import synth
    i8.ensure_built()
    ops = i8.ops
    torch.cuda.set_device(0)
    mark_buf = torch.empty((1,), dtype=torch.float64, device="cuda")

    def mark():
        torch.cuda.synchronize()
        mark_buf.fill_(1.0)
        torch.cuda.synchronize()

    done = []

    def section(name):
        """Start of a section's measured work (its end is the next end())."""
        mark()
        done.append(name)
        log("profile section " + name)

    def end():
        mark()

    # copy probe: a plain copy of known size (the counters' calibration)
    src = torch.empty((COPY_PROBE_BYTES,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(3)
    torch.cuda.synchronize()
    section("copy_probe")
    for _ in range(3):
        dst.copy_(src)
    end()
    del src, dst

    d = synth.ffn_175b()
    W = torch.from_numpy(d["W"]).cuda()
    X = torch.from_numpy(d["X"]).cuda()
    M, K = d["X"].shape
    N = W.shape[0]
    Wq, sw = ops.int8_quantize_colwise_weight(W)
    section("ffn175b_weight_quant")
    for _ in range(2):
        ops.int8_quantize_colwise_weight(W, Wq, sw)
    end()
    del W
    ws = torch.empty((ops.workspace_bytes(M, K),), dtype=torch.uint8, device="cuda")
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    section("ffn175b_layer")
    for _ in range(3):
        ops.linear_int8_mixed(X, Wq, sw, None, 6.0, ws, Y)
    end()
    del X, Wq, sw, ws, Y, d

    d = synth.opt_ffn_up()
    M, K = d["X"].shape
    N = d["W"].shape[0]
    Wq0, sw = ops.int8_quantize_colwise_weight(torch.from_numpy(d["W"]).cuda())
    sets = [(torch.from_numpy(d["X"]).cuda(), Wq0 if s == 0 else Wq0.clone(),
             torch.empty((ops.workspace_bytes(M, K),), dtype=torch.uint8, device="cuda"),
             torch.empty((M, N), dtype=torch.float16, device="cuda")) for s in range(4)]
    section("opt6.7b_layer")
    for i in range(4):
        Xs, Wqs, wss, Ys = sets[i]
        ops.linear_int8_mixed(Xs, Wqs, sw, None, 6.0, wss, Ys)
    end()
    del sets, Wq0, d

    for m in (1, 4, 16):
        d = synth.decode(m)
        X = torch.from_numpy(d["X"]).cuda()
        M, K = d["X"].shape
        Wq0, sw = ops.int8_quantize_colwise_weight(torch.from_numpy(d["W"]).cuda())
        N = Wq0.shape[0]
        copies = [Wq0] + [Wq0.clone() for _ in range(35)]
        ws = torch.empty((ops.workspace_bytes(M, K),), dtype=torch.uint8, device="cuda")
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        section("decode_m%d" % m)
        for i in range(3):
            ops.linear_int8_mixed(X, copies[7 * i + 3], sw, None, 6.0, ws, Y)
        end()
        del copies, X, ws, Y, d

    d = synth.mlp_sweep(32)
    X = torch.from_numpy(d["X"]).cuda()
    M, H = d["X"].shape
    F = d["W1"].shape[0]
    Wq1, sw1 = ops.int8_quantize_colwise_weight(torch.from_numpy(d["W1"]).cuda())
    Wq2, sw2 = ops.int8_quantize_colwise_weight(torch.from_numpy(d["W2"]).cuda())
    G = ops.gelu_f16(ops.linear_int8_mixed(X, Wq1, sw1, None, 6.0))
    ws2 = torch.empty((ops.workspace_bytes(M, F, H),), dtype=torch.uint8, device="cuda")
    Y2 = torch.empty((M, H), dtype=torch.float16, device="cuda")
    section("mlp_n32_layer2")
    for _ in range(2):
        ops.linear_int8_mixed(G, Wq2, sw2, None, 6.0, ws2, Y2)
    end()
    # the same layer with room in the workspace for every outlier column
    del ws2
    ws2 = torch.empty((ops.workspace_bytes_all_outliers(M, F, H),), dtype=torch.uint8,
                      device="cuda")
    section("mlp_n32_layer2_room_all")
    for _ in range(2):
        ops.linear_int8_mixed(G, Wq2, sw2, None, 6.0, ws2, Y2)
    end()
    torch.cuda.synchronize()
    print(json.dumps({"profile_sections": done}), flush=True)


def _dispatches(csv_path):
    """Dispatches of a rocprofv3 csv (counter collection or kernel trace) in
    dispatch order: [(dispatch id, kernel name, {counter: value}, duration ns
    or None)]. Rows without a dispatch id are ordered by start time."""
    import csv
    rows = list(csv.DictReader(open(csv_path)))
    out = {}
    for i, r in enumerate(rows):
        did = r.get("Dispatch_Id") or r.get("Dispatch_ID")
        if did in (None, ""):
            did = int(r["Start_Timestamp"]) if r.get("Start_Timestamp") else i
        did = int(did)
        e = out.setdefault(did, [r["Kernel_Name"], {}, None])
        if r.get("Counter_Name"):
            e[1][r["Counter_Name"]] = e[1].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        if r.get("Start_Timestamp") and r.get("End_Timestamp"):
            e[2] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return [(k, v[0], v[1], v[2]) for k, v in sorted(out.items())]


def _short(name):
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    base = name.split("(")[0]
    m = re.match(r"[\w:]*?(k_\w+)(<[^()]*>)?", base)
    return (m.group(1) + (m.group(2) or "")) if m else base[:60]


def _family(name):
    """Kernel family of a dispatch: the kernel's name without its template
    arguments, except the GEMM's two segment modes (its last template
    argument: 2 the compact outlier segment, 3 and 4 the dense one, with
    the weight as int8 codes or kept in fp16), which are listed apart: the
    layer launches the plain mode and a segment mode, and the one whose case
    it is not returns at once; other kernels (the copy probe) by what they
    are."""
    s = _short(name)
    if s.startswith("k_gemm_i8"):
        if re.search(r",\s*2>$", s):
            return "k_gemm_i8_outlier_seg"
        if re.search(r",\s*[34]>$", s):
            return "k_gemm_i8_dense_seg"
        return "k_gemm_i8"
    return s.split("<")[0] if s.startswith("k_") else ("copy" if "copy" in name.lower() else s)


def _is_marker(name):
    return "fill" in name.lower() and "double" in name.lower()


def _split_sections(disp, sections):
    """Dispatch list -> {section: [dispatches]}: section j is what lies between
    the marker fills 2j and 2j+1 (its start and end); the set-up work between
    one section's end and the next one's start belongs to none."""
    marks = [i for i, d in enumerate(disp) if _is_marker(d[1])]
    if len(marks) != 2 * len(sections):
        raise SystemExit("expected %d marker dispatches, found %d" % (2 * len(sections), len(marks)))
    return {name: disp[marks[2 * j] + 1:marks[2 * j + 1]] for j, name in enumerate(sections)}


SECTION_WORK = {
    # algorithmic bytes per dispatch of each kernel family, per section
    "copy_probe": {"copy": 2 * COPY_PROBE_BYTES},
}


def _write_counters(pmc_dir):
    """Per-kernel counter figures from five rocprofv3 runs of
    `bench.py --profile-kernels` (trace, mfma, dram, fetch, write under
    pmc_dir), written to profiles/pmc_counters.json and a markdown table.

    Bytes: DRAM-side requests (TCC_EA0_RDREQ_DRAM / TCC_EA0_WRREQ_DRAM) and
    FETCH_SIZE / WRITE_SIZE, each scaled by known bytes / the counter's
    reading on the copy probe. MFMA: busy cycles summed over all SIMDs over
    (active cycles of one XCD x 1024 SIMDs); effective clock = active cycles
    of one XCD / kernel duration."""
    sections = json.load(open(os.path.join(pmc_dir, "manifest.json")))["profile_sections"]
    runs = {}
    for run in ("trace", "mfma", "dram", "fetch", "write", "lds"):
        if run == "lds" and not os.path.isdir(os.path.join(pmc_dir, run)):
            continue
        sub = os.path.join(pmc_dir, run)
        f = [x for x in os.listdir(sub) if x.endswith(("counter_collection.csv", "kernel_trace.csv"))]
        runs[run] = _split_sections(_dispatches(os.path.join(sub, f[0])), sections)

    def mean(run, sec, fam, key):
        vals = [d[2].get(key) for d in runs[run][sec] if _family(d[1]) == fam and key in d[2]]
        return sum(vals) / len(vals) if vals else None

    def durs(sec, fam, run="trace"):
        v = [d[3] for d in runs[run][sec] if _family(d[1]) == fam and d[3]]
        return sum(v) / len(v) if v else None

    def per_dispatch(run, sec, fam, f):
        """Mean over the family's dispatches of f(counters, duration ns)."""
        v = [f(d[2], d[3]) for d in runs[run][sec] if _family(d[1]) == fam and d[3]]
        v = [x for x in v if x is not None]
        return sum(v) / len(v) if v else None

    cp = "copy_probe"
    known = 2.0 * COPY_PROBE_BYTES
    known_half = float(COPY_PROBE_BYTES)
    rd_scale = known_half / mean("dram", cp, "copy", "TCC_EA0_RDREQ_DRAM_sum")
    wr_scale = known_half / mean("dram", cp, "copy", "TCC_EA0_WRREQ_DRAM_sum")
    fe_scale = known_half / (1024.0 * mean("fetch", cp, "copy", "FETCH_SIZE"))
    wz_scale = known_half / (1024.0 * mean("write", cp, "copy", "WRITE_SIZE"))
    rec = {"kernel_code_sha256": _kernel_code_sha256(),
           "commands": [
               "rocprofv3 --kernel-trace --output-format csv -d %s/trace -o run -- "
               "python3 bench.py --profile-kernels" % pmc_dir,
               "rocprofv3 --pmc GRBM_GUI_ACTIVE GRBM_COUNT SQ_VALU_MFMA_BUSY_CYCLES "
               "SQ_INSTS_VALU_MFMA_MOPS_I8 SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_BUSY_CYCLES "
               "--output-format csv -d %s/mfma -o run -- python3 bench.py --profile-kernels"
               % pmc_dir,
               "rocprofv3 --pmc TCC_EA0_RDREQ_DRAM_sum TCC_EA0_WRREQ_DRAM_sum GRBM_GUI_ACTIVE "
               "--output-format csv -d %s/dram -o run -- python3 bench.py --profile-kernels"
               % pmc_dir,
               "rocprofv3 --pmc FETCH_SIZE --output-format csv -d %s/fetch -o run -- "
               "python3 bench.py --profile-kernels" % pmc_dir,
               "rocprofv3 --pmc WRITE_SIZE --output-format csv -d %s/write -o run -- "
               "python3 bench.py --profile-kernels" % pmc_dir,
               "rocprofv3 --pmc SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS_LOAD_BANDWIDTH "
               "SQ_LDS_DATA_FIFO_FULL SQ_WAIT_INST_LDS SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE "
               "--output-format csv -d %s/lds -o run -- python3 bench.py --profile-kernels"
               % pmc_dir,
               "python3 bench.py --profile-kernels > %s/manifest.json" % pmc_dir,
               "python3 bench.py --write-counters %s" % pmc_dir],
           "calibration": {
               "copy_probe_bytes_read": COPY_PROBE_BYTES, "copy_probe_bytes_written": COPY_PROBE_BYTES,
               "dram_read_bytes_per_request": round(rd_scale, 3),
               "dram_write_bytes_per_request": round(wr_scale, 3),
               "fetch_size_scale": round(fe_scale, 4), "write_size_scale": round(wz_scale, 4)},
           "notes": "DRAM-side counters count L2 requests to the memory fabric; the 256 MB "
                    "MALL sits behind them, so they bound HBM bytes from above. FETCH_SIZE and "
                    "WRITE_SIZE count L2-to-fabric traffic. MFMA busy: summed SQ_VALU_MFMA_BUSY_"
                    "CYCLES over (GRBM_GUI_ACTIVE of one XCD x 1024 SIMDs).",
           "sections": {}}
    for sec in sections:
        fams = []
        for d in runs["trace"][sec]:
            f = _family(d[1])
            if f not in fams and not ("fill" in d[1].lower() and "double" in d[1].lower()):
                fams.append(f)
        ks = {}
        for fam in fams:
            t_ns = durs(sec, fam)
            e = {"avg_duration_us": round(t_ns / 1e3, 3) if t_ns else None}
            rd = mean("dram", sec, fam, "TCC_EA0_RDREQ_DRAM_sum")
            wr = mean("dram", sec, fam, "TCC_EA0_WRREQ_DRAM_sum")
            if rd is not None:
                e["dram_read_bytes"] = round(rd * rd_scale)
                e["dram_write_bytes"] = round(wr * wr_scale)
            fe = mean("fetch", sec, fam, "FETCH_SIZE")
            wz = mean("write", sec, fam, "WRITE_SIZE")
            if fe is not None and wz is not None:
                e["fetch_bytes"] = round(fe * 1024.0 * fe_scale)
                e["write_bytes"] = round(wz * 1024.0 * wz_scale)
                e["fetch_write_bytes"] = e["fetch_bytes"] + e["write_bytes"]
            act = mean("mfma", sec, fam, "GRBM_GUI_ACTIVE")
            busy = mean("mfma", sec, fam, "SQ_VALU_MFMA_BUSY_CYCLES")
            mi8 = mean("mfma", sec, fam, "SQ_INSTS_VALU_MFMA_MOPS_I8")
            mf16 = mean("mfma", sec, fam, "SQ_INSTS_VALU_MFMA_MOPS_F16")
            if act:
                act1 = act / 8.0     # GRBM_GUI_ACTIVE summed over the 8 XCDs
                e["active_cycles_per_xcd"] = round(act1)
                # clock: active cycles of one XCD over the same dispatch's own
                # duration in the counter run
                clk = per_dispatch("mfma", sec, fam,
                                   lambda c, t: c["GRBM_GUI_ACTIVE"] / 8.0 / t
                                   if "GRBM_GUI_ACTIVE" in c else None)
                if clk is not None:
                    e["effective_clock_ghz"] = round(clk, 3)
                    e["duration_us_counter_run"] = round(durs(sec, fam, "mfma") / 1e3, 3)
                if busy is not None:
                    e["mfma_busy_frac"] = round(busy / (act1 * 1024.0), 4)
                if mi8 is not None:
                    e["mfma_i8_ops"] = round(mi8 * 512)
                if mf16 is not None:
                    e["mfma_f16_flops"] = round(mf16 * 512)
            if "lds" in runs:
                la = mean("lds", sec, fam, "GRBM_GUI_ACTIVE")
                if la:
                    la1 = la / 8.0
                    idx = mean("lds", sec, fam, "SQ_LDS_IDX_ACTIVE")
                    bc = mean("lds", sec, fam, "SQ_LDS_BANK_CONFLICT")
                    bw = mean("lds", sec, fam, "SQ_INSTS_LDS_LOAD_BANDWIDTH")
                    ff = mean("lds", sec, fam, "SQ_LDS_DATA_FIFO_FULL")
                    wl = mean("lds", sec, fam, "SQ_WAIT_INST_LDS")
                    bu = mean("lds", sec, fam, "SQ_BUSY_CU_CYCLES")
                    if idx is not None:
                        e["lds_active_frac"] = round(idx / (la1 * 256.0), 4)
                    if bc is not None and idx:
                        e["lds_bank_conflict_of_active"] = round(bc / idx, 4)
                    if bw is not None:
                        e["lds_load_bytes"] = round(bw * 64)
                        e["lds_load_bytes_per_cu_cycle"] = round(bw * 64 / (la1 * 256.0), 2)
                    if ff is not None:
                        e["lds_data_fifo_full_frac"] = round(ff / (la1 * 256.0), 4)
                    if wl is not None:
                        e["wait_inst_lds_wave_cycles"] = round(wl * 4)
                    if bu is not None:
                        e["cu_busy_frac"] = round(bu * 4 / (la1 * 256.0), 4)
            ks[fam] = e
        rec["sections"][sec] = {"kernels": ks}
    with open(COUNTERS_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    out = ["# rocprofv3 counters per kernel and workload", "",
           "Commands (from the repository root):", ""]
    out += ["    " + c for c in rec["commands"]]
    out += ["", "Calibration on the copy probe (%d bytes read and written): %s" % (
        COPY_PROBE_BYTES, json.dumps(rec["calibration"])), "", rec["notes"], "",
        "| section | kernel | avg us (trace) | DRAM read MB | DRAM write MB | fetch+write MB "
        "| clock GHz | MFMA busy | MFMA i8 ops | MFMA f16 flops | LDS active | LDS B/CU-clk |",
        "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for sec, v in rec["sections"].items():
        for fam, e in v["kernels"].items():
            g = lambda k, s=1e6: ("%.2f" % (e[k] / s)) if e.get(k) is not None else ""
            out.append("| %s | %s | %s | %s | %s | %s | %s | %s | %s | %s | %s | %s |" % (
                sec, fam, e.get("avg_duration_us", ""), g("dram_read_bytes"),
                g("dram_write_bytes"), g("fetch_write_bytes"), e.get("effective_clock_ghz", ""),
                e.get("mfma_busy_frac", ""), "%.4g" % e["mfma_i8_ops"] if e.get("mfma_i8_ops") else "",
                "%.4g" % e["mfma_f16_flops"] if e.get("mfma_f16_flops") else "",
                e.get("lds_active_frac", ""), e.get("lds_load_bytes_per_cu_cycle", "")))
    out += ["", "Kernel code SHA-256 (comments and whitespace ignored): " + rec["kernel_code_sha256"]]
    with open(COUNTERS_MD, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def _summarize_trace(trace_dir):
    """The committed kernel-trace summary from a rocprofv3 run of the default
    bench command (kernel trace + stats, csv output, -o bench): per-kernel
    statistics, and the headline GEMM's average over the launches of its timed
    GEMM-alone loop next to the HIP-event figure the bench printed."""
    import csv
    log_lines = open(os.path.join(trace_dir, "bench.log")).read().splitlines()
    line = [x for x in log_lines if x.startswith("{")][-1]
    b = json.loads(line)
    steps = b["steps"]
    grid = b["roofline"]["grid_threads"]
    tr = list(csv.DictReader(open(os.path.join(trace_dir, "bench_kernel_trace.csv"))))
    tr.sort(key=lambda r: int(r["Start_Timestamp"]))
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
    g = [r for r in tr if "k_gemm_i8" in r["Kernel_Name"] and int(r["Grid_Size_X"]) == grid]
    alone = g[-steps:]
    avg = lambda rs: sum(dur(r) for r in rs) / max(len(rs), 1)
    cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d %s -o bench -- "
           "python3 bench.py --steps %d --warmup %d" % (trace_dir, steps, b["warmup"]))
    out = ["# Kernel trace: k_gemm_i8 on the 175B-scale FFN layer (4096 x 12288 -> 49152) and "
           "every kernel of the bench run", "",
           "Command (from the repository root; bench.log is its stdout):", "",
           "    " + cmd + " > %s/bench.log" % trace_dir,
           "    python3 bench.py --summarize-trace %s" % trace_dir, "",
           "k_gemm_i8 (%s, grid %s threads, %s VGPR + %s AGPR, LDS %s B, scratch %s B):" % (
               _short(alone[0]["Kernel_Name"]), alone[0]["Grid_Size_X"], alone[0]["VGPR_Count"],
               alone[0]["Accum_VGPR_Count"], alone[0]["LDS_Block_Size"], alone[0]["Scratch_Size"]),
           "", "| measurement | launches | average (us) |", "|---|---|---|",
           "| rocprofv3, timed GEMM-alone loop | %d | %.2f |" % (len(alone), avg(alone)),
           "| HIP events on the launch stream, same loop (bench `roofline.ms_per_launch`) | %d | %.2f |"
           % (steps, 1000.0 * b["roofline"]["ms_per_launch"]), "",
           "Bench line printed under the profiler (whole layer step %.2f us):" % (
               1000.0 * b["ms_per_step"]), "", "    " + line, "",
           "rocprofv3 --stats (all launches of the run):", "",
           "| kernel | calls | average (us) | min (us) | max (us) | % of GPU time |",
           "|---|---|---|---|---|---|"]
    for r in csv.DictReader(open(os.path.join(trace_dir, "bench_kernel_stats.csv"))):
        out.append("| %s | %s | %.2f | %.2f | %.2f | %.2f |" % (
            _short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1000, float(r["MinNs"]) / 1000,
            float(r["MaxNs"]) / 1000, float(r["Percentage"])))
    with open(TRACE_FILE, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prewarm-ms", type=float, default=500.0,
                    help="untimed, time-based pre-warm before each timed loop")
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the headline workload (for profiler runs)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--profile-kernels", action="store_true",
                    help="eager runs of every kernel for rocprofv3 counter runs")
    ap.add_argument("--write-counters", metavar="PMC_DIR",
                    help="write the stored counter figures from rocprofv3 runs (no GPU) and exit")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="write the committed kernel-trace summary (no GPU) and exit")
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
    if args.profile_kernels:
        _profile_kernels()
        return

    import numpy as np
    import torch

    import int8_quantized_matmul_absmax_amd as i8

    i8.ensure_built()
    ops = i8.ops
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    wl = args.workload
    log("generating %s" % wl)
    d = _make(wl)
    log("headline layer %s" % wl)
    L = _measure_layer(ops, d, args.steps, args.warmup, args.prewarm_ms, stream, keep_pool=True)
    M, K, N, n_out = L["M"], L["K"], L["N"], L["n_outliers"]
    tiles = ((M + 255) // 256) * ((N + 255) // 256)
    grid_threads = tiles * 512 if tiles >= 256 else ((M + 127) // 128) * ((N + 127) // 128) * 256

    # parity host copies of the timed output (sampled rows, all features)
    rows_y = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(1).choice(M, 8)]))
    Y_last = L["_pool"][L["_last_set"]]["Y"]
    Y_rows = Y_last[torch.from_numpy(rows_y).cuda()].cpu().numpy()
    Wq_h = L["_Wq"].cpu().numpy() if not args.no_cpu_baseline else None
    del L["_pool"], L["_Wq"], L["_last_set"]
    torch.cuda.empty_cache()

    log("activation side alone")
    xside = _measure_x_side(ops, d["X"], args.prewarm_ms, stream)
    extras = {}
    if not args.no_extras:
        log("copy bandwidth")
        extras["copy"] = _measure_copy(args.prewarm_ms, stream)
        other = "opt6.7b_ffn_up" if wl == "ffn175b" else "ffn175b"
        log("layer %s" % other)
        d2 = _make(other)
        L2 = _measure_layer(ops, d2, min(args.steps, 100), args.warmup, args.prewarm_ms, stream)
        x2 = _measure_x_side(ops, d2["X"], args.prewarm_ms, stream)
        del d2
        torch.cuda.empty_cache()
        extras[other] = {
            "us_per_step": round(L2["ms_per_step"] * 1e3, 2), "eff_tops": round(L2["eff_tops"], 1),
            "n_outliers": L2["n_outliers"], "gemm_us": round(L2["gemm_ms"] * 1e3, 2),
            "gemm_achieved_tops": round(L2["gemm_achieved"], 1),
            "gemm_mfma_frac": round(L2["gemm_frac"], 4), "step_us_spread": L2["spread"],
            "x_side": x2, "weight_once_gbps": round(L2["weight_once_gbps"], 1),
            "weight_once_hbm_frac": round(L2["weight_once_gbps"] / PEAK_HBM_GBPS, 4),
            "rotation_sets": L2["rotation_sets"]}
        log("decode")
        extras["decode_4096x4096"] = _measure_decode(ops)
        torch.cuda.empty_cache()
        log("tiny layer")
        extras["tiny_16x256x256"] = _measure_tiny(ops)
        log("mlp sweep")
        extras["mlp_sweep"] = _measure_mlp(ops, args.prewarm_ms, stream)
        torch.cuda.empty_cache()

    cpu, parity = None, None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu, parity = _cpu_baseline(d, M, N, K, args.cpu_seconds, Wq_h, Y_rows, rows_y, wl)

    traffic = _traffic_from_counters(wl + "_layer")
    out = {
        "metric": "effective int8-mixed linear TOPS + % int8 MFMA peak; quantize kernel HBM GB/s",
        "value": round(L["eff_tops"], 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(L["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "%s_prefill" % wl, "description": DESCRIPTION[wl],
                   "M": M, "K": K, "N": N, "threshold": 6.0, "n_outliers": n_out,
                   "parallelism": "single_gpu"},
        "roofline": {"bound": "mfma",
                     "kernel": "k_gemm_i8 (int8 GEMM + fused dequant/fp16 outlier product)",
                     "achieved": round(L["gemm_achieved"], 3), "peak": round(L["gemm_peak"], 3),
                     "unit": "TOP/s", "frac": round(L["gemm_frac"], 4), "traffic": traffic,
                     "ms_per_launch": round(L["gemm_ms"], 6),
                     "ops_per_launch": int(L["gemm_ops"]),
                     "int8_ops_per_launch": 2 * M * N * (K - n_out),
                     "fp16_flops_per_launch": 2 * M * N * n_out,
                     "grid_threads": grid_threads,
                     "peak_note": "int8 ops at 5000 TOP/s and fp16 flops at 2500 TFLOP/s"},
        "int8_mfma_peak_frac": round(L["gemm_frac"], 4),
        "prewarm_ms": L["prewarm"]["ms"],
        "step_us_spread": L["spread"],
        "quantize": {"x_side": xside,
                     "weight_once": {"us": round(L["weight_once_ms"] * 1e3, 1),
                                     "gbps": round(L["weight_once_gbps"], 1),
                                     "hbm_frac": round(L["weight_once_gbps"] / PEAK_HBM_GBPS, 4),
                                     "algorithmic_bytes": 3 * N * K + 4 * N}},
        "parity": parity,
        "cpu_baseline": cpu,
        "rotation_sets": L["rotation_sets"],
        "timed_wall_s": round(L["wall_s"], 4),
    }
    out.update(extras)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
