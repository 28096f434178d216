"""Host-side checks of the benchmark script (no GPU): the one-GPU refusal and
the code hash that decides whether stored HBM counters still describe the
GEMM kernel."""

import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""   # no JSON line


def test_kernel_hash_ignores_comments_and_sees_code(tmp_path):
    bench = _bench_module()
    code = "int f(int x) {\n  return x + 1;\n}\n"
    variants = {
        "plain": code,
        "comments": "// header\n/* block\n comment */\nint f(int x) {  // note\n  return x + 1;\n}\n",
        "spacing": "int f(int x)\n{\n    return x + 1;   \n}\n\n",
        "changed": "int f(int x) {\n  return x + 2;\n}\n",
    }
    hashes = {}
    for name, text in variants.items():
        p = tmp_path / name / "gemm_kernel.hip"
        p.parent.mkdir()
        p.write_text(text)
        hashes[name] = bench._kernel_code_sha256([str(p)])
    assert hashes["plain"] == hashes["comments"] == hashes["spacing"]
    assert hashes["changed"] != hashes["plain"]


def test_kernel_hash_covers_every_source():
    bench = _bench_module()
    csrc = bench.CSRC
    srcs = sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".h")))
    assert "gemm_kernel.hip" in srcs and "quant_kernels.hip" in srcs
    full = bench._kernel_code_sha256()
    assert full == bench._kernel_code_sha256([os.path.join(csrc, f) for f in srcs])
    assert full != bench._kernel_code_sha256([os.path.join(csrc, f) for f in srcs[1:]])


def test_kernel_families_of_trace_names():
    bench = _bench_module()
    gemm = ("void i8mm::(anonymous namespace)::k_gemm_i8<i8mm::(anonymous namespace)::"
            "GemmCfg<256, 256, 64, 5, 4>, %d>(signed char const*, signed char const*)")
    assert bench._family(gemm % 0) == "k_gemm_i8"
    assert bench._family(gemm % 1) == "k_gemm_i8"
    assert bench._family(gemm % 2) == "k_gemm_i8_outlier_seg"
    assert bench._family(gemm % 3) == "k_gemm_i8_dense_seg"
    assert bench._family("void i8mm::(anonymous namespace)::k_rows<2, true>(unsigned short "
                         "const*, long)") == "k_rows"
    assert bench._family("void at::native::elementwise_kernel<128, 4, at::native::copy_"
                         "kernel_impl>(int)") == "copy"


def _write_csv(path, header, rows):
    import csv
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_counter_summary_from_rocprof_csvs(tmp_path, monkeypatch):
    """The counter summary assigns dispatches to the profiling sections by the
    marker fills, scales byte counters by the copy probe and derives clock and
    MFMA busy fraction; checked on synthetic rocprofv3-style csv files."""
    import json
    bench = _bench_module()
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(tmp_path / "out.json"))
    monkeypatch.setattr(bench, "COUNTERS_MD", str(tmp_path / "out.md"))
    mark = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<double>>(int)"
    copy = "void at::native::elementwise_kernel<128, 4, at::native::copy_kernel_impl>(int)"
    gemm = ("void i8mm::(anonymous namespace)::k_gemm_i8<i8mm::(anonymous namespace)::"
            "GemmCfg<256, 256, 64, 5, 4>, 0>(signed char const*)")
    rows_k = "void i8mm::(anonymous namespace)::k_rows<24, 2>(unsigned short const*)"
    seq = [mark, copy, copy, mark, rows_k, mark, rows_k, gemm, gemm, mark]
    sections = ["copy_probe", "layer"]
    (tmp_path / "pmc").mkdir()
    (tmp_path / "pmc" / "manifest.json").write_text(json.dumps({"profile_sections": sections}))
    # kernel trace: durations 1000 ns for everything, gemm 2000 ns
    trace = []
    t = 0
    for i, k in enumerate(seq):
        d = 2000 if k == gemm else 1000
        trace.append([i + 1, k, t, t + d])
        t += d + 10
    _write_csv(tmp_path / "pmc" / "trace" / "run_kernel_trace.csv",
               ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], trace)

    def counters(run, values):
        rows = []
        for i, k in enumerate(seq):
            for c, f in values.items():
                rows.append([i + 1, k, c, f(k), trace[i][2], trace[i][3]])
        _write_csv(tmp_path / "pmc" / run / "run_counter_collection.csv",
                   ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"], rows)

    half = bench.COPY_PROBE_BYTES
    counters("dram", {"TCC_EA0_RDREQ_DRAM_sum": lambda k: half / 64 if k == copy else 1000.0,
                      "TCC_EA0_WRREQ_DRAM_sum": lambda k: half / 64 if k == copy else 10.0,
                      "GRBM_GUI_ACTIVE": lambda k: 8000.0})
    counters("fetch", {"FETCH_SIZE": lambda k: half / 2048 if k == copy else 4.0})
    counters("write", {"WRITE_SIZE": lambda k: half / 1024 if k == copy else 1.0})
    # gemm: 8 XCDs x 4000 active cycles over 2000 ns -> 2 GHz; busy 1024 x 2000
    counters("mfma", {"GRBM_GUI_ACTIVE": lambda k: 32000.0 if k == gemm else 8000.0,
                      "GRBM_COUNT": lambda k: 32000.0,
                      "SQ_VALU_MFMA_BUSY_CYCLES": lambda k: 2048000.0 if k == gemm else 0.0,
                      "SQ_INSTS_VALU_MFMA_MOPS_I8": lambda k: 100.0 if k == gemm else 0.0,
                      "SQ_INSTS_VALU_MFMA_MOPS_F16": lambda k: 0.0,
                      "SQ_BUSY_CYCLES": lambda k: 1.0})
    bench._write_counters(str(tmp_path / "pmc"))
    rec = json.load(open(tmp_path / "out.json"))
    assert rec["calibration"]["dram_read_bytes_per_request"] == 64.0
    assert rec["calibration"]["fetch_size_scale"] == 2.0
    g = rec["sections"]["layer"]["kernels"]["k_gemm_i8"]
    assert g["avg_duration_us"] == 2.0
    assert g["dram_read_bytes"] == 64000 and g["dram_write_bytes"] == 640
    assert g["fetch_bytes"] == 4 * 1024 * 2 and g["write_bytes"] == 1024
    assert g["effective_clock_ghz"] == 2.0
    assert g["mfma_busy_frac"] == 0.5
    assert g["mfma_i8_ops"] == 51200
    assert set(rec["sections"]["layer"]["kernels"]) == {"k_rows", "k_gemm_i8"}
    # the set-up dispatch between the sections (a k_rows) belongs to neither
    assert rec["sections"]["layer"]["kernels"]["k_rows"]["dram_read_bytes"] == 64000
    assert set(rec["sections"]["copy_probe"]["kernels"]) == {"copy"}
    assert "k_gemm_i8" in open(tmp_path / "out.md").read()
