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


def test_kernel_hash_ignores_comments_and_sees_code(tmp_path, monkeypatch):
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
        p = tmp_path / (name + ".hip")
        p.write_text(text)
        monkeypatch.setattr(bench, "GEMM_SRC", str(p))
        hashes[name] = bench._kernel_code_sha256()
    assert hashes["plain"] == hashes["comments"] == hashes["spacing"]
    assert hashes["changed"] != hashes["plain"]
