"""Accuracy ablation report (needs the GPU): writes
profiles/accuracy_ablation.md.

    python3 -m tests.ablation_report

For each synthetic workload the error of every scheme against the exact
fp64 product X . W^T: the baselines the pages compare LLM.int8() with
(tensor-wise absmax, zero-point, vector-wise without decomposition) from the
CPU oracle, and LLM.int8() itself (threshold 6) and vector-wise (threshold
+inf) from both the oracle and the HIP path. Errors: max |dY| / max |Y| and
mean |dY| / mean |Y|.
"""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from int8_quantized_matmul_absmax_amd import synth  # noqa: E402
from oracle import ablations as A  # noqa: E402
from oracle import llm_int8 as O  # noqa: E402

OUT = os.path.join(ROOT, "profiles", "accuracy_ablation.md")


def workloads():
    d = synth.opt_ffn_up(M=256, K=4096, N=2048)
    yield "OPT-6.7B FFN up shape, 256 x 4096 -> 2048, 6 outlier dims on 25% of tokens", d["X"], d["W"]
    Xc = np.clip(d["X"].astype(np.float32), -5.0, 5.0).astype(np.float16)
    yield "same, outlier dims clipped to +-5 (no outliers)", Xc, d["W"]
    for n_in in (6, 32):
        m = synth.mlp_sweep(n_in)
        yield ("MLP input, %d dims planted on every token, 256 x 4096 -> 2048" % n_in,
               m["X"][:256], m["W1"][:2048])
    f = synth.ffn_175b(M=128, N=1024)
    yield "175B-scale hidden, 128 x 12288 -> 1024, 12 outlier dims", f["X"], f["W"]


def measure(ops, dev, host, X, W):
    """Errors of every scheme for one workload: {scheme: (max_rel, mean_rel)}."""
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    Wq, sw = O.quantize_weight_rows(W)
    r = {
        "tensor-wise absmax (oracle)": A.relative_errors(A.tensorwise_absmax_linear(X, W), exact),
        "zero-point (oracle)": A.relative_errors(A.zeropoint_linear(X, W), exact),
        "vector-wise, no decomposition (oracle)": A.relative_errors(A.vectorwise_linear(X, Wq, sw), exact),
        "LLM.int8() (oracle)": A.relative_errors(O.linear_int8_mixed(X, Wq, sw, 6.0)["Y"], exact),
    }
    Xd, Wqd, swd = dev(X), dev(Wq), dev(sw)
    Yv = host(ops.linear_int8_mixed(Xd, Wqd, swd, None, float("inf")))
    Ym = host(ops.linear_int8_mixed(Xd, Wqd, swd, None, 6.0))
    r["vector-wise, no decomposition (GPU, threshold +inf)"] = A.relative_errors(Yv, exact)
    r["LLM.int8() (GPU, threshold 6)"] = A.relative_errors(Ym, exact)
    return r


def main():
    import torch
    import int8_quantized_matmul_absmax_amd as i8
    i8.ensure_built()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    host = lambda t: t.detach().cpu().numpy().astype(np.float64)  # noqa: E731
    lines = ["# Accuracy ablation: LLM.int8() against the schemes the pages compare it with", "",
             "Command (from the repository root):", "", "    python3 -m tests.ablation_report", "",
             "Errors against the exact fp64 product X . W^T of the fp16 inputs "
             "(synthetic inputs, seeded): max |dY| / max |Y| and mean |dY| / mean |Y|. "
             "GPU rows come from the HIP path (fp16 output); oracle rows are fp64.", ""]
    for name, X, W in workloads():
        r = measure(i8.ops, dev, host, X, W)
        lines += ["## " + name, "", "| scheme | max rel. error | mean rel. error |", "|---|---|---|"]
        for k, (emax, emean) in r.items():
            lines.append("| %s | %.3e | %.3e |" % (k, emax, emean))
        lines.append("")
        print(name, {k: round(v[1], 5) for k, v in r.items()}, flush=True)
    with open(OUT, "w") as f:
        f.write("\n".join(lines))
    print("wrote", OUT, flush=True)


if __name__ == "__main__":
    main()
