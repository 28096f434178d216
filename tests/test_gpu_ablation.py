"""The accuracy ablation on the GPU: the HIP path's LLM.int8() and
vector-wise (threshold +inf) errors against the exact product match the
oracle's, and order as the pages report (decomposition < vector-wise alone <
tensor-wise) on synthetic outlier data."""

import numpy as np
import pytest

from int8_quantized_matmul_absmax_amd import synth
from oracle import ablations as A
from tests import ablation_report as R
from tests.gpu_helpers import dev, host, note

pytestmark = pytest.mark.gpu


def test_ablation_errors_on_gpu(gpu):
    note("ablation")
    d = synth.opt_ffn_up(M=128, K=1024, N=256)
    r = R.measure(gpu.ops, dev, lambda t: host(t).astype(np.float64), d["X"], d["W"])
    for scheme in ("LLM.int8()", "vector-wise, no decomposition"):
        g = [v for k, v in r.items() if k.startswith(scheme) and "GPU" in k][0]
        o = r[scheme + " (oracle)"]
        assert abs(g[1] - o[1]) <= 0.02 * o[1] + 1e-4, (scheme, g, o)
    g_m = r["LLM.int8() (GPU, threshold 6)"][1]
    g_v = r["vector-wise, no decomposition (GPU, threshold +inf)"][1]
    assert g_m < g_v < r["tensor-wise absmax (oracle)"][1]
    assert g_v > 2 * g_m
