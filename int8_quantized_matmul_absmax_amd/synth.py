"""Seeded synthetic inputs for the int8 mixed-precision linear layer.

This module draws inputs only: activations and weights in fp16 with planted
outlier columns. It holds none of the method's arithmetic (no thresholding,
quantization or matmul), so the same host buffers can feed both the HIP path
and an independent CPU reference.

Shapes and distributions follow the workloads the method is described on:
hidden 4096 / FFN 16384 (OPT-6.7B-shaped), hidden 12288 / FFN 49152
(175B-scale), and decode batches of 1-16 tokens. The outlier structure follows
the paper summary page "LLM.int8(): 8-Bit Matrix Multiplication for
Transformers at Scale", section "Discovery: emergent outlier features": a
handful of fixed hidden dimensions (about 6, at most 7; about 0.1% of the
features) whose values are about 20x the typical magnitude and that appear on
a large fraction of the tokens.

Every array is drawn in float32 from numpy's PCG64 and rounded to fp16 (round
to nearest even). Each tensor gets its own child stream of one SeedSequence, so
changing a size does not change the other tensors' streams.
"""

import numpy as np

# Seeds of the five named workloads: 1000 + workload index.
SEED_TINY = 1001
SEED_OPT_FFN_UP = 1002
SEED_DECODE = 1003
SEED_175B_FFN = 1004
SEED_MLP_SWEEP = 1005

_CHUNK_ELEMS = 1 << 24


def _rngs(seed, count):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(count)]


def normal_f16(rng, shape, std):
    """fp16 array of N(0, std^2) draws (float32 draw, scaled, rounded to fp16)."""
    out = np.empty(shape, np.float16)
    flat = out.reshape(-1)
    buf = np.empty(min(flat.size, _CHUNK_ELEMS), np.float32)
    for start in range(0, flat.size, _CHUNK_ELEMS):
        n = min(_CHUNK_ELEMS, flat.size - start)
        b = buf[:n]
        rng.standard_normal(out=b, dtype=np.float32)
        b *= np.float32(std)
        flat[start:start + n] = b
    return out


def plant_outlier_columns(rng, X, n_cols, lo, hi, token_fraction):
    """Overwrite n_cols seeded columns of X with +-U(lo, hi) on a seeded token subset.

    token_fraction is a float (same fraction for every column), a pair
    (pmin, pmax) (each column draws its own fraction from U(pmin, pmax)), or
    1.0 for every token. Each column gets its own seeded subset of
    round(p * M) rows. Returns the planted columns, ascending, and the row
    counts used.
    """
    M, K = X.shape
    cols = np.sort(rng.choice(K, size=n_cols, replace=False)).astype(np.int32)
    counts = []
    for c in cols:
        if isinstance(token_fraction, tuple):
            p = rng.uniform(token_fraction[0], token_fraction[1])
        else:
            p = float(token_fraction)
        cnt = int(round(p * M))
        rows = rng.choice(M, size=cnt, replace=False) if cnt < M else np.arange(M)
        mag = rng.uniform(lo, hi, size=rows.size).astype(np.float32)
        sign = np.where(rng.random(rows.size) < 0.5, -1.0, 1.0).astype(np.float32)
        X[rows, c] = (mag * sign).astype(np.float16)
        counts.append(cnt)
    return cols, counts


def tiny(seed=SEED_TINY, M=16, K=256, N=256):
    """Tiny layer: X and W entries 0.5 * N(0, 1); 2 fixed X columns set to
    +-U(8, 20) on every token (over the threshold 6.0)."""
    rx, rw, ro = _rngs(seed, 3)
    X = normal_f16(rx, (M, K), 0.5)
    planted, _ = plant_outlier_columns(ro, X, 2, 8.0, 20.0, 1.0)
    W = normal_f16(rw, (N, K), 0.5)
    return {"X": X, "W": W, "planted": planted, "name": "tiny_16x256x256"}


def opt_ffn_up(seed=SEED_OPT_FFN_UP, M=2048, K=4096, N=16384):
    """OPT-6.7B-shaped FFN up-projection at prefill: X ~ N(0, 1) [M, K],
    W ~ N(0, 0.02^2) [N, K]; 6 fixed hidden dims scaled to +-U(15, 25), each on
    its own 25% token subset."""
    rx, rw, ro = _rngs(seed, 3)
    X = normal_f16(rx, (M, K), 1.0)
    planted, _ = plant_outlier_columns(ro, X, 6, 15.0, 25.0, 0.25)
    W = normal_f16(rw, (N, K), 0.02)
    return {"X": X, "W": W, "planted": planted,
            "name": "opt6.7b_ffn_up_%dx%dx%d" % (M, K, N)}


def decode(M, seed=SEED_DECODE, K=4096, N=4096):
    """Decode-shaped layer: X ~ N(0, 1) [M, K] with M in {1, 4, 16} tokens and
    6 outlier dims at +-U(15, 25) on every token; W ~ N(0, 0.02^2) [N, K]
    (quantized once to int8 before the timed calls)."""
    rx, rw, ro = _rngs(seed, 3)
    W = normal_f16(rw, (N, K), 0.02)
    X = normal_f16(rx, (M, K), 1.0)
    planted, _ = plant_outlier_columns(ro, X, 6, 15.0, 25.0, 1.0)
    return {"X": X, "W": W, "planted": planted, "name": "decode_%dx%dx%d" % (M, K, N)}


def ffn_175b(seed=SEED_175B_FFN, M=4096, K=12288, N=49152):
    """175B-scale FFN layer on one GPU: X ~ N(0, 1) [M, K], W ~ N(0, 0.01^2)
    [N, K]; 12 hidden dims (~0.1% of K) at +-U(10, 60), each on its own token
    fraction drawn from U(0.2, 0.6)."""
    rx, rw, ro = _rngs(seed, 3)
    X = normal_f16(rx, (M, K), 1.0)
    planted, _ = plant_outlier_columns(ro, X, 12, 10.0, 60.0, (0.2, 0.6))
    W = normal_f16(rw, (N, K), 0.01)
    return {"X": X, "W": W, "planted": planted,
            "name": "ffn175b_%dx%dx%d" % (M, K, N)}


def mlp_sweep(n_in, seed=SEED_MLP_SWEEP, M=1024, H=4096, F=16384):
    """Two-layer MLP block (up H->F, GELU, down F->H): X ~ N(0, 1) [M, H],
    W1 [F, H] and W2 [H, F] ~ N(0, 0.02^2); n_in planted input columns at
    +-U(8, 40) on every token (n_in swept over 0, 6, 32, 128, 512)."""
    rx, r1, r2, ro = _rngs(seed, 4)
    X = normal_f16(rx, (M, H), 1.0)
    planted, _ = plant_outlier_columns(ro, X, n_in, 8.0, 40.0, 1.0)
    W1 = normal_f16(r1, (F, H), 0.02)
    W2 = normal_f16(r2, (H, F), 0.02)
    return {"X": X, "W1": W1, "W2": W2, "planted": planted,
            "name": "mlp_sweep_n%d_%dx%dx%d" % (n_in, M, H, F)}


def random_codes(seed, shape):
    """Uniform int8 codes in [-127, 127] (for direct GEMM parity cases)."""
    rng = np.random.default_rng(seed)
    return rng.integers(-127, 128, size=shape, dtype=np.int16).astype(np.int8)
