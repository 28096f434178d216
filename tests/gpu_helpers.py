"""Helpers shared by the GPU parity tests: moving seeded host buffers to the
device and back, and the comparison metrics. No arithmetic of the method."""

import sys

import numpy as np
import torch

from oracle import llm_int8 as O

Y_TOL = 1e-3   # max |Y_gpu - Y_ref| / max |Y_ref| (fp16 output vs fp64 oracle)


def dev(a):
    """numpy array -> contiguous CUDA tensor of the same dtype (fp16/int8/fp32/int32)."""
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def note(msg):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def bitmap_u32(t):
    return host(t).view(np.uint32)


def f16_ulp(a):
    """The fp16 ulp of each value of a (float16 array): the spacing of its
    binade. Finite at the largest finite fp16 (65504 lies in the binade
    [32768, 65536), whose ulp is 32), where np.spacing overflows to inf."""
    a16 = np.abs(np.asarray(a, np.float16))
    return np.spacing(np.minimum(a16, np.float16(32768.0))).astype(np.float64)


def y_err(Y_gpu, Y_ref):
    return O.max_abs_rel_error(np.asarray(Y_gpu, np.float64), Y_ref)


def sample_rows(M, count, seed, must=()):
    rng = np.random.default_rng(seed)
    rows = set(int(r) for r in must if 0 <= r < M)
    rows |= {0, M - 1}
    extra = rng.choice(M, size=min(M, count), replace=False)
    rows |= set(int(r) for r in extra)
    return np.array(sorted(rows))
