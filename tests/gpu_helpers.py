"""Helpers for the GPU parity tests: run the HIP path, run the oracle on the
same stored inputs, compare element by element."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import tiled_attention_amd as mx
import workloads

to_np = workloads.to_numpy_bits

# Tolerances stated for this method: max-abs error on O of 1e-5 (fp32 I/O) or
# 1e-2 (bf16 I/O, fp32 accumulate), and 1e-4 on the LSE.
TOL_O = {"f32": 1e-5, "bf16": 1e-2}
TOL_LSE = 1e-4


def dev():
    return torch.device("cuda:0")


def compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype, label=""):
    """Element-wise check; o_* are [n, d] arrays, lse_* [n] (fp64 reference)."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    masked = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), masked), f"{label}: fully-masked rows differ"
    assert np.all(o_gpu[masked] == 0.0), f"{label}: a row that sees no key must be zero"
    assert np.all(np.isfinite(o_gpu)), f"{label}: non-finite output"
    err_o = np.abs(o_gpu - o_ref)
    worst = float(err_o.max()) if err_o.size else 0.0
    fin = ~masked
    err_l = float(np.abs(lse_gpu[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    assert worst <= TOL_O[dtype], f"{label}: max |O - O_ref| = {worst:.3g} > {TOL_O[dtype]}"
    assert err_l <= TOL_LSE, f"{label}: max |LSE - LSE_ref| = {err_l:.3g} > {TOL_LSE}"
    return worst, err_l


def gpu_varlen(p, *, causal, window, softcap, scale):
    """Run mxfa_fwd_varlen on a problem dict from workloads.make_problem (CPU tensors)."""
    d = dev()
    q, k, v = p["q"].to(d), p["k"].to(d), p["v"].to(d)
    cq, ck = p["cu_seqlens_q"].to(d), p["cu_seqlens_k"].to(d)
    mq = max(p["lens_q"]) if p["lens_q"] else 0
    mk = max(p["lens_k"]) if p["lens_k"] else 0
    o, lse = mx.mxfa_fwd_varlen(q, k, v, cq, ck, mq, mk, causal=causal, window=window, softcap=softcap,
                                scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def oracle_varlen(p, *, causal, window, softcap, scale, rows=None):
    return oracle.attention_rows(to_np(p["q"]), to_np(p["k"]), to_np(p["v"]), p["cu_seqlens_q"].numpy(),
                                 p["cu_seqlens_k"].numpy(), causal=causal, window=window, softcap=softcap,
                                 scale=scale, rows=rows)


def sample_rows(lens, heads, n, seed, bm=128):
    """Seeded (token, head) rows: every segment's first/last rows and q-tile edges, plus random rows."""
    rng = np.random.RandomState(seed)
    rows = set()
    start = 0
    for L in lens:
        if L:
            for i in {0, 1, L - 1, L // 2, min(L - 1, bm - 1), min(L - 1, bm), min(L - 1, bm + 1)}:
                rows.add((start + i, int(rng.randint(heads))))
        start += L
    total = start
    while len(rows) < n and total:
        rows.add((int(rng.randint(total)), int(rng.randint(heads))))
    return np.array(sorted(rows), dtype=np.int64)
