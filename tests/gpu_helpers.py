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


def half_ulp_bf16(x):
    """Half a bf16 unit in the last place at |x|: 2^(e-8) for |x| in [2^e, 2^(e+1)), 0 at 0."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(a)  # a = m * 2^e with m in [0.5, 1)
    return np.where(a > 0, np.ldexp(1.0, e - 9), 0.0)


class Stats:
    """Running error statistics of one comparison, possibly over several chunks.

    Besides the max-abs errors it counts the O elements above the tolerance and,
    among them, those within the tolerance plus half a bf16 unit of |O_ref|
    (what rounding the output to bf16 alone can add).
    """

    def __init__(self, dtype, label):
        self.dtype, self.label = dtype, label
        self.rows = self.elems = 0
        self.max_o = self.max_l = 0.0
        self.over = self.over_within_half_ulp = 0

    def add(self, o_gpu, lse_gpu, o_ref, lse_ref):
        o_gpu = np.asarray(o_gpu, dtype=np.float64)
        lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
        masked = np.isneginf(lse_ref)
        assert np.array_equal(np.isneginf(lse_gpu), masked), f"{self.label}: fully-masked rows differ"
        assert np.all(o_gpu[masked] == 0.0), f"{self.label}: a row that sees no key must be zero"
        assert np.all(np.isfinite(o_gpu)), f"{self.label}: non-finite output"
        err_o = np.abs(o_gpu - o_ref)
        if err_o.size:
            self.max_o = max(self.max_o, float(err_o.max()))
            tol = TOL_O[self.dtype]
            over = err_o > tol
            self.over += int(over.sum())
            if over.any():
                self.over_within_half_ulp += int((err_o[over] <= tol + half_ulp_bf16(o_ref[over])).sum())
        fin = ~masked
        if fin.any():
            self.max_l = max(self.max_l, float(np.abs(lse_gpu[fin] - lse_ref[fin]).max()))
        self.rows += len(lse_ref)
        self.elems += err_o.size

    def report(self):
        return (f"{self.label}: {self.rows} rows, {self.elems} elements: max|O-O_ref| = {self.max_o:.4g}, "
                f"max|LSE-LSE_ref| = {self.max_l:.3g}, elements > {TOL_O[self.dtype]:g}: {self.over} "
                f"(of which within +half-ulp_bf16(|O_ref|): {self.over_within_half_ulp})")

    def check(self):
        print("[parity] " + self.report(), flush=True)
        assert self.max_o <= TOL_O[self.dtype], f"{self.label}: max |O - O_ref| = {self.max_o:.3g} > {TOL_O[self.dtype]}"
        assert self.max_l <= TOL_LSE, f"{self.label}: max |LSE - LSE_ref| = {self.max_l:.3g} > {TOL_LSE}"
        return self.max_o, self.max_l


def compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype, label=""):
    """Element-wise check; o_* are [n, d] arrays, lse_* [n] (fp64 reference)."""
    st = Stats(dtype, label)
    st.add(o_gpu, lse_gpu, o_ref, lse_ref)
    return st.check()


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
