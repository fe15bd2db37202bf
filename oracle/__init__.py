"""fp64 CPU oracle for softmax attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP product path never imports,
links or calls it; the two share no code (only the seeded input generators in
``workloads`` serve both).

The arithmetic lives in ``attention_oracle.c`` (plain C, double precision,
one materialised row at a time); this module only marshals numpy arrays into
it. Inputs are numpy arrays holding float32 values or bf16 bit patterns
(``uint16``); they are upcast to double exactly inside the C code.

Every function here is pinned by ``tests/test_oracle_pins.py`` against a
50-digit decimal brute force, torch's float64 scaled-dot-product attention
with an explicit mask, closed forms and invariants. Parity pinned: all rows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attention_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16, F64 = 0, 1, 2


class _Problem(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("dtype", ctypes.c_int),
        ("q_tok_stride", ctypes.c_int64), ("q_head_stride", ctypes.c_int64),
        ("k_tok_stride", ctypes.c_int64), ("k_head_stride", ctypes.c_int64),
        ("v_tok_stride", ctypes.c_int64), ("v_head_stride", ctypes.c_int64),
        ("cu_q", ctypes.c_void_p), ("cu_k", ctypes.c_void_p),
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
        ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("window_left", ctypes.c_int32), ("window_right", ctypes.c_int32),
        ("softcap", ctypes.c_double), ("scale", ctypes.c_double),
    ]


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, IEEE math) into liboracle.so."""
    with _lock:
        if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            tmp = _LIB_PATH + ".tmp%d" % os.getpid()
            cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
            subprocess.run(cmd, check=True)
            os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def load_library(path: str):
    """Open a compiled oracle library and declare its entry points."""
    lib = ctypes.CDLL(path)
    lib.oracle_rows.restype = ctypes.c_int
    lib.oracle_rows.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_int]
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_threads.argtypes = [ctypes.c_int]
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = load_library(_LIB_PATH)
    return _lib


def threads_used(threads: int = 0) -> int:
    """Thread count the oracle's OpenMP region uses for ``threads`` (0 = default)."""
    return int(_load().oracle_threads(int(threads)))


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle inputs must be float32, float64 or uint16 (bf16 bits), got {a.dtype}")


def attention_rows(q, k, v, cu_q, cu_k, *, causal=False, window=(-1, -1), softcap=0.0,
                   scale=None, rows=None, threads=0, lib=None):
    """Attention rows of a packed problem, in float64.

    q: [total_q, Hq, d_qk]; k: [total_k, Hkv, d_qk]; v: [total_k, Hkv, d_v]
    (v may be a strided view, e.g. the leading channels of a shared kv buffer).
    cu_q, cu_k: int32 cumulative lengths [batch+1].
    rows: None for every (token, head) row, or an int array [n, 2] of
    (token, head) pairs. Returns (O [n, d_v], LSE [n], max |sum P - 1|); with
    rows=None, O is [total_q, Hq, d_v] and LSE is [total_q, Hq].
    ``lib`` selects another compiled copy of the oracle (the tests use it to
    show that planted mistakes fail the pins).
    """
    lib = lib if lib is not None else _load()
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    code = _dtype_code(q)
    if _dtype_code(k) != code or _dtype_code(v) != code:
        raise TypeError("q, k and v must share a dtype")
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
        raise ValueError("q, k, v must be rank-3 [tokens, heads, dim]")
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    cu_q = np.ascontiguousarray(cu_q, dtype=np.int32)
    cu_k = np.ascontiguousarray(cu_k, dtype=np.int32)
    total_q, hq, dqk = q.shape
    _, hkv, _ = k.shape
    dv = v.shape[2]
    if k.shape[2] != dqk or v.shape[0] != k.shape[0] or v.shape[1] != hkv:
        raise ValueError("inconsistent q/k/v shapes")
    if v.size and v.strides[2] != v.itemsize:  # (an empty array's strides may all be 0)
        raise ValueError("v's last dimension must be contiguous")
    batch = len(cu_q) - 1
    if len(cu_k) != batch + 1:
        raise ValueError("cu_q and cu_k differ in length")
    if scale is None:
        scale = dqk ** -0.5
    p = _Problem()
    p.q, p.k, p.v = q.ctypes.data, k.ctypes.data, v.ctypes.data
    p.dtype = code
    p.q_tok_stride, p.q_head_stride = hq * dqk, dqk
    p.k_tok_stride, p.k_head_stride = hkv * dqk, dqk
    p.v_tok_stride, p.v_head_stride = v.strides[0] // v.itemsize, v.strides[1] // v.itemsize
    p.cu_q, p.cu_k = cu_q.ctypes.data, cu_k.ctypes.data
    p.batch, p.heads_q, p.heads_kv, p.d_qk, p.d_v = batch, hq, hkv, dqk, dv
    p.causal = 1 if causal else 0
    p.window_left, p.window_right = int(window[0]), int(window[1])
    p.softcap, p.scale = float(softcap), float(scale)
    full = rows is None
    if full:
        tok = np.repeat(np.arange(total_q, dtype=np.int64), hq)
        head = np.tile(np.arange(hq, dtype=np.int32), total_q)
    else:
        rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
        tok = np.ascontiguousarray(rows[:, 0])
        head = np.ascontiguousarray(rows[:, 1].astype(np.int32))
    n = len(tok)
    o = np.empty((n, dv), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    dev = ctypes.c_double(0.0)
    rc = lib.oracle_rows(ctypes.byref(p), tok.ctypes.data, head.ctypes.data, n,
                         o.ctypes.data, lse.ctypes.data, ctypes.addressof(dev), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_rows failed with code {rc} (bad row index or allocation)")
    if full:
        return o.reshape(total_q, hq, dv), lse.reshape(total_q, hq), dev.value
    return o, lse, dev.value


def attention_dense(q, k, v, *, causal=False, window=(-1, -1), softcap=0.0, scale=None, threads=0,
                    lib=None):
    """Dense ``[B, S, H, d]`` problem: returns O [B, Sq, Hq, d_v] and LSE [B, Hq, Sq]."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    b, sq, hq, _ = q.shape
    sk = k.shape[1]
    cu_q = np.arange(b + 1, dtype=np.int32) * sq
    cu_k = np.arange(b + 1, dtype=np.int32) * sk
    o, lse, dev = attention_rows(q.reshape(b * sq, hq, -1), k.reshape(b * sk, k.shape[2], -1),
                                 v.reshape(b * sk, v.shape[2], -1), cu_q, cu_k, causal=causal,
                                 window=window, softcap=softcap, scale=scale, threads=threads,
                                 lib=lib)
    return o.reshape(b, sq, hq, -1), lse.reshape(b, sq, hq).transpose(0, 2, 1), dev


def gather_paged(kv_cache, block_table, cache_seqlens):
    """Packed keys of a paged cache.

    The paged layout of the mxflashattn page's ``flash_attn_with_kvcache``
    (block_table argument): the cache is ``[num_pages, page_size, H, d]`` and
    key j of sequence b is row ``j mod page_size`` of page
    ``block_table[b, j div page_size]``; sequence b holds
    ``cache_seqlens[b]`` keys. Returns (kv ``[sum(cache_seqlens), H, d]``,
    cu_k int32 ``[batch + 1]``), one key at a time in sequence order. Raises
    ValueError for a page index outside the cache or a table row too short.
    """
    kv_cache = np.asarray(kv_cache)
    table = np.asarray(block_table)
    lens = [int(x) for x in np.asarray(cache_seqlens).reshape(-1)]
    num_pages, page_size = kv_cache.shape[0], kv_cache.shape[1]
    if table.ndim != 2 or table.shape[0] != len(lens):
        raise ValueError("block_table must be [batch, max_pages]")
    rows = []
    for b, n in enumerate(lens):
        if n < 0:
            raise ValueError("cache_seqlens must be >= 0")
        for j in range(n):
            logical = j // page_size
            if logical >= table.shape[1]:
                raise ValueError(f"sequence {b}: key {j} lies past its block_table row")
            page = int(table[b, logical])
            if not 0 <= page < num_pages:
                raise ValueError(f"sequence {b}: page index {page} outside the cache")
            rows.append(kv_cache[page, j % page_size])
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    if rows:
        kv = np.stack(rows)
    else:
        kv = np.zeros((0,) + kv_cache.shape[2:], dtype=kv_cache.dtype)
    return kv, cu


def e4m3_to_float64(codes):
    """Values of OCP 8-bit floating point E4M3 codes (uint8), exactly, as float64.

    The format of an fp8 latent cache (the kernelbot amd-mixed-mla submission
    588924 page names fp8 KV; the encoding is the OCP 8-bit floating point
    specification's E4M3): sign bit, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent 0 holds the subnormals m * 2^-9; the all-ones exponent is
    an ordinary binade (up to 448) except S.1111.111, which is NaN; there
    are no infinities.
    """
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = sign * val
    return np.where((e == 15) & (m == 7), np.nan, val)


def bf16_bits_to_float64(bits):
    """bf16 bit patterns (uint16) as float64, exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def attention_rows_fp8_latent(q, kv8, kv_scale, cu_q, cu_k, *, d_v, causal=False, window=(-1, -1), softcap=0.0,
                              scale=None, rows=None, threads=0, lib=None):
    """Attention over an fp8 (E4M3) shared latent cache with one per-tensor scale.

    Key j's row is kv_scale * e4m3(kv8[j]) (every channel), its value the
    first d_v channels of that row; q holds bf16 bits. The dequantised rows
    are formed exactly in float64 and passed to ``attention_rows``.
    """
    kv = e4m3_to_float64(kv8) * float(kv_scale)
    q64 = bf16_bits_to_float64(q)
    return attention_rows(q64, kv, kv[:, :, :d_v], cu_q, cu_k, causal=causal, window=window, softcap=softcap,
                          scale=scale, rows=rows, threads=threads, lib=lib)
