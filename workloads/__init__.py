"""Seeded synthetic inputs for attention problems.

This module is shared by the fp64 oracle tests, the GPU parity tests and the
bench. It only draws random numbers and lays them out; it holds none of the
attention arithmetic (no scores, masks, softmax or reductions).

Recipe (the same for every workload):

* one ``torch.Generator('cpu')`` seeded with the workload's seed;
* draw order: packed-batch lengths (when the workload has them), then q, then
  k, then v -- or q then the shared latent kv for the latent-KV decode, then
  (paged cache only) one permutation of the physical page indices;
* values are float32 ``randn`` (N(0, 1)); bf16 workloads cast them with
  round-to-nearest-even (torch's ``.to(torch.bfloat16)``); an fp8 latent
  cache holds the E4M3 codes of kv / scale with scale = amax / 448
  (``quantize_e4m3``). The stored, already-rounded tensors are the inputs to
  both sides of every comparison.

Layouts: dense ``[B, S, H, d]``; packed (varlen) ``[total, H, d]`` with int32
``cu_seqlens`` of length ``batch + 1`` starting at 0; latent-KV decode keeps a
single ``kv`` buffer ``[total_k, H_kv, d_qk]`` whose first ``d_v`` channels are
V; its paged form (``paginate``) is a cache ``[num_pages, page_size, H_kv,
d_qk]`` with an int32 ``block_table [B, max_pages]`` and ``cache_seqlens [B]``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import torch

__all__ = [
    "Workload",
    "WORKLOADS",
    "get",
    "make_inputs",
    "make_problem",
    "paginate",
    "quantize_e4m3",
    "varlen_lengths",
    "to_numpy_bits",
]


@dataclass(frozen=True)
class Workload:
    """One attention problem: shapes, options and the seed of its inputs."""

    name: str
    seed: int
    kind: str  # "dense" | "varlen" | "decode" (shared latent kv) | "gqa_decode" (separate k, v; packed)
    dtype: str  # "f32" | "bf16"
    batch: int
    heads_q: int
    heads_kv: int
    d_qk: int
    d_v: int
    seqlen_q: int = 0  # dense and decode: per-sequence length
    seqlen_k: int = 0
    len_lo: int = 0  # varlen: lengths drawn uniformly from [len_lo, len_hi]
    len_hi: int = 0
    causal: bool = False
    window: tuple = (-1, -1)
    softcap: float = 0.0
    scale: Optional[float] = None  # None -> d_qk ** -0.5
    page_size: int = 0  # decode: > 0 stores the latent kv in a paged cache of this many rows per page
    kv_dtype: str = ""  # decode: "fp8" stores the latent kv as OCP e4m3 codes with one per-tensor scale
    note: str = field(default="", compare=False)

    @property
    def softmax_scale(self) -> float:
        return float(self.scale) if self.scale is not None else 1.0 / math.sqrt(self.d_qk)


# The five workloads of the method's headline configurations (seeds are the
# configuration index), then further workloads.
WORKLOADS = {
    "single_head_f32": Workload(
        name="single_head_f32", seed=0, kind="dense", dtype="f32", batch=1, heads_q=1,
        heads_kv=1, d_qk=64, d_v=64, seqlen_q=128, seqlen_k=128, causal=False,
        note="B=1 H=1 S=128 d=64 fp32, non-causal"),
    "causal_prefill_bf16": Workload(
        name="causal_prefill_bf16", seed=1, kind="dense", dtype="bf16", batch=4, heads_q=16,
        heads_kv=16, d_qk=128, d_v=128, seqlen_q=2048, seqlen_k=2048, causal=True,
        note="B=4 H=16 S=2048 d=128 bf16, causal"),
    "varlen_gqa_causal_bf16": Workload(
        name="varlen_gqa_causal_bf16", seed=2, kind="varlen", dtype="bf16", batch=16,
        heads_q=32, heads_kv=8, d_qk=128, d_v=128, len_lo=64, len_hi=4096, causal=True,
        note="16 packed sequences, lengths U[64,4096], Hq=32 Hkv=8 d=128 bf16, causal"),
    "mla_decode_bf16": Workload(
        name="mla_decode_bf16", seed=3, kind="decode", dtype="bf16", batch=128, heads_q=16,
        heads_kv=1, d_qk=576, d_v=512, seqlen_q=4, seqlen_k=8192, causal=False,
        scale=1.0 / math.sqrt(576),
        note="batch 128, q_len 4, 16 heads, shared latent kv 576/512, kv_len 8192, bf16"),
    "window_softcap_bf16": Workload(
        name="window_softcap_bf16", seed=4, kind="dense", dtype="bf16", batch=1, heads_q=32,
        heads_kv=8, d_qk=128, d_v=128, seqlen_q=32768, seqlen_k=32768, causal=True,
        window=(4096, 0), softcap=50.0,
        note="B=1 Hq=32 Hkv=8 S=32768 d=128 bf16, causal, window (4096,0), softcap 50"),
    # Beyond the headline set: a prefill chunk of 2048 new tokens attending to
    # a 16384-token sequence whose first 14336 tokens are already cached
    # (Sq < Sk, bottom-right causal alignment).
    "chunked_prefill_bf16": Workload(
        name="chunked_prefill_bf16", seed=5, kind="dense", dtype="bf16", batch=2, heads_q=32,
        heads_kv=8, d_qk=128, d_v=128, seqlen_q=2048, seqlen_k=16384, causal=True,
        note="B=2 Hq=32 Hkv=8 Sq=2048 Sk=16384 d=128 bf16, causal (chunk after a 14336-token cache)"),
    # The latent-KV decode above with the cache in fp8 (e4m3) and one scale.
    "mla_decode_fp8": Workload(
        name="mla_decode_fp8", seed=8, kind="decode", dtype="bf16", batch=128, heads_q=16,
        heads_kv=1, d_qk=576, d_v=512, seqlen_q=4, seqlen_k=8192, causal=False,
        scale=1.0 / math.sqrt(576), kv_dtype="fp8",
        note="mla_decode_bf16's shapes, latent kv as e4m3 codes with a per-tensor scale"),
    # Decode for standard heads: one new token per sequence, 8 query heads per
    # kv head, separate K and V.
    "gqa_decode_bf16": Workload(
        name="gqa_decode_bf16", seed=7, kind="gqa_decode", dtype="bf16", batch=16, heads_q=32,
        heads_kv=4, d_qk=128, d_v=128, seqlen_q=1, seqlen_k=2048, causal=True,
        note="B=16, q_len 1, Hq=32 Hkv=4 d=128, kv_len 2048, bf16"),
    # The latent-KV decode above with its cache in 64-row pages, placed at
    # shuffled physical page indices.
    "paged_mla_decode_bf16": Workload(
        name="paged_mla_decode_bf16", seed=6, kind="decode", dtype="bf16", batch=128, heads_q=16,
        heads_kv=1, d_qk=576, d_v=512, seqlen_q=4, seqlen_k=8192, causal=False,
        scale=1.0 / math.sqrt(576), page_size=64,
        note="mla_decode_bf16's shapes, kv in a paged cache of 64-row pages, shuffled page order"),
}


def get(name: str, **overrides) -> Workload:
    """Return a named workload, optionally with fields replaced (smaller sizes)."""
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


def varlen_lengths(gen: torch.Generator, batch: int, lo: int, hi: int) -> torch.Tensor:
    """Segment lengths drawn uniformly from the inclusive range [lo, hi]."""
    return torch.randint(lo, hi + 1, (batch,), generator=gen, dtype=torch.int64)


def _cu(lengths) -> torch.Tensor:
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    if len(lengths):
        cu[1:] = torch.cumsum(torch.as_tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return cu


def _draw(gen: torch.Generator, shape, dtype: str, magnitude: float = 1.0) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if magnitude != 1.0:
        x.mul_(magnitude)
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def make_problem(seed: int, *, dtype: str, heads_q: int, heads_kv: int, d_qk: int, d_v: int,
                 lens_q, lens_k, shared_kv: bool = False, dense: bool = False,
                 magnitude: float = 1.0) -> dict:
    """Seeded random problem with explicit per-segment lengths.

    Returns CPU tensors: ``q``, ``k``, ``v`` (``kv`` instead of k/v when
    ``shared_kv``), ``cu_seqlens_q``, ``cu_seqlens_k`` and the lengths. With
    ``dense`` all segments must share one length and q/k/v come back in the
    dense ``[B, S, H, d]`` layout (the same memory as the packed layout).
    """
    gen = torch.Generator("cpu").manual_seed(int(seed))
    lens_q = [int(x) for x in lens_q]
    lens_k = [int(x) for x in lens_k]
    if len(lens_q) != len(lens_k):
        raise ValueError("lens_q and lens_k differ in length")
    tq, tk = sum(lens_q), sum(lens_k)
    out = {"lens_q": lens_q, "lens_k": lens_k, "cu_seqlens_q": _cu(lens_q), "cu_seqlens_k": _cu(lens_k)}
    out["q"] = _draw(gen, (tq, heads_q, d_qk), dtype, magnitude)
    if shared_kv:
        if d_v > d_qk:
            raise ValueError("shared kv needs d_v <= d_qk")
        out["kv"] = _draw(gen, (tk, heads_kv, d_qk), dtype, magnitude)
    else:
        out["k"] = _draw(gen, (tk, heads_kv, d_qk), dtype, magnitude)
        out["v"] = _draw(gen, (tk, heads_kv, d_v), dtype, magnitude)
    if dense:
        if len(set(lens_q)) > 1 or len(set(lens_k)) > 1:
            raise ValueError("dense layout needs equal lengths")
        b = len(lens_q)
        sq = lens_q[0] if b else 0
        sk = lens_k[0] if b else 0
        for key in ("q", "k", "v", "kv"):
            if key in out:
                t = out[key]
                s = sq if key == "q" else sk
                out[key] = t.view(b, s, t.shape[1], t.shape[2])
    return out


def paginate(kv: torch.Tensor, lens_k, page_size: int, gen: torch.Generator, *, spare_pages: int = 0,
             fill: float = 0.0, table_pad: int = 0, pad_value: int = -1) -> dict:
    """Scatter packed keys ``kv [sum(lens_k), H, d]`` into a paged cache.

    Sequence b takes ceil(len_b / page_size) pages; the physical page of each
    logical page comes from one ``torch.randperm`` (drawn from ``gen``) over
    all pages, ``spare_pages`` extra pages included. Rows no key fills (the
    tail of each sequence's last page, the spare pages) hold ``fill``; each
    table row is padded with ``pad_value`` to the longest sequence's page
    count plus ``table_pad``. Returns ``kv_cache [num_pages, page_size, H, d]``,
    ``block_table`` int32 ``[B, max_pages]`` and ``cache_seqlens`` int32 ``[B]``.
    """
    lens = [int(x) for x in lens_k]
    pages_of = [(n + page_size - 1) // page_size for n in lens]
    used = sum(pages_of)
    num_pages = used + spare_pages
    perm = torch.randperm(num_pages, generator=gen)
    cache = torch.full((num_pages, page_size) + tuple(kv.shape[1:]), fill, dtype=kv.dtype)
    max_pages = (max(pages_of) if pages_of else 0) + table_pad
    table = torch.full((len(lens), max_pages), pad_value, dtype=torch.int32)
    nxt = 0
    start = 0
    for b, n in enumerate(lens):
        for lp in range(pages_of[b]):
            phys = int(perm[nxt])
            nxt += 1
            table[b, lp] = phys
            rows = min(page_size, n - lp * page_size)
            cache[phys, :rows] = kv[start + lp * page_size:start + lp * page_size + rows]
        start += n
    return {"kv_cache": cache, "block_table": table, "cache_seqlens": torch.tensor(lens, dtype=torch.int32)}


def quantize_e4m3(x: torch.Tensor) -> dict:
    """Input preparation for an fp8 cache: one per-tensor scale, amax / 448
    (448 is the largest E4M3 value), and the codes of x / scale rounded to
    nearest-even by torch's float8_e4m3fn conversion. Returns ``kv8`` (uint8
    codes, same shape) and ``kv_scale`` (a Python float, exactly a float32)."""
    amax = float(x.abs().max()) if x.numel() else 1.0
    scale = float(torch.tensor(amax / 448.0 if amax > 0 else 1.0, dtype=torch.float32))
    codes = (x.to(torch.float32) / scale).to(torch.float8_e4m3fn).view(torch.uint8)
    return {"kv8": codes, "kv_scale": scale}


def make_inputs(w: Workload) -> dict:
    """The inputs of workload ``w`` (see the module docstring for the recipe)."""
    gen = torch.Generator("cpu").manual_seed(int(w.seed))
    if w.kind == "varlen":
        lens = varlen_lengths(gen, w.batch, w.len_lo, w.len_hi).tolist()
        lens_q = lens_k = lens
    else:
        lens_q = [w.seqlen_q] * w.batch
        lens_k = [w.seqlen_k] * w.batch
    tq, tk = sum(lens_q), sum(lens_k)
    out = {"lens_q": lens_q, "lens_k": lens_k, "cu_seqlens_q": _cu(lens_q), "cu_seqlens_k": _cu(lens_k)}
    out["q"] = _draw(gen, (tq, w.heads_q, w.d_qk), w.dtype)
    if w.kind == "decode" and w.kv_dtype == "fp8":
        out.update(quantize_e4m3(_draw(gen, (tk, w.heads_kv, w.d_qk), "f32")))
    elif w.kind == "decode":
        out["kv"] = _draw(gen, (tk, w.heads_kv, w.d_qk), w.dtype)
        if w.page_size:
            out.update(paginate(out["kv"], lens_k, w.page_size, gen))
    else:
        out["k"] = _draw(gen, (tk, w.heads_kv, w.d_qk), w.dtype)
        out["v"] = _draw(gen, (tk, w.heads_kv, w.d_v), w.dtype)
    if w.kind == "dense":
        for key, s in (("q", w.seqlen_q), ("k", w.seqlen_k), ("v", w.seqlen_k)):
            t = out[key]
            out[key] = t.view(w.batch, s, t.shape[1], t.shape[2])
    return out


def to_numpy_bits(t: torch.Tensor):
    """CPU tensor -> numpy array: float32 as is, bf16 as its uint16 bit pattern."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view("uint16")
    if t.dtype == torch.float32:
        return t.contiguous().numpy()
    if t.dtype in (torch.int32, torch.int64):
        return t.contiguous().numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")
