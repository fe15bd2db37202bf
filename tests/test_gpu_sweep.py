"""GPU parity on seeded random configurations of every entry point.

Each case draws its shape and options from a fixed seed: ragged segment
lengths (empty ones included), Sq below, equal to or above Sk, GQA ratios,
both head dims, causal / sliding-window / two-sided masks, softcap and the
softmax scale; the decode entry points also draw split counts, page sizes and
query tokens per sequence. Every output element and LSE is compared with the
fp64 oracle on the same stored inputs, to the tolerances of the method:
max |O - O_ref| <= 1e-5 (fp32) or 1e-2 (bf16), |LSE - LSE_ref| <= 1e-4.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from tests.gpu_helpers import compare, dev, gpu_varlen, oracle_varlen, to_np

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("tiled_attention_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mx.load_library()


def _mask(rng):
    """(causal, window, softcap) drawn from the supported options."""
    causal = bool(rng.random() < 0.6)
    u = rng.random()
    if u < 0.5:
        window = (-1, -1)
    elif u < 0.75:
        window = (int(rng.integers(0, 160)), 0)
    else:
        window = (int(rng.integers(-1, 120)), int(rng.integers(-1, 120)))
    cap = 0.0 if rng.random() < 0.6 else float(np.round(rng.uniform(5.0, 60.0), 2))
    return causal, window, cap


def _scale(rng, d):
    # Around the usual d^-1/2, where bf16 P keeps the stated tolerance.
    return float(d ** -0.5 * rng.uniform(0.5, 1.5))


def _lens_k(rng, lens_q, hi):
    """Key lengths: equal to the query lengths, longer (a cache prefix), or independent."""
    u = rng.random()
    if u < 0.4:
        return list(lens_q)
    if u < 0.75:
        return [int(x + rng.integers(0, hi)) for x in lens_q]
    return [int(rng.integers(0, hi + 100)) for _ in lens_q]


# ------------------------------------------------------------- prefill

def _prefill_case(i):
    rng = np.random.default_rng(41_000 + i)
    dtype = "f32" if i % 4 == 3 else "bf16"
    d = int(rng.choice([64, 128]))
    b = int(rng.integers(1, 5))
    lens_q = [int(rng.integers(0, 261)) if rng.random() > 0.1 else 0 for _ in range(b)]
    lens_k = _lens_k(rng, lens_q, 200)
    hkv = int(rng.choice([1, 2, 4]))
    hq = hkv * int(rng.choice([1, 2, 3, 4]))
    causal, window, cap = _mask(rng)
    return dict(seed=41_000 + i, dtype=dtype, d=d, lens_q=lens_q, lens_k=lens_k, hq=hq, hkv=hkv, causal=causal,
                window=window, cap=cap, scale=_scale(rng, d))


PREFILL = [_prefill_case(i) for i in range(64)]


@pytest.mark.parametrize("c", PREFILL, ids=[f"prefill{i}" for i in range(len(PREFILL))])
def test_random_varlen_prefill(c):
    print(f"[sweep-prefill] {c}", flush=True)
    p = workloads.make_problem(c["seed"], dtype=c["dtype"], heads_q=c["hq"], heads_kv=c["hkv"], d_qk=c["d"],
                               d_v=c["d"], lens_q=c["lens_q"], lens_k=c["lens_k"])
    kw = dict(causal=c["causal"], window=c["window"], softcap=c["cap"], scale=c["scale"])
    o_g, lse_g = gpu_varlen(p, **kw)
    o_ref, lse_ref, _ = oracle_varlen(p, **kw)
    compare(o_g.reshape(-1, c["d"]), lse_g.T.reshape(-1), o_ref.reshape(-1, c["d"]), lse_ref.reshape(-1),
            c["dtype"], str(c))


def _dense_case(i):
    rng = np.random.default_rng(42_000 + i)
    dtype = "f32" if i % 4 == 3 else "bf16"
    d = int(rng.choice([64, 128]))
    b = int(rng.integers(1, 4))
    sq = int(rng.integers(1, 300))
    sk = int(rng.choice([sq, sq + int(rng.integers(0, 300)), int(rng.integers(1, 300))]))
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    causal, window, cap = _mask(rng)
    return dict(seed=42_000 + i, dtype=dtype, d=d, b=b, sq=sq, sk=sk, hq=hq, hkv=hkv, causal=causal,
                window=window, cap=cap, scale=_scale(rng, d))


DENSE = [_dense_case(i) for i in range(32)]


@pytest.mark.parametrize("c", DENSE, ids=[f"dense{i}" for i in range(len(DENSE))])
def test_random_dense_prefill(c):
    print(f"[sweep-dense] {c}", flush=True)
    b, sq, sk, d, hq, hkv = c["b"], c["sq"], c["sk"], c["d"], c["hq"], c["hkv"]
    p = workloads.make_problem(c["seed"], dtype=c["dtype"], heads_q=hq, heads_kv=hkv, d_qk=d, d_v=d,
                               lens_q=[sq] * b, lens_k=[sk] * b, dense=True)
    kw = dict(causal=c["causal"], window=c["window"], softcap=c["cap"], scale=c["scale"])
    o, lse = mx.mxfa_fwd(p["q"].to(dev()), p["k"].to(dev()), p["v"].to(dev()), **kw)
    torch.cuda.synchronize()
    packed = {"q": p["q"].reshape(b * sq, hq, d), "k": p["k"].reshape(b * sk, hkv, d),
              "v": p["v"].reshape(b * sk, hkv, d), "cu_seqlens_q": p["cu_seqlens_q"],
              "cu_seqlens_k": p["cu_seqlens_k"]}
    o_ref, lse_ref, _ = oracle_varlen(packed, **kw)
    o_g = o.float().cpu().numpy().reshape(-1, d)
    lse_g = lse.cpu().numpy().transpose(0, 2, 1).reshape(-1)  # [B,Hq,Sq] -> token-major rows
    compare(o_g, lse_g, o_ref.reshape(-1, d), lse_ref.reshape(-1), c["dtype"], str(c))


# ------------------------------------------------------------- decode

def _decode_shape(rng, hq_choices, hi_k):
    b = int(rng.integers(1, 6))
    lens_q = [int(rng.integers(0, 9)) if rng.random() > 0.1 else 0 for _ in range(b)]
    lens_k = [int(rng.integers(0, hi_k)) if rng.random() > 0.1 else 0 for _ in range(b)]
    if max(lens_q) == 0:
        lens_q[0] = 1
    if max(lens_k) == 0:
        lens_k[-1] = 1
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice(hq_choices))
    return lens_q, lens_k, hq, hkv


def _latent_case(i, base):
    rng = np.random.default_rng(base + i)
    lens_q, lens_k, hq, hkv = _decode_shape(rng, [1, 4, 8, 16, 20], 1300)
    causal, window, cap = _mask(rng)
    splits = int(rng.choice([0, 0, 1, 2, 3, 5, 8]))
    return dict(seed=base + i, lens_q=lens_q, lens_k=lens_k, hq=hq, hkv=hkv, causal=causal, window=window,
                cap=cap, splits=splits, scale=_scale(rng, 576), page=int(rng.choice([32, 64, 128, 256])))


LATENT = [_latent_case(i, 43_000) for i in range(24)]
LATENT_FP8 = [_latent_case(i, 44_000) for i in range(16)]
LATENT_PAGED = [_latent_case(i, 45_000) for i in range(16)]


def _latent_problem(c):
    return workloads.make_problem(c["seed"], dtype="bf16", heads_q=c["hq"], heads_kv=c["hkv"], d_qk=576, d_v=512,
                                  lens_q=c["lens_q"], lens_k=c["lens_k"], shared_kv=True)


def _mask_kw(c):
    return dict(causal=c["causal"], window=c["window"], softcap=c["cap"], scale=c["scale"])


def _latent_oracle(p, c, kv=None, cu_k=None):
    import oracle

    kv = to_np(p["kv"]) if kv is None else kv
    cu_k = p["cu_seqlens_k"].numpy() if cu_k is None else cu_k
    return oracle.attention_rows(to_np(p["q"]), kv, kv[:, :, :512], p["cu_seqlens_q"].numpy(), cu_k, **_mask_kw(c))


def _check_latent(o, lse, o_ref, lse_ref, c):
    torch.cuda.synchronize()
    compare(o.float().cpu().numpy().reshape(-1, 512), lse.cpu().numpy().T.reshape(-1), o_ref.reshape(-1, 512),
            lse_ref.reshape(-1), "bf16", str(c))


@pytest.mark.parametrize("c", LATENT, ids=[f"latent{i}" for i in range(len(LATENT))])
def test_random_latent_decode(c):
    print(f"[sweep-latent] {c}", flush=True)
    p = _latent_problem(c)
    d = dev()
    o, lse = mx.mxfa_decode_splitkv(p["q"].to(d), p["kv"].to(d), p["cu_seqlens_q"].to(d), p["cu_seqlens_k"].to(d),
                                    max(c["lens_q"]), max(c["lens_k"]), head_dim_v=512, num_splits=c["splits"],
                                    **_mask_kw(c))
    o_ref, lse_ref, _ = _latent_oracle(p, c)
    _check_latent(o, lse, o_ref, lse_ref, c)


@pytest.mark.parametrize("c", LATENT_FP8, ids=[f"fp8-{i}" for i in range(len(LATENT_FP8))])
def test_random_fp8_latent_decode(c):
    print(f"[sweep-fp8] {c}", flush=True)
    p = _latent_problem(c)
    p.update(workloads.quantize_e4m3(p["kv"].float()))
    d = dev()
    o, lse = mx.mxfa_decode_splitkv_fp8(p["q"].to(d), p["kv8"].to(d), p["cu_seqlens_q"].to(d),
                                        p["cu_seqlens_k"].to(d), max(c["lens_q"]), max(c["lens_k"]), p["kv_scale"],
                                        head_dim_v=512, num_splits=c["splits"], **_mask_kw(c))
    import oracle

    o_ref, lse_ref, _ = oracle.attention_rows_fp8_latent(to_np(p["q"]), p["kv8"].numpy(), p["kv_scale"],
                                                         p["cu_seqlens_q"].numpy(), p["cu_seqlens_k"].numpy(),
                                                         d_v=512, **_mask_kw(c))
    _check_latent(o, lse, o_ref, lse_ref, c)


@pytest.mark.parametrize("c", LATENT_PAGED, ids=[f"paged{i}" for i in range(len(LATENT_PAGED))])
def test_random_paged_latent_decode(c):
    print(f"[sweep-paged] {c}", flush=True)
    p = _latent_problem(c)
    gen = torch.Generator("cpu").manual_seed(c["seed"] + 1)
    pg = workloads.paginate(p["kv"], c["lens_k"], c["page"], gen, spare_pages=2, fill=float("nan"), table_pad=1,
                            pad_value=1 << 30)
    d = dev()
    o, lse = mx.mxfa_decode_splitkv_paged(p["q"].to(d), pg["kv_cache"].to(d), p["cu_seqlens_q"].to(d),
                                          pg["cache_seqlens"].to(d), pg["block_table"].to(d), max(c["lens_q"]),
                                          max(c["lens_k"]), head_dim_v=512, num_splits=c["splits"], **_mask_kw(c))
    import oracle

    kv, cu_k = oracle.gather_paged(to_np(pg["kv_cache"]), pg["block_table"].numpy(), pg["cache_seqlens"].numpy())
    o_ref, lse_ref, _ = _latent_oracle(p, c, kv=kv, cu_k=cu_k)
    _check_latent(o, lse, o_ref, lse_ref, c)


def _gqa_case(i):
    rng = np.random.default_rng(46_000 + i)
    lens_q, lens_k, _, _ = _decode_shape(rng, [1], 3000)
    hkv = int(rng.choice([1, 2, 4, 8]))
    hq = hkv * int(rng.choice([1, 2, 4, 8, 12]))
    d = int(rng.choice([64, 128]))
    causal, window, cap = _mask(rng)
    splits = int(rng.choice([0, 0, 1, 2, 4, 7, 16]))
    return dict(seed=46_000 + i, lens_q=lens_q, lens_k=lens_k, hq=hq, hkv=hkv, d=d, causal=causal, window=window,
                cap=cap, splits=splits, scale=_scale(rng, d))


GQA = [_gqa_case(i) for i in range(32)]


@pytest.mark.parametrize("c", GQA, ids=[f"gqa{i}" for i in range(len(GQA))])
def test_random_gqa_decode(c):
    print(f"[sweep-gqa] {c}", flush=True)
    p = workloads.make_problem(c["seed"], dtype="bf16", heads_q=c["hq"], heads_kv=c["hkv"], d_qk=c["d"], d_v=c["d"],
                               lens_q=c["lens_q"], lens_k=c["lens_k"])
    d = dev()
    o, lse = mx.mxfa_decode_splitkv_gqa(p["q"].to(d), p["k"].to(d), p["v"].to(d), p["cu_seqlens_q"].to(d),
                                        p["cu_seqlens_k"].to(d), max(c["lens_q"]), max(c["lens_k"]),
                                        num_splits=c["splits"], **_mask_kw(c))
    torch.cuda.synchronize()
    o_ref, lse_ref, _ = oracle_varlen(p, **_mask_kw(c))
    compare(o.float().cpu().numpy().reshape(-1, c["d"]), lse.cpu().numpy().T.reshape(-1),
            o_ref.reshape(-1, c["d"]), lse_ref.reshape(-1), "bf16", str(c))
