"""Pins of the fp64 oracle to things other than itself (CPU only).

* a 50-digit decimal brute force on tiny problems (every mask option, GQA,
  packed batches with unequal/empty segments, Sq != Sk, shared latent kv);
* torch's float64 scaled_dot_product_attention with an explicit boolean mask,
  and torch.logsumexp for the LSE (library routines);
* closed forms: one visible key (O = v exactly), constant V, q = 0 (uniform
  weights: LSE = ln(number of visible keys), which pins every mask edge and
  the inclusive window), softcap limits and a two-key softcap row;
* invariants: GQA == MHA with repeated KV, packed == per-segment, causal last
  row == non-causal last row, window wider than the sequence == causal only,
  x50 inputs stay finite, shared-kv view == copied V;
* planted mistakes: compiled mutants of the oracle source each fail a pin.
"""
from __future__ import annotations

import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import bruteforce

to_np = workloads.to_numpy_bits


def _problem(seed, dtype, hq, hkv, dqk, dv, lens_q, lens_k, shared=False, magnitude=1.0):
    p = workloads.make_problem(seed, dtype=dtype, heads_q=hq, heads_kv=hkv, d_qk=dqk, d_v=dv,
                               lens_q=lens_q, lens_k=lens_k, shared_kv=shared, magnitude=magnitude)
    q = to_np(p["q"])
    if shared:
        kv = to_np(p["kv"])
        k, v = kv, kv[:, :, :dv]
    else:
        k, v = to_np(p["k"]), to_np(p["v"])
    return q, k, v, p["cu_seqlens_q"].numpy(), p["cu_seqlens_k"].numpy()


# (seed, dtype, hq, hkv, dqk, dv, lens_q, lens_k, causal, window, softcap, shared)
BRUTE_CASES = [
    (11, "f32", 1, 1, 8, 8, [5], [5], False, (-1, -1), 0.0, False),
    (12, "bf16", 2, 1, 8, 8, [7], [7], True, (-1, -1), 0.0, False),
    (13, "bf16", 4, 2, 4, 6, [3, 0, 6], [5, 2, 6], True, (-1, -1), 0.0, False),
    (14, "f32", 2, 2, 8, 8, [6], [6], True, (2, 0), 0.0, False),
    (15, "bf16", 2, 1, 8, 8, [8], [8], False, (1, 1), 0.0, False),
    (16, "f32", 1, 1, 8, 8, [4], [6], False, (-1, 1), 2.0, False),
    (17, "bf16", 3, 1, 8, 8, [5], [5], True, (3, -1), 0.5, False),
    (18, "bf16", 4, 1, 8, 6, [2, 3], [6, 4], False, (-1, -1), 0.0, True),
    (19, "f32", 2, 1, 4, 4, [6, 2], [3, 0], True, (-1, -1), 0.0, False),
    (20, "bf16", 2, 2, 8, 8, [5], [9], True, (2, 1), 3.0, False),
]

_BRUTE_CACHE = {}


def _brute(case):
    if case not in _BRUTE_CACHE:
        seed, dt, hq, hkv, dqk, dv, lq, lk, causal, window, cap, shared = case
        q, k, v, cq, ck = _problem(seed, dt, hq, hkv, dqk, dv, lq, lk, shared)
        _BRUTE_CACHE[case] = bruteforce.attention(q, k, v, cq, ck, causal=causal, window=window,
                                                  softcap=cap)
    return _BRUTE_CACHE[case]


def _case_key(case):
    seed, dt, hq, hkv, dqk, dv, lq, lk, causal, window, cap, shared = case
    return (seed, dt, hq, hkv, dqk, dv, tuple(lq), tuple(lk), causal, tuple(window), cap, shared)


def check_brute(case, lib=None):
    seed, dt, hq, hkv, dqk, dv, lq, lk, causal, window, cap, shared = case
    q, k, v, cq, ck = _problem(seed, dt, hq, hkv, dqk, dv, lq, lk, shared)
    o, lse, dev = oracle.attention_rows(q, k, v, cq, ck, causal=causal, window=window, softcap=cap,
                                        lib=lib)
    o_ref, lse_ref = _brute(_case_key(case))
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)), "fully-masked rows differ"
    fin = np.isfinite(lse_ref)
    np.testing.assert_allclose(lse[fin], lse_ref[fin], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    assert np.all(o[~fin] == 0.0), "a row that sees no key must be zero"
    assert dev <= 1e-12


@pytest.mark.parametrize("case", BRUTE_CASES, ids=[f"seed{c[0]}" for c in BRUTE_CASES])
def test_matches_decimal_bruteforce(case):
    check_brute(case)


def _torch_reference(q, k, v, causal, window, scale):
    """float64 SDPA with an explicit boolean mask + torch.logsumexp for LSE (dense)."""
    qt = torch.from_numpy(bruteforce._to_float(q)).permute(0, 2, 1, 3)  # B,H,S,d
    kt = torch.from_numpy(bruteforce._to_float(k)).permute(0, 2, 1, 3)
    vt = torch.from_numpy(bruteforce._to_float(v)).permute(0, 2, 1, 3)
    g = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(g, dim=1)
    vt = vt.repeat_interleave(g, dim=1)
    sq, sk = qt.shape[2], kt.shape[2]
    mask = torch.tensor([[bruteforce.visible(i, j, sq, sk, causal, window[0], window[1])
                          for j in range(sk)] for i in range(sq)])
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    s = torch.matmul(qt, kt.transpose(-1, -2)) * scale
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy()


@pytest.mark.parametrize("causal,window,sq,sk", [
    (False, (-1, -1), 37, 53), (True, (-1, -1), 41, 41), (True, (-1, -1), 29, 61),
    (True, (5, 0), 64, 64), (False, (3, 2), 40, 40), (True, (7, -1), 33, 70)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_matches_torch_sdpa_float64(causal, window, sq, sk, dtype):
    b, hq, hkv, d = 2, 4, 2, 16
    g = torch.Generator().manual_seed(sq * 100 + sk)
    mk = lambda s, h: torch.randn(b, s, h, d, generator=g)
    q, k, v = mk(sq, hq), mk(sk, hkv), mk(sk, hkv)
    if dtype == "bf16":
        q, k, v = q.bfloat16(), k.bfloat16(), v.bfloat16()
    q, k, v = to_np(q), to_np(k), to_np(v)
    scale = d ** -0.5
    o, lse, dev = oracle.attention_dense(q, k, v, causal=causal, window=window, scale=scale)
    o_ref, lse_ref = _torch_reference(q, k, v, causal, window, scale)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)
    assert dev <= 1e-12


def test_mla_matches_torch_materialised():
    """Shared latent kv (qk 576 / v 512): torch float64 bmm -> softmax -> bmm."""
    q, kv, _, cq, ck = _problem(31, "bf16", 16, 1, 576, 512, [4, 4], [100, 37], shared=True)
    v = kv[:, :, :512]
    scale = 1.0 / math.sqrt(576)
    o, lse, _ = oracle.attention_rows(q, kv, v, cq, ck, scale=scale)
    qf = torch.from_numpy(bruteforce._to_float(q))
    kvf = torch.from_numpy(bruteforce._to_float(kv))
    for b in range(2):
        qs = qf[cq[b]:cq[b + 1]].reshape(-1, 576)  # (token, head) rows
        ks = kvf[ck[b]:ck[b + 1], 0]
        s = (qs @ ks.T) * scale
        ref_o = torch.softmax(s, dim=-1) @ ks[:, :512]
        ref_lse = torch.logsumexp(s, dim=-1)
        np.testing.assert_allclose(o[cq[b]:cq[b + 1]].reshape(-1, 512), ref_o.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[cq[b]:cq[b + 1]].reshape(-1), ref_lse.numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms

def check_single_key(lib=None):
    """One visible key: O = v exactly and LSE = that key's (capped) score."""
    q, k, v, cq, ck = _problem(41, "bf16", 2, 1, 16, 16, [9], [9])
    qf, kf = bruteforce._to_float(q), bruteforce._to_float(k)
    vf = bruteforce._to_float(v)
    scale = 0.25
    for cap in (0.0, 1.5):
        o, lse, _ = oracle.attention_rows(q, k, v, cq, ck, causal=True, scale=scale, softcap=cap, lib=lib)
        t = scale * float(np.dot(qf[0, 0], kf[0, 0]))
        s = cap * math.tanh(t / cap) if cap else t
        assert np.array_equal(o[0, 0], vf[0, 0]), "first causal row must equal v_0 exactly"
        assert abs(lse[0, 0] - s) <= 1e-12
        o, lse, _ = oracle.attention_rows(q, k, v, cq, ck, causal=False, window=(0, 0), scale=scale,
                                          softcap=cap, lib=lib)
        for i in range(9):
            for h in range(2):
                t = scale * float(np.dot(qf[i, h], kf[i, 0]))
                s = cap * math.tanh(t / cap) if cap else t
                assert np.array_equal(o[i, h], vf[i, 0])
                assert abs(lse[i, h] - s) <= 1e-12


def test_single_visible_key():
    check_single_key()


def test_constant_v():
    q, k, v, cq, ck = _problem(42, "f32", 4, 2, 32, 32, [50, 17], [70, 17])
    v = np.full_like(v, 1.75)
    for causal, window in ((False, (-1, -1)), (True, (-1, -1)), (True, (8, 0))):
        o, lse, _ = oracle.attention_rows(q, k, v, cq, ck, causal=causal, window=window)
        assert np.all(np.isfinite(lse))
        np.testing.assert_allclose(o, 1.75, rtol=0, atol=1e-14)


def _counts(sq, sk, causal, window):
    """Closed-form visible-key count per row and first visible key."""
    wl, wr = window
    out = []
    for i in range(sq):
        pos = i + sk - sq
        lo = 0 if wl < 0 else max(0, pos - wl)
        hi = sk - 1
        if causal:
            hi = min(hi, pos)
        if wr >= 0:
            hi = min(hi, pos + wr)
        out.append((lo, hi))
    return out


def check_zero_query(lib=None):
    """q = 0: uniform weights, LSE = ln(count), O = mean of the visible V rows."""
    cases = [((5000, 5000), True, (4096, 0)), ((300, 300), True, (-1, -1)),
             ((100, 260), True, (-1, -1)), ((120, 120), False, (10, 20)),
             ((90, 150), False, (-1, -1)), ((64, 64), False, (-1, 5))]
    for (sq, sk), causal, window in cases:
        q, k, v, cq, ck = _problem(43, "bf16", 1, 1, 8, 8, [sq], [sk])
        q = np.zeros_like(q)
        vf = bruteforce._to_float(v)
        rows = sorted({0, 1, 2, sq // 2, sq - 2, sq - 1, min(sq - 1, 4096), min(sq - 1, 4097)})
        o, lse, _ = oracle.attention_rows(q, k, v, cq, ck, causal=causal, window=window,
                                          rows=[(i, 0) for i in rows], lib=lib)
        bounds = _counts(sq, sk, causal, window)
        for n, i in enumerate(rows):
            lo, hi = bounds[i]
            assert abs(lse[n] - math.log(hi - lo + 1)) <= 1e-12, (sq, sk, causal, window, i)
            np.testing.assert_allclose(o[n], vf[lo:hi + 1, 0].mean(axis=0), rtol=0, atol=1e-13)


def test_zero_query_counts_pin_mask_edges():
    check_zero_query()


def test_window_4096_is_inclusive():
    """An interior row of a (4096, 0) causal window sees 4097 keys: LSE = ln 4097."""
    q, k, v, cq, ck = _problem(44, "bf16", 1, 1, 8, 8, [4500], [4500])
    q = np.zeros_like(q)
    _, lse, _ = oracle.attention_rows(q, k, v, cq, ck, causal=True, window=(4096, 0), rows=[(4400, 0)])
    assert abs(lse[0] - math.log(4097)) < 1e-12
    assert abs(lse[0] - math.log(4096)) > 1e-4


def test_softcap_limits():
    q, k, v, cq, ck = _problem(45, "f32", 2, 2, 16, 16, [30], [30])
    o0, l0, _ = oracle.attention_rows(q, k, v, cq, ck, causal=True)
    o1, l1, _ = oracle.attention_rows(q, k, v, cq, ck, causal=True, softcap=1e9)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l0, rtol=0, atol=1e-12)


def test_softcap_two_key_row():
    """Row 1 of a causal problem sees two keys: closed form with capped scores."""
    q, k, v, cq, ck = _problem(46, "bf16", 1, 1, 16, 16, [2], [2], magnitude=6.0)
    qf, kf, vf = (bruteforce._to_float(a) for a in (q, k, v))
    cap, scale = 5.0, 0.5
    o, lse, _ = oracle.attention_rows(q, k, v, cq, ck, causal=True, softcap=cap, scale=scale)
    c = [cap * math.tanh(scale * float(np.dot(qf[1, 0], kf[j, 0])) / cap) for j in range(2)]
    m = max(c)
    e = [math.exp(x - m) for x in c]
    assert abs(lse[1, 0] - (m + math.log(sum(e)))) < 1e-12
    np.testing.assert_allclose(o[1, 0], (e[0] * vf[0, 0] + e[1] * vf[1, 0]) / sum(e), rtol=0, atol=1e-12)


# ------------------------------------------------------------------ invariants

def check_gqa_equals_mha(lib=None):
    q, k, v, cq, ck = _problem(51, "bf16", 8, 2, 16, 16, [20, 33], [25, 33])
    o, lse, _ = oracle.attention_rows(q, k, v, cq, ck, causal=True, lib=lib)
    k4, v4 = np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1)
    o2, lse2, _ = oracle.attention_rows(q, k4, v4, cq, ck, causal=True, lib=lib)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_gqa_equals_mha_with_repeated_kv():
    check_gqa_equals_mha()


def test_packed_equals_per_segment_and_detects_shift():
    lens_q, lens_k = [17, 1, 40, 9], [17, 5, 40, 30]
    q, k, v, cq, ck = _problem(52, "bf16", 4, 2, 16, 16, lens_q, lens_k)
    o, lse, _ = oracle.attention_rows(q, k, v, cq, ck, causal=True, window=(6, -1))
    for b in range(4):
        sl_q, sl_k = slice(cq[b], cq[b + 1]), slice(ck[b], ck[b + 1])
        ob, lb, _ = oracle.attention_rows(q[sl_q], k[sl_k], v[sl_k], np.array([0, lens_q[b]]),
                                          np.array([0, lens_k[b]]), causal=True, window=(6, -1))
        assert np.array_equal(o[sl_q], ob) and np.array_equal(lse[sl_q], lb)
    shifted = ck.copy()
    shifted[1:-1] += 1
    o2, _, _ = oracle.attention_rows(q, k, v, cq, shifted, causal=True, window=(6, -1))
    assert not np.allclose(o2, o), "shifting a segment boundary must change the result"


def test_causal_last_row_equals_noncausal():
    q, k, v, cq, ck = _problem(53, "f32", 2, 1, 16, 16, [31], [31])
    oc, lc, _ = oracle.attention_rows(q, k, v, cq, ck, causal=True)
    on, ln_, _ = oracle.attention_rows(q, k, v, cq, ck, causal=False)
    assert np.array_equal(oc[-1], on[-1]) and np.array_equal(lc[-1], ln_[-1])
    assert not np.allclose(oc[0], on[0])


def test_window_wider_than_sequence_is_causal():
    q, k, v, cq, ck = _problem(54, "bf16", 2, 2, 16, 16, [40], [40])
    oc, lc, _ = oracle.attention_rows(q, k, v, cq, ck, causal=True)
    ow, lw, _ = oracle.attention_rows(q, k, v, cq, ck, causal=True, window=(40, 0))
    assert np.array_equal(oc, ow) and np.array_equal(lc, lw)


def test_x50_inputs_stay_finite():
    case = (55, "f32", 2, 1, 8, 8, [6], [6], True, (-1, -1), 0.0, False)
    q, k, v, cq, ck = _problem(55, "f32", 2, 1, 8, 8, [6], [6], magnitude=50.0)
    o, lse, dev = oracle.attention_rows(q, k, v, cq, ck, causal=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)) and dev < 1e-12
    o_ref, lse_ref = bruteforce.attention(q, k, v, cq, ck, causal=True)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-9)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-13, atol=0)


def test_shared_kv_view_equals_copy():
    q, kv, v, cq, ck = _problem(56, "bf16", 16, 1, 64, 48, [3, 4], [20, 9], shared=True)
    o1, l1, _ = oracle.attention_rows(q, kv, v, cq, ck)
    o2, l2, _ = oracle.attention_rows(q, kv, np.ascontiguousarray(v), cq, ck)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_problem_with_no_tokens():
    """A packed problem whose segments hold no queries and no keys (the empty
    arrays torch hands over may carry strides that describe no layout)."""
    p = workloads.make_problem(58, dtype="bf16", heads_q=16, heads_kv=4, d_qk=64, d_v=64, lens_q=[0], lens_k=[0])
    q, k, v = (t.float().numpy() for t in (p["q"], p["k"], p["v"]))
    o, lse, _ = oracle.attention_rows(q, k, v, p["cu_seqlens_q"].numpy(), p["cu_seqlens_k"].numpy())
    assert o.shape == (0, 16, 64) and lse.shape == (0, 16)


def test_row_selection_matches_full():
    q, k, v, cq, ck = _problem(57, "bf16", 4, 2, 16, 16, [10, 20], [10, 25])
    o, lse, _ = oracle.attention_rows(q, k, v, cq, ck, causal=True)
    rows = [(0, 0), (29, 3), (12, 1), (9, 2)]
    os_, ls, _ = oracle.attention_rows(q, k, v, cq, ck, causal=True, rows=rows)
    for n, (t, h) in enumerate(rows):
        assert np.array_equal(os_[n], o[t, h]) and ls[n] == lse[t, h]


# -------------------------------------------------------------- paged cache

def test_gather_paged_worked_example():
    # Three pages of two rows; row r of page g holds the value 10 g + r. Key j
    # of sequence b is row j mod 2 of page table[b][j div 2]: sequence 0
    # (3 keys, pages 2 then 0) reads 20, 21, 0; sequence 1 (1 key, page 1)
    # reads 10, and its second table entry (7, outside the cache) lies past
    # its last page, so it is never read.
    cache = np.array([[[[10.0 * g + r]] for r in range(2)] for g in range(3)], dtype=np.float32)
    table = np.array([[2, 0], [1, 7]], dtype=np.int32)
    kv, cu = oracle.gather_paged(cache, table, [3, 1])
    assert cu.tolist() == [0, 3, 4]
    assert kv.reshape(-1).tolist() == [20.0, 21.0, 0.0, 10.0]


def test_gather_paged_rejects_bad_pages():
    cache = np.zeros((2, 4, 1, 8), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.gather_paged(cache, np.array([[0, 2]], dtype=np.int32), [5])  # page 2 of 2
    with pytest.raises(ValueError):
        oracle.gather_paged(cache, np.array([[1]], dtype=np.int32), [5])  # needs 2 table entries


@pytest.mark.parametrize("page_size,lens", [(32, [1, 70, 300]), (64, [64, 0, 128]), (128, [500, 65])])
def test_gather_paged_inverts_paginate(page_size, lens):
    # The input generator scatters packed keys into shuffled pages; gathering
    # them back through the table must give the packed keys exactly.
    gen = torch.Generator("cpu").manual_seed(77)
    kv = torch.randn(sum(lens), 2, 16, generator=gen).to(torch.bfloat16)
    pg = workloads.paginate(kv, lens, page_size, gen, spare_pages=3, fill=float("nan"), table_pad=2,
                            pad_value=1 << 30)
    back, cu = oracle.gather_paged(workloads.to_numpy_bits(pg["kv_cache"]), pg["block_table"].numpy(),
                                   pg["cache_seqlens"].numpy())
    assert np.array_equal(back, workloads.to_numpy_bits(kv))
    assert cu.tolist() == [0] + np.cumsum(lens).tolist()


# ------------------------------------------------------------ fp8 latent cache

def test_e4m3_decoder_worked_values():
    # Values fixed by the E4M3 definition (bias 7, 3 mantissa bits,
    # subnormals m * 2^-9, S.1111.111 = NaN).
    codes = [0x00, 0x80, 0x38, 0xB8, 0x7E, 0xFE, 0x01, 0x07, 0x08, 0x40, 0x3C, 0x77, 0x78]
    want = [0.0, -0.0, 1.0, -1.0, 448.0, -448.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 2.0, 1.5, 240.0, 256.0]
    got = oracle.e4m3_to_float64(codes)
    assert got.tolist() == want
    assert np.signbit(got[1]) and not np.signbit(got[0])
    assert np.isnan(oracle.e4m3_to_float64([0x7F, 0xFF])).all()


def test_e4m3_decoder_matches_torch_float8():
    # Every code against torch's own float8_e4m3fn conversion.
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_to_float64(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])


def test_float64_inputs_equal_bf16_inputs():
    # The float64 input path reads the same values as the bf16 path.
    q, kv, v, cq, ck = _problem(61, "bf16", 16, 1, 64, 48, [3, 4], [20, 9], shared=True)
    o1, l1, _ = oracle.attention_rows(q, kv, v, cq, ck, causal=True)
    q64, kv64 = oracle.bf16_bits_to_float64(q), oracle.bf16_bits_to_float64(kv)
    o2, l2, _ = oracle.attention_rows(q64, kv64, kv64[:, :, :48], cq, ck, causal=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_fp8_latent_with_power_of_two_scale_equals_bf16_cache():
    # With a power-of-two scale every dequantised value is a bf16 value, so
    # the fp8 path must give exactly the bf16 path's result on those values.
    gen = torch.Generator("cpu").manual_seed(62)
    q = torch.randn(7, 8, 64, generator=gen).to(torch.bfloat16)
    kv8 = (torch.randn(30, 1, 64, generator=gen) * 8).to(torch.float8_e4m3fn)
    kvb = (kv8.to(torch.float32) * 0.25).to(torch.bfloat16)
    cq = np.array([0, 3, 7], dtype=np.int32)
    ck = np.array([0, 12, 30], dtype=np.int32)
    bits = workloads.to_numpy_bits
    o1, l1, _ = oracle.attention_rows_fp8_latent(bits(q), kv8.view(torch.uint8).numpy(), 0.25, cq, ck, d_v=48,
                                                 causal=True, scale=0.125)
    kvn = bits(kvb)
    o2, l2, _ = oracle.attention_rows(bits(q), kvn, kvn[:, :, :48], cq, ck, causal=True, scale=0.125)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# Planted mistakes in the Python-side oracle functions: each mutant is a copy
# of the function's source with one plausible error, and each must fail one
# of the pins above.
PY_MUTANTS = {
    "gather_row_page_swapped": ("gather_paged", "rows.append(kv_cache[page, j % page_size])",
                                "rows.append(kv_cache[page, j // page_size])"),
    "gather_page_index_off": ("gather_paged", "logical = j // page_size", "logical = (j + 1) // page_size"),
    "gather_table_transposed": ("gather_paged", "page = int(table[b, logical])", "page = int(table[logical % table.shape[0], b % table.shape[1]])"),
    "e4m3_bias_8": ("e4m3_to_float64", "np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)"),
    "e4m3_subnormal_scale": ("e4m3_to_float64", "m * 2.0 ** -9", "m * 2.0 ** -10"),
    "e4m3_no_nan": ("e4m3_to_float64", "(e == 15) & (m == 7)", "(e == 16) & (m == 7)"),
    "e4m3_mantissa_4bits": ("e4m3_to_float64", "(1.0 + m / 8.0)", "(1.0 + m / 16.0)"),
}


def _python_pins_fail(name, fn) -> bool:
    saved = getattr(oracle, name)
    setattr(oracle, name, fn)
    try:
        checks = ([test_gather_paged_worked_example, test_gather_paged_rejects_bad_pages]
                  + [lambda ps=ps, ls=ls: test_gather_paged_inverts_paginate(ps, ls)
                     for ps, ls in [(32, [1, 70, 300]), (64, [64, 0, 128])]]
                  + [test_e4m3_decoder_worked_values, test_e4m3_decoder_matches_torch_float8])
        for chk in checks:
            try:
                chk()
            except (AssertionError, ValueError, IndexError, pytest.fail.Exception):
                return True
        return False
    finally:
        setattr(oracle, name, saved)


@pytest.mark.parametrize("mutant", sorted(PY_MUTANTS))
def test_planted_python_mistake_fails_a_pin(mutant):
    import inspect
    import textwrap
    name, before, after = PY_MUTANTS[mutant]
    src = textwrap.dedent(inspect.getsource(getattr(oracle, name)))
    assert src.count(before) == 1, f"mutation site for {mutant} not found exactly once"
    ns = {"np": np}
    exec(compile(src.replace(before, after), f"<mutant {mutant}>", "exec"), ns)
    assert _python_pins_fail(name, ns[name]), f"planted mistake {mutant} passed every pin"


def test_unmutated_python_oracle_passes_pins():
    for name in ("gather_paged", "e4m3_to_float64"):
        assert not _python_pins_fail(name, getattr(oracle, name))


# ----------------------------------------------------------- planted mistakes

MUTANTS = {
    "top_left_causal": ("if (p->causal && i + off < hi) hi = i + off;", "if (p->causal && i < hi) hi = i;"),
    "exclusive_window": ("lo = i + off - p->window_left;", "lo = i + off - p->window_left + 1;"),
    "gqa_modulo": ("const int g = h / group;", "const int g = h % p->heads_kv;"),
    "dropped_scale": ("double t = p->scale * dot;", "double t = dot;"),
    "cap_before_scale": ("if (p->softcap > 0.0) t = p->softcap * tanh(t / p->softcap);",
                         "if (p->softcap > 0.0) t = p->scale * p->softcap * tanh(dot / p->softcap);"),
    "lse_without_max": ("lse[r] = m + log(z);", "lse[r] = log(z);"),
    "v_row_offset": ("(p->cu_k[b] + lo + j) * p->v_tok_stride", "(p->cu_k[b] + j) * p->v_tok_stride"),
    "exp_sign": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "masked_row_lse": ("lse[r] = -INFINITY;", "lse[r] = 0.0;"),
    "k_strides_swapped": ("(p->cu_k[b] + j) * p->k_tok_stride + (int64_t)g * p->k_head_stride",
                          "(p->cu_k[b] + j) * p->k_head_stride + (int64_t)g * p->k_tok_stride"),
    "k_segment_from_q": ("(p->cu_k[b] + j) * p->k_tok_stride", "(p->cu_q[b] + j) * p->k_tok_stride"),
    "unnormalised": ("s[j] /= z;", "s[j] /= 1.0;"),
    "right_window_ignored": ("if (p->window_right >= 0 && i + off + p->window_right < hi)",
                             "if (0 && i + off + p->window_right < hi)"),
}


def _pins_fail(lib) -> bool:
    checks = [lambda c=c: check_brute(c, lib) for c in BRUTE_CASES]
    checks += [lambda: check_single_key(lib), lambda: check_zero_query(lib),
               lambda: check_gqa_equals_mha(lib)]
    for chk in checks:
        try:
            chk()
        except (AssertionError, ValueError):
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "attention_oracle.c")).read()
    assert src.count(before) == 1, f"mutation site for {name} not found exactly once"
    mutant_c = tmp_path / "mutant.c"
    mutant_c.write_text(src.replace(before, after))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-o", str(so),
                    str(mutant_c), "-lm"], check=True)
    lib = oracle.load_library(str(so))
    assert _pins_fail(lib), f"planted mistake {name} passed every pin"


def test_unmutated_oracle_passes_pins():
    assert not _pins_fail(oracle._load())
