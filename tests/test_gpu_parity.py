"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small problems compare every element; they span several q/k tiles with ragged
tails, GQA, Sq != Sk (bottom-right causal), fully-masked rows, empty
segments, windows and softcap. The five headline workloads run at full size
in the launch configuration the bench times, and every one of their rows is
compared with the oracle (the paged variant of the latent decode on seeded
sampled rows, plus bit equality with the contiguous call). Tolerances:
max |O - O_ref| <= 1e-5 (fp32) or 1e-2 (bf16), |LSE - LSE_ref| <= 1e-4.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import workloads
from tests.gpu_helpers import Stats, compare, dev, gpu_varlen, oracle_varlen, sample_rows, to_np

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("tiled_attention_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mx.load_library()


# (dtype, d, batch, sq, sk, hq, hkv, causal, window, softcap)
DENSE_CASES = [
    ("bf16", 128, 2, 1, 1, 2, 1, True, (-1, -1), 0.0),
    ("bf16", 128, 2, 15, 15, 4, 2, True, (-1, -1), 0.0),
    ("bf16", 128, 1, 129, 129, 8, 2, True, (-1, -1), 0.0),
    ("bf16", 128, 2, 300, 300, 4, 4, False, (-1, -1), 0.0),
    ("bf16", 64, 2, 65, 65, 4, 1, True, (-1, -1), 0.0),
    ("bf16", 64, 1, 127, 200, 2, 1, True, (-1, -1), 0.0),
    ("bf16", 128, 1, 200, 90, 2, 2, True, (-1, -1), 0.0),
    ("bf16", 128, 1, 333, 333, 4, 2, True, (50, 0), 0.0),
    ("bf16", 128, 1, 257, 257, 4, 1, True, (64, 0), 50.0),
    ("bf16", 128, 1, 190, 190, 2, 2, False, (17, 9), 0.0),
    ("bf16", 128, 1, 100, 100, 2, 1, False, (-1, -1), 5.0),
    ("bf16", 64, 3, 96, 160, 6, 3, False, (-1, 40), 0.0),
    ("f32", 64, 1, 128, 128, 1, 1, False, (-1, -1), 0.0),
    ("f32", 128, 2, 70, 70, 4, 2, True, (20, 0), 30.0),
    ("f32", 64, 1, 33, 80, 2, 1, True, (-1, -1), 0.0),
    ("f32", 64, 2, 100, 100, 2, 2, False, (5, 5), 0.0),
]


@pytest.mark.parametrize("case", DENSE_CASES, ids=[
    f"{c[0]}-d{c[1]}-b{c[2]}-{c[3]}x{c[4]}-h{c[5]}/{c[6]}-c{int(c[7])}-w{c[8][0]},{c[8][1]}-cap{c[9]:g}"
    for c in DENSE_CASES])
def test_dense_matches_oracle(case):
    dtype, d, b, sq, sk, hq, hkv, causal, window, cap = case
    seed = 1000 + DENSE_CASES.index(case)
    print(f"[dense] {case} seed={seed}", flush=True)
    p = workloads.make_problem(seed, dtype=dtype, heads_q=hq, heads_kv=hkv, d_qk=d, d_v=d,
                               lens_q=[sq] * b, lens_k=[sk] * b, dense=True)
    scale = d ** -0.5
    q, k, v = p["q"].to(dev()), p["k"].to(dev()), p["v"].to(dev())
    o, lse = mx.mxfa_fwd(q, k, v, causal=causal, window=window, softcap=cap, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref, _ = oracle_varlen(
        {"q": p["q"].reshape(b * sq, hq, d), "k": p["k"].reshape(b * sk, hkv, d),
         "v": p["v"].reshape(b * sk, hkv, d), "cu_seqlens_q": p["cu_seqlens_q"], "cu_seqlens_k": p["cu_seqlens_k"]},
        causal=causal, window=window, softcap=cap, scale=scale)
    o_g = o.float().cpu().numpy().reshape(b * sq * hq, d)
    lse_g = lse.cpu().numpy().transpose(0, 2, 1).reshape(-1)  # [B,Hq,Sq] -> token-major rows
    compare(o_g, lse_g, o_ref.reshape(-1, d), lse_ref.reshape(-1), dtype, str(case))


# (dtype, d, lens_q, lens_k, hq, hkv, causal, window, softcap)
VARLEN_CASES = [
    ("bf16", 128, [1, 0, 130, 64, 257], [1, 0, 130, 64, 257], 4, 2, True, (-1, -1), 0.0),
    ("bf16", 128, [50, 200, 7], [90, 200, 300], 8, 2, True, (-1, -1), 0.0),
    ("bf16", 64, [3, 129, 0, 65], [0, 129, 10, 80], 2, 1, True, (30, 0), 0.0),
    ("bf16", 128, [140, 33], [140, 33], 4, 1, True, (100, 0), 50.0),
    ("bf16", 128, [77, 250], [77, 250], 2, 2, False, (-1, -1), 0.0),
    ("f32", 64, [10, 0, 70], [10, 5, 70], 4, 4, True, (-1, -1), 0.0),
    ("f32", 128, [65, 31], [65, 40], 2, 1, False, (8, 3), 20.0),
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=[f"varlen{i}" for i in range(len(VARLEN_CASES))])
def test_varlen_matches_oracle(case):
    dtype, d, lq, lk, hq, hkv, causal, window, cap = case
    seed = 2000 + VARLEN_CASES.index(case)
    print(f"[varlen] {case} seed={seed}", flush=True)
    p = workloads.make_problem(seed, dtype=dtype, heads_q=hq, heads_kv=hkv, d_qk=d, d_v=d, lens_q=lq, lens_k=lk)
    scale = d ** -0.5
    o_g, lse_g = gpu_varlen(p, causal=causal, window=window, softcap=cap, scale=scale)
    o_ref, lse_ref, _ = oracle_varlen(p, causal=causal, window=window, softcap=cap, scale=scale)
    compare(o_g.reshape(-1, d), lse_g.T.reshape(-1), o_ref.reshape(-1, d), lse_ref.reshape(-1), dtype, str(case))


def test_varlen_work_list_many_segments_dirty_workspace():
    """The work list: more segments than its LDS holds (2500: lengths and prefix sums
    read from global memory), more than one pass of its scan (1500), empty q and k
    segments, a workspace full of garbage beforehand, then smaller problems in the
    same workspace -- every row against the oracle."""
    rng = np.random.RandomState(2600)
    for rep, batch in enumerate((2500, 1500, 37)):
        lq = [int(x) for x in rng.randint(0, 70, batch)]
        lk = [int(q + rng.randint(-5, 40)) if q else int(rng.randint(0, 3)) for q in lq]
        lk = [max(0, x) for x in lk]
        p = workloads.make_problem(2600 + rep, dtype="bf16", heads_q=4, heads_kv=2, d_qk=64, d_v=64, lens_q=lq,
                                   lens_k=lk)
        d = dev()
        if rep == 0:
            nbytes = mx.mxfa_fwd_varlen_workspace_bytes(batch, max(lq), 4, 64)
            ws = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device=d)
        print(f"[varlen] work list: {batch} segments, round {rep}", flush=True)
        o, lse = mx.mxfa_fwd_varlen(p["q"].to(d), p["k"].to(d), p["v"].to(d), p["cu_seqlens_q"].to(d),
                                    p["cu_seqlens_k"].to(d), max(lq), max(lk), causal=True, window=(20, 0),
                                    workspace=ws)
        torch.cuda.synchronize()
        o_ref, lse_ref, _ = oracle_varlen(p, causal=True, window=(20, 0), softcap=0.0, scale=64 ** -0.5)
        compare(o.float().cpu().numpy().reshape(-1, 64), lse.cpu().numpy().T.reshape(-1), o_ref.reshape(-1, 64),
                lse_ref.reshape(-1), "bf16", f"work list {batch} segments")


# The prefill kernel has a variant of its own for scale <= 0 (the logits are
# formed explicitly before the row max instead of folding the scale into the
# exponent): dense and packed, d 64 and 128, causal, windowed and capped.
NONPOS_CASES = [
    (scale_mul, d, causal, window, cap, packed)
    for scale_mul in (-1.0, 0.0)
    for d, causal, window, cap, packed in [
        (64, True, (-1, -1), 0.0, False),
        (128, True, (-1, -1), 0.0, False),
        (128, True, (70, 0), 0.0, True),
        (64, False, (33, 20), 0.0, True),
        (128, True, (-1, -1), 30.0, False),
    ]
]


@pytest.mark.parametrize("case", NONPOS_CASES, ids=[
    f"scale{c[0]:g}-d{c[1]}-c{int(c[2])}-w{c[3][0]},{c[3][1]}-cap{c[4]:g}-{'packed' if c[5] else 'dense'}"
    for c in NONPOS_CASES])
def test_prefill_nonpositive_scale(case):
    scale_mul, d, causal, window, cap, packed = case
    seed = 2500 + NONPOS_CASES.index(case)
    scale = scale_mul * d ** -0.5
    print(f"[prefill] scale={scale} case={case} seed={seed}", flush=True)
    if packed:
        lq, lk = [150, 0, 300], [200, 40, 300]
        p = workloads.make_problem(seed, dtype="bf16", heads_q=4, heads_kv=2, d_qk=d, d_v=d, lens_q=lq, lens_k=lk)
        o_g, lse_g = gpu_varlen(p, causal=causal, window=window, softcap=cap, scale=scale)
        o_ref, lse_ref, _ = oracle_varlen(p, causal=causal, window=window, softcap=cap, scale=scale)
        compare(o_g.reshape(-1, d), lse_g.T.reshape(-1), o_ref.reshape(-1, d), lse_ref.reshape(-1), "bf16",
                str(case))
        return
    b, sq, sk, hq, hkv = 2, 261, 261, 4, 2
    p = workloads.make_problem(seed, dtype="bf16", heads_q=hq, heads_kv=hkv, d_qk=d, d_v=d, lens_q=[sq] * b,
                               lens_k=[sk] * b, dense=True)
    q, k, v = p["q"].to(dev()), p["k"].to(dev()), p["v"].to(dev())
    o, lse = mx.mxfa_fwd(q, k, v, causal=causal, window=window, softcap=cap, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref, _ = oracle_varlen(
        {"q": p["q"].reshape(b * sq, hq, d), "k": p["k"].reshape(b * sk, hkv, d),
         "v": p["v"].reshape(b * sk, hkv, d), "cu_seqlens_q": p["cu_seqlens_q"], "cu_seqlens_k": p["cu_seqlens_k"]},
        causal=causal, window=window, softcap=cap, scale=scale)
    compare(o.float().cpu().numpy().reshape(-1, d), lse.cpu().numpy().transpose(0, 2, 1).reshape(-1),
            o_ref.reshape(-1, d), lse_ref.reshape(-1), "bf16", str(case))


def test_zero_length_calls_are_noops():
    q = torch.empty((0, 16, 4, 128), dtype=torch.bfloat16, device=dev())
    o, lse = mx.mxfa_fwd(q, q, q)
    assert o.numel() == 0
    k = torch.empty((2, 0, 4, 128), dtype=torch.bfloat16, device=dev())
    q = torch.randn((2, 5, 4, 128), device=dev()).bfloat16()
    o, lse = mx.mxfa_fwd(q, k, k)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_first_causal_row_is_v0_exactly():
    p = workloads.make_problem(7, dtype="bf16", heads_q=4, heads_kv=2, d_qk=128, d_v=128, lens_q=[300] * 2,
                               lens_k=[300] * 2, dense=True)
    q, k, v = (p[x].to(dev()) for x in "qkv")
    o, _ = mx.mxfa_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    for h in range(4):
        assert torch.equal(o[:, 0, h].cpu(), p["v"][:, 0, h // 2])


def test_zero_query_lse_counts_keys():
    """q = 0: LSE = ln(number of visible keys) at every row, window (64, 0) causal + Sq < Sk."""
    p = workloads.make_problem(8, dtype="bf16", heads_q=2, heads_kv=1, d_qk=128, d_v=128, lens_q=[300],
                               lens_k=[350], dense=True)
    q = torch.zeros_like(p["q"]).to(dev())
    k, v = p["k"].to(dev()), p["v"].to(dev())
    _, lse = mx.mxfa_fwd(q, k, v, causal=True, window=(64, 0))
    torch.cuda.synchronize()
    lse = lse.cpu().double()
    for i in range(300):
        pos = i + 50
        cnt = min(pos, 64) + 1
        assert abs(lse[0, 0, i].item() - math.log(cnt)) < 1e-4


def _one_key_expectation(q, k, v, lens_q, lens_k, hq, hkv, scale):
    """Window (0, 0): row i of a segment sees only key i + Sk - Sq (when that
    key exists). Then P is a single weight, O is that key's V row and the LSE
    is its scaled score (fp64 from the stored values); other rows see no key."""
    qn, kn, vn = (t.double().numpy() for t in (q, k, v))  # exact widening of the stored values
    g = hq // hkv
    o = np.zeros((qn.shape[0], hq, vn.shape[2]))
    lse = np.full((qn.shape[0], hq), -np.inf)
    sq0 = sk0 = 0
    for lq, lk in zip(lens_q, lens_k):
        for i in range(lq):
            pos = i + lk - lq
            if 0 <= pos < lk:
                for h in range(hq):
                    o[sq0 + i, h] = vn[sk0 + pos, h // g]
                    lse[sq0 + i, h] = scale * float(np.dot(qn[sq0 + i, h], kn[sk0 + pos, h // g]))
        sq0 += lq
        sk0 += lk
    return o, lse


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_window_zero_returns_the_diagonal_value(dtype):
    lens_q, lens_k = [5, 130, 0, 70, 40], [5, 200, 10, 300, 20]
    p = workloads.make_problem(11, dtype=dtype, heads_q=4, heads_kv=2, d_qk=128, d_v=128, lens_q=lens_q,
                               lens_k=lens_k)
    scale = 128 ** -0.5
    print(f"[closed form] window (0, 0) {dtype}", flush=True)
    o_g, lse_g = gpu_varlen(p, causal=True, window=(0, 0), softcap=0.0, scale=scale)
    o_x, lse_x = _one_key_expectation(p["q"], p["k"], p["v"], lens_q, lens_k, 4, 2, scale)
    assert np.array_equal(np.isneginf(lse_g.T), np.isneginf(lse_x))
    fin = np.isfinite(lse_x)
    assert np.abs(lse_g.T[fin] - lse_x[fin]).max() <= 1e-4
    if dtype == "bf16":
        assert np.array_equal(o_g, o_x)  # a single weight of 1 rounds back to the stored value
    else:
        assert np.abs(o_g - o_x).max() <= 1e-5


def test_window_zero_decodes_return_the_diagonal_value():
    scale = 1.0 / math.sqrt(576)
    lens_q, lens_k = [4, 1, 3], [300, 64, 700]
    p = workloads.make_problem(12, dtype="bf16", heads_q=16, heads_kv=1, d_qk=576, d_v=512, lens_q=lens_q,
                               lens_k=lens_k, shared_kv=True)
    print("[closed form] window (0, 0) latent decode", flush=True)
    o_g, lse_g = _run_decode(p, 16, False, (0, 0), 0.0, 3, scale)
    kv = p["kv"]
    o_x, lse_x = _one_key_expectation(p["q"], kv, kv[:, :, :512].contiguous(), lens_q, lens_k, 16, 1, scale)
    assert np.array_equal(o_g, o_x)
    assert np.abs(lse_g.T - lse_x).max() <= 1e-4

    scale = 128 ** -0.5
    lens_q, lens_k = [1, 3, 2], [2000, 70, 129]
    p = workloads.make_problem(13, dtype="bf16", heads_q=32, heads_kv=4, d_qk=128, d_v=128, lens_q=lens_q,
                               lens_k=lens_k)
    print("[closed form] window (0, 0) standard-head decode", flush=True)
    o_g, lse_g = _run_gqa(p, True, (0, 0), 0.0, 4, scale)
    o_x, lse_x = _one_key_expectation(p["q"], p["k"], p["v"], lens_q, lens_k, 32, 4, scale)
    assert np.array_equal(o_g, o_x)
    assert np.abs(lse_g.T - lse_x).max() <= 1e-4


def test_gqa_equals_mha_bitwise():
    p = workloads.make_problem(9, dtype="bf16", heads_q=8, heads_kv=2, d_qk=128, d_v=128, lens_q=[200] * 2,
                               lens_k=[200] * 2, dense=True)
    q, k, v = (p[x].to(dev()) for x in "qkv")
    o1, l1 = mx.mxfa_fwd(q, k, v, causal=True)
    o2, l2 = mx.mxfa_fwd(q, k.repeat_interleave(4, dim=2).contiguous(), v.repeat_interleave(4, dim=2).contiguous(),
                         causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_varlen_equals_per_segment_bitwise():
    lens = [100, 257, 1, 64]
    p = workloads.make_problem(10, dtype="bf16", heads_q=4, heads_kv=2, d_qk=128, d_v=128, lens_q=lens, lens_k=lens)
    d = dev()
    q, k, v = p["q"].to(d), p["k"].to(d), p["v"].to(d)
    o, lse = mx.mxfa_fwd_varlen(q, k, v, p["cu_seqlens_q"].to(d), p["cu_seqlens_k"].to(d), max(lens), max(lens),
                                causal=True)
    start = 0
    for L in lens:
        ob, lb = mx.mxfa_fwd(q[start:start + L][None].contiguous(), k[start:start + L][None].contiguous(),
                             v[start:start + L][None].contiguous(), causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o[start:start + L], ob[0])
        assert torch.equal(lse[:, start:start + L], lb[0])
        start += L


def test_deterministic_bitwise():
    w = workloads.get("causal_prefill_bf16", batch=1, heads_q=4, heads_kv=4, seqlen_q=1000, seqlen_k=1000)
    inp = workloads.make_inputs(w)
    q, k, v = (inp[x].to(dev()) for x in "qkv")
    o1, l1 = mx.mxfa_fwd(q, k, v, causal=True)
    o2, l2 = mx.mxfa_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ------------------------------------------------------------------ decode

# (lens_q, lens_k, hq, hkv, causal, window, softcap, splits)
DECODE_CASES = [
    ([1, 4, 2], [1, 70, 300], 16, 1, False, (-1, -1), 0.0, 0),
    ([4, 4], [1000, 129], 16, 1, False, (-1, -1), 0.0, 3),
    ([9, 1], [200, 64], 16, 2, False, (-1, -1), 0.0, 2),
    ([4, 3], [500, 65], 16, 1, True, (-1, -1), 0.0, 4),
    ([4], [700], 16, 1, True, (100, 0), 30.0, 5),
    ([2, 0, 5], [64, 10, 0], 8, 1, False, (-1, -1), 0.0, 1),
]


def _run_decode(p, hq, causal, window, cap, splits, scale):
    d = dev()
    q, kv = p["q"].to(d), p["kv"].to(d)
    cq, ck = p["cu_seqlens_q"].to(d), p["cu_seqlens_k"].to(d)
    o, lse = mx.mxfa_decode_splitkv(q, kv, cq, ck, max(p["lens_q"]), max(p["lens_k"]), head_dim_v=512,
                                    causal=causal, window=window, softcap=cap, scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"decode{i}" for i in range(len(DECODE_CASES))])
def test_decode_matches_oracle(case):
    lq, lk, hq, hkv, causal, window, cap, splits = case
    seed = 3000 + DECODE_CASES.index(case)
    print(f"[decode] {case} seed={seed}", flush=True)
    p = workloads.make_problem(seed, dtype="bf16", heads_q=hq, heads_kv=hkv, d_qk=576, d_v=512, lens_q=lq,
                               lens_k=lk, shared_kv=True)
    scale = 1.0 / math.sqrt(576)
    o_g, lse_g = _run_decode(p, hq, causal, window, cap, splits, scale)
    kv = to_np(p["kv"])
    import oracle

    o_ref, lse_ref, _ = oracle.attention_rows(to_np(p["q"]), kv, kv[:, :, :512], p["cu_seqlens_q"].numpy(),
                                              p["cu_seqlens_k"].numpy(), causal=causal, window=window,
                                              softcap=cap, scale=scale)
    compare(o_g.reshape(-1, 512), lse_g.T.reshape(-1), o_ref.reshape(-1, 512), lse_ref.reshape(-1), "bf16",
            str(case))


@pytest.mark.parametrize("scale", [-1.0 / math.sqrt(576), 0.0])
def test_decode_nonpositive_scale(scale):
    # A negative scale turns the largest score into the smallest logit; zero
    # gives uniform weights. Both must follow the oracle like any other scale.
    p = workloads.make_problem(3200, dtype="bf16", heads_q=16, heads_kv=1, d_qk=576, d_v=512, lens_q=[4, 2],
                               lens_k=[300, 97], shared_kv=True)
    print(f"[decode] scale={scale}", flush=True)
    o_g, lse_g = _run_decode(p, 16, False, (-1, -1), 0.0, 2, scale)
    kv = to_np(p["kv"])
    import oracle

    o_ref, lse_ref, _ = oracle.attention_rows(to_np(p["q"]), kv, kv[:, :, :512], p["cu_seqlens_q"].numpy(),
                                              p["cu_seqlens_k"].numpy(), causal=False, window=(-1, -1),
                                              softcap=0.0, scale=scale)
    compare(o_g.reshape(-1, 512), lse_g.T.reshape(-1), o_ref.reshape(-1, 512), lse_ref.reshape(-1), "bf16",
            f"scale={scale}")


def test_decode_independent_of_split_count():
    p = workloads.make_problem(3100, dtype="bf16", heads_q=16, heads_kv=1, d_qk=576, d_v=512, lens_q=[4, 4, 1],
                               lens_k=[2000, 333, 64], shared_kv=True)
    scale = 1.0 / math.sqrt(576)
    ref_o, ref_l = _run_decode(p, 16, False, (-1, -1), 0.0, 1, scale)
    for s in (2, 3, 4, 8, 32):
        o, l = _run_decode(p, 16, False, (-1, -1), 0.0, s, scale)
        assert np.abs(o - ref_o).max() <= 1e-2
        assert np.abs(l - ref_l).max() <= 1e-4
    o2, l2 = _run_decode(p, 16, False, (-1, -1), 0.0, 4, scale)
    o3, l3 = _run_decode(p, 16, False, (-1, -1), 0.0, 4, scale)
    assert np.array_equal(o2, o3) and np.array_equal(l2, l3)


# -------------------------------------------------------- fp8 latent decode

# (lens_q, lens_k, hq, hkv, causal, window, softcap, splits)
FP8_CASES = [
    ([1, 4, 2], [1, 70, 300], 16, 1, False, (-1, -1), 0.0, 0),
    ([4, 3], [500, 65], 16, 1, True, (-1, -1), 0.0, 4),
    ([4], [700], 16, 1, True, (100, 0), 30.0, 5),
    ([9, 1], [200, 64], 16, 2, False, (-1, -1), 0.0, 2),
    ([2, 0, 5], [64, 10, 0], 8, 1, False, (-1, -1), 0.0, 1),
    ([4, 4], [1000, 129], 16, 1, False, (-1, -1), 0.0, 3),
]


def _fp8_problem(seed, lq, lk, hq, hkv, magnitude=1.0):
    p = workloads.make_problem(seed, dtype="bf16", heads_q=hq, heads_kv=hkv, d_qk=576, d_v=512, lens_q=lq,
                               lens_k=lk, shared_kv=True)
    p.update(workloads.quantize_e4m3(p["kv"].float() * magnitude))
    return p


def _run_fp8(p, causal, window, cap, splits, scale, kv_scale=None):
    d = dev()
    o, lse = mx.mxfa_decode_splitkv_fp8(p["q"].to(d), p["kv8"].to(d), p["cu_seqlens_q"].to(d),
                                        p["cu_seqlens_k"].to(d), max(p["lens_q"]), max(p["lens_k"]),
                                        p["kv_scale"] if kv_scale is None else kv_scale, head_dim_v=512,
                                        causal=causal, window=window, softcap=cap, scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("case", FP8_CASES, ids=[f"fp8-{i}" for i in range(len(FP8_CASES))])
def test_fp8_decode_matches_oracle(case):
    lq, lk, hq, hkv, causal, window, cap, splits = case
    seed = 3700 + FP8_CASES.index(case)
    print(f"[fp8-decode] {case} seed={seed}", flush=True)
    p = _fp8_problem(seed, lq, lk, hq, hkv)
    scale = 1.0 / math.sqrt(576)
    o_g, lse_g = _run_fp8(p, causal, window, cap, splits, scale)
    import oracle

    o_ref, lse_ref, _ = oracle.attention_rows_fp8_latent(to_np(p["q"]), p["kv8"].numpy(), p["kv_scale"],
                                                         p["cu_seqlens_q"].numpy(), p["cu_seqlens_k"].numpy(),
                                                         d_v=512, causal=causal, window=window, softcap=cap,
                                                         scale=scale)
    compare(o_g.reshape(-1, 512), lse_g.T.reshape(-1), o_ref.reshape(-1, 512), lse_ref.reshape(-1), "bf16",
            str(case))


def test_fp8_decode_equals_bf16_decode_of_dequantised_cache():
    # With a power-of-two scale the dequantised rows are bf16 values and every
    # step of the arithmetic matches the bf16 cache's: equal bit for bit.
    p = _fp8_problem(3790, [4, 2], [600, 97], 16, 1)
    kv_scale = 0.125
    kvb = (p["kv8"].view(torch.float8_e4m3fn).float() * kv_scale).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(576)
    print("[fp8-decode] equals bf16", flush=True)
    o8, l8 = _run_fp8(p, True, (-1, -1), 0.0, 3, scale, kv_scale=kv_scale)
    pb = dict(p, kv=kvb)
    ob, lb = _run_decode(pb, 16, True, (-1, -1), 0.0, 3, scale)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)


# ------------------------------------------------------- paged-cache decode

# (lens_q, lens_k, hq, hkv, causal, window, softcap, splits, page_size)
PAGED_CASES = [
    ([1, 4, 2], [1, 70, 300], 16, 1, False, (-1, -1), 0.0, 0, 32),
    ([4, 4], [1000, 129], 16, 1, True, (-1, -1), 0.0, 3, 64),
    ([4, 1, 3], [500, 0, 65], 16, 2, True, (100, 0), 30.0, 4, 128),
    ([9, 1], [700, 256], 16, 1, False, (-1, -1), 0.0, 5, 256),
]


def _paged_problem(seed, lq, lk, hq, hkv, page_size):
    p = workloads.make_problem(seed, dtype="bf16", heads_q=hq, heads_kv=hkv, d_qk=576, d_v=512, lens_q=lq,
                               lens_k=lk, shared_kv=True)
    gen = torch.Generator("cpu").manual_seed(seed + 1)
    # Rows no key fills hold NaN and table entries past each sequence's last
    # page point far outside the cache: a read of either would show.
    pg = workloads.paginate(p["kv"], lk, page_size, gen, spare_pages=3, fill=float("nan"), table_pad=2,
                            pad_value=1 << 30)
    return p, pg


def _run_paged(p, pg, causal, window, cap, splits, scale):
    d = dev()
    o, lse = mx.mxfa_decode_splitkv_paged(p["q"].to(d), pg["kv_cache"].to(d), p["cu_seqlens_q"].to(d),
                                          pg["cache_seqlens"].to(d), pg["block_table"].to(d), max(p["lens_q"]),
                                          max(p["lens_k"]), head_dim_v=512, causal=causal, window=window,
                                          softcap=cap, scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("case", PAGED_CASES, ids=[f"paged{i}" for i in range(len(PAGED_CASES))])
def test_paged_decode_matches_oracle(case):
    lq, lk, hq, hkv, causal, window, cap, splits, page = case
    seed = 3300 + PAGED_CASES.index(case)
    print(f"[paged] {case} seed={seed}", flush=True)
    p, pg = _paged_problem(seed, lq, lk, hq, hkv, page)
    scale = 1.0 / math.sqrt(576)
    o_g, lse_g = _run_paged(p, pg, causal, window, cap, splits, scale)
    import oracle

    kv, ck = oracle.gather_paged(to_np(pg["kv_cache"]), pg["block_table"].numpy(), pg["cache_seqlens"].numpy())
    o_ref, lse_ref, _ = oracle.attention_rows(to_np(p["q"]), kv, kv[:, :, :512], p["cu_seqlens_q"].numpy(), ck,
                                              causal=causal, window=window, softcap=cap, scale=scale)
    compare(o_g.reshape(-1, 512), lse_g.T.reshape(-1), o_ref.reshape(-1, 512), lse_ref.reshape(-1), "bf16",
            str(case))
    # Same split plan, same arithmetic: the paged call equals the contiguous one bit for bit.
    o_c, lse_c = _run_decode(p, hq, causal, window, cap, splits, scale)
    assert np.array_equal(o_g, o_c) and np.array_equal(lse_g, lse_c)


def test_paged_decode_bad_page_index_touches_only_its_sequence():
    # A page index outside the cache in a page that holds keys: that tile
    # reads as zeros (no memory outside the cache is read); the other
    # sequences stay exact.
    p, pg = _paged_problem(3390, [4, 4], [300, 200], 16, 1, 64)
    pg["block_table"][0, 1] = pg["kv_cache"].shape[0] + 5
    print("[paged] bad page index", flush=True)
    scale = 1.0 / math.sqrt(576)
    o_g, lse_g = _run_paged(p, pg, False, (-1, -1), 0.0, 2, scale)
    assert np.all(np.isfinite(o_g)) and np.all(np.isfinite(lse_g))
    import oracle

    kv = to_np(p["kv"])
    o_ref, lse_ref, _ = oracle.attention_rows(to_np(p["q"]), kv, kv[:, :, :512], p["cu_seqlens_q"].numpy(),
                                              p["cu_seqlens_k"].numpy(), scale=scale)
    compare(o_g[4:].reshape(-1, 512), lse_g[:, 4:].T.reshape(-1), o_ref[4:].reshape(-1, 512),
            lse_ref[4:].reshape(-1), "bf16", "sequence 1")


# ----------------------------------------------------- standard-head decode

# (lens_q, lens_k, hq, hkv, d, causal, window, softcap, splits)
GQA_CASES = [
    ([1, 1, 1], [1, 70, 300], 32, 4, 128, False, (-1, -1), 0.0, 0),
    ([1, 1], [2048, 129], 32, 4, 128, True, (-1, -1), 0.0, 3),
    ([2, 4], [500, 65], 16, 2, 128, True, (100, 0), 30.0, 4),
    ([1, 3], [700, 256], 8, 8, 64, False, (-1, -1), 0.0, 1),
    ([5, 1, 0], [300, 0, 10], 64, 4, 128, False, (-1, -1), 0.0, 2),
    ([1], [4096], 32, 4, 64, True, (-1, -1), 0.0, 0),
    ([3, 2], [190, 64], 12, 3, 64, False, (17, 9), 0.0, 5),
    ([1, 1, 1, 1], [64, 65, 127, 128], 8, 1, 128, True, (-1, -1), 5.0, 1),
]


def _run_gqa(p, causal, window, cap, splits, scale):
    d = dev()
    o, lse = mx.mxfa_decode_splitkv_gqa(p["q"].to(d), p["k"].to(d), p["v"].to(d), p["cu_seqlens_q"].to(d),
                                        p["cu_seqlens_k"].to(d), max(p["lens_q"]), max(p["lens_k"]),
                                        causal=causal, window=window, softcap=cap, scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("case", GQA_CASES, ids=[f"gqa{i}" for i in range(len(GQA_CASES))])
def test_gqa_decode_matches_oracle(case):
    lq, lk, hq, hkv, d, causal, window, cap, splits = case
    seed = 3500 + GQA_CASES.index(case)
    print(f"[gqa-decode] {case} seed={seed}", flush=True)
    p = workloads.make_problem(seed, dtype="bf16", heads_q=hq, heads_kv=hkv, d_qk=d, d_v=d, lens_q=lq, lens_k=lk)
    scale = 1.0 / math.sqrt(d)
    o_g, lse_g = _run_gqa(p, causal, window, cap, splits, scale)
    o_ref, lse_ref, _ = oracle_varlen(p, causal=causal, window=window, softcap=cap, scale=scale)
    compare(o_g.reshape(-1, d), lse_g.T.reshape(-1), o_ref.reshape(-1, d), lse_ref.reshape(-1), "bf16", str(case))


def test_gqa_decode_independent_of_split_count():
    p = workloads.make_problem(3600, dtype="bf16", heads_q=32, heads_kv=4, d_qk=128, d_v=128, lens_q=[1, 2, 1],
                               lens_k=[3000, 333, 64])
    scale = 1.0 / math.sqrt(128)
    ref_o, ref_l = _run_gqa(p, True, (-1, -1), 0.0, 1, scale)
    for s in (2, 3, 8, 24, 64):
        o, l = _run_gqa(p, True, (-1, -1), 0.0, s, scale)
        assert np.abs(o - ref_o).max() <= 1e-2
        assert np.abs(l - ref_l).max() <= 1e-4
    o2, l2 = _run_gqa(p, True, (-1, -1), 0.0, 8, scale)
    o3, l3 = _run_gqa(p, True, (-1, -1), 0.0, 8, scale)
    assert np.array_equal(o2, o3) and np.array_equal(l2, l3)


# --------------------------------------------------- headline workloads, full size

def _oracle_all_rows(label, dtype, o_c, lse_c, run_rows, total_tokens, heads, chunk_tokens):
    """Compare every (token, head) row of a GPU result with the oracle, a chunk of tokens at a time.

    o_c [T, H, d_v] and lse_c [T, H] are the GPU outputs (token-major); run_rows(rows) returns the
    oracle's (O, LSE) for an int array of (token, head) rows.
    """
    st = Stats(dtype, label)
    for t0 in range(0, total_tokens, chunk_tokens):
        t1 = min(total_tokens, t0 + chunk_tokens)
        tok = np.repeat(np.arange(t0, t1, dtype=np.int64), heads)
        head = np.tile(np.arange(heads, dtype=np.int64), t1 - t0)
        rows = np.stack([tok, head], axis=1)
        o_ref, lse_ref = run_rows(rows)
        st.add(o_c[t0:t1].reshape(-1, o_c.shape[-1]), lse_c[t0:t1].reshape(-1), o_ref, lse_ref)
        print(f"[full] {label}: tokens {t0}..{t1 - 1} of {total_tokens}: max|dO| so far {st.max_o:.4g}, "
              f"max|dLSE| {st.max_l:.3g}", flush=True)
    return st.check()


def _full_dense_or_varlen(name, chunk_tokens):
    """The whole workload on the GPU in the launch configuration the bench times; every row against the oracle."""
    w = workloads.get(name)
    print(f"[full] {name}: generating inputs", flush=True)
    inp = workloads.make_inputs(w)
    d = dev()
    scale = w.softmax_scale
    if w.kind == "dense":
        q, k, v = (inp[x].to(d) for x in "qkv")
        o, lse = mx.mxfa_fwd(q, k, v, causal=w.causal, window=w.window, softcap=w.softcap, scale=scale)
        torch.cuda.synchronize()
        o = o.reshape(-1, w.heads_q, w.d_v)
        lse = lse.permute(0, 2, 1).reshape(-1, w.heads_q)  # token-major
        qn = inp["q"].reshape(-1, w.heads_q, w.d_qk)
        kn = inp["k"].reshape(-1, w.heads_kv, w.d_qk)
        vn = inp["v"].reshape(-1, w.heads_kv, w.d_v)
    else:
        q, k, v = (inp[x].to(d) for x in "qkv")
        o, lse = mx.mxfa_fwd_varlen(q, k, v, inp["cu_seqlens_q"].to(d), inp["cu_seqlens_k"].to(d),
                                    max(inp["lens_q"]), max(inp["lens_k"]), causal=w.causal, window=w.window,
                                    softcap=w.softcap, scale=scale)
        torch.cuda.synchronize()
        lse = lse.T
        qn, kn, vn = inp["q"], inp["k"], inp["v"]
    import oracle

    o_c = o.float().cpu().numpy()
    lse_c = lse.cpu().numpy()
    del o, lse, q, k, v
    assert np.all(np.isfinite(lse_c)), "every row of these workloads sees at least one key"
    qn, kn, vn = to_np(qn), to_np(kn), to_np(vn)
    cq, ck = inp["cu_seqlens_q"].numpy(), inp["cu_seqlens_k"].numpy()

    def run_rows(rows):
        o_ref, lse_ref, _ = oracle.attention_rows(qn, kn, vn, cq, ck, causal=w.causal, window=w.window,
                                                  softcap=w.softcap, scale=scale, rows=rows)
        return o_ref, lse_ref

    return _oracle_all_rows(name, w.dtype, o_c, lse_c, run_rows, o_c.shape[0], w.heads_q, chunk_tokens)


def test_full_single_head_f32():
    w = workloads.get("single_head_f32")
    inp = workloads.make_inputs(w)
    q, k, v = (inp[x].to(dev()) for x in "qkv")
    o, lse = mx.mxfa_fwd(q, k, v, causal=False, scale=w.softmax_scale)
    torch.cuda.synchronize()
    import oracle

    o_ref, lse_ref, _ = oracle.attention_dense(to_np(inp["q"]), to_np(inp["k"]), to_np(inp["v"]),
                                               scale=w.softmax_scale)
    compare(o.cpu().numpy().reshape(-1, 64), lse.cpu().numpy().transpose(0, 2, 1).reshape(-1),
            o_ref.reshape(-1, 64), lse_ref.transpose(0, 2, 1).reshape(-1), "f32", "single_head_f32")


# Every row of each full-size workload is compared. The oracle takes about
# 2.5 s (causal prefill), 19 s (varlen), 75 s (window + softcap) and 40 s
# (chunked prefill) on 16 host cores.
@pytest.mark.timeout(600)
def test_full_causal_prefill_bf16():
    _full_dense_or_varlen("causal_prefill_bf16", 2048)


@pytest.mark.timeout(600)
def test_full_varlen_gqa_causal_bf16():
    _full_dense_or_varlen("varlen_gqa_causal_bf16", 4096)


@pytest.mark.timeout(900)
def test_full_window_softcap_bf16():
    _full_dense_or_varlen("window_softcap_bf16", 4096)


@pytest.mark.timeout(900)
def test_full_chunked_prefill_bf16():
    # Sq < Sk: the chunk's rows see the whole cached prefix plus their causal part.
    _full_dense_or_varlen("chunked_prefill_bf16", 512)


def test_decode_long_context():
    # 131072 keys per sequence (151 MB of latent rows each): large offsets and
    # the automatic split plan at long range, checked on sampled rows.
    lq, lk = [4, 1], [131072, 70001]
    p = workloads.make_problem(3800, dtype="bf16", heads_q=16, heads_kv=1, d_qk=576, d_v=512, lens_q=lq,
                               lens_k=lk, shared_kv=True)
    print("[decode] long context", flush=True)
    scale = 1.0 / math.sqrt(576)
    o_g, lse_g = _run_decode(p, 16, True, (-1, -1), 0.0, 0, scale)
    rows = np.array([(t, h) for t in range(5) for h in (0, 5, 15)], dtype=np.int64)
    import oracle

    kv = to_np(p["kv"])
    o_ref, lse_ref, _ = oracle.attention_rows(to_np(p["q"]), kv, kv[:, :, :512], p["cu_seqlens_q"].numpy(),
                                              p["cu_seqlens_k"].numpy(), causal=True, scale=scale, rows=rows)
    compare(o_g[rows[:, 0], rows[:, 1]], lse_g.T[rows[:, 0], rows[:, 1]], o_ref, lse_ref, "bf16", "long context")


@pytest.mark.parametrize("window,cap", [((-1, -1), 0.0), ((4096, 0), 30.0)])
def test_prefill_long_context(window, cap):
    # Chunked prefill against 131072 and 100003 keys per segment (packed, GQA):
    # large offsets, thousands of tiles per work group, checked on sampled rows
    # (first, last and tile-edge rows of each segment included).
    lq, lk = [200, 77], [131072, 100003]
    p = workloads.make_problem(3820, dtype="bf16", heads_q=8, heads_kv=2, d_qk=128, d_v=128, lens_q=lq, lens_k=lk)
    scale = 128 ** -0.5
    print(f"[prefill] long context window={window} cap={cap}", flush=True)
    o_g, lse_g = gpu_varlen(p, causal=True, window=window, softcap=cap, scale=scale)
    rows = sample_rows(lq, 8, 48, seed=3821)
    o_ref, lse_ref, _ = oracle_varlen(p, causal=True, window=window, softcap=cap, scale=scale, rows=rows)
    compare(o_g[rows[:, 0], rows[:, 1]], lse_g.T[rows[:, 0], rows[:, 1]], o_ref, lse_ref, "bf16",
            f"long context {window} {cap}")


def test_gqa_decode_long_context():
    lq, lk = [1, 2], [65536, 40000]
    p = workloads.make_problem(3810, dtype="bf16", heads_q=32, heads_kv=4, d_qk=128, d_v=128, lens_q=lq, lens_k=lk)
    print("[gqa-decode] long context", flush=True)
    scale = 1.0 / math.sqrt(128)
    o_g, lse_g = _run_gqa(p, True, (-1, -1), 0.0, 0, scale)
    rows = np.array([(t, h) for t in range(3) for h in (0, 7, 8, 31)], dtype=np.int64)
    o_ref, lse_ref, _ = oracle_varlen(p, causal=True, window=(-1, -1), softcap=0.0, scale=scale, rows=rows)
    compare(o_g[rows[:, 0], rows[:, 1]], lse_g.T[rows[:, 0], rows[:, 1]], o_ref, lse_ref, "bf16", "long context")


def test_prefill_after_kernels_that_leave_other_data_in_lds():
    # Regression: a tile is loaded into LDS by all waves of a work group, and a
    # wave's own wait covers only its part, so every read of a tile must come
    # after a barrier that follows every wave's wait. A read that came too
    # early picked up what the previous kernel on that CU left in LDS. The
    # standard-head decode leaves fp32 partials there (whose low halves are
    # arbitrary bf16 patterns, NaN included); the prefill right after it must
    # still give finite, correct rows everywhere.
    w = workloads.get("varlen_gqa_causal_bf16")
    inp = workloads.make_inputs(w)
    d = dev()
    q, k, v = (inp[x].to(d) for x in "qkv")
    cq, ck = inp["cu_seqlens_q"].to(d), inp["cu_seqlens_k"].to(d)
    gp = workloads.make_problem(3610, dtype="bf16", heads_q=32, heads_kv=4, d_qk=128, d_v=128, lens_q=[1] * 64,
                                lens_k=[1024] * 64)
    gq, gk, gv = (gp[x].to(d) for x in "qkv")
    gcq, gck = gp["cu_seqlens_q"].to(d), gp["cu_seqlens_k"].to(d)
    ref = None
    for rep in range(3):
        print(f"[lds-reuse] round {rep}", flush=True)
        mx.mxfa_decode_splitkv_gqa(gq, gk, gv, gcq, gck, 1, 1024, num_splits=8)
        o, lse = mx.mxfa_fwd_varlen(q, k, v, cq, ck, max(inp["lens_q"]), max(inp["lens_k"]), causal=True)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(lse).all()) and bool(torch.isfinite(o.float()).all())
        if ref is None:
            ref = (o.clone(), lse.clone())
        else:
            assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1])


def _nan_latent_decode(d):
    """A latent decode over an all-NaN cache, one work group per CU: it leaves NaN
    in every byte of LDS its tiles and partial-score exchange use (160 KB per CU)."""
    p = workloads.make_problem(3620, dtype="bf16", heads_q=16, heads_kv=1, d_qk=576, d_v=512, lens_q=[1] * 128,
                               lens_k=[512] * 128, shared_kv=True)
    q = p["q"].to(d)
    kv = torch.full_like(p["kv"], float("nan")).to(d)
    cq, ck = p["cu_seqlens_q"].to(d), p["cu_seqlens_k"].to(d)

    def run():
        mx.mxfa_decode_splitkv(q, kv, cq, ck, 1, 512, head_dim_v=512, num_splits=2)

    return run


def test_decodes_after_kernels_that_leave_other_data_in_lds():
    # The decode kernels also load each tile cooperatively (every wave a part),
    # so the same rule holds: a tile is read only after a barrier that follows
    # every wave's wait. Each decode runs right after a kernel that leaves NaN
    # in the LDS of every CU (a latent decode over a NaN cache, and the prefill
    # over NaN keys and values); its rows must be finite, match the oracle and
    # repeat bit for bit.
    d = dev()
    dirty_decode = _nan_latent_decode(d)
    pf = workloads.make_problem(3621, dtype="bf16", heads_q=16, heads_kv=16, d_qk=128, d_v=128, lens_q=[2048] * 4,
                                lens_k=[2048] * 4, dense=True)
    pq = pf["q"].to(d)
    pk = torch.full_like(pf["k"], float("nan")).to(d)
    pv = torch.full_like(pf["v"], float("nan")).to(d)

    def dirty_prefill():
        mx.mxfa_fwd(pq, pk, pv, causal=False)

    scale_l = 1.0 / math.sqrt(576)
    scale_g = 1.0 / math.sqrt(128)
    lat = workloads.make_problem(3622, dtype="bf16", heads_q=16, heads_kv=1, d_qk=576, d_v=512, lens_q=[4, 4, 2],
                                 lens_k=[1000, 129, 700], shared_kv=True)
    f8 = _fp8_problem(3623, [4, 3], [900, 200], 16, 1)
    pgp, pgt = _paged_problem(3624, [4, 4], [600, 333], 16, 1, 64)
    gq = workloads.make_problem(3625, dtype="bf16", heads_q=32, heads_kv=4, d_qk=128, d_v=128, lens_q=[1, 2, 1],
                                lens_k=[2000, 700, 129])
    cases = {
        "latent": lambda: _run_decode(lat, 16, True, (-1, -1), 0.0, 3, scale_l),
        "fp8": lambda: _run_fp8(f8, True, (-1, -1), 0.0, 3, scale_l),
        "paged": lambda: _run_paged(pgp, pgt, True, (-1, -1), 0.0, 3, scale_l),
        "gqa": lambda: _run_gqa(gq, True, (-1, -1), 0.0, 3, scale_g),
    }
    import oracle

    kv = to_np(lat["kv"])
    ref_lat = oracle.attention_rows(to_np(lat["q"]), kv, kv[:, :, :512], lat["cu_seqlens_q"].numpy(),
                                    lat["cu_seqlens_k"].numpy(), causal=True, scale=scale_l)[:2]
    ref_f8 = oracle.attention_rows_fp8_latent(to_np(f8["q"]), f8["kv8"].numpy(), f8["kv_scale"],
                                              f8["cu_seqlens_q"].numpy(), f8["cu_seqlens_k"].numpy(), d_v=512,
                                              causal=True, scale=scale_l)[:2]
    kvp, ckp = oracle.gather_paged(to_np(pgt["kv_cache"]), pgt["block_table"].numpy(), pgt["cache_seqlens"].numpy())
    ref_pg = oracle.attention_rows(to_np(pgp["q"]), kvp, kvp[:, :, :512], pgp["cu_seqlens_q"].numpy(), ckp,
                                   causal=True, scale=scale_l)[:2]
    ref_gq = oracle_varlen(gq, causal=True, window=(-1, -1), softcap=0.0, scale=scale_g)[:2]
    refs = {"latent": ref_lat, "fp8": ref_f8, "paged": ref_pg, "gqa": ref_gq}
    for name, run in cases.items():
        first = None
        for rep, dirty in enumerate((dirty_decode, dirty_prefill, dirty_decode)):
            print(f"[lds-reuse] {name} after {'decode' if dirty is dirty_decode else 'prefill'} (round {rep})",
                  flush=True)
            dirty()
            o, lse = run()
            assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), name
            if first is None:
                first = (o, lse)
                o_ref, lse_ref = refs[name]
                dv = o_ref.shape[-1]
                compare(o.reshape(-1, dv), lse.T.reshape(-1), o_ref.reshape(-1, dv), lse_ref.reshape(-1), "bf16",
                        name)
            else:
                assert np.array_equal(o, first[0]) and np.array_equal(lse, first[1]), name


@pytest.mark.timeout(600)
def test_full_mla_decode_bf16():
    w = workloads.get("mla_decode_bf16")
    print("[full] mla_decode_bf16: generating inputs", flush=True)
    inp = workloads.make_inputs(w)
    d = dev()
    q, kv = inp["q"].to(d), inp["kv"].to(d)
    o, lse = mx.mxfa_decode_splitkv(q, kv, inp["cu_seqlens_q"].to(d), inp["cu_seqlens_k"].to(d), w.seqlen_q,
                                    w.seqlen_k, head_dim_v=w.d_v, scale=w.softmax_scale)
    torch.cuda.synchronize()
    o_c = o.float().cpu().numpy()
    lse_c = lse.T.cpu().numpy()
    del q, kv, o, lse
    import oracle

    qn, kvn = to_np(inp["q"]), to_np(inp["kv"])
    cq, ck = inp["cu_seqlens_q"].numpy(), inp["cu_seqlens_k"].numpy()

    def run_rows(rows):
        o_ref, lse_ref, _ = oracle.attention_rows(qn, kvn, kvn[:, :, :w.d_v], cq, ck, scale=w.softmax_scale,
                                                  rows=rows)
        return o_ref, lse_ref

    # Every one of the 512 x 16 rows.
    _oracle_all_rows("mla_decode_bf16", "bf16", o_c, lse_c, run_rows, o_c.shape[0], w.heads_q, 128)


def test_full_paged_mla_decode_bf16():
    w = workloads.get("paged_mla_decode_bf16")
    print("[full] paged_mla_decode_bf16: generating inputs", flush=True)
    inp = workloads.make_inputs(w)
    d = dev()
    q = inp["q"].to(d)
    cq = inp["cu_seqlens_q"].to(d)
    cache = inp["kv_cache"].to(d)
    o, lse = mx.mxfa_decode_splitkv_paged(q, cache, cq, inp["cache_seqlens"].to(d), inp["block_table"].to(d),
                                          w.seqlen_q, w.seqlen_k, head_dim_v=w.d_v, scale=w.softmax_scale)
    torch.cuda.synchronize()
    del cache
    rows = sample_rows(inp["lens_q"], w.heads_q, 256, seed=w.seed)
    import oracle

    # The oracle reads the keys through the block table only for the sampled
    # rows' sequences: gather those, then run the rows against them.
    seqs = sorted({int(t) // w.seqlen_q for t in rows[:, 0]})
    kv_parts = []
    for b in seqs:
        kv_b, _ = oracle.gather_paged(to_np(inp["kv_cache"]), inp["block_table"][b:b + 1].numpy(),
                                      inp["cache_seqlens"][b:b + 1].numpy())
        kv_parts.append(kv_b)
    kvn = np.concatenate(kv_parts)
    q_n = to_np(inp["q"]).reshape(w.batch, w.seqlen_q, w.heads_q, w.d_qk)[seqs].reshape(-1, w.heads_q, w.d_qk)
    cu = np.arange(len(seqs) + 1, dtype=np.int32)
    slot = {b: i for i, b in enumerate(seqs)}
    local = np.stack([[slot[int(t) // w.seqlen_q] * w.seqlen_q + int(t) % w.seqlen_q, h] for t, h in rows])
    o_ref, lse_ref, _ = oracle.attention_rows(q_n, kvn, kvn[:, :, :w.d_v], cu * w.seqlen_q, cu * w.seqlen_k,
                                              scale=w.softmax_scale, rows=local)
    o_c = o.float().cpu().numpy()
    lse_c = lse.T.cpu().numpy()
    compare(o_c[rows[:, 0], rows[:, 1]], lse_c[rows[:, 0], rows[:, 1]], o_ref, lse_ref, "bf16",
            "paged_mla_decode_bf16")
    # Bit for bit the contiguous call on the packed keys (same split plan).
    o2, lse2 = mx.mxfa_decode_splitkv(q, inp["kv"].to(d), cq, inp["cu_seqlens_k"].to(d), w.seqlen_q, w.seqlen_k,
                                      head_dim_v=w.d_v, scale=w.softmax_scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_full_gqa_decode_bf16():
    w = workloads.get("gqa_decode_bf16")
    print("[full] gqa_decode_bf16: generating inputs", flush=True)
    inp = workloads.make_inputs(w)
    d = dev()
    q, k, v = (inp[x].to(d) for x in "qkv")
    o, lse = mx.mxfa_decode_splitkv_gqa(q, k, v, inp["cu_seqlens_q"].to(d), inp["cu_seqlens_k"].to(d), w.seqlen_q,
                                        w.seqlen_k, causal=w.causal, scale=w.softmax_scale)
    torch.cuda.synchronize()
    # Every row: 16 x 32 (token, head) rows of 2048 keys each.
    o_ref, lse_ref, _ = oracle_varlen(inp, causal=w.causal, window=w.window, softcap=w.softcap,
                                      scale=w.softmax_scale)
    compare(o.float().cpu().numpy().reshape(-1, w.d_v), lse.T.cpu().numpy().reshape(-1), o_ref.reshape(-1, w.d_v),
            lse_ref.reshape(-1), "bf16", "gqa_decode_bf16")


@pytest.mark.timeout(600)
def test_full_mla_decode_fp8():
    w = workloads.get("mla_decode_fp8")
    print("[full] mla_decode_fp8: generating inputs", flush=True)
    inp = workloads.make_inputs(w)
    d = dev()
    o, lse = mx.mxfa_decode_splitkv_fp8(inp["q"].to(d), inp["kv8"].to(d), inp["cu_seqlens_q"].to(d),
                                        inp["cu_seqlens_k"].to(d), w.seqlen_q, w.seqlen_k, inp["kv_scale"],
                                        head_dim_v=w.d_v, scale=w.softmax_scale)
    torch.cuda.synchronize()
    o_c = o.float().cpu().numpy()
    lse_c = lse.T.cpu().numpy()
    del o, lse
    import oracle

    qn, kv8 = to_np(inp["q"]), inp["kv8"].numpy()
    cq, ck = inp["cu_seqlens_q"].numpy(), inp["cu_seqlens_k"].numpy()

    def run_rows(rows):
        o_ref, lse_ref, _ = oracle.attention_rows_fp8_latent(qn, kv8, inp["kv_scale"], cq, ck, d_v=w.d_v,
                                                             scale=w.softmax_scale, rows=rows)
        return o_ref, lse_ref

    # Every one of the 512 x 16 rows, in one oracle call (the cache is dequantised once per call).
    _oracle_all_rows("mla_decode_fp8", "bf16", o_c, lse_c, run_rows, o_c.shape[0], w.heads_q, o_c.shape[0])


# ------------------------------------------------ offsets past 4 GiB
#
# Segments whose K/V (or latent rows, or cache pages) start more than 2^32
# bytes into their tensors: the visible keys are a small seeded problem placed
# at the end of a long, zero-filled sequence, so that the oracle runs on the
# small problem alone (with bottom-right alignment and a left window, the
# query of the long sequence sees exactly the last 256 keys in both).

def _embed_tail(small_rows, total_rows, tail_len, head_rows):
    """A [total_rows, ...] zero GPU tensor: small_rows[:tail_len] at the end of the
    first sequence (ending at head_rows), the rest right after it."""
    d = dev()
    big = torch.zeros((total_rows,) + tuple(small_rows.shape[1:]), dtype=small_rows.dtype, device=d)
    big[head_rows - tail_len:head_rows] = small_rows[:tail_len].to(d)
    big[head_rows:] = small_rows[tail_len:].to(d)
    return big


def test_prefill_offsets_past_4gib():
    long_k = 17_000_000  # 256 B of K per key: the second segment starts 4.35 GB in
    lq, lk = [1, 300], [256, 300]
    p = workloads.make_problem(3900, dtype="bf16", heads_q=2, heads_kv=1, d_qk=128, d_v=128, lens_q=lq, lens_k=lk)
    d = dev()
    print("[prefill] offsets past 4 GiB", flush=True)
    k = _embed_tail(p["k"], long_k + 300, 256, long_k)
    v = _embed_tail(p["v"], long_k + 300, 256, long_k)
    cq = p["cu_seqlens_q"].to(d)
    ck = torch.tensor([0, long_k, long_k + 300], dtype=torch.int32, device=d)
    scale = 128 ** -0.5
    o, lse = mx.mxfa_fwd_varlen(p["q"].to(d), k, v, cq, ck, 300, long_k, causal=True, window=(255, 0),
                                scale=scale)
    torch.cuda.synchronize()
    o_g, lse_g = o.float().cpu().numpy(), lse.cpu().numpy()
    del k, v, o, lse
    torch.cuda.empty_cache()
    o_ref, lse_ref, _ = oracle_varlen(p, causal=True, window=(255, 0), softcap=0.0, scale=scale)
    compare(o_g.reshape(-1, 128), lse_g.T.reshape(-1), o_ref.reshape(-1, 128), lse_ref.reshape(-1), "bf16",
            "prefill past 4 GiB")


def test_latent_decode_offsets_past_4gib():
    long_k = 3_800_000  # 1152 B per latent row: the second sequence starts 4.38 GB in
    lq, lk = [1, 4], [256, 300]
    p = workloads.make_problem(3910, dtype="bf16", heads_q=16, heads_kv=1, d_qk=576, d_v=512, lens_q=lq,
                               lens_k=lk, shared_kv=True)
    d = dev()
    print("[decode] offsets past 4 GiB", flush=True)
    scale = 1.0 / math.sqrt(576)
    kv = _embed_tail(p["kv"], long_k + 300, 256, long_k)
    cq = p["cu_seqlens_q"].to(d)
    ck = torch.tensor([0, long_k, long_k + 300], dtype=torch.int32, device=d)
    o, lse = mx.mxfa_decode_splitkv(p["q"].to(d), kv, cq, ck, 4, long_k, head_dim_v=512, causal=True,
                                    window=(255, 0), scale=scale)
    torch.cuda.synchronize()
    o_g, lse_g = o.float().cpu().numpy(), lse.cpu().numpy()
    del kv, o, lse
    torch.cuda.empty_cache()
    import oracle

    kvn = to_np(p["kv"])
    o_ref, lse_ref, _ = oracle.attention_rows(to_np(p["q"]), kvn, kvn[:, :, :512], p["cu_seqlens_q"].numpy(),
                                              p["cu_seqlens_k"].numpy(), causal=True, window=(255, 0), scale=scale)
    compare(o_g.reshape(-1, 512), lse_g.T.reshape(-1), o_ref.reshape(-1, 512), lse_ref.reshape(-1), "bf16",
            "latent decode past 4 GiB")


def test_paged_decode_pages_past_4gib():
    # 60,000 pages of 64 latent rows (73,728 B each): the visible pages of both
    # sequences lie past page 58,255, i.e. more than 2^32 bytes into the cache.
    page, num_pages, long_k = 64, 60_000, 3_800_000
    lq, lk = [1, 4], [256, 300]
    p = workloads.make_problem(3920, dtype="bf16", heads_q=16, heads_kv=1, d_qk=576, d_v=512, lens_q=lq,
                               lens_k=lk, shared_kv=True)
    d = dev()
    print("[paged] pages past 4 GiB", flush=True)
    scale = 1.0 / math.sqrt(576)
    cache = torch.zeros((num_pages, page, 1, 576), dtype=torch.bfloat16, device=d)
    max_pages = long_k // page
    table = torch.zeros((2, max_pages), dtype=torch.int32)
    # sequence 0: its last 4 logical pages hold the small problem's 256 keys
    for i in range(4):
        phys = 59_990 + i
        table[0, max_pages - 4 + i] = phys
        cache[phys] = p["kv"][i * page:(i + 1) * page].to(d)
    # sequence 1: 300 keys in 5 pages
    for i in range(5):
        phys = 59_995 + i
        table[1, i] = phys
        rows = p["kv"][256 + i * page:min(556, 256 + (i + 1) * page)]
        cache[phys, :rows.shape[0]] = rows.to(d)
    seqlens = torch.tensor([long_k, 300], dtype=torch.int32, device=d)
    o, lse = mx.mxfa_decode_splitkv_paged(p["q"].to(d), cache, p["cu_seqlens_q"].to(d), seqlens, table.to(d), 4,
                                          long_k, head_dim_v=512, causal=True, window=(255, 0), scale=scale)
    torch.cuda.synchronize()
    o_g, lse_g = o.float().cpu().numpy(), lse.cpu().numpy()
    del cache, o, lse
    torch.cuda.empty_cache()
    import oracle

    kvn = to_np(p["kv"])
    o_ref, lse_ref, _ = oracle.attention_rows(to_np(p["q"]), kvn, kvn[:, :, :512], p["cu_seqlens_q"].numpy(),
                                              p["cu_seqlens_k"].numpy(), causal=True, window=(255, 0), scale=scale)
    compare(o_g.reshape(-1, 512), lse_g.T.reshape(-1), o_ref.reshape(-1, 512), lse_ref.reshape(-1), "bf16",
            "paged decode past 4 GiB")
