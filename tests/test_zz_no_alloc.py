"""The allocation-free packed forward (mxfa_fwd_varlen_noalloc), through the C ABI, against
mxfa_fwd_varlen with a caller workspace: the two run the same kernels, so the results must be
identical bit for bit -- on two calls in a row, the second smaller than the first (the static
scratch array keeps the first call's list, which the second must not depend on)."""
from __future__ import annotations

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("tiled_attention_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mx.load_library()


# (dtype, d, lens_q, lens_k, hq, hkv, causal, window, softcap)
CALLS = [
    ("bf16", 128, [300, 0, 1, 777, 129, 4000], [333, 40, 1, 777, 129, 4100], 8, 2, True, (200, 0), 0.0),
    ("bf16", 128, [65, 3], [65, 90], 8, 2, True, (200, 0), 0.0),
    ("f32", 64, [130, 31, 0, 64], [130, 40, 5, 64], 4, 4, False, (-1, -1), 20.0),
    ("f32", 64, [7], [9], 4, 4, False, (-1, -1), 20.0),
]


def test_noalloc_matches_workspace_call_twice_in_a_row():
    d_ = torch.device("cuda:0")
    for i, (dtype, d, lq, lk, hq, hkv, causal, window, cap) in enumerate(CALLS):
        print(f"[noalloc] call {i}: {dtype} d={d} lens_q={lq}", flush=True)
        p = workloads.make_problem(5100 + i, dtype=dtype, heads_q=hq, heads_kv=hkv, d_qk=d, d_v=d, lens_q=lq,
                                   lens_k=lk)
        q, k, v = p["q"].to(d_), p["k"].to(d_), p["v"].to(d_)
        cq, ck = p["cu_seqlens_q"].to(d_), p["cu_seqlens_k"].to(d_)
        o_ref, l_ref = mx.mxfa_fwd_varlen(q, k, v, cq, ck, max(lq), max(lk), causal=causal, window=window,
                                          softcap=cap)
        out = torch.full_like(q, float("nan"))
        lse = torch.full((hq, q.shape[0]), float("nan"), dtype=torch.float32, device=d_)
        o, l = mx.mxfa_fwd_varlen_noalloc(q, k, v, cq, ck, max(lq), max(lk), causal=causal, window=window,
                                          softcap=cap, out=out, lse=lse)
        torch.cuda.synchronize()
        assert o.data_ptr() == out.data_ptr() and l.data_ptr() == lse.data_ptr()
        assert torch.equal(o.view(torch.int16) if dtype == "bf16" else o, o_ref.view(torch.int16)
                           if dtype == "bf16" else o_ref), f"call {i}: O differs"
        assert torch.equal(l, l_ref), f"call {i}: LSE differs"
