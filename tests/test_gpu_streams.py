"""Stream semantics of the C ABI.

Every call is enqueued on the caller's stream, allocates nothing and never
synchronises. Two checks show it: the calls give bit-identical results on a
side stream, and they can be captured into a HIP graph whose replays (with
eager work and synchronisations between them, and after the captured inputs
are overwritten in place) match eager calls bit for bit.
"""
from __future__ import annotations

import math

import pytest
import torch

import workloads
from tests.gpu_helpers import dev

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("tiled_attention_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mx.load_library()


class Calls:
    """Inputs, outputs and workspaces of one prefill, one latent decode and one
    standard-head decode, all preallocated on the GPU."""

    def __init__(self, seed):
        d = dev()
        pre = workloads.make_problem(seed, dtype="bf16", heads_q=4, heads_kv=2, d_qk=128, d_v=128,
                                     lens_q=[300] * 2, lens_k=[300] * 2, dense=True)
        lat = workloads.make_problem(seed + 1, dtype="bf16", heads_q=16, heads_kv=1, d_qk=576, d_v=512,
                                     lens_q=[4, 2], lens_k=[700, 300], shared_kv=True)
        gqa = workloads.make_problem(seed + 2, dtype="bf16", heads_q=32, heads_kv=4, d_qk=128, d_v=128,
                                     lens_q=[1, 1, 1], lens_k=[2000, 64, 513])
        self.q, self.k, self.v = (pre[x].to(d) for x in "qkv")
        self.lq, self.lkv = lat["q"].to(d), lat["kv"].to(d)
        self.lcq, self.lck = lat["cu_seqlens_q"].to(d), lat["cu_seqlens_k"].to(d)
        self.gq, self.gk, self.gv = gqa["q"].to(d), gqa["k"].to(d), gqa["v"].to(d)
        self.gcq, self.gck = gqa["cu_seqlens_q"].to(d), gqa["cu_seqlens_k"].to(d)
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((2, 4, 300), dtype=torch.float32, device=d)
        self.lo = torch.empty((6, 16, 512), dtype=torch.bfloat16, device=d)
        self.llse = torch.empty((16, 6), dtype=torch.float32, device=d)
        nb = mx.mxfa_decode_splitkv_workspace_bytes(2, 4, 700, 16, 1, 512, 3)
        self.lws = torch.empty(max(nb, 16), dtype=torch.uint8, device=d)
        self.go = torch.empty_like(self.gq)
        self.glse = torch.empty((32, 3), dtype=torch.float32, device=d)
        nb = mx.mxfa_decode_splitkv_gqa_workspace_bytes(3, 1, 2000, 32, 4, 128, 4)
        self.gws = torch.empty(max(nb, 16), dtype=torch.uint8, device=d)

    def run(self):
        mx.mxfa_fwd(self.q, self.k, self.v, causal=True, scale=128 ** -0.5, out=self.o, lse=self.lse)
        mx.mxfa_decode_splitkv(self.lq, self.lkv, self.lcq, self.lck, 4, 700, scale=1.0 / math.sqrt(576),
                               num_splits=3, workspace=self.lws, out=self.lo, lse=self.llse)
        mx.mxfa_decode_splitkv_gqa(self.gq, self.gk, self.gv, self.gcq, self.gck, 1, 2000, causal=True,
                                   scale=128 ** -0.5, num_splits=4, workspace=self.gws, out=self.go,
                                   lse=self.glse)

    def outputs(self):
        return [t.clone() for t in (self.o, self.lse, self.lo, self.llse, self.go, self.glse)]


def _assert_same(a, b, what):
    for i, (x, y) in enumerate(zip(a, b)):
        assert torch.equal(x, y), f"{what}: output {i} differs"


def test_side_stream_matches_default_stream():
    c = Calls(7100)
    c.run()
    torch.cuda.synchronize()
    ref = c.outputs()
    for t in (c.o, c.lse, c.lo, c.llse, c.go, c.glse):
        t.fill_(float("nan"))
    s = torch.cuda.Stream()  # default priority
    s.wait_stream(torch.cuda.current_stream())
    print("[streams] side stream", flush=True)
    with torch.cuda.stream(s):
        c.run()
    s.synchronize()
    _assert_same(c.outputs(), ref, "side stream")


def test_graph_capture_replays_match_eager():
    c = Calls(7200)
    c.run()
    torch.cuda.synchronize()
    ref = c.outputs()
    g = torch.cuda.CUDAGraph()
    print("[streams] capture", flush=True)
    with torch.cuda.graph(g):
        c.run()
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device=dev())
    for r in range(3):
        for t in (c.o, c.lse, c.lo, c.llse, c.go, c.glse):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        print(f"[streams] replay {r}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        _assert_same(c.outputs(), ref, f"replay {r}")
        scratch.mul_(1.5).add_(1.0)  # eager work between replays
        torch.cuda.synchronize()
    # The graph reads its inputs through their addresses at replay time.
    c2 = Calls(7300)
    c2.run()
    torch.cuda.synchronize()
    ref2 = c2.outputs()
    for a, b in ((c.q, c2.q), (c.k, c2.k), (c.v, c2.v), (c.lq, c2.lq), (c.lkv, c2.lkv), (c.gq, c2.gq),
                 (c.gk, c2.gk), (c.gv, c2.gv)):
        a.copy_(b)
    torch.cuda.synchronize()
    print("[streams] replay on new inputs", flush=True)
    g.replay()
    torch.cuda.synchronize()
    _assert_same(c.outputs(), ref2, "replay on new inputs")
