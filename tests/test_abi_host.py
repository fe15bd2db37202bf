"""The C-ABI library on the host (CPU only, no GPU compute).

* libmxfa.so loads and exports every function include/mxfa.h declares;
* the Python binding's ctypes signatures match the header's prototypes;
* host-side argument checks return the documented status before anything is
  enqueued (fake device addresses are never dereferenced on these paths);
* the workspace-size query is plain arithmetic for an explicit split count.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import tiled_attention_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfa.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
A = 0x100000  # 16-byte aligned fake device address (never dereferenced here)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mx.library_path()):
        import __graft_entry__

        __graft_entry__.build()
    return mx.load_library()


def _prototypes():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    protos = {}
    for m in re.finditer(r"([A-Za-z_][\w\s\*]*?)\b(mxfa_\w+)\s*\(([^;{]*?)\)\s*;", text):
        ret, name, args = m.group(1).strip(), m.group(2), m.group(3).strip()
        if name.endswith("_t") or name == "mxfa_status":
            continue
        params = [] if args in ("void", "") else [a.strip() for a in args.split(",")]
        protos[name] = (ret, params)
    return protos


def _ctype_of(decl: str, named: bool = True):
    decl = decl.strip()
    if named:
        decl = re.sub(r"\b\w+$", "", decl).strip()
    if "*" in decl:
        return ctypes.c_char_p if decl.replace(" ", "").startswith("constchar*") else ctypes.c_void_p
    base = decl.replace("const", "").strip()
    return {"int": ctypes.c_int, "mxfa_dtype": ctypes.c_int, "mxfa_status": ctypes.c_int,
            "float": ctypes.c_float, "size_t": ctypes.c_size_t, "mxfa_stream_t": ctypes.c_void_p}[base]


def test_header_declares_the_entry_points():
    names = set(_prototypes())
    for n in ("mxfa_fwd", "mxfa_fwd_varlen", "mxfa_fwd_varlen_workspace_bytes", "mxfa_decode_splitkv", "mxfa_decode_splitkv_paged",
              "mxfa_decode_splitkv_fp8",
              "mxfa_decode_splitkv_gqa", "mxfa_decode_splitkv_gqa_workspace_bytes",
              "mxfa_decode_splitkv_gqa_num_splits",
              "mxfa_decode_splitkv_workspace_bytes",
              "mxfa_decode_splitkv_num_splits", "mxfa_last_error", "mxfa_version", "mxfa_clock_probe"):
        assert n in names, n


def test_library_exports_every_declared_symbol(lib):
    for name in _prototypes():
        assert hasattr(lib, name), f"libmxfa.so does not export {name}"


def test_binding_signatures_match_header():
    for name, (ret, params) in _prototypes().items():
        res, args = mx._SIGNATURES[name]
        assert [_ctype_of(p) for p in params] == list(args), name
        want_ret = _ctype_of(ret, named=False)
        assert res == want_ret, name


def test_version(lib):
    assert mx.mxfa_version().startswith("mxfa")


@pytest.mark.parametrize("out,us", [(None, 50), (A + 4, 50), (A, 0), (A, 1001), (A, -5)])
def test_clock_probe_host_checks(lib, out, us):
    assert lib.mxfa_clock_probe(out, us, None) == INVALID
    assert lib.mxfa_last_error().decode()


def fwd(lib, **kw):
    a = dict(q=A, k=A, v=A, o=A, lse=A, batch=1, sq=16, sk=16, hq=4, hkv=2, d=128, dtype=1, causal=1,
             wl=-1, wr=-1, softcap=0.0, scale=0.1, stream=None)
    a.update(kw)
    return lib.mxfa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["batch"], a["sq"], a["sk"], a["hq"],
                        a["hkv"], a["d"], a["dtype"], a["causal"], a["wl"], a["wr"], a["softcap"], a["scale"],
                        a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(dtype=7), UNSUPPORTED),
    (dict(hq=6, hkv=4), INVALID), (dict(hkv=0), INVALID), (dict(wl=-2), INVALID), (dict(wr=-5), INVALID),
    (dict(softcap=-1.0), INVALID), (dict(softcap=float("nan")), INVALID), (dict(softcap=float("inf")), INVALID),
    (dict(scale=float("inf")), INVALID), (dict(scale=float("nan")), INVALID), (dict(batch=-1), INVALID),
    (dict(sq=-3), INVALID), (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(k=None), INVALID),
    (dict(q=A + 2), INVALID), (dict(v=A + 8), INVALID), (dict(lse=A + 2), INVALID),
    (dict(batch=1 << 20, sq=1 << 12), INVALID), (dict(hq=16386, hkv=2), UNSUPPORTED),
    (dict(hq=32768, hkv=32768), UNSUPPORTED),
    (dict(batch=0), OK), (dict(sq=0), OK), (dict(batch=0, q=None, k=None, v=None, o=None), OK),
])
def test_fwd_host_checks(lib, kw, status):
    assert fwd(lib, **kw) == status
    if status != OK:
        assert lib.mxfa_last_error().decode()


def varlen(lib, **kw):
    a = dict(q=A, k=A, v=A, o=A, lse=A, cq=A, ck=A, batch=2, mq=16, mk=16, tq=20, tk=20, hq=4, hkv=2,
             d=64, dtype=1, causal=1, wl=-1, wr=-1, softcap=0.0, scale=0.1, ws=A, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.mxfa_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"], a["batch"], a["mq"],
                               a["mk"], a["tq"], a["tk"], a["hq"], a["hkv"], a["d"], a["dtype"], a["causal"],
                               a["wl"], a["wr"], a["softcap"], a["scale"], a["ws"], a["ws_bytes"], a["stream"])


# Every case fails on the host before anything is enqueued (the workspace
# cases because it is missing, too small or misaligned), or is an empty call.
@pytest.mark.parametrize("kw,status", [
    (dict(cq=None), INVALID), (dict(ck=A + 2), INVALID), (dict(mq=30), INVALID), (dict(tk=-1), INVALID),
    (dict(d=80), UNSUPPORTED), (dict(hq=3), INVALID), (dict(hq=32768, hkv=2), UNSUPPORTED), (dict(batch=0), OK),
    (dict(tq=0, mq=0), OK),
    (dict(ws=None, ws_bytes=1 << 20), WORKSPACE), (dict(ws_bytes=15), WORKSPACE),
    (dict(ws=A + 8, ws_bytes=1 << 20), INVALID), (dict(batch=0, ws=None), OK),
])
def test_varlen_host_checks(lib, kw, status):
    assert varlen(lib, **kw) == status
    if status != OK:
        assert lib.mxfa_last_error().decode()


@pytest.mark.parametrize("batch,mq", [(16, 3991), (1, 1), (3, 32), (3, 33), (0, 100), (5, 0)])
def test_varlen_workspace_bytes_is_arithmetic(lib, batch, mq):
    # count + 3 unused ints, batch + 1 prefix sums (padded to an even count),
    # one (segment, q tile) int pair per 32-row tile of every segment.
    want = 0 if batch == 0 or mq == 0 else 4 * (4 + ((batch + 2) & ~1)) + 8 * batch * -(-mq // 32)
    for hq, d in ((32, 128), (4, 64)):
        assert mx.mxfa_fwd_varlen_workspace_bytes(batch, mq, hq, d) == want


def decode(lib, **kw):
    a = dict(q=A, kv=A, o=A, lse=A, cq=A, ck=A, batch=2, mq=4, mk=100, tq=8, tk=200, hq=16, hkv=1, dqk=576,
             dv=512, causal=0, wl=-1, wr=-1, softcap=0.0, scale=0.04, splits=2, ws=A, ws_bytes=1 << 30,
             stream=None)
    a.update(kw)
    return lib.mxfa_decode_splitkv(a["q"], a["kv"], a["o"], a["lse"], a["cq"], a["ck"], a["batch"], a["mq"],
                                   a["mk"], a["tq"], a["tk"], a["hq"], a["hkv"], a["dqk"], a["dv"], a["causal"],
                                   a["wl"], a["wr"], a["softcap"], a["scale"], a["splits"], a["ws"],
                                   a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dqk=128, dv=128), UNSUPPORTED), (dict(dv=256), UNSUPPORTED), (dict(splits=65), INVALID),
    (dict(splits=-1), INVALID), (dict(ws=None), WORKSPACE), (dict(ws_bytes=1000), WORKSPACE),
    (dict(ws=A + 4), INVALID), (dict(kv=None), INVALID), (dict(hq=16, hkv=3), INVALID),
    (dict(hq=20000, hkv=1), UNSUPPORTED), (dict(batch=0), OK),
])
def test_decode_host_checks(lib, kw, status):
    assert decode(lib, **kw) == status


def fp8(lib, **kw):
    a = dict(q=A, kv=A, o=A, lse=A, cq=A, ck=A, batch=2, mq=4, mk=100, tq=8, tk=200, hq=16, hkv=1, dqk=576,
             dv=512, causal=0, wl=-1, wr=-1, softcap=0.0, scale=0.04, kv_scale=0.01, splits=2, ws=A,
             ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.mxfa_decode_splitkv_fp8(a["q"], a["kv"], a["o"], a["lse"], a["cq"], a["ck"], a["batch"], a["mq"],
                                       a["mk"], a["tq"], a["tk"], a["hq"], a["hkv"], a["dqk"], a["dv"], a["causal"],
                                       a["wl"], a["wr"], a["softcap"], a["scale"], a["kv_scale"], a["splits"],
                                       a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(kv_scale=float("nan")), INVALID), (dict(kv_scale=float("inf")), INVALID),
    (dict(kv_scale=3e38, scale=10.0), INVALID), (dict(dqk=128, dv=128), UNSUPPORTED), (dict(kv=None), INVALID),
    (dict(kv=A + 8), INVALID), (dict(ws=None), WORKSPACE), (dict(mk=300), INVALID), (dict(batch=0), OK),
])
def test_fp8_decode_host_checks(lib, kw, status):
    assert fp8(lib, **kw) == status
    if status != OK:
        assert lib.mxfa_last_error().decode()


def paged(lib, **kw):
    a = dict(q=A, kv=A, o=A, lse=A, cq=A, seqlens=A, table=A, batch=2, mq=4, mk=100, tq=8, pages=10, page=64,
             max_pages=2, hq=16, hkv=1, dqk=576, dv=512, causal=0, wl=-1, wr=-1, softcap=0.0, scale=0.04,
             splits=2, ws=A, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.mxfa_decode_splitkv_paged(a["q"], a["kv"], a["o"], a["lse"], a["cq"], a["seqlens"], a["table"],
                                         a["batch"], a["mq"], a["mk"], a["tq"], a["pages"], a["page"],
                                         a["max_pages"], a["hq"], a["hkv"], a["dqk"], a["dv"], a["causal"],
                                         a["wl"], a["wr"], a["softcap"], a["scale"], a["splits"], a["ws"],
                                         a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(page=48), INVALID), (dict(page=0), INVALID), (dict(page=-32), INVALID), (dict(pages=-1), INVALID),
    (dict(max_pages=-1), INVALID), (dict(max_pages=1), INVALID), (dict(mk=129), INVALID),
    (dict(pages=1 << 26, page=64), INVALID), (dict(table=None), INVALID), (dict(seqlens=None), INVALID),
    (dict(table=A + 2), INVALID), (dict(kv=None), INVALID), (dict(dqk=128, dv=128), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(splits=65), INVALID), (dict(batch=0), OK),
])
def test_paged_decode_host_checks(lib, kw, status):
    assert paged(lib, **kw) == status
    if status != OK:
        assert lib.mxfa_last_error().decode()


def gqa(lib, **kw):
    a = dict(q=A, k=A, v=A, o=A, lse=A, cq=A, ck=A, batch=2, mq=1, mk=100, tq=2, tk=200, hq=32, hkv=4, d=128,
             causal=1, wl=-1, wr=-1, softcap=0.0, scale=0.09, splits=2, ws=A, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.mxfa_decode_splitkv_gqa(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"], a["batch"],
                                       a["mq"], a["mk"], a["tq"], a["tk"], a["hq"], a["hkv"], a["d"], a["causal"],
                                       a["wl"], a["wr"], a["softcap"], a["scale"], a["splits"], a["ws"],
                                       a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(hq=30), INVALID), (dict(hkv=0), INVALID),
    (dict(wl=-2), INVALID), (dict(softcap=-1.0), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(splits=65), INVALID), (dict(splits=-1), INVALID), (dict(ws=None), WORKSPACE),
    (dict(ws_bytes=100), WORKSPACE), (dict(ws=A + 4), INVALID), (dict(k=None), INVALID),
    (dict(v=A + 2), INVALID), (dict(cq=None), INVALID), (dict(mq=3), INVALID), (dict(tk=-1), INVALID),
    (dict(hq=32768, hkv=4), UNSUPPORTED), (dict(batch=0), OK), (dict(tq=0, mq=0), OK),
])
def test_gqa_decode_host_checks(lib, kw, status):
    assert gqa(lib, **kw) == status
    if status != OK:
        assert lib.mxfa_last_error().decode()


@pytest.mark.parametrize("batch,mq,mk,hq,hkv,d,splits", [(16, 1, 2048, 32, 4, 128, 8), (3, 9, 100, 16, 2, 64, 5),
                                                        (1, 1, 64, 8, 8, 128, 1)])
def test_gqa_workspace_bytes_is_arithmetic(lib, batch, mq, mk, hq, hkv, d, splits):
    groups = -(-mq * (hq // hkv) // 32)
    # per row: d fp32 accumulators plus (max, sum of p, sum of bf16(p))
    want = batch * hkv * groups * splits * 32 * (d + 3) * 4 if splits > 1 else 0
    assert mx.mxfa_decode_splitkv_gqa_workspace_bytes(batch, mq, mk, hq, hkv, d, splits) == want
    assert mx.mxfa_decode_splitkv_gqa_num_splits(batch, mq, mk, hq, hkv, splits) == splits


@pytest.mark.parametrize("batch,mq,mk,hq,hkv,splits", [(128, 4, 8192, 16, 1, 2), (3, 9, 100, 16, 2, 5),
                                                      (1, 1, 1, 16, 1, 1)])
def test_workspace_bytes_is_arithmetic(lib, batch, mq, mk, hq, hkv, splits):
    groups = -(-mq * (hq // hkv) // 64)
    want = batch * hkv * groups * splits * 64 * (512 + 3) * 4
    assert mx.mxfa_decode_splitkv_workspace_bytes(batch, mq, mk, hq, hkv, 512, splits) == want
    assert mx.mxfa_decode_splitkv_num_splits(batch, mq, mk, hq, hkv, splits) == splits


def test_noalloc_varlen_rejects_lists_beyond_its_static_array(lib):
    # 64 segments of up to 2^21 tokens: about 2^20 query tiles, far beyond the
    # static array's 2^20 bytes. Refused on the host, before any HIP call.
    st = lib.mxfa_fwd_varlen_noalloc(A, A, A, A, A, A, A, 64, 1 << 21, 1 << 21, 1 << 27, 1 << 27, 4, 2, 128, 1, 1,
                                     -1, -1, 0.0, 0.1, None)
    assert st == WORKSPACE
    assert "allocation-free" in lib.mxfa_last_error().decode()
    # Empty calls do nothing and succeed; bad arguments are refused as by mxfa_fwd_varlen.
    assert lib.mxfa_fwd_varlen_noalloc(A, A, A, A, A, A, A, 0, 0, 0, 0, 0, 4, 2, 128, 1, 1, -1, -1, 0.0, 0.1,
                                       None) == OK
    assert lib.mxfa_fwd_varlen_noalloc(A, A, A, A, A, A, A, 2, 16, 16, 20, 20, 4, 2, 80, 1, 1, -1, -1, 0.0, 0.1,
                                       None) == UNSUPPORTED
