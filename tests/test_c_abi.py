"""The boundary from C: include/mxfa.h compiles as C11 and C++17, and a plain
C program (tests/c_abi/caller.c, HIP runtime C API only) links libmxfa.so.

* CPU: the program runs the host-side argument checks and reads the version.
* GPU: it runs the dense prefill and the latent decode on a stream of its own;
  its outputs equal the Python binding's, bit for bit, on the same inputs.
"""
from __future__ import annotations

import math
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import tiled_attention_amd as mx
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SRC = os.path.join(ROOT, "tests", "c_abi", "caller.c")


def _need_gcc():
    if shutil.which("gcc") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")):
        pytest.skip("gcc or the HIP headers are not available")


def _library():
    if not os.path.exists(mx.library_path()):
        import __graft_entry__

        __graft_entry__.build()
    return mx.library_path()


def _build_caller(tmp_path):
    _need_gcc()
    libdir = os.path.dirname(_library())
    exe = str(tmp_path / "caller")
    subprocess.run(["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROCM, "include"), "-D__HIP_PLATFORM_AMD__", SRC, "-o", exe, "-L", libdir,
                    "-lmxfa", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{libdir}",
                    f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"], check=True, capture_output=True, text=True)
    return exe


@pytest.mark.parametrize("lang", ["c", "c++"])
def test_header_compiles_alone(lang, tmp_path):
    _need_gcc()
    src = tmp_path / ("h.c" if lang == "c" else "h.cpp")
    src.write_text('#include "mxfa.h"\nint main(void) { return mxfa_last_error()[0] != 0; }\n')
    cc = "gcc" if lang == "c" else "g++"
    std = "-std=c11" if lang == "c" else "-std=c++17"
    subprocess.run([cc, std, "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-I", os.path.join(ROOT, "include"),
                    str(src)], check=True, capture_output=True, text=True)


def test_c_caller_host_checks(tmp_path):
    exe = _build_caller(tmp_path)
    r = subprocess.run([exe, "checks"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stderr)
    assert r.stdout.startswith("mxfa ")


def _save(d, name, t):
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    (d / name).write_bytes(t.numpy().tobytes())


@pytest.mark.gpu
def test_c_caller_matches_python_binding(tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mx.load_library()
    exe = _build_caller(tmp_path)
    dev = torch.device("cuda:0")

    # Dense causal prefill, GQA, ragged tiles.
    b, sq, sk, hq, hkv, d = 2, 300, 333, 4, 2, 128
    p = workloads.make_problem(7400, dtype="bf16", heads_q=hq, heads_kv=hkv, d_qk=d, d_v=d, lens_q=[sq] * b,
                               lens_k=[sk] * b, dense=True)
    fd = tmp_path / "fwd"
    fd.mkdir()
    for x in "qkv":
        _save(fd, f"{x}.bin", p[x])
    scale = d ** -0.5
    (fd / "args.txt").write_text(f"{b} {sq} {sk} {hq} {hkv} {d} 1 -1 -1 0.0 {scale!r}\n")
    print("[c-abi] fwd", flush=True)
    r = subprocess.run([exe, "fwd", str(fd)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stderr)
    o, lse = mx.mxfa_fwd(p["q"].to(dev), p["k"].to(dev), p["v"].to(dev), causal=True, scale=scale)
    torch.cuda.synchronize()
    o_c = np.frombuffer((fd / "o.bin").read_bytes(), dtype=np.int16).reshape(b, sq, hq, d)
    l_c = np.frombuffer((fd / "lse.bin").read_bytes(), dtype=np.float32).reshape(b, hq, sq)
    assert np.array_equal(o_c, o.cpu().view(torch.int16).numpy())
    assert np.array_equal(l_c, lse.cpu().numpy())

    # Latent split-KV decode.
    lq, lk, hq, hkv, splits = [4, 1, 3], [700, 64, 300], 16, 1, 3
    p = workloads.make_problem(7401, dtype="bf16", heads_q=hq, heads_kv=hkv, d_qk=576, d_v=512, lens_q=lq,
                               lens_k=lk, shared_kv=True)
    dd = tmp_path / "decode"
    dd.mkdir()
    _save(dd, "q.bin", p["q"])
    _save(dd, "kv.bin", p["kv"])
    _save(dd, "cu_q.bin", p["cu_seqlens_q"])
    _save(dd, "cu_k.bin", p["cu_seqlens_k"])
    scale = 1.0 / math.sqrt(576)
    tq, tk = sum(lq), sum(lk)
    (dd / "args.txt").write_text(f"{len(lq)} {max(lq)} {max(lk)} {tq} {tk} {hq} {hkv} 0 -1 -1 0.0 {scale!r} {splits}\n")
    print("[c-abi] decode", flush=True)
    r = subprocess.run([exe, "decode", str(dd)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stderr)
    o, lse = mx.mxfa_decode_splitkv(p["q"].to(dev), p["kv"].to(dev), p["cu_seqlens_q"].to(dev),
                                    p["cu_seqlens_k"].to(dev), max(lq), max(lk), scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    o_c = np.frombuffer((dd / "o.bin").read_bytes(), dtype=np.int16).reshape(tq, hq, 512)
    l_c = np.frombuffer((dd / "lse.bin").read_bytes(), dtype=np.float32).reshape(hq, tq)
    assert np.array_equal(o_c, o.cpu().view(torch.int16).numpy())
    assert np.array_equal(l_c, lse.cpu().numpy())


def _run_caller(exe, mode, d):
    print(f"[c-abi] {mode}", flush=True)
    r = subprocess.run([exe, mode, str(d)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (mode, r.returncode, r.stderr)
    return d


def _same(d, o, lse, o_shape, lse_shape):
    o_c = np.frombuffer((d / "o.bin").read_bytes(), dtype=np.int16).reshape(o_shape)
    l_c = np.frombuffer((d / "lse.bin").read_bytes(), dtype=np.float32).reshape(lse_shape)
    assert np.array_equal(o_c, o.cpu().view(torch.int16).numpy())
    assert np.array_equal(l_c, lse.cpu().numpy())


@pytest.mark.gpu
def test_c_caller_covers_the_other_entry_points(tmp_path):
    """Packed forward, fp8, paged and standard-head decode from C, bit for bit the binding's result."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mx.load_library()
    exe = _build_caller(tmp_path)
    dev = torch.device("cuda:0")

    # Packed forward: GQA, causal + window, an empty segment, ragged tiles.
    lq, lk, hq, hkv, d = [300, 0, 129], [333, 40, 129], 4, 2, 128
    p = workloads.make_problem(7402, dtype="bf16", heads_q=hq, heads_kv=hkv, d_qk=d, d_v=d, lens_q=lq, lens_k=lk)
    vd = tmp_path / "varlen"
    vd.mkdir()
    for x in "qkv":
        _save(vd, f"{x}.bin", p[x])
    _save(vd, "cu_q.bin", p["cu_seqlens_q"])
    _save(vd, "cu_k.bin", p["cu_seqlens_k"])
    scale = d ** -0.5
    tq, tk = sum(lq), sum(lk)
    (vd / "args.txt").write_text(f"{len(lq)} {max(lq)} {max(lk)} {tq} {tk} {hq} {hkv} {d} 1 100 0 0.0 {scale!r} 0\n")
    _run_caller(exe, "varlen", vd)
    o, lse = mx.mxfa_fwd_varlen(p["q"].to(dev), p["k"].to(dev), p["v"].to(dev), p["cu_seqlens_q"].to(dev),
                                p["cu_seqlens_k"].to(dev), max(lq), max(lk), causal=True, window=(100, 0),
                                scale=scale)
    torch.cuda.synchronize()
    _same(vd, o, lse, (tq, hq, d), (hq, tq))

    # Standard-head decode, three splits.
    lq, lk, hq, hkv, d, splits = [1, 2, 1], [700, 64, 300], 16, 2, 128, 3
    p = workloads.make_problem(7403, dtype="bf16", heads_q=hq, heads_kv=hkv, d_qk=d, d_v=d, lens_q=lq, lens_k=lk)
    gd = tmp_path / "gqa"
    gd.mkdir()
    for x in "qkv":
        _save(gd, f"{x}.bin", p[x])
    _save(gd, "cu_q.bin", p["cu_seqlens_q"])
    _save(gd, "cu_k.bin", p["cu_seqlens_k"])
    scale = d ** -0.5
    tq, tk = sum(lq), sum(lk)
    (gd / "args.txt").write_text(f"{len(lq)} {max(lq)} {max(lk)} {tq} {tk} {hq} {hkv} {d} 1 -1 -1 0.0 {scale!r} "
                                 f"{splits}\n")
    _run_caller(exe, "gqa", gd)
    o, lse = mx.mxfa_decode_splitkv_gqa(p["q"].to(dev), p["k"].to(dev), p["v"].to(dev), p["cu_seqlens_q"].to(dev),
                                        p["cu_seqlens_k"].to(dev), max(lq), max(lk), causal=True, scale=scale,
                                        num_splits=splits)
    torch.cuda.synchronize()
    _same(gd, o, lse, (tq, hq, d), (hq, tq))

    # Latent decode over an fp8 cache, two splits.
    lq, lk, hq, hkv, splits = [4, 1], [500, 77], 16, 1, 2
    p = workloads.make_problem(7404, dtype="bf16", heads_q=hq, heads_kv=hkv, d_qk=576, d_v=512, lens_q=lq,
                               lens_k=lk, shared_kv=True)
    p.update(workloads.quantize_e4m3(p["kv"].float()))
    fd = tmp_path / "fp8"
    fd.mkdir()
    _save(fd, "q.bin", p["q"])
    _save(fd, "kv.bin", p["kv8"].view(torch.uint8))
    _save(fd, "cu_q.bin", p["cu_seqlens_q"])
    _save(fd, "cu_k.bin", p["cu_seqlens_k"])
    scale = 1.0 / math.sqrt(576)
    tq, tk = sum(lq), sum(lk)
    kv_scale = float(p["kv_scale"])
    (fd / "args.txt").write_text(f"{len(lq)} {max(lq)} {max(lk)} {tq} {tk} {hq} {hkv} 0 -1 -1 0.0 {scale!r} "
                                 f"{splits} {kv_scale!r}\n")
    _run_caller(exe, "fp8", fd)
    o, lse = mx.mxfa_decode_splitkv_fp8(p["q"].to(dev), p["kv8"].to(dev), p["cu_seqlens_q"].to(dev),
                                        p["cu_seqlens_k"].to(dev), max(lq), max(lk), kv_scale, scale=scale,
                                        num_splits=splits)
    torch.cuda.synchronize()
    _same(fd, o, lse, (tq, hq, 512), (hq, tq))

    # Latent decode over a paged cache (64-row pages at shuffled indices).
    lq, lk, hq, hkv, splits, page = [4, 2], [300, 130], 16, 1, 2, 64
    p = workloads.make_problem(7405, dtype="bf16", heads_q=hq, heads_kv=hkv, d_qk=576, d_v=512, lens_q=lq,
                               lens_k=lk, shared_kv=True)
    pg = workloads.paginate(p["kv"], lk, page, torch.Generator("cpu").manual_seed(7406))
    pd = tmp_path / "paged"
    pd.mkdir()
    _save(pd, "q.bin", p["q"])
    _save(pd, "kv.bin", pg["kv_cache"])
    _save(pd, "cu_q.bin", p["cu_seqlens_q"])
    _save(pd, "seqlens.bin", pg["cache_seqlens"])
    _save(pd, "table.bin", pg["block_table"])
    tq = sum(lq)
    num_pages, max_pages = pg["kv_cache"].shape[0], pg["block_table"].shape[1]
    (pd / "args.txt").write_text(f"{len(lq)} {max(lq)} {max(lk)} {tq} {num_pages} {page} {max_pages} {hq} {hkv} "
                                 f"0 -1 -1 0.0 {scale!r} {splits}\n")
    _run_caller(exe, "paged", pd)
    o, lse = mx.mxfa_decode_splitkv_paged(p["q"].to(dev), pg["kv_cache"].to(dev), p["cu_seqlens_q"].to(dev),
                                          pg["cache_seqlens"].to(dev), pg["block_table"].to(dev), max(lq), max(lk),
                                          scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    _same(pd, o, lse, (tq, hq, 512), (hq, tq))
