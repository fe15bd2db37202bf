"""Host-side logic of bench.py, on the CPU: the work counts behind the reported
rates, the single-GPU guard, the PMC traffic summary and its source tagging."""
from __future__ import annotations

import csv
import json
import os
import shutil
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _pairs_by_loops(lens_q, lens_k, causal, window):
    wl, wr = window
    n = 0
    for sq, sk in zip(lens_q, lens_k):
        for i in range(sq):
            row = i + sk - sq  # query i sits at key position row (bottom-right alignment)
            for j in range(sk):
                if causal and j > row:
                    continue
                if wl >= 0 and j < row - wl:
                    continue
                if wr >= 0 and j > row + wr:
                    continue
                n += 1
    return n


@pytest.mark.parametrize("causal,window", [(False, (-1, -1)), (True, (-1, -1)), (False, (5, 2)), (True, (7, 0)),
                                           (True, (0, 0)), (False, (0, -1)), (False, (-1, 0))])
def test_visible_pairs_counts_every_unmasked_pair(causal, window):
    lens_q = [1, 17, 40, 0, 33, 5]
    lens_k = [1, 17, 29, 9, 64, 0]
    assert bench.visible_pairs(lens_q, lens_k, causal, window) == _pairs_by_loops(lens_q, lens_k, causal, window)


def test_visible_pairs_closed_forms():
    # full square causal: n(n+1)/2 per sequence; non-causal: sq*sk
    assert bench.visible_pairs([2048] * 4, [2048] * 4, True, (-1, -1)) == 4 * 2048 * 2049 // 2
    assert bench.visible_pairs([4] * 3, [8192] * 3, False, (-1, -1)) == 3 * 4 * 8192


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_code_only_drops_comments_and_whitespace_keeps_literals():
    src = 'int a = 1; // note\n/* block\n comment */ const char* s = "x // y /* z */";\nchar q = \'"\';\n'
    assert bench._code_only(src) == 'inta=1;constchar*s="x // y /* z */";charq=\'"\';'
    assert bench._code_only("a /* unterminated") == "a"


def _copy_sources(dst):
    for rel in set(bench.KERNEL_SOURCES.values()) | set(bench.SHARED_SOURCES):
        os.makedirs(os.path.join(dst, os.path.dirname(rel)), exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), os.path.join(dst, rel))
    os.makedirs(os.path.join(dst, "profiles"), exist_ok=True)


def test_source_hash_follows_code_not_comments(tmp_path, monkeypatch):
    _copy_sources(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    before = bench.source_sha("decode_mla")
    path = tmp_path / bench.KERNEL_SOURCES["decode_mla"]
    text = path.read_text()
    path.write_text("// a new comment line\n" + text.replace("\n", "  \n", 3))
    assert bench.source_sha("decode_mla") == before
    path.write_text(text + "\nstatic int extra_symbol;\n")
    assert bench.source_sha("decode_mla") != before
    assert bench.source_sha("fwd_bf16") != bench.source_sha("decode_mla")


def _write_pmc_csv(path, counter, readings):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, vals in readings.items():
            for v in vals:
                w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_pmc_summary_scales_by_the_copy_and_tags_the_source(tmp_path, monkeypatch, capsys):
    _copy_sources(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    copy_mb = 64
    # The copy reads 64 MiB but FETCH_SIZE shows half of it; WRITE_SIZE shows all of it.
    fetch = {"void fwd_bf16_kernel<128, 0>(Args)": [1000.0, 1002.0],
             "__amd_rocclr_copyBuffer": [16.0, copy_mb * 1024 / 2],
             "void decode_gqa_split_kernel<128, false>(P)": [300.0],
             "void decode_gqa_combine_kernel<128>(P)": [10.0]}
    write = {"void fwd_bf16_kernel<128, 0>(Args)": [500.0, 500.0],
             "__amd_rocclr_copyBuffer": [copy_mb * 1024.0],
             "void decode_gqa_split_kernel<128, false>(P)": [20.0],
             "void decode_gqa_combine_kernel<128>(P)": [2.0]}
    _write_pmc_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _write_pmc_csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    bench.pmc_summarize(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), copy_mb)
    capsys.readouterr()
    out = json.loads((tmp_path / "profiles" / "pmc_traffic.json").read_text())
    assert out["_calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert out["_calibration"]["write_scale"] == pytest.approx(1.0)
    assert out["fwd_bf16"]["fetch_bytes"] == round(1001.0 * 1024 * 2)
    assert out["fwd_bf16"]["write_bytes"] == round(500.0 * 1024)
    assert out["decode_gqa"]["bytes_per_launch"] == round((300.0 + 10.0) * 2048 + (20.0 + 2.0) * 1024)
    assert "decode_mla" not in out  # no readings for its kernels in these files
    assert bench.load_traffic("fwd_bf16") == out["fwd_bf16"]["bytes_per_launch"]
    assert bench.load_traffic("decode_mla") is None
    src = tmp_path / bench.KERNEL_SOURCES["fwd_bf16"]
    src.write_text(src.read_text() + "\nstatic int extra_symbol;\n")
    assert bench.load_traffic("fwd_bf16") is None  # stale once the kernel's code changes


def test_committed_traffic_figures_are_tagged_with_a_known_family():
    with open(os.path.join(ROOT, "profiles", "pmc_traffic.json")) as f:
        rec = json.load(f)
    fams = [k for k in rec if not k.startswith("_")]
    assert fams and set(fams) <= set(bench.PMC_KERNELS)
    for k in fams:
        assert abs(rec[k]["bytes_per_launch"] - rec[k]["fetch_bytes"] - rec[k]["write_bytes"]) <= 1


def test_trace_summary_cuts_workloads_at_their_clock_probes(tmp_path, capsys):
    # Two workloads of the bench: A's 5 + 3 + 3 calls around its 2 probes, then
    # B, whose first kernel A never launched. A torch fill is left out.
    cols = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Workgroup_Size_X"]
    rows, t = [], 0

    def add(name, dur_ns, grid=256 * 4):
        nonlocal t
        rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur_ns,
                     "Grid_Size_X": grid, "Workgroup_Size_X": 256})
        t += dur_ns + 100

    A = "void mxfa::(anonymous namespace)::fwd_bf16_kernel<128, 0>(mxfa::FwdParams)"
    P = "mxfa::(anonymous namespace)::clock_probe_kernel(unsigned long long*, unsigned int)"
    B = "void mxfa::(anonymous namespace)::decode_split_kernel<false, false, false>(mxfa::DecodeParams)"
    for _ in range(5):
        add(A, 90_000)
    for _ in range(2):
        for _ in range(3):
            add(A, 80_000)
        add(P, 1_000_000, grid=64)
    add("void at::native::vectorized_elementwise_kernel<4>(int)", 2_000)
    for d in (70_000, 71_000, 72_000):
        add(A, d)
    for _ in range(4):
        add(B, 200_000)
    path = tmp_path / "trace.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        w.writerows(rows)
    bench.trace_summarize(str(path), ["wa", "wb"], tail=3, probes=2)
    out = capsys.readouterr().out.splitlines()
    body = [l for l in out[2:] if l.startswith("|")]
    assert len(body) == 2
    assert body[0].startswith("| wa | `fwd_bf16_kernel<128, 0>` | 4 | 14 |")
    assert "| 71.0 | 70.0 | 72.0 |" in body[0]  # median / min / max of the last three calls, us
    assert body[1].startswith("| wb | `decode_split_kernel<false, false, false>` | 4 | 4 |")
