"""Host logic of bench.py on the CPU: the work and byte counts its metrics
divide by, the block-sparse pair counts, the rocprofv3 counter scaling, the
guard that drops traffic figures taken on other kernel sources, and the
refusal of a multi-GPU run.  Counts are pinned to brute force over the mask
definition and to sizes worked out by hand."""

import json
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import bench
from attn_workloads import DECODE_WORKLOADS, HEADLINE, WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SHAPES = [(1, 1), (7, 7), (5, 9), (9, 5), (16, 3), (3, 16), (130, 70)]
WINDOWS = [(-1, -1), (0, 0), (2, -1), (-1, 1), (3, 2), (0, -1), (40, 5)]


def brute_pairs(Nq, Nk, causal, left, right):
    """Kept (query, key) pairs, one pair at a time: key j is kept for row i
    iff its distance i + (Nk - Nq) - j is >= 0 (causal), <= left and
    >= -right (when those are >= 0)."""
    n = 0
    for i in range(Nq):
        for j in range(Nk):
            dist = i + (Nk - Nq) - j
            if causal and dist < 0:
                continue
            if left >= 0 and dist > left:
                continue
            if right >= 0 and -dist > right:
                continue
            n += 1
    return n


@pytest.mark.parametrize("Nq,Nk", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_visible_pairs_against_brute_force(Nq, Nk, causal):
    for left, right in WINDOWS:
        assert bench.visible_pairs(Nq, Nk, causal, left, right) == brute_pairs(Nq, Nk, causal, left, right), (
            Nq, Nk, causal, left, right)


def test_flop_counts_of_the_headline():
    w = WORKLOADS[HEADLINE]  # B 4, H 16, N 4096, d 128, non-causal
    assert bench.flops(w) == 4 * 4 * 16 * 4096 * 4096 * 128 == 549_755_813_888
    assert bench.bwd_flops(w) == 2.5 * 549_755_813_888
    # with no window every pair is kept: the variant count is the plain one
    assert bench.variant_flops(w, -1, -1) == bench.flops(w)


def test_causal_flops_halve_and_kept_pairs_count_the_diagonal():
    w = WORKLOADS["causal_mha_b2_h32_n8192_d128_bf16"]
    full = 4.0 * w.B * w.Hq * w.Nq * w.Nk * w.d
    assert bench.flops(w) == full / 2
    # the kept-pair count includes the diagonal: N (N + 1) / 2 pairs per head
    N = w.Nq
    assert bench.variant_flops(w, -1, -1) == 4.0 * w.B * w.Hq * w.d * N * (N + 1) // 2


@pytest.mark.parametrize("Nq,Nk", [(7, 7), (130, 70), (300, 300), (257, 513), (513, 257)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [4, 128])
def test_blocksparse_pair_counts_against_brute_force(Nq, Nk, causal, block):
    counts = bench.blocksparse_pair_counts(Nq, Nk, causal, block)
    nqb, nkb = -(-Nq // block), -(-Nk // block)
    assert counts.shape == (nqb, nkb)
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    keep = np.ones((Nq, Nk), dtype=bool) if not causal else (j <= i + (Nk - Nq))
    for qb in range(nqb):
        for kb in range(nkb):
            want = keep[qb * block:(qb + 1) * block, kb * block:(kb + 1) * block].sum()
            assert counts[qb, kb] == want, (qb, kb)
    assert counts.sum() == bench.visible_pairs(Nq, Nk, causal, -1, -1)


def test_algorithmic_bytes_by_hand():
    w = WORKLOADS[HEADLINE]
    tensor = 4 * 4096 * 16 * 128 * 2  # one [B, N, H, d] bf16 tensor: 64 MiB
    vec = 4 * 16 * 4096 * 4          # one [B, H, N] fp32 vector: 1 MiB
    assert tensor == 67_108_864 and vec == 1_048_576
    # forward: q, k, v read, out written, lse written
    assert bench.algorithmic_bytes(w) == 4 * tensor + vec == 269_484_032
    # backward: q, k, v, out, dout read, dq, dk, dv written, lse read, delta written
    assert bench.bwd_algorithmic_bytes(w) == 8 * tensor + 2 * vec == 538_968_064


def test_decode_bytes_by_hand():
    w = DECODE_WORKLOADS["decode_b1_hq32_hkv8_cache131072_d128_bf16"]
    cache = 131072 * 8 * 128 * 2 * 2   # K and V caches read once
    q_out = 1 * 32 * 128 * 2 * 2       # one query row per head read, out written
    lse = 32 * 4
    new_rows = 8 * 128 * 2 * 4         # one new K and V row per KV head, read and appended
    assert bench.decode_bytes(w) == cache + q_out + lse + new_rows == 536_895_616


def _write_counter_csv(path, counter, rows):
    with open(path, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for name, value in rows:
            f.write(f"\"{name}\",{counter},{value}\n")


def test_traffic_summary_scales_counters_by_the_copy(tmp_path, monkeypatch):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the forward kernel,
    averaged over its dispatches and scaled by copy bytes / copy counter."""
    out = tmp_path / "attn_fwd_traffic.json"
    monkeypatch.setitem(bench.TRAFFIC_FILES, "fwd", str(out))
    kern = "void eta::attn_fwd_kernel<128, true, false, false, false, false>(...)"
    copy = "void at::native::neg_kernel(...)"
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # a 1 MiB copy reads as 512 KiB of FETCH_SIZE (factor 2) and 1024 KiB of WRITE_SIZE (factor 1)
    _write_counter_csv(fetch, "FETCH_SIZE", [(kern, 100.0), (kern, 140.0), (copy, 512.0)])
    _write_counter_csv(write, "WRITE_SIZE", [(kern, 30.0), (copy, 1024.0)])
    bench.write_traffic_summary(str(fetch), str(write), 1, workload=HEADLINE, op="fwd")
    rec = json.loads(out.read_text())
    assert rec["kernel_source_hash"] == bench.kernel_source_hash("fwd")
    r = rec["workloads"][HEADLINE]
    assert r["FETCH_SIZE_copy_scale"] == 2.0 and r["WRITE_SIZE_copy_scale"] == 1.0
    assert r["bytes_read_per_launch"] == 120.0 * 1024 * 2.0
    assert r["bytes_written_per_launch"] == 30.0 * 1024
    assert r["hbm_bytes_per_launch"] == 120.0 * 1024 * 2.0 + 30.0 * 1024
    assert r["algorithmic_bytes"] == 269_484_032
    # the guard: figures apply only to the sources they were taken on
    assert bench.measured_traffic(HEADLINE, "fwd") == r["hbm_bytes_per_launch"]
    rec["kernel_source_hash"] = "0" * 16
    out.write_text(json.dumps(rec))
    assert bench.measured_traffic(HEADLINE, "fwd") is None


def test_traffic_summary_needs_the_kernel_and_the_copy(tmp_path, monkeypatch):
    monkeypatch.setitem(bench.TRAFFIC_FILES, "fwd", str(tmp_path / "t.json"))
    kern = "void eta::attn_fwd_kernel<128, true, false, false, false, false>(...)"
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _write_counter_csv(fetch, "FETCH_SIZE", [(kern, 100.0)])  # no copy dispatch
    _write_counter_csv(write, "WRITE_SIZE", [(kern, 30.0), ("neg_kernel", 1024.0)])
    with pytest.raises(SystemExit, match="no copy dispatch"):
        bench.write_traffic_summary(str(fetch), str(write), 1, workload=HEADLINE, op="fwd")
    _write_counter_csv(fetch, "FETCH_SIZE", [("neg_kernel", 512.0)])  # no kernel dispatch
    with pytest.raises(SystemExit, match="no forward kernel dispatches"):
        bench.write_traffic_summary(str(fetch), str(write), 1, workload=HEADLINE, op="fwd")
    # the d = 256 workloads run the 16x16x32 kernel
    k256 = "void eta::attn_fwd_k16_kernel<256, false, true, false, false, false, false>(...)"
    _write_counter_csv(fetch, "FETCH_SIZE", [(k256, 200.0), ("neg_kernel", 512.0)])
    _write_counter_csv(write, "WRITE_SIZE", [(k256, 30.0), ("neg_kernel", 1024.0)])
    bench.write_traffic_summary(str(fetch), str(write), 1, workload=HEADLINE, op="fwd")
    rec = json.load(open(tmp_path / "t.json"))["workloads"][HEADLINE]
    assert rec["FETCH_SIZE_KiB_per_launch"] == 200.0
    # the plain d = 128 workloads run the 16x16x32 kernel
    k16 = "void eta::attn_fwd_k16_kernel<128, true, false>(...)"
    _write_counter_csv(fetch, "FETCH_SIZE", [(k16, 300.0), ("neg_kernel", 512.0)])
    _write_counter_csv(write, "WRITE_SIZE", [(k16, 30.0), ("neg_kernel", 1024.0)])
    bench.write_traffic_summary(str(fetch), str(write), 1, workload=HEADLINE, op="fwd")
    rec = json.load(open(tmp_path / "t.json"))["workloads"][HEADLINE]
    assert rec["FETCH_SIZE_KiB_per_launch"] == 300.0


def test_kernel_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    csrc = tmp_path / "csrc"
    shutil.copytree(bench._CSRC, csrc)
    monkeypatch.setattr(bench, "_CSRC", str(csrc))
    base = {op: bench.kernel_source_hash(op) for op in bench.OP_SOURCES}
    f = csrc / "attn_fwd_kernel.hpp"
    text = f.read_text()
    f.write_text("// a new comment line\n/* and a block\n   comment */\n" + text.replace("\n", "\n  ", 3))
    assert bench.kernel_source_hash("fwd") == base["fwd"]
    f.write_text(text.replace("kLeanTiles = true", "kLeanTiles = false", 1))
    assert bench.kernel_source_hash("fwd") != base["fwd"]
    # the backward and decode sources do not include the forward kernel
    assert bench.kernel_source_hash("bwd") == base["bwd"]
    assert bench.kernel_source_hash("decode") == base["decode"]


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_launch_stats_median_min_max(capsys):
    st = bench.launch_stats([0.5, 0.7, 0.4, 0.6])  # milliseconds
    assert st == {"median_us": 550.0, "min_us": 400.0, "max_us": 700.0}
    assert bench.launch_stats([0.3, 0.1, 0.2])["median_us"] == 200.0
    # every launch, in launch order, goes to stderr
    assert "500.0 700.0 400.0 600.0" in capsys.readouterr().err


def test_clock_summary_keeps_one_sample_per_refresh_under_load():
    # the table refreshes about once per second: repeated reads of one refresh
    # count once, the pre-load refresh and the first 0.5 s are left out
    S = [
        {"t": 0.9, "acc": 100, "clk": 150.0, "clk_min": 140.0, "power": 250},    # before the load
        {"t": 1.2, "acc": 100, "clk": 150.0, "clk_min": 140.0, "power": 250},    # stale
        {"t": 1.3, "acc": 101, "clk": 1900.0, "clk_min": 1800.0, "power": 900},  # < 0.5 s in
        {"t": 1.7, "acc": 102, "clk": 1700.0, "clk_min": 1600.0, "power": 1300},
        {"t": 1.8, "acc": 102, "clk": 1700.0, "clk_min": 1600.0, "power": 1300},  # same refresh
        {"t": 2.7, "acc": 103, "clk": 1660.0, "clk_min": 1550.0, "power": 1350},
    ]
    c = bench.clock_summary(S, t0=1.0, achieved=1000.0, peak=2500.0)
    assert c["refreshes_under_load"] == 2
    assert c["gfxclk_mhz_mean_over_xcds"] == 1680.0 and c["gfxclk_mhz_slowest_xcd"] == 1550.0
    assert c["socket_power_w"] == 1325.0
    assert c["frac_of_peak_at_this_clock"] == round(1000.0 / (2500.0 * 1680.0 / 2400.0), 4)
    # a timed region too short for any refresh: reported, not invented
    assert "error" in bench.clock_summary(S[:3], t0=1.0, achieved=1000.0, peak=2500.0)


def test_host_info_names_cores_and_versions():
    info = bench.host_info("fwd")
    assert info["cores"] == len(os.sched_getaffinity(0))
    assert info["kernel_source_hash"] == bench.kernel_source_hash("fwd")
    assert "torch" in info and "rocm" in info


def test_host_info_names_the_build_on_a_tree_without_git(monkeypatch):
    # The library's build records the revision it was built from; a copy of
    # the tree without .git (git fails) reports that one, marked as such.
    from exact_tiled_attention_35_amd import build as b

    b.write_build_info()
    with open(b.BUILD_INFO) as f:
        built = json.load(f)["git_rev"]

    def no_git(*args, **kwargs):
        raise OSError("no git here")

    monkeypatch.setattr(subprocess, "run", no_git)
    info = bench.host_info("fwd")
    assert info["git_rev"] == (f"{built} (at build)" if built else None)
