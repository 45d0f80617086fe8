#!/usr/bin/env python3
"""Throughput of the exact attention forward on one MI355X.

One step = one ``attn_fwd`` call over the whole workload (all query blocks
of every (batch, head)), with q, k, v already resident in device memory.
Default workload: B=4, H=16, N=4096, d=128, bf16, non-causal -- the hidden
2048 / batch 16k/seq setup of the README benchmark described on the
hysenlabs.com page (section "Leistungs- und Speicherangaben im README").

Prints ONE JSON line on stdout.  ``value`` is TFLOP/s with the flop count
4*B*Hq*Nq*Nk*d (halved for causal).  ``roofline`` compares the kernel's
average duration (HIP events around every launch inside the timed region,
on the launch stream) with MI355X's dense bf16/fp16 MFMA peak.
``cpu_baseline`` times the fp64 CPU oracle on a bounded sample of the same
workload (rank 0 only).

``--op bwd`` measures the backward pass instead: one step = one ``attn_bwd``
call (its two kernels) from the forward's out and lse, with a seeded dout;
flops = 10*B*Hq*Nq*Nk*d (the five products S, dP, dV, dK, dQ; halved for
causal).  The default (forward) is the headline metric.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (bf16, d=128) and % of MI355X bf16 MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0}  # MI355X dense MFMA, published
METRIC_BWD = ("attention bwd TFLOP/s (10*B*Hq*Nq*Nk*d per call, halved for causal) and % of "
              "MI355X bf16 MFMA peak")
# Sources of each operation's kernels and launch code (the committed HBM
# traffic figures are valid only for these), the file that holds those
# figures, and the kernels one call launches.
_CSRC = os.path.join(ROOT, "exact_tiled_attention_35_amd", "csrc")
OP_SOURCES = {
    "fwd": ("gfx950_ops.hpp", "attn_fwd_kernel.hpp", "attn_fwd_splitk_kernel.hpp",
            "attn_fwd_k16_kernel.hpp", "attn_api.hip", "attn_host.hpp"),
    "bwd": ("gfx950_ops.hpp", "attn_bwd_kernel.hpp", "attn_bwd_api.hip", "attn_host.hpp"),
    "decode": ("gfx950_ops.hpp", "attn_decode_kernel.hpp", "attn_decode_api.hip", "attn_host.hpp"),
}
KERNEL_SOURCES = [os.path.join(_CSRC, n) for n in OP_SOURCES["fwd"]]
TRAFFIC_FILES = {op: os.path.join(ROOT, "profiles", f"attn_{op}_traffic.json") for op in OP_SOURCES}
TRAFFIC_FILE = TRAFFIC_FILES["fwd"]
OP_KERNELS = {
    # one of these per forward call: the tile kernel, or (plain d = 128 and
    # d = 256, windows at d = 128) its 16x16x32 form (small grids use
    # attn_fwd_splitk_kernel)
    "fwd": ("attn_fwd_kernel", "attn_fwd_k16_kernel"),
    "bwd": ("attn_bwd_dq_kernel", "attn_bwd_dkdv_kernel"),
    # the split attention kernel appends the new rows itself
    "decode": ("attn_decode_kernel", "attn_decode_merge_kernel"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def flops(w) -> float:
    f = 4.0 * w.B * w.Hq * w.Nq * w.Nk * w.d
    return f / 2 if w.causal else f


def decode_bytes(w) -> int:
    """HBM bytes one decode step must move: the whole K/V cache of every
    (batch, KV head) read once, q and the new K/V rows read, out, lse and the
    appended cache rows written."""
    el = 2
    return (w.B * w.Nk * w.Hkv * w.d * el * 2
            + w.B * w.Nq * w.Hq * w.d * el * 2 + w.B * w.Hq * w.Nq * 4
            + w.B * 1 * w.Hkv * w.d * el * 4)


def visible_pairs(Nq: int, Nk: int, causal: bool, left: int, right: int) -> int:
    """Number of (query, key) pairs a row-wise window / causal mask keeps
    (bottom-right aligned: key j kept for row i iff lo_i <= j <= hi_i)."""
    import numpy as np

    i = np.arange(Nq, dtype=np.int64)
    dg = i + (Nk - Nq)
    hi = np.full(Nq, Nk - 1, dtype=np.int64)
    if causal:
        hi = np.minimum(hi, dg)
    if right >= 0:
        hi = np.minimum(hi, dg + right)
    lo = np.maximum(0, dg - left) if left >= 0 else np.zeros(Nq, dtype=np.int64)
    return int(np.maximum(0, hi - lo + 1).sum())


def variant_flops(w, left, right) -> float:
    """4 d flops per kept (query, key) pair and head (both products)."""
    return 4.0 * w.B * w.Hq * w.d * visible_pairs(w.Nq, w.Nk, w.causal, left, right)


def bwd_flops(w) -> float:
    """Five products of the forward's size: S, dP, dV, dK, dQ."""
    return 2.5 * flops(w)


def bwd_algorithmic_bytes(w) -> int:
    el = 2
    return (w.B * w.Nq * w.Hq * w.d * el * 4          # q, out, dout read; dq written
            + w.B * w.Nk * w.Hkv * w.d * el * 4       # k, v read; dk, dv written
            + w.B * w.Hq * w.Nq * 4 * 2)              # lse read, delta written


def algorithmic_bytes(w) -> int:
    el = 2
    return (w.B * w.Nq * w.Hq * w.d * el * 2          # q read, out written
            + w.B * w.Nk * w.Hkv * w.d * el * 2       # k, v read
            + w.B * w.Hq * w.Nq * 4)                  # lse written


def kernel_source_hash(op: str = "fwd") -> str:
    """Hash of an operation's kernel sources with comments and whitespace
    removed, so that edits to comments alone keep the measured figures."""
    import re

    h = hashlib.sha256()
    for n in OP_SOURCES[op]:
        with open(os.path.join(_CSRC, n)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload_name: str, op: str = "fwd"):
    """HBM bytes per call from the committed rocprofv3 counter runs, or None
    if they were taken on another version of the kernel sources."""
    try:
        with open(TRAFFIC_FILES[op]) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get("workloads", {}).get(workload_name)
    if not rec or t.get("kernel_source_hash") != kernel_source_hash(op):
        return None
    return rec.get("hbm_bytes_per_launch")



def host_cores() -> int:
    """Cores this process may run on (its CPU affinity)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        return os.cpu_count() or 1


def blas_threads_in_use() -> int:
    try:
        from threadpoolctl import threadpool_info

        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover - informational only
        return host_cores()


def host_info(op: str = "fwd") -> dict:
    """What ran where: host cores, ROCm / HIP / torch versions, the kernel
    sources' hash and, where a git checkout is present, its revision."""
    import subprocess

    import torch

    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    rev = None
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short=12", "HEAD"],
                           capture_output=True, text=True, timeout=10)
        if r.returncode == 0:
            rev = r.stdout.strip()
            d = subprocess.run(["git", "-C", ROOT, "status", "--porcelain", "--untracked-files=no"],
                               capture_output=True, text=True, timeout=10)
            if d.returncode == 0 and d.stdout.strip():
                rev += "+modified"
    except (OSError, subprocess.SubprocessError):
        pass
    if rev is None:  # a copy of the tree without .git: the revision the library was built from
        try:
            with open(os.path.join(ROOT, "exact_tiled_attention_35_amd", "libattn.build.json")) as f:
                built = json.load(f).get("git_rev")
            rev = f"{built} (at build)" if built else None
        except (OSError, ValueError):
            pass
    src = op if op in OP_SOURCES else "fwd"
    return {"cores": host_cores(), "rocm": rocm, "hip_runtime": torch.version.hip,
            "torch": torch.__version__, "git_rev": rev,
            "kernel_source_hash": kernel_source_hash(src)}


def launch_stats(kernel_ms) -> dict:
    """Median, min and max of the per-launch event times (microseconds); every
    launch's time goes to stderr, so that a clock ramp over the timed steps
    can be told apart from a slower box."""
    us = sorted(1e3 * t for t in kernel_ms)
    n = len(us)
    med = us[n // 2] if n % 2 else 0.5 * (us[n // 2 - 1] + us[n // 2])
    log("[bench] per-launch us, in launch order: " + " ".join(f"{1e3 * t:.1f}" for t in kernel_ms))
    return {"median_us": round(med, 2), "min_us": round(us[0], 2), "max_us": round(us[-1], 2)}


def sustained_clock(step, stream, seconds: float, achieved: float, peak: float,
                    nominal_mhz: float = 2400.0):
    """The GPU's graphics clock and socket power under this step's load, read
    from amdsmi's GPU metrics while the step runs back to back for `seconds`
    after the timed region (outside it).  The firmware refreshes that table
    about once per second, so only refreshes at least 0.5 s into the load
    count; a timed region of milliseconds cannot be sampled this way.  The
    clock also rescales the peak: frac_of_peak_at_this_clock is the timed
    steps' achieved rate against the peak at this clock.  Best effort: without
    amdsmi, or without a refresh, the summary says so."""
    import threading

    import torch

    out = {"source": "amdsmi GPU metrics, refreshed by the firmware about once per second, "
                     "sampled while the step ran back to back after the timed region",
           "seconds": seconds, "nominal_mhz": nominal_mhz}
    if seconds <= 0:
        out["error"] = "disabled"
        return out
    try:
        import amdsmi

        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception as e:  # pragma: no cover - depends on the box
        out["error"] = f"{type(e).__name__}: {e}"
        return out
    samples, stop = [], threading.Event()

    def read():
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
        except Exception:  # pragma: no cover
            return
        clks = [float(c) for c in (m.get("current_gfxclks") or [])
                if isinstance(c, (int, float)) and 0 < c < 0xFFFF]
        samples.append({"t": time.perf_counter(), "acc": m.get("accumulation_counter"),
                         "clk": sum(clks) / len(clks) if clks else None,
                         "clk_min": min(clks) if clks else None,
                         "power": m.get("current_socket_power")})

    def loop():
        while not stop.is_set():
            read()
            stop.wait(0.02)

    read()
    th = threading.Thread(target=loop, daemon=True)
    t0 = time.perf_counter()
    th.start()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        n += 10
    stop.set()
    th.join(timeout=2.0)
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:  # pragma: no cover
        pass
    out["steps_run"] = n
    out.update(clock_summary(samples, t0, achieved, peak, nominal_mhz))
    return out


def clock_summary(samples, t0: float, achieved: float, peak: float, nominal_mhz: float = 2400.0):
    """Keep one sample per refresh of the GPU metrics table (its
    accumulation counter changes at each refresh) taken at least 0.5 s after
    the load started at t0, the first sample (before the load) excluded, and
    average the mean-over-XCDs clock and the socket power over them."""
    first_acc = samples[0]["acc"] if samples else None
    fresh, seen = [], set()
    for r in samples:
        if r["t"] >= t0 + 0.5 and r["acc"] != first_acc and r["acc"] not in seen and r["clk"]:
            seen.add(r["acc"])
            fresh.append(r)
    out = {"refreshes_under_load": len(fresh)}
    if not fresh:
        out["error"] = "no refresh of the GPU metrics under the load"
        return out
    clk = sum(r["clk"] for r in fresh) / len(fresh)
    out["gfxclk_mhz_mean_over_xcds"] = round(clk, 1)
    out["gfxclk_mhz_slowest_xcd"] = round(min(r["clk_min"] for r in fresh), 1)
    pw = [r["power"] for r in fresh if isinstance(r["power"], (int, float))]
    if pw:
        out["socket_power_w"] = round(sum(pw) / len(pw), 1)
    out["frac_of_peak_at_this_clock"] = round(achieved / (peak * clk / nominal_mhz), 4)
    return out


def cpu_baseline(w, q, k, v, budget_s: float, out=None, lse=None):
    """Time the fp64 oracle head by head (all rows of each) on this host until
    ``budget_s`` is spent, with BLAS on every core of the process's affinity.
    Given this run's GPU ``out`` / ``lse`` (CPU copies), also compare them
    with the oracle on every head it evaluated (outside the oracle's timing):
    max-abs and mean-abs over all those output elements, the logsumexp error
    over their rows, and the floor max |dtype(O_64) - O_64|."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle

    cores = host_cores()
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    done, t_oracle = 0, 0.0
    par = {"max_abs": 0.0, "sum_abs": 0.0, "n": 0, "lse_abs": 0.0, "floor": 0.0}
    with threadpool_limits(limits=cores, user_api="blas"):
        blas = blas_threads_in_use()
        for (b, h) in heads:
            t0 = time.perf_counter()
            O, L = oracle.attention_rows(q, k, v, w.scale, w.causal, b, h, np.arange(w.Nq))
            t_oracle += time.perf_counter() - t0
            done += 1
            if out is not None:
                err = np.abs(out[b, :, h, :].double().numpy() - O)
                par["max_abs"] = max(par["max_abs"], float(err.max()))
                par["sum_abs"] += float(err.sum())
                par["n"] += err.size
                fin = np.isfinite(L)
                lg = lse[b, h].double().numpy()
                if fin.any():
                    par["lse_abs"] = max(par["lse_abs"], float(np.abs(lg[fin] - L[fin]).max()))
                rounded = torch.from_numpy(O).to(out.dtype).double().numpy()
                par["floor"] = max(par["floor"], float(np.abs(rounded - O).max()))
            if t_oracle >= budget_s:
                break
    f = flops(w) * done / len(heads)
    res = {
        "value": f / t_oracle / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "blas_threads": blas,
        "kind": "oracle",
        "sample": f"{done} of {len(heads)} (batch, head) pairs, all {w.Nq} query rows each, "
                  f"fp64 NumPy, {t_oracle:.1f} s of oracle time",
    }
    if out is not None:
        res["parity"] = {
            "compared": f"this run's GPU output on every row of the {done} oracle heads",
            "max_abs": par["max_abs"], "mean_abs": par["sum_abs"] / max(1, par["n"]),
            "lse_abs": par["lse_abs"], "floor": par["floor"],
            "tolerance": {"max_abs": 1e-2, "mean_abs": 1e-3, "lse_abs": 1e-3},
        }
        res["parity"]["pass"] = bool(res["parity"]["max_abs"] <= 1e-2
                                     and res["parity"]["mean_abs"] <= 1e-3
                                     and res["parity"]["lse_abs"] <= 1e-3)
    return res


def cpu_baseline_bwd(w, q, k, v, do, budget_s: float):
    """Time the fp64 backward oracle on whole KV groups until ``budget_s`` is spent."""
    import numpy as np

    import oracle

    G = w.Hq // w.Hkv
    groups = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    done = 0
    t0 = time.perf_counter()
    for (b, g) in groups:
        hs = slice(g * G, (g + 1) * G)
        oracle.attention_backward(q[b:b + 1, :, hs], k[b:b + 1, :, g:g + 1], v[b:b + 1, :, g:g + 1],
                                  do[b:b + 1, :, hs], w.scale, w.causal)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    f = bwd_flops(w) * done / len(groups)
    return {
        "value": f / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": host_cores(),
        "blas_threads": blas_threads_in_use(),
        "kind": "oracle",
        "sample": f"{done} of {len(groups)} (batch, KV head) groups, all rows, fp64 NumPy, "
                  f"{dt:.1f} s wall",
    }


def cpu_baseline_decode(w, q, kc, vc, budget_s: float):
    """Time the fp64 oracle on whole sequences of the decode workload."""
    import oracle

    done = 0
    t0 = time.perf_counter()
    for b in range(w.B):
        oracle.attention(q[b:b + 1], kc[b:b + 1], vc[b:b + 1], w.scale, w.causal)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": decode_bytes(w) * done / w.B / dt / 1e9,
        "unit": "GB/s",
        "cores": host_cores(),
        "blas_threads": blas_threads_in_use(),
        "kind": "oracle",
        "sample": f"{done} of {w.B} sequences, every query head, fp64 NumPy, {dt:.1f} s wall",
    }


def calibration_copy(mib: int):
    """One elementwise kernel that reads mib MiB and writes mib MiB (a negated
    copy), the yardstick that scales FETCH_SIZE / WRITE_SIZE to bytes."""
    import torch

    n = mib * 2**20 // 4
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()


def _pmc_rows(path: str, counter: str):
    """(kernel name, counter value) per dispatch from rocprofv3 output: a
    counter_collection.csv, or the SQLite database rocprofv3 writes by default."""
    rows = []
    if path.endswith(".db"):
        import sqlite3

        con = sqlite3.connect(path)
        q = "select kernel_name, value from counters_collection where counter_name = ? order by start"
        rows = [(k, float(v)) for (k, v) in con.execute(q, (counter,))]
        con.close()
        return rows
    import csv

    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def write_traffic_summary(fetch_csv: str, write_csv: str, copy_mib, workload=None, op="fwd"):
    """Per-call HBM bytes of an operation from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch; a call's kernels are summed), each scaled by the factor that
    maps the same counter onto a plain copy of known size."""
    from attn_workloads import DECODE_WORKLOADS, HEADLINE, WORKLOADS

    copy_bytes = int(copy_mib) * 2**20
    if op == "decode":
        name = workload or next(iter(DECODE_WORKLOADS))
        w = DECODE_WORKLOADS[name]
        algo = decode_bytes(w)
    else:
        name = workload or HEADLINE
        w = WORKLOADS[name]
        algo = algorithmic_bytes(w) if op == "fwd" else bwd_algorithmic_bytes(w)
    path = TRAFFIC_FILES[op]
    out = {"kernel_source_hash": kernel_source_hash(op), "workloads": {}}
    if os.path.exists(path):
        with open(path) as f:
            old = json.load(f)
        if old.get("kernel_source_hash") == out["kernel_source_hash"]:
            out = old
    rec = {"kernels": list(OP_KERNELS[op])} if op != "fwd" else {}
    for csv_path, counter, key in ((fetch_csv, "FETCH_SIZE", "read"), (write_csv, "WRITE_SIZE", "written")):
        rows = _pmc_rows(csv_path, counter)
        copy = [v for (k, v) in rows if "neg_kernel" in k]
        per_kernel = []
        for kern in OP_KERNELS[op]:
            vals = [v for (k, v) in rows if kern + "<" in k]
            if not vals and op != "fwd":
                raise SystemExit(f"{csv_path}: no {kern} dispatches for {counter}")
            if vals:
                per_kernel.append(sum(vals) / len(vals))
        if not per_kernel:
            raise SystemExit(f"{csv_path}: no forward kernel dispatches for {counter}")
        if not copy:
            raise SystemExit(f"{csv_path}: no copy dispatch for {counter}")
        factor = copy_bytes / (max(copy) * 1024.0)
        kib = sum(per_kernel)
        rec[f"{counter}_KiB_per_launch"] = kib
        rec[f"{counter}_copy_scale"] = factor
        rec[f"bytes_{key}_per_launch"] = kib * 1024.0 * factor
    rec["hbm_bytes_per_launch"] = rec["bytes_read_per_launch"] + rec["bytes_written_per_launch"]
    rec["algorithmic_bytes"] = algo
    out["workloads"][name] = rec
    with open(path, "w") as f:
        json.dump(out, f, indent=2)
    print(json.dumps(rec, indent=2))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default=None, help="workload name (default: the headline one)")
    ap.add_argument("--op", choices=("fwd", "bwd", "decode", "varlen", "varlen_bwd", "blocksparse",
                                     "blocksparse_bwd"),
                    default="fwd",
                    help="fwd: attn_fwd (the headline metric); bwd: attn_bwd, the backward pass; "
                         "decode: attn_decode on a KV-cache decode workload; varlen: "
                         "attn_fwd_varlen on packed variable-length sequences; varlen_bwd: "
                         "attn_bwd_varlen on them; blocksparse: "
                         "attn_fwd_blocksparse with a random block mask; blocksparse_bwd: "
                         "attn_bwd_blocksparse on the same workloads")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time")
    ap.add_argument("--window", nargs=2, type=int, default=(-1, -1), metavar=("LEFT", "RIGHT"),
                    help="fwd/bwd: sliding window (attn_fwd_ext / attn_bwd_ext); flops count the "
                         "kept pairs")
    ap.add_argument("--softcap", type=float, default=0.0,
                    help="fwd/bwd: softcap (attn_fwd_ext / attn_bwd_ext)")
    ap.add_argument("--alibi", action="store_true",
                    help="fwd/bwd: ALiBi slopes (attn_fwd_ext / attn_bwd_ext)")
    ap.add_argument("--splits", type=int, default=0,
                    help="decode only: number of key splits (0: the library's heuristic)")
    ap.add_argument("--cold-mib", type=int, default=0, metavar="MIB",
                    help="fwd/bwd diagnostic: after the timed steps, time the same number of "
                         "steps again with MIB MiB of scratch read before each one (evicts L2 "
                         "and the Infinity Cache; outside the timed region) and report them "
                         "as \"cold\"; the headline figures stay the warm ones")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--clock-seconds", type=float, default=2.5,
                    help="after the timed steps, run the step back to back this long and read "
                         "the GPU clock and power from amdsmi's GPU metrics (0: skip)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0, metavar="MIB",
                    help="after the timed steps, run one plain elementwise copy kernel that "
                         "reads and writes MIB MiB (the reference for scaling HBM byte counters "
                         "under rocprofv3 --pmc)")
    ap.add_argument("--traffic-from", nargs=3, metavar=("FETCH_OUT", "WRITE_OUT", "COPY_MIB"),
                    help="turn the rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE outputs (.db or "
                         "counter_collection.csv) of runs made with --calibration-copy-mib "
                         "COPY_MIB into the committed per-launch traffic summary, then exit")
    args = ap.parse_args()

    if args.traffic_from:
        write_traffic_summary(*args.traffic_from, workload=args.workload,
                              op=args.op if args.op in OP_SOURCES else "fwd")
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(sharding is described in the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from attn_workloads import DECODE_WORKLOADS, HEADLINE, VARLEN_WORKLOADS, WORKLOADS, make_workload
    from exact_tiled_attention_35_amd import attn_bwd_ptr, attn_fwd, attn_version
    from exact_tiled_attention_35_amd.attention import _DTYPE_CODE

    if args.op in ("varlen", "varlen_bwd"):
        if not torch.cuda.is_available():
            log("no GPU visible")
            sys.exit(1)
        return bench_varlen(args, VARLEN_WORKLOADS[args.workload or next(iter(VARLEN_WORKLOADS))],
                            backward=args.op == "varlen_bwd")
    if args.op in ("blocksparse", "blocksparse_bwd"):
        from attn_workloads import BLOCKSPARSE_WORKLOADS

        if not torch.cuda.is_available():
            log("no GPU visible")
            sys.exit(1)
        return bench_blocksparse(args, args.workload or next(iter(BLOCKSPARSE_WORKLOADS)),
                                 backward=args.op == "blocksparse_bwd")
    if args.op == "decode":
        w = DECODE_WORKLOADS[args.workload or next(iter(DECODE_WORKLOADS))]
    else:
        w = WORKLOADS[args.workload or HEADLINE]
    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] workload {w.name}; library {attn_version()}")
    if args.op == "decode":
        return bench_decode(args, w, dev)
    q, k, v = make_workload(w)
    dq, dk, dv = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(dq)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    variants = tuple(args.window) != (-1, -1) or args.softcap != 0.0 or args.alibi
    if args.op == "fwd":
        slopes = None
        if args.alibi:
            slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / w.Hq) for h in range(w.Hq)],
                                  dtype=torch.float32, device=dev)

        def step():
            attn_fwd(dq, dk, dv, w.scale, w.causal, out=out, lse=lse, window=tuple(args.window),
                     alibi_slopes=slopes, softcap=args.softcap)
    else:
        from attn_workloads import make_qkv

        do = make_qkv(w.B, w.Nq, w.Nq, w.Hq, w.Hq, w.d, w.dtype, w.sigma, w.seed + 100)[0]
        ddo = do.to(dev)
        attn_fwd(dq, dk, dv, w.scale, w.causal, out=out, lse=lse)
        gq, gk, gv = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
        delta = torch.empty_like(lse)
        ptrs = [t.data_ptr() for t in (dq, dk, dv, out, ddo, lse, gq, gk, gv, delta)]
        code_dt = _DTYPE_CODE[dq.dtype]

        slopes = None
        if args.alibi:
            slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / w.Hq) for h in range(w.Hq)],
                                  dtype=torch.float32, device=dev)
        if variants:
            from exact_tiled_attention_35_amd.attention import attn_bwd_ext_ptr

            attn_fwd(dq, dk, dv, w.scale, w.causal, out=out, lse=lse, window=tuple(args.window),
                     alibi_slopes=slopes, softcap=args.softcap)

        def step():
            if variants:
                code = attn_bwd_ext_ptr(*ptrs, w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.scale, w.causal,
                                        args.window[0], args.window[1],
                                        slopes.data_ptr() if slopes is not None else 0,
                                        args.softcap, code_dt, stream.cuda_stream)
            else:
                code = attn_bwd_ptr(*ptrs, w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.scale, w.causal,
                                    code_dt, stream.cuda_stream)
            if code != 0:
                raise SystemExit(f"attn_bwd failed with status {code}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    torch.cuda.synchronize()  # one rank: the barrier is this synchronisation
    t0 = time.perf_counter()
    for i in range(K):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    kernel_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_kernel_s = sum(kernel_ms) / K / 1e3
    ms_per_step = wall / K * 1e3
    per_launch = launch_stats(kernel_ms)

    F = flops(w) if args.op == "fwd" else bwd_flops(w)
    if variants:
        F = variant_flops(w, *args.window) * (1.0 if args.op == "fwd" else 2.5)
    value = F / (wall / K) / 1e12
    achieved = F / avg_kernel_s / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    traffic = None if variants else measured_traffic(w.name, args.op)
    log(f"[bench] {K} steps: {ms_per_step:.4f} ms/step wall, kernel avg {avg_kernel_s*1e6:.1f} us "
        f"(median {per_launch['median_us']:.1f}, min {per_launch['min_us']:.1f} us), "
        f"{achieved:.1f} TFLOP/s = {100*achieved/peak:.1f}% of peak")

    result = {
        "metric": METRIC if args.op == "fwd" else METRIC_BWD,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0, sigma^2) inputs rounded to the element type)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk,
                   "d": w.d, "causal": w.causal, "seed": w.seed, "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "algorithmic_bytes": algorithmic_bytes(w) if args.op == "fwd" else bwd_algorithmic_bytes(w),
            "kernel_avg_us": round(avg_kernel_s * 1e6, 2),
            "kernel_median_us": per_launch["median_us"],
            "kernel_min_us": per_launch["min_us"],
            "kernel_max_us": per_launch["max_us"],
            "achieved_at_median": round(F / (per_launch["median_us"] * 1e-6) / 1e12, 3),
        },
        "clock": sustained_clock(step, stream, args.clock_seconds, achieved, peak),
        "host": host_info(args.op),
        "cpu_baseline": None,
        "context": "FlexAttention with the FA4 backend reports 1.2x-3.2x speedups on NVIDIA "
                   "Hopper/Blackwell (liora.io news item); other hardware, not a target",
    }
    if args.cold_mib > 0:
        result["cold"] = cold_timing(step, stream, K, args.cold_mib, F, peak)
    if args.calibration_copy_mib:
        calibration_copy(args.calibration_copy_mib)
        result["calibration_copy_bytes"] = args.calibration_copy_mib * 2**20
    if variants:
        result["config"]["variants"] = {"window": list(args.window), "softcap": args.softcap,
                                         "alibi": bool(args.alibi)}
        if args.op == "fwd":
            result["metric"] = ("attention fwd TFLOP/s with score variants (4*d per kept "
                                "(query, key) pair and head)")
            result["context"] = "score variants (attn_fwd_ext); the headline metric is plain attn_fwd"
        else:
            result["metric"] = ("attention bwd TFLOP/s with score variants (10*d per kept "
                                "(query, key) pair and head)")
            result["context"] = "score variants in the backward (attn_bwd_ext)"
    if args.op == "bwd":
        result["roofline"]["unit_of_work"] = ("one attn_bwd call: the dQ kernel and the dK/dV "
                                              "kernel back to back")
        result["context"] = "backward pass; the headline metric is the forward (--op fwd)"
    if not args.no_cpu_baseline:
        del dq, dk, dv
        if args.op == "fwd" and variants:
            result["cpu_baseline"] = None  # the oracle baseline is timed on the plain forward
        elif args.op == "fwd":
            # the output of the last timed step, compared with the oracle
            out_c, lse_c = out.cpu(), lse.cpu()
            result["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_budget, out_c, lse_c)
        else:
            result["cpu_baseline"] = cpu_baseline_bwd(w, q, k, v, do, args.cpu_budget)
    print(json.dumps(result), flush=True)


def cold_timing(step, stream, K, mib, F, peak):
    """Diagnostic: K steps, each after MIB MiB of scratch has been read on the
    same stream (a reduction, outside the events), so that no input is left in
    L2 or the Infinity Cache when the step starts.  The scratch is written once
    beforehand and then only read, so no dirty lines are left to be written
    back during a step.  Returns the event-timed kernel average and its
    fraction of the peak."""
    import torch

    scratch = torch.ones(mib * 2**20 // 4, dtype=torch.float32, device=stream.device)
    sums = [scratch.sum() for _ in range(2)]  # flush the initial writes
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for i in range(K):
        sums.append(scratch.sum())
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    avg_s = sum(s.elapsed_time(e) for s, e in zip(starts, ends)) / K / 1e3
    achieved = F / avg_s / 1e12
    log(f"[bench] cold ({mib} MiB read before each step): kernel avg {avg_s * 1e6:.1f} us, "
        f"{achieved:.1f} TFLOP/s = {100 * achieved / peak:.1f}% of peak")
    return {"scratch_mib": mib, "kernel_avg_us": round(avg_s * 1e6, 2),
            "achieved": round(achieved, 3), "frac": round(achieved / peak, 4)}


def bench_decode(args, w, dev):
    """One step = one attn_decode call: append one K/V row per sequence at row
    Nk - 1 of a cache holding Nk - 1 rows, then attend over all Nk rows."""
    import torch

    from attn_workloads import make_qkv
    from exact_tiled_attention_35_amd import (attn_decode_num_splits, attn_decode_ptr,
                                              attn_decode_workspace_size)
    from exact_tiled_attention_35_amd.attention import _DTYPE_CODE

    q = make_qkv(w.B, w.Nq, w.Nq, w.Hq, w.Hq, w.d, w.dtype, w.sigma, w.seed)[0]
    _, kc, vc = make_qkv(w.B, 1, w.Nk, 1, w.Hkv, w.d, w.dtype, w.sigma, w.seed + 1)
    _, kn, vn = make_qkv(w.B, 1, 1, 1, w.Hkv, w.d, w.dtype, w.sigma, w.seed + 2)
    stream = torch.cuda.current_stream(dev)
    gq, gkc, gvc, gkn, gvn = (t.to(dev) for t in (q, kc, vc, kn, vn))
    sl = torch.full((w.B,), w.Nk - 1, dtype=torch.int32, device=dev)
    out = torch.empty_like(gq)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
    splits = args.splits or attn_decode_num_splits(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d)
    ws_bytes = attn_decode_workspace_size(w.B, w.Hq, w.Nq, w.d, splits)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    args_c = [t.data_ptr() for t in (gq, gkc, gvc, sl, gkn, gvn, out, lse, ws)]

    def step():
        code = attn_decode_ptr(*args_c, ws_bytes, w.B, w.Hq, w.Hkv, w.Nq, w.Nk, 1, w.d, w.scale,
                               w.causal, _DTYPE_CODE[gq.dtype], splits, stream.cuda_stream)
        if code != 0:
            raise SystemExit(f"attn_decode failed with status {code}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    kernel_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_s = sum(kernel_ms) / K / 1e3
    per_launch = launch_stats(kernel_ms)
    nbytes = decode_bytes(w)
    value = nbytes / (wall / K) / 1e9
    achieved = nbytes / avg_s / 1e9
    peak = 8000.0
    log(f"[bench] {K} steps: {wall / K * 1e3:.4f} ms/step wall, call avg {avg_s * 1e6:.1f} us "
        f"(min {min(kernel_ms) * 1e3:.1f} us), {achieved:.1f} GB/s = {100 * achieved / peak:.1f}% "
        f"of HBM peak, {splits} splits")
    result = {
        "metric": "attention decode GB/s (K/V cache read once plus q, out, lse and the appended "
                  "rows, per call) and % of MI355X HBM peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0, sigma^2) inputs rounded to the element type)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq,
                   "cache_rows": w.Nk, "appended_rows": 1, "d": w.d, "causal": w.causal,
                   "splits": splits, "seed": w.seed, "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "GB/s",
            "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(w.name, "decode"),
            "algorithmic_bytes": nbytes,
            "kernel_avg_us": round(avg_s * 1e6, 2),
            "kernel_median_us": per_launch["median_us"],
            "kernel_min_us": per_launch["min_us"],
            "unit_of_work": "one attn_decode call: split attention (appending the new rows) and merge kernels",
        },
        "clock": sustained_clock(step, stream, args.clock_seconds, achieved, peak),
        "host": host_info("decode"),
        "cpu_baseline": None,
        "context": "KV-cache decode; the headline metric is the forward (--op fwd)",
    }
    if args.calibration_copy_mib:
        calibration_copy(args.calibration_copy_mib)
        result["calibration_copy_bytes"] = args.calibration_copy_mib * 2**20
    if not args.no_cpu_baseline:
        del gq, gkc, gvc
        kcf = kc.clone()
        kcf[:, w.Nk - 1] = kn[:, 0]
        vcf = vc.clone()
        vcf[:, w.Nk - 1] = vn[:, 0]
        result["cpu_baseline"] = cpu_baseline_decode(w, q, kcf, vcf, args.cpu_budget)
    print(json.dumps(result), flush=True)


def cpu_baseline_varlen(wl, lens, q, k, v, scale, budget_s: float):
    """Time the fp64 oracle sequence by sequence and head by head (all rows of
    each) until ``budget_s`` is spent."""
    import numpy as np

    import oracle

    starts = [0]
    for n in lens:
        starts.append(starts[-1] + n)
    done, f = 0, 0.0
    t0 = time.perf_counter()
    for b, n in enumerate(lens):
        s = starts[b]
        for h in range(wl["H"]):
            oracle.attention_rows(q[None, s:s + n], k[None, s:s + n], v[None, s:s + n], scale,
                                  wl["causal"], 0, h, np.arange(n))
            f += 4.0 * wl["d"] * visible_pairs(n, n, wl["causal"], -1, -1)
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": f / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": host_cores(),
        "blas_threads": blas_threads_in_use(),
        "kind": "oracle",
        "sample": f"{done} of {len(lens) * wl['H']} (sequence, head) pairs in packing order, all "
                  f"rows each, fp64 NumPy, {dt:.1f} s wall",
    }


def bench_varlen(args, wl, backward=False):
    """One step = one attn_fwd_varlen call over the packed batch (or,
    ``backward``, one attn_bwd_varlen call from its out and lse with a seeded
    dout); flops count 4*d (backward: 10*d) per kept (query, key) pair and
    head, sequence by sequence."""
    import torch

    from attn_workloads import make_varlen, varlen_lengths
    from exact_tiled_attention_35_amd import attn_bwd_varlen, attn_fwd_varlen, attn_version

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] workload {wl['name']}; library {attn_version()}")
    lens = varlen_lengths(wl["total"], wl["lo"], wl["hi"], wl["seed"])
    H, d, causal = wl["H"], wl["d"], wl["causal"]
    q, k, v, cu_q, cu_k = make_varlen(lens, lens, H, H, d, wl["dtype"], 1.0, wl["seed"])
    scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
    gq, gk, gv, gcq, gck = (t.to(dev) for t in (q, k, v, cu_q, cu_k))
    stream = torch.cuda.current_stream(dev)
    max_q = max(lens)

    def step():
        return attn_fwd_varlen(gq, gk, gv, gcq, gck, max_q, scale, causal)

    if backward:
        out, lse = step()
        gdo = make_varlen(lens, lens, H, H, d, wl["dtype"], 1.0, wl["seed"] + 100)[0].to(dev)

        def step():  # noqa: F811
            attn_bwd_varlen(gq, gk, gv, out, gdo, lse, gcq, gck, max_q, max_q, scale, causal)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    kernel_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_s = sum(kernel_ms) / K / 1e3
    per_launch = launch_stats(kernel_ms)
    F = sum((10.0 if backward else 4.0) * H * d * visible_pairs(n, n, causal, -1, -1) for n in lens)
    value = F / (wall / K) / 1e12
    achieved = F / avg_s / 1e12
    peak = PEAK_TFLOPS[wl["dtype"]]
    total = wl["total"]
    nbytes = total * H * d * 2 * 4 + H * total * 4 + (len(lens) + 1) * 4 * 2
    if backward:  # q, k, v, out, dout, lse read once; dq, dk, dv, delta written once
        nbytes = total * H * d * 2 * 8 + H * total * 4 * 2 + (len(lens) + 1) * 4 * 2
    log(f"[bench] {K} steps: {wall / K * 1e3:.4f} ms/step wall, kernel avg {avg_s * 1e6:.1f} us "
        f"(min {min(kernel_ms) * 1e3:.1f} us), {achieved:.1f} TFLOP/s = {100 * achieved / peak:.1f}% "
        f"of peak; lengths {lens}")
    result = {
        "metric": ("attention bwd TFLOP/s over packed variable-length sequences (10*d per kept "
                   "(query, key) pair and head)" if backward else
                   "attention fwd TFLOP/s over packed variable-length sequences (4*d per kept "
                   "(query, key) pair and head)"),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl["dtype"],
        "data": "synthetic (seeded N(0, 1) inputs rounded to the element type; seeded lengths)",
        "config": {"workload": wl["name"], "total_tokens": total, "lengths": lens, "H": H,
                   "d": d, "causal": causal, "seed": wl["seed"], "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": None,
            "algorithmic_bytes": nbytes,
            "kernel_avg_us": round(avg_s * 1e6, 2),
            "kernel_median_us": per_launch["median_us"],
            "kernel_min_us": per_launch["min_us"],
        },
        "clock": sustained_clock(step, stream, args.clock_seconds, achieved, peak),
        "host": host_info("bwd" if backward else "fwd"),
        "cpu_baseline": None,
        "context": ("packed variable-length backward" if backward else
                    "packed variable-length forward") + "; the headline metric is the forward (--op fwd)",
    }
    if not args.no_cpu_baseline and not backward:
        del gq, gk, gv
        result["cpu_baseline"] = cpu_baseline_varlen(wl, lens, q, k, v, scale, args.cpu_budget)
    print(json.dumps(result), flush=True)


def blocksparse_pair_counts(Nq: int, Nk: int, causal: bool, block: int):
    """[nqb, nkb] numbers of (query, key) pairs a fully kept block pair holds
    (the causal bound applied inside it; bottom-right aligned)."""
    import numpy as np

    nqb, nkb = -(-Nq // block), -(-Nk // block)
    i = np.arange(Nq)
    hi = np.minimum(i + (Nk - Nq) + 1, Nk) if causal else np.full(Nq, Nk)  # keys [0, hi) per row
    counts = np.zeros((nqb, nkb), dtype=np.int64)
    for kb in range(nkb):
        js, je = kb * block, min(Nk, kb * block + block)
        per_row = np.clip(hi - js, 0, je - js)
        counts[:, kb] = np.add.reduceat(per_row, np.arange(0, Nq, block))
    return counts


def cpu_baseline_blocksparse(w, q, k, v, mask, counts, budget_s: float):
    """Time the fp64 oracle on whole query blocks of the workload, (batch,
    head) pairs in order, until ``budget_s`` is spent."""
    import numpy as np

    import oracle
    from attn_workloads import BLOCK

    m = mask.numpy() != 0
    done, f = 0, 0.0
    t0 = time.perf_counter()
    for b in range(w.B):
        for h in range(w.Hq):
            oracle.attention_block_sparse_rows(q, k, v, mask, w.scale, w.causal, b, h,
                                               np.arange(w.Nq), block=BLOCK)
            f += 4.0 * w.d * float((m[b, h] * counts).sum())
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": f / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": host_cores(),
        "blas_threads": blas_threads_in_use(),
        "kind": "oracle",
        "sample": f"{done} of {w.B * w.Hq} (batch, head) pairs, all rows each, fp64 NumPy, "
                  f"{dt:.1f} s wall",
    }


def bench_blocksparse(args, name, backward=False):
    """One step = one attn_fwd_blocksparse call (or, ``backward``, one
    attn_bwd_blocksparse call from the forward's out and lse with a seeded
    dout); flops count 4*d (backward: 10*d) per kept (query, key) pair and
    head (the mask's kept blocks, with the causal bound inside them)."""
    import torch

    from attn_workloads import (BLOCK, BLOCKSPARSE_WORKLOADS, WORKLOADS, make_block_mask, make_qkv,
                                make_workload)
    from exact_tiled_attention_35_amd import attn_bwd_blocksparse, attn_fwd_blocksparse, attn_version

    spec = BLOCKSPARSE_WORKLOADS[name]
    w = WORKLOADS[spec["base"]]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] workload {name}; library {attn_version()}")
    q, k, v = make_workload(w)
    nqb, nkb = -(-w.Nq // BLOCK), -(-w.Nk // BLOCK)
    mask = make_block_mask(w.B, w.Hq, nqb, nkb, spec["density"], spec["mask_seed"])
    gq, gk, gv, gm = q.to(dev), k.to(dev), v.to(dev), mask.to(dev)
    out = torch.empty_like(gq)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        attn_fwd_blocksparse(gq, gk, gv, gm, w.scale, w.causal, out=out, lse=lse)

    if backward:
        step()
        gdo = make_qkv(w.B, w.Nq, w.Nk, w.Hq, w.Hkv, w.d, w.dtype, w.sigma, w.seed + 100)[0].to(dev)

        def step():  # noqa: F811
            attn_bwd_blocksparse(gq, gk, gv, out, gdo, lse, gm, w.scale, w.causal)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    kernel_ms = [s_.elapsed_time(e) for s_, e in zip(starts, ends)]
    avg_s = sum(kernel_ms) / K / 1e3
    per_launch = launch_stats(kernel_ms)
    counts = blocksparse_pair_counts(w.Nq, w.Nk, w.causal, BLOCK)
    kept_blocks = mask.numpy() != 0
    pairs = float((kept_blocks * counts[None, None]).sum())
    F = (10.0 if backward else 4.0) * w.d * pairs
    value = F / (wall / K) / 1e12
    achieved = F / avg_s / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    log(f"[bench] {K} steps: {wall / K * 1e3:.4f} ms/step wall, kernel avg {avg_s * 1e6:.1f} us "
        f"(min {min(kernel_ms) * 1e3:.1f} us), {achieved:.1f} TFLOP/s = {100 * achieved / peak:.1f}% "
        f"of peak; kept block pairs {kept_blocks.mean():.3f}, kept (query, key) pairs "
        f"{pairs / (w.B * w.Hq * w.Nq * w.Nk):.3f}")
    result = {
        "metric": ("attention bwd TFLOP/s with a block mask (10*d per kept (query, key) pair and head)"
                   if backward else
                   "attention fwd TFLOP/s with a block mask (4*d per kept (query, key) pair and head)"),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0, sigma^2) inputs rounded to the element type; seeded "
                "random block mask)",
        "config": {"workload": name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk,
                   "d": w.d, "causal": w.causal, "seed": w.seed, "block": BLOCK,
                   "mask_density": spec["density"], "mask_seed": spec["mask_seed"],
                   "kept_block_fraction": round(float(kept_blocks.mean()), 4),
                   "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": None,
            "kernel_avg_us": round(avg_s * 1e6, 2),
            "kernel_median_us": per_launch["median_us"],
            "kernel_min_us": per_launch["min_us"],
        },
        "clock": sustained_clock(step, stream, args.clock_seconds, achieved, peak),
        "host": host_info("bwd" if backward else "fwd"),
        "cpu_baseline": None,
        "context": ("block-sparse backward (the dQ and dK/dV kernels)" if backward else
                    "block-sparse forward") + "; the headline metric is the plain forward (--op fwd)",
    }
    if not args.no_cpu_baseline and not backward:
        del gq, gk, gv
        result["cpu_baseline"] = cpu_baseline_blocksparse(w, q, k, v, mask, counts, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
