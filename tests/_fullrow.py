"""Every-row comparison of a GPU forward result with the fp64 oracle.

Test infrastructure.  For each (batch, query head) the oracle is evaluated on
every query row, in slabs of rows (each slab writes out its rows' scores over
all keys), and the GPU output of those rows is compared with it.  The
statistics are taken over ALL output elements and ALL logsumexp rows of the
workload:

* ``max_abs``, ``mean_abs``: |O_gpu - O_64| with O_gpu widened to fp64 and O_64
  the unrounded oracle output;
* ``lse_abs``: max |lse_gpu - lse_64| over rows with a visible key; rows
  without one must be -inf on both sides;
* ``floor``: max |dtype(O_64) - O_64|, the error a perfectly rounded output
  would have (what no kernel can go below), so that a failure can be told
  apart from the output's own rounding.

Heads run on a pool of threads (NumPy releases the interpreter lock inside
its array operations) with one BLAS thread each; no worker processes.
"""

from __future__ import annotations

import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle


def host_threads() -> int:
    """Cores this process may run on (its CPU affinity), at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _head_stats(q, k, v, out, lse, scale, causal, b, h, slab, tdtype):
    """Statistics of one (b, h) pair over all its rows."""
    Nq = q.shape[1]
    Hq, Hkv = q.shape[2], k.shape[2]
    g = oracle.kv_head_of(h, Hq, Hkv)
    # One head of each input, widened exactly to fp64 once for all slabs.
    qh = q[b, :, h, :].double().numpy()[None, :, None, :]
    kh = k[b, :, g, :].double().numpy()[None, :, None, :]
    vh = v[b, :, g, :].double().numpy()[None, :, None, :]
    oh = out[b, :, h, :]
    lh = lse[b, h, :].double().numpy()
    st = {"max_abs": 0.0, "sum_abs": 0.0, "n": 0, "lse_abs": 0.0, "floor": 0.0,
          "worst": None, "nonfinite": 0, "inf_mismatch": 0}
    for r0 in range(0, Nq, slab):
        rows = np.arange(r0, min(Nq, r0 + slab))
        O, L = oracle.attention_rows(qh, kh, vh, scale, causal, 0, 0, rows)
        o = oh[r0:r0 + len(rows)].double().numpy()
        st["nonfinite"] += int((~np.isfinite(o)).sum())
        err = np.abs(o - O)
        i = int(err.argmax())
        if err.flat[i] > st["max_abs"]:
            st["max_abs"] = float(err.flat[i])
            st["worst"] = (b, int(rows[i // O.shape[1]]), h, int(i % O.shape[1]))
        st["sum_abs"] += float(err.sum())
        st["n"] += err.size
        rounded = torch.from_numpy(O).to(tdtype).double().numpy()
        st["floor"] = max(st["floor"], float(np.abs(rounded - O).max()))
        lg = lh[r0:r0 + len(rows)]
        fin = np.isfinite(L)
        st["inf_mismatch"] += int((np.isfinite(lg) != fin).sum() + (lg[~fin] != -np.inf).sum())
        if fin.any():
            st["lse_abs"] = max(st["lse_abs"], float(np.abs(lg[fin] - L[fin]).max()))
    return st


def compare_every_row(q, k, v, out, lse, scale, causal, slab=512, threads=None):
    """Compare out [B, Nq, Hq, d] and lse [B, Hq, Nq] (CPU tensors) with the
    oracle on every row of every head.  Returns the merged statistics plus
    ``mean_abs``, ``heads``, ``rows``, ``threads`` and ``seconds``."""
    from threadpoolctl import threadpool_limits

    B, Nq, Hq, _ = q.shape
    threads = threads or host_threads()
    heads = [(b, h) for b in range(B) for h in range(Hq)]
    t0 = time.perf_counter()
    with threadpool_limits(limits=1, user_api="blas"):
        with ThreadPoolExecutor(max_workers=threads) as ex:
            parts = list(ex.map(lambda bh: _head_stats(q, k, v, out, lse, scale, causal,
                                                       bh[0], bh[1], slab, out.dtype), heads))
    tot = {"max_abs": 0.0, "sum_abs": 0.0, "n": 0, "lse_abs": 0.0, "floor": 0.0, "worst": None,
           "nonfinite": 0, "inf_mismatch": 0}
    for p in parts:
        if p["max_abs"] >= tot["max_abs"]:
            tot["max_abs"], tot["worst"] = p["max_abs"], p["worst"]
        for key in ("sum_abs", "n", "nonfinite", "inf_mismatch"):
            tot[key] += p[key]
        tot["lse_abs"] = max(tot["lse_abs"], p["lse_abs"])
        tot["floor"] = max(tot["floor"], p["floor"])
    tot["mean_abs"] = tot["sum_abs"] / max(1, tot["n"])
    tot["heads"] = len(heads)
    tot["rows"] = len(heads) * Nq
    tot["threads"] = threads
    tot["seconds"] = time.perf_counter() - t0
    return tot
