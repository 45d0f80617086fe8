"""fp64 exact-attention oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module.  It is deliberately slow and plain: for every
(batch, query head) it writes out the scaled score matrix row by row over all
keys, masks it, and applies the textbook softmax and the product with V.
No tiling, no online rescaling, no fusion: that is what the GPU path does,
and this module exists to check it.

Sources (the pages, cited by title and section):

* hysenlabs.com, "FlashAttention: exakte Attention-Kernel fuer CUDA und ROCm",
  section "Die Schnittstellen von flash_attn_func bis KV-Cache": the functions
  compute scaled dot-product attention as softmax(Q @ K^T * softmax_scale) @ V,
  take a ``causal`` flag and a ``softmax_scale``, and accept fewer KV heads than
  query heads when the query head count is divisible by it (MQA/GQA).
* same page, section "Von 2.0 bis 2.7": since version 2.1 the causal mask is
  aligned to the bottom-right corner when query and key lengths differ.
* tokenwerk.de, "FlashAttention", section "Was FlashAttention veraendert":
  the method is exact attention -- not an approximate substitute -- and
  differences against a reference are floating-point effects judged with
  tolerances.
* tokenwerk.de, "FlashAttention", section "Warum Kacheln beim
  Speicherzugriff helfen" and its table: the dense score matrix of one head
  has N x N cells (2 bytes per cell in the page's arithmetic).

Readings where the pages are silent (each is listed in the design notes):

* layout: q, out are [B, Nq, Hq, d]; k, v are [B, Nk, Hkv, d]; lse is
  [B, Hq, Nq].  The oracle indexes logical (b, i, h, c) so it does not depend
  on strides.
* GQA grouping: query head h reads KV head floor(h / (Hq / Hkv)) -- each KV
  head serves a contiguous run of Hq/Hkv query heads.
* causal: key j is visible to query i iff j <= i + (Nk - Nq).
* scale: the value the library receives is an fp32; the oracle uses that same
  fp32 value, widened to fp64.
* logsumexp: natural log of the sum of exp over the scaled, masked scores.
* a query row with no visible key (causal, Nq > Nk) has output 0 and
  logsumexp -inf (the empty-sum limit).
* score variants (the interface section lists ``window_size`` and
  ``alibi_slopes`` among the parameters; section "Von 2.0 bis 2.7" dates
  sliding windows to 2.3, ALiBi to 2.4 and softcapping to 2.6): with
  diag = Nk - Nq, a window (left, right) keeps key j for row i iff
  i + diag - left <= j <= i + diag + right (a negative bound is no bound);
  softcapping replaces the scaled score t by cap * tanh(t / cap); ALiBi then
  adds -slope_h * |i + diag - j|.  The softmax runs over the result.

Block sparsity (``attention_block_sparse``; the liora.io item on
FlexAttention's new backend names block sparsity among its features, in the
section on its limitations, and gives 128 x 128 as the Hopper kernel's
block size): a mask of flags over (query block, key block) pairs decides
which blocks of the score matrix take part.  Reading: row i lies in query
block floor(i / 128), key j in key block floor(j / 128); key j is visible to
row i iff the flag of that pair is nonzero and j is causally visible (when
causal); everything else is the definition above.  The mask is
[B, Hm, ceil(Nq / 128), ceil(Nk / 128)] with Hm = 1 (shared by all query
heads) or Hm = Hq.

The backward pass (``attention_backward``): the pages say the library
computes gradients (hysenlabs.com page, section "GPU-Abdeckung: Ampere,
Hopper und AMD-Backends" on the backward pass for head dimension 256;
section "Von 2.0 bis 2.7" on a deterministic backward pass) and that its tests compare outputs *and
gradients* with a reference (section "Tests, BSD-3-Clause und
Zitierpraxis"); they do not write the gradients out.  Those are fixed by the
mathematics: the derivatives of the forward definition above with respect
to q, k and v for the loss L = sum(dout * out), written out by the chain
rule with the full probability matrix (no tiling, no recomputation).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "attention",
    "attention_rows",
    "attention_backward",
    "attention_varlen",
    "attention_backward_varlen",
    "attention_block_sparse",
    "attention_block_sparse_rows",
    "kv_head_of",
    "allowed_keys",
    "visible_range",
    "materialised_score_bytes",
]


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head ``h`` (GQA/MQA, contiguous groups).

    The interface page only requires Hq to be divisible by Hkv; the grouping
    below (query heads [g*G, (g+1)*G) share KV head g, G = Hq/Hkv) is the
    reading used throughout.
    """
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} must be a positive multiple of Hkv={Hkv}")
    return h // (Hq // Hkv)


def allowed_keys(i: int, Nq: int, Nk: int, causal: bool) -> int:
    """Number of keys visible to query row ``i``; they are keys [0, count).

    Non-causal rows see every key.  Causal rows see key j iff
    j <= i + (Nk - Nq): the mask is aligned to the bottom-right corner
    (hysenlabs.com page, section "Von 2.0 bis 2.7", version 2.1).
    """
    if not causal:
        return Nk
    return int(max(0, min(Nk, i + (Nk - Nq) + 1)))


def visible_range(i: int, Nq: int, Nk: int, causal: bool, window=(-1, -1)):
    """Keys [lo, hi) visible to query row ``i``: the causal bound of
    ``allowed_keys`` intersected with a (left, right) window around the
    bottom-right aligned diagonal key i + (Nk - Nq)."""
    left, right = window
    diag = Nk - Nq
    hi = allowed_keys(i, Nq, Nk, causal)
    if right >= 0:
        hi = min(hi, max(0, min(Nk, i + diag + right + 1)))
    lo = max(0, i + diag - left) if left >= 0 else 0
    return lo, max(lo, hi)


def materialised_score_bytes(Nq: int, Nk: int, bytes_per_cell: int = 2) -> int:
    """Size of one head's dense score matrix, as in the tokenwerk.de page's
    table (section "Warum Kacheln beim Speicherzugriff helfen"): Nq*Nk cells
    at ``bytes_per_cell`` bytes each."""
    return int(Nq) * int(Nk) * int(bytes_per_cell)


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor on the CPU: widen exactly
        import torch

        x = x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _check_shapes(q: np.ndarray, k: np.ndarray, v: np.ndarray):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D: [B, N, H, d]")
    B, Nq, Hq, d = q.shape
    Bk, Nk, Hkv, dk = k.shape
    if v.shape != k.shape or Bk != B or dk != d:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    return B, Nq, Nk, Hq, Hkv, d


def _rows_of_one_head(qh, kg, vg, sigma, rows, Nq, Nk, causal, want_p,
                      window=(-1, -1), slope=0.0, softcap=0.0, key_mask=None):
    """Exact attention for the query rows ``rows`` of one (b, h) pair.

    qh: [Nq, d]; kg, vg: [Nk, d] (already the KV head this query head reads).
    key_mask: optional [R, Nk] booleans; a key takes part only where it is
    True (in addition to the causal and window bounds).
    Returns (O [R, d], lse [R], S [R, Nk], P [R, Nk] or None).
    """
    rows = np.asarray(rows, dtype=np.int64)
    # Scores over ALL keys: s_ij = sigma * <q_i, k_j>.
    S = sigma * (qh[rows] @ kg.T)
    if softcap > 0.0:
        S = softcap * np.tanh(S / softcap)
    if slope != 0.0:
        S = S - slope * np.abs(rows[:, None] + (Nk - Nq) - np.arange(Nk)[None, :])
    # Mask: key j visible to row i iff lo(i) <= j < hi(i).
    rng = np.array([visible_range(int(i), Nq, Nk, causal, window) for i in rows],
                   dtype=np.int64).reshape(len(rows), 2)
    kidx = np.arange(Nk)[None, :]
    visible = (kidx >= rng[:, :1]) & (kidx < rng[:, 1:])
    if key_mask is not None:
        visible = visible & np.asarray(key_mask, dtype=bool)
    S = np.where(visible, S, -np.inf)
    # Row-wise softmax over keys.  Subtracting the row maximum is the usual
    # stable evaluation; it does not change the value.
    m = S.max(axis=1) if Nk > 0 else np.full(len(rows), -np.inf)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    E = np.exp(S - m_safe[:, None])  # exp(-inf) = 0 for masked keys
    l = E.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        P = np.where(empty[:, None], 0.0, E / np.where(empty, 1.0, l)[:, None])
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    O = P @ vg
    return O, lse, S, (P if want_p else None)


def attention(q, k, v, scale: float, causal: bool = False, *,
              return_scores: bool = False, return_probs: bool = False,
              slab_rows: int = 512, window=(-1, -1), alibi_slopes=None,
              softcap: float = 0.0):
    """Exact attention in fp64.

    Args:
      q: [B, Nq, Hq, d]; k, v: [B, Nk, Hkv, d] -- numpy arrays or CPU torch
         tensors holding the exact input values (bf16/fp16 values widen to
         fp64 without loss).
      scale: the softmax scale as passed to the library (an fp32 value).
      causal: apply the bottom-right aligned causal mask.
      return_scores / return_probs: also return the materialised score matrix
         S and the probabilities P, shaped [B, Hq, Nq, Nk] (small inputs only).
      slab_rows: how many query rows are written out at once.  Every row is
         independent of the others, so this only bounds memory.
      window: (left, right) sliding window around the diagonal; -1 = none.
      alibi_slopes: one slope per query head (fp32 values), or None.
      softcap: cap > 0 applies cap * tanh(t / cap) to the scaled scores.

    Returns:
      (O [B, Nq, Hq, d] fp64, lse [B, Hq, Nq] fp64[, S][, P]).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, Nq, Nk, Hq, Hkv, d = _check_shapes(q, k, v)
    sigma = float(np.float32(scale))
    cap = float(np.float32(softcap))
    slopes = (np.zeros(Hq) if alibi_slopes is None
              else np.asarray(alibi_slopes, dtype=np.float32).astype(np.float64).reshape(Hq))
    O = np.zeros((B, Nq, Hq, d))
    lse = np.full((B, Hq, Nq), -np.inf)
    S_all = np.full((B, Hq, Nq, Nk), -np.inf) if return_scores else None
    P_all = np.zeros((B, Hq, Nq, Nk)) if return_probs else None
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            qh, kg, vg = q[b, :, h, :], k[b, :, g, :], v[b, :, g, :]
            for r0 in range(0, Nq, max(1, slab_rows)):
                rows = np.arange(r0, min(Nq, r0 + slab_rows))
                Or, lr, Sr, Pr = _rows_of_one_head(qh, kg, vg, sigma, rows, Nq, Nk,
                                                   causal, return_probs, tuple(window),
                                                   float(slopes[h]), cap)
                O[b, rows, h, :] = Or
                lse[b, h, rows] = lr
                if return_scores:
                    S_all[b, h, rows, :] = Sr
                if return_probs:
                    P_all[b, h, rows, :] = Pr
    out = (O, lse)
    if return_scores:
        out = out + (S_all,)
    if return_probs:
        out = out + (P_all,)
    return out


def attention_rows(q, k, v, scale: float, causal: bool, b: int, h: int, rows, *,
                   window=(-1, -1), alibi_slopes=None, softcap: float = 0.0):
    """Exact attention for selected query rows of one (b, h) pair.

    Each output row depends only on its own query row and on all keys and
    values of the KV head it reads, so evaluating a subset of rows is the
    same definition restricted to those rows.  ``q`` needs only to provide
    q[b, rows, h, :]; pass full tensors or views.

    Returns (O [R, d] fp64, lse [R] fp64).
    """
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    g = kv_head_of(h, Hq, Hkv)
    qh = _as_f64(q[b, :, h, :])
    kg = _as_f64(k[b, :, g, :])
    vg = _as_f64(v[b, :, g, :])
    sigma = float(np.float32(scale))
    slope = 0.0 if alibi_slopes is None else float(np.float32(np.asarray(alibi_slopes).reshape(-1)[h]))
    O, lse, _, _ = _rows_of_one_head(qh, kg, vg, sigma, rows, Nq, Nk, causal, False,
                                     tuple(window), slope, float(np.float32(softcap)))
    return O, lse


def _softmax_rows_backward(P, dP):
    """Row-wise softmax Jacobian applied to dP: for p = softmax(s),
    ds_j = p_j (dp_j - sum_k p_k dp_k).  Returns (dS, D) with D the row sums
    sum_k p_k dp_k."""
    D = (P * dP).sum(axis=1)
    return P * (dP - D[:, None]), D


def attention_backward(q, k, v, dout, scale: float, causal: bool = False, *,
                       block_mask=None, block: int = 128, window=(-1, -1), alibi_slopes=None,
                       softcap: float = 0.0):
    """Exact gradients of L = sum(dout * attention(q, k, v)) in fp64.

    Per (b, h) with KV head g, probabilities P (rows over the visible keys,
    exactly as in ``attention``) and upstream gradient dO = dout[b, :, h, :]:

      dV_g += P^T dO                      (the output is P V)
      dP    = dO V_g^T                    (gradient w.r.t. the probabilities)
      D_i   = sum_j P_ij dP_ij            (= dO_i . O_i)
      dS    = P * (dP - D[:, None])       (softmax Jacobian applied row-wise)
      dQ    = sigma * dS K_g              (s_ij = sigma q_i . k_j)
      dK_g += sigma * dS^T Q

    KV heads shared by a group of query heads (GQA/MQA) receive the sum over
    the group.  Masked keys have P = 0, so they get no gradient, and rows with
    no visible key contribute nothing.

    Args: q [B, Nq, Hq, d]; k, v [B, Nk, Hkv, d]; dout like q (numpy arrays
    or CPU torch tensors); scale as passed to the library (an fp32 value);
    block_mask: None, or the flags of ``attention_block_sparse`` (the
    gradients of that function: P is its probability matrix).
    window, alibi_slopes, softcap: the score variants of ``attention``.  The
    window and ALiBi enter through P only (the bias does not depend on q or
    k); with a softcap the final score is cap * tanh(s / cap) of the scaled
    score s, so dS is multiplied by its derivative 1 - tanh(s / cap)^2 before
    the products with K and Q.

    Returns (dq [B, Nq, Hq, d], dk [B, Nk, Hkv, d], dv [B, Nk, Hkv, d],
    delta [B, Hq, Nq]) in fp64, where delta holds D.
    """
    q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    B, Nq, Nk, Hq, Hkv, d = _check_shapes(q, k, v)
    if dout.shape != q.shape:
        raise ValueError(f"dout{dout.shape} must match q{q.shape}")
    sigma = float(np.float32(scale))
    cap = float(np.float32(softcap))
    slopes = (np.zeros(Hq) if alibi_slopes is None
              else np.asarray(alibi_slopes, dtype=np.float32).astype(np.float64).reshape(Hq))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = np.zeros((B, Hq, Nq))
    rows = np.arange(Nq)
    bm = None
    if block_mask is not None:
        if hasattr(block_mask, "detach"):
            block_mask = block_mask.detach().cpu().numpy()
        bm = np.asarray(block_mask) != 0
        if bm.ndim != 4 or bm.shape[0] != B or bm.shape[1] not in (1, Hq) or \
                bm.shape[2] != -(-Nq // block) or bm.shape[3] != -(-Nk // block):
            raise ValueError(f"block_mask{bm.shape} does not match the shapes")
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            qh, kg, vg = q[b, :, h, :], k[b, :, g, :], v[b, :, g, :]
            dO = dout[b, :, h, :]
            key_mask = None
            if bm is not None:
                flags = bm[b, 0 if bm.shape[1] == 1 else h]
                key_mask = flags[(rows // block)[:, None], (np.arange(Nk) // block)[None, :]]
            _, _, _, P = _rows_of_one_head(qh, kg, vg, sigma, rows, Nq, Nk, causal, True,
                                           tuple(window), float(slopes[h]), cap,
                                           key_mask=key_mask)
            dv[b, :, g, :] += P.T @ dO
            dP = dO @ vg.T
            dS, D = _softmax_rows_backward(P, dP)
            if cap > 0.0:
                dS = dS * (1.0 - np.tanh(sigma * (qh @ kg.T) / cap) ** 2)
            dq[b, :, h, :] = sigma * (dS @ kg)
            dk[b, :, g, :] += sigma * (dS.T @ qh)
            delta[b, h, :] = D
    return dq, dk, dv, delta


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale: float, causal: bool = False):
    """Exact attention over packed variable-length sequences: sequence b is
    query rows [cu_q[b], cu_q[b+1]) of q [total_q, Hq, d] attending to key
    rows [cu_k[b], cu_k[b+1]) of k, v [total_k, Hkv, d], each on its own with
    ``attention`` (the unpadded layout of the hysenlabs.com page's version
    history, section "Von 2.0 bis 2.7").

    Returns (O [total_q, Hq, d], lse [Hq, total_q]) in fp64.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    cq = [int(x) for x in np.asarray(cu_seqlens_q).reshape(-1)]
    ck = [int(x) for x in np.asarray(cu_seqlens_k).reshape(-1)]
    total_q, Hq, d = q.shape
    O = np.zeros((total_q, Hq, d))
    lse = np.full((Hq, total_q), -np.inf)
    for b in range(len(cq) - 1):
        qs, qe, ks, ke = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if qe <= qs:
            continue
        if ke <= ks:  # no keys: rows stay 0 / -inf
            continue
        Ob, Lb = attention(q[None, qs:qe], k[None, ks:ke], v[None, ks:ke], scale, causal)
        O[qs:qe] = Ob[0]
        lse[:, qs:qe] = Lb[0]
    return O, lse


def attention_backward_varlen(q, k, v, dout, cu_seqlens_q, cu_seqlens_k, scale: float,
                              causal: bool = False):
    """Gradients of L = sum(dout * attention_varlen(...)) in fp64: sequence by
    sequence, ``attention_backward`` on that sequence's rows (the sequences
    share no rows, so their gradients do not interact).  Key rows of a
    sequence without query rows, and query rows of a sequence without keys,
    get zero gradients.

    Returns (dq [total_q, Hq, d], dk, dv [total_k, Hkv, d], delta [Hq, total_q]).
    """
    q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    cq = [int(x) for x in np.asarray(cu_seqlens_q).reshape(-1)]
    ck = [int(x) for x in np.asarray(cu_seqlens_k).reshape(-1)]
    total_q, Hq, d = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    delta = np.zeros((Hq, total_q))
    for b in range(len(cq) - 1):
        qs, qe, ks, ke = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if qe <= qs or ke <= ks:
            continue
        g = attention_backward(q[None, qs:qe], k[None, ks:ke], v[None, ks:ke], dout[None, qs:qe],
                               scale, causal)
        dq[qs:qe], dk[ks:ke], dv[ks:ke] = g[0][0], g[1][0], g[2][0]
        delta[:, qs:qe] = g[3][0]
    return dq, dk, dv, delta


def attention_block_sparse_rows(q, k, v, block_mask, scale: float, causal: bool, b: int, h: int,
                                rows, block: int = 128):
    """``attention_block_sparse`` for selected query rows of one (b, h) pair:
    each row depends only on its own query row, its mask flags and the keys
    and values of its KV head, so this is the same definition restricted to
    those rows.  Returns (O [R, d], lse [R]) in fp64."""
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    if hasattr(block_mask, "detach"):
        block_mask = block_mask.detach().cpu().numpy()
    bm = np.asarray(block_mask) != 0
    rows = np.asarray(rows, dtype=np.int64)
    flags = bm[b, 0 if bm.shape[1] == 1 else h]
    key_mask = flags[(rows // block)[:, None], (np.arange(Nk) // block)[None, :]]
    g = kv_head_of(h, Hq, Hkv)
    O, lse, _, _ = _rows_of_one_head(_as_f64(q[b, :, h, :]), _as_f64(k[b, :, g, :]),
                                     _as_f64(v[b, :, g, :]), float(np.float32(scale)), rows, Nq,
                                     Nk, causal, False, key_mask=key_mask)
    return O, lse


def attention_block_sparse(q, k, v, block_mask, scale: float, causal: bool = False,
                           block: int = 128):
    """Exact attention restricted by a block mask, in fp64.

    block_mask: [B, Hm, ceil(Nq / block), ceil(Nk / block)] (numpy or CPU
    torch), Hm = 1 or Hq; query row i and key j interact iff
    block_mask[b, hm, i // block, j // block] != 0 (hm = 0 when Hm = 1, else
    the query head) and, when ``causal``, j <= i + (Nk - Nq).  The flags are
    expanded to one boolean per (row, key) and the softmax runs over the
    scores of the keys they keep, exactly as in ``attention``; a row that
    keeps no key gets O = 0 and lse = -inf.  ``block`` is 128 for the
    library; smaller values serve tiny test shapes.

    Returns (O [B, Nq, Hq, d], lse [B, Hq, Nq]) in fp64.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, Nq, Nk, Hq, Hkv, d = _check_shapes(q, k, v)
    if hasattr(block_mask, "detach"):
        block_mask = block_mask.detach().cpu().numpy()
    bm = np.asarray(block_mask) != 0
    nqb, nkb = -(-Nq // block), -(-Nk // block)
    if bm.ndim != 4 or bm.shape[0] != B or bm.shape[1] not in (1, Hq) or \
            bm.shape[2] != nqb or bm.shape[3] != nkb:
        raise ValueError(f"block_mask{bm.shape} must be [B, 1 or Hq, {nqb}, {nkb}]")
    sigma = float(np.float32(scale))
    O = np.zeros((B, Nq, Hq, d))
    lse = np.full((B, Hq, Nq), -np.inf)
    rows = np.arange(Nq)
    qblk, kblk = rows // block, np.arange(Nk) // block
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            flags = bm[b, 0 if bm.shape[1] == 1 else h]
            key_mask = flags[qblk[:, None], kblk[None, :]]  # [Nq, Nk]
            Or, lr, _, _ = _rows_of_one_head(q[b, :, h, :], k[b, :, g, :], v[b, :, g, :], sigma,
                                             rows, Nq, Nk, causal, False, key_mask=key_mask)
            O[b, :, h, :] = Or
            lse[b, h, :] = lr
    return O, lse
