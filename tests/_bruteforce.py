"""Pure-Python brute-force attention for tiny shapes (a pin for the oracle).

Written independently of ``oracle/``: plain loops, ``math.exp`` and
``math.fsum``, no NumPy, no max subtraction, and its own index rules
(KV head by ``h * Hkv // Hq``; causal visibility by ``j - i <= Nk - Nq``).
For tiny inputs with moderate scores this is the definition evaluated as
directly as it can be: weight_j = exp(s_j) / sum_k exp(s_k).
"""

import math


def brute_attention(q, k, v, scale, causal, left=-1, right=-1, slopes=None, cap=0.0, keep=None):
    """q: nested lists [B][Nq][Hq][d]; k, v: [B][Nk][Hkv][d]; python floats.

    Optional score variants: a window of ``left`` keys before and ``right``
    keys after the diagonal key i + Nk - Nq (negative = unbounded); per-head
    ALiBi ``slopes`` (bias -slope * distance to that diagonal key); a softcap
    ``cap`` (cap * tanh(score / cap), before the bias); ``keep(b, h, i, j)``,
    a predicate that a key must also satisfy (an explicit element mask).

    Returns (O as nested lists [B][Nq][Hq][d], lse as [B][Hq][Nq])."""
    B, Nq, Hq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Nk, Hkv = len(k[0]), len(k[0][0])
    O = [[[[0.0] * d for _ in range(Hq)] for _ in range(Nq)] for _ in range(B)]
    lse = [[[0.0] * Nq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h * Hkv // Hq
            for i in range(Nq):
                dk = i + Nk - Nq  # the key on this row's diagonal
                keys = [j for j in range(Nk)
                        if (not causal or j <= dk) and (left < 0 or dk - j <= left)
                        and (right < 0 or j - dk <= right)
                        and (keep is None or keep(b, h, i, j))]
                if not keys:
                    lse[b][h][i] = -math.inf
                    continue
                w = []
                for j in keys:
                    s = math.fsum(q[b][i][h][c] * k[b][j][g][c] for c in range(d)) * scale
                    if cap > 0:
                        s = cap * math.tanh(s / cap)
                    if slopes is not None:
                        s -= slopes[h] * abs(dk - j)
                    w.append(math.exp(s))
                Z = math.fsum(w)
                for c in range(d):
                    O[b][i][h][c] = math.fsum(wj * v[b][j][g][c] for wj, j in zip(w, keys)) / Z
                lse[b][h][i] = math.log(Z)
    return O, lse
