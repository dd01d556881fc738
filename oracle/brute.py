"""Brute-force attention in pure Python -- TEST INFRASTRUCTURE ONLY.

An independent formulation of the same definition, for tiny shapes only:
every output element is computed on its own as

    o[b,h,i,c] = fsum_j exp(s_ij) * v[j,c]  /  fsum_j exp(s_ij)

with exactly rounded sums (math.fsum) and no max subtraction, so it shares
neither code nor numerical structure with the C oracle (which subtracts the row
max, normalises the probabilities first and accumulates in index order).
Scores must stay small enough for exp() not to overflow, which holds for the
tiny N(0,1) inputs it is used on.
"""
from __future__ import annotations

import math


def attention(q, k, v, scale, causal):
    """q: nested lists [B][Hq][Sq][d]; k, v: [B][Hkv][Skv][d]. Returns o as nested lists."""
    B = len(q)
    Hq = len(q[0])
    Sq = len(q[0][0])
    d = len(q[0][0][0])
    Hkv = len(k[0])
    Skv = len(k[0][0])
    out = []
    for b in range(B):
        ob = []
        for h in range(Hq):
            g = (h * Hkv) // Hq
            oh = []
            for i in range(Sq):
                last = i + Skv - Sq if causal else Skv - 1
                keys = range(0, last + 1)
                w = [math.exp(scale * math.fsum(q[b][h][i][c] * k[b][g][j][c] for c in range(d))) for j in keys]
                den = math.fsum(w)
                row = []
                for c in range(d):
                    num = math.fsum(w[t] * v[b][g][j][c] for t, j in enumerate(keys))
                    row.append(num / den if w else 0.0)
                oh.append(row)
            ob.append(oh)
        out.append(ob)
    return out
