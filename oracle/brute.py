"""Pure-Python scalar attention for tiny shapes — TEST INFRASTRUCTURE ONLY.

The textbook definition (FlashAttention interview canvas, panel 1, "standard
attention" box) written as nested loops over Python floats, with math.exp and
math.fsum (correctly rounded sums), so it shares nothing with the numpy oracle
it pins.  Causal reading: key j visible from row i iff j <= i + Sk - Sq.
"""

from __future__ import annotations

import math


def attention_brute(q, k, v, causal=False, scale=None):
    """q [B][Hq][Sq][d], k/v [B][Hkv][Sk][d] as nested lists (or anything that
    indexes like them and yields floats).  Returns (O, LSE) as nested lists."""
    B = len(q)
    Hq = len(q[0])
    Sq = len(q[0][0])
    d = len(q[0][0][0])
    Hkv = len(k[0])
    Sk = len(k[0][0])
    dv = len(v[0][0][0])
    G = Hq // Hkv
    tau = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = []
    lses = []
    for b in range(B):
        ob, lb = [], []
        for h in range(Hq):
            kh = k[b][h // G]
            vh = v[b][h // G]
            oh, lh = [], []
            for i in range(Sq):
                last = i + Sk - Sq if causal else Sk - 1
                js = [j for j in range(Sk) if j <= last]
                if not js:
                    oh.append([0.0] * dv)
                    lh.append(-math.inf)
                    continue
                s = [tau * math.fsum(float(q[b][h][i][c]) * float(kh[j][c]) for c in range(d))
                     for j in js]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                l = math.fsum(e)
                row = [math.fsum(e[n] * float(vh[j][c]) for n, j in enumerate(js)) / l
                       for c in range(dv)]
                oh.append(row)
                lh.append(m + math.log(l))
            ob.append(oh)
            lb.append(lh)
        out.append(ob)
        lses.append(lb)
    return out, lses
