"""Tiled online-softmax attention on the CPU in float64.  TEST INFRASTRUCTURE.

This is the recurrence of "From standard Attention to FlashAttention and paged
execution" (dlog.com.cn), section 2.2 (online softmax), restated: each query row
keeps a running max m, a running sum l and an unnormalised output o; for every
key block the old l and o are rescaled by exp(m - m_new) and the block's
exp(s - m_new) terms are added; at the end o / l is the output.  The -inf start
value of m and the rule that exp(m - m_new) is 0 (not NaN) while m is still -inf
follow the troubleshooting section 5.1 of the m.lqnn.cn FlashAttention article.

It exists only to pin the two-pass oracle (``attention.py``) against an
independent algorithm, including the per-block (m, l) trace printed in section
2.3 of the dlog.com.cn page.  Scalar loops: tiny inputs only.
"""
from __future__ import annotations

import math

import numpy as np


def online_attention(q, k, v, scale: float, block: int, causal: bool = False, trace: bool = False):
    """q [Lq, d], k [Lk, d], v [Lk, dv] float64.  Returns (O, lse[, trace]) where trace
    [row] is the list of (m, l) after each key block."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lq, lk = q.shape[0], k.shape[0]
    dv = v.shape[1]
    out = np.zeros((lq, dv))
    lse = np.full(lq, -math.inf)
    tr = []
    for i in range(lq):
        m = -math.inf
        l = 0.0
        o = [0.0] * dv
        row_trace = []
        for j0 in range(0, lk, block):
            s = []
            for j in range(j0, min(lk, j0 + block)):
                if causal and j > i + (lk - lq):
                    s.append(-math.inf)
                else:
                    s.append(scale * sum(q[i, c] * k[j, c] for c in range(q.shape[1])))
            m_new = max([m] + s)
            if m_new == -math.inf:          # nothing admissible yet: state stays (−inf, 0, 0)
                row_trace.append((m, l))
                continue
            alpha = 0.0 if m == -math.inf else math.exp(m - m_new)
            p = [0.0 if x == -math.inf else math.exp(x - m_new) for x in s]
            l = l * alpha + sum(p)
            for c in range(dv):
                o[c] = o[c] * alpha + sum(p[t] * v[j0 + t, c] for t in range(len(p)))
            m = m_new
            row_trace.append((m, l))
        if l > 0:
            out[i] = [x / l for x in o]
            lse[i] = m + math.log(l)
        tr.append(row_trace)
    if trace:
        return out, lse, tr
    return out, lse
