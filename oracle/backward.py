"""Gradients of exact attention in float64 (the oracle for the backward pass).
TEST INFRASTRUCTURE.

What is differentiated: O = softmax(scale * Q K^T) V row-wise, with the causal mask of
the forward oracle (key j admissible for row i iff j <= i + (Lk - Lq)).  Given dO, the
chain rule through the softmax gives, with P the probabilities:

    dV = P^T dO,   dP = dO V^T,   D_i = sum_j P_ij dP_ij = dO_i . O_i,
    dS = P * (dP - D),   dQ = scale * dS K,   dK = scale * dS^T Q.

The pages describe the backward as recomputing S and P from the forward's stored
statistics and dO, subtracting the row sums in dS, and keeping dQ in registers rather
than adding it atomically (m.lqnn.cn FlashAttention article, section 4.3 and the
pitfall list of section 6.4; "L2.5 SOTA Kernel", yulong.wang, section 2.3: P is
recomputed from the O(N) logsumexp).  Here P is formed by the plain two-pass softmax,
not from a stored statistic, so the oracle does not depend on the forward kernel.

Grouped-query attention: the gradient of a KV head sums the contributions of every
query head that reads it (query head h reads KV head h // (H / H_kv)).

`o` (optional): the forward output the backward is handed, as the GPU entry points take
it.  Then D_i is formed as dO_i . O_i from that O (the same row sum; the pages form it
from the stored O), so that a kernel fed a rounded (bf16) O is compared against the
gradient of the same inputs.  Without `o`, D_i comes from P and dP (exact O).
"""
from __future__ import annotations

import numpy as np

from .attention import _as_f64, kv_head, probabilities


def attention_backward_rows(q, k, v, do, scale: float, causal: bool = False, o=None):
    """One head: q [Lq, d], k [Lk, d], v [Lk, dv], do [Lq, dv] (floats or bf16 bits);
    o [Lq, dv] or None (see the module note).  Returns (dq [Lq, d], dk [Lk, d],
    dv [Lk, dv]) in float64."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    lq, lk = q.shape[0], k.shape[0]
    if lq == 0 or lk == 0:
        return np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    p = probabilities(q, k, scale, causal)          # rows without keys are all zero
    dv = p.T @ do
    dp = do @ v.T
    if o is None:
        dsum = (p * dp).sum(axis=1, keepdims=True)  # D_i
    else:
        dsum = (do * _as_f64(o)).sum(axis=1, keepdims=True)  # D_i = dO_i . O_i, the given O
    ds = p * (dp - dsum)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attention_backward_dense(q, k, v, do, scale: float, causal: bool = False, o=None):
    """Q, dO [B, H, N, d]; K, V [B, H_kv, Nk, d]; O as dO or None.  Returns dQ [B, H, N, d]
    and dK, dV [B, H_kv, Nk, d] in float64 (KV-head gradients summed over their group)."""
    B, H, N, d = q.shape
    H_kv, Nk = k.shape[1], k.shape[2]
    dq = np.zeros((B, H, N, d))
    dk = np.zeros((B, H_kv, Nk, d))
    dv = np.zeros((B, H_kv, Nk, v.shape[3]))
    for b in range(B):
        for h in range(H):
            hk = kv_head(h, H, H_kv)
            a, bk, bv = attention_backward_rows(q[b, h], k[b, hk], v[b, hk], do[b, h], scale, causal,
                                                None if o is None else o[b, h])
            dq[b, h] = a
            dk[b, hk] += bk
            dv[b, hk] += bv
    return dq, dk, dv


def attention_backward_varlen(q, k, v, do, cu_q, cu_k, scale: float, causal: bool = False, o=None):
    """Variable-length packed batch ("From standard Attention to FlashAttention and paged
    execution", section 3.3: sequence s owns rows [cu_q[s], cu_q[s+1]) of Q, dO
    [total_q, H, d] and [cu_k[s], cu_k[s+1]) of K, V [total_k, H_kv, d]; each sequence
    attends independently, causal bottom-right aligned).  The gradient of the packed
    batch is each sequence's gradient in its own rows; rows outside every sequence get
    zero.  O as dO or None.  Returns dQ [total_q, H, d], dK, dV [total_k, H_kv, d] in
    float64."""
    tq, H, d = q.shape
    tk, H_kv = k.shape[0], k.shape[1]
    dq = np.zeros((tq, H, d))
    dk = np.zeros((tk, H_kv, d))
    dv = np.zeros((tk, H_kv, v.shape[2]))
    for s in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[s]), int(cu_q[s + 1])
        k0, k1 = int(cu_k[s]), int(cu_k[s + 1])
        for h in range(H):
            hk = kv_head(h, H, H_kv)
            a, bk, bv = attention_backward_rows(q[q0:q1, h], k[k0:k1, hk], v[k0:k1, hk], do[q0:q1, h], scale, causal,
                                                None if o is None else o[q0:q1, h])
            dq[q0:q1, h] = a
            dk[k0:k1, hk] += bk
            dv[k0:k1, hk] += bv
    return dq, dk, dv
