"""Plain two-pass exact attention in float64 (the oracle).  TEST INFRASTRUCTURE.

Definition followed: Attention(Q, K, V) = softmax(Q K^T * scale) V, row-wise
softmax over keys ("From standard Attention to FlashAttention and paged
execution", dlog.com.cn, section "the memory bottleneck of standard attention";
the 1/sqrt(d) scale is the one in that section's code, passed explicitly here
because the page's worked example of section 2.1 omits it).  The per-row
logsumexp is the statistic the tiled forward writes next to O ("L2.5 SOTA
Kernel", yulong.wang, sections 2.1 and 2.3).

Readings where the pages are silent:

* causal mask: key j is admissible for query row i iff j <= i + (Lk - Lq)
  (bottom-right alignment; j <= i when Lq == Lk);
* a row with no admissible key has O = 0 and lse = -inf;
* lse = m + ln(l), natural log, in units of the scaled score;
* keys past a sequence's end simply do not exist (never a zero-filled key).

Grouped-query attention ("From standard Attention to FlashAttention and paged
execution", section "GQA: handled natively by the kernel, K/V not expanded"): K/V
hold H_kv heads, H_kv divides H, and query head h uses KV head h // (H // H_kv) --
the head order the page's explicit expansion of each KV head into H // H_kv copies
produces.

Rows are independent (dlog.com.cn, section 2.1), so computing a chunk of rows at
a time is exact; it only bounds memory.
"""
from __future__ import annotations

import numpy as np

NEG_INF = float("-inf")


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns (uint16) to float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _as_f64(x: np.ndarray) -> np.ndarray:
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return np.asarray(x, dtype=np.float64)


def attention_rows(q, k, v, scale: float, causal: bool = False, row_chunk: int = 512,
                   rows=None):
    """Exact attention for one head.

    q [Lq, d], k [Lk, d], v [Lk, dv] (float arrays or bf16 bits).  Returns
    (O [n, dv] float64, lse [n] float64) for query rows ``rows`` (default all).

    Pass 1: m_i = max_j s_ij.  Pass 2: P_ij = exp(s_ij - m_i), l_i = sum_j P_ij,
    O_i = sum_j P_ij v_j / l_i, lse_i = m_i + ln l_i.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    lq, lk = q.shape[0], k.shape[0]
    rows = np.arange(lq) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((len(rows), v.shape[1]), dtype=np.float64)
    lse = np.full(len(rows), NEG_INF, dtype=np.float64)
    if lk == 0 or len(rows) == 0:
        return o, lse
    for a in range(0, len(rows), row_chunk):
        r = rows[a:a + row_chunk]
        # under a causal mask no row of this chunk sees keys past the last row's limit
        kmax = lk if not causal else int(min(lk, max(0, r.max() + (lk - lq) + 1)))
        if kmax <= 0:
            continue
        s = (q[r] @ k[:kmax].T) * scale
        if causal:
            # admissible iff j <= i + (Lk - Lq)
            s = np.where(np.arange(kmax)[None, :] <= (r[:, None] + (lk - lq)), s, NEG_INF)
        m = s.max(axis=1)                                  # pass 1
        has = np.isfinite(m)
        m_safe = np.where(has, m, 0.0)
        p = np.exp(s - m_safe[:, None])                    # pass 2 (exp(-inf) = 0)
        l = p.sum(axis=1)
        pv = p @ v[:kmax]
        with np.errstate(divide="ignore", invalid="ignore"):
            o[a:a + len(r)] = np.where(has[:, None], pv / np.where(has, l, 1.0)[:, None], 0.0)
            lse[a:a + len(r)] = np.where(has, m_safe + np.log(np.where(has, l, 1.0)), NEG_INF)
    return o, lse


def probabilities(q, k, scale: float, causal: bool = False) -> np.ndarray:
    """Debug hook for tiny inputs: the full softmax matrix P [Lq, Lk] (two-pass)."""
    q, k = _as_f64(q), _as_f64(k)
    lq, lk = q.shape[0], k.shape[0]
    s = (q @ k.T) * scale
    if causal:
        s = np.where(np.arange(lk)[None, :] <= (np.arange(lq)[:, None] + (lk - lq)), s, NEG_INF)
    m = s.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(l > 0, p / np.where(l > 0, l, 1.0), 0.0)


def kv_head(h: int, H: int, H_kv: int) -> int:
    """KV head read by query head h under grouped-query attention (H_kv divides H)."""
    if H_kv < 1 or H % H_kv != 0:
        raise ValueError(f"H_kv={H_kv} must divide H={H}")
    return h // (H // H_kv)


def attention_dense(q, k, v, scale: float, causal: bool = False, heads=None, rows=None):
    """Dense batched attention, Q [B, H, N, d], K/V [B, H_kv, Nk, d] (the [B, H, N, d]
    layout of the pages' Triton kernels; H_kv = H unless grouped-query).  Returns
    O [B, H, N, d] and lse [B, H, N] float64.  ``heads`` restricts to a list of (b, h)
    pairs (the other entries stay NaN); ``rows`` restricts the query rows (same for
    each head)."""
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    dv = v.shape[3]
    o = np.full((B, H, N, dv), np.nan)
    lse = np.full((B, H, N), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in pairs:
        hk = kv_head(h, H, H_kv)
        ob, lb = attention_rows(q[b, h], k[b, hk], v[b, hk], scale, causal, rows=rows)
        if rows is None:
            o[b, h], lse[b, h] = ob, lb
        else:
            o[b, h, rows], lse[b, h, rows] = ob, lb
    return o, lse


def attention_varlen(q, k, v, cu_q, cu_k, scale: float, causal: bool = False, seqs=None,
                     heads=None, rows_per_seq=None):
    """Variable-length packed attention ("From standard Attention to FlashAttention
    and paged execution", section 3.3): tokens of all sequences are flattened to
    Q [total_q, H, d] and K/V [total_k, H, d]; sequence s owns rows
    [cu_q[s], cu_q[s+1]) of Q and [cu_k[s], cu_k[s+1]) of K/V (the page's example
    cu_seqlens [0, 3, 7] means ranges [0,3) and [3,7)).  Each sequence is attended
    independently.  K/V may hold fewer (grouped-query) heads.  Returns
    O [total_q, H, d], lse [total_q, H] (NaN where not computed when restricted by
    ``seqs``/``heads``/``rows_per_seq``)."""
    tq, H, d = q.shape
    H_kv = k.shape[1]
    dv = v.shape[2]
    o = np.full((tq, H, dv), np.nan)
    lse = np.full((tq, H), np.nan)
    S = len(cu_q) - 1
    seqs = range(S) if seqs is None else seqs
    heads = range(H) if heads is None else heads
    for s in seqs:
        q0, q1 = int(cu_q[s]), int(cu_q[s + 1])
        k0, k1 = int(cu_k[s]), int(cu_k[s + 1])
        rows = None
        if rows_per_seq is not None:
            rows = np.asarray(rows_per_seq(s, q1 - q0), dtype=np.int64)
        for h in heads:
            hk = kv_head(h, H, H_kv)
            ob, lb = attention_rows(q[q0:q1, h], k[k0:k1, hk], v[k0:k1, hk], scale, causal,
                                    rows=rows)
            if rows is None:
                o[q0:q1, h], lse[q0:q1, h] = ob, lb
            else:
                o[q0 + rows, h], lse[q0 + rows, h] = ob, lb
    return o, lse


def gather_paged(cache, block_table_row, ctx: int, page: int):
    """Contiguous [ctx, ...] copy of one sequence's cached keys (or values): token t
    lives in physical page block_table[t // page], slot t % page ("From standard
    Attention to FlashAttention and paged execution", sections "PagedAttention" and
    "the two functions v3 calls")."""
    n = (ctx + page - 1) // page
    pages = np.asarray(block_table_row[:n], dtype=np.int64)
    g = cache[pages]  # [n, page, ...]
    return g.reshape(n * page, *cache.shape[2:])[:ctx]


def attention_decode_paged(q, k_cache, v_cache, block_table, context_lens, scale: float,
                           seqs=None, heads=None):
    """Decode over a paged KV cache: sequence b's single query q[b] [H, d] attends
    its context_lens[b] cached tokens, gathered through block_table[b] (page size =
    k_cache.shape[1]).  With one query token, bottom-right causal and non-causal
    coincide.  The pools hold H_kv (grouped-query) heads: [pages, page, H_kv, d].
    Returns O [B, H, d], lse [B, H] (NaN where not computed)."""
    B, H, d = q.shape
    H_kv = k_cache.shape[2]
    page = k_cache.shape[1]
    dv = v_cache.shape[3]
    o = np.full((B, H, dv), np.nan)
    lse = np.full((B, H), np.nan)
    seqs = range(B) if seqs is None else seqs
    heads = list(range(H)) if heads is None else list(heads)
    for b in seqs:
        ctx = int(context_lens[b])
        for h in heads:
            # gather one head at a time: [ctx, d] instead of [ctx, H, d]
            hk = kv_head(h, H, H_kv)
            kb = gather_paged(k_cache[:, :, hk], block_table[b], ctx, page)
            vb = gather_paged(v_cache[:, :, hk], block_table[b], ctx, page)
            ob, lb = attention_rows(q[b, h][None, :], kb, vb, scale, False)
            o[b, h], lse[b, h] = ob[0], lb[0]
    return o, lse


def store_kvcache(k, v, k_cache, v_cache, slot_mapping):
    """Write one step's new K/V rows into the paged pools ("From standard Attention to
    FlashAttention and paged execution", the attention step of the v3 engine: the
    step's k/v are first written into the paged KV cache through slot_mapping, every
    step, prefill and decode alike).  k, v [T, H_kv, d]; pools [pages, page, H_kv, d].
    Reading where the page is silent: slot_mapping[t] is the flat slot
    page * page_size + offset of token t's row; a slot outside [0, pages * page) (for
    instance -1, padding) is skipped.  Returns new pool arrays; the inputs are not
    modified."""
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    pages, page = kc.shape[0], kc.shape[1]
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if 0 <= slot < pages * page:
            kc[slot // page, slot % page] = k[t]
            vc[slot // page, slot % page] = v[t]
    return kc, vc


def attention_varlen_paged(q, k_cache, v_cache, cu_q, cu_k, block_table, scale: float,
                           causal: bool = False, seqs=None, heads=None, rows_per_seq=None):
    """Variable-length attention whose keys and values live in the paged pools (paged
    prefill: "From standard Attention to FlashAttention and paged execution", the
    prefill entry of the v3 engine: a continued chunk passes the KV cache and its
    block_table to the varlen function, with cu_seqlens_q != cu_seqlens_k).
    Sequence s has Lq = cu_q[s+1] - cu_q[s] new query rows and Lk = cu_k[s+1] - cu_k[s]
    keys; key j is token j of the sequence, in page block_table[s][j // page], slot
    j % page (the pools [pages, page, H_kv, d]).  Under the causal mask the query rows
    are the last Lq tokens (bottom-right).  Returns O [total_q, H, d], lse [total_q, H]."""
    tq, H, d = q.shape
    H_kv = k_cache.shape[2]
    page = k_cache.shape[1]
    dv = v_cache.shape[3]
    o = np.full((tq, H, dv), np.nan)
    lse = np.full((tq, H), np.nan)
    S = len(cu_q) - 1
    seqs = range(S) if seqs is None else seqs
    heads = range(H) if heads is None else heads
    for s in seqs:
        q0, q1 = int(cu_q[s]), int(cu_q[s + 1])
        lk = int(cu_k[s + 1]) - int(cu_k[s])
        rows = None
        if rows_per_seq is not None:
            rows = np.asarray(rows_per_seq(s, q1 - q0), dtype=np.int64)
        for h in heads:
            hk = kv_head(h, H, H_kv)
            kb = gather_paged(k_cache[:, :, hk], block_table[s], lk, page)
            vb = gather_paged(v_cache[:, :, hk], block_table[s], lk, page)
            ob, lb = attention_rows(q[q0:q1, h], kb, vb, scale, causal, rows=rows)
            if rows is None:
                o[q0:q1, h], lse[q0:q1, h] = ob, lb
            else:
                o[q0 + rows, h], lse[q0 + rows, h] = ob, lb
    return o, lse
