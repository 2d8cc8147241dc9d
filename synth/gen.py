"""Seeded synthetic workloads for exact attention (dense, varlen, paged decode).

Recipe (stated once, used everywhere):

* Small integer draws (sequence lengths, context lengths, the page permutation)
  come from ``numpy.random.default_rng(seed)`` in the order listed per workload.
* Tensor values are iid standard normals drawn as float32.  Each tensor has a
  fixed id; its flat buffer is cut into chunks of ``CHUNK`` elements and chunk
  ``c`` of tensor ``t`` is drawn by ``PCG64(SeedSequence(seed, spawn_key=(t, c)))``.
  The result therefore does not depend on how many threads draw it.
* bf16 tensors are the float32 draws rounded to nearest-even (RNE) once, here,
  and handed out as raw ``uint16`` bit patterns.  The GPU receives those bits and
  the oracle upcasts the same bits exactly.
* For paged decode the pool has one extra page, id ``num_pages``: block-table
  padding points at it.  In correctness runs it is filled with NaN so any read of
  it poisons the output.

Nothing here performs any step of the attention method.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK = 1 << 22
BF16_NAN = np.uint16(0x7FC0)

# tensor ids (part of the recipe: changing one changes every drawn value)
T_Q, T_K, T_V, T_KCACHE, T_VCACHE, T_DO = 1, 2, 3, 4, 5, 6


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 with round-to-nearest-even; return uint16 bits.

    NaN inputs stay NaN (quiet).  Used only for input preparation.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = BF16_NAN
    return r


def _fill_chunk(seed: int, tid: int, c: int, n: int, out: np.ndarray, as_bf16: bool) -> None:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tid, c))))
    x = g.standard_normal(n, dtype=np.float32)
    if as_bf16:
        out[:] = f32_to_bf16_bits(x)
    else:
        out[:] = x


def normal(seed: int, tid: int, shape, bf16: bool) -> np.ndarray:
    """iid N(0,1) tensor of ``shape``: uint16 bf16 bits if ``bf16`` else float32."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK
    jobs = [(c, c * CHUNK, min(n, (c + 1) * CHUNK)) for c in range(nchunks)]
    if nchunks <= 1:
        for c, a, b in jobs:
            _fill_chunk(seed, tid, c, b - a, out[a:b], bf16)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(lambda j: _fill_chunk(seed, tid, j[0], j[2] - j[1], out[j[1]:j[2]], bf16), jobs))
    return out.reshape(shape)


# --------------------------------------------------------------------------- workloads


@dataclass
class Dense:
    """Q, K, V as [B, H, N, d] (float32 values or bf16 bits)."""
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32" | "bf16"
    causal: bool
    scale: float
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    Nk: int = -1  # key length (defaults to N)

    def __post_init__(self):
        if self.Nk < 0:
            self.Nk = self.N


def dense(B: int, H: int, N: int, d: int, dtype: str = "bf16", causal: bool = False,
          scale: float | None = None, seed: int = 0, Nk: int | None = None,
          H_kv: int | None = None) -> Dense:
    """Q [B, H, N, d]; K, V [B, H_kv, Nk, d] (H_kv defaults to H)."""
    Nk = N if Nk is None else Nk
    H_kv = H if H_kv is None else H_kv
    bf = dtype == "bf16"
    q = normal(seed, T_Q, (B, H, N, d), bf)
    k = normal(seed, T_K, (B, H_kv, Nk, d), bf)
    v = normal(seed, T_V, (B, H_kv, Nk, d), bf)
    return Dense(B, H, N, d, dtype, causal, 1.0 / math.sqrt(d) if scale is None else scale, q, k, v, Nk)


@dataclass
class Varlen:
    """Packed token-major Q [total_q, H, d], K/V [total_k, H, d] (bf16 bits)."""
    H: int
    d: int
    causal: bool
    scale: float
    lens_q: np.ndarray
    lens_k: np.ndarray
    cu_q: np.ndarray  # int32 [S+1]
    cu_k: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray

    @property
    def num_seqs(self) -> int:
        return len(self.lens_q)

    @property
    def max_q(self) -> int:
        return int(self.lens_q.max()) if len(self.lens_q) else 0

    @property
    def max_k(self) -> int:
        return int(self.lens_k.max()) if len(self.lens_k) else 0


def cu_from_lens(lens) -> np.ndarray:
    lens = np.asarray(lens, dtype=np.int64)
    cu = np.zeros(len(lens) + 1, dtype=np.int64)
    np.cumsum(lens, out=cu[1:])
    assert cu[-1] < 2**31
    return cu.astype(np.int32)


def varlen(num_seqs: int = 16, lmin: int = 128, lmax: int = 4096, H: int = 32, d: int = 128,
           causal: bool = True, scale: float | None = None, seed: int = 0,
           lens=None, lens_k=None, H_kv: int | None = None) -> Varlen:
    """Draw order: lengths = rng.integers(lmin, lmax, num_seqs, endpoint=True); then Q, K, V.

    ``lens`` / ``lens_k`` override the drawn lengths (edge-case tests).  K and V carry
    H_kv heads (default H)."""
    H_kv = H if H_kv is None else H_kv
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = rng.integers(lmin, lmax, size=num_seqs, endpoint=True)
    lens = np.asarray(lens, dtype=np.int64)
    lens_k = lens if lens_k is None else np.asarray(lens_k, dtype=np.int64)
    cu_q, cu_k = cu_from_lens(lens), cu_from_lens(lens_k)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    q = normal(seed, T_Q, (tq, H, d), True)
    k = normal(seed, T_K, (tk, H_kv, d), True)
    v = normal(seed, T_V, (tk, H_kv, d), True)
    return Varlen(H, d, causal, 1.0 / math.sqrt(d) if scale is None else scale,
                  lens, lens_k, cu_q, cu_k, q, k, v)


@dataclass
class Paged:
    """Decode batch over a paged KV pool.

    q [B, H, d]; k_cache / v_cache [num_pages + 1, page, H, d]; block_table
    [B, max_pages] int32 padded with the poison page id ``num_pages``;
    context_lens [B] int32.  Values are bf16 bits.
    """
    B: int
    H: int
    d: int
    page: int
    scale: float
    context_lens: np.ndarray
    block_table: np.ndarray
    num_pages: int
    q: np.ndarray
    k_cache: np.ndarray | None = field(repr=False, default=None)
    v_cache: np.ndarray | None = field(repr=False, default=None)

    @property
    def max_pages(self) -> int:
        return self.block_table.shape[1]

    @property
    def pool_pages(self) -> int:
        return self.num_pages + 1


def paged(B: int = 64, H: int = 32, d: int = 128, ctx_min: int = 512, ctx_max: int = 8192,
          page: int = 16, scale: float | None = None, seed: int = 0, poison: bool = True,
          ctx=None, identity: bool = False, with_pool: bool = True, H_kv: int | None = None) -> Paged:
    """Draw order: ctx = rng.integers(ctx_min, ctx_max, B, endpoint=True); then the page
    permutation rng.permutation(num_pages), dealt out to sequences in order; then q,
    k_cache, v_cache.  ``identity`` uses pages 0..n-1 in order instead of the permutation.
    The pools carry H_kv heads (default H)."""
    H_kv = H if H_kv is None else H_kv
    rng = np.random.default_rng(seed)
    if ctx is None:
        ctx = rng.integers(ctx_min, ctx_max, size=B, endpoint=True)
    ctx = np.asarray(ctx, dtype=np.int64)
    B = len(ctx)
    pages_b = (ctx + page - 1) // page
    num_pages = int(pages_b.sum())
    perm = np.arange(num_pages) if identity else rng.permutation(num_pages)
    maxp = max(1, int(pages_b.max()) if B else 1)
    bt = np.full((B, maxp), num_pages, dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(pages_b[b])
        bt[b, :n] = perm[off:off + n]
        off += n
    q = normal(seed, T_Q, (B, H, d), True)
    kc = vc = None
    if with_pool:
        kc = normal(seed, T_KCACHE, (num_pages + 1, page, H_kv, d), True)
        vc = normal(seed, T_VCACHE, (num_pages + 1, page, H_kv, d), True)
        if poison:
            kc[num_pages] = BF16_NAN
            vc[num_pages] = BF16_NAN
            # slots past the context in each sequence's last page are poisoned too
            for b in range(B):
                tail = int(ctx[b] % page)
                if tail and pages_b[b]:
                    p = int(bt[b, pages_b[b] - 1])
                    kc[p, tail:] = BF16_NAN
                    vc[p, tail:] = BF16_NAN
    return Paged(B, H, d, page, 1.0 / math.sqrt(d) if scale is None else scale,
                 ctx.astype(np.int32), bt, num_pages, q, kc, vc)


@dataclass
class PagedPrefill:
    """Paged prefill: new query rows q [sum(lens_q), H, d] of sequences whose keys (the
    cached prefix and the new tokens, lens_k in all) sit in pools [num_pages + 1, page,
    H_kv, d] through block_table [S, max_pages] (padded with the poison page
    num_pages).  Values are bf16 bits."""
    H: int
    H_kv: int
    d: int
    page: int
    causal: bool
    scale: float
    lens_q: np.ndarray
    lens_k: np.ndarray
    cu_q: np.ndarray
    cu_k: np.ndarray
    block_table: np.ndarray
    num_pages: int
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray

    @property
    def max_q(self) -> int:
        return int(self.lens_q.max()) if len(self.lens_q) else 0

    @property
    def max_k(self) -> int:
        return int(self.lens_k.max()) if len(self.lens_k) else 0


def paged_prefill(lens_q, lens_k, H: int = 32, d: int = 128, page: int = 16, causal: bool = True,
                  scale: float | None = None, seed: int = 0, H_kv: int | None = None,
                  poison: bool = True) -> PagedPrefill:
    """Draw order: the page permutation rng.permutation(num_pages) dealt out to the
    sequences in order, then q, k_cache, v_cache.  With ``poison`` the padding page and
    the slots past each sequence's last key are NaN (a kernel that reads them fails)."""
    H_kv = H if H_kv is None else H_kv
    rng = np.random.default_rng(seed)
    lens_q = np.asarray(lens_q, dtype=np.int64)
    lens_k = np.asarray(lens_k, dtype=np.int64)
    pages_b = (lens_k + page - 1) // page
    num_pages = int(pages_b.sum())
    perm = rng.permutation(num_pages)
    maxp = max(1, int(pages_b.max()) if len(pages_b) else 1)
    bt = np.full((len(lens_k), maxp), num_pages, dtype=np.int32)
    off = 0
    for s_, n in enumerate(pages_b):
        bt[s_, :int(n)] = perm[off:off + int(n)]
        off += int(n)
    cu_q, cu_k = cu_from_lens(lens_q), cu_from_lens(lens_k)
    q = normal(seed, T_Q, (int(cu_q[-1]), H, d), True)
    kc = normal(seed, T_KCACHE, (num_pages + 1, page, H_kv, d), True)
    vc = normal(seed, T_VCACHE, (num_pages + 1, page, H_kv, d), True)
    if poison:
        kc[num_pages] = BF16_NAN
        vc[num_pages] = BF16_NAN
        for s_, L in enumerate(lens_k):
            tail = int(L % page)
            if tail:
                pg = int(bt[s_, pages_b[s_] - 1])
                kc[pg, tail:] = BF16_NAN
                vc[pg, tail:] = BF16_NAN
    return PagedPrefill(H, H_kv, d, page, causal, 1.0 / math.sqrt(d) if scale is None else scale,
                        lens_q, lens_k, cu_q, cu_k, bt, num_pages, q, kc, vc)


@dataclass
class KVStore:
    """New K/V rows [T, H_kv, d] (bf16 bits) to be written into pools [P, page, H_kv, d]
    through slot_mapping int64 [T] (slot = page * page_size + offset, -1 = padding)."""
    T: int
    H_kv: int
    d: int
    page: int
    num_pages: int
    k: np.ndarray
    v: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    slot_mapping: np.ndarray


def kvstore(lens, H_kv: int = 32, d: int = 128, page: int = 16, extra_pages: int = 0, pad: int = 0,
            seed: int = 0) -> KVStore:
    """Tokens of sequences with lengths ``lens`` laid out page by page: draw order is
    the page permutation rng.permutation(num_pages) dealt out to sequences in order
    (as for the decode pools), then ``pad`` padding positions rng.choice(T + pad, pad)
    whose slot is -1, then K, V and the two pools (random bits of the old contents)."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    pages_b = (lens + page - 1) // page
    used = int(pages_b.sum())
    num_pages = used + extra_pages
    perm = rng.permutation(num_pages)
    slots = []
    off = 0
    for L, n in zip(lens, pages_b):
        pg = perm[off:off + int(n)]
        off += int(n)
        t = np.arange(int(L))
        slots.append(pg[t // page] * page + t % page)
    slots = np.concatenate(slots) if slots else np.zeros(0, dtype=np.int64)
    T = len(slots) + pad
    if pad:
        where = np.sort(rng.choice(T, size=pad, replace=False))
        full = np.full(T, -1, dtype=np.int64)
        keep = np.ones(T, dtype=bool)
        keep[where] = False
        full[keep] = slots
        slots = full
    k = normal(seed, T_K, (T, H_kv, d), True)
    v = normal(seed, T_V, (T, H_kv, d), True)
    kc = normal(seed, T_KCACHE, (num_pages, page, H_kv, d), True)
    vc = normal(seed, T_VCACHE, (num_pages, page, H_kv, d), True)
    return KVStore(T, H_kv, d, page, num_pages, k, v, kc, vc, slots.astype(np.int64))


# --------------------------------------------------------------------------- named workloads

HAND_Q = np.array([[1, 0, 2], [0, 1, 1]], dtype=np.float32)
HAND_K = np.array([[2, 1, 0], [1, 1, 2]], dtype=np.float32)
HAND_V = np.array([[1, 0, 1], [0, 2, 1]], dtype=np.float32)

WORKLOADS = {
    "c1": "single-head fp32 B=1 H=1 N=256 d=64 non-causal, scale 1/8",
    "c2": "batched MHA bf16 B=4 H=16 N=2048 d=128 non-causal",
    "c3": "long causal bf16 B=1 H=32 N=8192 d=128",
    "c4": "varlen causal bf16 16 seqs len U[128,4096] H=32 d=128",
    "c5": "paged decode bf16 64 seqs ctx U[512,8192] H=32 d=128 page 16",
    "gqa_decode": "paged decode bf16 64 seqs ctx U[512,8192] H=16 H_kv=8 d=128 page 16 "
                  "(the page's 16-query-head / 8-KV-head model shape)",
    "store_prefill": "store_kvcache of a prefill batch: the 16 varlen lengths (34069 tokens), "
                     "H_kv=32 d=128 bf16, 16-token pages in a random page order",
    "prefill_paged": "paged prefill: the 16 varlen lengths as contexts in 16-token pages, the "
                     "second half of each (ceil(L/2) tokens) as new causal query rows, H=32 d=128",
}


def workload(name: str, seed: int = 0, **kw):
    if name == "c1":
        return dense(1, 1, 256, 64, "f32", False, seed=seed)
    if name == "c2":
        return dense(4, 16, 2048, 128, "bf16", False, seed=seed)
    if name == "c3":
        return dense(1, 32, 8192, 128, "bf16", True, seed=seed)
    if name == "c4":
        return varlen(16, 128, 4096, 32, 128, True, seed=seed)
    if name == "c5":
        return paged(64, 32, 128, 512, 8192, 16, seed=seed, **kw)
    if name == "gqa_decode":
        return paged(64, 16, 128, 512, 8192, 16, seed=seed, H_kv=8, **kw)
    if name == "prefill_paged":
        lens = np.random.default_rng(seed).integers(128, 4096, size=16, endpoint=True)
        return paged_prefill((lens + 1) // 2, lens, 32, 128, 16, True, seed=seed, **kw)
    if name == "store_prefill":
        lens = np.random.default_rng(seed).integers(128, 4096, size=16, endpoint=True)
        return kvstore(lens, 32, 128, 16, seed=seed)
    raise KeyError(name)
