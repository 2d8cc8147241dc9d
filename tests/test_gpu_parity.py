"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle on the same
seeded inputs, element by element.  bf16 runs feed the oracle the same bf16 values.

Small shapes are compared everywhere.  The five workloads (and the paged-prefill and
grouped-query decode workloads the bench also times) are compared in full: every
output element of every (batch, head) pair, in the launch configuration the bench
times.  Only the 65536-row causal sequence is compared on sampled rows.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from tests.golden.load import load
from tests.util import TOL_BF16_LSE, TOL_BF16_O, TOL_F32, assert_close, dev, host, max_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    import torch
    import exact_attention_attn_amd as attn
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    attn.load()
    return attn


def run_dense(A, w, causal=None, layout="bhnd"):
    import torch
    causal = w.causal if causal is None else causal
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    if layout == "bnhd":   # same values, [B, N, H, d] memory order through strides
        q = q.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        k = k.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        v = v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    o, lse = A.attn_fwd(q, k, v, scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    return host(o), host(lse)


def tol(w):
    return (TOL_F32, TOL_F32) if w.dtype == "f32" else (TOL_BF16_O, TOL_BF16_LSE)


# ------------------------------------------------------------------ page examples

def test_hand_example_fp32(A):
    """The dlog.com.cn section 2.1 example (N=2, d=3, scale 1), zero-padded to d=64:
    zero columns change neither the scores nor O[:, :3]."""
    import torch
    g = load("hand_example.txt")
    pad = lambda x: np.pad(x, ((0, 0), (0, 61))).astype(np.float32)[None, None]
    q, k, v = (dev(pad(g[n])) for n in "QKV")
    o, lse = A.attn_fwd(q, k, v, scale=1.0)
    torch.cuda.synchronize()
    e3, e2 = math.exp(3), math.exp(2)
    P = np.array([[1 / (1 + e3), e3 / (1 + e3)], [1 / (1 + e2), e2 / (1 + e2)]])
    assert_close("O", host(o)[0, 0, :, :3], P @ g["V"], TOL_F32)
    assert np.all(host(o)[0, 0, :, 3:] == 0)
    assert_close("lse", host(lse)[0, 0], np.array([5 + math.log1p(math.exp(-3)), 3 + math.log1p(math.exp(-2))]), TOL_F32)


# ------------------------------------------------------------------ full workloads

def test_c1_fp32_full(A):
    w = synth.workload("c1")
    o, lse = run_dense(A, w)
    ro, rl = oracle.attention_dense(w.q, w.k, w.v, w.scale, w.causal)
    assert_close("O", o, ro, TOL_F32)
    assert_close("lse", lse, rl, TOL_F32)


def _dense_sampled(A, w, pairs, rows):
    o, lse = run_dense(A, w)
    ro, rl = oracle.attention_dense(w.q, w.k, w.v, w.scale, w.causal, heads=pairs, rows=rows)
    to, tl = tol(w)
    assert_close("O", o, ro, to)
    assert_close("lse", lse, rl, tl)
    return o, lse


def _rows(N, rng, extra=48):
    fixed = [0, 1, 2, 31, 32, 63, 64, 127, 128, 129, 255, 256, N // 2, N - 129, N - 128, N - 65, N - 64, N - 2, N - 1]
    r = set(x for x in fixed if 0 <= x < N) | set(rng.integers(0, N, extra).tolist())
    return np.array(sorted(r))


def test_c2_bf16_full(A):
    """Batched 4 x 16 x 2048 x 128 non-causal: all 64 (b, h) pairs, every row."""
    w = synth.workload("c2")
    o, lse = run_dense(A, w)
    ro, rl = oracle.attention_dense(w.q, w.k, w.v, w.scale, w.causal)
    assert_close("O", o, ro, TOL_BF16_O)
    assert_close("lse", lse, rl, TOL_BF16_LSE)


def test_c3_bf16_causal_full(A):
    """Causal 1 x 32 x 8192 x 128 (the headline workload): all 32 heads, every row."""
    w = synth.workload("c3")
    o, lse = run_dense(A, w)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    ro, rl = oracle.attention_dense(w.q, w.k, w.v, w.scale, w.causal)
    assert_close("O", o, ro, TOL_BF16_O)
    assert_close("lse", lse, rl, TOL_BF16_LSE)


def test_dense_long_sequence_sampled(A):
    """The longest dense sequence tested: causal N = 65536 (1024 key tiles for the last
    row block), sampled rows including the last ones."""
    w = synth.dense(B=1, H=2, N=65536, d=128, causal=True, seed=95)
    rng = np.random.default_rng(105)
    o, lse = _dense_sampled(A, w, [(0, 0), (0, 1)], _rows(w.N, rng, 16))
    assert np.isfinite(o).all() and np.isfinite(lse).all()


def test_c4_varlen_full(A):
    """16 packed causal sequences (34069 tokens, H = 32): every sequence, head and row."""
    import torch
    w = synth.workload("c4")
    o, lse = A.attn_fwd_varlen(dev(w.q), dev(w.k), dev(w.v), dev(w.cu_q), dev(w.cu_k), w.max_q, w.max_k,
                               scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    ro, rl = oracle.attention_varlen(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal)
    assert_close("O", o, ro, TOL_BF16_O)
    assert_close("lse", lse, rl, TOL_BF16_LSE)


@pytest.mark.parametrize("d", [64, 128])
def test_varlen_long_causal_sampled(A, d):
    """A causal varlen batch whose longest sequence exceeds 4096 rows: the 64-key tile
    configuration of the varlen entry (shorter batches take 32-key tiles)."""
    import torch
    w = synth.varlen(H=2, d=d, causal=True, seed=90 + d, lens=[4100, 300, 5003], lens_k=[4100, 301, 5003])
    o, lse = A.attn_fwd_varlen(dev(w.q), dev(w.k), dev(w.v), dev(w.cu_q), dev(w.cu_k), w.max_q, w.max_k,
                               scale=w.scale, causal=True)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    rng = np.random.default_rng(104)
    ro, rl = oracle.attention_varlen(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, True,
                                     rows_per_seq=lambda s, L: _rows(L, rng, 24))
    assert_close("O", o, ro, TOL_BF16_O)
    assert_close("lse", lse, rl, TOL_BF16_LSE)


def test_c5_decode_full(A):
    """64 sequences over the paged pool (NaN poison page and tail slots): every
    sequence and head."""
    import torch
    w = synth.workload("c5")
    o, lse = A.attn_decode_paged(dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_table),
                                 dev(w.context_lens), int(w.context_lens.max()), scale=w.scale)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    assert np.isfinite(o).all() and np.isfinite(lse).all()   # no NaN page or tail slot was read
    ro, rl = oracle.attention_decode_paged(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, w.scale)
    assert_close("O", o, ro, TOL_BF16_O)
    assert_close("lse", lse, rl, TOL_BF16_LSE)


# ------------------------------------------------------------------ edge cases, small shapes

@pytest.mark.parametrize("N,Nk,causal", [(1, 1, False), (1, 1, True), (2, 2, True), (63, 63, True),
                                         (65, 65, False), (129, 129, True), (200, 200, True),
                                         (300, 300, False), (513, 513, True), (77, 300, True),
                                         (300, 77, True), (300, 77, False), (128, 1, False),
                                         (5, 1000, True)])
@pytest.mark.parametrize("d", [64, 128])
def test_dense_ragged_bf16(A, N, Nk, causal, d):
    w = synth.dense(2, 3, N, d, "bf16", causal, seed=N * 7 + Nk, Nk=Nk)
    o, lse = run_dense(A, w)
    ro, rl = oracle.attention_dense(w.q, w.k, w.v, w.scale, causal)
    assert_close("O", o, ro, TOL_BF16_O)
    assert_close("lse", lse, rl, TOL_BF16_LSE)


@pytest.mark.parametrize("N,Nk,causal,d", [(1, 1, False, 64), (100, 100, True, 64), (130, 70, True, 128),
                                           (70, 130, True, 128), (257, 257, False, 128),
                                           # several key tiles per wavefront of the fp32 kernel
                                           (300, 1100, True, 64), (1000, 1000, False, 64)])
def test_dense_ragged_fp32(A, N, Nk, causal, d):
    w = synth.dense(2, 2, N, d, "f32", causal, seed=N + 3 * Nk, Nk=Nk)
    o, lse = run_dense(A, w)
    ro, rl = oracle.attention_dense(w.q, w.k, w.v, w.scale, causal)
    assert_close("O", o, ro, TOL_F32)
    assert_close("lse", lse, rl, TOL_F32)


@pytest.mark.parametrize("N,Nk,causal,d", [(100, 77, False, 64), (100, 77, True, 128), (33, 200, True, 64),
                                           (1, 1, False, 128), (130, 300, False, 128)])
def test_dense_tail_poison(A, N, Nk, causal, d):
    """K/V rows past Nk hold NaN in the same allocation (the tensors passed are views of
    larger buffers): no such row may reach the output."""
    import torch
    w = synth.dense(1, 2, N, d, "bf16", causal, seed=N + Nk + d, Nk=Nk)
    q = dev(w.q)
    pad = 64
    kb = torch.full((1, 2, Nk + pad, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    vb = torch.full((1, 2, Nk + pad, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    kb[:, :, :Nk] = dev(w.k)
    vb[:, :, :Nk] = dev(w.v)
    o, lse = A.attn_fwd(q, kb[:, :, :Nk], vb[:, :, :Nk], scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_dense(w.q, w.k, w.v, w.scale, causal)
    assert_close("O", host(o), ro, TOL_BF16_O)
    assert_close("lse", host(lse), rl, TOL_BF16_LSE)


def test_varlen_tail_poison(A):
    """Tokens after the last sequence are NaN: reading past a sequence's keys shows up."""
    import torch
    w = synth.varlen(H=2, d=128, causal=False, seed=11, lens=[70, 5, 33])
    tk = int(w.cu_k[-1])
    kb = torch.full((tk + 64, 2, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    vb = torch.full((tk + 64, 2, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    kb[:tk] = dev(w.k)
    vb[:tk] = dev(w.v)
    o, lse = A.attn_fwd_varlen(dev(w.q), kb[:tk], vb[:tk], dev(w.cu_q), dev(w.cu_k), w.max_q, w.max_k,
                               scale=w.scale, causal=False)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_varlen(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, False)
    assert_close("O", host(o), ro, TOL_BF16_O)
    assert_close("lse", host(lse), rl, TOL_BF16_LSE)


def test_dense_strided_layout(A):
    """[B, N, H, d] memory order passed through the stride arguments."""
    w = synth.dense(2, 4, 190, 128, "bf16", True, seed=5)
    o, lse = run_dense(A, w, layout="bnhd")
    ro, rl = oracle.attention_dense(w.q, w.k, w.v, w.scale, True)
    assert_close("O", o, ro, TOL_BF16_O)
    assert_close("lse", lse, rl, TOL_BF16_LSE)


def test_dense_deterministic(A):
    import torch
    w = synth.dense(1, 8, 1000, 128, "bf16", True, seed=9)
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    o1, l1 = A.attn_fwd(q, k, v, causal=True)
    o2, l2 = A.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_dense_causal_prefix_invariance(A):
    """Changing K/V rows after row i leaves rows <= i bit-identical."""
    import torch
    w = synth.dense(1, 2, 500, 128, "bf16", True, seed=10)
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    o1, l1 = A.attn_fwd(q, k, v, causal=True)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, 300:] = torch.randn_like(k2[:, :, 300:]) * 3
    v2[:, :, 300:] = torch.randn_like(v2[:, :, 300:]) * 3
    o2, l2 = A.attn_fwd(q, k2, v2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :, :300], o2[:, :, :300]) and torch.equal(l1[:, :, :300], l2[:, :, :300])
    assert not torch.equal(o1[:, :, 300:], o2[:, :, 300:])


@pytest.mark.parametrize("lens,lens_k,causal", [
    ([3, 4], None, True), ([3, 4], None, False),
    ([0, 1, 64, 65, 127, 128, 129, 300], None, True),
    ([0, 1, 64, 65, 127, 128, 129, 300], None, False),
    ([10, 200, 0, 7], [50, 200, 5, 0], True),
    ([10, 200, 0, 7], [50, 200, 5, 0], False),
    ([500], [1], True),
])
@pytest.mark.parametrize("d", [64, 128])
def test_varlen_edges(A, lens, lens_k, causal, d):
    import torch
    w = synth.varlen(H=3, d=d, causal=causal, seed=len(lens) + d, lens=lens, lens_k=lens_k)
    o, lse = A.attn_fwd_varlen(dev(w.q), dev(w.k), dev(w.v), dev(w.cu_q), dev(w.cu_k), w.max_q, w.max_k,
                               scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_varlen(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, causal)
    assert_close("O", host(o), ro, TOL_BF16_O)
    assert_close("lse", host(lse), rl, TOL_BF16_LSE)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equals_dense_per_sequence(A, causal):
    # Each packed sequence against the dense entry on that sequence alone.  Non-causal
    # launches use the same tile configuration in both entries: bit-exact.  Causal
    # varlen batches of short sequences take 32-key tiles where the dense entry keeps
    # 64-key ones (another summation order): both within the bf16 tolerance of each
    # other, which still catches any row or key taken from a neighbouring sequence.
    import torch
    w = synth.varlen(H=4, d=128, causal=causal, seed=3, lens=[130, 257, 64])
    o, lse = A.attn_fwd_varlen(dev(w.q), dev(w.k), dev(w.v), dev(w.cu_q), dev(w.cu_k), w.max_q, w.max_k,
                               scale=w.scale, causal=causal)
    for s in range(3):
        a, b = int(w.cu_q[s]), int(w.cu_q[s + 1])
        qd = dev(np.ascontiguousarray(w.q[a:b].transpose(1, 0, 2))[None])
        kd = dev(np.ascontiguousarray(w.k[a:b].transpose(1, 0, 2))[None])
        vd = dev(np.ascontiguousarray(w.v[a:b].transpose(1, 0, 2))[None])
        od, ld = A.attn_fwd(qd, kd, vd, scale=w.scale, causal=causal)
        torch.cuda.synchronize()
        if not causal:
            assert torch.equal(od[0].transpose(0, 1), o[a:b]) and torch.equal(ld[0].transpose(0, 1), lse[a:b])
        else:
            assert_close(f"O seq {s}", host(o[a:b]), host(od[0].transpose(0, 1)), TOL_BF16_O)
            assert_close(f"lse seq {s}", host(lse[a:b]), host(ld[0].transpose(0, 1)), TOL_BF16_LSE)


@pytest.mark.parametrize("ctx,page", [([1, 15, 16, 17, 0, 511, 512, 513, 1024, 1500], 16),
                                      ([33, 64, 100, 0, 600], 32), ([2000, 3], 64)])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_edges(A, ctx, page, d):
    import torch
    w = synth.paged(H=4, d=d, ctx=ctx, page=page, seed=len(ctx) + page)
    o, lse = A.attn_decode_paged(dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_table),
                                 dev(w.context_lens), int(max(ctx)), scale=w.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_decode_paged(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, w.scale)
    assert_close("O", host(o), ro, TOL_BF16_O)
    assert_close("lse", host(lse), rl, TOL_BF16_LSE)


@pytest.mark.parametrize("H,H_kv", [(8, 8), (8, 2)])
def test_decode_long_context(A, H, H_kv):
    """The longest contexts tested: 65536 and 40001 tokens, 128 splits of the longest
    sequence merged by the combine (one query head per KV head, and grouped-query)."""
    import torch
    ctx = [65536, 40001]
    w = synth.paged(H=H, d=128, ctx=ctx, page=16, seed=96, H_kv=H_kv)
    o, lse = A.attn_decode_paged(dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_table),
                                 dev(w.context_lens), max(ctx), scale=w.scale)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    ro, rl = oracle.attention_decode_paged(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, w.scale)
    assert_close("O", o, ro, TOL_BF16_O)
    assert_close("lse", lse, rl, TOL_BF16_LSE)


@pytest.mark.parametrize("H,H_kv,d", [(4, 4, 64), (8, 2, 128)])
def test_decode_split_counts_at_combine_boundaries(A, H, H_kv, d):
    """The combine reads the splits' (m, l) one split per lane in chunks of 64 and the
    partial outputs eight splits at a time: 512-token splits counts of 8, 9, 64 and 65
    (and one single-token context) put a sequence on each of those boundaries."""
    import torch
    ctx = [4096, 4097, 32768, 32769, 1]
    w = synth.paged(H=H, d=d, ctx=ctx, page=16, seed=97, H_kv=H_kv)
    o, lse = A.attn_decode_paged(dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_table),
                                 dev(w.context_lens), max(ctx), scale=w.scale)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    ro, rl = oracle.attention_decode_paged(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, w.scale)
    assert_close("O", o, ro, TOL_BF16_O)
    assert_close("lse", lse, rl, TOL_BF16_LSE)


def test_decode_context_above_max_is_truncated(A):
    """A context length above max_context_len (a caller error) is truncated to
    max_context_len, in the split kernels and in the combine.  The block table and the
    workspace are sized for the full lengths, so even without the truncation every read
    would stay inside them (it would only give a different result)."""
    import torch
    ctx = [100, 5000, 777, 2048]
    maxc = 1000
    w = synth.paged(H=4, d=128, ctx=ctx, page=16, seed=99, H_kv=2)
    ws = torch.empty(10 * A.attn_decode_paged_workspace_size(4, 4, 128, 5000, 16), dtype=torch.uint8, device="cuda")
    o, lse = A.attn_decode_paged(dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_table),
                                 dev(w.context_lens), maxc, scale=w.scale, workspace=ws)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    clamped = np.minimum(w.context_lens, maxc).astype(np.int32)
    ro, rl = oracle.attention_decode_paged(w.q, w.k_cache, w.v_cache, w.block_table, clamped, w.scale)
    assert_close("O", o, ro, TOL_BF16_O)
    assert_close("lse", lse, rl, TOL_BF16_LSE)


def test_decode_identity_table_equals_dense_last_row(A):
    """Paged decode with pages in order == the last row of a causal dense run."""
    import torch
    ctx = [700, 129]
    w = synth.paged(H=2, d=128, ctx=ctx, identity=True, poison=False, seed=4)
    o, lse = A.attn_decode_paged(dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_table),
                                 dev(w.context_lens), max(ctx), scale=w.scale)
    torch.cuda.synchronize()
    flat_k = w.k_cache[:-1].reshape(-1, 2, 128)
    flat_v = w.v_cache[:-1].reshape(-1, 2, 128)
    start = 0
    for b, c in enumerate(ctx):
        ro, rl = oracle.attention_rows(w.q[b, 0][None], flat_k[start:start + c, 0], flat_v[start:start + c, 0], w.scale)
        assert_close("O", host(o)[b, 0], ro[0], TOL_BF16_O)
        assert_close("lse", host(lse)[b, 0:1], rl, TOL_BF16_LSE)
        start += ((c + 15) // 16) * 16


def test_decode_deterministic(A):
    import torch
    w = synth.paged(B=8, H=8, d=128, ctx_min=100, ctx_max=3000, seed=6)
    args = (dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_table), dev(w.context_lens),
            int(w.context_lens.max()))
    o1, l1 = A.attn_decode_paged(*args, scale=w.scale)
    o2, l2 = A.attn_decode_paged(*args, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ------------------------------------------------------------------ grouped-query attention

@pytest.mark.parametrize("H,Hkv,N,Nk,causal,d", [
    (16, 8, 1000, 1000, True, 128),    # the page's 16 query heads sharing 8 KV heads
    (16, 8, 777, 1333, False, 128),
    (32, 4, 513, 513, True, 128),
    (8, 1, 300, 300, True, 64),        # multi-query
    (6, 3, 200, 257, True, 64),        # 12 (b, h) pairs: not a multiple of 8
])
def test_dense_gqa_bf16(A, H, Hkv, N, Nk, causal, d):
    w = synth.dense(2, H, N, d, "bf16", causal, seed=40, Nk=Nk, H_kv=Hkv)
    o, lse = run_dense(A, w)
    ro, rl = oracle.attention_dense(w.q, w.k, w.v, w.scale, w.causal)
    assert_close("O", o, ro, TOL_BF16_O)
    assert_close("lse", lse, rl, TOL_BF16_LSE)


@pytest.mark.parametrize("H,Hkv,causal", [(4, 2, True), (4, 1, False)])
def test_dense_gqa_fp32(A, H, Hkv, causal):
    w = synth.dense(2, H, 100, 64, "f32", causal, seed=41, Nk=130, H_kv=Hkv)
    o, lse = run_dense(A, w)
    ro, rl = oracle.attention_dense(w.q, w.k, w.v, w.scale, w.causal)
    assert_close("O", o, ro, TOL_F32)
    assert_close("lse", lse, rl, TOL_F32)


@pytest.mark.parametrize("H,Hkv,d", [(8, 2, 128), (16, 8, 64), (4, 1, 128)])
def test_varlen_gqa(A, H, Hkv, d):
    import torch
    w = synth.varlen(H=H, d=d, causal=True, seed=42, lens=[5, 130, 64, 1, 700, 257], H_kv=Hkv)
    o, lse = A.attn_fwd_varlen(dev(w.q), dev(w.k), dev(w.v), dev(w.cu_q), dev(w.cu_k), w.max_q, w.max_k,
                               scale=w.scale, causal=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_varlen(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, True)
    assert_close("O", host(o), ro, TOL_BF16_O)
    assert_close("lse", host(lse), rl, TOL_BF16_LSE)


@pytest.mark.parametrize("H,Hkv,d,page", [(16, 8, 128, 16), (8, 1, 64, 16), (32, 4, 128, 16), (6, 2, 128, 16),
                                          (32, 1, 128, 16), (48, 1, 128, 16), (64, 1, 64, 16), (12, 3, 64, 48),
                                          (16, 4, 128, 32)])
def test_decode_gqa(A, H, Hkv, d, page):
    """Groups of 2 .. 64 query heads per KV head (one and several blocks of 32 heads,
    partial blocks, an odd group), d = 64 and 128, page sizes 16, 32 and 48."""
    import torch
    w = synth.paged(H=H, d=d, seed=43, ctx=[1, 17, 600, 1024, 33, 512, 513, 2000], H_kv=Hkv, page=page)
    o, lse = A.attn_decode_paged(dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_table),
                                 dev(w.context_lens), int(w.context_lens.max()), scale=w.scale)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    ro, rl = oracle.attention_decode_paged(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, w.scale)
    assert_close("O", o, ro, TOL_BF16_O)
    assert_close("lse", lse, rl, TOL_BF16_LSE)


def test_gqa_decode_full(A):
    """The grouped-query decode workload the bench times (64 sequences, 16 query heads
    on 8 KV heads): every sequence and head."""
    import torch
    w = synth.workload("gqa_decode")
    o, lse = A.attn_decode_paged(dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_table),
                                 dev(w.context_lens), int(w.context_lens.max()), scale=w.scale)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    ro, rl = oracle.attention_decode_paged(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, w.scale)
    assert_close("O", o, ro, TOL_BF16_O)
    assert_close("lse", lse, rl, TOL_BF16_LSE)


# ------------------------------------------------------------------ store_kvcache (bit-exact)

def _bits(t):
    """Device tensor -> host uint16 bit patterns (bf16) or uint32 (fp32)."""
    import torch
    h = t.detach().cpu().contiguous()
    return h.view(torch.int16).numpy().view(np.uint16) if h.dtype == torch.bfloat16 else h.view(torch.int32).numpy().view(np.uint32)


def _store_and_compare(A, w, k=None, v=None):
    import torch
    kd = dev(w.k) if k is None else k
    vd = dev(w.v) if v is None else v
    kc, vc = dev(w.k_cache), dev(w.v_cache)
    A.attn_store_kvcache(kd, vd, kc, vc, torch.from_numpy(w.slot_mapping).cuda())
    torch.cuda.synchronize()
    ek, ev = oracle.store_kvcache(w.k, w.v, w.k_cache, w.v_cache, w.slot_mapping)
    assert np.array_equal(_bits(kc), ek), "k_cache differs"
    assert np.array_equal(_bits(vc), ev), "v_cache differs"


@pytest.mark.parametrize("lens,Hkv,d,pad,extra", [
    ([1], 1, 64, 0, 0),
    ([5, 17, 3, 40], 2, 128, 3, 2),
    ([64] * 8, 8, 128, 0, 4),               # decode-like: whole pages
    ([300, 1, 77], 8, 64, 20, 1),
])
def test_store_kvcache_bitexact(A, lens, Hkv, d, pad, extra):
    w = synth.kvstore(lens, Hkv, d, 16, extra_pages=extra, pad=pad, seed=50)
    _store_and_compare(A, w)


def test_store_kvcache_out_of_pool_slots_skipped(A):
    w = synth.kvstore([20, 9], 2, 64, 16, extra_pages=1, seed=51)
    w.slot_mapping[3] = w.num_pages * 16          # one past the pool
    w.slot_mapping[7] = 1 << 40
    w.slot_mapping[11] = -5
    _store_and_compare(A, w)


def test_store_kvcache_fused_qkv_slices(A):
    """K and V read as strided slices of a fused [T, (H + 2 H_kv) d] projection output."""
    import torch
    H, Hkv, d = 8, 2, 128
    w = synth.kvstore([33, 100], Hkv, d, 16, seed=52)
    q = synth.normal(52, synth.T_Q, (w.T, H, d), True)
    fused = np.concatenate([q.reshape(w.T, -1), w.k.reshape(w.T, -1), w.v.reshape(w.T, -1)], axis=1)
    f = dev(fused)
    k = f[:, H * d:(H + Hkv) * d].view(w.T, Hkv, d)
    v = f[:, (H + Hkv) * d:].view(w.T, Hkv, d)
    assert k.stride(0) == (H + 2 * Hkv) * d
    _store_and_compare(A, w, k, v)


def test_store_kvcache_fp32(A):
    import torch
    w = synth.kvstore([21, 5], 2, 64, 16, pad=2, seed=53)
    as32 = lambda b: oracle.bf16_bits_to_f64(b).astype(np.float32)
    k, v, kc0, vc0 = as32(w.k), as32(w.v), as32(w.k_cache), as32(w.v_cache)
    kc, vc = torch.from_numpy(kc0).cuda(), torch.from_numpy(vc0).cuda()
    A.attn_store_kvcache(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), kc, vc,
                         torch.from_numpy(w.slot_mapping).cuda())
    torch.cuda.synchronize()
    ek, ev = oracle.store_kvcache(k, v, kc0, vc0, w.slot_mapping)
    assert np.array_equal(kc.cpu().numpy().view(np.uint32), ek.view(np.uint32))
    assert np.array_equal(vc.cpu().numpy().view(np.uint32), ev.view(np.uint32))


def test_store_kvcache_full_prefill(A):
    """The prefill store the bench times: 34069 tokens, 32 KV heads, d = 128, every slot."""
    w = synth.workload("store_prefill")
    _store_and_compare(A, w)


# ------------------------------------------------------------------ paged prefill

def _run_prefill(A, w):
    import torch
    o, lse = A.attn_fwd_varlen(dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.cu_q), dev(w.cu_k), w.max_q,
                               w.max_k, scale=w.scale, causal=w.causal, block_table=dev(w.block_table))
    torch.cuda.synchronize()
    return host(o), host(lse)


@pytest.mark.parametrize("lq,lk,H,Hkv,d,page,causal", [
    ([5, 130, 1, 64], [100, 130, 1000, 364], 8, 2, 128, 16, True),     # continued chunks
    ([64, 65, 63], [64, 65, 63], 4, 4, 128, 16, True),                   # first chunks (no prefix)
    ([200, 7], [777, 2000], 16, 8, 128, 32, True),
    ([33, 1, 100], [33, 300, 101], 4, 1, 64, 64, True),
    ([50, 129], [1000, 129], 8, 2, 64, 256, True),
    ([40, 90], [300, 90], 4, 2, 128, 16, False),
    ([0, 12, 3], [16, 12, 0], 4, 2, 128, 16, True),                      # empty query / empty context
    ([4200, 30], [4500, 30], 2, 1, 128, 16, True),                       # > 4096 rows: 64-key tiles
])
def test_paged_prefill(A, lq, lk, H, Hkv, d, page, causal):
    w = synth.paged_prefill(lq, lk, H, d, page, causal, seed=60, H_kv=Hkv)
    o, lse = _run_prefill(A, w)
    ro, rl = oracle.attention_varlen_paged(w.q, w.k_cache, w.v_cache, w.cu_q, w.cu_k, w.block_table, w.scale,
                                           causal)
    assert np.isfinite(o).all()   # no NaN-poisoned slot or padding page was read
    assert_close("O", o, ro, TOL_BF16_O)
    assert_close("lse", lse, rl, TOL_BF16_LSE)


def test_paged_prefill_equals_contiguous_varlen(A):
    """Identity-ordered pages hold the same keys as a contiguous varlen batch."""
    import torch
    lens = [70, 300, 17]
    w = synth.varlen(H=8, d=128, causal=True, seed=61, lens=lens, H_kv=2)
    page = 16
    n = [(L + page - 1) // page for L in lens]
    kc = np.zeros((sum(n), page, 2, 128), dtype=np.uint16)
    vc = np.zeros_like(kc)
    bt = np.zeros((3, max(n)), dtype=np.int32)
    off = 0
    for s, L in enumerate(lens):
        t = np.arange(L)
        pages = off + t // page
        kc[pages, t % page] = w.k[w.cu_k[s]:w.cu_k[s + 1]]
        vc[pages, t % page] = w.v[w.cu_k[s]:w.cu_k[s + 1]]
        bt[s, :n[s]] = np.arange(off, off + n[s])
        off += n[s]
    o1, l1 = A.attn_fwd_varlen(dev(w.q), dev(w.k), dev(w.v), dev(w.cu_q), dev(w.cu_k), w.max_q, w.max_k,
                               scale=w.scale, causal=True)
    o2, l2 = A.attn_fwd_varlen(dev(w.q), dev(kc), dev(vc), dev(w.cu_q), dev(w.cu_k), w.max_q, w.max_k,
                               scale=w.scale, causal=True, block_table=dev(bt))
    torch.cuda.synchronize()
    assert np.array_equal(host(o1), host(o2)) and np.array_equal(host(l1), host(l2))


def test_prefill_paged_full(A):
    """The paged prefill the bench times: 16 sequences, the second half of each as new
    causal query rows over its whole context in 16-token pages; every sequence, head
    and row."""
    w = synth.workload("prefill_paged")
    o, lse = _run_prefill(A, w)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    ro, rl = oracle.attention_varlen_paged(w.q, w.k_cache, w.v_cache, w.cu_q, w.cu_k, w.block_table, w.scale,
                                           True)
    assert_close("O", o, ro, TOL_BF16_O)
    assert_close("lse", lse, rl, TOL_BF16_LSE)


# ------------------------------------------------------------------ backward

# Gradient tolerance (none is stated for gradients; derived here).  The backward is handed
# O and lse; both the kernel and the oracle get the oracle forward's O rounded to bf16 and
# its lse in float32 (_fwd_outputs), so both form D_i = dO_i . O_i from the same O.  What
# is left are the kernel's own roundings: dQ, dK, dV are written in bf16, whose
# round-to-nearest-even error is at most 2^-8 = 3.9e-3 of the entry itself, from fp32 sums
# whose terms carry bf16 roundings of P and dS (2^-8 relative each, random in sign) and P
# recomputed in fp32 from lse.  Whole tensor: max-abs error <= TOL_BWD_REL x max
# |reference| (measured at most 5.4e-3 over every case below).  Each gradient ROW (a query
# row of dQ, a key row of dK or dV, per head) is also held to a bound on its own scale,
#     max-abs error <= row_tol x max |reference row| + floor x max |reference tensor|,
# so that a wrong low-magnitude row (late causal keys, rows with few keys) fails even
# when the tensor-wide bound would not see it.  Measured over every case below, the worst
# row used 0.47 (dV), 0.28 (dK) and 0.29 (dQ) of these bounds: a margin of 2-3.
# (Before the O handed to both sides was the same, a dQ row also carried the bf16 rounding
# of the kernel's own O inside D_i, scale (dO_i . dO_i-rounding) sum_j P_ij K_j, which does
# not shrink with the row's magnitude; that term needed a floor of 2e-3 and failed on a
# batch of 70 short sequences.)
TOL_BWD_REL = 1e-2
TOL_BWD_ROWS = {"dQ": (2e-2, 1e-3), "dK": (2e-2, 1e-3), "dV": (1e-2, 1e-3)}   # (row_tol, floor)


def _fwd_outputs(o, lse):
    """The oracle forward's O and lse as the backward's O and lse inputs, in the formats
    the kernels exchange: O rounded to bf16 (bits), lse to float32.  The kernel and the
    oracle backward are both handed these, so each side forms D_i = dO_i . O_i from the
    same O."""
    return synth.f32_to_bf16_bits(o.astype(np.float32)), lse.astype(np.float32)


def _bwd_case(A, B, H, Hkv, N, Nk, d, causal, seed):
    import torch
    w = synth.dense(B, H, N, d, "bf16", causal, seed=seed, Nk=Nk, H_kv=Hkv)
    do = synth.normal(seed, synth.T_DO, (B, H, N, d), True)
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    o_in, lse_in = _fwd_outputs(*oracle.attention_dense(w.q, w.k, w.v, w.scale, causal))
    dq, dk, dv = A.attn_bwd(q, k, v, dev(o_in), dev(lse_in), dev(do), scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    return w, do, o_in, host(dq), host(dk), host(dv)


def _assert_grad(name, got, want):
    """``got``/``want`` [..., rows, d]: the last axis is one gradient row; ``name`` starts
    with dQ, dK or dV."""
    row_tol, floor = TOL_BWD_ROWS[name[:2]]
    scale = max(1e-30, float(np.abs(want).max()))
    err, where, _ = max_err(got, want)
    assert np.isfinite(got).all(), f"{name}: non-finite entries"
    g = got.reshape(-1, got.shape[-1])
    w = want.reshape(-1, want.shape[-1])
    row_err = np.abs(g - w).max(axis=1)
    row_ref = np.abs(w).max(axis=1)
    bound = row_tol * row_ref + floor * scale
    worst = int(np.argmax(row_err / bound))
    print(f"  {name}: max|err| = {err:.3e} at {where}, max|ref| = {scale:.3e}, rel {err / scale:.2e}; "
          f"worst row {worst}: err {row_err[worst]:.2e}, row max|ref| {row_ref[worst]:.2e}, "
          f"{row_err[worst] / bound[worst]:.2f} of its bound", flush=True)
    assert err <= TOL_BWD_REL * scale, f"{name}: max|err| {err:.3e} > {TOL_BWD_REL} x {scale:.3e}"
    assert row_err[worst] <= bound[worst], (f"{name}: row {worst} max|err| {row_err[worst]:.3e} > "
                                            f"{row_tol} x {row_ref[worst]:.3e} + {floor} x {scale:.3e}")


@pytest.mark.parametrize("B,H,Hkv,N,Nk,d,causal", [
    (2, 4, 4, 256, 256, 128, True),
    (1, 8, 2, 300, 300, 64, True),      # grouped-query, ragged tiles
    (1, 4, 4, 200, 333, 128, False),     # Nk != N
    (1, 2, 1, 333, 200, 128, True),      # rows without keys (bottom-right), multi-query
    (2, 2, 2, 64, 64, 64, False),
    (1, 2, 2, 1, 77, 128, True),         # one query row
])
def test_backward(A, B, H, Hkv, N, Nk, d, causal):
    w, do, o_in, dq, dk, dv = _bwd_case(A, B, H, Hkv, N, Nk, d, causal, seed=80)
    rq, rk, rv = oracle.attention_backward_dense(w.q, w.k, w.v, do, w.scale, causal, o=o_in)
    _assert_grad("dQ", dq, rq)
    _assert_grad("dK", dk, rk)
    _assert_grad("dV", dv, rv)


def test_backward_deterministic(A):
    a = _bwd_case(A, 1, 4, 2, 257, 257, 128, True, seed=81)
    b = _bwd_case(A, 1, 4, 2, 257, 257, 128, True, seed=81)
    for x, y in zip(a[3:], b[3:]):
        assert np.array_equal(x, y)


def _bwd_varlen_case(A, lens, lens_k, H, Hkv, d, causal, seed):
    import torch
    w = synth.varlen(H=H, d=d, causal=causal, seed=seed, lens=lens, lens_k=lens_k, H_kv=Hkv)
    tq = int(w.cu_q[-1])
    do = synth.normal(seed, synth.T_DO, (tq, H, d), True)
    q, k, v, cq, ck = dev(w.q), dev(w.k), dev(w.v), dev(w.cu_q), dev(w.cu_k)
    mq, mk = w.max_q, w.max_k
    o_in, lse_in = _fwd_outputs(*oracle.attention_varlen(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, causal))
    dq, dk, dv = A.attn_bwd_varlen(q, k, v, dev(o_in), dev(lse_in), dev(do), cq, ck, mq, mk, scale=w.scale,
                                   causal=causal)
    torch.cuda.synchronize()
    return w, do, o_in, host(dq), host(dk), host(dv)


@pytest.mark.parametrize("lens,lens_k,H,Hkv,d,causal", [
    ([1, 17, 64, 130, 33], None, 4, 2, 128, True),          # ragged, grouped-query
    ([100, 7, 250], [300, 7, 400], 4, 4, 64, True),          # Lk > Lq: bottom-right causal
    ([100, 7, 250], [60, 50, 400], 2, 1, 128, True),         # Lq > Lk: rows without keys
    ([64, 0, 96], [64, 10, 0], 4, 4, 128, False),            # empty query range, empty key range
    ([300], None, 8, 8, 128, True),                          # one sequence
    ([50, 300, 0, 129, 128, 1], None, 16, 8, 128, True),     # compact grids, KV heads dealt over the XCDs
    ([int(x) for x in np.random.default_rng(7).integers(0, 150, 70)], None, 4, 2, 64, True),  # 70 sequences: plain grids
])
def test_backward_varlen(A, lens, lens_k, H, Hkv, d, causal):
    w, do, o_in, dq, dk, dv = _bwd_varlen_case(A, lens, lens_k, H, Hkv, d, causal, seed=82)
    rq, rk, rv = oracle.attention_backward_varlen(w.q, w.k, w.v, do, w.cu_q, w.cu_k, w.scale, causal, o=o_in)
    _assert_grad("dQ", dq, rq)
    _assert_grad("dK", dk, rk)
    _assert_grad("dV", dv, rv)


def test_backward_varlen_one_sequence_equals_dense(A):
    """A one-sequence packed batch runs the same backward arithmetic as the dense entry on
    the transposed tensors (given the same O and lse): the gradients are bit-identical."""
    import torch
    w = synth.varlen(H=4, d=128, causal=True, seed=83, lens=[333], lens_k=[400], H_kv=2)
    do = synth.normal(83, synth.T_DO, (333, 4, 128), True)
    q, k, v, cq, ck = dev(w.q), dev(w.k), dev(w.v), dev(w.cu_q), dev(w.cu_k)
    o, lse = A.attn_fwd_varlen(q, k, v, cq, ck, w.max_q, w.max_k, scale=w.scale, causal=True)
    dq, dk, dv = A.attn_bwd_varlen(q, k, v, o, lse, dev(do), cq, ck, w.max_q, w.max_k, scale=w.scale, causal=True)
    t = lambda x: x.transpose(0, 1).contiguous()[None]  # [total, H, d] -> [1, H, N, d]
    gq, gk, gv = A.attn_bwd(t(q), t(k), t(v), t(o), lse.transpose(0, 1).contiguous()[None], t(dev(do)),
                            scale=w.scale, causal=True)
    torch.cuda.synchronize()
    for a, b in ((dq, gq), (dk, gk), (dv, gv)):
        assert torch.equal(a, b[0].transpose(0, 1))


def test_backward_varlen_deterministic(A):
    a = _bwd_varlen_case(A, [70, 129, 5], None, 4, 2, 128, True, seed=84)
    b = _bwd_varlen_case(A, [70, 129, 5], None, 4, 2, 128, True, seed=84)
    for x, y in zip(a[3:], b[3:]):
        assert np.array_equal(x, y)


def test_backward_varlen_c4_sampled(A):
    """The 16-sequence varlen batch (34069 tokens, H = 32, causal): every gradient finite;
    the shortest and the longest sequence checked in full for two heads."""
    import torch
    w = synth.workload("c4")
    tq = int(w.cu_q[-1])
    do = synth.normal(0, synth.T_DO, (tq, 32, 128), True)
    q, k, v, cq, ck = dev(w.q), dev(w.k), dev(w.v), dev(w.cu_q), dev(w.cu_k)
    o_in, lse_in = _fwd_outputs(*oracle.attention_varlen(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, True))
    dq, dk, dv = A.attn_bwd_varlen(q, k, v, dev(o_in), dev(lse_in), dev(do), cq, ck, w.max_q, w.max_k,
                                   scale=w.scale, causal=True)
    torch.cuda.synchronize()
    dq, dk, dv = host(dq), host(dk), host(dv)
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()
    lens = np.diff(w.cu_q)
    for s in (int(np.argmin(lens)), int(np.argmax(lens))):
        a, b = int(w.cu_q[s]), int(w.cu_q[s + 1])
        for h in (0, 31):
            rq, rk, rv = oracle.attention_backward_rows(w.q[a:b, h], w.k[a:b, h], w.v[a:b, h], do[a:b, h], w.scale, True,
                                                        o=o_in[a:b, h])
            _assert_grad(f"dQ[s={s},h={h}]", dq[a:b, h], rq)
            _assert_grad(f"dK[s={s},h={h}]", dk[a:b, h], rk)
            _assert_grad(f"dV[s={s},h={h}]", dv[a:b, h], rv)


def test_backward_full_causal_8192(A):
    """The backward the bench times: causal B=1 H=32 N=8192 d=128, two heads checked
    in full against the oracle."""
    import torch
    w = synth.workload("c3")
    do = synth.normal(0, synth.T_DO, (1, 32, 8192, 128), True)
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    o_in, lse_in = _fwd_outputs(*oracle.attention_dense(w.q, w.k, w.v, w.scale, True))
    dq, dk, dv = A.attn_bwd(q, k, v, dev(o_in), dev(lse_in), dev(do), scale=w.scale, causal=True)
    torch.cuda.synchronize()
    dq, dk, dv = host(dq), host(dk), host(dv)
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()
    for h in (0, 31):
        rq, rk, rv = oracle.attention_backward_rows(w.q[0, h], w.k[0, h], w.v[0, h], do[0, h], w.scale, True,
                                                    o=o_in[0, h])
        _assert_grad(f"dQ[h={h}]", dq[0, h], rq)
        _assert_grad(f"dK[h={h}]", dk[0, h], rk)
        _assert_grad(f"dV[h={h}]", dv[0, h], rv)


def test_side_stream_matches_default_stream(A):
    """Launches go to the stream the caller names (torch's current stream by default):
    the same calls on a side stream (default priority), implicitly and explicitly, give
    the default stream's bits."""
    import torch
    w = synth.dense(B=1, H=4, N=300, d=128, causal=True, seed=97)
    q, k, v = dev(w.q), dev(w.k), dev(w.v)
    wp = synth.paged(H=4, d=128, ctx=[700, 33], page=16, seed=98)
    pq, kc, vc, bt, cl = dev(wp.q), dev(wp.k_cache), dev(wp.v_cache), dev(wp.block_table), dev(wp.context_lens)
    do = dev(synth.normal(97, synth.T_DO, (1, 4, 300, 128), True))

    def run(stream=None):
        o, lse = A.attn_fwd(q, k, v, scale=w.scale, causal=True, stream=stream)
        od, ld = A.attn_decode_paged(pq, kc, vc, bt, cl, 700, scale=wp.scale, stream=stream)
        g = A.attn_bwd(q, k, v, o, lse, do, scale=w.scale, causal=True, stream=stream)
        return (o, lse, od, ld) + tuple(g)

    ref = run()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        implicit = run()
    explicit = run(stream=s)
    s.synchronize()
    for a, b, c in zip(ref, implicit, explicit):
        assert torch.equal(a, b) and torch.equal(a, c)
