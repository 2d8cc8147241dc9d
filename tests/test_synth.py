"""The seeded generators: recorded derived statistics (drift detection), RNE rounding,
thread-count independence and the poison-page layout."""
import numpy as np
import pytest

import synth


def test_c4_lengths_recorded():
    v = synth.varlen(16, 128, 4096, H=1, d=8)   # same draw order, tiny tensors
    assert v.lens_q.tolist() == [3504, 2656, 2156, 1198, 1349, 290, 426, 193, 823, 3355,
                                 2705, 3750, 2126, 2535, 3980, 3023]
    assert int(v.cu_q[-1]) == 34069 and v.max_q == 3980
    assert v.cu_q.dtype == np.int32 and np.array_equal(v.cu_q, v.cu_k)


def test_c5_tables_recorded():
    p = synth.paged(with_pool=False)
    c = p.context_lens.astype(np.int64)
    assert c.sum() == 283360 and c.min() == 533 and c.max() == 8171
    assert p.num_pages == 17742 and p.max_pages == 511
    used = np.concatenate([p.block_table[b, :(c[b] + 15) // 16] for b in range(p.B)])
    assert np.array_equal(np.sort(used), np.arange(p.num_pages))       # a permutation
    pad = np.concatenate([p.block_table[b, (c[b] + 15) // 16:] for b in range(p.B)])
    assert np.all(pad == p.num_pages)                                   # padding -> poison page
    algorithmic = c.sum() * 32 * 128 * 2 * 2 + 64 * 32 * 128 * 2 * 2 + 64 * 32 * 4 + \
        ((c + 15) // 16).sum() * 4 + 64 * 4
    assert algorithmic == 4643698232


def test_bf16_rne_matches_torch_and_ties():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(0).standard_normal(1 << 16).astype(np.float32) * 7
    ties = np.array([1.00390625, 1.01171875, -1.00390625, 3.0 + 2 ** -7, 65504.0, 1e-30],
                    dtype=np.float32)
    x = np.concatenate([x, ties])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert synth.f32_to_bf16_bits(np.array([1.00390625], np.float32))[0] == 0x3F80  # tie -> even
    assert synth.f32_to_bf16_bits(np.array([1.01171875], np.float32))[0] == 0x3F82
    assert synth.f32_to_bf16_bits(np.array([np.nan], np.float32))[0] == 0x7FC0


def test_values_independent_of_threads(monkeypatch):
    a = synth.normal(3, synth.T_K, (3, synth.CHUNK // 2 + 5), True)
    monkeypatch.setattr(synth.gen, "_threads", lambda: 1)
    b = synth.normal(3, synth.T_K, (3, synth.CHUNK // 2 + 5), True)
    assert np.array_equal(a, b)
    c = synth.normal(4, synth.T_K, (3, synth.CHUNK // 2 + 5), True)
    assert not np.array_equal(a, c)


def test_poison_layout():
    p = synth.paged(B=3, H=2, d=8, ctx=[5, 16, 17], page=16)
    nan = p.k_cache.view(np.uint16) == synth.BF16_NAN
    assert nan[p.num_pages].all()
    last0 = p.block_table[0, 0]
    assert nan[last0, 5:].all() and not nan[last0, :5].any()
    assert not nan[p.block_table[1, 0]].any()
    last2 = p.block_table[2, 1]
    assert nan[last2, 1:].all() and not nan[last2, :1].any()
