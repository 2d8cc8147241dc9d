"""attn_decode_paged_noalloc (the paged decode through the library's fixed device
scratch, for callers that cannot allocate) against attn_decode_paged with a caller
workspace: the same kernels, so the results must be bit-identical; and both against the
oracle at the bf16 tolerances.  Two calls in a row, the second on a smaller batch, show
that the reused scratch carries nothing from one call into the next."""
import numpy as np
import pytest

import oracle
import synth
from tests.util import TOL_BF16_LSE, TOL_BF16_O, assert_close, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    import torch
    import exact_attention_attn_amd as attn
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    attn.load()
    return attn


def _both(A, w, maxctx):
    import torch
    args = (dev(w.q), dev(w.k_cache), dev(w.v_cache), dev(w.block_table), dev(w.context_lens))
    B, H, d = w.q.shape
    o_na = torch.full((B, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    l_na = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    A.attn_decode_paged_noalloc(*args, maxctx, o_na, scale=w.scale, lse=l_na)
    o_ws, l_ws = A.attn_decode_paged(*args, maxctx, scale=w.scale)
    torch.cuda.synchronize()
    return o_na, l_na, o_ws, l_ws


@pytest.mark.parametrize("H,H_kv", [(8, 8), (16, 4)])
def test_noalloc_matches_workspace_entry_twice(A, H, H_kv):
    import torch
    # first call: 24 sequences up to 9000 tokens; second: 5 shorter sequences
    for seed, B, cmin, cmax in ((71, 24, 1, 9000), (72, 5, 1, 700)):
        w = synth.paged(B=B, H=H, d=128, ctx_min=cmin, ctx_max=cmax, seed=seed, H_kv=H_kv)
        maxctx = int(w.context_lens.max())
        print(f"  B={B} H={H} H_kv={H_kv} max context {maxctx}", flush=True)
        o_na, l_na, o_ws, l_ws = _both(A, w, maxctx)
        assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws), "no-allocation entry differs from the workspace entry"
        ro, rl = oracle.attention_decode_paged(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, w.scale)
        assert_close("O", host(o_na), ro, TOL_BF16_O)
        assert_close("lse", host(l_na), rl, TOL_BF16_LSE)


def test_noalloc_rejects_batches_beyond_its_scratch(A):
    import torch
    w = synth.paged(B=2, H=2, d=128, ctx=[40, 17], seed=73)
    o = torch.empty((2, 2, 128), dtype=torch.bfloat16, device="cuda")
    big = 200000 * 512   # a max_context_len whose partials exceed the fixed scratch
    bt = torch.zeros((2, big // 16), dtype=torch.int32, device="cuda")
    with pytest.raises(A.AttnError) as e:
        A.attn_decode_paged_noalloc(dev(w.q), dev(w.k_cache), dev(w.v_cache), bt, dev(w.context_lens), big, o,
                                    scale=w.scale)
    assert e.value.status == A.ATTN_ERR_SCRATCH_LIMIT
