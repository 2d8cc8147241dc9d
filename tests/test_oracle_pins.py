"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  None of them re-types the oracle's formula:
each compares it with a printed value, a closed form, an invariant, a brute-force
loop or a second algorithm (the online recurrence).
"""
import math

import numpy as np
import pytest

import oracle
from tests.golden.load import load

TIGHT = 1e-12


def rng(seed=0):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- worked example (page 1, §2.1)

def test_hand_example_closed_form():
    g = load("hand_example.txt")
    Q, K, V = g["Q"], g["K"], g["V"]
    # scores are integers: S = Q K^T exactly as printed
    P = oracle.probabilities(Q, K, 1.0)
    e3, e2 = math.exp(3), math.exp(2)
    P_exact = np.array([[1 / (1 + e3), e3 / (1 + e3)], [1 / (1 + e2), e2 / (1 + e2)]])
    assert np.abs(P - P_exact).max() < TIGHT
    O, lse = oracle.attention_rows(Q, K, V, 1.0)
    O_exact = P_exact @ V
    assert np.abs(O - O_exact).max() < TIGHT
    assert abs(O_exact[0, 1] - 1.9051483) < 1e-7
    lse_exact = np.array([5 + math.log1p(math.exp(-3)), 3 + math.log1p(math.exp(-2))])
    assert np.abs(lse - lse_exact).max() < TIGHT
    # third column of V is all ones -> third column of O is exactly a row sum of P
    assert np.abs(O[:, 2] - 1.0).max() < 1e-15


def test_hand_example_printed_values():
    """Printed P (2 dp) and O (2 dp).  The page multiplied its rounded P, so O[0,1] is
    printed 1.90 while the exact value is 1.905; hence the ±0.01 bound on O."""
    g = load("hand_example.txt")
    S = g["Q"] @ g["K"].T
    assert np.array_equal(S, g["S"])
    P = oracle.probabilities(g["Q"], g["K"], 1.0)
    assert np.abs(P - g["P"]).max() <= 0.005 + 1e-12
    O, _ = oracle.attention_rows(g["Q"], g["K"], g["V"], 1.0)
    assert np.abs(O - g["O"]).max() <= 0.01


def test_hand_example_transposed_operand_is_caught():
    """A swapped Q/K (S^T instead of S) would give a different O on this example."""
    g = load("hand_example.txt")
    O, _ = oracle.attention_rows(g["Q"], g["K"], g["V"], 1.0)
    Ot, _ = oracle.attention_rows(g["K"], g["Q"], g["V"], 1.0)
    assert np.abs(O - Ot).max() > 0.1


# ----------------------------------------------------------------- FA2 trace (page 1, §2.3)

def _fa2_inputs():
    g = load("fa2_trace.txt")
    Q = np.stack([g["s0"], g["s1"]])      # with K = I, S = Q K^T = Q: scores as printed
    K = np.eye(4)
    return g, Q, K, g["Vread"]


def test_fa2_trace_online_recurrence():
    g, Q, K, V = _fa2_inputs()
    O, lse, tr = oracle.online_attention(Q, K, V, 1.0, block=1, trace=True)
    for r, key in ((0, "ml0"), (1, "ml1")):
        assert np.abs(np.array(tr[r]) - g[key]).max() < 5e-5
    assert np.abs(O[0] - g["O0"]).max() < 5e-5
    assert np.abs(O[1] - g["O1"]).max() < 5e-5
    l0 = 1 + math.exp(-1) + math.exp(-2) + math.exp(-3)
    l1 = 1 + math.exp(-2) + math.exp(-3) + math.exp(-4)
    assert abs(tr[0][-1][1] - l0) < TIGHT and abs(tr[1][-1][1] - l1) < TIGHT
    assert abs(lse[0] - (3 + math.log(l0))) < TIGHT and abs(lse[1] - (4 + math.log(l1))) < TIGHT


def test_fa2_trace_two_pass():
    g, Q, K, V = _fa2_inputs()
    O, lse = oracle.attention_rows(Q, K, V, 1.0)
    assert np.abs(O[0] - g["O0"]).max() < 5e-5
    assert np.abs(O[1] - g["O1"]).max() < 5e-5
    assert abs(lse[0] - 3.4401897) < 1e-7 and abs(lse[1] - 4.1851825) < 1e-7


# ----------------------------------------------------------------- invariants and closed forms

@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one_and_output_is_convex(causal):
    r = rng(1)
    q, k, v = r.normal(size=(9, 5)), r.normal(size=(9, 5)), r.normal(size=(9, 3))
    P = oracle.probabilities(q, k, 0.7, causal)
    assert np.abs(P.sum(1) - 1).max() < 1e-14
    assert (P >= 0).all()
    if causal:
        assert np.all(P[np.triu_indices(9, 1)] == 0)
    O, _ = oracle.attention_rows(q, k, v, 0.7, causal)
    assert (O >= v.min(0) - 1e-15).all() and (O <= v.max(0) + 1e-15).all()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lq,lk", [(7, 7), (5, 9), (1, 6), (13, 13)])
@pytest.mark.parametrize("block", [1, 2, 3, 7, None])
def test_online_recurrence_equals_two_pass(causal, lq, lk, block):
    r = rng(lq * 100 + lk)
    q, k, v = r.normal(size=(lq, 6)), r.normal(size=(lk, 6)), r.normal(size=(lk, 4))
    o1, l1 = oracle.online_attention(q, k, v, 0.45, block=block or lk, causal=causal)
    o2, l2 = oracle.attention_rows(q, k, v, 0.45, causal)
    assert np.abs(o1 - o2).max() < TIGHT
    assert np.abs(l1 - l2).max() < TIGHT


def _brute(q, k, v, scale, causal):
    """Pure-Python attention with math.exp, no NumPy arithmetic and no max-subtraction
    (inputs are small enough for exp not to overflow)."""
    lq, lk, d, dv = len(q), len(k), len(q[0]), len(v[0])
    O, L = [], []
    for i in range(lq):
        w = []
        for j in range(lk):
            if causal and j > i + (lk - lq):
                continue
            s = 0.0
            for c in range(d):
                s += float(q[i][c]) * float(k[j][c])
            w.append((j, math.exp(scale * s)))
        z = sum(x for _, x in w)
        O.append([sum(x * float(v[j][c]) for j, x in w) / z if w else 0.0 for c in range(dv)])
        L.append(math.log(z) if w else -math.inf)
    return np.array(O), np.array(L)


@pytest.mark.parametrize("lq,lk,d,causal", [(1, 1, 1, False), (1, 5, 3, False), (4, 4, 8, True),
                                            (16, 16, 8, False), (16, 16, 8, True), (3, 11, 2, True),
                                            (11, 3, 5, False), (7, 13, 4, True)])
def test_brute_force_small(lq, lk, d, causal):
    r = rng(lq + 7 * lk + 31 * d)
    q, k, v = r.normal(size=(lq, d)), r.normal(size=(lk, d)), r.normal(size=(lk, 3))
    scale = 1 / math.sqrt(d)
    ob, lb = _brute(q.tolist(), k.tolist(), v.tolist(), scale, causal)
    o, l = oracle.attention_rows(q, k, v, scale, causal)
    assert np.array_equal(np.isinf(l), np.isinf(lb))
    fin = np.isfinite(lb)
    assert np.abs(o - ob).max() < TIGHT
    assert np.abs(l[fin] - lb[fin]).max() < TIGHT


def test_causal_invariants():
    r = rng(3)
    n, d = 12, 6
    q, k, v = r.normal(size=(n, d)), r.normal(size=(n, d)), r.normal(size=(n, d))
    s = 0.4
    o, l = oracle.attention_rows(q, k, v, s, True)
    # row 0 sees only key 0
    assert np.abs(o[0] - v[0]).max() < 1e-15
    assert abs(l[0] - s * (q[0] @ k[0])) < TIGHT
    # last causal row == last non-causal row
    o2, l2 = oracle.attention_rows(q, k, v, s, False)
    assert np.abs(o[-1] - o2[-1]).max() < TIGHT and abs(l[-1] - l2[-1]) < TIGHT
    # changing keys/values after row i leaves row i unchanged
    i = 5
    k2, v2 = k.copy(), v.copy()
    k2[i + 1:] = r.normal(size=k2[i + 1:].shape) * 10
    v2[i + 1:] = r.normal(size=v2[i + 1:].shape) * 10
    o3, l3 = oracle.attention_rows(q, k2, v2, s, True)
    assert np.abs(o3[:i + 1] - o[:i + 1]).max() == 0 and np.abs(l3[:i + 1] - l[:i + 1]).max() == 0
    assert np.abs(o3[i + 1:] - o[i + 1:]).max() > 1e-3
    # a single query row with causal (bottom-right) == non-causal
    oa, la = oracle.attention_rows(q[:1], k, v, s, True)
    ob, lb = oracle.attention_rows(q[:1], k, v, s, False)
    assert np.abs(oa - ob).max() == 0 and np.abs(la - lb).max() == 0
    # Lq < Lk: row i (bottom-right aligned) sees keys 0..i+(Lk-Lq)
    oc, lc = oracle.attention_rows(q[:4], k, v, s, True)
    for i in range(4):
        lim = i + (n - 4)
        od, ld = oracle.attention_rows(q[i:i + 1], k[:lim + 1], v[:lim + 1], s, False)
        assert np.abs(oc[i] - od[0]).max() < TIGHT and abs(lc[i] - ld[0]) < TIGHT


def test_rows_without_keys():
    r = rng(4)
    q, k, v = r.normal(size=(6, 4)), r.normal(size=(3, 4)), r.normal(size=(3, 4))
    # Lq > Lk under bottom-right causal: rows 0..2 have no admissible key
    o, l = oracle.attention_rows(q, k, v, 0.5, True)
    assert np.all(o[:3] == 0) and np.all(np.isneginf(l[:3]))
    assert np.all(np.isfinite(l[3:]))
    # no keys at all
    o, l = oracle.attention_rows(q, k[:0], v[:0], 0.5, False)
    assert np.all(o == 0) and np.all(np.isneginf(l))


def test_closed_forms():
    r = rng(5)
    q, v = r.normal(size=(5, 4)), r.normal(size=(9, 3))
    # zero keys -> uniform attention: O = mean(V), lse = ln(Lk)
    o, l = oracle.attention_rows(q, np.zeros((9, 4)), v, 0.3)
    assert np.abs(o - v.mean(0)).max() < TIGHT and np.abs(l - math.log(9)).max() < TIGHT
    # one key -> O = v0, lse = scale q.k
    k1 = r.normal(size=(1, 4))
    o, l = oracle.attention_rows(q, k1, v[:1], 0.3)
    assert np.abs(o - v[0]).max() < 1e-15 and np.abs(l - 0.3 * (q @ k1[0])).max() < TIGHT
    # two keys: O = sigma(a-b) v0 + sigma(b-a) v1 with a, b the scaled scores
    k2 = r.normal(size=(2, 4))
    o, l = oracle.attention_rows(q, k2, v[:2], 0.3)
    a, b = 0.3 * (q @ k2[0]), 0.3 * (q @ k2[1])
    w0 = 1 / (1 + np.exp(b - a))
    assert np.abs(o - (w0[:, None] * v[0] + (1 - w0)[:, None] * v[1])).max() < TIGHT
    assert np.abs(l - np.logaddexp(a, b)).max() < TIGHT
    # very sharp softmax picks the arg-max key
    k = r.normal(size=(9, 4))
    o, _ = oracle.attention_rows(q, k, v, 1e4)
    assert np.abs(o - v[np.argmax(q @ k.T, axis=1)]).max() < 1e-9


def test_algebraic_invariants():
    r = rng(6)
    q, k, v = r.normal(size=(7, 5)), r.normal(size=(10, 5)), r.normal(size=(10, 4))
    s = 0.6
    o, l = oracle.attention_rows(q, k, v, s)
    perm = r.permutation(10)
    op, lp = oracle.attention_rows(q, k[perm], v[perm], s)
    assert np.abs(o - op).max() < TIGHT and np.abs(l - lp).max() < TIGHT
    u = r.normal(size=5)
    os_, ls = oracle.attention_rows(q, k + u, v, s)
    assert np.abs(o - os_).max() < 1e-11 and np.abs(ls - (l + s * (q @ u))).max() < 1e-11
    v2 = r.normal(size=(10, 4))
    o2, _ = oracle.attention_rows(q, k, v2, s)
    o3, _ = oracle.attention_rows(q, k, 2.5 * v - 0.5 * v2, s)
    assert np.abs(o3 - (2.5 * o - 0.5 * o2)).max() < 1e-11


def test_scale_matters():
    r = rng(7)
    q, k, v = r.normal(size=(4, 8)), r.normal(size=(6, 8)), r.normal(size=(6, 2))
    o1, l1 = oracle.attention_rows(q, k, v, 1 / math.sqrt(8))
    o2, l2 = oracle.attention_rows(q * (1 / math.sqrt(8)), k, v, 1.0)
    assert np.abs(o1 - o2).max() < TIGHT and np.abs(l1 - l2).max() < TIGHT
    o3, _ = oracle.attention_rows(q, k, v, 1.0)
    assert np.abs(o1 - o3).max() > 1e-3


def test_bf16_upcast_exact():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F80, 0xFF80], dtype=np.uint16)
    x = oracle.bf16_bits_to_f64(bits)
    assert x[0] == 1.0 and x[1] == -2.0 and x[2] == 1.0078125
    assert x[3] == 2.0 ** -133 and x[4] == np.inf and x[5] == -np.inf


# ----------------------------------------------------------------- structural reductions

def test_varlen_is_per_sequence_dense():
    r = rng(8)
    cu = np.array([0, 3, 7], dtype=np.int32)     # the page's example (section 3.3)
    H, d = 2, 4
    q, k, v = (r.normal(size=(7, H, d)) for _ in range(3))
    for causal in (False, True):
        o, l = oracle.attention_varlen(q, k, v, cu, cu, 0.5, causal)
        for a, b in ((0, 3), (3, 7)):
            for h in range(H):
                od, ld = oracle.attention_rows(q[a:b, h], k[a:b, h], v[a:b, h], 0.5, causal)
                assert np.abs(o[a:b, h] - od).max() == 0 and np.abs(l[a:b, h] - ld).max() == 0
    # tokens of one sequence never see another sequence's keys
    k2 = k.copy()
    k2[3:] += 100
    o2, _ = oracle.attention_varlen(q, k2, v, cu, cu, 0.5, False)
    o1, _ = oracle.attention_varlen(q, k, v, cu, cu, 0.5, False)
    assert np.abs(o2[:3] - o1[:3]).max() == 0


def test_varlen_q_shorter_than_k_bottom_right():
    r = rng(9)
    cq = np.array([0, 2, 5], dtype=np.int32)
    ck = np.array([0, 6, 8], dtype=np.int32)
    q, k, v = r.normal(size=(5, 1, 3)), r.normal(size=(8, 1, 3)), r.normal(size=(8, 1, 3))
    o, l = oracle.attention_varlen(q, k, v, cq, ck, 1.0, True)
    # seq 0: Lq=2, Lk=6 -> row t sees keys 0..t+4
    for t in range(2):
        od, _ = oracle.attention_rows(q[t:t + 1, 0], k[:t + 5, 0], v[:t + 5, 0], 1.0, False)
        assert np.abs(o[t, 0] - od[0]).max() < TIGHT
    # seq 1: Lq=3, Lk=2 -> row 0 sees nothing
    assert np.all(o[2, 0] == 0) and np.isneginf(l[2, 0])


def _paged_small(seed, ctx, page=4, H=2, d=3, identity=False):
    r = rng(seed)
    n = [(c + page - 1) // page for c in ctx]
    P = sum(n)
    perm = np.arange(P) if identity else r.permutation(P)
    bt = np.full((len(ctx), max(n)), P, dtype=np.int32)
    off = 0
    for b, m in enumerate(n):
        bt[b, :m] = perm[off:off + m]
        off += m
    kc = r.normal(size=(P + 1, page, H, d))
    vc = r.normal(size=(P + 1, page, H, d))
    kc[P] = np.nan
    vc[P] = np.nan
    q = r.normal(size=(len(ctx), H, d))
    return q, kc, vc, bt, np.array(ctx, dtype=np.int32)


def test_paged_decode_gathers_through_block_table():
    q, kc, vc, bt, ctx = _paged_small(10, [1, 4, 5, 11, 16])
    o, l = oracle.attention_decode_paged(q, kc, vc, bt, ctx, 0.7)
    assert np.isfinite(o).all() and np.isfinite(l).all()   # never touches the NaN page
    page = kc.shape[1]
    for b, c in enumerate(ctx):
        # brute-force gather token by token
        ks = np.stack([kc[bt[b, t // page], t % page] for t in range(c)])
        vs = np.stack([vc[bt[b, t // page], t % page] for t in range(c)])
        for h in range(q.shape[1]):
            ob, lb = _brute([q[b, h].tolist()], ks[:, h].tolist(), vs[:, h].tolist(), 0.7, False)
            assert np.abs(o[b, h] - ob[0]).max() < TIGHT and abs(l[b, h] - lb[0]) < TIGHT


def test_paged_identity_equals_contiguous_and_last_causal_row():
    q, kc, vc, bt, ctx = _paged_small(11, [7, 9], identity=True)
    o, l = oracle.attention_decode_paged(q, kc, vc, bt, ctx, 0.3)
    page = kc.shape[1]
    flat_k = kc[:-1].reshape(-1, *kc.shape[2:])
    flat_v = vc[:-1].reshape(-1, *vc.shape[2:])
    start = 0
    for b, c in enumerate(ctx):
        for h in range(q.shape[1]):
            kk = flat_k[start:start + c, h]
            vv = flat_v[start:start + c, h]
            od, ld = oracle.attention_rows(q[b, h][None], kk, vv, 0.3, False)
            assert np.abs(o[b, h] - od[0]).max() < TIGHT and abs(l[b, h] - ld[0]) < TIGHT
            # decode == last row of a causal run whose last query is q
            qq = np.concatenate([np.random.default_rng(0).normal(size=(c - 1, q.shape[2])), q[b, h][None]])
            oc, lc = oracle.attention_rows(qq, kk, vv, 0.3, True)
            assert np.abs(oc[-1] - od[0]).max() < TIGHT and abs(lc[-1] - ld[0]) < TIGHT
        start += ((c + page - 1) // page) * page


def test_dense_wrapper_layout():
    r = rng(12)
    q, k, v = (r.normal(size=(2, 3, 5, 4)) for _ in range(3))
    o, l = oracle.attention_dense(q, k, v, 0.5, True)
    for b in range(2):
        for h in range(3):
            od, ld = oracle.attention_rows(q[b, h], k[b, h], v[b, h], 0.5, True)
            assert np.array_equal(o[b, h], od) and np.array_equal(l[b, h], ld)


def test_optional_sdpa_crosscheck():
    """Non-authoritative: PyTorch's CPU math SDPA in float64 agrees with the oracle."""
    torch = pytest.importorskip("torch")
    r = rng(13)
    q, k, v = (r.normal(size=(1, 2, 33, 16)) for _ in range(3))
    for causal in (False, True):
        o, _ = oracle.attention_dense(q, k, v, 0.25, causal)
        t = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal, scale=0.25)
        assert np.abs(o - t.numpy()).max() < 1e-12


# ----------------------------------------------------------------- grouped-query attention

def _expand_kv(x, groups, axis):
    """The page's explicit GQA expansion (section "GQA: handled natively by the kernel"):
    each KV head repeated `groups` times along the head axis, KV head-major."""
    shp = list(x.shape)
    y = np.expand_dims(x, axis + 1)
    y = np.broadcast_to(y, shp[:axis + 1] + [groups] + shp[axis + 1:])
    return y.reshape(shp[:axis] + [shp[axis] * groups] + shp[axis + 1:])


@pytest.mark.parametrize("H,Hkv", [(4, 2), (8, 2), (6, 3), (4, 1), (4, 4)])
def test_gqa_dense_equals_expanded_kv(H, Hkv):
    r = rng(20 + H + Hkv)
    q = r.normal(size=(2, H, 9, 5))
    k, v = r.normal(size=(2, Hkv, 11, 5)), r.normal(size=(2, Hkv, 11, 5))
    for causal in (False, True):
        o, l = oracle.attention_dense(q, k, v, 0.4, causal)
        g = H // Hkv
        oe, le = oracle.attention_dense(q, _expand_kv(k, g, 1), _expand_kv(v, g, 1), 0.4, causal)
        assert np.array_equal(o, oe) and np.array_equal(l, le)


def test_gqa_head_mapping_brute_force():
    """Query head h must read KV head h // (H / H_kv): heads 0,1 -> 0 and 2,3 -> 1 here
    (a modulo mapping h % H_kv would pair heads 0,2 and 1,3 and fails)."""
    r = rng(30)
    q = r.normal(size=(1, 4, 3, 2))
    k, v = r.normal(size=(1, 2, 4, 2)), r.normal(size=(1, 2, 4, 2))
    o, l = oracle.attention_dense(q, k, v, 0.8, False)
    for h, hk in ((0, 0), (1, 0), (2, 1), (3, 1)):
        ob, lb = _brute(q[0, h].tolist(), k[0, hk].tolist(), v[0, hk].tolist(), 0.8, False)
        assert np.abs(o[0, h] - ob).max() < TIGHT and np.abs(l[0, h] - lb).max() < TIGHT


def test_gqa_rejects_non_dividing_heads():
    r = rng(31)
    with pytest.raises(ValueError):
        oracle.attention_dense(r.normal(size=(1, 4, 2, 2)), r.normal(size=(1, 3, 2, 2)),
                               r.normal(size=(1, 3, 2, 2)), 1.0)


def test_gqa_varlen_equals_expanded_kv():
    r = rng(32)
    cu = np.array([0, 3, 7, 12], dtype=np.int32)
    q = r.normal(size=(12, 8, 4))
    k, v = r.normal(size=(12, 2, 4)), r.normal(size=(12, 2, 4))
    for causal in (False, True):
        o, l = oracle.attention_varlen(q, k, v, cu, cu, 0.5, causal)
        oe, le = oracle.attention_varlen(q, _expand_kv(k, 4, 1), _expand_kv(v, 4, 1), cu, cu, 0.5, causal)
        assert np.array_equal(o, oe) and np.array_equal(l, le)


def test_gqa_paged_decode_brute_force():
    r = rng(33)
    page, H, Hkv, d = 4, 4, 2, 3
    ctx = np.array([5, 9], dtype=np.int32)
    P = 5
    bt = np.array([[3, 0, 5], [1, 4, 2]], dtype=np.int32)   # page 5 = poison, never read
    kc, vc = r.normal(size=(P + 1, page, Hkv, d)), r.normal(size=(P + 1, page, Hkv, d))
    kc[P] = np.nan
    vc[P] = np.nan
    q = r.normal(size=(2, H, d))
    o, l = oracle.attention_decode_paged(q, kc, vc, bt, ctx, 0.6)
    for b, c in enumerate(ctx):
        for h in range(H):
            hk = h // (H // Hkv)
            ks = [kc[bt[b, t // page], t % page, hk].tolist() for t in range(c)]
            vs = [vc[bt[b, t // page], t % page, hk].tolist() for t in range(c)]
            ob, lb = _brute([q[b, h].tolist()], ks, vs, 0.6, False)
            assert np.abs(o[b, h] - ob[0]).max() < TIGHT and abs(l[b, h] - lb[0]) < TIGHT


# ----------------------------------------------------------------- store_kvcache

def test_store_kvcache_then_gather_round_trip():
    """Rows scattered through slot_mapping come back, in token order, from the block-
    table gather of the paged layout (token t of a sequence in page block_table[t //
    page], slot t % page)."""
    r = rng(40)
    page, Hkv, d = 4, 2, 3
    P = 6
    bt = np.array([4, 1, 5], dtype=np.int32)         # one sequence, 10 tokens, 3 pages
    T = 10
    slots = np.array([bt[t // page] * page + t % page for t in range(T)], dtype=np.int64)
    k, v = r.normal(size=(T, Hkv, d)), r.normal(size=(T, Hkv, d))
    kc0, vc0 = r.normal(size=(P, page, Hkv, d)), r.normal(size=(P, page, Hkv, d))
    kc, vc = oracle.store_kvcache(k, v, kc0, vc0, slots)
    for h in range(Hkv):
        assert np.array_equal(oracle.gather_paged(kc[:, :, h], bt, T, page), k[:, h])
        assert np.array_equal(oracle.gather_paged(vc[:, :, h], bt, T, page), v[:, h])
    # every other slot is untouched, and the inputs are not modified
    written = np.zeros((P, page), dtype=bool)
    written[slots // page, slots % page] = True
    assert np.array_equal(kc[~written], kc0[~written]) and np.array_equal(vc[~written], vc0[~written])


def test_store_kvcache_skips_padding_and_out_of_range_slots():
    r = rng(41)
    k, v = r.normal(size=(4, 1, 2)), r.normal(size=(4, 1, 2))
    kc0, vc0 = r.normal(size=(2, 4, 1, 2)), r.normal(size=(2, 4, 1, 2))
    kc, vc = oracle.store_kvcache(k, v, kc0, vc0, np.array([-1, 8, 3, -7]))
    expect_k = kc0.copy()
    expect_k[0, 3] = k[2]                             # only slot 3 is in range
    assert np.array_equal(kc, expect_k)
    assert np.array_equal(vc[0, 3], v[2]) and np.array_equal(np.delete(vc.reshape(8, 1, 2), 3, 0),
                                                              np.delete(vc0.reshape(8, 1, 2), 3, 0))


# ----------------------------------------------------------------- paged prefill

def _pages_for(lens, page, r, extra=1):
    n = [(L + page - 1) // page for L in lens]
    P = sum(n) + extra
    perm = r.permutation(P)
    bt = np.full((len(lens), max(n)), P - 1, dtype=np.int32)
    off = 0
    for s, m in enumerate(n):
        bt[s, :m] = perm[off:off + m]
        off += m
    return bt, P


def test_paged_prefill_brute_force_gather():
    """Keys gathered token by token through the block table; query rows are the last
    Lq tokens (bottom-right causal), e.g. a continued chunk after a cached prefix."""
    r = rng(60)
    page, H, Hkv, d = 4, 4, 2, 3
    lq, lk = [2, 5, 1], [9, 5, 6]
    bt, P = _pages_for(lk, page, r)
    kc, vc = r.normal(size=(P, page, Hkv, d)), r.normal(size=(P, page, Hkv, d))
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q = r.normal(size=(cq[-1], H, d))
    for causal in (False, True):
        o, l = oracle.attention_varlen_paged(q, kc, vc, cq, ck, bt, 0.9, causal)
        for s in range(3):
            for h in range(H):
                hk = h // (H // Hkv)
                ks = [kc[bt[s, t // page], t % page, hk].tolist() for t in range(lk[s])]
                vs = [vc[bt[s, t // page], t % page, hk].tolist() for t in range(lk[s])]
                ob, lb = _brute(q[cq[s]:cq[s + 1], h].tolist(), ks, vs, 0.9, causal)
                assert np.abs(o[cq[s]:cq[s + 1], h] - ob).max() < TIGHT
                assert np.abs(l[cq[s]:cq[s + 1], h] - lb).max() < TIGHT


def test_paged_prefill_last_row_is_decode():
    """With one new query token per sequence, paged prefill is the paged decode."""
    r = rng(61)
    page, H, d = 4, 2, 3
    lk = [7, 12]
    bt, P = _pages_for(lk, page, r)
    kc, vc = r.normal(size=(P, page, H, d)), r.normal(size=(P, page, H, d))
    q = r.normal(size=(2, H, d))
    o, l = oracle.attention_varlen_paged(q, kc, vc, np.array([0, 1, 2]), np.concatenate([[0], np.cumsum(lk)]),
                                         bt, 0.5, True)
    od, ld = oracle.attention_decode_paged(q, kc, vc, bt, np.array(lk), 0.5)
    assert np.abs(o - od).max() < TIGHT and np.abs(l - ld).max() < TIGHT


# ----------------------------------------------------------------- backward (gradients)

def _loss(q, k, v, do, scale, causal):
    o, _ = oracle.attention_rows(q, k, v, scale, causal)
    return float((o * do).sum())


@pytest.mark.parametrize("lq,lk,d,causal", [(3, 4, 2, False), (4, 4, 3, True), (2, 5, 2, True), (5, 3, 2, True)])
def test_backward_matches_finite_differences(lq, lk, d, causal):
    """Central differences of <O, dO> in float64 (independent of the chain rule)."""
    r = rng(70 + lq * 10 + lk)
    q, k, v, do = r.normal(size=(lq, d)), r.normal(size=(lk, d)), r.normal(size=(lk, d)), r.normal(size=(lq, d))
    dq, dk, dv = oracle.attention_backward_rows(q, k, v, do, 0.7, causal)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + eps
            up = _loss(q, k, v, do, 0.7, causal)
            x[idx] = x0 - eps
            dn = _loss(q, k, v, do, 0.7, causal)
            x[idx] = x0
            assert abs((up - dn) / (2 * eps) - g[idx]) < 1e-7


def test_backward_row_sum_identity():
    """D_i = sum_j P_ij dP_ij equals dO_i . O_i: the row sum the backward subtracts."""
    r = rng(75)
    q, k, v, do = (r.normal(size=(6, 4)) for _ in range(4))
    p = oracle.probabilities(q, k, 0.5, True)
    o, _ = oracle.attention_rows(q, k, v, 0.5, True)
    assert np.abs((p * (do @ v.T)).sum(axis=1) - (do * o).sum(axis=1)).max() < TIGHT


@pytest.mark.parametrize("causal", [False, True])
def test_backward_given_exact_o_matches_default(causal):
    """Handed the exact forward output, the backward forms D_i = dO_i . O_i from it and
    gets the same gradients as from P and dP (rows without keys included)."""
    r = rng(76)
    q, do = r.normal(size=(7, 4)), r.normal(size=(7, 3))
    k, v = r.normal(size=(5, 4)), r.normal(size=(5, 3))
    o, _ = oracle.attention_rows(q, k, v, 0.6, causal)
    a = oracle.attention_backward_rows(q, k, v, do, 0.6, causal)
    b = oracle.attention_backward_rows(q, k, v, do, 0.6, causal, o=o)
    for x, y in zip(a, b):
        assert np.abs(x - y).max() < TIGHT


def test_backward_given_o_shifts_only_the_row_sum():
    """A perturbed O moves D_i by dO_i . delta_i and nothing else: dQ_i shifts by
    -scale (dO_i . delta_i) sum_j P_ij K_j, dK_j by -scale sum_i P_ij (dO_i . delta_i) Q_i,
    and dV does not move (closed forms from dS = P (dP - D))."""
    r = rng(77)
    q, do = r.normal(size=(6, 4)), r.normal(size=(6, 3))
    k, v = r.normal(size=(6, 4)), r.normal(size=(6, 3))
    scale = 0.7
    o, _ = oracle.attention_rows(q, k, v, scale, True)
    delta = 1e-3 * r.normal(size=o.shape)
    dq0, dk0, dv0 = oracle.attention_backward_rows(q, k, v, do, scale, True, o=o)
    dq1, dk1, dv1 = oracle.attention_backward_rows(q, k, v, do, scale, True, o=o + delta)
    p = oracle.probabilities(q, k, scale, True)
    dd = (do * delta).sum(axis=1)                      # shift of D_i
    assert np.abs((dq1 - dq0) - (-scale * dd[:, None] * (p @ k))).max() < TIGHT
    assert np.abs((dk1 - dk0) - (-scale * (p * dd[:, None]).T @ q)).max() < TIGHT
    assert np.abs(dv1 - dv0).max() == 0.0


def test_backward_given_o_dense_and_varlen_pass_it_per_head():
    """The dense and varlen entries hand each head its own rows of O."""
    r = rng(78)
    q, do = r.normal(size=(1, 4, 5, 3)), r.normal(size=(1, 4, 5, 3))
    k, v = r.normal(size=(1, 2, 5, 3)), r.normal(size=(1, 2, 5, 3))
    o = r.normal(size=(1, 4, 5, 3))
    got = oracle.attention_backward_dense(q, k, v, do, 0.5, True, o=o)
    for h in range(4):
        hk = h // 2
        want = oracle.attention_backward_rows(q[0, h], k[0, hk], v[0, hk], do[0, h], 0.5, True, o=o[0, h])
        assert np.abs(got[0][0, h] - want[0]).max() < TIGHT
    t = lambda x: x[0].transpose(1, 0, 2)  # [1, H, N, d] -> [N, H, d]
    cu = np.array([0, 5])
    gv = oracle.attention_backward_varlen(t(q), t(k), t(v), t(do), cu, cu, 0.5, True, o=t(o))
    assert np.abs(gv[0] - t(got[0])).max() < TIGHT
    assert np.abs(gv[1] - t(got[1])).max() < TIGHT


def test_backward_gqa_sums_group_gradients():
    """A KV head's gradient is the sum over the query heads reading it: equal to the
    gradient of the explicitly expanded K/V summed back over the copies."""
    r = rng(76)
    q, do = r.normal(size=(1, 4, 5, 3)), r.normal(size=(1, 4, 5, 3))
    k, v = r.normal(size=(1, 2, 6, 3)), r.normal(size=(1, 2, 6, 3))
    dq, dk, dv = oracle.attention_backward_dense(q, k, v, do, 0.6, True)
    dqe, dke, dve = oracle.attention_backward_dense(q, _expand_kv(k, 2, 1), _expand_kv(v, 2, 1), do, 0.6, True)
    assert np.abs(dq - dqe).max() < TIGHT
    assert np.abs(dk - dke.reshape(1, 2, 2, 6, 3).sum(axis=2)).max() < TIGHT
    assert np.abs(dv - dve.reshape(1, 2, 2, 6, 3).sum(axis=2)).max() < TIGHT


def test_backward_optional_autograd_crosscheck():
    """torch autograd of the plain formula in float64 on the CPU (skipped without torch)."""
    torch = pytest.importorskip("torch")
    r = rng(77)
    q, k, v, do = r.normal(size=(7, 4)), r.normal(size=(9, 4)), r.normal(size=(9, 4)), r.normal(size=(7, 4))
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = (tq @ tk.T) * 0.5
    mask = torch.arange(9)[None, :] <= torch.arange(7)[:, None] + 2
    o = torch.softmax(s.masked_fill(~mask, float("-inf")), dim=1) @ tv
    o.backward(torch.tensor(do))
    dq, dk, dv = oracle.attention_backward_rows(q, k, v, do, 0.5, True)
    for a, b in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.abs(a - b.numpy()).max() < 1e-12


def _varlen_loss(q, k, v, do, cu_q, cu_k, scale, causal):
    o, _ = oracle.attention_varlen(q, k, v, cu_q, cu_k, scale, causal)
    return float(np.nansum(o * do))


def test_backward_varlen_matches_finite_differences():
    """Central differences of <O, dO> through the varlen forward oracle, on a ragged
    batch with grouped-query heads, Lq != Lk (bottom-right causal), an empty query
    range and a trailing row outside every sequence (its gradient must be zero)."""
    r = rng(78)
    cu_q = np.array([0, 2, 2, 5])      # lengths 2, 0, 3; row 5 belongs to no sequence
    cu_k = np.array([0, 3, 5, 7])      # lengths 3, 2, 2
    H, H_kv, d = 2, 1, 2
    q, do = r.normal(size=(6, H, d)), r.normal(size=(6, H, d))
    k, v = r.normal(size=(7, H_kv, d)), r.normal(size=(7, H_kv, d))
    dq, dk, dv = oracle.attention_backward_varlen(q, k, v, do, cu_q, cu_k, 0.8, True)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + eps
            up = _varlen_loss(q, k, v, do, cu_q, cu_k, 0.8, True)
            x[idx] = x0 - eps
            dn = _varlen_loss(q, k, v, do, cu_q, cu_k, 0.8, True)
            x[idx] = x0
            assert abs((up - dn) / (2 * eps) - g[idx]) < 1e-7, (idx, g[idx])
    assert not dq[5].any()                   # outside every sequence
    assert not dk[3:5].any() and not dv[3:5].any()  # keys of the sequence without queries


def test_backward_varlen_one_sequence_is_dense():
    """A one-sequence packed batch is the dense [1, H, N, d] case transposed."""
    r = rng(79)
    q, do = r.normal(size=(5, 4, 3)), r.normal(size=(5, 4, 3))
    k, v = r.normal(size=(7, 2, 3)), r.normal(size=(7, 2, 3))
    dq, dk, dv = oracle.attention_backward_varlen(q, k, v, do, np.array([0, 5]), np.array([0, 7]), 0.6, True)
    t = lambda x: np.ascontiguousarray(x.transpose(1, 0, 2))[None]
    rq, rk, rv = oracle.attention_backward_dense(t(q), t(k), t(v), t(do), 0.6, True)
    assert np.abs(dq - rq[0].transpose(1, 0, 2)).max() < TIGHT
    assert np.abs(dk - rk[0].transpose(1, 0, 2)).max() < TIGHT
    assert np.abs(dv - rv[0].transpose(1, 0, 2)).max() < TIGHT
