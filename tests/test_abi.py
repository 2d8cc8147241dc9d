"""The C ABI: the library loads, exports every function the header declares, and
rejects invalid requests on the host before any launch (runs without a GPU)."""
import ctypes
import os
import re

import pytest

import exact_attention_attn_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", src)))


def test_header_declares_the_three_entries():
    names = header_functions()
    for n in ("attn_fwd", "attn_fwd_varlen", "attn_decode_paged", "attn_decode_paged_workspace_size"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = attn.load()
    for n in header_functions():
        assert hasattr(lib, n), n
    assert set(header_functions()) == set(attn.EXPORTS)
    assert lib.attn_version() >= 200   # 2.0: grouped-query heads in all three entries


FAKE = ctypes.c_void_p(1 << 20)        # never dereferenced: validation fails first
FAKE_ODD = ctypes.c_void_p((1 << 20) + 2)


def fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, H=4, Hkv=4, N=64, Nk=64, d=128,
             dtype=attn.ATTN_DTYPE_BF16, qs=None, ks=None, vs=None, os_=None, scale=0.1, causal=0)
    a.update(kw)
    return attn.load().attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["N"], a["Nk"],
                                a["d"], a["dtype"], a["qs"], a["ks"], a["vs"], a["os_"], a["scale"],
                                a["causal"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=80), attn.ATTN_ERR_UNSUPPORTED),
    (dict(d=96), attn.ATTN_ERR_UNSUPPORTED),
    (dict(d=3), attn.ATTN_ERR_UNSUPPORTED),
    (dict(dtype=7), attn.ATTN_ERR_UNSUPPORTED),
    (dict(B=-1), attn.ATTN_ERR_INVALID_ARG),
    (dict(N=-5), attn.ATTN_ERR_INVALID_ARG),
    (dict(scale=0.0), attn.ATTN_ERR_INVALID_ARG),
    (dict(scale=-1.0), attn.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), attn.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("inf")), attn.ATTN_ERR_INVALID_ARG),
    (dict(causal=2), attn.ATTN_ERR_INVALID_ARG),
    (dict(q=None), attn.ATTN_ERR_INVALID_ARG),
    (dict(o=None), attn.ATTN_ERR_INVALID_ARG),
    (dict(k=None), attn.ATTN_ERR_INVALID_ARG),
    (dict(q=FAKE_ODD), attn.ATTN_ERR_UNSUPPORTED),
    (dict(v=FAKE_ODD), attn.ATTN_ERR_UNSUPPORTED),
    (dict(qs=(ctypes.c_int64 * 3)(64 * 128, 128 * 64, 129)), attn.ATTN_ERR_UNSUPPORTED),
    (dict(ks=(ctypes.c_int64 * 3)(-128, 128, 128)), attn.ATTN_ERR_UNSUPPORTED),
    (dict(lse=ctypes.c_void_p((1 << 20) + 1)), attn.ATTN_ERR_INVALID_ARG),
    (dict(Hkv=0), attn.ATTN_ERR_INVALID_ARG),      # grouped-query heads must divide H
    (dict(Hkv=3), attn.ATTN_ERR_INVALID_ARG),
    (dict(Hkv=8), attn.ATTN_ERR_INVALID_ARG),
    (dict(Hkv=-4), attn.ATTN_ERR_INVALID_ARG),
    (dict(B=0), attn.ATTN_OK),          # nothing to do: no launch
    (dict(N=0), attn.ATTN_OK),
    (dict(N=0, Hkv=2), attn.ATTN_OK),
    (dict(N=0, Hkv=1), attn.ATTN_OK),
])
def test_fwd_rejects_before_launch(kw, status):
    assert fwd(**kw) == status


def varlen(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, cq=FAKE, ck=FAKE, S=2, mq=16, mk=16, H=2, Hkv=2, d=128,
             dtype=attn.ATTN_DTYPE_BF16, bt=None, maxp=0, page=0, scale=0.1, causal=1)
    a.update(kw)
    return attn.load().attn_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"], a["S"],
                                       a["mq"], a["mk"], a["H"], a["Hkv"], a["d"], a["dtype"], a["bt"], a["maxp"],
                                       a["page"], a["scale"], a["causal"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=attn.ATTN_DTYPE_F32), attn.ATTN_ERR_UNSUPPORTED),
    (dict(d=32), attn.ATTN_ERR_UNSUPPORTED),
    (dict(cq=None), attn.ATTN_ERR_INVALID_ARG),
    (dict(ck=None), attn.ATTN_ERR_INVALID_ARG),
    (dict(S=-1), attn.ATTN_ERR_INVALID_ARG),
    (dict(mq=-1), attn.ATTN_ERR_INVALID_ARG),
    (dict(scale=0.0), attn.ATTN_ERR_INVALID_ARG),
    (dict(q=FAKE_ODD), attn.ATTN_ERR_UNSUPPORTED),
    (dict(Hkv=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(Hkv=3), attn.ATTN_ERR_INVALID_ARG),
    (dict(bt=FAKE, maxp=1, page=24), attn.ATTN_ERR_UNSUPPORTED),    # paged: power-of-two pages >= 16
    (dict(bt=FAKE, maxp=4, page=8), attn.ATTN_ERR_UNSUPPORTED),
    (dict(bt=FAKE, maxp=0, page=16), attn.ATTN_ERR_INVALID_ARG),     # 0 pages < 16 keys
    (dict(bt=FAKE, maxp=1, page=16, mk=17), attn.ATTN_ERR_INVALID_ARG),
    (dict(S=0), attn.ATTN_OK),
    (dict(mq=0), attn.ATTN_OK),
])
def test_varlen_rejects_before_launch(kw, status):
    assert varlen(**kw) == status


def decode(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, o=FAKE, lse=None, bt=FAKE, maxp=8, cl=FAKE, B=2, P=16, page=16, H=2,
             Hkv=2, d=128, maxctx=128, scale=0.1, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return attn.load().attn_decode_paged(a["q"], a["kc"], a["vc"], a["o"], a["lse"], a["bt"], a["maxp"], a["cl"],
                                         a["B"], a["P"], a["page"], a["H"], a["Hkv"], a["d"], a["maxctx"],
                                         a["scale"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(page=8), attn.ATTN_ERR_UNSUPPORTED),
    (dict(page=24), attn.ATTN_ERR_UNSUPPORTED),
    (dict(page=0), attn.ATTN_ERR_UNSUPPORTED),
    (dict(d=256), attn.ATTN_ERR_UNSUPPORTED),
    (dict(ws=None), attn.ATTN_ERR_INVALID_ARG),
    (dict(wsb=16), attn.ATTN_ERR_INVALID_ARG),
    (dict(bt=None), attn.ATTN_ERR_INVALID_ARG),
    (dict(cl=None), attn.ATTN_ERR_INVALID_ARG),
    (dict(maxp=4), attn.ATTN_ERR_INVALID_ARG),      # 4 pages * 16 < 128 tokens
    (dict(B=-2), attn.ATTN_ERR_INVALID_ARG),
    (dict(scale=-0.5), attn.ATTN_ERR_INVALID_ARG),
    (dict(kc=FAKE_ODD), attn.ATTN_ERR_UNSUPPORTED),
    (dict(Hkv=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(Hkv=4), attn.ATTN_ERR_INVALID_ARG),
    (dict(B=0), attn.ATTN_OK),
])
def test_decode_rejects_before_launch(kw, status):
    assert decode(**kw) == status


def decode_noalloc(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, o=FAKE, lse=None, bt=FAKE, maxp=8, cl=FAKE, B=2, P=16, page=16, H=2,
             Hkv=2, d=128, maxctx=128, scale=0.1)
    a.update(kw)
    return attn.load().attn_decode_paged_noalloc(a["q"], a["kc"], a["vc"], a["o"], a["lse"], a["bt"], a["maxp"],
                                                 a["cl"], a["B"], a["P"], a["page"], a["H"], a["Hkv"], a["d"],
                                                 a["maxctx"], a["scale"], None)


# d = 128: 520 bytes of partials per (sequence, head, 512-token split)
_SLOTS = attn.NOALLOC_SCRATCH_BYTES // 520


@pytest.mark.parametrize("kw,status", [
    (dict(page=8), attn.ATTN_ERR_UNSUPPORTED),
    (dict(d=80), attn.ATTN_ERR_UNSUPPORTED),
    (dict(bt=None), attn.ATTN_ERR_INVALID_ARG),
    (dict(maxp=4), attn.ATTN_ERR_INVALID_ARG),
    (dict(scale=0.0), attn.ATTN_ERR_INVALID_ARG),
    (dict(Hkv=3), attn.ATTN_ERR_INVALID_ARG),
    (dict(B=0), attn.ATTN_OK),
    # one split slot past the fixed scratch: B * H * splits = _SLOTS + 1
    (dict(B=_SLOTS + 1, H=1, Hkv=1, maxctx=512, maxp=32), attn.ATTN_ERR_SCRATCH_LIMIT),
    (dict(B=4, H=32, Hkv=8, maxctx=512 * (_SLOTS // 128 + 1), maxp=32 * (_SLOTS // 128 + 1)),
     attn.ATTN_ERR_SCRATCH_LIMIT),
])
def test_decode_noalloc_rejects_before_launch(kw, status):
    """The no-allocation decode entry checks its arguments like attn_decode_paged and
    refuses a batch whose split partials exceed its fixed scratch, before any launch."""
    assert decode_noalloc(**kw) == status


def test_noalloc_scratch_limit_matches_header():
    src = open(os.path.join(ROOT, "include", "attn.h")).read()
    assert "#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in src
    assert attn.NOALLOC_SCRATCH_BYTES == 64 << 20
    assert attn.status_string(attn.ATTN_ERR_SCRATCH_LIMIT).startswith("needs more scratch")


def test_workspace_size():
    ws = attn.attn_decode_paged_workspace_size
    assert ws(0, 32, 128, 8192, 16) == 0
    assert ws(64, 32, 128, 0, 16) == 0
    one = ws(1, 1, 128, 1, 16)
    assert one == 130 * 4
    assert ws(64, 32, 128, 8192, 16) == 64 * 32 * 16 * 130 * 4   # 512-token splits
    assert ws(64, 32, 128, 8193, 16) == 64 * 32 * 17 * 130 * 4
    assert ws(2, 2, 64, 100, 16) == 2 * 2 * 1 * 66 * 4


def test_status_strings():
    assert attn.status_string(0) == "ok"
    assert "unsupported" in attn.status_string(2)
    assert attn.status_string(99) == "unknown status"


def store(**kw):
    a = dict(k=FAKE, v=FAKE, kc=FAKE, vc=FAKE, slots=FAKE, T=16, Hkv=8, d=128, ks=8 * 128, vs=8 * 128,
             P=32, page=16, dtype=attn.ATTN_DTYPE_BF16)
    a.update(kw)
    return attn.load().attn_store_kvcache(a["k"], a["v"], a["kc"], a["vc"], a["slots"], a["T"], a["Hkv"], a["d"],
                                          a["ks"], a["vs"], a["P"], a["page"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), attn.ATTN_ERR_UNSUPPORTED),
    (dict(T=-1), attn.ATTN_ERR_INVALID_ARG),
    (dict(slots=None), attn.ATTN_ERR_INVALID_ARG),
    (dict(kc=None), attn.ATTN_ERR_INVALID_ARG),
    (dict(ks=8 * 128 - 8), attn.ATTN_ERR_INVALID_ARG),    # rows would overlap
    (dict(ks=8 * 128 + 4), attn.ATTN_ERR_UNSUPPORTED),    # 8-byte aligned only
    (dict(Hkv=1, d=4, ks=4, vs=4), attn.ATTN_ERR_UNSUPPORTED),   # 8-byte rows
    (dict(k=FAKE_ODD), attn.ATTN_ERR_UNSUPPORTED),
    (dict(slots=ctypes.c_void_p((1 << 20) + 4)), attn.ATTN_ERR_INVALID_ARG),
    (dict(T=0), attn.ATTN_OK),
    (dict(P=0), attn.ATTN_OK),
])
def test_store_kvcache_rejects_before_launch(kw, status):
    assert store(**kw) == status


def bwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, H=4, Hkv=2, N=64,
             Nk=64, d=128, dtype=attn.ATTN_DTYPE_BF16, scale=0.1, causal=1, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return attn.load().attn_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                                a["B"], a["H"], a["Hkv"], a["N"], a["Nk"], a["d"], a["dtype"], a["scale"],
                                a["causal"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=attn.ATTN_DTYPE_F32), attn.ATTN_ERR_UNSUPPORTED),
    (dict(d=96), attn.ATTN_ERR_UNSUPPORTED),
    (dict(Hkv=3), attn.ATTN_ERR_INVALID_ARG),
    (dict(scale=0.0), attn.ATTN_ERR_INVALID_ARG),
    (dict(causal=3), attn.ATTN_ERR_INVALID_ARG),
    (dict(lse=None), attn.ATTN_ERR_INVALID_ARG),
    (dict(dk=None), attn.ATTN_ERR_INVALID_ARG),
    (dict(do=None), attn.ATTN_ERR_INVALID_ARG),
    (dict(ws=None), attn.ATTN_ERR_INVALID_ARG),
    (dict(wsb=64 * 4 * 8 - 1), attn.ATTN_ERR_INVALID_ARG),
    (dict(dq=FAKE_ODD), attn.ATTN_ERR_UNSUPPORTED),
    (dict(B=-1), attn.ATTN_ERR_INVALID_ARG),
    (dict(B=0), attn.ATTN_OK),
    (dict(N=0, Nk=0), attn.ATTN_OK),
])
def test_bwd_rejects_before_launch(kw, status):
    assert bwd(**kw) == status


def test_bwd_workspace_size():
    assert attn.attn_bwd_workspace_size(2, 3, 5) == 2 * 3 * 5 * 8
    assert attn.attn_bwd_workspace_size(0, 3, 5) == 0


def bwd_varlen(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, cq=FAKE, ck=FAKE, S=3,
             Tq=300, Tk=400, mq=200, mk=250, H=4, Hkv=2, d=128, dtype=attn.ATTN_DTYPE_BF16, scale=0.1, causal=1,
             ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return attn.load().attn_bwd_varlen(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                                       a["cq"], a["ck"], a["S"], a["Tq"], a["Tk"], a["mq"], a["mk"], a["H"], a["Hkv"],
                                       a["d"], a["dtype"], a["scale"], a["causal"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=attn.ATTN_DTYPE_F32), attn.ATTN_ERR_UNSUPPORTED),
    (dict(d=96), attn.ATTN_ERR_UNSUPPORTED),
    (dict(Hkv=3), attn.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), attn.ATTN_ERR_INVALID_ARG),
    (dict(causal=2), attn.ATTN_ERR_INVALID_ARG),
    (dict(cq=None), attn.ATTN_ERR_INVALID_ARG),
    (dict(ck=None), attn.ATTN_ERR_INVALID_ARG),
    (dict(lse=None), attn.ATTN_ERR_INVALID_ARG),
    (dict(dv=None), attn.ATTN_ERR_INVALID_ARG),
    (dict(ws=None), attn.ATTN_ERR_INVALID_ARG),
    (dict(wsb=300 * 4 * 8 - 1), attn.ATTN_ERR_INVALID_ARG),
    (dict(mq=301), attn.ATTN_ERR_INVALID_ARG),          # longer than the tensor
    (dict(mk=401), attn.ATTN_ERR_INVALID_ARG),
    (dict(k=FAKE_ODD), attn.ATTN_ERR_UNSUPPORTED),
    (dict(S=-1), attn.ATTN_ERR_INVALID_ARG),
    (dict(S=0), attn.ATTN_OK),
    (dict(mq=0, mk=0), attn.ATTN_OK),
])
def test_bwd_varlen_rejects_before_launch(kw, status):
    assert bwd_varlen(**kw) == status


def test_bwd_varlen_workspace_size():
    assert attn.attn_bwd_varlen_workspace_size(300, 4) == 300 * 4 * 8
    assert attn.attn_bwd_varlen_workspace_size(0, 4) == 0


def test_binding_refuses_host_tensors():
    """The binding raises before the library is called when a tensor argument is not in
    GPU memory (a host address given to a kernel would fault the device)."""
    import torch
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        attn.attn_fwd(q, q, q)
    x = torch.zeros((8, 1, 64), dtype=torch.bfloat16)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        attn.attn_fwd_varlen(x, x, x, cu, cu, 8, 8)
    kc = torch.zeros((2, 16, 1, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        attn.attn_decode_paged(torch.zeros((1, 1, 64), dtype=torch.bfloat16), kc, kc,
                               torch.zeros((1, 2), dtype=torch.int32), torch.ones(1, dtype=torch.int32), 1)
    with pytest.raises(ValueError, match="GPU tensor"):
        attn.attn_store_kvcache(x[:, :, :], x, torch.zeros((1, 16, 1, 64), dtype=torch.bfloat16),
                                torch.zeros((1, 16, 1, 64), dtype=torch.bfloat16), torch.zeros(8, dtype=torch.int64))
