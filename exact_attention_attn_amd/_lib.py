"""ctypes binding of libattn.so (the C ABI in include/attn.h).

Argument marshalling only: torch tensors are turned into device pointers, sizes,
strides and the current HIP stream, and passed to the library.  Every step of the
computation runs in the library's kernels; there is no fallback of any kind.  If
libattn.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_LAUNCH, ATTN_ERR_SCRATCH_LIMIT = 0, 1, 2, 3, 4
NOALLOC_SCRATCH_BYTES = 64 << 20   # ATTN_NOALLOC_SCRATCH_BYTES
ATTN_DTYPE_F32, ATTN_DTYPE_BF16 = 0, 1

EXPORTS = ("attn_fwd", "attn_fwd_varlen", "attn_decode_paged", "attn_decode_paged_workspace_size",
           "attn_decode_paged_noalloc",
           "attn_store_kvcache", "attn_bwd", "attn_bwd_workspace_size", "attn_bwd_varlen",
           "attn_bwd_varlen_workspace_size", "attn_status_string", "attn_version")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


def load() -> ctypes.CDLL:
    """Load libattn.so (once).  Raises ImportError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m exact_attention_attn_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64p, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int64), ctypes.c_float, ctypes.c_size_t
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i64p, i64p, i64p, i64p, f32, i32, vp]
    lib.attn_fwd.restype = i32
    lib.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                    vp, i32, i32, f32, i32, vp]
    lib.attn_fwd_varlen.restype = i32
    lib.attn_decode_paged_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.attn_decode_paged_workspace_size.restype = sz
    lib.attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, i32, f32, vp, sz, vp]
    lib.attn_decode_paged.restype = i32
    lib.attn_decode_paged_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, i32, f32,
                                              vp]
    lib.attn_decode_paged_noalloc.restype = i32
    i64 = ctypes.c_int64
    lib.attn_store_kvcache.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i64, i64, i32, i32, i32, vp]
    lib.attn_store_kvcache.restype = i32
    lib.attn_bwd_workspace_size.argtypes = [i32, i32, i32]
    lib.attn_bwd_workspace_size.restype = sz
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    lib.attn_bwd.restype = i32
    lib.attn_bwd_varlen_workspace_size.argtypes = [i32, i32]
    lib.attn_bwd_varlen_workspace_size.restype = sz
    lib.attn_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                    i32, i32, f32, i32, vp, sz, vp]
    lib.attn_bwd_varlen.restype = i32
    lib.attn_status_string.argtypes = [i32]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().attn_status_string(status).decode()


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return ATTN_DTYPE_BF16
    if t.dtype == torch.float32:
        return ATTN_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _strides3(t):
    if t.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    return (ctypes.c_int64 * 3)(*t.stride()[:3])


def _check(rc: int, where: str):
    if rc != ATTN_OK:
        raise AttnError(rc, where)


def _on_device(where: str, device, **tensors):
    """Every tensor argument must live in GPU memory on ``device``: the library takes
    raw device pointers, and a host address handed to a kernel would fault."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda or t.device != device:
            raise ValueError(f"{where}: {name} must be a GPU tensor on {device} (got {t.device})")


def _check_out(where: str, name: str, t, shape, dtype, contiguous: bool = True):
    """A caller-given output must have the shape, dtype (and contiguity) the kernels
    write: they store every element of the expected shape."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{where}: {name} must be {dtype} {tuple(shape)} (got {t.dtype} {tuple(t.shape)})")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{where}: {name} must be contiguous")


def _check_workspace(where: str, ws, need: int):
    if ws is None:
        return
    if not ws.is_contiguous():
        raise ValueError(f"{where}: workspace must be contiguous")
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"{where}: workspace holds {ws.numel() * ws.element_size()} bytes, needs {need}")


def attn_fwd(q, k, v, scale: float | None = None, causal: bool = False, out=None, lse=None,
             with_lse: bool = True, stream=None):
    """Dense attention.  q [B, H, N, d], k/v [B, H_kv, Nk, d] (bf16 or fp32, any strides
    with a contiguous last dim; H_kv divides H: grouped-query attention when smaller).
    Returns (o, lse) with o like q and lse float32 [B, H, N] (None when ``with_lse``
    is false)."""
    torch = _torch()
    lib = load()
    B, H, N, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, Nk, d) or v.shape != (B, Hkv, Nk, d):
        raise ValueError("k and v must be [B, H_kv, Nk, d] matching q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    _on_device("attn_fwd", q.device, q=q, k=k, v=v, out=out, lse=lse)
    _check_out("attn_fwd", "out", out, (B, H, N, d), q.dtype, contiguous=False)
    _check_out("attn_fwd", "lse", lse, (B, H, N), torch.float32)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty((B, H, N, d), dtype=q.dtype, device=q.device) if out is None else out
    if with_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    rc = lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse) if with_lse else None,
                      B, H, Hkv, N, Nk, d, _dtype_code(q), _strides3(q), _strides3(k), _strides3(v),
                      _strides3(o), scale, int(bool(causal)), _stream(stream))
    _check(rc, "attn_fwd")
    return o, (lse if with_lse else None)


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                    scale: float | None = None, causal: bool = False, out=None, lse=None,
                    with_lse: bool = True, stream=None, block_table=None):
    """Packed variable-length attention.  q [total_q, H, d]; k/v [total_k, H_kv, d]
    contiguous bf16 (H_kv divides H), or with ``block_table`` (int32 [num_seqs,
    max_pages]) the page pools [num_pages, page, H_kv, d] (paged prefill);
    cu_seqlens_* int32 device tensors [num_seqs + 1].  Returns (o [total_q, H, d],
    lse float32 [total_q, H])."""
    torch = _torch()
    lib = load()
    tq, H, d = q.shape
    if block_table is None:
        Hkv = k.shape[1]
        if k.shape[2] != d or v.shape != k.shape:
            raise ValueError("k and v must be [total_k, H_kv, d] matching q")
        bt, maxp, page = None, 0, 0
    else:
        Hkv, page = k.shape[2], k.shape[1]
        if k.dim() != 4 or k.shape[3] != d or v.shape != k.shape:
            raise ValueError("paged k and v must be [num_pages, page, H_kv, d] matching q")
        if block_table.dtype != torch.int32 or not block_table.is_contiguous():
            raise TypeError("block_table must be a contiguous int32 tensor")
        bt, maxp = block_table, block_table.shape[1]
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("varlen tensors must be contiguous [tokens, H, d]")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    num_seqs = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != num_seqs + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    if not cu_seqlens_q.is_contiguous() or not cu_seqlens_k.is_contiguous():
        raise ValueError("cu_seqlens must be contiguous")
    _on_device("attn_fwd_varlen", q.device, q=q, k=k, v=v, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k,
               block_table=block_table, out=out, lse=lse)
    _check_out("attn_fwd_varlen", "out", out, (tq, H, d), q.dtype)
    _check_out("attn_fwd_varlen", "lse", lse, (tq, H), torch.float32)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    if with_lse and lse is None:
        lse = torch.empty((tq, H), dtype=torch.float32, device=q.device)
    rc = lib.attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse) if with_lse else None,
                             _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), num_seqs, int(max_seqlen_q),
                             int(max_seqlen_k), H, Hkv, d, _dtype_code(q), _ptr(bt), maxp, page, scale,
                             int(bool(causal)), _stream(stream))
    _check(rc, "attn_fwd_varlen")
    return o, (lse if with_lse else None)


def attn_decode_paged_workspace_size(B: int, H: int, d: int, max_context_len: int, page_size: int = 16) -> int:
    return int(load().attn_decode_paged_workspace_size(B, H, d, max_context_len, page_size))


def attn_decode_paged(q, k_cache, v_cache, block_table, context_lens, max_context_len: int,
                      scale: float | None = None, workspace=None, out=None, lse=None,
                      with_lse: bool = True, stream=None):
    """Decode over a paged KV pool.  q [B, H, d]; k_cache/v_cache [num_pages, page, H_kv, d]
    bf16 contiguous (H_kv divides H); block_table int32 [B, max_pages]; context_lens int32 [B].
    ``workspace`` (uint8 device tensor) is allocated here when not given.  Returns
    (o [B, H, d], lse float32 [B, H])."""
    torch = _torch()
    lib = load()
    B, H, d = q.shape
    num_pages, page, Hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape[3] != d or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must be [num_pages, page, H_kv, d] matching q")
    for t in (q, k_cache, v_cache, block_table, context_lens):
        if not t.is_contiguous():
            raise ValueError("decode tensors must be contiguous")
    if block_table.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_table and context_lens must be int32")
    _on_device("attn_decode_paged", q.device, q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
               context_lens=context_lens, workspace=workspace, out=out, lse=lse)
    _check_out("attn_decode_paged", "out", out, (B, H, d), q.dtype)
    _check_out("attn_decode_paged", "lse", lse, (B, H), torch.float32)
    if context_lens.numel() != B or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("context_lens must be [B] and block_table [B, max_pages]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = attn_decode_paged_workspace_size(B, H, d, int(max_context_len), page)
    _check_workspace("attn_decode_paged", workspace, need)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q) if out is None else out
    if with_lse and lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    rc = lib.attn_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse) if with_lse else None,
                               _ptr(block_table), block_table.shape[1], _ptr(context_lens), B, num_pages,
                               page, H, Hkv, d, int(max_context_len), scale, _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "attn_decode_paged")
    return o, (lse if with_lse else None)


def attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, context_lens, max_context_len: int, out,
                              scale: float | None = None, lse=None, stream=None):
    """attn_decode_paged through the library's fixed device scratch: no workspace, and
    nothing is allocated here either (``out`` [B, H, d] and the optional ``lse``
    float32 [B, H] are the caller's).  Raises AttnError (ATTN_ERR_SCRATCH_LIMIT) when the
    batch needs more than NOALLOC_SCRATCH_BYTES of split partials.  Calls that overlap on
    one GPU share its scratch and race.  Returns (out, lse)."""
    torch = _torch()
    lib = load()
    B, H, d = q.shape
    num_pages, page, Hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape[3] != d or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must be [num_pages, page, H_kv, d] matching q")
    for t in (q, k_cache, v_cache, block_table, context_lens):
        if not t.is_contiguous():
            raise ValueError("decode tensors must be contiguous")
    if block_table.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_table and context_lens must be int32")
    if out is None:
        raise ValueError("attn_decode_paged_noalloc: out must be given (nothing is allocated)")
    _on_device("attn_decode_paged_noalloc", q.device, q=q, k_cache=k_cache, v_cache=v_cache,
               block_table=block_table, context_lens=context_lens, out=out, lse=lse)
    _check_out("attn_decode_paged_noalloc", "out", out, (B, H, d), q.dtype)
    _check_out("attn_decode_paged_noalloc", "lse", lse, (B, H), torch.float32)
    if context_lens.numel() != B or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("context_lens must be [B] and block_table [B, max_pages]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rc = lib.attn_decode_paged_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse),
                                       _ptr(block_table), block_table.shape[1], _ptr(context_lens), B, num_pages,
                                       page, H, Hkv, d, int(max_context_len), scale, _stream(stream))
    _check(rc, "attn_decode_paged_noalloc")
    return out, lse


def attn_store_kvcache(k, v, k_cache, v_cache, slot_mapping, stream=None):
    """Write new K/V rows into the page pools.  k, v [T, H_kv, d] (token stride free,
    [H_kv, d] contiguous; e.g. slices of a fused QKV output); k_cache/v_cache
    [num_pages, page, H_kv, d] contiguous, written in place; slot_mapping int64 [T]
    (slot = page * page_size + offset; out-of-pool slots such as -1 are skipped)."""
    torch = _torch()
    lib = load()
    T, Hkv, d = k.shape
    if v.shape != k.shape:
        raise ValueError("k and v must have the same shape [T, H_kv, d]")
    num_pages, page = k_cache.shape[0], k_cache.shape[1]
    if k_cache.shape[2:] != (Hkv, d) or v_cache.shape != k_cache.shape:
        raise ValueError("pools must be [num_pages, page, H_kv, d] matching k")
    for t in (k, v):
        if t.stride(2) != 1 or t.stride(1) != d:
            raise ValueError("each token's [H_kv, d] row must be contiguous")
    for t in (k_cache, v_cache, slot_mapping):
        if not t.is_contiguous():
            raise ValueError("pools and slot_mapping must be contiguous")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != T:
        raise TypeError("slot_mapping must be int64 [T]")
    if k.dtype != k_cache.dtype or v.dtype != k.dtype or v_cache.dtype != k.dtype:
        raise TypeError("k, v and the pools must share a dtype")
    _on_device("attn_store_kvcache", k.device, k=k, v=v, k_cache=k_cache, v_cache=v_cache, slot_mapping=slot_mapping)
    rc = lib.attn_store_kvcache(_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), T, Hkv, d,
                                k.stride(0), v.stride(0), num_pages, page, _dtype_code(k), _stream(stream))
    _check(rc, "attn_store_kvcache")
    return k_cache, v_cache


def attn_bwd_workspace_size(B: int, H: int, N: int) -> int:
    return int(load().attn_bwd_workspace_size(B, H, N))


def attn_bwd(q, k, v, o, lse, dout, scale: float | None = None, causal: bool = False, dq=None, dk=None,
             dv=None, workspace=None, stream=None):
    """Gradients of attn_fwd.  q, o, dout [B, H, N, d]; k, v [B, H_kv, Nk, d] (contiguous
    bf16); lse float32 [B, H, N] from the forward.  Returns (dq, dk, dv)."""
    torch = _torch()
    lib = load()
    B, H, N, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, Nk, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, H_kv, Nk, d] matching q")
    if o.shape != q.shape or dout.shape != q.shape or lse.shape != (B, H, N):
        raise ValueError("o and dout must match q, lse must be [B, H, N]")
    for t in (q, k, v, o, dout, lse):
        if not t.is_contiguous():
            raise ValueError("backward tensors must be contiguous")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    _on_device("attn_bwd", q.device, q=q, k=k, v=v, o=o, lse=lse, dout=dout, dq=dq, dk=dk, dv=dv,
               workspace=workspace)
    _check_out("attn_bwd", "dq", dq, q.shape, q.dtype)
    _check_out("attn_bwd", "dk", dk, k.shape, k.dtype)
    _check_out("attn_bwd", "dv", dv, v.shape, v.dtype)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = attn_bwd_workspace_size(B, H, N)
    _check_workspace("attn_bwd", workspace, need)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=q.device)
    rc = lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                      B, H, Hkv, N, Nk, d, _dtype_code(q), scale, int(bool(causal)), _ptr(workspace),
                      workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "attn_bwd")
    return dq, dk, dv


def attn_bwd_varlen_workspace_size(total_q: int, H: int) -> int:
    return int(load().attn_bwd_varlen_workspace_size(total_q, H))


def attn_bwd_varlen(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                    scale: float | None = None, causal: bool = False, dq=None, dk=None, dv=None, workspace=None,
                    stream=None):
    """Gradients of attn_fwd_varlen.  q, o, dout [total_q, H, d]; k, v [total_k, H_kv, d]
    (contiguous bf16); lse float32 [total_q, H] from the forward; cu_seqlens int32
    [num_seqs + 1] on the device.  Returns (dq, dk, dv); rows outside every sequence are
    left as they were in dq, dk, dv (zeros when they are allocated here)."""
    torch = _torch()
    lib = load()
    Tq, H, d = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    if k.shape != (Tk, Hkv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [total_k, H_kv, d] matching q")
    if o.shape != q.shape or dout.shape != q.shape or lse.shape != (Tq, H):
        raise ValueError("o and dout must match q, lse must be [total_q, H]")
    for t in (q, k, v, o, dout, lse, cu_seqlens_q, cu_seqlens_k):
        if not t.is_contiguous():
            raise ValueError("backward tensors must be contiguous")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    _on_device("attn_bwd_varlen", q.device, q=q, k=k, v=v, o=o, lse=lse, dout=dout, cu_seqlens_q=cu_seqlens_q,
               cu_seqlens_k=cu_seqlens_k, dq=dq, dk=dk, dv=dv, workspace=workspace)
    _check_out("attn_bwd_varlen", "dq", dq, q.shape, q.dtype)
    _check_out("attn_bwd_varlen", "dk", dk, k.shape, k.dtype)
    _check_out("attn_bwd_varlen", "dv", dv, v.shape, v.dtype)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.zeros_like(q) if dq is None else dq
    dk = torch.zeros_like(k) if dk is None else dk
    dv = torch.zeros_like(v) if dv is None else dv
    need = attn_bwd_varlen_workspace_size(Tq, H)
    _check_workspace("attn_bwd_varlen", workspace, need)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=q.device)
    rc = lib.attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                             _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), cu_seqlens_q.numel() - 1, Tq, Tk,
                             int(max_seqlen_q), int(max_seqlen_k), H, Hkv, d, _dtype_code(q), scale, int(bool(causal)),
                             _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "attn_bwd_varlen")
    return dq, dk, dv
