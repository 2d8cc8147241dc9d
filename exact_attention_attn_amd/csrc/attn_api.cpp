// Host side of libattn.so: argument validation, launch geometry and the C ABI
// declared in include/attn.h.  Nothing here allocates device memory, synchronises a
// stream or keeps state between calls.
#include "../../include/attn.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include "attn_internal.h"

namespace {

constexpr float kLog2e = 1.4426950408889634074f;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int fail(attn_status s) { return static_cast<int>(s); }

inline bool scale_ok(float scale) { return isfinite(scale) && scale > 0.f; }

// Strides (b, h, n) of a tensor, defaulting to contiguous [B, H, N, d].
inline void strides_or_default(const int64_t* s, int H, int N, int d, int64_t out[3]) {
  if (s) {
    out[0] = s[0];
    out[1] = s[1];
    out[2] = s[2];
  } else {
    out[2] = d;
    out[1] = (int64_t)N * d;
    out[0] = (int64_t)H * N * d;
  }
}

// Every row start must be 16-byte aligned for the vector loads/stores.
inline bool strides_aligned(const int64_t s[3], int esize) {
  for (int i = 0; i < 3; ++i)
    if (s[i] < 0 || ((s[i] * esize) & 15) != 0) return false;
  return true;
}

inline int check_launch(hipError_t e, hipStream_t stream) {
  if (e != hipSuccess) return fail(ATTN_ERR_LAUNCH);
  if (getenv("ATTN_DEBUG") != nullptr) {
    // test aid: surface asynchronous faults at the call that caused them (only the
    // caller's stream is waited for, as every launch of the call went there)
    if (hipStreamSynchronize(stream) != hipSuccess || hipGetLastError() != hipSuccess) return fail(ATTN_ERR_LAUNCH);
  }
  return ATTN_OK;
}

inline int n_splits(int max_ctx) { return (max_ctx + attn::kDecodeSplit - 1) / attn::kDecodeSplit; }

// Grouped-query heads: H_kv in [1, H] and dividing H (H == 0 launches nothing).
inline bool heads_ok(int H, int H_kv) { return H == 0 || (H_kv >= 1 && H_kv <= H && H % H_kv == 0); }

// Argument checks shared by the two paged-decode entries (host only: no device call).
// *nothing is set when there is nothing to launch (B * H == 0).
int decode_check(const void* q, const void* k_cache, const void* v_cache, const void* o, const float* lse,
                 const int32_t* block_table, int max_pages_per_seq, const int32_t* context_lens, int B,
                 int num_pages, int page_size, int H, int H_kv, int d, int max_context_len, float scale,
                 bool* nothing) {
  *nothing = false;
  if (B < 0 || H < 0 || num_pages < 0 || max_pages_per_seq < 0 || max_context_len < 0)
    return fail(ATTN_ERR_INVALID_ARG);
  if (!heads_ok(H, H_kv)) return fail(ATTN_ERR_INVALID_ARG);
  if (!scale_ok(scale)) return fail(ATTN_ERR_INVALID_ARG);
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED);
  if (page_size <= 0 || (page_size % 16) != 0) return fail(ATTN_ERR_UNSUPPORTED);
  if ((int64_t)B * H == 0) {
    *nothing = true;
    return ATTN_OK;
  }
  if (!q || !o || !context_lens) return fail(ATTN_ERR_INVALID_ARG);
  if (!aligned16(q) || !aligned16(o)) return fail(ATTN_ERR_UNSUPPORTED);
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(ATTN_ERR_INVALID_ARG);
  if (max_context_len > 0) {
    if (!k_cache || !v_cache || !block_table) return fail(ATTN_ERR_INVALID_ARG);
    if (!aligned16(k_cache) || !aligned16(v_cache)) return fail(ATTN_ERR_UNSUPPORTED);
    if ((int64_t)max_pages_per_seq * page_size < max_context_len) return fail(ATTN_ERR_INVALID_ARG);
  }
  return ATTN_OK;
}

// Launch of a checked paged decode with its split partials in `workspace`.
int decode_launch(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                  const int32_t* block_table, int max_pages_per_seq, const int32_t* context_lens, int B,
                  int page_size, int H, int H_kv, int d, int max_context_len, float scale, void* workspace,
                  void* stream) {
  attn::DecodeParams p{};
  p.q = q; p.k_cache = k_cache; p.v_cache = v_cache; p.o = o; p.lse = lse;
  p.block_table = block_table; p.context_lens = context_lens;
  p.B = B; p.H = H; p.H_kv = H_kv; p.max_pages = max_pages_per_seq; p.page_size = page_size;
  p.split_len = attn::kDecodeSplit;
  p.max_ctx = max_context_len;
  p.max_splits = max_context_len > 0 ? n_splits(max_context_len) : 0;
  const size_t slots = (size_t)B * H * p.max_splits;
  p.ws_acc = static_cast<float*>(workspace);
  p.ws_ml = p.ws_acc ? p.ws_acc + slots * d : nullptr;
  p.scale_log2 = scale * kLog2e;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return check_launch(attn::launch_decode_paged(p, d, s), s);
}

static_assert(attn::kNoAllocScratchBytes == ATTN_NOALLOC_SCRATCH_BYTES, "scratch size of include/attn.h");

}  // namespace

extern "C" {

int attn_version(void) { return 300; }

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_SCRATCH_LIMIT: return "needs more scratch than the fixed device array of the no-allocation entry holds";
    default: return "unknown status";
  }
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int H_kv, int N, int Nk, int d, int dtype,
             const int64_t* q_strides, const int64_t* k_strides,
             const int64_t* v_strides, const int64_t* o_strides,
             float scale, int causal, void* stream) {
  if (B < 0 || H < 0 || N < 0 || Nk < 0) return fail(ATTN_ERR_INVALID_ARG);
  if (!heads_ok(H, H_kv)) return fail(ATTN_ERR_INVALID_ARG);
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG);
  if (!scale_ok(scale)) return fail(ATTN_ERR_INVALID_ARG);
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F32) return fail(ATTN_ERR_UNSUPPORTED);
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED);
  if ((int64_t)B * H * N == 0) return ATTN_OK;  // no query rows: nothing to write
  if (!q || !o || (Nk > 0 && (!k || !v))) return fail(ATTN_ERR_INVALID_ARG);
  const int esize = dtype == ATTN_DTYPE_BF16 ? 2 : 4;
  int64_t qs[3], ks[3], vs[3], os[3];
  strides_or_default(q_strides, H, N, d, qs);
  strides_or_default(k_strides, H_kv, Nk, d, ks);
  strides_or_default(v_strides, H_kv, Nk, d, vs);
  strides_or_default(o_strides, H, N, d, os);
  if (!aligned16(q) || !aligned16(o) || (Nk > 0 && (!aligned16(k) || !aligned16(v))))
    return fail(ATTN_ERR_UNSUPPORTED);
  if (!strides_aligned(qs, esize) || !strides_aligned(ks, esize) || !strides_aligned(vs, esize) ||
      !strides_aligned(os, esize))
    return fail(ATTN_ERR_UNSUPPORTED);
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(ATTN_ERR_INVALID_ARG);
  // key-tile byte offsets are 32-bit: 64 rows of K/V must span less than 2 GiB
  if (64 * ks[2] * esize > INT32_MAX || 64 * vs[2] * esize > INT32_MAX) return fail(ATTN_ERR_UNSUPPORTED);

  attn::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.q_sb = qs[0]; p.q_sh = qs[1]; p.q_sn = qs[2];
  p.k_sb = ks[0]; p.k_sh = ks[1]; p.k_sn = ks[2];
  p.v_sb = vs[0]; p.v_sh = vs[1]; p.v_sn = vs[2];
  p.o_sb = os[0]; p.o_sh = os[1]; p.o_sn = os[2];
  p.l_sb = (int64_t)H * N; p.l_sh = N; p.l_sn = 1;
  p.B = B; p.H = H; p.Nq = N; p.Nk = Nk;
  p.kv_group = H / H_kv;
  p.scale_log2 = scale * kLog2e;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == ATTN_DTYPE_BF16) {
    p.n_rb = (N + attn::kFwdBM - 1) / attn::kFwdBM;
    return check_launch(attn::launch_fwd_bf16(p, d, causal != 0, false, s), s);
  }
  p.n_rb = (N + attn::kFwdF32BM - 1) / attn::kFwdF32BM;
  return check_launch(attn::launch_fwd_f32(p, d, causal != 0, s), s);
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int num_seqs,
                    int max_seqlen_q, int max_seqlen_k, int H, int H_kv, int d, int dtype,
                    const int32_t* block_table, int max_pages_per_seq, int page_size,
                    float scale, int causal, void* stream) {
  if (num_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || H < 0) return fail(ATTN_ERR_INVALID_ARG);
  if (!heads_ok(H, H_kv)) return fail(ATTN_ERR_INVALID_ARG);
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG);
  if (!scale_ok(scale)) return fail(ATTN_ERR_INVALID_ARG);
  if (dtype != ATTN_DTYPE_BF16) return fail(ATTN_ERR_UNSUPPORTED);
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED);
  if ((int64_t)num_seqs * H * max_seqlen_q == 0) return ATTN_OK;
  if (!q || !o || !cu_seqlens_q || !cu_seqlens_k) return fail(ATTN_ERR_INVALID_ARG);
  if (max_seqlen_k > 0 && (!k || !v)) return fail(ATTN_ERR_INVALID_ARG);
  if (!aligned16(q) || !aligned16(o) || (max_seqlen_k > 0 && (!aligned16(k) || !aligned16(v))))
    return fail(ATTN_ERR_UNSUPPORTED);
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(ATTN_ERR_INVALID_ARG);
  int page_shift = 0;
  if (block_table != nullptr) {  // paged K/V: page size a power of two, at least 16
    if (page_size < 16 || (page_size & (page_size - 1)) != 0) return fail(ATTN_ERR_UNSUPPORTED);
    if (max_pages_per_seq < 0 || (int64_t)max_pages_per_seq * page_size < max_seqlen_k)
      return fail(ATTN_ERR_INVALID_ARG);
    while ((1 << page_shift) < page_size) ++page_shift;
  }

  attn::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.block_table = block_table;
  p.bt_stride = max_pages_per_seq;
  p.page_shift = page_shift;
  const int64_t tok = (int64_t)H * d, ktok = (int64_t)H_kv * d;
  p.q_sn = tok; p.q_sh = d;
  p.k_sn = ktok; p.k_sh = d;
  p.v_sn = ktok; p.v_sh = d;
  p.o_sn = tok; p.o_sh = d;
  p.l_sn = H; p.l_sh = 1;
  p.cu_q = cu_seqlens_q; p.cu_k = cu_seqlens_k;
  p.B = num_seqs; p.H = H; p.Nq = max_seqlen_q; p.Nk = max_seqlen_k;
  p.kv_group = H / H_kv;
  p.n_rb = (max_seqlen_q + attn::kFwdBM - 1) / attn::kFwdBM;
  p.scale_log2 = scale * kLog2e;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return check_launch(attn::launch_fwd_bf16(p, d, causal != 0, true, s), s);
}

size_t attn_decode_paged_workspace_size(int B, int H, int d, int max_context_len, int page_size) {
  (void)page_size;
  if (B <= 0 || H <= 0 || max_context_len <= 0 || (d != 64 && d != 128)) return 0;
  const size_t slots = (size_t)B * H * n_splits(max_context_len);
  return slots * (size_t)d * sizeof(float) + slots * 2 * sizeof(float);
}

int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                      const int32_t* block_table, int max_pages_per_seq,
                      const int32_t* context_lens, int B, int num_pages, int page_size,
                      int H, int H_kv, int d, int max_context_len, float scale,
                      void* workspace, size_t workspace_bytes, void* stream) {
  bool nothing = false;
  const int rc = decode_check(q, k_cache, v_cache, o, lse, block_table, max_pages_per_seq, context_lens, B,
                              num_pages, page_size, H, H_kv, d, max_context_len, scale, &nothing);
  if (rc != ATTN_OK || nothing) return rc;
  const size_t need = attn_decode_paged_workspace_size(B, H, d, max_context_len, page_size);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(ATTN_ERR_INVALID_ARG);
  return decode_launch(q, k_cache, v_cache, o, lse, block_table, max_pages_per_seq, context_lens, B, page_size, H,
                       H_kv, d, max_context_len, scale, workspace, stream);
}

int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                              const int32_t* block_table, int max_pages_per_seq,
                              const int32_t* context_lens, int B, int num_pages, int page_size,
                              int H, int H_kv, int d, int max_context_len, float scale, void* stream) {
  bool nothing = false;
  const int rc = decode_check(q, k_cache, v_cache, o, lse, block_table, max_pages_per_seq, context_lens, B,
                              num_pages, page_size, H, H_kv, d, max_context_len, scale, &nothing);
  if (rc != ATTN_OK || nothing) return rc;
  const size_t need = attn_decode_paged_workspace_size(B, H, d, max_context_len, page_size);
  if (need > attn::kNoAllocScratchBytes) return fail(ATTN_ERR_SCRATCH_LIMIT);
  void* ws = nullptr;
  if (need > 0 && attn::noalloc_scratch(&ws) != hipSuccess) return fail(ATTN_ERR_LAUNCH);
  return decode_launch(q, k_cache, v_cache, o, lse, block_table, max_pages_per_seq, context_lens, B, page_size, H,
                       H_kv, d, max_context_len, scale, ws, stream);
}

size_t attn_bwd_workspace_size(int B, int H, int N) {
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  return (size_t)B * H * N * 2 * sizeof(float);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             void* dq, void* dk, void* dv, int B, int H, int H_kv, int N, int Nk, int d, int dtype,
             float scale, int causal, void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || H < 0 || N < 0 || Nk < 0) return fail(ATTN_ERR_INVALID_ARG);
  if (!heads_ok(H, H_kv)) return fail(ATTN_ERR_INVALID_ARG);
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG);
  if (!scale_ok(scale)) return fail(ATTN_ERR_INVALID_ARG);
  if (dtype != ATTN_DTYPE_BF16) return fail(ATTN_ERR_UNSUPPORTED);
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED);
  if ((int64_t)B * H == 0 || (int64_t)N + Nk == 0) return ATTN_OK;  // no gradient entries
  const bool rows = N > 0, keys = Nk > 0;
  if (rows && (!q || !o || !dout || !lse || !dq)) return fail(ATTN_ERR_INVALID_ARG);
  if (keys && (!k || !v || !dk || !dv)) return fail(ATTN_ERR_INVALID_ARG);
  const void* ptrs[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(ATTN_ERR_UNSUPPORTED);
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(ATTN_ERR_INVALID_ARG);
  const size_t need = attn_bwd_workspace_size(B, H, N);
  if (need > 0 && (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 7u)))
    return fail(ATTN_ERR_INVALID_ARG);
  // 32-bit byte offsets of one 32-row tile
  if ((int64_t)32 * d * 2 > INT32_MAX) return fail(ATTN_ERR_UNSUPPORTED);

  attn::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse;
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.ws = static_cast<float*>(workspace);
  p.rows = (int64_t)B * H * N;
  p.B = B; p.H = H; p.H_kv = H_kv; p.N = N; p.Nk = Nk;
  p.kv_group = H / H_kv;
  p.scale = scale;
  p.scale_log2 = scale * kLog2e;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return check_launch(attn::launch_bwd(p, d, causal != 0, false, s), s);
}

size_t attn_bwd_varlen_workspace_size(int total_q, int H) {
  if (total_q <= 0 || H <= 0) return 0;
  return (size_t)total_q * H * 2 * sizeof(float);
}

int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    void* dq, void* dk, void* dv, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                    int num_seqs, int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int H, int H_kv,
                    int d, int dtype, float scale, int causal, void* workspace, size_t workspace_bytes,
                    void* stream) {
  if (num_seqs < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || H < 0)
    return fail(ATTN_ERR_INVALID_ARG);
  if (max_seqlen_q > total_q || max_seqlen_k > total_k) return fail(ATTN_ERR_INVALID_ARG);
  if (!heads_ok(H, H_kv)) return fail(ATTN_ERR_INVALID_ARG);
  if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG);
  if (!scale_ok(scale)) return fail(ATTN_ERR_INVALID_ARG);
  if (dtype != ATTN_DTYPE_BF16) return fail(ATTN_ERR_UNSUPPORTED);
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED);
  if ((int64_t)num_seqs * H == 0 || (int64_t)max_seqlen_q + max_seqlen_k == 0) return ATTN_OK;
  if (!cu_seqlens_q || !cu_seqlens_k) return fail(ATTN_ERR_INVALID_ARG);
  const bool rows = max_seqlen_q > 0, keys = max_seqlen_k > 0;
  if (rows && (!q || !o || !dout || !lse || !dq)) return fail(ATTN_ERR_INVALID_ARG);
  if (keys && (!k || !v || !dk || !dv)) return fail(ATTN_ERR_INVALID_ARG);
  const void* ptrs[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(ATTN_ERR_UNSUPPORTED);
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(ATTN_ERR_INVALID_ARG);
  const size_t need = attn_bwd_varlen_workspace_size(total_q, H);
  if (need > 0 && (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 7u)))
    return fail(ATTN_ERR_INVALID_ARG);
  // 32-bit byte offsets of one 32-row tile of token rows
  if ((int64_t)32 * H * d * 2 > INT32_MAX) return fail(ATTN_ERR_UNSUPPORTED);

  attn::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse;
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.ws = static_cast<float*>(workspace);
  p.cu_q = cu_seqlens_q; p.cu_k = cu_seqlens_k;
  p.rows = (int64_t)total_q * H;
  p.B = num_seqs; p.H = H; p.H_kv = H_kv; p.N = max_seqlen_q; p.Nk = max_seqlen_k;
  p.total_q = total_q; p.total_k = total_k;
  p.kv_group = H / H_kv;
  p.scale = scale;
  p.scale_log2 = scale * kLog2e;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return check_launch(attn::launch_bwd(p, d, causal != 0, true, s), s);
}

int attn_store_kvcache(const void* k, const void* v, void* k_cache, void* v_cache,
                       const int64_t* slot_mapping, int T, int H_kv, int d,
                       int64_t k_token_stride, int64_t v_token_stride,
                       int num_pages, int page_size, int dtype, void* stream) {
  if (T < 0 || H_kv < 0 || d < 0 || num_pages < 0 || page_size < 0) return fail(ATTN_ERR_INVALID_ARG);
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F32) return fail(ATTN_ERR_UNSUPPORTED);
  const int esize = dtype == ATTN_DTYPE_BF16 ? 2 : 4;
  const int64_t row = (int64_t)H_kv * d * esize;
  if (T == 0 || row == 0 || (int64_t)num_pages * page_size == 0) return ATTN_OK;  // nothing to write
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return fail(ATTN_ERR_INVALID_ARG);
  if (k_token_stride < (int64_t)H_kv * d || v_token_stride < (int64_t)H_kv * d) return fail(ATTN_ERR_INVALID_ARG);
  if ((row & 15) != 0 || row > INT32_MAX || ((k_token_stride * esize) & 15) != 0 || ((v_token_stride * esize) & 15) != 0)
    return fail(ATTN_ERR_UNSUPPORTED);
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache)) return fail(ATTN_ERR_UNSUPPORTED);
  if (reinterpret_cast<uintptr_t>(slot_mapping) & 7u) return fail(ATTN_ERR_INVALID_ARG);

  attn::StoreParams p{};
  p.k = k; p.v = v; p.k_cache = k_cache; p.v_cache = v_cache;
  p.slot_mapping = slot_mapping;
  p.k_stride_bytes = k_token_stride * esize;
  p.v_stride_bytes = v_token_stride * esize;
  p.num_slots = (int64_t)num_pages * page_size;
  p.T = T;
  p.row_bytes = (int)row;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return check_launch(attn::launch_store_kvcache(p, s), s);
}

}  // extern "C"
