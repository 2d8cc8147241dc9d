/*
 * attn.h — C ABI of libattn.so: exact attention, forward and backward, for AMD Instinct
 * MI355X (gfx950).
 *
 * Three forward entry points, one per way the attention library is called on the
 * dlog.com.cn page "From standard Attention to FlashAttention and paged execution",
 * the KV-cache write that precedes them (attn_store_kvcache), and the backward of the
 * first two:
 *
 *   attn_fwd            fixed-length batched attention (section 3.1, the basic
 *                       fixed-length interface), layout [B, H, N, d] by default;
 *   attn_fwd_varlen     variable-length packed batch described by cumulative
 *                       sequence lengths (section 3.3, cu_seqlens);
 *   attn_decode_paged   one new query token per sequence attending its cached
 *                       K/V, read page by page through a block table
 *                       (sections 3.4 and "PagedAttention");
 *   attn_store_kvcache  the step's new K/V rows written into the page pools
 *                       through slot_mapping;
 *   attn_bwd            the gradients dQ, dK, dV of attn_fwd by recomputation;
 *   attn_bwd_varlen     the same for attn_fwd_varlen's packed batches.
 *
 * Each computes, per query row i, O_i = sum_j softmax_j(scale * q_i . k_j) v_j over
 * the admissible keys j, and the row's logsumexp lse_i = ln sum_j exp(scale * q_i . k_j)
 * (the statistic the tiled forward keeps for the backward pass: "L2.5 SOTA Kernel",
 * yulong.wang, sections 2.1 and 2.3).  S and P never reach memory.
 *
 * Conventions shared by all entry points
 * --------------------------------------
 * - Every pointer argument except the stride arrays is a DEVICE pointer, allocated
 *   and owned by the caller.  The library allocates nothing, frees nothing and keeps
 *   no state between calls; calls are reentrant and thread-safe.
 * - Element types: ATTN_DTYPE_BF16 (raw bfloat16) or ATTN_DTYPE_F32.  lse is always
 *   float32.  Accumulation is float32.
 * - Every call is asynchronous on `stream` (a hipStream_t passed as void*; NULL means
 *   the null stream).  Results are valid once the caller has synchronised that stream.
 * - Arguments are validated on the host before any launch; an invalid call returns a
 *   non-zero status and launches nothing.  Device-array CONTENTS (cu_seqlens,
 *   block_table, context_lens) are the caller's contract and are not checked: reading
 *   them would need a device-to-host copy.
 * - Causal masking: key j is admissible for query row i iff j <= i + (Lk - Lq)
 *   (bottom-right alignment; j <= i when Lq == Lk).  A row with no admissible key
 *   gets O = 0 and lse = -inf.
 * - Supported head dimension d: 64 or 128.  Other values are rejected
 *   (ATTN_ERR_UNSUPPORTED), never computed on a truncated tile.
 * - scale must be finite and > 0 (the pages use 1/sqrt(d)).
 * - Grouped-query attention (dlog.com.cn page, section "GQA: handled natively by the
 *   kernel, K/V not expanded"): K and V carry H_kv heads, H_kv divides H, and query
 *   head h reads KV head h / (H / H_kv) -- the head order of expanding each KV head
 *   H / H_kv times.  H_kv == H is plain multi-head attention, H_kv == 1 multi-query.
 *   K/V are never expanded in memory.  H_kv < 1 or H not a multiple of H_kv returns
 *   ATTN_ERR_INVALID_ARG (when H > 0).
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad scale, short workspace */
  ATTN_ERR_UNSUPPORTED = 2, /* valid request the library does not implement (d, dtype, alignment, page size) */
  ATTN_ERR_LAUNCH = 3,      /* the HIP runtime reported an error at launch */
  ATTN_ERR_SCRATCH_LIMIT = 4 /* attn_decode_paged_noalloc: the batch needs more than its fixed scratch */
} attn_status;

/* Bytes of the fixed device scratch array of attn_decode_paged_noalloc (one per GPU). */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

typedef enum { ATTN_DTYPE_F32 = 0, ATTN_DTYPE_BF16 = 1 } attn_dtype;

/*
 * attn_fwd — dense batched attention.
 *
 * q, o : logical [B, H, N, d];  k, v : logical [B, H_kv, Nk, d]; element type `dtype`
 *        (o has q's type).  The d dimension must be contiguous.
 * *_strides : three int64 element strides for the (b, h, n) dimensions of that tensor,
 *        or NULL for a contiguous [B, H, N, d] (q, o) / [B, H_kv, Nk, d] (k, v)
 *        tensor.  Strides make the
 *        [B, N, H, d] layout of the flash-attn interface and packed QKV / KV
 *        tensors ([B, N, 3, H, d], [B, N, 2, H, d]; page section 3.2) usable
 *        without copies.  Every row start must be 16-byte aligned.
 * lse  : float32 [B, H, N] contiguous, or NULL to skip it.
 * causal : 0 or 1 (bottom-right aligned when N != Nk).
 * B, H, N, Nk may be 0 (nothing is launched).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int H_kv, int N, int Nk, int d, int dtype,
             const int64_t* q_strides, const int64_t* k_strides,
             const int64_t* v_strides, const int64_t* o_strides,
             float scale, int causal, void* stream);

/*
 * attn_fwd_varlen — packed variable-length batch (bfloat16), keys contiguous or paged.
 *
 * q, o : [total_q, H, d] contiguous;  k, v : [total_k, H_kv, d] contiguous, or, when
 *        block_table is not NULL, the page pools [num_pages, page_size, H_kv, d].
 * cu_seqlens_q, cu_seqlens_k : int32 [num_seqs + 1] device arrays of prefix sums;
 *        sequence s owns Q rows [cu_seqlens_q[s], cu_seqlens_q[s+1]) and K/V rows
 *        [cu_seqlens_k[s], cu_seqlens_k[s+1]) (the page's example [0, 3, 7] is two
 *        sequences of 3 and 4 tokens).  Sequences never attend to each other.
 * max_seqlen_q / max_seqlen_k : upper bounds of the per-sequence lengths (they size
 *        the launch grid; a smaller value than the truth is a contract violation).
 * block_table, max_pages_per_seq, page_size : paged prefill (the page's v3 prefill
 *        entry continuing a chunk on the KV cache).  NULL block_table: contiguous K/V
 *        and the other two are ignored.  Otherwise sequence s's key j is slot
 *        j % page_size of page block_table[s * max_pages_per_seq + j / page_size];
 *        only cu_seqlens_k's differences (the key counts) are used; cu_seqlens_q may
 *        differ from cu_seqlens_k, and under the causal mask the query rows are the
 *        sequence's last tokens (bottom-right).  page_size must be a power of two
 *        >= 16 (else ATTN_ERR_UNSUPPORTED) and max_pages_per_seq * page_size >=
 *        max_seqlen_k (else ATTN_ERR_INVALID_ARG).  Every block-table entry a sequence
 *        uses must name a page of the pools (the pages are gathered by address).
 * lse  : float32 [total_q, H], or NULL.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int num_seqs,
                    int max_seqlen_q, int max_seqlen_k, int H, int H_kv, int d, int dtype,
                    const int32_t* block_table, int max_pages_per_seq, int page_size,
                    float scale, int causal, void* stream);

/*
 * attn_decode_paged_workspace_size — bytes of device workspace attn_decode_paged
 * needs for this batch shape (0 when nothing needs to be launched).
 */
size_t attn_decode_paged_workspace_size(int B, int H, int d, int max_context_len, int page_size);

/*
 * attn_decode_paged — decode step over a paged KV cache (bfloat16).
 *
 * q, o : [B, H, d] contiguous (one new query token per sequence).
 * k_cache, v_cache : [num_pages, page_size, H_kv, d] contiguous page pools.
 * block_table : int32 [B, max_pages_per_seq]; token t of sequence b lives in page
 *        block_table[b][t / page_size], slot t % page_size.  Entries past
 *        ceil(context_lens[b] / page_size) are never read.
 * context_lens : int32 [B], each in [0, max_context_len]; sequence b's query attends
 *        its keys [0, context_lens[b]) (with one query token, causal and non-causal
 *        coincide).  Slots past the context in the last page are never read.  A length
 *        above max_context_len is a caller error: the kernels truncate it to
 *        max_context_len (no read outside the block-table row or the workspace); a
 *        length of zero or below gives O = 0 and lse = -inf.
 * page_size : a positive multiple of 16.
 * lse  : float32 [B, H], or NULL.
 * workspace : device buffer of at least attn_decode_paged_workspace_size(...) bytes,
 *        owned by the caller; its contents on entry do not matter.  Concurrent calls
 *        must not share one workspace.
 */
int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                      const int32_t* block_table, int max_pages_per_seq,
                      const int32_t* context_lens, int B, int num_pages, int page_size,
                      int H, int H_kv, int d, int max_context_len, float scale,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged_noalloc — attn_decode_paged without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  The call allocates and frees
 * nothing; the caller still passes every input and output (same meaning, layout and
 * ownership as attn_decode_paged, and the same results bit for bit).
 *
 * The split partials go to a fixed device array inside the library,
 * ATTN_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held by each GPU the library runs on until
 * the process ends.  Limit: attn_decode_paged_workspace_size(B, H, d, max_context_len,
 * page_size) must not exceed it (at d = 128: B * H * ceil(max_context_len / 512) split
 * slots of 520 bytes, at most 129055), else ATTN_ERR_SCRATCH_LIMIT is returned before any
 * launch.  Nothing in the array needs to start at zero.
 * Every call on a GPU shares that GPU's array and leaves its partials there: calls that
 * overlap in time on one GPU (on different streams or from different host threads)
 * race, and the caller must serialise them.
 * The first call on a device looks up the array's device address (once per device, with
 * that device current); `stream` must belong to the current device.
 */
int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                              const int32_t* block_table, int max_pages_per_seq,
                              const int32_t* context_lens, int B, int num_pages, int page_size,
                              int H, int H_kv, int d, int max_context_len, float scale, void* stream);

/*
 * attn_store_kvcache — write one step's new K/V rows into the paged pools.
 *
 * The engine's attention step on the dlog.com.cn page first stores the step's k/v into
 * the paged KV cache through slot_mapping (prefill: a batch of new tokens; decode: one
 * token per sequence), then runs attention over the pools.
 *
 * k, v : token-major rows; token t's [H_kv, d] row starts at element t * k_token_stride
 *        (v_token_stride) and is contiguous.  Strides >= H_kv * d, so the K and V parts of
 *        a fused [T, (H + 2 H_kv) * d] projection output are accepted without copies.
 * slot_mapping : int64 [T] device array; token t's row goes to pool slot
 *        slot_mapping[t] = page * page_size + offset (block_table[b][i] = page holds
 *        tokens i * page_size ... of sequence b).  Slots outside [0, num_pages *
 *        page_size), -1 for padding among them, are skipped: nothing is written for them.
 *        Two tokens naming the same slot is a caller error (which row lands is not
 *        specified).
 * k_cache, v_cache : [num_pages, page_size, H_kv, d] contiguous pools, written in place.
 * dtype : ATTN_DTYPE_BF16 or ATTN_DTYPE_F32 (a byte copy; rows and strides must be
 *        multiples of 16 bytes, else ATTN_ERR_UNSUPPORTED).
 */
int attn_store_kvcache(const void* k, const void* v, void* k_cache, void* v_cache,
                       const int64_t* slot_mapping, int T, int H_kv, int d,
                       int64_t k_token_stride, int64_t v_token_stride,
                       int num_pages, int page_size, int dtype, void* stream);

/*
 * attn_bwd_workspace_size — bytes of device workspace attn_bwd needs (0 if none).
 */
size_t attn_bwd_workspace_size(int B, int H, int N);

/*
 * attn_bwd — gradients of dense attention by recomputation (bfloat16).
 *
 * The forward keeps only O and lse; the backward recomputes S and P from them and dO
 * and applies the chain rule through the softmax (m.lqnn.cn FlashAttention article,
 * section 4.3; yulong.wang "L2.5 SOTA Kernel", section 2.3).  With D_i = dO_i . O_i:
 * dV = P^T dO, dS = P (dO V^T - D), dQ = scale dS K, dK = scale dS^T Q; the gradient of
 * a KV head sums over the query heads that read it (grouped-query attention).
 *
 * q, o, dout, dq : [B, H, N, d] contiguous;  k, v, dk, dv : [B, H_kv, Nk, d] contiguous;
 * lse : float32 [B, H, N], the forward's logsumexp (natural log) for the same q, k, v,
 *       scale and causal flag (attn_fwd's lse output).
 * dq, dk, dv are overwritten (not accumulated into).  Every gradient entry is written
 * exactly once, without atomics, so the result is deterministic.
 * workspace : at least attn_bwd_workspace_size(B, H, N) bytes, 8-byte aligned, owned by
 *       the caller; its contents on entry do not matter.
 * dtype : ATTN_DTYPE_BF16 only; d 64 or 128; causal bottom-right as in attn_fwd.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             void* dq, void* dk, void* dv, int B, int H, int H_kv, int N, int Nk, int d, int dtype,
             float scale, int causal, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_bwd_varlen_workspace_size — bytes of device workspace attn_bwd_varlen needs
 * (0 if none): 8 bytes per query row and head.
 */
size_t attn_bwd_varlen_workspace_size(int total_q, int H);

/*
 * attn_bwd_varlen — gradients of variable-length attention by recomputation (bfloat16):
 * attn_bwd's method (same passages) applied to attn_fwd_varlen's packed batches
 * (dlog.com.cn page, section 3.3: sequence s owns rows [cu_seqlens_q[s],
 * cu_seqlens_q[s+1]) of the query-side tensors and [cu_seqlens_k[s], cu_seqlens_k[s+1])
 * of the key-side ones, and attends only to its own keys; causal bottom-right per
 * sequence).
 *
 * q, o, dout, dq : [total_q, H, d] contiguous;  k, v, dk, dv : [total_k, H_kv, d]
 *       contiguous (contiguous K/V only: the paged layout has no backward here);
 * lse : float32 [total_q, H], attn_fwd_varlen's logsumexp for the same inputs;
 * cu_seqlens_q, cu_seqlens_k : int32 [num_seqs + 1] on the device, non-decreasing,
 *       starting at 0, ending at most total_q / total_k;
 * max_seqlen_q, max_seqlen_k : upper bounds of the per-sequence lengths (they size the
 *       grid); total_q, total_k : the row counts of the tensors.
 * Rows of dq (dk, dv) outside every sequence are not written; every other gradient
 * entry is written exactly once, without atomics (deterministic), including zeros for
 * keys no query row attends.
 * workspace : at least attn_bwd_varlen_workspace_size(total_q, H) bytes, 8-byte aligned.
 * dtype : ATTN_DTYPE_BF16 only; d 64 or 128.  ATTN_ERR_UNSUPPORTED when 32 H d * 2
 * exceeds 2^31 - 1 (a tile's byte offsets are 32-bit).
 */
int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, const int32_t* cu_seqlens_q,
                    const int32_t* cu_seqlens_k, int num_seqs, int total_q, int total_k,
                    int max_seqlen_q, int max_seqlen_k, int H, int H_kv, int d, int dtype, float scale,
                    int causal, void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable name of a status code (static storage). */
const char* attn_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
