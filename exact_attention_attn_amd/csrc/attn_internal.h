// Internal declarations shared by the host entry points and the kernel launchers of
// libattn.so.  Not part of the C ABI (that is include/attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Parameters of one dense or varlen forward launch.  Strides are in elements.
// Dense: tensor (b, h, n, :) starts at b*sb + h*sh + n*sn.
// Varlen: token t of head h starts at t*sn + h*sh (sb unused); sequence s owns
// tokens [cu[s], cu[s+1]).  For K and V, h is the KV head: query head h reads KV head
// h / kv_group.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int64_t l_sb, l_sh, l_sn;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int B;      // batch (dense) or number of sequences (varlen)
  int H;
  int Nq;     // dense: query length; varlen: max_seqlen_q
  int Nk;     // dense: key length;   varlen: max_seqlen_k
  int n_rb;   // query row blocks per (b, h)
  int kv_group;  // query heads per KV head (1: multi-head attention)
  // Paged K/V (varlen only): sequence b's key j is slot j & (2^page_shift - 1) of page
  // block_table[b * bt_stride + (j >> page_shift)]; k/v point at the pools and the
  // token stride k_sn / v_sn is the slot stride.  block_table == nullptr: contiguous.
  const int32_t* block_table;
  int bt_stride;
  int page_shift;
  float scale_log2;  // scale * log2(e): scores are handled in base-2 units
};

struct DecodeParams {
  const void* q;        // [B, H, d]
  const void* k_cache;  // [P, page, H_kv, d]
  const void* v_cache;
  void* o;              // [B, H, d]
  float* lse;           // [B, H] or null
  const int32_t* block_table;  // [B, max_pages]
  const int32_t* context_lens; // [B]
  float* ws_acc;        // [B, H, max_splits, d]   unnormalised partial outputs
  float* ws_ml;         // [B, H, max_splits, 2]   partial (m, l), base-2 units
  int B, H;
  int H_kv;             // query head h reads KV head h / (H / H_kv)
  int max_pages;
  int page_size;
  int split_len;        // tokens per split, a multiple of 16
  int max_splits;
  int max_ctx;          // context lengths are clamped to this (max_context_len)
  float scale_log2;
};

// Parameters of one store_kvcache launch.  Byte strides; rows are 16-byte multiples.
struct StoreParams {
  const void* k;            // token t's K row at k + t * k_stride_bytes
  const void* v;
  void* k_cache;            // slot s's row at k_cache + s * row_bytes
  void* v_cache;
  const int64_t* slot_mapping;  // [T]
  int64_t k_stride_bytes, v_stride_bytes;
  int64_t num_slots;        // num_pages * page_size
  int T;
  int row_bytes;            // H_kv * d * element size
};

// Parameters of one backward launch (contiguous bf16 tensors).
struct BwdParams {
  const void* q;      // [B, H, N, d]; varlen: [total_q, H, d]
  const void* k;      // [B, H_kv, Nk, d]; varlen: [total_k, H_kv, d]
  const void* v;
  const void* o;      // as q
  const void* dout;   // as q
  const float* lse;   // [B, H, N] (natural log); varlen: [total_q, H]
  void* dq;           // as q
  void* dk;           // as k
  void* dv;
  float* ws;          // (lse * log2 e, dO . O) per query row, in lse order
  const int32_t* cu_q;  // varlen: [B + 1] row starts of the B sequences (else null)
  const int32_t* cu_k;
  int64_t rows;       // query rows x heads: B H N, or total_q H
  int B, H, H_kv;
  int N, Nk;          // rows / keys per sequence; varlen: of the longest sequence
  int total_q, total_k;  // varlen: rows of the packed query-side / key-side tensors
  int units_q, units_k;  // varlen compact grids: blocks per head (0: one per max_seqlen block; set by the launcher)
  int kv_group;       // H / H_kv
  float scale;
  float scale_log2;
};

// Launchers (return the hipError_t of the launch).
hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, bool varlen, hipStream_t s);  // paged iff p.block_table
hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, hipStream_t s);
hipError_t launch_decode_paged(const DecodeParams& p, int d, hipStream_t s);

// Bytes of the fixed device scratch array used by attn_decode_paged_noalloc (one per GPU,
// held for the life of the process; the ATTN_NOALLOC_SCRATCH_BYTES of include/attn.h).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
// Device address of the current device's scratch array.  The first call on a device
// looks it up with that device current; later calls return the kept pointer.
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_store_kvcache(const StoreParams& p, hipStream_t s);
hipError_t launch_bwd(const BwdParams& p, int d, bool causal, bool varlen, hipStream_t s);

// Wavefronts per workgroup of the bf16 forward kernel; each owns 32 query rows.
#ifndef ATTN_FWD_NW
#define ATTN_FWD_NW 4
#endif
constexpr int kFwdNW = ATTN_FWD_NW;
// Tile configurations of the bf16 forward kernel: keys per K/V tile and wavefronts per
// SIMD (the register budget).  64-key tiles at 2 wavefronts per SIMD by default; causal
// variable-length (and paged) launches whose longest sequence is at most kFwdShortLen use
// 32-key tiles at 3 wavefronts per SIMD (less masked work on the many diagonal tiles of
// short sequences, and a third wavefront to cover the per-tile latencies).
constexpr int kFwdBN = 64, kFwdWPE = 2;
constexpr int kFwdShortBN = 32, kFwdShortWPE = 3;
constexpr int kFwdShortLen = 4096;
// Row-block height of the bf16 forward kernel (query rows per workgroup).
constexpr int kFwdBM = 32 * kFwdNW;
// Row-block height of the fp32 forward kernel (its four wavefronts split the keys).
constexpr int kFwdF32BM = 16;
// Tokens per decode split (a multiple of 16).
#ifndef ATTN_DECODE_SPLIT
#define ATTN_DECODE_SPLIT 512
#endif
constexpr int kDecodeSplit = ATTN_DECODE_SPLIT;

}  // namespace attn
