// Paged-KV decode for gfx950: one query token per sequence attends its cached keys,
// which are gathered page by page through the block table ("From standard Attention
// to FlashAttention and paged execution" (dlog.com.cn), sections 3.4 "Decode and the
// KV cache" and "PagedAttention": one kernel covers the whole batch).
//
// The work is HBM-bound (about one flop per byte read), so the design is about
// keeping many bytes in flight, not about matrix cores:
//  * split-KV: each (sequence, split of kDecodeSplit tokens, head) is one wavefront,
//    so a batch with a long-tailed length mix still yields thousands of equal-sized
//    work units;
//  * a wavefront reads 16-token chunks: 16 lanes x 16 bytes cover one token's
//    d = 128 head row, 4 token rows per load instruction, whole 256-byte segments;
//    the next two chunks are already in flight while one is reduced;
//  * q.k is a per-lane 8-term packed bf16 dot product (four v_dot2_f32_bf16) plus a
//    4-step DPP reduction inside each 16-lane row; P V pairs two tokens per packed dot;
//  * every lane-row runs the online-softmax recurrence (section 2.2 of the same page)
//    on its own tokens; the four rows are merged at the end with the same rescale;
//  * grouped-query attention (section "GQA" of the same page): query head h reads KV
//    head h / (H / H_kv) in place; a wavefront serves GW query heads of one KV head
//    from each K/V row it loads, and further heads of the group run in adjacent
//    wavefronts of the workgroup, so their reads of the same rows hit in cache.
// The second kernel merges the splits of each (sequence, head): with M = max_c m_c,
// O = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c, lse = (M + log2 L) ln 2, in split
// order (deterministic).  This is the online-softmax rescale applied to partial
// states ("L2.5 SOTA Kernel", yulong.wang, section 2.2).
#include "attn_internal.h"
#include "attn_tile.h"

namespace attn {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// a.lo * b.lo + a.hi * b.hi + c for packed bf16 pairs, fp32 accumulate
__device__ __forceinline__ float dot2(unsigned a, unsigned b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}
// (lo, hi) rounded to bf16 (nearest even) and packed
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(unsigned, bf16x2{(__bf16)lo, (__bf16)hi});
}

// DPP helpers inside 16-lane rows.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Sum over groups of LPT lanes (LPT = 8 or 16), result in every lane of the group.
template <int LPT>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kRowHalfMirror>(x);
  if (LPT == 16) x += dpp<kRowMirror>(x);
  return x;
}

template <int D>
struct Chunk {
  static constexpr int LPT = D / 8;       // lanes per token row (16 B each)
  static constexpr int TPI = 64 / LPT;    // token rows per load instruction
  static constexpr int NI = 16 / TPI;     // load instructions per 16-token chunk
  u32x4 k[NI];
  u32x4 v[NI];
};

// One wavefront per (sequence, split, GW consecutive query heads).  The GW heads share
// one KV head (GW divides H / H_kv), so each K/V row is loaded once for all of them.
template <int D, int GW>
__global__ __launch_bounds__(256) void decode_split_kernel(const DecodeParams p) {
  using C = Chunk<D>;
  constexpr int LPT = C::LPT, TPI = C::TPI, NI = C::NI;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hw = blockIdx.x * 4 + wave;  // head group of this wave; the groups of one
  const int split = blockIdx.y;          // (sequence, split) are adjacent in dispatch
                                         // order, so a page is read by all of them at
                                         // about the same time
  const int b = blockIdx.z;
  const int h0 = hw * GW;                // first query head of this wave
  if (h0 >= p.H) return;  // no barriers in this kernel: waves are independent
  const int ctx = p.context_lens[b];
  const int t_begin = split * p.split_len;
  if (t_begin >= ctx) return;
  const int t_end = min(ctx, t_begin + p.split_len);
  const int nchunks = (t_end - t_begin + 15) >> 4;

  const int g = lane / LPT;        // token row within an instruction
  const int cl = lane % LPT;       // 16-byte column chunk
  const int64_t tok_stride = (int64_t)p.H_kv * D;        // elements between slots
  const int64_t page_stride = (int64_t)p.page_size * tok_stride;
  const int hk = h0 / (p.H / p.H_kv);                     // the KV head of all GW heads
  const int64_t lane_off = (int64_t)hk * D + cl * 8;
  const uint16_t* __restrict__ Kc = (const uint16_t*)p.k_cache;
  const uint16_t* __restrict__ Vc = (const uint16_t*)p.v_cache;
  const int32_t* __restrict__ bt = p.block_table + (int64_t)b * p.max_pages;

  // q slices of this lane, one per head, as packed bf16 pairs; scores are scaled after
  // the sum
  u32x4 qp[GW];
#pragma unroll
  for (int j = 0; j < GW; ++j)
    qp[j] = *(const u32x4*)((const uint16_t*)p.q + ((int64_t)b * p.H + h0 + j) * D + cl * 8);

  auto load_chunk = [&](int u, C& c) {
    const int t0 = t_begin + 16 * u;  // multiple of 16, inside one page
    const int page = bt[t0 / p.page_size];
    const int slot0 = t0 % p.page_size;
    const int64_t base = (int64_t)page * page_stride + (int64_t)slot0 * tok_stride + lane_off;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = i * TPI + g;  // token within the chunk
      const bool ok = t0 + r < t_end;
      u32x4 kz = {0u, 0u, 0u, 0u}, vz = {0u, 0u, 0u, 0u};
      if (ok) {
        kz = *(const u32x4*)(Kc + base + (int64_t)r * tok_stride);
        vz = *(const u32x4*)(Vc + base + (int64_t)r * tok_stride);
      }
      c.k[i] = kz;
      c.v[i] = vz;
    }
  };

  float m2[GW], l[GW], acc[GW][8];
#pragma unroll
  for (int j = 0; j < GW; ++j) {
    m2[j] = kNegInf;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  }
  const float c2 = p.scale_log2;

  // q.k and the P V sums use packed bf16 dot products (v_dot2_f32_bf16, fp32
  // accumulate): q.k straight from the K words; for P V the lane's tokens of two
  // consecutive load instructions are paired, P rounded to bf16 (as for the matrix-core
  // product of the prefill kernel) and the two tokens' V elements packed by byte
  // permutes shared by all GW heads.
  static_assert(NI % 2 == 0, "token pairs");
  auto consume = [&](int u, const C& c) {
    const int t0 = t_begin + 16 * u;
    unsigned vpair[NI / 2][8];  // (token 2 i, token 2 i + 1) of element e, bf16 pairs
#pragma unroll
    for (int i = 0; i < NI / 2; ++i) {
      const u32x4 x = c.v[2 * i], y = c.v[2 * i + 1];
      const unsigned xw[4] = {x.x, x.y, x.z, x.w}, yw[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        vpair[i][2 * w] = __builtin_amdgcn_perm(yw[w], xw[w], 0x05040100u);      // low halves
        vpair[i][2 * w + 1] = __builtin_amdgcn_perm(yw[w], xw[w], 0x07060302u);  // high halves
      }
    }
#pragma unroll
    for (int j = 0; j < GW; ++j) {
      float s[NI];
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const u32x4 w = c.k[i];
        float d = dot2(w.x, qp[j].x, 0.f);
        d = dot2(w.y, qp[j].y, d);
        d = dot2(w.z, qp[j].z, d);
        d = dot2(w.w, qp[j].w, d);
        d = group_sum<LPT>(d);
        const bool ok = t0 + i * TPI + g < t_end;
        s[i] = ok ? d * c2 : kNegInf;
        mx = fmaxf(mx, s[i]);
      }
      const float mnew = fmaxf(m2[j], mx);
      const float muse = (mnew == kNegInf) ? 0.f : mnew;
      const float alpha = exp2_fast(m2[j] - muse);
      float rs = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] *= alpha;
#pragma unroll
      for (int i = 0; i < NI / 2; ++i) {
        const float p0 = exp2_fast(s[2 * i] - muse), p1 = exp2_fast(s[2 * i + 1] - muse);
        rs += p0 + p1;
        const unsigned pp = pack_bf16(p0, p1);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = dot2(pp, vpair[i][e], acc[j][e]);
      }
      l[j] = l[j] * alpha + rs;
      m2[j] = mnew;
    }
  };

  // three chunks in flight: consume u while u+1 and u+2 load
  C c0, c1, c2b;
  load_chunk(0, c0);
  if (nchunks > 1) load_chunk(1, c1);
  int u = 0;
  for (; u + 2 < nchunks; u += 3) {
    load_chunk(u + 2, c2b);
    consume(u, c0);
    if (u + 3 < nchunks) load_chunk(u + 3, c0);
    consume(u + 1, c1);
    if (u + 4 < nchunks) load_chunk(u + 4, c1);
    consume(u + 2, c2b);
  }
  if (u < nchunks) consume(u, c0);
  if (u + 1 < nchunks) consume(u + 1, c1);

  // merge the lane rows (token rows g) of this wavefront, head by head
#pragma unroll
  for (int j = 0; j < GW; ++j) {
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
      const float mo = __shfl_xor(m2[j], off);
      const float lo = __shfl_xor(l[j], off);
      const float mm = fmaxf(m2[j], mo);
      const float mu = (mm == kNegInf) ? 0.f : mm;
      const float a0 = exp2_fast(m2[j] - mu), a1 = exp2_fast(mo - mu);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ao = __shfl_xor(acc[j][e], off);
        acc[j][e] = acc[j][e] * a0 + ao * a1;
      }
      l[j] = l[j] * a0 + lo * a1;
      m2[j] = mm;
    }
    const int64_t slot = ((int64_t)b * p.H + h0 + j) * p.max_splits + split;
    if (g == 0) {
      float* dst = p.ws_acc + slot * D + cl * 8;
      *(float4*)dst = make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
      *(float4*)(dst + 4) = make_float4(acc[j][4], acc[j][5], acc[j][6], acc[j][7]);
    }
    if (lane == 0) *(float2*)(p.ws_ml + slot * 2) = make_float2(m2[j], l[j]);
  }
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;
__device__ __forceinline__ const lds_u8* lds_at(unsigned a) { return (const lds_u8*)a; }

// 16 bytes per lane from a per-lane global address into LDS at byte address `lds` +
// 16 lane (global_load_lds; the wait states after the M0 write are spelled out, as the
// hazard recognizer does not see inside the asm).
__device__ __forceinline__ void dma16_at(const void* src, unsigned lds) {
  const unsigned m0v = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(m0v), "v"(src)
               : "memory", "m0");
}

// Grouped-query decode on the matrix cores, for groups large enough that the per-head
// VALU work of decode_split_kernel would dominate: one wavefront per (sequence, split,
// KV head, block of up to 32 of the query heads that read it).  Those query heads are
// the rows of the forward kernel's tile products (padded to 32): S^T = K Q^T and
// O^T += V^T P^T on v_mfma_f32_32x32x16_bf16, so one K/V read serves every head of the
// block, with no cross-lane reductions and a cost that does not grow with the group.
// The split's tokens stream through LDS in tiles of 32, gathered from their pages
// (global_load_lds with per-lane addresses: the pools may exceed a buffer resource's
// reach), three tiles in flight per wavefront; each wavefront owns its LDS and runs
// without barriers.  K tiles are row-major with the 16-byte chunk index XOR-swizzled by
// the token, so that each lane quad loads 64 contiguous bytes of one token row and the
// operand reads (one token per lane) hit distinct banks; V tiles use the forward
// kernel's [32-column block][token][64 B] layout for the transposing reads.  The partial
// (acc, m, l) per (sequence, head, split) has the same form as decode_split_kernel's,
// so decode_combine_kernel merges either.
template <int D>
__global__ __launch_bounds__(64) void decode_mfma_kernel(const DecodeParams p) {
  constexpr int BN = 32;                // tokens per tile
  constexpr int DT = D / 16, DB = D / 32;
  constexpr int TILE = BN * D * 2;      // bytes of one K or V tile
  constexpr int NBLK = TILE / 1024;     // 1 KiB blocks per K or V tile
  constexpr int CPR = D / 8;            // 16-byte chunks per token row
  constexpr int RPB = 64 / CPR;         // token rows per K block
  constexpr int STAGES = 3;
  constexpr int VBLK = BN * 64;         // bytes per 32-column block of the V tile
  // per stage: K tile (swizzled row-major), V tile ([32-column block][token][64 B])
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * 2 * TILE];

  const int lane = threadIdx.x, half = lane >> 5, col = lane & 31;
  const int G = p.H / p.H_kv;
  const int gblocks = (G + 31) / 32;
  const int hk = blockIdx.x / gblocks, gb = blockIdx.x - hk * gblocks;
  const int split = blockIdx.y, b = blockIdx.z;
  const int ctx = p.context_lens[b];
  const int t_begin = split * p.split_len;
  if (t_begin >= ctx) return;  // no barriers in this kernel
  const int t_end = min(ctx, t_begin + p.split_len);
  const int ntiles = (t_end - t_begin + BN - 1) / BN;
  const int g = gb * 32 + col;  // query head (within the group) of this lane's column
  const bool hv = g < G;
  const int h = hk * G + g;

  // B operand Q^T: lane's column is head h; k-step t covers columns 16 t + 8 half ...
  bf16x8 qreg[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    u32x4 u = {0u, 0u, 0u, 0u};
    if (hv) u = *(const u32x4*)((const uint16_t*)p.q + ((int64_t)b * p.H + h) * D + 16 * t + 8 * half);
    qreg[t] = as_bf16x8(u);
  }
#pragma unroll
  for (int t = 0; t < DT; ++t) asm volatile("" : "+v"(qreg[t]));  // wait for Q here, once

  // swizzle of token row r: chunk c sits at slot c ^ sw(r)
  auto sw = [](int r) { return (r / (16 / CPR)) % CPR; };
  // DMA.  K block i: token RPB i + lane / CPR, slot lane % CPR (chunk slot ^ sw).
  // V block i: column block i / 2, token 16 (i % 2) + lane / 4, chunk 4 (i / 2) + lane % 4.
  // Each 16-token group of the tile lies in one page.
  const int64_t tok_bytes = (int64_t)p.H_kv * D * 2;
  const int64_t page_bytes = (int64_t)p.page_size * tok_bytes;
  const int gpp = p.page_size / 16;  // 16-token groups per page
  const int32_t* __restrict__ bt = p.block_table + (int64_t)b * p.max_pages;
  const uint8_t* const kpool = (const uint8_t*)p.k_cache + (int64_t)hk * D * 2;
  const uint8_t* const vpool = (const uint8_t*)p.v_cache + (int64_t)hk * D * 2;
  const unsigned lsm = (unsigned)(uintptr_t)(const lds_void*)smem;
  auto group_row = [&](int gi) -> int64_t {  // byte offset of the first token row of group gi
    const int pg = bt[gi / gpp];
    return (int64_t)pg * page_bytes + (int64_t)((gi % gpp) * 16) * tok_bytes;
  };
  auto row_of = [&](int tok, int64_t r0, int64_t r1) { return (tok < 16 ? r0 : r1) + (int64_t)(tok & 15) * tok_bytes; };
  auto issue = [&](int j) {
    const int t0 = t_begin + j * BN;              // a multiple of 32
    const int last = t_end - t0 - 1;              // last valid token of the tile (>= 0)
    const int gi = t0 >> 4;
    const int64_t r0 = group_row(gi);
    const int64_t r1 = last >= 16 ? group_row(gi + 1) : r0;
    const unsigned st = lsm + (unsigned)((j % STAGES) * 2 * TILE);
#pragma unroll
    for (int i = 0; i < NBLK; ++i) {
      const int tok = RPB * i + lane / CPR;
      const int chunk = (lane % CPR) ^ sw(tok);
      dma16_at(kpool + row_of(min(tok, last), r0, r1) + 16 * chunk, st + 1024 * i);
    }
    const int64_t vrow0 = row_of(min(lane >> 2, last), r0, r1);
    const int64_t vrow1 = row_of(min(16 + (lane >> 2), last), r0, r1);
#pragma unroll
    for (int i = 0; i < NBLK; ++i)
      dma16_at(vpool + ((i & 1) ? vrow1 : vrow0) + 16 * (lane & 3) + 64 * (i >> 1), st + TILE + 1024 * i);
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m2 = kNegInf, l = 0.f;
  const float c2 = p.scale_log2;
  // K operand of k-step t: token col, chunk 2 t + half, at col * 2 D + ((2 t ^ ks) * 16)
  const int ks = half ^ sw(col);
  const unsigned krow = (unsigned)(col * D * 2);
  const unsigned vread = (unsigned)((4 * half + (lane & 15) / 4) * 64 + 32 * ((lane >> 4) & 1) + 8 * (lane & 3));

#pragma unroll
  for (int j = 0; j < STAGES - 1; ++j)
    if (j < ntiles) issue(j);
  for (int j = 0; j < ntiles; ++j) {
    // this tile's 2 NBLK loads have landed; up to STAGES - 2 younger tiles stay in flight
    if (j + 1 < ntiles)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NBLK) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (j + STAGES - 1 < ntiles) issue(j + STAGES - 1);
    const unsigned st = lsm + (unsigned)((j % STAGES) * 2 * TILE);
    // S^T = K Q^T
    f32x16 s = f32x16{};
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const bf16x8 a = as_bf16x8(*(const lds_u32x4*)lds_at(st + krow + (unsigned)(((2 * t) ^ ks) * 16)));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[t], s, 0, 0, 0);
    }
    // online softmax per column (query head), base 2; tokens past the end -> -inf
    const int rem = t_end - (t_begin + j * BN);  // valid tokens in this tile
    float mx = kNegInf;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int tok = 8 * (v >> 2) + 4 * half + (v & 3);
      if (tok >= rem) s[v] = kNegInf;
      mx = fmaxf(mx, s[v]);
    }
    mx = fmaxf(mx, xor32(mx)) * c2;
    const float mnew = fmaxf(m2, mx);  // finite: every tile holds a valid token
    if (__builtin_amdgcn_ballot_w64(mnew > m2) != 0) {
      const float alpha = exp2_fast(m2 - mnew);  // 0 on the first tile
      l *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
      m2 = mnew;
    }
    bf16x8 pb[2];
    float rs = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float pv = exp2_fast(__builtin_fmaf(s[v], c2, -m2));
      rs += pv;
      pb[v >> 3][v & 7] = (__bf16)pv;
    }
    l += rs + xor32(rs);
    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int t4 = 0; t4 < 2; ++t4) {
        const unsigned vp = st + TILE + vread + db * VBLK + t4 * 1024;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)lds_at(vp));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)lds_at(vp + 512));
        const bf16x8 a = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[t4], oacc[db], 0, 0, 0);
      }
  }

  if (hv) {  // the partial state of head h: O^T column, (m, l)
    const int64_t slot = ((int64_t)b * p.H + h) * p.max_splits + split;
    float* dst = p.ws_acc + slot * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(float4*)(dst + 32 * db + 8 * i + 4 * half) =
            make_float4(oacc[db][4 * i], oacc[db][4 * i + 1], oacc[db][4 * i + 2], oacc[db][4 * i + 3]);
    if (half == 0) *(float2*)(p.ws_ml + slot * 2) = make_float2(m2, l);
  }
}

// One wavefront per (sequence, head); lane owns D/64 columns.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(const DecodeParams p) {
  constexpr int CPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= p.B * p.H) return;
  const int b = bh / p.H;
  const int ctx = p.context_lens[b];
  const int ns = (ctx + p.split_len - 1) / p.split_len;
  const int64_t base = (int64_t)bh * p.max_splits;

  float M = kNegInf;
  for (int c = 0; c < ns; ++c) M = fmaxf(M, p.ws_ml[(base + c) * 2]);
  const float Mu = (M == kNegInf) ? 0.f : M;
  float L = 0.f, o[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) o[e] = 0.f;
  for (int c = 0; c < ns; ++c) {
    const float2 ml = *(const float2*)(p.ws_ml + (base + c) * 2);
    const float w = exp2_fast(ml.x - Mu);
    L = __builtin_fmaf(w, ml.y, L);
    const float* a = p.ws_acc + (base + c) * D + lane * CPL;
#pragma unroll
    for (int e = 0; e < CPL; ++e) o[e] = __builtin_fmaf(w, a[e], o[e]);
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  uint16_t* O = (uint16_t*)p.o + (int64_t)bh * D + lane * CPL;
#pragma unroll
  for (int e = 0; e < CPL; ++e) O[e] = __builtin_bit_cast(uint16_t, (__bf16)(o[e] * inv));
  if (p.lse != nullptr && lane == 0) p.lse[bh] = L > 0.f ? (M + __log2f(L)) * kLn2 : kNegInf;
}

template <int D, int GW>
hipError_t launch_split(const DecodeParams& p, hipStream_t s) {
  const int waves = p.H / GW;  // head groups per (sequence, split)
  dim3 grid((unsigned)((waves + 3) / 4), (unsigned)p.max_splits, (unsigned)p.B);
  hipLaunchKernelGGL((decode_split_kernel<D, GW>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_t(const DecodeParams& p, hipStream_t s) {
  if (p.B <= 0 || p.H <= 0) return hipSuccess;
  if (p.max_splits > 0) {
    const int group = p.H / p.H_kv;
    hipError_t e;
#ifndef ATTN_DECODE_MFMA_MIN_GROUP
#define ATTN_DECODE_MFMA_MIN_GROUP 4
#endif
    if (group >= ATTN_DECODE_MFMA_MIN_GROUP) {  // larger groups: the matrix-core kernel
      dim3 grid((unsigned)(p.H_kv * ((group + 31) / 32)), (unsigned)p.max_splits, (unsigned)p.B);
      hipLaunchKernelGGL((decode_mfma_kernel<D>), grid, dim3(64), 0, s, p);
      e = hipGetLastError();
    } else if (D == 64 && group % 4 == 0)  // query heads per wavefront of the VALU kernel:
                                           // the largest of 4 (d = 64 only: register
                                           // budget), 2, 1 that divides the group size
      e = launch_split<D, 4>(p, s);
    else if (group % 2 == 0)
      e = launch_split<D, 2>(p, s);
    else
      e = launch_split<D, 1>(p, s);
    if (e != hipSuccess) return e;
  }
  const int nbh = p.B * p.H;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)((nbh + 3) / 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_paged(const DecodeParams& p, int d, hipStream_t s) {
  return d == 128 ? launch_t<128>(p, s) : launch_t<64>(p, s);
}

}  // namespace attn
