// Paged-KV decode for gfx950: one query token per sequence attends its cached keys,
// which are gathered page by page through the block table ("From standard Attention
// to FlashAttention and paged execution" (dlog.com.cn), sections 3.4 "Decode and the
// KV cache" and "PagedAttention": one kernel covers the whole batch).
//
// The work is HBM-bound (about one flop per byte read per query head), so the design is
// about keeping many bytes in flight:
//  * split-KV: each (sequence, split of kDecodeSplit tokens, KV head or head) is one
//    wavefront, so a batch with a long-tailed length mix still yields thousands of
//    equal-sized work units;
//  * one query head per KV head (decode_split_kernel, VALU): a wavefront reads 16-token
//    chunks, 16 lanes x 16 bytes covering one token's d = 128 head row, 4 token rows per
//    load instruction, the next two chunks in flight while one is reduced; q.k is a
//    per-lane packed bf16 dot product (four v_dot2_f32_bf16) plus a 4-step DPP
//    reduction inside each 16-lane row, P V pairs two tokens per packed dot; every
//    lane-row runs the online-softmax recurrence (section 2.2 of the same page) on its
//    own tokens and the four rows are merged at the end with the same rescale;
//  * grouped-query attention (section "GQA" of the same page; query head h reads KV head
//    h / (H / H_kv)): decode_mfma_kernel runs the query heads of one KV head as the rows
//    of matrix-core tiles, so each K/V row is read once for the whole group and the
//    per-head cost is absorbed by the MFMA.
// The combine kernel merges the splits of each (sequence, head): with M = max_c m_c,
// O = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c, lse = (M + log2 L) ln 2; the O
// sums run in split order and L by a fixed reduction tree (deterministic).  This is the
// online-softmax rescale applied to partial states ("L2.5 SOTA Kernel", yulong.wang,
// section 2.2).
#include "attn_internal.h"
#include "attn_tile.h"

#include <mutex>

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
// one KV head (GW divides H / H_kv), so each K/V row is loaded once for all of them
// (launched with GW = 1: grouped-query decode uses decode_mfma_kernel).
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
  const int ctx = min(p.context_lens[b], p.max_ctx);  // a longer length is a caller error: truncated
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
      if (ok) {  // read once: non-temporal loads (measured: 789 -> 721 us on the 64-sequence batch)
        kz = __builtin_nontemporal_load((const u32x4*)(Kc + base + (int64_t)r * tok_stride));
        vz = __builtin_nontemporal_load((const u32x4*)(Vc + base + (int64_t)r * tok_stride));
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
__device__ __forceinline__ const lds_u8* lds_at(unsigned a) { return (const lds_u8*)(uintptr_t)a; }

// Grouped-query decode on the matrix cores (the per-head VALU work of
// decode_split_kernel grows with the group): one wavefront per (sequence, split,
// KV head, block of up to 32 of the query heads that read it).  Those query heads are
// the rows of the forward kernel's tile products (padded to 32): S^T = K Q^T and
// O^T += V^T P^T on v_mfma_f32_32x32x16_bf16, so one K/V read serves every head of the
// block, with no cross-lane reductions and a cost that does not grow with the group.
// Memory side, as in decode_split_kernel: 16-token halves of a tile (one page group
// each) load into registers with whole-row coalesced loads, the next tile's two halves
// in flight while a tile is computed;
// each tile is then written to the wavefront's own LDS stage in the layouts the
// products read (no barriers: a wavefront reads only what it wrote).  K: row-major with
// the 16-byte chunk index XOR-swizzled by the token (conflict-free operand reads, one
// token per lane).  V: chunk c of token r at c * 512 + (r ^ 4 (c % 4)) * 16, read by
// ds_read_b64_tr_b16 as the V^T operand.  The partial (acc, m, l) per (sequence, head,
// split) has the same form as decode_split_kernel's, so decode_combine_kernel merges
// either.
template <int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_mfma_kernel(const DecodeParams p) {
  constexpr int BN = 32;                // tokens per tile
  constexpr int DT = D / 16, DB = D / 32;
  constexpr int TILE = BN * D * 2;      // bytes of one K or V tile
  constexpr int CPR = D / 8;            // 16-byte chunks per token row
  constexpr int TPI = 64 / CPR;         // token rows per load instruction
  constexpr int NI = 16 / TPI;          // load instructions per tensor per 16-token half
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * TILE];  // K tile, V tile

  const int lane = threadIdx.x, half = lane >> 5, col = lane & 31;
  const int G = p.H / p.H_kv;
  const int gblocks = (G + 31) / 32;
  const int hk = blockIdx.x / gblocks, gb = blockIdx.x - hk * gblocks;
  const int split = blockIdx.y, b = blockIdx.z;
  const int ctx = min(p.context_lens[b], p.max_ctx);  // a longer length is a caller error: truncated
  const int t_begin = split * p.split_len;
  if (t_begin >= ctx) return;  // no barriers in this kernel
  const int t_end = min(ctx, t_begin + p.split_len);
  const int nt = t_end - t_begin;            // tokens of this split
  const int ntiles = (nt + BN - 1) / BN;
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
  // wait for Q here, once: a wait left to the compiler would land in the tile loop as a
  // vmcnt(0) that also drains the next tile's loads
#pragma unroll
  for (int t = 0; t < DT; ++t) asm volatile("" : "+v"(qreg[t]));

  // swizzle of K token row r: chunk c sits at slot c ^ sw(r)
  auto sw = [](int r) { return (r / (16 / CPR)) % CPR; };
  const int lr = lane / CPR, lc = lane % CPR;  // token row within an instruction, chunk
  const int64_t tok_stride = (int64_t)p.H_kv * D;  // elements
  const int64_t page_stride = (int64_t)p.page_size * tok_stride;
  const int gpp = p.page_size / 16;                // 16-token groups per page
  const int32_t* __restrict__ bt = p.block_table + (int64_t)b * p.max_pages;
  const uint16_t* const Kc = (const uint16_t*)p.k_cache + (int64_t)hk * D + lc * 8;
  const uint16_t* const Vc = (const uint16_t*)p.v_cache + (int64_t)hk * D + lc * 8;
  // The pages of halves hf and hf + 1 (lanes 0 and 1 of one vector load, fetched a tile
  // ahead of use so that the load loop's own wait covers it); indices past the split's
  // last token group are clamped to it.
  const int gi0 = t_begin >> 4, gi_last = (t_end - 1) >> 4;
  auto fetch_pages = [&](int hf) { return bt[min(gi0 + hf + (lane & 1), gi_last) / gpp]; };
  // half hf of the split (tokens 16 hf .. 16 hf + 15, in page `page`) into registers;
  // tokens past the end read as zero (they are masked, and zero V rows keep 0 * V finite)
  auto load_half = [&](int hf, int page, u32x4* kr, u32x4* vr) {
    const int gi = gi0 + hf;
    const int64_t base = (int64_t)page * page_stride + (int64_t)((gi % gpp) * 16) * tok_stride;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = TPI * i + lr;
      u32x4 kz = {0u, 0u, 0u, 0u}, vz = {0u, 0u, 0u, 0u};
      if (16 * hf + r < nt) {  // read once: non-temporal loads (measured: 232 -> 206 us on the 16/8 batch)
        kz = __builtin_nontemporal_load((const u32x4*)(Kc + base + (int64_t)r * tok_stride));
        vz = __builtin_nontemporal_load((const u32x4*)(Vc + base + (int64_t)r * tok_stride));
      }
      kr[i] = kz;
      vr[i] = vz;
    }
  };
  const unsigned lsm = (unsigned)(uintptr_t)(const lds_void*)smem;
  // registers of half hf (position ph = 0 / 1 in the tile) -> the LDS tile
  auto store_half = [&](int ph, const u32x4* kr, const u32x4* vr) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = 16 * ph + TPI * i + lr;  // token row in the tile
      *(lds_u32x4*)lds_at(lsm + (unsigned)(r * D * 2 + ((lc ^ sw(r)) * 16))) = kr[i];
      *(lds_u32x4*)lds_at(lsm + TILE + (unsigned)(lc * 512 + ((r ^ (4 * (lc & 3))) * 16))) = vr[i];
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m2 = kNegInf, l = 0.f;
  const float c2 = p.scale_log2;
  // K operand of k-step t: token col, chunk 2 t + half, at col * 2 D + ((2 t ^ ks) * 16)
  const int ks = half ^ sw(col);
  const unsigned kread = lsm + (unsigned)(col * D * 2);
  // V^T operand: 8 bytes of chunk 4 db + j of rows 16 t4 + x and 16 t4 + x + 8
  const int vx = 4 * half + (lane & 15) / 4, vj = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const unsigned vlo = lsm + TILE + (unsigned)(vj * 512 + ((vx ^ (4 * vj)) * 16) + 8 * (lane & 1));
  const unsigned vhi = lsm + TILE + (unsigned)(vj * 512 + (((vx ^ (4 * vj)) ^ 8) * 16) + 8 * (lane & 1));

  auto compute = [&](int j) {
    // S^T = K Q^T
    f32x16 s = f32x16{};
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const bf16x8 a = as_bf16x8(*(const lds_u32x4*)lds_at(kread + (unsigned)(((2 * t) ^ ks) * 16)));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[t], s, 0, 0, 0);
    }
    // online softmax per column (query head), base 2; tokens past the end -> -inf
    const int rem = nt - j * BN;  // valid tokens in this tile
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
        const unsigned off = (unsigned)(db * 2048 + t4 * 256);
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)lds_at(vlo + off));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)lds_at(vhi + off));
        const bf16x8 a = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[t4], oacc[db], 0, 0, 0);
      }
  };

  // Two halves in registers: tile j's halves are written to LDS, then the next tile's
  // halves load into the same registers while tile j is computed.
  u32x4 kA[NI], vA[NI], kB[NI], vB[NI];
  int pg = fetch_pages(0);
  load_half(0, __builtin_amdgcn_readlane(pg, 0), kA, vA);
  load_half(1, __builtin_amdgcn_readlane(pg, 1), kB, vB);
  pg = fetch_pages(2);
  for (int j = 0; j < ntiles; ++j) {
    store_half(0, kA, vA);
    store_half(1, kB, vB);
    if (j + 1 < ntiles) {
      load_half(2 * j + 2, __builtin_amdgcn_readlane(pg, 0), kA, vA);
      load_half(2 * j + 3, __builtin_amdgcn_readlane(pg, 1), kB, vB);
      pg = fetch_pages(2 * j + 4);
    }
    compute(j);
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

// One wavefront per (sequence, head); lane owns D/64 columns.  The splits' (m, l) are read
// one split per lane (64 at a time) and reduced across the wavefront; each split's weight
// 2^(m_c - M) is then broadcast from its lane while the lanes add up their columns of the
// partial outputs in split order, with those loads issued eight splits at a time, so the
// combine costs a few memory round trips instead of one per split.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(const DecodeParams p) {
  constexpr int CPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= p.B * p.H) return;
  const int b = bh / p.H;
  const int ctx = min(p.context_lens[b], p.max_ctx);  // a longer length is a caller error: truncated
  const int ns = (ctx + p.split_len - 1) / p.split_len;
  const int64_t base = (int64_t)bh * p.max_splits;

  float M = kNegInf;
  for (int c0 = 0; c0 < ns; c0 += 64)
    if (c0 + lane < ns) M = fmaxf(M, p.ws_ml[(base + c0 + lane) * 2]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) M = fmaxf(M, __shfl_xor(M, d));
  const float Mu = (M == kNegInf) ? 0.f : M;
  float L = 0.f, o[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) o[e] = 0.f;
  for (int c0 = 0; c0 < ns; c0 += 64) {
    // this chunk's weights and row sums, one split per lane
    float w = 0.f, lw = 0.f;
    if (c0 + lane < ns) {
      const float2 ml = *(const float2*)(p.ws_ml + (base + c0 + lane) * 2);
      w = exp2_fast(ml.x - Mu);
      lw = w * ml.y;
    }
    L += lw;
    const int n = min(64, ns - c0);
    for (int c = 0; c < n; c += 8) {
      float a[8][CPL];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < CPL; ++e)
          a[u][e] = c + u < n ? p.ws_acc[(base + c0 + c + u) * D + lane * CPL + e] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), min(c + u, 63)));
        if (c + u < n) {
#pragma unroll
          for (int e = 0; e < CPL; ++e) o[e] = __builtin_fmaf(wu, a[u][e], o[e]);
        }
      }
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) L += __shfl_xor(L, d);
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
    // grouped-query attention: the matrix-core kernel (measured faster than the VALU
    // kernel from two query heads per KV head on); one head per KV head: the VALU kernel
    const int group = p.H / p.H_kv;
    hipError_t e;
    if (group >= 2) {
      dim3 grid((unsigned)(p.H_kv * ((group + 31) / 32)), (unsigned)p.max_splits, (unsigned)p.B);
      hipLaunchKernelGGL((decode_mfma_kernel<D>), grid, dim3(64), 0, s, p);
      e = hipGetLastError();
    } else {
      e = launch_split<D, 1>(p, s);
    }
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

// ----------------------------------------------------------------------------------
// Fixed scratch of the no-allocation decode entry: the split partials (acc, m, l) of one
// call, for callers that cannot allocate device memory.  Every GPU the library runs on
// holds its own copy of the array until the process ends; every call on a GPU reuses it
// (calls that overlap in time on one GPU race).  In host code `scratch` names only a
// host-side stand-in: its device address is looked up per device and kept.
// ----------------------------------------------------------------------------------
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {  // with device `dev` current
    void* a = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = a;
  });
  *ptr = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

}  // namespace attn
