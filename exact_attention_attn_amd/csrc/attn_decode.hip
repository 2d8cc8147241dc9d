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
//  * q.k is a per-lane 8-term FMA plus a 4-step DPP reduction inside each 16-lane row;
//  * every lane-row runs the online-softmax recurrence (section 2.2 of the same page)
//    on its own tokens; the four rows are merged at the end with the same rescale;
//  * grouped-query attention (section "GQA" of the same page): query head h reads KV
//    head h / (H / H_kv) in place; the query heads sharing a KV head are adjacent
//    wavefronts of one workgroup, so the repeated reads of a KV row hit in cache.
// The second kernel merges the splits of each (sequence, head): with M = max_c m_c,
// O = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c, lse = (M + log2 L) ln 2, in split
// order (deterministic).  This is the online-softmax rescale applied to partial
// states ("L2.5 SOTA Kernel", yulong.wang, section 2.2).
#include "attn_internal.h"

namespace attn {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float bf_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

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

  // q slices of this lane, one per head; scores are scaled after the sum
  float qf[GW][8];
#pragma unroll
  for (int j = 0; j < GW; ++j) {
    const u32x4 u = *(const u32x4*)((const uint16_t*)p.q + ((int64_t)b * p.H + h0 + j) * D + cl * 8);
    qf[j][0] = bf_lo(u.x); qf[j][1] = bf_hi(u.x); qf[j][2] = bf_lo(u.y); qf[j][3] = bf_hi(u.y);
    qf[j][4] = bf_lo(u.z); qf[j][5] = bf_hi(u.z); qf[j][6] = bf_lo(u.w); qf[j][7] = bf_hi(u.w);
  }

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

  auto consume = [&](int u, const C& c) {
    const int t0 = t_begin + 16 * u;
#pragma unroll
    for (int j = 0; j < GW; ++j) {
      float s[NI];
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const u32x4 w = c.k[i];
        float d = qf[j][0] * bf_lo(w.x);
        d = __builtin_fmaf(qf[j][1], bf_hi(w.x), d);
        d = __builtin_fmaf(qf[j][2], bf_lo(w.y), d);
        d = __builtin_fmaf(qf[j][3], bf_hi(w.y), d);
        d = __builtin_fmaf(qf[j][4], bf_lo(w.z), d);
        d = __builtin_fmaf(qf[j][5], bf_hi(w.z), d);
        d = __builtin_fmaf(qf[j][6], bf_lo(w.w), d);
        d = __builtin_fmaf(qf[j][7], bf_hi(w.w), d);
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
      for (int i = 0; i < NI; ++i) {
        const float pv = exp2_fast(s[i] - muse);
        rs += pv;
        const u32x4 w = c.v[i];
        acc[j][0] = __builtin_fmaf(pv, bf_lo(w.x), acc[j][0]);
        acc[j][1] = __builtin_fmaf(pv, bf_hi(w.x), acc[j][1]);
        acc[j][2] = __builtin_fmaf(pv, bf_lo(w.y), acc[j][2]);
        acc[j][3] = __builtin_fmaf(pv, bf_hi(w.y), acc[j][3]);
        acc[j][4] = __builtin_fmaf(pv, bf_lo(w.z), acc[j][4]);
        acc[j][5] = __builtin_fmaf(pv, bf_hi(w.z), acc[j][5]);
        acc[j][6] = __builtin_fmaf(pv, bf_lo(w.w), acc[j][6]);
        acc[j][7] = __builtin_fmaf(pv, bf_hi(w.w), acc[j][7]);
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
    // query heads per wavefront: the largest of 4 (d = 64 only: register budget), 2, 1
    // that divides the group size
    const int group = p.H / p.H_kv;
    hipError_t e;
    if (D == 64 && group % 4 == 0)
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
