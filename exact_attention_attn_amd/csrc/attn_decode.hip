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
//    on its own tokens; the four rows are merged at the end with the same rescale.
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

template <int D>
__global__ __launch_bounds__(256) void decode_split_kernel(const DecodeParams p) {
  using C = Chunk<D>;
  constexpr int LPT = C::LPT, TPI = C::TPI, NI = C::NI;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = blockIdx.x * 4 + wave;  // head groups of one (sequence, split) are adjacent
  const int split = blockIdx.y;          // in dispatch order, so a page is read by all of
                                         // them at about the same time
  const int b = blockIdx.z;
  if (h >= p.H) return;  // no barriers in this kernel: waves are independent
  const int ctx = p.context_lens[b];
  const int t_begin = split * p.split_len;
  if (t_begin >= ctx) return;
  const int t_end = min(ctx, t_begin + p.split_len);
  const int nchunks = (t_end - t_begin + 15) >> 4;

  const int g = lane / LPT;        // token row within an instruction
  const int cl = lane % LPT;       // 16-byte column chunk
  const int64_t tok_stride = (int64_t)p.H * D;           // elements between slots
  const int64_t page_stride = (int64_t)p.page_size * tok_stride;
  const int64_t lane_off = (int64_t)h * D + cl * 8;
  const uint16_t* __restrict__ Kc = (const uint16_t*)p.k_cache;
  const uint16_t* __restrict__ Vc = (const uint16_t*)p.v_cache;
  const int32_t* __restrict__ bt = p.block_table + (int64_t)b * p.max_pages;

  // q slice of this lane, pre-multiplied by nothing: scores are scaled after the sum
  float qf[8];
  {
    const u32x4 u = *(const u32x4*)((const uint16_t*)p.q + ((int64_t)b * p.H + h) * D + cl * 8);
    qf[0] = bf_lo(u.x); qf[1] = bf_hi(u.x); qf[2] = bf_lo(u.y); qf[3] = bf_hi(u.y);
    qf[4] = bf_lo(u.z); qf[5] = bf_hi(u.z); qf[6] = bf_lo(u.w); qf[7] = bf_hi(u.w);
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

  float m2 = kNegInf, l = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  const float c2 = p.scale_log2;

  auto consume = [&](int u, const C& c) {
    const int t0 = t_begin + 16 * u;
    float s[NI];
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const u32x4 w = c.k[i];
      float d = qf[0] * bf_lo(w.x);
      d = __builtin_fmaf(qf[1], bf_hi(w.x), d);
      d = __builtin_fmaf(qf[2], bf_lo(w.y), d);
      d = __builtin_fmaf(qf[3], bf_hi(w.y), d);
      d = __builtin_fmaf(qf[4], bf_lo(w.z), d);
      d = __builtin_fmaf(qf[5], bf_hi(w.z), d);
      d = __builtin_fmaf(qf[6], bf_lo(w.w), d);
      d = __builtin_fmaf(qf[7], bf_hi(w.w), d);
      d = group_sum<LPT>(d);
      const bool ok = t0 + i * TPI + g < t_end;
      s[i] = ok ? d * c2 : kNegInf;
      mx = fmaxf(mx, s[i]);
    }
    const float mnew = fmaxf(m2, mx);
    const float muse = (mnew == kNegInf) ? 0.f : mnew;
    const float alpha = exp2_fast(m2 - muse);
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float pv = exp2_fast(s[i] - muse);
      rs += pv;
      const u32x4 w = c.v[i];
      acc[0] = __builtin_fmaf(pv, bf_lo(w.x), acc[0]);
      acc[1] = __builtin_fmaf(pv, bf_hi(w.x), acc[1]);
      acc[2] = __builtin_fmaf(pv, bf_lo(w.y), acc[2]);
      acc[3] = __builtin_fmaf(pv, bf_hi(w.y), acc[3]);
      acc[4] = __builtin_fmaf(pv, bf_lo(w.z), acc[4]);
      acc[5] = __builtin_fmaf(pv, bf_hi(w.z), acc[5]);
      acc[6] = __builtin_fmaf(pv, bf_lo(w.w), acc[6]);
      acc[7] = __builtin_fmaf(pv, bf_hi(w.w), acc[7]);
    }
    l = l * alpha + rs;
    m2 = mnew;
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

  // merge the lane rows (token rows g) of this wavefront
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
    const float mo = __shfl_xor(m2, off);
    const float lo = __shfl_xor(l, off);
    const float mm = fmaxf(m2, mo);
    const float mu = (mm == kNegInf) ? 0.f : mm;
    const float a0 = exp2_fast(m2 - mu), a1 = exp2_fast(mo - mu);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float ao = __shfl_xor(acc[e], off);
      acc[e] = acc[e] * a0 + ao * a1;
    }
    l = l * a0 + lo * a1;
    m2 = mm;
  }

  const int64_t slot = ((int64_t)b * p.H + h) * p.max_splits + split;
  if (g == 0) {
    float* dst = p.ws_acc + slot * D + cl * 8;
    *(float4*)dst = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *(float4*)(dst + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
  if (lane == 0) *(float2*)(p.ws_ml + slot * 2) = make_float2(m2, l);
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

template <int D>
hipError_t launch_t(const DecodeParams& p, hipStream_t s) {
  if (p.B <= 0 || p.H <= 0) return hipSuccess;
  if (p.max_splits > 0) {
    dim3 grid((unsigned)((p.H + 3) / 4), (unsigned)p.max_splits, (unsigned)p.B);
    hipLaunchKernelGGL((decode_split_kernel<D>), grid, dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
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
