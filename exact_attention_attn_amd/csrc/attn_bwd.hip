// Backward pass of exact attention for gfx950: dQ, dK, dV by recomputation.
//
// Method: the forward keeps only O and the per-row logsumexp; the backward recomputes
// S and P from them, takes dO, and applies the chain rule through the softmax
// (m.lqnn.cn FlashAttention article, section 4.3: recompute P, use dO, subtract the row
// sums in dS; "L2.5 SOTA Kernel", yulong.wang, section 2.3: P from the stored
// logsumexp).  With D_i = dO_i . O_i:
//     P = exp(scale q k^T - lse),  dV = P^T dO,  dP = dO V^T,  dS = P (dP - D),
//     dQ = scale dS K,             dK = scale dS^T Q.
// No float atomics (the same article's advice against atomically accumulating dQ):
//  * bwd_delta_kernel writes (lse log2 e, D) per query row into the workspace;
//  * bwd_dq_kernel owns query rows (4 wavefronts x 32 rows) and streams key tiles of 32,
//    holding dQ in registers: S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T;
//  * bwd_dkdv_kernel owns keys (4 wavefronts x 32 keys) and streams query tiles of 32
//    of every query head that reads its KV head, holding dK and dV in registers:
//    S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS.  Each wavefront
//    software-pipelines the tiles: the S and dP products of tile st+1 run on the matrix
//    cores while the VALU turns tile st's S and dP into P and dS.
// Both recompute S and P (seven tile products per pair of tiles instead of five) so
// that every gradient is written exactly once.
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16): as in the forward kernel, a 32x32 accumulator
// gives each lane one column (a query in the dQ kernel, a key in the dK/dV kernel) and
// 16 rows; the bf16 P or dS feeds the next product as the B operand straight from the
// accumulator, and the A operand of that product (K^T, dO^T, Q^T) is read from LDS with
// transposing reads in the accumulator's row order.  Tiles go global -> LDS with
// direct-to-LDS loads into one swizzled layout per tensor that serves both the 16-byte
// operand reads and the ds_read_b64_tr_b16 transposing reads without bank conflicts.
#include "attn_internal.h"
#include <algorithm>
#include <type_traits>

#include "attn_tile.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634074f;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) uint8_t lds_u8;  // byte address in LDS

// LDS reads at a per-lane byte address plus a compile-time offset.  The per-lane base
// (stage + lane offset) is formed once per tile and passed through an empty asm
// statement, so that the compiler keeps one base register and folds every constant into
// the instruction's offset field instead of re-deriving each address.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const lds_void*)p;
}
__device__ __forceinline__ unsigned opaque(unsigned a) {
  asm volatile("" : "+v"(a));
  return a;
}
__device__ __forceinline__ const lds_u8* lds_at(unsigned a) { return (const lds_u8*)(uintptr_t)a; }

// Swizzled [32 rows, D] bf16 tile serving both read patterns without bank conflicts:
// 16-byte chunk c (columns 8 c .. 8 c + 7) of row r sits at c * 512 + (r ^ 4 (c % 4)) * 16.
// Operand-order A operand of k-step t: lane l reads chunk 2 t + l / 32 of row l % 32,
// at sw_op_lane(l, t % 2) + 1024 t.
__device__ __forceinline__ unsigned sw_op_lane(int lane, int parity) {
  const int half = lane >> 5;
  return (unsigned)(half * 512 + (((lane & 31) ^ (4 * half) ^ (8 * parity)) * 16));
}
// Transposing reads: lane l reads 8 bytes of chunk 4 db + j of row 16 t4 + x (first
// read) and row 16 t4 + x + 8 (second), with x = 4 (l / 32) + (l % 16) / 4 and
// j = 2 ((l / 16) % 2) + (l % 4) / 2, byte 8 (l % 2) of the chunk.
__device__ __forceinline__ unsigned sw_tr_lane(int lane, int second) {
  const int x = 4 * (lane >> 5) + (lane & 15) / 4;
  const int j = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  return (unsigned)(j * 512 + (((x ^ (4 * j)) ^ (8 * second)) * 16) + 8 * (lane & 1));
}
__device__ __forceinline__ bf16x8 sw_tr_read(unsigned lo_base, unsigned hi_base, int db, int t4) {
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)lds_at(lo_base + db * 2048 + t4 * 256));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)lds_at(hi_base + db * 2048 + t4 * 256));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Operand-order A operand of k-step t from a swizzled tile; `base` = tile address +
// sw_op_lane(lane, t % 2)
__device__ __forceinline__ bf16x8 op_read(unsigned base, int t) {
  return as_bf16x8(*(const lds_u32x4*)lds_at(base + t * 1024));
}

// Accumulator element v of lane (half = lane / 32) sits in row 8 (v / 4) + 4 half + v % 4.
__device__ __forceinline__ int acc_row(int v, int half) { return 8 * (v >> 2) + 4 * half + (v & 3); }

// acc += A B on an AGPR-pinned accumulator (the dK / dV accumulators: the dK/dV kernel
// needs more than 256 registers).  The hazard recognizer does not see inside inline
// asm, so the callers spell out the wait states: after VALU writes of an operand before
// the first of these MFMAs, and after the last of them before a VALU read of the
// accumulator (agpr_settle).  MFMAs chained on the same accumulator need none.
__device__ __forceinline__ void mfma_agpr(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void agpr_settle() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// Registers loaded from global memory before the tile loop are passed through an empty
// asm statement, so the compiler waits for those loads here, once.  Otherwise its wait
// for them lands inside the loop as a vmcnt(0), which would also wait for every
// direct-to-LDS prefetch in flight.
template <int N>
__device__ __forceinline__ void settle(bf16x8 (&r)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(r[i]));
}

// Four 1 KiB direct-to-LDS blocks from one M0 write: the instruction offset i * 1024
// moves both the memory address and the LDS destination of block i (the 12-bit field
// reaches block 3), so the per-lane memory offsets passed in have i * 1024 taken out,
// biased by kDmaBias (the descriptor's base sits that many bytes before the tile).  The
// wait states after the M0 write and after SGPR writes by VALU are spelled out, as the
// hazard recognizer does not see inside the asm.
constexpr int kDmaBias = 4096;
__device__ __forceinline__ void dma4(u32x4s r, unsigned m0, int v0, int v1, int v2, int v3) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\t"
               "buffer_load_dwordx4 %2, %1, 0 offen lds\n\t"
               "buffer_load_dwordx4 %3, %1, 0 offen offset:1024 lds\n\t"
               "buffer_load_dwordx4 %4, %1, 0 offen offset:2048 lds\n\t"
               "buffer_load_dwordx4 %5, %1, 0 offen offset:3072 lds"
               :
               : "s"(m0), "s"(r), "v"(v0), "v"(v1), "v"(v2), "v"(v3)
               : "memory", "m0");
}
// Descriptor over [base - kDmaBias, +2 GiB): every row read is a valid one (the last
// tile's rows are clamped), so the range is not used as a guard.
__device__ __forceinline__ u32x4s biased_rsrc(const void* base) {
  const uint64_t a = (uint64_t)base - kDmaBias;
  u32x4s r;
  r.x = (unsigned)a;
  r.y = (unsigned)(a >> 32) & 0xFFFFu;
  r.z = 0x7FFFFFFFu;
  r.w = 0x00020000u;
  return r;
}

// Direct-to-LDS loads of two [32, D] bf16 tiles (tensor 0 then tensor 1, each
// TILE bytes) into the swizzled layout (sw_op_lane): 2 NB 1 KiB blocks, wavefront
// w < NWU carrying blocks 4 w .. 4 w + 3, which all belong to one tensor.  Block i of a
// tile holds chunks 2 i and 2 i + 1 of every row: lane l carries chunk c = 2 i + l / 32
// of row (l % 32) ^ 4 (c % 4).
template <int D>
struct TilePairDma {
  static constexpr int TILE = 32 * D * 2, NB = TILE / 1024, NWU = NB / 2;
  static_assert(NB % 4 == 0, "whole groups of four blocks");
  int tsr;  // tensor of this wavefront's blocks
  int rs;   // row stride of both tensors, elements
  int brow[4], bcol[4], voff[4];
  __device__ void init(int wave, int lane, int row_stride) {
    rs = row_stride;
    tsr = min(1, 4 * wave / NB);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 2 * ((4 * wave + i) % NB) + (lane >> 5);
      brow[i] = (lane & 31) ^ (4 * (c & 3));
      bcol[i] = c * 16;
      voff[i] = brow[i] * (rs * 2) + bcol[i] - i * 1024 + kDmaBias;
    }
  }
  // rows [r0, r0 + 32) of this wavefront's tensor (row stride rs, `nrows` valid rows:
  // later rows are clamped to the last one) into the stage at LDS byte address `stage`
  __device__ void issue(const uint16_t* src, int r0, int nrows, unsigned stage, int wave) const {
    issue_at(src + (int64_t)r0 * rs, nrows - r0 - 1, stage, wave);
  }
  // the same from the tile's first row `tile` with `last` = index of its last valid row
  __device__ void issue_at(const uint16_t* tile, int last, unsigned stage, int wave) const {
    if (wave >= NWU) return;
    const u32x4s r = biased_rsrc(tile);
    const unsigned m0 = stage + (unsigned)(wave * 4096);
    if (last >= 31) {
      dma4(r, m0, voff[0], voff[1], voff[2], voff[3]);
    } else {
      int vo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) vo[i] = min(brow[i], last) * (rs * 2) + bcol[i] - i * 1024 + kDmaBias;
      dma4(r, m0, vo[0], vo[1], vo[2], vo[3]);
    }
  }
};

// s_waitcnt vmcnt(N): at most N of this wavefront's loads still in flight (loads
// complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Variable-length launches in compact form: the batch's blocks of 128 rows (or keys),
// sequence by sequence, are numbered without gaps; block u -> sequence s (-1 past the
// last block), its block index blk and its row ranges [q0, q1) and [k0, k1) in the packed
// tensors.  scan_q: the blocks are row blocks (else key blocks).  Lane i reads sequence
// i's bounds (B <= 64), the wavefront takes an inclusive prefix sum of the block counts,
// and the first lane whose sum exceeds u holds the block: one round of loads and
// register work, instead of a walk over the sequences.
__device__ __forceinline__ void seq_block(const BwdParams& p, bool scan_q, int u, int lane, int& s, int& blk,
                                          int& q0, int& q1, int& k0, int& k1) {
  const int i = min(lane, p.B - 1);
  const int qa = p.cu_q[i], qe = p.cu_q[i + 1], ka = p.cu_k[i], ke = p.cu_k[i + 1];
  const int n = lane < p.B ? ((scan_q ? qe - qa : ke - ka) + 127) >> 7 : 0;
  int incl = n;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(incl, d);
    if (lane >= d) incl += t;
  }
  const unsigned long long m = __builtin_amdgcn_ballot_w64(incl > u);
  s = -1;
  blk = q0 = q1 = k0 = k1 = 0;
  if (m == 0) return;
  s = (int)__builtin_ctzll(m);
  blk = u - __builtin_amdgcn_readlane(incl - n, s);
  q0 = __builtin_amdgcn_readlane(qa, s);
  q1 = __builtin_amdgcn_readlane(qe, s);
  k0 = __builtin_amdgcn_readlane(ka, s);
  k1 = __builtin_amdgcn_readlane(ke, s);
}

// Extents and offsets of (sequence b, query head h, KV head hk).  Dense tensors are
// [B, H, N, d] / [B, H_kv, Nk, d]; variable-length ones are token-major [total, H, d] /
// [total, H_kv, d] with sequence b's rows from cu_q[b] / cu_k[b] (the forward's varlen
// layout).  The lse and the workspace pairs follow the lse layout ([B, H, N] or
// [total_q, H]); r0 / rrs index them.
template <int D, bool VARLEN>
struct BwdGeo {
  int Lq, Lk;
  int64_t q0, k0;  // element offsets of query row 0 of head h, key 0 of KV head hk
  int qrs, krs;    // row strides, elements
  int64_t qhs;     // element stride between consecutive query heads
  int64_t r0;      // lse / workspace index of query row 0 of head h
  int rrs;         // ... its stride between rows
  int64_t rhs;     // ... and between consecutive query heads
  __device__ BwdGeo(const BwdParams& p, int b, int h, int hk)
      : BwdGeo(p, h, hk, VARLEN ? p.cu_q[b] : 0, VARLEN ? p.cu_q[b + 1] : 0, VARLEN ? p.cu_k[b] : 0,
               VARLEN ? p.cu_k[b + 1] : 0, b) {}
  // varlen: the sequence's rows [qs, qe) and keys [ks, ke) given; dense: batch b
  __device__ BwdGeo(const BwdParams& p, int h, int hk, int qs, int qe, int ks, int ke, int b) {
    if (VARLEN) {
      Lq = qe - qs;
      Lk = ke - ks;
      q0 = ((int64_t)qs * p.H + h) * D;
      k0 = ((int64_t)ks * p.H_kv + hk) * D;
      qrs = p.H * D;
      krs = p.H_kv * D;
      qhs = D;
      r0 = (int64_t)qs * p.H + h;
      rrs = p.H;
      rhs = 1;
    } else {
      Lq = p.N;
      Lk = p.Nk;
      q0 = ((int64_t)b * p.H + h) * Lq * D;
      k0 = ((int64_t)b * p.H_kv + hk) * Lk * D;
      qrs = D;
      krs = D;
      qhs = (int64_t)Lq * D;
      r0 = ((int64_t)b * p.H + h) * Lq;
      rrs = 1;
      rhs = Lq;
    }
  }
};

// ------------------------------------------------------------------------------------
// (lse log2 e, D = dO . O) per query row
// ------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const BwdParams p) {
  constexpr int LPR = D / 8;            // lanes per row, 8 elements each
  constexpr int RPB = 256 / LPR;        // rows per workgroup
  const int64_t rows = p.rows;  // B H N, or total_q H (varlen): o, dO rows of D elements
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  float s = 0.f;
  if (row < rows) {
    const u32x4 a = *(const u32x4*)((const uint16_t*)p.dout + row * D + 8 * c);
    const u32x4 b = *(const u32x4*)((const uint16_t*)p.o + row * D + 8 * c);
    const unsigned av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s = __builtin_fmaf(__builtin_bit_cast(float, av[i] << 16), __builtin_bit_cast(float, bv[i] << 16), s);
      s = __builtin_fmaf(__builtin_bit_cast(float, av[i] & 0xFFFF0000u), __builtin_bit_cast(float, bv[i] & 0xFFFF0000u), s);
    }
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) s += __shfl_xor(s, off);
  if (row < rows && c == 0) *(float2*)(p.ws + 2 * row) = make_float2(p.lse[row] * kLog2e, s);
}

// ------------------------------------------------------------------------------------
// dQ: 4 wavefronts x 32 query rows of one (b, h); key tiles of 32
// ------------------------------------------------------------------------------------
template <int D, bool CAUSAL, bool VARLEN>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) bwd_dq_kernel(const BwdParams p) {
  constexpr int NW = 4, BM = 32 * NW, BN = 32;
  constexpr int DT = D / 16, DB = D / 32;
  constexpr int TILE = BN * D * 2;          // bytes of one [32, D] bf16 tile
  // two stages: tile j in use, tile j+1 loading (deeper rings, and tiles loaded in
  // pairs with a barrier every second step, measured no faster)
  constexpr int STAGES = 2;
  // per stage: the K tile and the V tile, swizzled (sw_op_lane)
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * 2 * TILE];

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_rb = (p.N + BM - 1) / BM;  // p.N: the longest sequence's rows (varlen)
  int b, h, rb;
  int sq0 = 0, sq1 = 0, sk0 = 0, sk1 = 0;  // compact grid: the sequence's row and key ranges
  const bool compact = VARLEN && p.units_q > 0;
  if (compact) {
    // compact varlen grid (seq_block): units_q blocks per query head; XCD x takes KV
    // heads x, x + 8, ... (when H_kv is a multiple of 8), each with every query head of
    // its group back to back, each with its blocks in sequence order
    const int G = p.kv_group, nu = p.units_q;
    const int bid = blockIdx.x;
    int u;
    if ((p.H_kv & 7) == 0) {
      const int x = bid & 7, i = bid >> 3;
      const int per = G * nu;
      const int hk = x + 8 * (i / per);
      const int r = i - (i / per) * per;
      const int member = r / nu;
      u = r - member * nu;
      h = hk * G + member;
    } else {
      h = bid % p.H;
      u = bid / p.H;
    }
    int rbi;
    seq_block(p, true, u, lane, b, rbi, sq0, sq1, sk0, sk1);
    if (b < 0) return;  // past the batch's last block; no barrier passed yet
    rb = CAUSAL ? ((sq1 - sq0 + 127) >> 7) - 1 - rbi : rbi;  // heaviest row block of the sequence first
  } else {
    int rbi;
    // Workgroups go round-robin to the 8 XCDs (blockIdx % 8), each with its own L2.  For
    // variable-length batches (many (sequence, KV head) pairs), when the pairs are a
    // multiple of 8, XCD x takes pairs x, x + 8, ... one after the other, and for each
    // the row blocks of every query head of the group back to back, so the pair's K and
    // V tiles stay in that XCD's L2 (measured: varlen dQ -3 %; the dense batch's 32 pairs
    // run 5 % faster in the plain order, head-major within each row-block level).
    const int G = p.kv_group, hkv = p.H_kv, nkv = p.B * hkv;
    const int bid = blockIdx.x;
    if (VARLEN && (nkv & 7) == 0) {
      const int x = bid & 7, i = bid >> 3;
      const int per = G * n_rb;  // blocks per KV pair
      const int kvp = x + 8 * (i / per);
      const int r = i - (i / per) * per;
      const int member = r / n_rb;
      rbi = r - member * n_rb;
      b = kvp / hkv;
      h = (kvp - b * hkv) * G + member;
    } else {
      const int npairs = p.B * p.H;
      const int pair = bid % npairs;
      rbi = bid / npairs;
      b = pair / p.H;
      h = pair - b * p.H;
    }
    rb = CAUSAL ? n_rb - 1 - rbi : rbi;  // heaviest row block first
  }
  const int hk = h / p.kv_group;
  const BwdGeo<D, VARLEN> geo = compact ? BwdGeo<D, VARLEN>(p, h, hk, sq0, sq1, sk0, sk1, b) : BwdGeo<D, VARLEN>(p, b, h, hk);
  const int Lq = geo.Lq, Lk = geo.Lk, shift = Lk - Lq;
  const int row0 = rb * BM;
  if (row0 >= Lq) return;  // uniform over the workgroup; no barrier passed yet
  const int qi = row0 + wave * 32 + (lane & 31);
  const uint16_t* Q = (const uint16_t*)p.q + geo.q0;
  const uint16_t* dO = (const uint16_t*)p.dout + geo.q0;
  const uint16_t* K = (const uint16_t*)p.k + geo.k0;
  const uint16_t* V = (const uint16_t*)p.v + geo.k0;

  int kend = Lk;
  if (CAUSAL) kend = min(Lk, max(0, row0 + BM + shift));
  const int ntiles = (kend + BN - 1) / BN;
  int nfull = Lk / BN;  // tiles that need no mask for any row of this workgroup
  if (CAUSAL) nfull = min(nfull, max(0, (row0 + shift + 1) / BN));

  // Rows past the end load the last row (no divergent branch around the loads) and are
  // zeroed; their results are never stored.
  const bool qin = qi < Lq;
  const int64_t qrow = min(qi, Lq - 1);
  bf16x8 qreg[DT], dreg[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 a = *(const u32x4*)(Q + qrow * geo.qrs + 16 * t + 8 * half);
    const u32x4 c = *(const u32x4*)(dO + qrow * geo.qrs + 16 * t + 8 * half);
    qreg[t] = as_bf16x8(qin ? a : z);
    dreg[t] = as_bf16x8(qin ? c : z);
  }
  const float2 ld = *(const float2*)(p.ws + 2 * (geo.r0 + qrow * geo.rrs));
  float lse2 = qin ? ld.x : 0.f, dsum = qin ? ld.y : 0.f;
  const float c2 = p.scale_log2;

  const unsigned lsm = lds_addr(smem);
  TilePairDma<D> dma;
  dma.init(wave, lane, geo.krs);
  const uint16_t* const src = dma.tsr ? V : K;
  // tile j's rows: a cursor advanced by one tile per load
  const uint16_t* ld_src = src;
  const int64_t src_tile = (int64_t)BN * geo.krs;
  auto issue = [&](int j) {
    dma.issue_at(ld_src, Lk - j * BN - 1, lsm + (unsigned)((j % STAGES) * 2 * TILE), wave);
    ld_src += src_tile;
  };

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x16{};

  if (ntiles > 0) issue(0);
  // the register loads above are waited for here, after the first tile's loads are
  // issued, so that the two memory latencies overlap
  settle(qreg);
  settle(dreg);
  asm volatile("" : "+v"(lse2), "+v"(dsum));
  for (int j = 0; j < ntiles; ++j) {
    wait_vm<0>();     // this wave's share of tile j landed
    __syncthreads();  // ... and every wave's; the stage of tile j-1 is free
    if (j + 1 < ntiles) issue(j + 1);
    const unsigned sbase = lsm + (unsigned)((j % STAGES) * 2 * TILE);
    const unsigned o0 = opaque(sbase + sw_op_lane(lane, 0)), o1 = opaque(sbase + sw_op_lane(lane, 1));
    const unsigned t0 = opaque(sbase + sw_tr_lane(lane, 0)), t1 = opaque(sbase + sw_tr_lane(lane, 1));
    // S^T = K Q^T and dP^T = V dO^T, operands read KPF k-steps ahead of their products
    constexpr int KPF = 3;
    bf16x8 ka[KPF], va[KPF];
#pragma unroll
    for (int u = 0; u < KPF; ++u) {
      ka[u] = op_read((u & 1) ? o1 : o0, u);
      va[u] = op_read(((u & 1) ? o1 : o0) + TILE, u);
    }
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      bf16x8 kn = ka[t % KPF], vn = va[t % KPF];
      if (t + KPF < DT) {
        kn = op_read(((t + KPF) & 1) ? o1 : o0, t + KPF);
        vn = op_read((((t + KPF) & 1) ? o1 : o0) + TILE, t + KPF);
      }
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[t % KPF], qreg[t], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t % KPF], dreg[t], dp, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      ka[t % KPF] = kn;
      va[t % KPF] = vn;
    }
    // the dQ product's operands are requested while S and dP are computed
    bf16x8 kt[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int t4 = 0; t4 < 2; ++t4) kt[db][t4] = sw_tr_read(t0, t1, db, t4);
    __builtin_amdgcn_sched_barrier(0);
    // dS^T = P^T (dP^T - D); keys past the end or above the diagonal have P = 0
    bf16x8 dsb[2];
    if (j < nfull) {  // no row of the workgroup needs a mask in this tile
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float pv = exp2_fast(__builtin_fmaf(s[v], c2, -lse2));
        dsb[v >> 3][v & 7] = (__bf16)(pv * (dp[v] - dsum));
      }
    } else {
      const int base = j * BN + 4 * half;
      int lim = Lk - 1 - base;  // element offsets <= lim are admissible
      if (CAUSAL) lim = min(lim, qi + shift - base);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int off = 8 * (v >> 2) + (v & 3);
        const float pv = exp2_fast(off <= lim ? __builtin_fmaf(s[v], c2, -lse2) : kNegInf);  // exp2(-inf) = 0
        dsb[v >> 3][v & 7] = (__bf16)(pv * (dp[v] - dsum));
      }
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int t4 = 0; t4 < 2; ++t4)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[db][t4], dsb[t4], acc[db], 0, 0, 0);
  }
  __syncthreads();  // every wave is done with the last K / V stage: the LDS stages dQ
  const int wrow0 = row0 + wave * 32;
  store_rows_lds<D>(lsm + (unsigned)(wave * 32 * D * 2), (uint16_t*)p.dq + geo.q0 + (int64_t)wrow0 * geo.qrs,
                    geo.qrs, Lq - wrow0, acc, p.scale, lane);
}

// ------------------------------------------------------------------------------------
// dK, dV: 4 wavefronts x 32 keys of one (b, KV head); query tiles of 32 of every query
// head of the group
// ------------------------------------------------------------------------------------
template <int D, bool CAUSAL, bool VARLEN>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) bwd_dkdv_kernel(const BwdParams p) {
  constexpr int NW = 4, BK = 32 * NW, BQ = 32;
  constexpr int DT = D / 16, DB = D / 32;
  constexpr int TILE = BQ * D * 2;
  // per stage: the Q tile, the dO tile (swizzled layout, see sw_op_lane), then the
  // tile's 32 (lse log2 e, D) pairs
  constexpr int BUF = 2 * TILE + 256;
  // Tiles load in pairs and the workgroup synchronises every second step: the barrier
  // of an even step st publishes tiles st+1 and st+2 (phase 1 of steps st and st+1)
  // and then the pair st+3, st+4 is issued into the stages of tiles st-2 and st-1,
  // which every wave finished before reaching that barrier.  Five stages.
  // (a barrier every third or fourth step, with rings of 7 or 9 stages, measured slower)
  constexpr int STAGES = 5;
  // after the ring: each wavefront's K and V rows, staged on their way into registers
  // (one workgroup per CU, so the LDS this adds costs no occupancy)
  constexpr int KV_STAGE = 2 * TILE;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * BUF + NW * KV_STAGE];

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nkb = (p.Nk + BK - 1) / BK;  // p.Nk: the longest sequence's keys (varlen)
  int b, hk, kb;  // sequence, KV head and key block; low (heaviest causal) key blocks first
  int sq0 = 0, sq1 = 0, sk0 = 0, sk1 = 0;  // compact grid: the sequence's row and key ranges
  const bool compact = VARLEN && p.units_k > 0;
  if (compact) {
    // compact varlen grid (seq_block): units_k key blocks per KV head; XCD x takes KV
    // heads x, x + 8, ... (when H_kv is a multiple of 8), each with its blocks in sequence
    // order, so a sequence's blocks run side by side and share its query-side tiles in L2
    const int nu = p.units_k;
    const int bid = blockIdx.x;
    int u;
    if ((p.H_kv & 7) == 0) {
      const int x = bid & 7, i = bid >> 3;
      hk = x + 8 * (i / nu);
      u = i - (i / nu) * nu;
    } else {
      hk = bid % p.H_kv;
      u = bid / p.H_kv;
    }
    seq_block(p, false, u, lane, b, kb, sq0, sq1, sk0, sk1);
    if (b < 0) return;  // past the batch's last block; no barrier passed yet
  } else {
    int pair;
    // As in the dQ kernel, for variable-length batches: XCD x takes pairs x, x + 8, ...
    // one after the other with all their key blocks, so the pair's query-side tiles stay
    // in that XCD's L2 (measured: varlen dK/dV -7 %; the dense batch unchanged).
    const int npairs = p.B * p.H_kv;
    const int bid = blockIdx.x;
    if (VARLEN && (npairs & 7) == 0) {
      const int x = bid & 7, i = bid >> 3;
      pair = x + 8 * (i / nkb);
      kb = i - (i / nkb) * nkb;
    } else {
      pair = bid % npairs;
      kb = bid / npairs;
    }
    b = pair / p.H_kv;
    hk = pair - b * p.H_kv;
  }
  const int G = p.kv_group;
  // query head: the group's first
  const BwdGeo<D, VARLEN> geo =
      compact ? BwdGeo<D, VARLEN>(p, hk * G, hk, sq0, sq1, sk0, sk1, b) : BwdGeo<D, VARLEN>(p, b, hk * G, hk);
  const int Lq = geo.Lq, Lk = geo.Lk, shift = Lk - Lq;
  const int k0 = kb * BK;
  if (k0 >= Lk) return;  // uniform over the workgroup; no barrier passed yet
  const int key = k0 + wave * 32 + (lane & 31);  // this lane's key (accumulator column)
  const uint16_t* K = (const uint16_t*)p.k + geo.k0;
  const uint16_t* V = (const uint16_t*)p.v + geo.k0;

  // This wavefront's 32 K rows and 32 V rows come through LDS: direct-to-LDS loads of
  // whole rows (1 KiB blocks) into its staging slot, in the swizzled tile layout that
  // op_read reads as the B operands (one key per lane).  Loads straight into the operand
  // layout would make each load instruction touch 32 rows for 32 bytes each; this way
  // the registers are filled about 2.5 us sooner after the workgroup starts.  Keys past
  // the end load the last key (their P and dS are masked to zero, their dK / dV never
  // stored).
  const unsigned kv_slot = lds_addr(smem) + (unsigned)(STAGES * BUF + wave * KV_STAGE);
  {
    const int wk0 = k0 + wave * 32;
    const int last = max(0, min(31, Lk - 1 - wk0));  // last valid row of this wavefront's keys
    const u32x4s kr = biased_rsrc(K + (int64_t)min(wk0, Lk - 1) * geo.krs);
    const u32x4s vr = biased_rsrc(V + (int64_t)min(wk0, Lk - 1) * geo.krs);
    constexpr int NBT = TILE / 1024;  // 1 KiB blocks per tensor
    static_assert(NBT % 4 == 0, "whole groups of four blocks");
#pragma unroll
    for (int g = 0; g < NBT / 4; ++g) {
      int vo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 2 * (4 * g + i) + (lane >> 5);
        const int row = min((lane & 31) ^ (4 * (c & 3)), last);
        vo[i] = row * (geo.krs * 2) + c * 16 - i * 1024 + kDmaBias;
      }
      dma4(kr, kv_slot + (unsigned)(g * 4096), vo[0], vo[1], vo[2], vo[3]);
      dma4(vr, kv_slot + (unsigned)(TILE + g * 4096), vo[0], vo[1], vo[2], vo[3]);
    }
  }
  bf16x8 kreg[DT], vreg[DT];  // filled from the staging slot once the loads landed
  const float c2 = p.scale_log2;

  // query tiles of one head that can see any key of this block
  const int qfirst = CAUSAL ? max(0, k0 - shift) / BQ : 0;
  const int nqt = (Lq + BQ - 1) / BQ;
  const int per_head = max(0, nqt - qfirst);
  const int nsteps = G * per_head;

  const unsigned lsm = lds_addr(smem);
  // DMA: the Q and dO tiles through TilePairDma; one wavefront also brings the tile's 32
  // (lse log2 e, D) pairs
  TilePairDma<D> dma;
  dma.init(wave, lane, geo.qrs);
  const uint16_t* const src0 = (const uint16_t*)(dma.tsr ? p.dout : p.q) + geo.q0;
  const float* const ws0 = p.ws + 2 * geo.r0;
  // Cursors of the next tile to load, advanced by increments (with one wavefront per
  // SIMD, every scalar instruction here delays this wavefront's MFMAs): its first query
  // row, its rows in this wavefront's tensor and in the (lse, D) pairs, its ring stage.
  int ld_q0 = qfirst * BQ;
  const uint16_t* ld_src = src0 + (int64_t)ld_q0 * geo.qrs;
  const float* ld_ws = ws0 + 2 * (int64_t)ld_q0 * geo.rrs;
  unsigned ld_lds = lsm;
  int ld_n = 0;  // tiles issued
  const int64_t src_tile = (int64_t)BQ * geo.qrs, ws_tile = 2 * (int64_t)BQ * geo.rrs;
  // from one past the last tile of a head to the first tile of the next
  const int64_t src_head = geo.qhs - (int64_t)per_head * src_tile;
  const int64_t ws_head = 2 * geo.rhs - (int64_t)per_head * ws_tile;
  const int pv_full = (lane >> 1) * geo.rrs * 8 + (lane & 1) * 4;  // pair rows of a full tile
  auto issue = [&]() {
    const int last = Lq - ld_q0 - 1;  // last valid row of the tile (>= 0)
    dma.issue_at(ld_src, last, ld_lds, wave);
    // 32 (lse2, D) pairs: 64 dwords, lane i -> dword i; rows clamped.  The wavefront that
    // loads them rotates with the tile, so that no wavefront is always the last at the
    // barrier (each waits for its own loads before it).
    if (wave == (ld_n & 3)) {
      const u32x4s pr = buffer_rsrc(ld_ws, 0x7FFFFFFF);
      const int pv = last >= 31 ? pv_full : min(lane >> 1, last) * geo.rrs * 8 + (lane & 1) * 4;
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dword %1, %2, 0 offen lds"
                   :
                   : "s"(ld_lds + (unsigned)(2 * TILE)), "v"(pv), "s"(pr)
                   : "memory", "m0");
    }
    ++ld_n;
    ld_lds = ld_lds + (unsigned)BUF == lsm + (unsigned)(STAGES * BUF) ? lsm : ld_lds + (unsigned)BUF;
    ld_q0 += BQ;
    ld_src += src_tile;
    ld_ws += ws_tile;
    if (ld_q0 >= Lq) {  // next head of the group
      ld_q0 = qfirst * BQ;
      ld_src += src_head;
      ld_ws += ws_head;
    }
  };

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  auto products = [&](f32x16& s, f32x16& dp) {  // S, dP of the first tile (stage 0)
    const unsigned o0 = opaque(lsm + sw_op_lane(lane, 0)), o1 = opaque(lsm + sw_op_lane(lane, 1));
    s = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const unsigned ob = (t & 1) ? o1 : o0;
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op_read(ob, t), kreg[t], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op_read(ob + TILE, t), vreg[t], dp, 0, 0, 0);
    }
  };
  // Admissible query rows of this lane's key: q in [qlo, Lq), none when key >= Lk.  A
  // row q is admissible iff (unsigned)(q - qlo) < span.
  const int qlo = CAUSAL ? key - shift : 0;
  const unsigned span = key < Lk ? (unsigned)max(0, Lq - qlo) : 0u;
  constexpr int KPF = 2;               // k-steps of S / dP operands in flight
  constexpr int EPK = 16 / DT;         // P / dS elements per k-step (2 at d = 128)
  constexpr int PPK = EPK / 2;         // (lse, D) 16-byte reads per k-step
  constexpr int NTR = 4 * DB;          // dV / dK operands (two transposing reads each)
  constexpr int TPK = NTR / DT;        // of them requested per k-step of the second half
  // the 16-byte (lse log2 e, D) pair read pp of a tile: rows 8 (pp / 2) + 4 half + 2 (pp % 2) + {0, 1}
  // (`base` = stage address + 32 half)
  auto pair_read = [&](unsigned base, int pp) -> f32x4 {
    return *(const lds_f32x4*)lds_at(base + 2 * TILE + (16 * (pp >> 1) + 4 * (pp & 1)) * 4);
  };
  const int kw_last = k0 + 32 * wave + 31;  // this wavefront's last key
  int c_s = 0, c_t = qfirst;  // ring stage and query tile of the tile being finished
  auto step = [&](int st, const f32x16& sc, const f32x16& dpc, f32x16& sn, f32x16& dpn, bool sync) {
    if (sync) {       // st even
      wait_vm<0>();   // this wave's share of tiles st+1 and st+2 landed
      __syncthreads();  // ... and every wave's; tiles st-2 and st-1 are finished
      if (st + 3 < nsteps) issue();
      if (st + 4 < nsteps) issue();
    }
    const int c_n = c_s + 1 == STAGES ? 0 : c_s + 1;  // stage of tile st+1
    const unsigned cst = lsm + (unsigned)(c_s * BUF);
    const unsigned nst = lsm + (unsigned)(c_n * BUF);
    const unsigned o0 = opaque(nst + sw_op_lane(lane, 0));  // operand reads of tile st+1,
    const unsigned o1 = opaque(nst + sw_op_lane(lane, 1));  // even and odd k-steps
    const unsigned t0 = opaque(cst + sw_tr_lane(lane, 0));  // transposing reads of tile st,
    const unsigned t1 = opaque(cst + sw_tr_lane(lane, 1));  // rows +0 and +8
    const unsigned lb = opaque(cst + 32u * half);           // (lse, D) pairs of tile st
    const int qt0 = c_t * BQ;
    c_s = c_n;  // the cursors move on to tile st+1
    if (++c_t == nqt) c_t = qfirst;
    const int d0 = qt0 + 4 * half - qlo;  // (q - qlo) of accumulator row 0 of this lane
    bf16x8 qa[KPF], da[KPF];
#pragma unroll
    for (int u = 0; u < KPF; ++u) {
      qa[u] = op_read((u & 1) ? o1 : o0, u);
      da[u] = op_read(((u & 1) ? o1 : o0) + TILE, u);
    }
    f32x4 lp[PPK];
#pragma unroll
    for (int i = 0; i < PPK; ++i) lp[i] = pair_read(lb, i);
    bf16x8 trop[NTR];  // operand 4 db + 2 t4 + 0: dO^T, + 1: Q^T
    bf16x8 pb[2], dsb[2];
    sn = f32x16{};
    dpn = f32x16{};
    // phase 1: S, dP of tile st+1; P, dS of tile st.  Two copies: tiles whose 32 rows
    // see all 32 keys of this wavefront skip the mask (three VALU ops per element, a
    // third of this kernel's VALU work).  Only phase 1 is duplicated: the dK / dV
    // accumulators, written by inline-asm MFMAs, must not be joined by copies after a
    // branch (the hazard recognizer cannot see that those asm statements are MFMAs).
    auto phase1 = [&](auto masked) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      bf16x8 qn = qa[t % KPF], dn = da[t % KPF];
      if (t + KPF < DT) {
        qn = op_read(((t + KPF) & 1) ? o1 : o0, t + KPF);
        dn = op_read((((t + KPF) & 1) ? o1 : o0) + TILE, t + KPF);
      }
      f32x4 ln[PPK];
#pragma unroll
      for (int i = 0; i < PPK; ++i) ln[i] = (t + 1 < DT) ? pair_read(lb, (t + 1) * PPK + i) : lp[i];
      if (t >= DT / 2) {  // the first half of the phase-2 operands
#pragma unroll
        for (int i = 0; i < TPK; ++i) {
          const int idx = (t - DT / 2) * TPK + i;
          const unsigned tt = (idx & 1) ? 0u : (unsigned)TILE;  // Q^T or dO^T
          trop[idx] = sw_tr_read(t0 + tt, t1 + tt, idx >> 2, (idx >> 1) & 1);
        }
      }
      sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[t % KPF], kreg[t], sn, 0, 0, 0);
      dpn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[t % KPF], vreg[t], dpn, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < EPK; ++e) {
        const int v = t * EPK + e;
        const f32x4 pr = lp[e >> 1];
        const float l2 = (v & 1) ? pr.z : pr.x, dd = (v & 1) ? pr.w : pr.y;
        const bool ok = !MASKED || (unsigned)(d0 + acc_row(v, 0)) < span;
        const float x = ok ? __builtin_fmaf(sc[v], c2, -l2) : kNegInf;  // exp2(-inf) = 0
        const float pv = exp2_fast(x);
        pb[v >> 3][v & 7] = (__bf16)pv;
        dsb[v >> 3][v & 7] = (__bf16)(pv * (dpc[v] - dd));
      }
      __builtin_amdgcn_sched_barrier(0);
      qa[t % KPF] = qn;
      da[t % KPF] = dn;
#pragma unroll
      for (int i = 0; i < PPK; ++i) lp[i] = ln[i];
    }
    };
    if (qt0 + BQ <= Lq && kw_last < Lk && (!CAUSAL || qt0 >= kw_last - shift)) phase1(std::false_type{});
    else phase1(std::true_type{});
    // the second half of the phase-2 operands
#pragma unroll
    for (int idx = NTR / 2; idx < NTR; ++idx)
      trop[idx] = sw_tr_read(t0 + ((idx & 1) ? 0u : (unsigned)TILE), t1 + ((idx & 1) ? 0u : (unsigned)TILE),
                             idx >> 2, (idx >> 1) & 1);
    // The asm MFMAs below read P and dS, just written by VALU: the hazard recognizer does
    // not see them, so five wait states are spelled out here, after the last write (the
    // operands are tied to this statement so that no write can move past it).
    asm volatile("s_nop 4" : "+v"(pb[0]), "+v"(pb[1]), "+v"(dsb[0]), "+v"(dsb[1]));
    // phase 2: dV^T += dO^T P,  dK^T += Q^T dS
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int t4 = 0; t4 < 2; ++t4) {
        mfma_agpr(dv[db], trop[4 * db + 2 * t4], pb[t4]);
        mfma_agpr(dk[db], trop[4 * db + 2 * t4 + 1], dsb[t4]);
      }
  };

  // tiles 0, 1 and 2 before the loop (the first step's barrier publishes 1 and 2 again)
#pragma unroll
  for (int st = 0; st < 3; ++st)
    if (st < nsteps) issue();
  wait_vm<0>();  // this wave's K / V rows (and its share of the first tiles) landed
  {
    const unsigned o0 = opaque(kv_slot + sw_op_lane(lane, 0)), o1 = opaque(kv_slot + sw_op_lane(lane, 1));
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      kreg[t] = op_read((t & 1) ? o1 : o0, t);
      vreg[t] = op_read(((t & 1) ? o1 : o0) + TILE, t);
    }
  }
  f32x16 sA, dA, sB, dB;
  if (nsteps > 0) {
    __syncthreads();
    products(sA, dA);
  }
  // unrolled by two so that the two S / dP sets swap roles without copies; the even
  // step of each pair synchronises
  int st = 0;
  for (; st + 1 < nsteps; st += 2) {
    step(st, sA, dA, sB, dB, true);
    step(st + 1, sB, dB, sA, dA, false);
  }
  if (st < nsteps) step(st, sA, dA, sB, dB, true);
  agpr_settle();
  __syncthreads();  // every wave is done with the ring: the LDS stages dK and dV
  {
    const int wk0 = k0 + wave * 32;
    const int64_t row = geo.k0 + (int64_t)wk0 * geo.krs;
    const unsigned slice = lsm + (unsigned)(wave * 2 * 32 * D * 2);
    store_rows_lds<D>(slice, (uint16_t*)p.dk + row, geo.krs, Lk - wk0, dk, p.scale, lane);
    store_rows_lds<D>(slice + 32 * D * 2, (uint16_t*)p.dv + row, geo.krs, Lk - wk0, dv, 1.0f, lane);
  }
}

// Variable-length batches of at most kCompactSeqs sequences launch compact grids
// (seq_block): an upper bound of the batch's 128-row (key) blocks per head, from the
// packed row counts (sum over s of ceil(L_s / 128) <= (total + 127 B) / 128), instead of
// ceil(max_seqlen / 128) blocks for every sequence.  At one dK/dV workgroup per CU,
// each of the empty workgroups of the plain grid held a CU for its launch, its
// parameter and cu_seqlens reads and its exit (a per-workgroup timeline showed 5-6 us
// between a CU's consecutive real workgroups against 1 us in the dense case).
constexpr int kCompactSeqs = 64;  // seq_block: one sequence per lane

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t s) {
  // p.N, p.Nk: rows and keys per sequence (dense) or of the longest sequence (varlen)
  BwdParams q = p;
  q.units_q = q.units_k = 0;
  if (VARLEN && p.B <= kCompactSeqs) {
    q.units_q = (int)std::min<int64_t>((int64_t)p.B * ((p.N + 127) / 128), ((int64_t)p.total_q + 127 * (int64_t)p.B) / 128);
    q.units_k = (int)std::min<int64_t>((int64_t)p.B * ((p.Nk + 127) / 128), ((int64_t)p.total_k + 127 * (int64_t)p.B) / 128);
  }
  if (p.rows > 0) {
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)((p.rows + RPB - 1) / RPB)), dim3(256), 0, s, q);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nq = (VARLEN && q.units_q > 0 ? (int64_t)q.units_q : (int64_t)((p.N + 127) / 128) * p.B) * p.H;
    if (nq > 0) {
      hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, VARLEN>), dim3((unsigned)nq), dim3(256), 0, s, q);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  const int64_t nk = (VARLEN && q.units_k > 0 ? (int64_t)q.units_k : (int64_t)((p.Nk + 127) / 128) * p.B) * p.H_kv;
  if (nk > 0) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, VARLEN>), dim3((unsigned)nk), dim3(256), 0, s, q);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, bool causal, bool varlen, hipStream_t s) {
  if (varlen) return causal ? launch_bwd_t<D, true, true>(p, s) : launch_bwd_t<D, false, true>(p, s);
  return causal ? launch_bwd_t<D, true, false>(p, s) : launch_bwd_t<D, false, false>(p, s);
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int d, bool causal, bool varlen, hipStream_t s) {
  return d == 128 ? launch_bwd_d<128>(p, causal, varlen, s) : launch_bwd_d<64>(p, causal, varlen, s);
}

}  // namespace attn
