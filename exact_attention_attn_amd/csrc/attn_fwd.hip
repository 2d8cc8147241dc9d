// Tiled exact-attention forward for gfx950 (MI355X): dense and variable-length.
//
// Method: "From standard Attention to FlashAttention and paged execution"
// (dlog.com.cn), sections 2.1-2.3: Q is cut into row blocks that are independent
// work units; each block streams every K/V column block through on-chip memory;
// an online softmax (running max m, running sum l) rescales the accumulator so that
// only O and the per-row logsumexp are written.  Each wavefront owns its own query
// rows for the whole key loop, so no softmax state is ever exchanged between
// wavefronts (section 2.3, the FA2 split).
//
// gfx950 mapping (bf16 kernel):
//  * workgroup = NW wavefronts x 32 query rows; key tiles of 64 at 2 wavefronts per
//    SIMD, or of 32 at 3 wavefronts per SIMD for causal varlen / paged batches of short
//    sequences (kFwdShortLen).
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: A = K rows read from LDS, B = Q held in
//    VGPRs for the whole loop.  In the 32x32 accumulator each lane then owns ONE
//    query (column) and 16 keys, so the row max / row sum are 15 in-lane ops plus a
//    single exchange with lane^32.
//  * O^T += V^T P^T on the same MFMA: P^T is taken straight from the S^T
//    accumulator (converted to bf16) as the B operand; the order in which keys enter
//    the contraction follows the accumulator's layout, and V^T is read from LDS in
//    that same order.  The O^T accumulator again gives each lane one query row, so
//    the per-row rescale by exp(m_old - m_new) is a per-lane scalar multiply.
//  * K and V tiles go global -> LDS with direct-to-LDS loads (no VGPR staging),
//    double-buffered; rows past the sequence end are clamped to its last row and
//    masked.  K tile: 1 KiB blocks of 16 keys x 64 B (one page group each, 64
//    contiguous bytes per lane quad), the chunk order XOR-swizzled by key so that the
//    MFMA operand reads hit distinct banks.  V tile: [32-column block][key][64 B]; the
//    V^T operand comes from two LDS transposing reads (ds_read_b64_tr_b16), each
//    covering 256 contiguous bytes.
//  * Scores are kept in base-2 units: p = exp2(s * scale*log2(e) - m2), using the
//    hardware exp2.
//
// The fp32 kernel (used for float32 inputs) is a plain VALU version of the same
// recurrence: 4 lanes per query row, K/V tiles broadcast from LDS.
#include "attn_internal.h"
#include "attn_tile.h"

#include <type_traits>

namespace attn {
namespace {

// 16 bytes per lane from a uniform base plus a 32-bit lane offset into LDS at `lds` +
// 16 lane (global_load_lds with a scalar base: the paged gather, whose pools may exceed
// a buffer resource's reach).  The wait states after the M0 write and after VALU writes
// of the SGPR base are spelled out, as the hazard recognizer does not see inside the asm.
__device__ __forceinline__ void dma16s(const void* sbase, int voff, const uint8_t* lds) {
  const unsigned m0v = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(const lds_void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(m0v), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// Block index -> (row block, batch/sequence, head).  Workgroups are dispatched
// round-robin over the 8 XCDs (bid % 8), each with its own L2.  When the number of
// (batch, KV head) pairs is a multiple of 8, XCD x takes KV pairs x, x+8, x+16, ... one
// after the other; for each, the query heads reading that KV head (one under multi-head
// attention, H / H_kv under grouped-query attention) run back to back, each with all
// its row blocks, so the K/V in flight stay in that XCD's L2 and every XCD gets an even
// share of heads and sequences.  Causal launches take the heaviest (last) row block of
// a head first.
template <bool CAUSAL>
__device__ __forceinline__ void block_coords(const FwdParams& p, int& rb, int& b, int& h) {
  const int G = p.kv_group;
  const int hkv = p.H / G;
  const int nkv = hkv * p.B;
  const int bid = blockIdx.x;
  int rbi;
  if ((nkv & 7) == 0) {
    const int x = bid & 7, i = bid >> 3;
    const int per = G * p.n_rb;        // blocks per KV pair
    const int kvp = x + 8 * (i / per);
    const int r = i - (i / per) * per;
    const int member = r / p.n_rb;
    rbi = r - member * p.n_rb;
    b = kvp / hkv;
    h = (kvp - b * hkv) * G + member;
  } else {
    const int npairs = p.H * p.B;
    const int pair = bid % npairs;
    rbi = bid / npairs;
    b = pair / p.H;
    h = pair - b * p.H;
  }
  rb = CAUSAL ? (p.n_rb - 1 - rbi) : rbi;
}

// Dense causal launches: the row blocks of a head come in pairs (n_rb - 1 - j, j), one
// pair per workgroup, so every workgroup does the same work (n_rb + 1 key tiles of 128
// rows for a 128-row block), whatever the row block.  The hardware places workgroups on
// the CUs in dispatch order without regard to their length, so with one row block per
// workgroup the CUs that drew the long blocks of the diagonal ran on after the others;
// equal pairs leave no such tail.  Block order as in block_coords (KV pairs round-robin
// over the XCDs, the query heads of a KV head back to back).  rb1 == rb0 for the middle
// block of an odd count.
__device__ __forceinline__ void block_coords_pair(const FwdParams& p, int& rb0, int& rb1, int& b, int& h) {
  const int G = p.kv_group;
  const int hkv = p.H / G;
  const int nkv = hkv * p.B;
  const int npr = (p.n_rb + 1) >> 1;  // pairs per head
  const int bid = blockIdx.x;
  int j;
  if ((nkv & 7) == 0) {
    const int x = bid & 7, i = bid >> 3;
    const int per = G * npr;
    const int kvp = x + 8 * (i / per);
    const int r = i - (i / per) * per;
    const int member = r / npr;
    j = r - member * npr;
    b = kvp / hkv;
    h = (kvp - b * hkv) * G + member;
  } else {
    const int npairs = p.H * p.B;
    const int pair = bid % npairs;
    j = bid / npairs;
    b = pair / p.H;
    h = pair - b * p.H;
  }
  rb0 = p.n_rb - 1 - j;
  rb1 = j;
}

// Per-(sequence, head) extents and element offsets.  Paged K/V: koff / voff only select
// the KV head inside a slot; the page comes from the block table per key.
template <bool VARLEN, bool PAGED = false>
__device__ __forceinline__ void seq_bounds(const FwdParams& p, int b, int h, int& Lq, int& Lk,
                                           int64_t& qoff, int64_t& koff, int64_t& voff,
                                           int64_t& ooff, int64_t& loff) {
  const int hk = h / p.kv_group;  // KV head of query head h (grouped-query attention)
  if (VARLEN) {
    const int q0 = p.cu_q[b], q1 = p.cu_q[b + 1];
    const int k0 = p.cu_k[b], k1 = p.cu_k[b + 1];
    Lq = q1 - q0;
    Lk = k1 - k0;
    qoff = (int64_t)q0 * p.q_sn + (int64_t)h * p.q_sh;
    koff = (PAGED ? 0 : (int64_t)k0 * p.k_sn) + (int64_t)hk * p.k_sh;
    voff = (PAGED ? 0 : (int64_t)k0 * p.v_sn) + (int64_t)hk * p.v_sh;
    ooff = (int64_t)q0 * p.o_sn + (int64_t)h * p.o_sh;
    loff = (int64_t)q0 * p.l_sn + (int64_t)h * p.l_sh;
  } else {
    Lq = p.Nq;
    Lk = p.Nk;
    qoff = (int64_t)b * p.q_sb + (int64_t)h * p.q_sh;
    koff = (int64_t)b * p.k_sb + (int64_t)hk * p.k_sh;
    voff = (int64_t)b * p.v_sb + (int64_t)hk * p.v_sh;
    ooff = (int64_t)b * p.o_sb + (int64_t)h * p.o_sh;
    loff = (int64_t)b * p.l_sb + (int64_t)h * p.l_sh;
  }
}

// ----------------------------------------------------------------------------------
// bf16 MFMA kernel
// ----------------------------------------------------------------------------------
// Deferred rescale: the reference max m2 (base-2 units) only moves when a row's new
// maximum exceeds it by more than kRescaleSlack.  Probabilities are then bounded by
// 2^kRescaleSlack instead of 1, which fp32 accumulators and bf16 operands carry
// without loss; O = acc / l and lse = m2 + log2 l hold for any reference value, so
// the result is the same function.  Most tiles then skip the O^T rescale.
constexpr float kRescaleSlack = 8.0f;

template <int D, int NW, int BN, int WPE, bool CAUSAL, bool VARLEN, bool PAGED>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) fwd_bf16_kernel(const FwdParams p) {
  constexpr int BM = 32 * NW;       // query rows per workgroup
  constexpr int NS = BN / 32;       // 32-key blocks per key tile
  constexpr int NP = BN / 16;       // 16-key groups per key tile (B operands of O^T += V^T P^T)
  constexpr int DT = D / 16;        // k-steps of the S^T contraction
  constexpr int DB = D / 32;        // 32-column blocks of O^T
  constexpr int TILE_BYTES = BN * D * 2;
  constexpr int VBLK = BN * 64;             // bytes of one 32-column block of a V tile
  constexpr int NBLK = TILE_BYTES / 1024;   // 1 KiB direct-to-LDS blocks per K (or V) tile
  constexpr int BPW = NBLK / NW;            // blocks per wavefront
  static_assert(BPW * NW == NBLK, "tile split");
  // LDS: K and V tiles, each double-buffered.  K runs one tile ahead of V: while
  // tile j's V feeds P_j V_j, tile j+1's K feeds S_{j+1} = K_{j+1} Q^T.
  //   K tile: [BN / 16 key groups][NQ = D / 32 chunk quads] blocks of 1 KiB, each 16
  //           keys x 64 B with the chunk within the quad XOR-swizzled by key bits 2-3:
  //           chunk c of key k at ((k / 16) NQ + c / 4) 1024 + (k % 16) 64 +
  //           ((c % 4) ^ ((k / 4) % 4)) 16.  A load block is one 16-key group (one page
  //           of a paged pool) and each lane quad reads 64 contiguous bytes; the A operand
  //           reads (one key per lane) hit distinct banks from two lane bases.
  //   V tile: [DB blocks][BN keys][4 chunks]  (32 columns of one key = 64 B)
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TILE_BYTES];  // K0 K1 V0 V1
  uint8_t* const kbuf0 = smem;
  uint8_t* const kbuf1 = smem + TILE_BYTES;
  uint8_t* const vbuf0 = smem + 2 * TILE_BYTES;
  uint8_t* const vbuf1 = smem + 3 * TILE_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: LDS DMA bases stay in SGPRs
  const int col = lane & 31;
  const int half = lane >> 5;

  // dense causal: two row blocks of equal total work per workgroup (block_coords_pair)
  constexpr bool PAIRED = CAUSAL && !VARLEN;
  int rbs[2], b, h;
  if constexpr (PAIRED) {
    block_coords_pair(p, rbs[0], rbs[1], b, h);
  } else {
    block_coords<CAUSAL>(p, rbs[0], b, h);
    rbs[1] = rbs[0];
  }
  int Lq, Lk;
  int64_t qoff, koff, voff, ooff, loff;
  seq_bounds<VARLEN, PAGED>(p, b, h, Lq, Lk, qoff, koff, voff, ooff, loff);

  // One row block: its Q rows against every admissible K/V tile, then O and lse.
  auto row_block = [&](const int rb) {
    const int row0 = rb * BM;
    if (row0 >= Lq) return;  // uniform over the workgroup

    const int shift = Lk - Lq;  // bottom-right causal alignment
    int kend = Lk;
    if (CAUSAL) kend = min(Lk, max(0, row0 + BM + shift));
    const int ntiles = (kend + BN - 1) / BN;
    // tiles [0, nfull) need no mask for any row of this workgroup
    int nfull = Lk / BN;
    if (CAUSAL) nfull = min(nfull, max(0, (row0 + shift + 1) / BN));

    const uint16_t* __restrict__ Qg = (const uint16_t*)p.q + qoff;
    const uint16_t* __restrict__ Kg = (const uint16_t*)p.k + koff;
    const uint16_t* __restrict__ Vg = (const uint16_t*)p.v + voff;
    const int64_t ksn = p.k_sn, vsn = p.v_sn;

    const int wrow0 = row0 + wave * 32;
    const int qi = wrow0 + col;

    bf16x8 qreg[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      u32x4 u = {0u, 0u, 0u, 0u};
      if (qi < Lq) u = *(const u32x4*)(Qg + (int64_t)qi * p.q_sn + 16 * t + 8 * half);
      qreg[t] = as_bf16x8(u);
    }

    // Per-lane source rows and in-row byte offsets of this wavefront's direct-to-LDS loads.
    // In the last tile, rows past the sequence end are clamped to its last row: the
    // direct-to-LDS path does not reliably write zeros for out-of-range rows, and stale LDS
    // data times a zero probability could be NaN.  Clamped keys are masked to -inf.
    int kkey[BPW], kcol[BPW], vkey[BPW], vcol[BPW], kdoff[BPW], vdoff[BPW];
    const int krow_bytes = (int)ksn * 2, vrow_bytes = (int)vsn * 2;
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int bi = wave * BPW + i;
      {  // K block bi = (key group g, chunk quad q): key 16 g + lane / 4, chunk
         // 4 q + ((lane % 4) ^ ((lane / 16) % 4))
        constexpr int NQ = D / 32;
        const int g = bi / NQ, q = bi % NQ;
        kkey[i] = 16 * g + (lane >> 2);
        kcol[i] = (4 * q + ((lane & 3) ^ ((lane >> 4) & 3))) * 16;
      }
      {  // V block bi: column block bi / (BN / 16), keys 16 * (bi % (BN / 16)) + lane / 4, chunk lane % 4
        const int db = bi / (BN / 16);
        vkey[i] = 16 * (bi % (BN / 16)) + lane / 4;
        vcol[i] = (32 * db + 8 * (lane % 4)) * 2;
      }
      kdoff[i] = kkey[i] * krow_bytes + kcol[i];
      vdoff[i] = vkey[i] * vrow_bytes + vcol[i];
    }

    // Paged K/V: every 1 KiB load block covers one 16-key group of its tile, and a group
    // lies in one page (page sizes are powers of two >= 16), so a block's source is a
    // uniform base (its group's page, read from the block table one step before the load)
    // plus a loop-invariant lane offset.  In the last tile, keys past the end are clamped
    // to the last key, whose group then serves the whole block.
    const int32_t* __restrict__ bt_row = PAGED ? p.block_table + (int64_t)b * p.bt_stride : nullptr;
    const int pshift = PAGED ? p.page_shift : 0;
    const int pmask = (1 << pshift) - 1;
    int kgrp[BPW], vgrp[BPW], kloff[BPW], vloff[BPW];
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int bi = wave * BPW + i;
      kgrp[i] = bi / (D / 32);
      vgrp[i] = bi % (BN / 16);
      kloff[i] = (kkey[i] & 15) * krow_bytes + kcol[i];
      vloff[i] = (vkey[i] & 15) * vrow_bytes + vcol[i];
    }
    // Page of block i's group.  A wavefront's K blocks are the NQ chunk quads of one key
    // group, so K needs one page per tile (entry 0); V blocks span the tile's groups.
    static_assert(BPW <= D / 32 && (D / 32) % BPW == 0, "a wavefront's K blocks share one key group");
    int kpg[1], vpg[PAGED ? BPW : 1];
    // The page ids are uniform per wavefront: read through the constant address space,
    // they become scalar loads into SGPRs (no VGPRs: the 32-key, 3-wavefront configuration
    // spilled with them in VGPRs) whose wait counter is not the one of the tile loads.
    // They are issued a step ahead and pass through an empty asm right after the step's
    // barrier, so that the compiler's wait for them lands there.
    auto load_pages = [&](int j, const int* grp, int* pg, int n) {
      const int kt0 = j * BN;
      const int glast = (Lk - 1 - kt0) >> 4;  // last group holding a valid key
#pragma unroll
      for (int i = 0; i < BPW; ++i)
        if (i < n)
          pg[i] = *(const __attribute__((address_space(4))) int32_t*)(bt_row + ((kt0 + 16 * min(grp[i], glast)) >> pshift));
    };
    auto settle_pages = [&]() {
      asm volatile("" : "+s"(kpg[0]));
#pragma unroll
      for (int i = 0; i < BPW; ++i) asm volatile("" : "+s"(vpg[i]));
    };
    auto issue_paged = [&](int j, uint8_t* buf, const uint16_t* base, const int* grp, const int* loff,
                           const int* key, const int* colb, const int* pg, bool one_page, int row_bytes) {
      const int kt0 = j * BN;
      const int last = Lk - kt0 - 1;
      const int glast = last >> 4;
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        const int geff = min(grp[i], glast);
        const int page = pg[one_page ? 0 : i];  // scalar, loaded a step earlier
        const uint8_t* gbase =
            (const uint8_t*)base + (((int64_t)page << pshift) + ((kt0 + 16 * geff) & pmask)) * row_bytes;
        const int vo = last >= BN - 1 ? loff[i] : (min(key[i], last) - 16 * geff) * row_bytes + colb[i];
        dma16s(gbase, vo, buf + (wave * BPW + i) * 1024);
      }
    };

    auto issue_k = [&](int j, uint8_t* kb) {
      if (PAGED) {
        issue_paged(j, kb, Kg, kgrp, kloff, kkey, kcol, kpg, true, krow_bytes);
        return;
      }
      const int kt0 = j * BN;
      const int last = Lk - kt0 - 1;  // last valid row of this tile (>= 0)
      const int64_t krem = ((int64_t)last * ksn + D) * 2;  // bytes of valid keys from kt0 on
      const u32x4s kr = buffer_rsrc(Kg + (int64_t)kt0 * ksn, krem);
      if (last >= BN - 1) {
#pragma unroll
        for (int i = 0; i < BPW; ++i) dma16(kr, kb + (wave * BPW + i) * 1024, kdoff[i]);
      } else {
#pragma unroll
        for (int i = 0; i < BPW; ++i)
          dma16(kr, kb + (wave * BPW + i) * 1024, min(kkey[i], last) * krow_bytes + kcol[i]);
      }
    };
    auto issue_v = [&](int j, uint8_t* vb) {
      if (PAGED) {
        issue_paged(j, vb, Vg, vgrp, vloff, vkey, vcol, vpg, false, vrow_bytes);
        return;
      }
      const int kt0 = j * BN;
      const int last = Lk - kt0 - 1;
      const int64_t vrem = ((int64_t)last * vsn + D) * 2;
      const u32x4s vr = buffer_rsrc(Vg + (int64_t)kt0 * vsn, vrem);
      if (last >= BN - 1) {
#pragma unroll
        for (int i = 0; i < BPW; ++i) dma16(vr, vb + (wave * BPW + i) * 1024, vdoff[i]);
      } else {
#pragma unroll
        for (int i = 0; i < BPW; ++i)
          dma16(vr, vb + (wave * BPW + i) * 1024, min(vkey[i], last) * vrow_bytes + vcol[i]);
      }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
    float m2 = kNegInf;  // reference max, base-2 units
    float l = 0.f;
    const float c2 = p.scale_log2;

    // LDS read offsets
    // K operand of k-step t, key block c: lane l reads chunk 2 t + l / 32 of key 32 c + l % 32,
    // at kread[t % 2] + (2 c NQ + t / 2) 1024
    constexpr int NQ = D / 32;
    int kread[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int m = (lane >> 2) & 3;
      kread[par] = ((lane >> 4) & 1) * NQ * 1024 + (lane & 15) * 64 + (2 * (par ^ (m >> 1)) + (half ^ (m & 1))) * 16;
    }
    const int vread = (4 * half + (lane & 15) / 4) * 64 + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);

    // K operand of S^T = K Q^T for k-step t and key block c (16 bytes per lane)
    auto kop = [&](const uint8_t* kb, int t, int c) -> u32x4 {
      return *(const lds_u32x4*)(kb + kread[t & 1] + (2 * c * NQ + (t >> 1)) * 1024);
    };
    // V^T operand of O^T += V^T P^T for column block db and key group t4 (two transposing reads)
    auto vop = [&](const uint8_t* vb, int db, int t4) -> bf16x8 {
      const uint8_t* vp = vb + vread + db * VBLK + t4 * 1024;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vp + 512));
      return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    // Tail keys and (causal) keys above the diagonal -> -inf.  A key is admissible for
    // this lane's query iff key <= klim; element (c, v) of the tile
    // at kt0 holds key kt0 + 4 half + 32 c + 8 (v / 4) + v % 4, so the test is one compare
    // of that compile-time offset with klim - kt0 - 4 half.
    const int klim = CAUSAL ? min(Lk - 1, qi + shift) : Lk - 1;
    auto mask1 = [&](int rel, float x, int c, int v) -> float {
      return 32 * c + 8 * (v >> 2) + (v & 3) <= rel ? x : kNegInf;
    };
    auto finish_max = [&](float mx, float& mnew, bool& grow) {
      mx = fmaxf(mx, xor32(mx)) * c2;
      grow = mx > m2 + kRescaleSlack;  // also true on a row's first admissible key
      mnew = grow ? mx : m2;
    };

    if (ntiles > 0) {
      // prologue: K0, V0, K1 in flight; S_0 and its row max
      if (PAGED) {
        load_pages(0, kgrp, kpg, 1);
        load_pages(0, vgrp, vpg, BPW);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        settle_pages();
      }
      issue_k(0, kbuf0);
      issue_v(0, vbuf0);
      if (ntiles > 1) {
        if (PAGED) {
          load_pages(1, kgrp, kpg, 1);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          settle_pages();
        }
        issue_k(1, kbuf1);
      }
      if (PAGED) {  // pages of the first step's loads: K_2 and V_1
        if (ntiles > 2) load_pages(2, kgrp, kpg, 1);
        if (ntiles > 1) load_pages(1, vgrp, vpg, BPW);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      f32x16 sA[NS], sB[NS];  // S of the current and the next tile, alternating roles
#pragma unroll
      for (int c = 0; c < NS; ++c) sA[c] = f32x16{};
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int c = 0; c < NS; ++c)
          sA[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kop(kbuf0, t, c)), qreg[t], sA[c], 0, 0, 0);
      float mnew;
      bool grow;
      {
        float mx = kNegInf;
#pragma unroll
        for (int c = 0; c < NS; ++c)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            if (nfull < 1) sA[c][v] = mask1(klim - 4 * half, sA[c][v], c, v);
            mx = fmaxf(mx, sA[c][v]);
          }
        finish_max(mx, mnew, grow);
      }

      // Step j, software-pipelined inside one wavefront (MFMA and VALU work of the same
      // wavefront overlap; separate wavefronts on a SIMD barely do):
      //   phase 1: S_{j+1} = K_{j+1} Q^T (NS MFMAs per k-step) interleaved with the
      //            exponentials, row sums and bf16 packing of tile j;
      //   phase 2: O^T += V_j^T P_j^T (1 MFMA per chunk) interleaved with masking and the
      //            row max of tile j+1.
      // Scheduling barriers keep each chunk's MFMAs next to its VALU share.  Tiles that
      // cross the diagonal or the sequence end are masked after phase 2 (a few per row
      // block).  The last step's S_{j+1} is computed on a stale buffer and discarded.
      // Step j: see the comment above.  Buffers: K_j in kbuf[j % 2], V_j in vbuf[j % 2].
      auto step = [&](int j, const uint8_t* kcur, uint8_t* kdma, const uint8_t* vcur, uint8_t* vdma,
                      f32x16* s_cur, f32x16* sn) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's K_{j+1}, V_j landed
        __syncthreads();                                   // ... and every wave's
        if (PAGED) settle_pages();  // the page ids loaded with them too
        // the first two k-steps' K operands are requested before anything else
        constexpr int KPF = 2;  // k-steps of K operands in flight
        u32x4 a[KPF][NS];
#pragma unroll
        for (int u = 0; u < KPF; ++u)
#pragma unroll
          for (int c = 0; c < NS; ++c) a[u][c] = kop(kcur, u, c);
        if (j + 2 < ntiles) issue_k(j + 2, kdma);
        if (j + 1 < ntiles) issue_v(j + 1, vdma);
        if (PAGED) {  // pages of the next step's loads, landing with this step's tiles
          if (j + 3 < ntiles) load_pages(j + 3, kgrp, kpg, 1);
          if (j + 2 < ntiles) load_pages(j + 2, vgrp, vpg, BPW);
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {      // deferred rescale (rare)
          const float alpha = exp2_fast(m2 - (mnew == kNegInf ? 0.f : mnew));
          l *= alpha;
#pragma unroll
          for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
          m2 = mnew;
        }
        const float muse = (m2 == kNegInf) ? 0.f : m2;  // no admissible key yet: p = 0

        // phase 1
#pragma unroll
        for (int c = 0; c < NS; ++c) sn[c] = f32x16{};
        bf16x8 pb[NP];
        // Row sum of P_j: with 64-key tiles at 2 wavefronts per SIMD the fp32 P values stay
        // in registers and are summed in phase 2, whose VALU share is light (phase 1 carries
        // the exponentials; measured +1 %); the 3-wavefront configuration has no registers
        // to spare and sums in phase 1.
        constexpr bool DEFER_SUM = WPE == 2;
        // In that configuration the last MV elements of P_j are also computed in phase 2:
        // its MFMAs then run key-group-major, so the last group's P operand is first needed
        // at chunk (NP - 1) DB, after those elements (measured +0.7 %).
        constexpr int MV = DEFER_SUM ? ((NP - 1) * DB < 4 ? (NP - 1) * DB : 4) : 0;
        constexpr int P1 = 16 * NS - MV;  // elements of P_j computed in phase 1
        float rs = 0.f;
        float pvs[DEFER_SUM ? 16 * NS : 1];
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          u32x4 n[NS];
#pragma unroll
          for (int c = 0; c < NS; ++c) n[c] = (t + KPF < DT) ? kop(kcur, t + KPF, c) : a[t % KPF][c];
#pragma unroll
          for (int c = 0; c < NS; ++c)
            sn[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[t % KPF][c]), qreg[t], sn[c], 0, 0, 0);
          const int e0 = (t * P1) / DT, e1 = ((t + 1) * P1) / DT;
#pragma unroll
          for (int idx = e0; idx < e1; ++idx) {  // key group idx / 8, element idx % 8
            const float pv = exp2_fast(__builtin_fmaf(s_cur[idx >> 4][idx & 15], c2, -muse));
            if constexpr (DEFER_SUM) pvs[idx] = pv;
            else rs += pv;
            pb[idx >> 3][idx & 7] = (__bf16)pv;
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int c = 0; c < NS; ++c) a[t % KPF][c] = n[c];
        }
        if constexpr (!DEFER_SUM) l += rs + xor32(rs);

        // phase 2
        constexpr int NCH = NP * DB;          // O^T MFMAs per tile
        constexpr int SPC = 16 * NS / NCH;    // tile j+1 scores handled per chunk
        const int kt1 = (j + 1) * BN;
        float mx = kNegInf;
        // V^T operands are read two MFMAs ahead: the transposing LDS reads take longer
        // than one MFMA, and a one-ahead read made every MFMA of this phase wait for them
        constexpr int VPF = 2;
        bf16x8 vq[VPF];
        // chunk k's (column block, key group): key-group-major when elements moved here
        auto cdb = [](int k) { return MV ? k % DB : k / NP; };
        auto ct4 = [](int k) { return MV ? k / DB : k % NP; };
#pragma unroll
        for (int u = 0; u < VPF; ++u) vq[u] = vop(vcur, cdb(u), ct4(u));
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
          const int db = cdb(k), t4 = ct4(k);
          if (k < MV) {  // element P1 + k of P_j
            const int idx = P1 + k;
            const float pv = exp2_fast(__builtin_fmaf(s_cur[idx >> 4][idx & 15], c2, -muse));
            pvs[idx] = pv;
            pb[idx >> 3][idx & 7] = (__bf16)pv;
          }
          const bf16x8 va = vq[k % VPF];
          if (k + VPF < NCH) vq[k % VPF] = vop(vcur, cdb(k + VPF), ct4(k + VPF));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[t4], oacc[db], 0, 0, 0);
#pragma unroll
          for (int e = 0; e < SPC; ++e) {
            const int idx = k * SPC + e;
            const int c = idx >> 4, v = idx & 15;
            mx = fmaxf(mx, sn[c][v]);
            if constexpr (DEFER_SUM) rs += pvs[idx];
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (DEFER_SUM) l += rs + xor32(rs);
        // a use of the row max here keeps its max3 chain between the MFMAs above; otherwise
        // the compiler sinks it past them into the unmasked branch below
        asm volatile("" : "+v"(mx));
        if (j + 1 >= nfull) {  // tile j+1 crosses the diagonal or the tail: mask, redo the max
          mx = kNegInf;
#pragma unroll
          for (int c = 0; c < NS; ++c)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              sn[c][v] = mask1(klim - kt1 - 4 * half, sn[c][v], c, v);
              mx = fmaxf(mx, sn[c][v]);
            }
        }
        finish_max(mx, mnew, grow);
      };
      // unrolled by two so every buffer address is a compile-time offset and S alternates
      // between sA and sB without copies; an odd last step runs after the loop
      int j = 0;
      for (; j + 1 < ntiles; j += 2) {
        step(j, kbuf1, kbuf0, vbuf0, vbuf1, sA, sB);
        step(j + 1, kbuf0, kbuf1, vbuf1, vbuf0, sB, sA);
      }
      if (j < ntiles) step(j, kbuf1, kbuf0, vbuf0, vbuf1, sA, sB);
    }

    // ---- epilogue: O = O_acc / l, lse = (m2 + log2 l) * ln 2.  O goes through the
    // wavefront's LDS slice (store_rows_lds): whole rows per store instruction.
    __syncthreads();  // every wave is done with the K / V tiles
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    store_rows_lds<D>((unsigned)(uintptr_t)(const lds_void*)(smem + wave * 32 * D * 2),
                      (uint16_t*)p.o + ooff + (int64_t)wrow0 * p.o_sn, p.o_sn, Lq - wrow0, oacc, inv, lane);
    if (qi < Lq && p.lse != nullptr && half == 0)
      p.lse[loff + (int64_t)qi * p.l_sn] = l > 0.f ? (m2 + __log2f(l)) * kLn2 : kNegInf;
  };  // row_block

  row_block(rbs[0]);
  if (rbs[1] != rbs[0]) {
    __syncthreads();  // every wave is done with the first block's LDS (its O slices)
    row_block(rbs[1]);
  }
}

// ----------------------------------------------------------------------------------
// fp32 VALU kernel (dense only): kFwdF32BM = 16 query rows per workgroup, 4 lanes per row
// in each of its NWV wavefronts (8 at d = 64, 4 at d = 128: one K / V slot each in LDS).
// The wavefronts take the key tiles in turn (tile j to wavefront j mod NWV), each
// through its own slot with no barrier in the loop, so a row block's keys are walked NWV
// tiles at a time; the partial states (m, l, O) merge through LDS at the end, as the
// decode combine merges splits.
// ----------------------------------------------------------------------------------
template <int D>
constexpr int f32_waves() { return D == 64 ? 8 : 4; }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * f32_waves<D>()) void fwd_f32_kernel(const FwdParams p) {
  constexpr int DL = D / 4;   // columns per lane
  constexpr int KT = 32;      // keys per LDS tile
  constexpr int RS = D + 4;   // LDS row stride (floats)
  constexpr int NWV = f32_waves<D>();  // wavefronts, each with its own K / V slot
  constexpr int SLOT = 2 * KT * RS;
  constexpr int PS = D + 2;   // merge record of a row: O, m, l
  static_assert(kFwdF32BM * PS <= SLOT, "a wavefront's merge records fit its slot");
  __shared__ __attribute__((aligned(16))) float sm[NWV * SLOT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane >> 2;
  const int part = lane & 3;
  int rb, b, h;
  block_coords<CAUSAL>(p, rb, b, h);
  int Lq, Lk;
  int64_t qoff, koff, voff, ooff, loff;
  seq_bounds<false>(p, b, h, Lq, Lk, qoff, koff, voff, ooff, loff);
  const int row0 = rb * kFwdF32BM;
  if (row0 >= Lq) return;  // uniform over the workgroup
  const int shift = Lk - Lq;
  int kend = Lk;
  if (CAUSAL) kend = min(Lk, max(0, row0 + kFwdF32BM + shift));
  const int ntiles = (kend + KT - 1) / KT;

  const float* Qg = (const float*)p.q + qoff;
  const float* Kg = (const float*)p.k + koff;
  const float* Vg = (const float*)p.v + voff;
  const int qi = row0 + row;

  float q[DL], o[DL];
#pragma unroll
  for (int c = 0; c < DL; ++c) {
    q[c] = qi < Lq ? Qg[(int64_t)qi * p.q_sn + part * DL + c] : 0.f;
    o[c] = 0.f;
  }
  float m2 = kNegInf, l = 0.f;
  const float c2 = p.scale_log2;
  float* const Ksh = sm + wave * SLOT;
  float* const Vsh = Ksh + KT * RS;

  for (int j = wave; j < ntiles; j += NWV) {
    const int kt0 = j * KT;
    // The slot's reads of the previous tile precede these writes in this wavefront's
    // program, and LDS instructions of one wavefront complete in order.
    asm volatile("" ::: "memory");
    for (int idx = lane; idx < KT * (D / 4); idx += 64) {
      const int key = idx / (D / 4), c4 = idx % (D / 4);
      const int gk = kt0 + key;
      float4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (gk < Lk) {
        kv = *(const float4*)(Kg + (int64_t)gk * p.k_sn + 4 * c4);
        vv = *(const float4*)(Vg + (int64_t)gk * p.v_sn + 4 * c4);
      }
      *(float4*)(Ksh + key * RS + 4 * c4) = kv;
      *(float4*)(Vsh + key * RS + 4 * c4) = vv;
    }
    asm volatile("" ::: "memory");

    float s[KT];
    float mx = kNegInf;
#pragma unroll
    for (int jj = 0; jj < KT; ++jj) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < DL; ++c) acc = __builtin_fmaf(q[c], Ksh[jj * RS + part * DL + c], acc);
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      const int key = kt0 + jj;
      const bool ok = key < Lk && (!CAUSAL || key <= qi + shift);
      s[jj] = ok ? acc : kNegInf;
      mx = fmaxf(mx, s[jj]);
    }
    const float mnew = fmaxf(m2, mx * c2);
    const float muse = (mnew == kNegInf) ? 0.f : mnew;
    const float alpha = exp2f(m2 - muse);
    float rs = 0.f;
#pragma unroll
    for (int jj = 0; jj < KT; ++jj) {
      s[jj] = exp2f(__builtin_fmaf(s[jj], c2, -muse));
      rs += s[jj];
    }
    l = l * alpha + rs;
    m2 = mnew;
#pragma unroll
    for (int c = 0; c < DL; ++c) o[c] *= alpha;
    // key by key, so that one key's V values are live at a time
#pragma unroll
    for (int jj = 0; jj < KT; ++jj) {
      const float* vr = Vsh + jj * RS + part * DL;
#pragma unroll
      for (int c = 0; c < DL; ++c) o[c] = __builtin_fmaf(s[jj], vr[c], o[c]);
    }
  }

  // Merge: each wavefront's (O, m, l) per row into its slot; wavefront 0 combines them,
  // M = max_w m_w, O = sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w, in wavefront order.
  __syncthreads();  // every wavefront is done with its tiles
  {
    float* rec = sm + wave * SLOT + row * PS;
#pragma unroll
    for (int c = 0; c < DL; ++c) rec[part * DL + c] = o[c];
    if (part == 0) {
      rec[D] = m2;
      rec[D + 1] = l;
    }
  }
  __syncthreads();
  if (wave != 0 || qi >= Lq) return;
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < NWV; ++w) M = fmaxf(M, sm[w * SLOT + row * PS + D]);
  const float Mu = (M == kNegInf) ? 0.f : M;
  float L = 0.f, acc[DL];
#pragma unroll
  for (int c = 0; c < DL; ++c) acc[c] = 0.f;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    const float* rec = sm + w * SLOT + row * PS;
    const float wt = exp2f(rec[D] - Mu);  // 0 for a wavefront that saw no admissible key
    L = __builtin_fmaf(wt, rec[D + 1], L);
#pragma unroll
    for (int c = 0; c < DL; ++c) acc[c] = __builtin_fmaf(wt, rec[part * DL + c], acc[c]);
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  float* Og = (float*)p.o + ooff + (int64_t)qi * p.o_sn + part * DL;
#pragma unroll
  for (int c = 0; c < DL; ++c) Og[c] = acc[c] * inv;
  if (p.lse != nullptr && part == 0) p.lse[loff + (int64_t)qi * p.l_sn] = L > 0.f ? (M + log2f(L)) * kLn2 : kNegInf;
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_bf16_t(const FwdParams& p, hipStream_t s) {
  constexpr int NW = kFwdNW;
  // dense causal: one workgroup per pair of row blocks (block_coords_pair)
  const int64_t nblk = (int64_t)(CAUSAL && !VARLEN ? (p.n_rb + 1) / 2 : p.n_rb) * p.H * p.B;
  if (nblk <= 0) return hipSuccess;
  const bool paged = VARLEN && p.block_table != nullptr;
  // causal varlen / paged batches of short sequences: 32-key tiles at 3 wavefronts per
  // SIMD (dense batches keep 64-key tiles: measured faster there, e.g. -10 % with 32-key
  // tiles on a causal 4 x 16 x 2048 batch, whose 1024 workgroups fill the chip in two
  // waves of two per CU)
  // (compile-time branches: only causal varlen instantiates the 32-key configuration,
  // only varlen the paged one)
  if constexpr (VARLEN && CAUSAL) {
    if ((int64_t)p.n_rb * kFwdBM <= kFwdShortLen) {
      constexpr int BN = kFwdShortBN, WPE = kFwdShortWPE;
      if (paged)
        hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, BN, WPE, CAUSAL, true, true>), dim3((unsigned)nblk), dim3(NW * 64), 0, s, p);
      else
        hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, BN, WPE, CAUSAL, true, false>), dim3((unsigned)nblk), dim3(NW * 64), 0, s, p);
      return hipGetLastError();
    }
  }
  if constexpr (VARLEN) {
    if (paged) {
      hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, kFwdBN, kFwdWPE, CAUSAL, true, true>), dim3((unsigned)nblk), dim3(NW * 64), 0, s, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, kFwdBN, kFwdWPE, CAUSAL, VARLEN, false>), dim3((unsigned)nblk), dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_f32_t(const FwdParams& p, hipStream_t s) {
  const int64_t nblk = (int64_t)p.n_rb * p.H * p.B;
  if (nblk <= 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)nblk), dim3(64 * f32_waves<D>()), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, bool varlen, hipStream_t s) {
  if (d == 128) {
    if (varlen) return causal ? launch_bf16_t<128, true, true>(p, s) : launch_bf16_t<128, false, true>(p, s);
    return causal ? launch_bf16_t<128, true, false>(p, s) : launch_bf16_t<128, false, false>(p, s);
  }
  if (varlen) return causal ? launch_bf16_t<64, true, true>(p, s) : launch_bf16_t<64, false, true>(p, s);
  return causal ? launch_bf16_t<64, true, false>(p, s) : launch_bf16_t<64, false, false>(p, s);
}

hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, hipStream_t s) {
  if (d == 128) return causal ? launch_f32_t<128, true>(p, s) : launch_f32_t<128, false>(p, s);
  return causal ? launch_f32_t<64, true>(p, s) : launch_f32_t<64, false>(p, s);
}

}  // namespace attn
