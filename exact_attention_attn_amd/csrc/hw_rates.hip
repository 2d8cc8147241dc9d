// Hardware rates behind the forward kernel's roofline on gfx950: how fast one SIMD
// issues 32x32x16 bf16 MFMAs alone and next to the rest of the forward's tile loop --
// LDS operand reads (16-byte reads as for K, pairs of transposing 8-byte reads as for
// V^T), VALU instructions (FMA and exp2), a workgroup barrier per tile, and the K/V tile
// loads that fill LDS -- at one and two wavefronts per SIMD, in the forward's layout of two
// 4-wavefront workgroups per CU and in one 8-wavefront workgroup; what vector-memory loads
// of each kind cost next to MFMAs; and 16x16x32 MFMAs whose LDS operand serves 2-4 query
// blocks.  A measurement aid, not part of libattn.so.
//
// Each test runs one workgroup per CU (the LDS array is sized above half of a CU's LDS),
// or two of 4 wavefronts with 64 KiB each, and times its loop with the shader's s_memtime
// counter ("ticks"; its rate against the 100 MHz s_memrealtime counter is printed).  The
// MFMA pipe counts as full at the rate two wavefronts reach with nothing but MFMAs to issue
// (the first row).  Every LDS read is the A operand of an MFMA and is issued two MFMAs ahead
// of it, as in the forward kernel; the VALU work runs on 8 independent chains.  Operand
// values are constant (0.5 and 0.25 in bf16), so these are the chip's unthrottled rates.
// Tile loads read a 2 MiB device buffer (L2-resident); every LDS and global address stays
// inside its array or buffer.
//
// Build: hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops
//        hw_rates.hip -o hw_rates        (build.py does this)
#include <hip/hip_runtime.h>

#include <cstdio>
#include <vector>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kTiles = 128;       // tiles of 32 MFMAs per wavefront and launch
constexpr int kLdsBytes = 81920;  // > 80 KiB: one workgroup per CU
constexpr int kBlocks = 256;      // one per CU

// Operand source of MFMA m (0..31) of a tile, by test mode:
//   0 none (register operands only); 1 all from 16-byte reads; 2 all from transposing
//   reads; 3 the forward's tile: the first 16 (S^T = K Q^T) from 16-byte reads, the last 16
//   (O^T += V^T P^T) from transposing reads; 4 as 3 for every second MFMA only (512 B per
//   MFMA: the operand shared by two 32-row query blocks).
// Returns 0 register, 1 16-byte read, 2 transposing pair.
constexpr int src_of(int mode, int m) {
  return mode == 0   ? 0
         : mode == 1 ? 1
         : mode == 2 ? 2
         : mode == 3 ? (m < 16 ? 1 : 2)
                     : ((m & 1) ? 0 : (m < 16 ? 1 : 2));
}

constexpr int lds_kib_per_tile(int mode) {
  int n = 0;
  for (int m = 0; m < 32; ++m) n += src_of(mode, m) != 0;
  return n;
}

__device__ __forceinline__ bf16x8 read_b128(unsigned a) {
  return __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(uintptr_t)a);
}

__device__ __forceinline__ bf16x8 read_tr(unsigned a) {
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)a);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)(a + 512u));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ void fill_lds(unsigned char* sm) {
  for (int i = threadIdx.x * 16; i < 65536; i += blockDim.x * 16)
    *(u32x4*)(sm + i) = u32x4{0x3f003e80u, 0x3e803f00u, 0x3f003e80u, 0x3e803f00u};
  __syncthreads();
}

// One tile = 32 MFMAs over CH accumulator chains, operands as `MODE` says; after each
// MFMA, NF FMAs and NE exp2s; BAR: a workgroup barrier after each tile.  LDSB: the LDS
// array's size (kLdsBytes: one workgroup per CU; 64 KiB: two).
// TL: the tile loads each wavefront issues per tile, NB blocks of 1 KiB from a 2 MiB
// global buffer (L2-resident) into its own 8 KiB of LDS, issued after the barrier and
// waited for before the next one, as in the forward:
//   0 none; 1 direct-to-LDS loads (buffer_load_dwordx4 ... lds), 16 rows x 64 B per
//   block (the forward's K blocks); 2 the same, 4 whole 256-byte rows per block; 3
//   global_load_dwordx4 into registers, written to LDS by ds_write_b128 before the barrier;
//   4 global_load_lds_dwordx4 (per-lane 64-bit addresses), 16 rows x 64 B; 5 buffer_load_dwordx4
//   into registers only (no LDS write); 7 buffer_load_dwordx2 into registers, two per 1 KiB
//   block; 8 as 5 from an 8 KiB source that every wavefront of the CU reads (L1 hits).
// With TL != 0 the workgroup has 4 wavefronts and LDSB = 64 KiB: tile buffers in the low
// 32 KiB, operand reads in the high 32 KiB.
// SH (8 wavefronts per workgroup): wavefronts 4-7 reach the barrier after MFMA 15 of their
// tile instead of 31, so the two wavefronts of each SIMD stay half a tile apart (each wavefront
// still issues its tile loads right after its barrier and lands them before the next).
// TLV (tile-load variant, direct-to-LDS only): 0 as the forward (s_nop 4 after the M0 write,
// all blocks issued after the barrier, waited for before the next); 1 s_nop 0; 2 one block
// issued after every fourth MFMA instead; 3 no wait before the barrier (timing only).
// BE: tiles per barrier (2: the loads of two tiles issued after each barrier, a four-stage ring).
template <int MODE, int CH, int NF, int NE, bool BAR, int LDSB = kLdsBytes, int TL = 0, int NB = 8, bool SH = false,
          int TLV = 0, int BE = 1>
__global__ void __launch_bounds__(512) tile_loop(long long* ticks, float* sink, float a, float b,
                                                 const unsigned char* gbuf) {
  __shared__ __attribute__((aligned(1024))) unsigned char sm[LDSB];
  fill_lds(sm);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  f32x16 c[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) c[i] = f32x16{};
  bf16x8 A0, B0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    A0[i] = (__bf16)0.5f;
    B0[i] = (__bf16)0.25f;
  }
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = a + 0.01f * lane + 0.1f * i;
  const unsigned base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)sm;
  // 1 KiB operand blocks k = 0..15 of the wavefront's 16 KiB stretch (stretches overlap:
  // all reads, so sharing is harmless); the last byte read is below 45 KiB
  const unsigned w0 = base + (unsigned)(wave * 4096) + (TL ? 32768u : 0u);
  // tile loads: lane offsets within a 1 KiB block, in the 2 MiB source
  const unsigned goff = TL == 2 ? (unsigned)((lane >> 4) * 256 + (lane & 15) * 16)
                                : (unsigned)((lane >> 2) * 256 + (lane & 3) * 16);
  const unsigned gwave = (unsigned)((blockIdx.x * (blockDim.x / 64) + wave) & 63) * 32768u;  // 32 KiB per wavefront
  u32x4 rsrc;
  rsrc.x = (unsigned)(uintptr_t)gbuf;
  rsrc.y = (unsigned)((uintptr_t)gbuf >> 32) & 0xFFFFu;
  rsrc.z = 2u << 20;
  rsrc.w = 0x00020000u;
  const unsigned ldst = base + (unsigned)(wave * NB * 1024);  // this wavefront's NB KiB of tile buffer
  u32x4 stage[TL == 3 || TL == 5 || TL == 7 || TL == 8 ? NB : 1];
  auto issue_block = [&](int t, int i) {
    // block i of tile t: 4 KiB of source rows per block (16 rows of 256 B) in the wavefront's 32 KiB
    const unsigned src = gwave + (unsigned)(((t * NB + i) & 7) * 4096) + goff +
                         (TL == 1 || TL == 4 ? (unsigned)((i & 3) * 64) : 0u);
    if constexpr (TL == 7) {
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)gbuf, (short)0, 2 << 20, 0x00020000);
      typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
      const unsigned o2 = gwave + (unsigned)(((t * NB + i) & 7) * 4096) + (unsigned)(lane * 8);
      const u32x2_t lo = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)o2, 0, 0));
      const u32x2_t hi = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)(o2 + 512u), 0, 0));
      stage[i] = u32x4{lo.x, lo.y, hi.x, hi.y};
    } else if constexpr (TL == 8) {
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)gbuf, (short)0, 2 << 20, 0x00020000);
      stage[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)((unsigned)(i * 1024) + goff), 0, 0));
    } else if constexpr (TL == 4) {
      const unsigned m0v = __builtin_amdgcn_readfirstlane(ldst + (unsigned)(i * 1024));
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %1, off"
                   :
                   : "s"(m0v), "v"(gbuf + src)
                   : "memory", "m0");
    } else if constexpr (TL == 5) {
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)gbuf, (short)0, 2 << 20, 0x00020000);
      stage[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)src, 0, 0));
    } else if constexpr (TL == 1 || TL == 2) {
      const unsigned m0v = __builtin_amdgcn_readfirstlane(ldst + (unsigned)(i * 1024));
      if constexpr (TLV == 1)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :
                     : "s"(m0v), "v"(src), "s"(rsrc)
                     : "memory", "m0");
      else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :
                     : "s"(m0v), "v"(src), "s"(rsrc)
                     : "memory", "m0");
    } else if constexpr (TL == 3) {
      stage[i] = *(const u32x4*)(gbuf + src);
    }
  };
  auto issue_tile = [&](int t) {
    if constexpr (TLV != 2) {
#pragma unroll
      for (int i = 0; i < NB; ++i) issue_block(t, i);
    }
  };
  auto land_tile = [&]() {
    if constexpr (TL != 0 && TLV != 3) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if constexpr (TL == 5 || TL == 7 || TL == 8) {
#pragma unroll
      for (int i = 0; i < NB; ++i) asm volatile("" : : "v"(stage[i]));
    }
    if constexpr (TL == 3) {
#pragma unroll
      for (int i = 0; i < NB; ++i) *(lds_u32x4*)(uintptr_t)(ldst + (unsigned)(i * 1024 + lane * 16)) = stage[i];
    }
  };
  auto fetch = [&](int src, int k) -> bf16x8 {
    if (src == 1) return read_b128(w0 + (unsigned)((k & 15) * 1024 + lane * 16));
    if (src == 2) return read_tr(w0 + (unsigned)((k & 15) * 1024 + lane * 8));
    return A0;
  };
  bf16x8 p0 = fetch(src_of(MODE, 0), 0), p1 = fetch(src_of(MODE, 1), 1);
  const long long t0 = clock64();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  const int barpos = SH && wave >= 4 ? 15 : 31;  // MFMA after which this wavefront meets the barrier
  if constexpr (TL != 0) issue_tile(0);
  for (int t = 0; t < kTiles; ++t) {
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const bf16x8 A = p0;
      p0 = p1;
      p1 = fetch(src_of(MODE, (m + 2) & 31), t * 32 + m + 2);
      c[m % CH] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B0, c[m % CH], 0, 0, 0);
#pragma unroll
      for (int v = 0; v < NF + NE; ++v) {
        const int i = (m * (NF + NE) + v) & 7;
        if (v < NE) x[i] = __builtin_amdgcn_exp2f(-x[i]);
        else x[i] = __builtin_fmaf(x[i], a, b);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (TL != 0 && TLV == 2) {
        if (m % 4 == 0 && m / 4 < NB) issue_block(t, m / 4);
      }
      if (m == 15 || m == 31) {
        if (m == barpos && t % BE == BE - 1) {  // uniform per wavefront; every wavefront meets the same barriers
          land_tile();
          if (BAR) __syncthreads();
          if constexpr (TL != 0)
#pragma unroll
            for (int u = 1; u <= BE; ++u) issue_tile(t + u);
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  const long long t1 = clock64();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = (float)p0[0] + (float)p1[0];
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
#pragma unroll
  for (int i = 0; i < CH; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += c[i][j];
  if (s == 1234.5f) sink[tid] = s;  // keeps the work; never true
  if (lane == 0) {
    ticks[blockIdx.x * (blockDim.x / 64) + wave] = t1 - t0;
    ticks[kBlocks * 8 + blockIdx.x * (blockDim.x / 64) + wave] = r1 - r0;  // 100 MHz counter
  }
}

// 16x16x32 MFMAs (half the flops of a 32x32x16): per iteration NA 1 KiB LDS reads, each
// (one read ahead) the A operand of R MFMAs (R query blocks of 16 rows sharing it); NV
// VALU instructions after each MFMA (FMA and exp2, two to one).
template <int NA, int R, int NV>
__global__ void __launch_bounds__(512) mix16(long long* ticks, float* sink, float a, float b) {
  __shared__ __attribute__((aligned(1024))) unsigned char sm[kLdsBytes];
  fill_lds(sm);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  f32x4 c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = f32x4{};
  bf16x8 B[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < 8; ++i) B[r][i] = (__bf16)(0.25f - i * 0.01f + r);
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = a + 0.01f * lane + 0.1f * i;
  const unsigned base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)sm;
  const unsigned off = (unsigned)(wave * 4096 + lane * 16);
  constexpr int kIters = kTiles * 32 / (NA * R);  // the same flops as the 32x32x16 loops
  const long long t0 = clock64();
  for (int it = 0; it < kIters; ++it) {
    u32x4 nxt = *(const lds_u32x4*)(uintptr_t)(base + off + (unsigned)(((it * 7) & 15) * 1024));
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const u32x4 cur = nxt;
      if (i + 1 < NA) nxt = *(const lds_u32x4*)(uintptr_t)(base + off + (unsigned)(((it * 7 + i + 1) & 15) * 1024));
      const bf16x8 A = __builtin_bit_cast(bf16x8, cur);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int ci = (i * R + r) & 7;
        c[ci] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B[r], c[ci], 0, 0, 0);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int j = (r * NV + v) & 7;
          if (v % 3 == 1) x[j] = __builtin_amdgcn_exp2f(-x[j]);
          else x[j] = __builtin_fmaf(x[j], a, b);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  const long long t1 = clock64();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i] + c[i][0] + c[i][1] + c[i][2] + c[i][3];
  if (s == 1234.5f) sink[tid] = s;
  if (lane == 0) ticks[blockIdx.x * 8 + wave] = t1 - t0;
}

double g_full = 0.0;                   // ticks per MFMA per SIMD with the pipe full (set by the first row)
const unsigned char* g_buf = nullptr;  // 2 MiB source of the tile-load tests

void launch(void (*k)(long long*, float*, float, float, const unsigned char*), int blocks, int threads,
            long long* ticks, float* sink) {
  hipLaunchKernelGGL(k, dim3(blocks), dim3(threads), 0, 0, ticks, sink, 0.3f, 0.7f, g_buf);
}
void launch(void (*k)(long long*, float*, float, float), int blocks, int threads, long long* ticks, float* sink) {
  hipLaunchKernelGGL(k, dim3(blocks), dim3(threads), 0, 0, ticks, sink, 0.3f, 0.7f);
}

double g_mhz = 0.0;  // s_memtime ticks per microsecond of the 100 MHz counter, last tile_loop run

// Mean ticks per launch of one wavefront (last of three launches), or -1 on failure.
template <typename K>
double mean_ticks(K kernel, int threads, long long* ticks, float* sink, int blocks = kBlocks) {
  double mean = -1.0;
  for (int rep = 0; rep < 3; ++rep) {
    launch(kernel, blocks, threads, ticks, sink);
    if (hipDeviceSynchronize() != hipSuccess) {
      fprintf(stderr, "launch failed\n");
      return -1.0;
    }
    const int n = blocks * (threads / 64);  // at most kBlocks * 8 entries
    std::vector<long long> h(n);
    if (hipMemcpy(h.data(), ticks, h.size() * sizeof(long long), hipMemcpyDeviceToHost) != hipSuccess) return -1.0;
    double s = 0.0;
    for (long long v : h) s += (double)v;
    mean = s / n;
    if (hipMemcpy(h.data(), ticks + kBlocks * 8, h.size() * sizeof(long long), hipMemcpyDeviceToHost) != hipSuccess)
      return -1.0;
    double r = 0.0;
    for (long long v : h) r += (double)v;
    g_mhz = r > 0.0 ? 100.0 * s / r : 0.0;
  }
  return mean;
}

// wps wavefronts per SIMD: one workgroup of 4 wps wavefronts per CU, or (two_wg) two
// workgroups of 4 wavefronts per CU, whose wavefronts pair up on the SIMDs as in the
// forward kernel.
template <int MODE, int CH, int NF, int NE, bool BAR, bool TWO_WG = false, int TL = 0, int NB = 8, bool SH = false,
          int TLV = 0, int BE = 1>
void run(int wps, long long* ticks, float* sink, const char* what) {
  const double t = TWO_WG ? mean_ticks(tile_loop<MODE, CH, NF, NE, BAR, 65536, TL, NB, false, TLV, BE>, 256, ticks, sink, 2 * kBlocks)
                          : mean_ticks(tile_loop<MODE, CH, NF, NE, BAR, kLdsBytes, TL, NB, SH, 0, BE>, 256 * wps, ticks, sink);
  if (t < 0) return;
  const double per = t / (kTiles * 32.0);  // ticks per MFMA per wavefront
  if (g_full == 0.0) g_full = per / wps;
  const double lds = lds_kib_per_tile(MODE) * 1024.0 * 4 * wps / (per * 32.0);  // B/tick/CU
  printf("| %-62s | %d | %6.1f | %5.1f %% | %6.1f | %5.0f |\n", what, wps, per, 100.0 * g_full * wps / per, lds, g_mhz);
}

template <int NA, int R, int NV>
void run16(long long* ticks, float* sink, const char* what) {
  const double t = mean_ticks(mix16<NA, R, NV>, 512, ticks, sink);
  if (t < 0) return;
  constexpr int kIters = kTiles * 32 / (NA * R);
  const double per = t / (kIters * NA * R / 2.0);  // ticks per 32 Kflop per wavefront
  const double lds = 1024.0 * NA * 8 / (per * NA * R / 2.0);
  printf("| %-62s | 2 | %6.1f | %5.1f %% | %6.1f |\n", what, per, 100.0 * g_full * 2 / per, lds);
}

}  // namespace

void header(const char* title) {
  printf("\n%s\n\n", title);
  printf("| loop | wavefronts per SIMD | ticks per MFMA per wavefront | MFMA pipe busy | LDS B/tick/CU | s_memtime MHz |\n");
  printf("|---|---|---|---|---|---|\n");
}

int main() {
  long long* ticks = nullptr;
  float* sink = nullptr;
  if (hipMalloc(&ticks, 2 * kBlocks * 8 * sizeof(long long)) != hipSuccess) return 1;
  if (hipMalloc(&sink, 512 * sizeof(float)) != hipSuccess) return 1;
  unsigned char* gb = nullptr;
  if (hipMalloc(&gb, 2u << 20) != hipSuccess || hipMemset(gb, 0x3f, 2u << 20) != hipSuccess) return 1;
  g_buf = gb;
  printf("32x32x16 bf16 MFMAs in tiles of 32; one operand per MFMA from LDS where stated, read two MFMAs ahead.\n");
  header("A. MFMA issue next to LDS operand reads and VALU work (one workgroup of 4 or 8 wavefronts per CU):");
  run<0, 4, 0, 0, false>(2, ticks, sink, "MFMA only, 4 chains per wavefront (defines the full pipe)");
  run<0, 8, 0, 0, false>(1, ticks, sink, "MFMA only, 8 chains");
  run<1, 4, 0, 0, false>(2, ticks, sink, "1 KiB 16-byte-read operand per MFMA");
  run<2, 4, 0, 0, false>(2, ticks, sink, "1 KiB transposing-read operand per MFMA");
  run<3, 4, 0, 0, false>(2, ticks, sink, "forward operands: 16 x K (16-byte), 16 x V^T (transposing)");
  run<0, 4, 4, 1, false>(2, ticks, sink, "no LDS, 5 VALU (1 exp2 + 4 FMA)");
  run<3, 4, 3, 1, false>(2, ticks, sink, "forward operands + 4 VALU (1 exp2 + 3 FMA)");
  run<3, 4, 4, 1, false>(2, ticks, sink, "forward operands + 5 VALU (1 exp2 + 4 FMA)");
  run<3, 4, 5, 0, false>(2, ticks, sink, "forward operands + 5 FMA (no exp2)");
  run<3, 4, 5, 1, false>(2, ticks, sink, "forward operands + 6 VALU (1 exp2 + 5 FMA)");
  run<3, 4, 4, 1, true>(2, ticks, sink, "forward operands + 5 VALU + barrier per tile (8 wavefronts)");
  header("B. The forward's layout: two workgroups of 4 wavefronts per CU, forward operands + 5 VALU:");
  run<3, 4, 4, 1, false, true>(2, ticks, sink, "no barrier, no tile loads");
  run<3, 4, 4, 1, true, true>(2, ticks, sink, "barrier per tile");
  run<3, 4, 4, 1, true, true, 1>(2, ticks, sink, "barrier + 8 KiB tile loads per wavefront: direct-to-LDS, 16 x 64 B");
  run<3, 4, 4, 1, true, true, 2>(2, ticks, sink, "the same, direct-to-LDS in whole rows");
  run<3, 4, 4, 1, true, true, 3>(2, ticks, sink, "the same, through registers and ds_write_b128");
  run<3, 4, 4, 1, true, true, 1, 8, false, 1>(2, ticks, sink, "direct-to-LDS, s_nop 0 after the M0 write");
  run<3, 4, 4, 1, true, true, 1, 8, false, 2>(2, ticks, sink, "direct-to-LDS, one block after every 4th MFMA");
  run<3, 4, 4, 1, true, true, 1, 8, false, 3>(2, ticks, sink, "direct-to-LDS, no wait before the barrier");
  run<3, 4, 4, 1, true, true, 1, 4>(2, ticks, sink, "4 KiB of tile loads per wavefront (256 rows per tile)");
  header("C. Vector-memory loads next to MFMAs alone (two workgroups of 4 per CU, barrier per tile):");
  run<0, 4, 0, 0, true, true>(2, ticks, sink, "no loads");
  run<0, 4, 0, 0, true, true, 1>(2, ticks, sink, "8 KiB per wavefront and tile, direct-to-LDS (8 x 1 KiB)");
  run<0, 4, 0, 0, true, true, 1, 8, false, 3>(2, ticks, sink, "the same, no wait before the barrier");
  run<0, 4, 0, 0, true, true, 4>(2, ticks, sink, "8 KiB, global_load_lds_dwordx4 (64-bit lane addresses)");
  run<0, 4, 0, 0, true, true, 5>(2, ticks, sink, "8 KiB into registers, 16 bytes per lane (8 loads)");
  run<0, 4, 0, 0, true, true, 7>(2, ticks, sink, "8 KiB into registers, 8 bytes per lane (16 loads)");
  run<0, 4, 0, 0, true, true, 8>(2, ticks, sink, "8 KiB into registers, 16 bytes per lane, L1 hits");
  header("D. More query rows per loaded tile:");
  run<3, 4, 4, 1, true, false, 1, 4>(2, ticks, sink, "8 wavefronts (256 rows), barrier, 4 KiB direct-to-LDS");
  run<3, 4, 4, 1, true, false, 1, 4, true>(2, ticks, sink, "the same, wavefronts 4-7 half a tile behind");
  run<3, 4, 4, 1, false, false, 1, 4>(2, ticks, sink, "8 wavefronts, 4 KiB direct-to-LDS, no barrier");
  run<3, 4, 4, 1, true, false, 1, 4, false, 0, 2>(2, ticks, sink, "8 wavefronts, 4 KiB direct-to-LDS, barrier every 2nd tile");
  run<3, 4, 4, 1, true, true, 1, 8, false, 0, 2>(2, ticks, sink, "two workgroups of 4, 8 KiB, barrier every 2nd tile");
  run<4, 4, 4, 1, false>(2, ticks, sink, "512 B operand per MFMA (64 rows per wavefront) + 5 VALU");
  run<0, 8, 4, 1, false>(1, ticks, sink, "no LDS, 5 VALU, 8 chains");
  run<4, 8, 4, 1, false>(1, ticks, sink, "512 B per MFMA + 5 VALU, 8 chains (64 rows per wavefront)");
  run<4, 8, 4, 1, true>(1, ticks, sink, "the same + barrier per tile");
  printf("\nE. 16x16x32 MFMAs, per 32 Kflop (two of them), LDS A operand shared by R MFMAs:\n\n");
  printf("| loop | wavefronts per SIMD | ticks per 32 Kflop per wavefront | MFMA pipe busy | LDS B/tick/CU |\n");
  printf("|---|---|---|---|---|\n");
  run16<8, 2, 0>(ticks, sink, "R = 2 (1 KiB LDS per 32 Kflop)");
  run16<8, 2, 3>(ticks, sink, "R = 2, 3 VALU per 16x16x32 (6 per 32 Kflop)");
  run16<6, 3, 0>(ticks, sink, "R = 3 (1 KiB per 48 Kflop, 48 rows per wavefront)");
  run16<6, 3, 3>(ticks, sink, "R = 3, 3 VALU per 16x16x32");
  run16<4, 4, 3>(ticks, sink, "R = 4 (1 KiB per 64 Kflop), 3 VALU per 16x16x32");
  return 0;
}
