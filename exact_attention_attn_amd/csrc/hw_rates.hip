// Hardware rates behind the forward kernel's roofline on gfx950: how fast one SIMD
// issues 32x32x16 bf16 MFMAs alone, next to VALU work, and next to LDS operand reads of
// the two sizes a wavefront tile can have (1 KiB per MFMA with 32 query rows per
// wavefront, 512 B with 64); the same for 16x16x32 MFMAs whose LDS operand serves 2-4
// query blocks of 16 rows; operands from global memory; and a forward split by role (one
// wavefront computes S and P for 64 rows, its partner accumulates O).  A measurement aid,
// not part of libattn.so.
//
// Each test runs one workgroup per CU (the LDS array is sized above half of a CU's LDS)
// of 4 or 8 wavefronts, i.e. 1 or 2 wavefronts per SIMD, and times its loop with the
// shader's s_memtime counter ("ticks").  The MFMA pipe is full when the SIMD retires one
// MFMA per kFullTicks ticks: the rate two wavefronts reach with nothing else to do.  The
// operands are constant, so these are the chip's unthrottled rates.  Every LDS address
// stays inside the workgroup's array; every store goes to one slot per wavefront.
//
// Build: hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops
//        hw_rates.hip -o hw_rates        (build.py does this)
#include <hip/hip_runtime.h>

#include <cstdio>
#include <vector>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int kIters = 256;
constexpr int kLdsBytes = 81920;  // > 80 KiB: one workgroup per CU
constexpr int kBlocks = 256;      // one per CU

// Per iteration: 16 MFMAs over CH accumulator chains; RD LDS reads of 16 B per lane
// (1 KiB per wavefront each) issued ahead of them; NV VALU instructions after each MFMA
// (FMA and exp2, two to one, on 8 independent chains).
template <int CH, int RD, int NV>
__global__ void __launch_bounds__(512) mix(long long* ticks, float* sink, float a, float b) {
  __shared__ __attribute__((aligned(1024))) unsigned char sm[kLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid * 16; i < 65536; i += blockDim.x * 16) *(u32x4*)(sm + i) = u32x4{(unsigned)i, 1u, 2u, 3u};
  __syncthreads();
  f32x16 c[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) c[i] = f32x16{};
  bf16x8 A, B;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    A[i] = (__bf16)(0.5f + i * 0.01f);
    B[i] = (__bf16)(0.25f - i * 0.01f);
  }
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = a + 0.01f * lane + 0.1f * i;
  const unsigned base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)sm;
  const unsigned off = (unsigned)(wave * 4096 + lane * 16);
  u32x4 acc = {0u, 0u, 0u, 0u};
  const long long t0 = clock64();
  for (int it = 0; it < kIters; ++it) {
    u32x4 r[RD > 0 ? RD : 1];
#pragma unroll
    for (int i = 0; i < RD; ++i) r[i] = *(const lds_u32x4*)(base + ((off + ((it * 7 + i) & 15) * 1024) & 0xFFF0u));
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      c[m % CH] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, c[m % CH], 0, 0, 0);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int i = (m * NV + v) & 7;
        if (v % 3 == 1) x[i] = __builtin_amdgcn_exp2f(-x[i]);
        else x[i] = __builtin_fmaf(x[i], a, b);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < RD; ++i) acc ^= r[i];
  }
  __builtin_amdgcn_s_waitcnt(0);
  const long long t1 = clock64();
  float s = (float)(acc.x + acc.y + acc.z + acc.w);
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
#pragma unroll
  for (int i = 0; i < CH; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += c[i][j];
  if (s == 1234.5f) sink[tid] = s;  // keeps the work; never true
  if (lane == 0) ticks[blockIdx.x * 8 + wave] = t1 - t0;
}

// The same with v_mfma_f32_16x16x32_bf16 (half the flops of a 32x32x16): NA LDS reads of
// 1 KiB per iteration, each the A operand of R MFMAs (R query blocks of 16 rows sharing
// it), NV VALU instructions after each MFMA.
template <int NA, int R, int NV>
__global__ void __launch_bounds__(512) mix16(long long* ticks, float* sink, float a, float b) {
  __shared__ __attribute__((aligned(1024))) unsigned char sm[kLdsBytes];
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid * 16; i < 65536; i += blockDim.x * 16) *(u32x4*)(sm + i) = u32x4{(unsigned)i, 1u, 2u, 3u};
  __syncthreads();
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
  const long long t0 = clock64();
  for (int it = 0; it < kIters; ++it) {
    u32x4 nxt = *(const lds_u32x4*)(base + ((off + ((it * 7) & 15) * 1024) & 0xFFF0u));
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const u32x4 cur = nxt;
      if (i + 1 < NA) nxt = *(const lds_u32x4*)(base + ((off + ((it * 7 + i + 1) & 15) * 1024) & 0xFFF0u));
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

// The same loop with GL of the 1 KiB operand reads per iteration taken from global
// memory (a 64 KiB buffer, L1/L2 resident) into registers instead of from LDS, one
// iteration ahead (consumed, like the LDS reads, by an XOR into a sink).  PAT 0: the
// MFMA operand pattern (lane l: row l % 32, 32 bytes of each of 32 rows of 256 B); PAT 1:
// whole rows (lane l: row l / 16, 16 bytes; 4 complete rows per instruction).
template <int RD, int GL, int PAT>
__global__ void __launch_bounds__(512) mixg(long long* ticks, float* sink, const u32x4* __restrict__ gbuf) {
  __shared__ __attribute__((aligned(1024))) unsigned char sm[kLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid * 16; i < 65536; i += blockDim.x * 16) *(u32x4*)(sm + i) = u32x4{(unsigned)i, 1u, 2u, 3u};
  __syncthreads();
  f32x16 c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = f32x16{};
  bf16x8 A, B;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    A[i] = (__bf16)(0.5f + i * 0.01f);
    B[i] = (__bf16)(0.25f - i * 0.01f);
  }
  const unsigned base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)sm;
  const unsigned off = (unsigned)(wave * 4096 + lane * 16);
  // byte offset of this lane's 16 bytes in a 1 KiB operand block (a 4 KiB stretch of rows)
  const unsigned goff = PAT == 0 ? (unsigned)((lane & 31) * 256 + (lane >> 5) * 16) : (unsigned)((lane >> 4) * 256 + (lane & 15) * 16);
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 g[GL > 0 ? GL : 1];
#pragma unroll
  for (int i = 0; i < GL; ++i) g[i] = gbuf[(goff + i * 32u) / 16];
  const long long t0 = clock64();
  for (int it = 0; it < kIters; ++it) {
    u32x4 r[RD > 0 ? RD : 1], gn[GL > 0 ? GL : 1];
#pragma unroll
    for (int i = 0; i < RD; ++i) r[i] = *(const lds_u32x4*)(base + ((off + ((it * 7 + i) & 15) * 1024) & 0xFFF0u));
    const unsigned blk = (unsigned)(((it + 1) * 5) & 15) * 4096u;  // 4 KiB stretch in the 64 KiB buffer
#pragma unroll
    for (int i = 0; i < GL; ++i) gn[i] = gbuf[(blk + goff + (unsigned)(i % 8) * 32u + (unsigned)(i / 8) * 8192u) % 65536u / 16u];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      c[m % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, c[m % 4], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < RD; ++i) acc ^= r[i];
#pragma unroll
    for (int i = 0; i < GL; ++i) {
      acc ^= g[i];
      g[i] = gn[i];
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  const long long t1 = clock64();
  float s = (float)(acc.x + acc.y + acc.z + acc.w);
#pragma unroll
  for (int i = 0; i < GL; ++i) s += (float)(g[i].x ^ g[i].w);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += c[i][j];
  if (s == 1234.5f) sink[tid] = s;  // keeps the work; never true
  if (lane == 0) ticks[blockIdx.x * 8 + wave] = t1 - t0;
}

// A forward split by role, two wavefronts per SIMD (8 per workgroup; wavefronts w and
// w + 4 share a SIMD, which the test reads back from HW_ID): wavefronts 0-3 play "S"
// (16 MFMAs per tile whose 1 KiB LDS operand serves two 32-row query blocks: RDS reads;
// NVS VALU instructions per MFMA, the whole softmax of 64 rows; WRS 16-byte LDS writes
// per lane, P for the partner) and wavefronts 4-7 play "PV" (16 MFMAs, RDP reads: the
// V^T operands shared by two query blocks and the partner's P; NVP VALU per MFMA).
// BAR: a workgroup barrier per tile, as the hand-over of P needs.  The same template
// with equal roles is the present kernel's mix.
template <int RDS, int NVS, int WRS, int RDP, int NVP, bool BAR>
__global__ void __launch_bounds__(512) mixrole(long long* ticks, unsigned* simd, float* sink, float a, float b) {
  __shared__ __attribute__((aligned(1024))) unsigned char sm[kLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid * 16; i < 65536; i += blockDim.x * 16) *(u32x4*)(sm + i) = u32x4{(unsigned)i, 1u, 2u, 3u};
  __syncthreads();
  const bool S = wave < 4;
  const int RD = S ? RDS : RDP;
  f32x16 c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = f32x16{};
  bf16x8 A, B;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    A[i] = (__bf16)(0.5f + i * 0.01f);
    B[i] = (__bf16)(0.25f - i * 0.01f);
  }
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = a + 0.01f * lane + 0.1f * i;
  const unsigned base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)sm;
  const unsigned off = (unsigned)(wave * 4096 + lane * 16);
  // P slots: 2 KiB per wavefront from byte 65536 on (the last ends at 81920)
  const unsigned woff = 65536u + (unsigned)(wave * 2048 + lane * 16);
  u32x4 acc = {0u, 0u, 0u, 0u};
  const long long t0 = clock64();
  for (int it = 0; it < kIters; ++it) {
    u32x4 r[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i < RD) r[i] = *(const lds_u32x4*)(base + ((off + ((it * 7 + i) & 15) * 1024) & 0xFFF0u));
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      c[m % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, c[m % 4], 0, 0, 0);
      if (S) {
#pragma unroll
        for (int v = 0; v < NVS; ++v) {
          const int i = (m * NVS + v) & 7;
          if (v % 3 == 1) x[i] = __builtin_amdgcn_exp2f(-x[i]);
          else x[i] = __builtin_fmaf(x[i], a, b);
        }
      } else {
#pragma unroll
        for (int v = 0; v < NVP; ++v) {
          const int i = (m * NVP + v) & 7;
          if (v % 3 == 1) x[i] = __builtin_amdgcn_exp2f(-x[i]);
          else x[i] = __builtin_fmaf(x[i], a, b);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i < RD) acc ^= r[i];
    if (S) {
#pragma unroll
      for (int w = 0; w < WRS; ++w)
        *(lds_u32x4*)(base + woff + (unsigned)((w & 1) * 1024)) = u32x4{__builtin_bit_cast(unsigned, x[w & 7]), acc.x, 0u, 0u};
    }
    if (BAR) __syncthreads();
  }
  __builtin_amdgcn_s_waitcnt(0);
  const long long t1 = clock64();
  float s = (float)(acc.x + acc.y + acc.z + acc.w);
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += c[i][j];
  if (s == 1234.5f) sink[tid] = s;  // keeps the work; never true
  if (lane == 0) {
    unsigned hw;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    ticks[blockIdx.x * 8 + wave] = t1 - t0;
    simd[blockIdx.x * 8 + wave] = (hw >> 4) & 3u;  // SIMD_ID
  }
}

constexpr double kFullTicks = 24.0;  // measured below: two wavefronts, MFMA only

template <int CH, int RD, int NV>
double run(int waves_per_simd, long long* ticks, float* sink, const char* what, bool print = true) {
  const int threads = 256 * waves_per_simd;
  double per = 0.0;
  for (int rep = 0; rep < 3; ++rep) {
    hipLaunchKernelGGL((mix<CH, RD, NV>), dim3(kBlocks), dim3(threads), 0, 0, ticks, sink, 0.3f, 0.7f);
    if (hipDeviceSynchronize() != hipSuccess) {
      fprintf(stderr, "launch failed\n");
      return -1.0;
    }
    std::vector<long long> h(kBlocks * 8);
    if (hipMemcpy(h.data(), ticks, h.size() * sizeof(long long), hipMemcpyDeviceToHost) != hipSuccess) return -1.0;
    double s = 0.0;
    int n = 0;
    for (int b = 0; b < kBlocks; ++b)
      for (int w = 0; w < threads / 64; ++w) {
        s += (double)h[b * 8 + w];
        ++n;
      }
    per = s / n / kIters / 16.0;  // ticks per MFMA per wavefront (last repetition)
  }
  const double pipe = kFullTicks * waves_per_simd / per;
  const double lds = RD * 1024.0 * 4 * waves_per_simd / (per * 16.0);  // LDS bytes per tick per CU
  if (print)
    printf("| %-58s | %d | %6.1f | %5.1f %% | %6.1f |\n", what, waves_per_simd, per, 100.0 * pipe, lds);
  return per;
}

}  // namespace

template <int RD, int GL, int PAT>
void rung(long long* ticks, float* sink, const u32x4* gbuf, const char* what) {
  double per = 0.0;
  for (int rep = 0; rep < 3; ++rep) {
    hipLaunchKernelGGL((mixg<RD, GL, PAT>), dim3(kBlocks), dim3(512), 0, 0, ticks, sink, gbuf);
    if (hipDeviceSynchronize() != hipSuccess) return;
    std::vector<long long> h(kBlocks * 8);
    if (hipMemcpy(h.data(), ticks, h.size() * sizeof(long long), hipMemcpyDeviceToHost) != hipSuccess) return;
    double s = 0.0;
    for (long long v : h) s += (double)v;
    per = s / h.size() / kIters / 16.0;  // ticks per MFMA per wavefront
  }
  const double lds = RD * 1024.0 * 8 / (per * 16.0), glb = GL * 1024.0 * 8 / (per * 16.0);
  printf("| %-58s | 2 | %6.1f | %5.1f %% | %6.1f | %6.1f |\n", what, per, 100.0 * kFullTicks * 2 / per, lds, glb);
}

// 16x16x32 loops at two wavefronts per SIMD, reported per 32 Kflop (one 32x32x16's work).
template <int NA, int R, int NV>
void run16(long long* ticks, float* sink, const char* what) {
  double per = 0.0;
  for (int rep = 0; rep < 3; ++rep) {
    hipLaunchKernelGGL((mix16<NA, R, NV>), dim3(kBlocks), dim3(512), 0, 0, ticks, sink, 0.3f, 0.7f);
    if (hipDeviceSynchronize() != hipSuccess) return;
    std::vector<long long> h(kBlocks * 8);
    if (hipMemcpy(h.data(), ticks, h.size() * sizeof(long long), hipMemcpyDeviceToHost) != hipSuccess) return;
    double s = 0.0;
    for (long long v : h) s += (double)v;
    per = s / h.size() / kIters / (NA * R / 2.0);  // ticks per 32 Kflop per wavefront
  }
  const double lds = 1024.0 * NA * 8 / (per * NA * R / 2.0);
  printf("| %-58s | 2 | %6.1f | %5.1f %% | %6.1f |\n", what, per, 100.0 * kFullTicks * 2 / per, lds);
}

// Role-split loops: ticks per MFMA of the slowest wavefront (the tile loop's pace when
// the roles are coupled), and in how many workgroups wavefronts w and w + 4 shared a SIMD.
template <int RDS, int NVS, int WRS, int RDP, int NVP, bool BAR>
void runrole(long long* ticks, unsigned* simd, float* sink, const char* what) {
  double per = 0.0;
  int shared = 0;
  for (int rep = 0; rep < 3; ++rep) {
    hipLaunchKernelGGL((mixrole<RDS, NVS, WRS, RDP, NVP, BAR>), dim3(kBlocks), dim3(512), 0, 0, ticks, simd, sink,
                       0.3f, 0.7f);
    if (hipDeviceSynchronize() != hipSuccess) return;
    std::vector<long long> h(kBlocks * 8);
    std::vector<unsigned> sd(kBlocks * 8);
    if (hipMemcpy(h.data(), ticks, h.size() * sizeof(long long), hipMemcpyDeviceToHost) != hipSuccess) return;
    if (hipMemcpy(sd.data(), simd, sd.size() * sizeof(unsigned), hipMemcpyDeviceToHost) != hipSuccess) return;
    long long mx = 0;
    for (long long v : h) mx = v > mx ? v : mx;
    per = (double)mx / kIters / 16.0;
    shared = 0;
    for (int b = 0; b < kBlocks; ++b) {
      bool ok = true;
      for (int w = 0; w < 4; ++w) ok = ok && sd[b * 8 + w] == sd[b * 8 + w + 4];
      shared += ok ? 1 : 0;
    }
  }
  printf("| %-58s | 2 | %6.1f | %5.1f %% | %d / %d |\n", what, per, 100.0 * kFullTicks * 2 / per, shared, kBlocks);
}

int main() {
  long long* ticks = nullptr;
  float* sink = nullptr;
  if (hipMalloc(&ticks, kBlocks * 8 * sizeof(long long)) != hipSuccess) return 1;
  if (hipMalloc(&sink, 512 * sizeof(float)) != hipSuccess) return 1;
  printf("| loop (per MFMA: LDS bytes read / VALU instructions) | wavefronts per SIMD | ticks per MFMA per wavefront | MFMA pipe busy | LDS B/tick/CU |\n");
  printf("|---|---|---|---|---|\n");
  run<4, 0, 0>(2, ticks, sink, "MFMA only, 4 chains per wavefront");
  run<8, 0, 0>(1, ticks, sink, "MFMA only, 8 chains");
  run<8, 0, 4>(1, ticks, sink, "MFMA + 4 VALU, 8 chains");
  run<4, 16, 0>(2, ticks, sink, "MFMA + 1 KiB LDS");
  run<4, 16, 5>(2, ticks, sink, "MFMA + 1 KiB LDS + 5 VALU (32 rows per wavefront)");
  run<4, 8, 0>(2, ticks, sink, "MFMA + 512 B LDS");
  run<4, 8, 5>(2, ticks, sink, "MFMA + 512 B LDS + 5 VALU (64 rows, if it fit 2/SIMD)");
  run<8, 8, 4>(1, ticks, sink, "MFMA + 512 B LDS + 4 VALU, 8 chains (64 rows per wavefront)");
  printf("\n16x16x32 MFMAs, per 32 Kflop (two of them), LDS A operand shared by R MFMAs:\n\n");
  printf("| loop | wavefronts per SIMD | ticks per 32 Kflop per wavefront | MFMA pipe busy | LDS B/tick/CU |\n");
  printf("|---|---|---|---|---|\n");
  run16<8, 2, 0>(ticks, sink, "R = 2 (1 KiB LDS per 32 Kflop)");
  run16<6, 3, 0>(ticks, sink, "R = 3 (1 KiB per 48 Kflop, 48 rows per wavefront)");
  run16<6, 3, 3>(ticks, sink, "R = 3, 3 VALU per 16x16x32 (6 per 32 Kflop)");
  run16<4, 4, 3>(ticks, sink, "R = 4 (1 KiB per 64 Kflop), 3 VALU per 16x16x32");
  u32x4* gbuf = nullptr;
  if (hipMalloc(&gbuf, 65536) != hipSuccess || hipMemset(gbuf, 0, 65536) != hipSuccess) return 1;
  printf("\nOperands from global memory (L1/L2-resident 64 KiB) instead of LDS, 16 MFMAs per iteration:\n\n");
  printf("| loop (per MFMA) | wavefronts per SIMD | ticks per MFMA per wavefront | MFMA pipe busy | LDS B/tick/CU | global B/tick/CU |\n");
  printf("|---|---|---|---|---|---|\n");
  rung<16, 0, 0>(ticks, sink, gbuf, "1 KiB LDS (reference)");
  rung<8, 8, 0>(ticks, sink, gbuf, "512 B LDS + 512 B global, operand pattern");
  rung<8, 8, 1>(ticks, sink, gbuf, "512 B LDS + 512 B global, whole rows");
  rung<0, 16, 0>(ticks, sink, gbuf, "1 KiB global, operand pattern");
  rung<0, 16, 1>(ticks, sink, gbuf, "1 KiB global, whole rows");
  rung<0, 8, 1>(ticks, sink, gbuf, "512 B global, whole rows");
  unsigned* simd = nullptr;
  if (hipMalloc(&simd, kBlocks * 8 * sizeof(unsigned)) != hipSuccess) return 1;
  printf("\nA forward split by role (per SIMD one S and one PV wavefront, 16 MFMAs each per tile), against the\n"
         "present mix (every wavefront: 16 MFMAs, 16 KiB of LDS reads, 5 VALU per MFMA); slowest wavefront:\n\n");
  printf("| loop per tile | wavefronts per SIMD | ticks per MFMA | MFMA pipe busy | workgroups with w, w + 4 on one SIMD |\n");
  printf("|---|---|---|---|---|\n");
  runrole<16, 5, 0, 16, 5, false>(ticks, simd, sink, "present mix");
  runrole<16, 5, 0, 16, 5, true>(ticks, simd, sink, "present mix, barrier per tile");
  runrole<8, 10, 4, 12, 0, true>(ticks, simd, sink, "split: S 8 KiB + 10 VALU/MFMA + P, PV 12 KiB; barrier");
  runrole<8, 10, 4, 12, 0, false>(ticks, simd, sink, "split as above, no barrier");
  runrole<8, 0, 0, 12, 0, true>(ticks, simd, sink, "split without the softmax VALU; barrier");
  return 0;
}
