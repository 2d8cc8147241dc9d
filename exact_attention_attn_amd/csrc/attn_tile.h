// Device helpers shared by the forward and backward attention kernels of libattn.so
// (gfx950): vector types, the direct-to-LDS tile loads and small math helpers.
// Internal to the library; every translation unit gets its own copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

typedef unsigned u32x4s __attribute__((ext_vector_type(4)));

// Buffer resource for raw (unstrided) 16-byte loads of `bytes` bytes from `base`; reads
// past the end return zero.  Word 3 is the gfx9 raw-buffer format.
__device__ __forceinline__ u32x4s buffer_rsrc(const void* base, int64_t bytes) {
  // bytes > 0 here; clamp with 32-bit compares (the scalar unit has no 64-bit ordered compare)
  const unsigned hi = (unsigned)((uint64_t)bytes >> 32), lo = (unsigned)bytes;
  const unsigned nrec = (hi != 0u || lo > 0x7FFFFFFFu) ? 0x7FFFFFFFu : lo;
  const uint64_t a = (uint64_t)base;
  u32x4s r;
  r.x = (unsigned)a;
  r.y = (unsigned)(a >> 32) & 0xFFFFu;
  r.z = nrec;
  r.w = 0x00020000u;
  return r;
}

// 16-byte direct-to-LDS load per lane: lane i's data lands at lds + 16 i.  Issued as
// inline asm so the compiler does not see an asynchronous LDS write: it would otherwise
// make every later LDS read wait for all outstanding loads, which serialises the
// prefetch.  Completion is tracked explicitly (s_waitcnt vmcnt(0) before the barrier that
// publishes a buffer).
__device__ __forceinline__ void dma16(u32x4s r, const uint8_t* lds, int voffset) {
  const unsigned m0v = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(const lds_void*)lds);
  // The compiler's hazard recognizer does not look inside inline asm, so the wait states
  // the load needs are spelled out: one after the SALU write of M0, and five after a
  // VALU write of an SGPR it reads (v_readfirstlane of the descriptor or of M0's value).
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0v), "v"(voffset), "s"(r)
               : "memory", "m0");
}

// Same, from a per-lane 64-bit address (global_load_lds): the gather of paged K/V, whose
// rows may lie anywhere in pools larger than a buffer resource's 32-bit offsets reach.
// The address must be valid: paged keys past a sequence's end are clamped to its last
// key, so only block-table entries of the sequence's own pages are used.
__device__ __forceinline__ void dma16g(const void* src, const uint8_t* lds) {
  const unsigned m0v = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(const lds_void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(m0v), "v"(src)
               : "memory", "m0");
}

// The 32 rows held by a wavefront's 32x32 accumulators (lane l: row l % 32; D / 32
// accumulators of 32 columns each, element 4 i + e of accumulator db in column
// 32 db + 8 i + 4 (l / 32) + e), each multiplied by the lane's `mul` -> bf16 rows
// [0, nrows) of a row-major tensor at dst0 (row stride in elements, 16-byte aligned rows),
// through the wavefront's own LDS slice of 64 D bytes at byte address `slice`: written in
// the accumulators' layout with the 16-byte chunk index XOR-swizzled by the row
// (conflict-free), read back as whole rows, and stored 16 bytes per lane, so that each
// store instruction writes 64 / (D / 8) complete rows instead of 16 bytes of 32 rows.
template <int D>
__device__ __forceinline__ void store_rows_lds(unsigned slice, uint16_t* dst0, int64_t stride, int nrows,
                                               const f32x16* acc, float mul, int lane) {
  typedef __attribute__((address_space(3))) u32x2 lds_u32x2_t;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;
  constexpr int DB = D / 32, CPR = D / 8, RB = D * 2, RPI = 64 / CPR;
  const int half = lane >> 5, row = lane & 31;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 r0 = (__bf16)(acc[db][4 * i + 0] * mul), r1 = (__bf16)(acc[db][4 * i + 1] * mul);
      const __bf16 r2 = (__bf16)(acc[db][4 * i + 2] * mul), r3 = (__bf16)(acc[db][4 * i + 3] * mul);
      const unsigned u0 = (unsigned)__builtin_bit_cast(uint16_t, r0) | ((unsigned)__builtin_bit_cast(uint16_t, r1) << 16);
      const unsigned u1 = (unsigned)__builtin_bit_cast(uint16_t, r2) | ((unsigned)__builtin_bit_cast(uint16_t, r3) << 16);
      const int c = 4 * db + i;  // chunk of columns 32 db + 8 i .. +7; this lane's half is 4 of them
      *(lds_u32x2_t*)(uintptr_t)(slice + (unsigned)(row * RB + ((c ^ (row % CPR)) * 16) + 8 * half)) = u32x2{u0, u1};
    }
#pragma unroll
  for (int n = 0; n < 32 / RPI; ++n) {
    const int r = n * RPI + lane / CPR, c = lane % CPR;
    const u32x4 v = *(const lds_u32x4_t*)(uintptr_t)(slice + (unsigned)(r * RB + ((c ^ (r % CPR)) * 16)));
    if (r < nrows) *(u32x4*)(dst0 + (int64_t)r * stride + c * 8) = v;
  }
}

}  // namespace
}  // namespace attn
