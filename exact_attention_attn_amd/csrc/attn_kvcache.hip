// store_kvcache for gfx950: one step's new K/V rows are written into the paged KV pools
// through slot_mapping ("From standard Attention to FlashAttention and paged execution"
// (dlog.com.cn), the engine's attention step: store_kvcache runs before every attention
// call, prefill and decode alike).
//
// A pure copy, bound by HBM bandwidth: one wavefront moves one token's [H_kv, d] row of K
// and of V at a time, 64 lanes x 16 bytes per load, with the slot read once per token
// into a scalar register.  Slots outside the pool (padding, -1) are skipped, so no
// write can leave the pools whatever slot_mapping holds.
#include "attn_internal.h"

namespace attn {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kStoreWaves = 4;  // wavefronts per workgroup

__global__ __launch_bounds__(kStoreWaves * 64) void store_kvcache_kernel(const StoreParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int units = p.row_bytes >> 4;  // 16-byte units per token row
  const uint8_t* __restrict__ K = (const uint8_t*)p.k;
  const uint8_t* __restrict__ V = (const uint8_t*)p.v;
  uint8_t* __restrict__ Kc = (uint8_t*)p.k_cache;
  uint8_t* __restrict__ Vc = (uint8_t*)p.v_cache;
  for (int t = blockIdx.x * kStoreWaves + wave; t < p.T; t += gridDim.x * kStoreWaves) {
    const int64_t slot = p.slot_mapping[t];  // uniform over the wavefront
    if (slot < 0 || slot >= p.num_slots) continue;
    const uint8_t* ks = K + (int64_t)t * p.k_stride_bytes;
    const uint8_t* vs = V + (int64_t)t * p.v_stride_bytes;
    uint8_t* kd = Kc + slot * p.row_bytes;
    uint8_t* vd = Vc + slot * p.row_bytes;
    for (int c = lane; c < units; c += 64) {
      const u32x4 a = *(const u32x4*)(ks + 16 * c);
      const u32x4 b = *(const u32x4*)(vs + 16 * c);
      *(u32x4*)(kd + 16 * c) = a;
      *(u32x4*)(vd + 16 * c) = b;
    }
  }
}

}  // namespace

hipError_t launch_store_kvcache(const StoreParams& p, hipStream_t s) {
  if (p.T <= 0) return hipSuccess;
  // enough workgroups to keep every CU busy; the rest is covered by the token loop
  const int64_t want = ((int64_t)p.T + kStoreWaves - 1) / kStoreWaves;
  const unsigned blocks = (unsigned)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(store_kvcache_kernel, dim3(blocks), dim3(kStoreWaves * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace attn
