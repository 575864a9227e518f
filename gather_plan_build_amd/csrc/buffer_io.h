// Buffer-resource loads and stores shared by the per-layer kernels.
#pragma once

#include "gpb_common.h"

#ifndef GPB_LOAD_POLICY
#define GPB_LOAD_POLICY 2      // cache-policy bits of the buffer loads (nt)
#endif
#ifndef GPB_STORE_POLICY
// cache-policy bits of the buffer stores: sc1.  Measured on the traced
// workload (interleaved runs, 30 steps each): sc1 on every per-layer store
// 93.7 us per layer, nt 94.5 us, sc1 on the scatter alone 94.8 us (the scatter
// itself is 5% faster with sc1, but mixed policies cost more between the two
// kernels than that saves).
#define GPB_STORE_POLICY 16
#endif

namespace gpb {

// Raw buffer resources: a base address plus a byte range the hardware checks
// on every access.  A load outside the range returns zeros and a store
// outside it is dropped, so ragged tails, -1 sentinels and bad rows need no
// branches around the memory instructions (branches around them would make
// the compiler wait for each store before the next).
constexpr int kRsrcWord3 = 0x00020000;         // 32-bit data format, raw addressing
constexpr uint32_t kDropOffset = 0x80000000u;  // beyond every range we build

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, kRsrcWord3);
}
__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, GPB_LOAD_POLICY);
}
__device__ __forceinline__ void st16(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, GPB_STORE_POLICY);
}

}  // namespace gpb
