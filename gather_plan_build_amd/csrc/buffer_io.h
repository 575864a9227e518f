// Buffer-resource loads and stores shared by the per-layer kernels.
#pragma once

#include "gpb_common.h"

#ifndef GPB_LOAD_POLICY
#define GPB_LOAD_POLICY 2      // cache-policy bits of the buffer loads (nt)
#endif
#ifndef GPB_STORE_POLICY
// cache-policy bits of the row stores (scatter, fused fill, staging clear):
// sc1.  Measured on the traced workload (interleaved runs, 30 steps each): the
// scatter takes 16.0 us with sc1 and 16.8-17.1 us with nt or nt|sc1.
#define GPB_STORE_POLICY 16
#endif
#ifndef GPB_DENSE_STORE_POLICY
// cache-policy bits of the gather's dense-page stores: nt|sc1.  Interleaved
// A/B on MI355X, 3 runs of 30 steps per variant, scatter stores sc1 in all:
//   dense stores   traced us/layer   opaque us/layer
//   sc1            93.45             169.1
//   nt             94.78             165.3
//   nt|sc1         93.02-93.23       163.5-163.6
//   nt|sc0|sc1     93.24             163.4
//   sc0|sc1        93.82             169.4
//   nt|sc0         94.88             165.1
#define GPB_DENSE_STORE_POLICY 18
#endif

#ifndef GPB_LAYER_STAGING_POLICY
// cache-policy bits of the one-launch layer's staging stores and of its
// read-back of those bytes: plain (write-back L2, cached loads), so a store
// completes in L2 and the wave's read-back of the chunk does not wait on a
// write through to memory.  Interleaved probe on MI355X, traced workload,
// us per layer (staging store / read-back):
//   sc1 / nt 96.0   plain / nt 89.4   plain / plain 87.4   sc0 / sc0 87.4
//   sc0|sc1 / nt 96.0
#define GPB_LAYER_STAGING_POLICY 0
#endif
#ifndef GPB_LAYER_READBACK_POLICY
#define GPB_LAYER_READBACK_POLICY 0
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
__device__ __forceinline__ void st16_dense(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, GPB_DENSE_STORE_POLICY);
}
__device__ __forceinline__ void st16_staged(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, GPB_LAYER_STAGING_POLICY);
}
__device__ __forceinline__ u32x4 ld16_staged(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, GPB_LAYER_READBACK_POLICY);
}

}  // namespace gpb
