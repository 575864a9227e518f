// Internal helpers shared by the libgpb translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "gpb.h"

namespace gpb {

// 16-byte chunk: the unit every row copy moves (one global_load_dwordx4 /
// global_store_dwordx4 per lane).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;  // 4 wave64 per workgroup

inline bool aligned(const void *p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// The HIP error of the last refused launch on this thread (for gpb_strerror).
void note_hip_error(hipError_t e);

// Launch `kernel` with arguments converted to its parameter types and report
// the status of exactly this launch (hipGetLastError would also report errors
// that earlier, unrelated HIP calls on the thread left behind).  The launch
// is asynchronous: faults inside the kernel surface at the next
// synchronisation, not here.
template <typename... KArgs, typename... Args>
int launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
           Args &&...args) {
  std::tuple<KArgs...> values(static_cast<KArgs>(args)...);
  void *ptrs[sizeof...(KArgs)];
  std::apply([&ptrs](auto &...v) {
    int i = 0;
    ((ptrs[i++] = static_cast<void *>(&v)), ...);
  }, values);
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid,
                                       block, ptrs, 0, stream);
  if (e != hipSuccess) {
    note_hip_error(e);
    return GPB_EHIP;
  }
  return GPB_OK;
}

inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// compose.hip: the one-launch layer (with_prefix) or its consume half, after
// every host check; with d_pool and n_pool_rows >= 0 the fused fill, with
// clear_staging a clear of all n_staging_rows staging rows launched first.
int compose_layer(void *d_dense, void *d_dense_pre, const gpb_sources *table,
                  const gpb_plan *plan, int32_t n_slots, int32_t n_cur_pages,
                  void *d_staging, int64_t n_staging_rows, const void *d_cur_rows,
                  int32_t n_rows, int32_t page_rows, int32_t row_bytes, int32_t *d_status,
                  void *stream, bool with_prefix, void *d_pool, int64_t n_pool_rows,
                  bool clear_staging);

}  // namespace gpb
