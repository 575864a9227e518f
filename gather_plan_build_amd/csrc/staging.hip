// staging.hip -- the per-batch staging clear (gfx950).
//
// Page d63fbd4, commit "current rows written straight into staging": the
// current rows are copied into staging that holds zeros, so a last current
// page's rows beyond its request's tokens reach the dense buffer as zeros.
// A batch's scatter writes the same staging rows in every layer, so clearing
// once per batch is enough for all of its layers.
//
// A pure store stream: 256-lane workgroups, one 16-byte store per lane, 4 KiB
// per workgroup.  Stores alone are bound by the workgroup launch rate when a
// workgroup is a single wave with one KiB; four waves per workgroup clear
// 105 MiB in 13.5 us on MI355X (7.8 TB/s, partly absorbed by the 256 MB
// MALL) against 18.5 us for four non-temporal stores per lane.  The stores
// carry the per-layer kernels' policy, so the cleared lines the scatter then
// rewrites are handled like its own stores.
#include "buffer_io.h"
#include "gpb_common.h"

namespace gpb {
namespace {

constexpr int kClearBytes = kBlock * 16;  // bytes per workgroup

// The buffer range of the last workgroup ends at the region's end: its
// stores past it are dropped by the hardware range check.
__global__ __launch_bounds__(kBlock) void k_fill_zero(uint8_t *__restrict__ p,
                                                      int64_t n_bytes) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kClearBytes;
  const int64_t left = n_bytes - base;
  const int32_t range = left < kClearBytes ? static_cast<int32_t>(left) : kClearBytes;
  st16(u32x4{0, 0, 0, 0}, rsrc(p + base, range), threadIdx.x * 16u);
}

}  // namespace
}  // namespace gpb

extern "C" int gpb_staging_clear(void *d_ptr, int64_t n_bytes, void *stream) {
  using namespace gpb;
  if (n_bytes < 0) return GPB_EINVAL;
  if (n_bytes == 0) return GPB_OK;
  if (!d_ptr) return GPB_EINVAL;
  if (n_bytes % 16 != 0 || !aligned(d_ptr, 16)) return GPB_EALIGN;
  const int64_t grid = ceil_div64(n_bytes, kClearBytes);
  if (grid > INT32_MAX) return GPB_ERANGE;
  return launch(k_fill_zero, dim3(static_cast<uint32_t>(grid)), dim3(kBlock),
                as_stream(stream), static_cast<uint8_t *>(d_ptr), n_bytes);
}
