// noalloc.hip -- the one-launch layer for callers that cannot allocate
// device memory (gfx950).
//
// gpb_compose_layer takes its staging region from the caller: the slabs the
// current rows are copied into before their pages are read back into the
// dense buffer.  gpb_compose_layer_noalloc takes it from a fixed array of
// the library's own instead, GPB_SCRATCH_BYTES on every GPU it runs on, so
// a caller that cannot call hipMalloc (code under HIP graph capture, a tight
// serving loop, a harness that forbids allocation) passes only its inputs
// and outputs.  The array keeps what the last call on that GPU wrote, so
// each call first clears the part it uses (a kernel, not a memset node),
// then runs the kernel of gpb_compose_layer on it.  Calls that overlap on
// one GPU share the array and race.
#include <mutex>

#include "gpb_common.h"

// The staging region of gpb_compose_layer_noalloc, one copy per GPU, held
// from the first call on a device until the process ends.  In host code the
// name only identifies the variable to the runtime; the device address of a
// GPU's copy comes from hipGetSymbolAddress and is the only one host code
// passes on.
static __device__ __align__(256) uint8_t scratch[GPB_SCRATCH_BYTES];

namespace gpb {
namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_base[kMaxDevices];  // address of `scratch` on device d, once known

// The address of the scratch array on `device`, which is the current device
// of the calling thread: looked up once per device, then cached.
int scratch_on(int device, uint8_t **out) {
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_base[device]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) {
      note_hip_error(e);
      return GPB_EHIP;
    }
    if (!p) return GPB_EHIP;
    scratch_base[device] = p;
  }
  *out = static_cast<uint8_t *>(scratch_base[device]);
  return GPB_OK;
}

}  // namespace
}  // namespace gpb

extern "C" int gpb_compose_layer_noalloc(void *d_dense, const gpb_sources *pools,
                                         int32_t n_writers, int32_t staging_cap_pages,
                                         const gpb_plan *plan, int32_t n_slots,
                                         int32_t n_cur_pages, const void *d_cur_rows,
                                         int32_t n_rows, int32_t page_rows,
                                         int32_t row_bytes, int32_t *d_status,
                                         void *stream) {
  using namespace gpb;
  if (!pools || pools->n < 1 || n_writers < 1 || staging_cap_pages < 1 || page_rows < 1 ||
      row_bytes < 1)
    return GPB_EINVAL;
  if (pools->n > GPB_MAX_SOURCES - n_writers) return GPB_EINVAL;  // table of pools + slabs
  if (row_bytes % 16 != 0) return GPB_EALIGN;
  // W slabs of CAP pages: every slab row is at least 16 bytes, so a slab of
  // more rows than the array has bytes is refused before any product can
  // overflow
  const int64_t slab_rows = static_cast<int64_t>(staging_cap_pages) * page_rows;
  if (slab_rows > GPB_SCRATCH_BYTES) return GPB_ESCRATCH;
  const int64_t slab_bytes = slab_rows * row_bytes;
  const int64_t n_staging_rows = slab_rows * n_writers;
  if (n_staging_rows * row_bytes > GPB_SCRATCH_BYTES) return GPB_ESCRATCH;

  // the scratch copy of the device the work runs on: the current device,
  // which the stream must belong to
  int device = -1;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) {
    note_hip_error(e);
    return GPB_EHIP;
  }
  if (device < 0 || device >= kMaxDevices) return GPB_EINVAL;
  if (stream) {
    int stream_device = -1;
    e = hipStreamGetDevice(as_stream(stream), &stream_device);
    if (e != hipSuccess) {
      note_hip_error(e);
      return GPB_EHIP;
    }
    if (stream_device != device) return GPB_EINVAL;
  }
  uint8_t *base = nullptr;
  const int rc = scratch_on(device, &base);
  if (rc != GPB_OK) return rc;

  gpb_sources table;
  table.n = pools->n + n_writers;
  for (int i = 0; i < GPB_MAX_SOURCES; ++i) {
    table.base[i] = nullptr;
    table.n_pages[i] = 0;
  }
  for (int i = 0; i < pools->n; ++i) {
    table.base[i] = pools->base[i];
    table.n_pages[i] = pools->n_pages[i];
  }
  for (int w = 0; w < n_writers; ++w) {
    table.base[pools->n + w] = base + w * slab_bytes;
    table.n_pages[pools->n + w] = staging_cap_pages;
  }
  return compose_layer(d_dense, d_dense, &table, plan, n_slots, n_cur_pages, base,
                       n_staging_rows, d_cur_rows, n_rows, page_rows, row_bytes, d_status,
                       stream, true, nullptr, -1, true);
}
