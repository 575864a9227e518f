// compose.hip -- per-layer current-row scatter and slot-dense page gather
// (gfx950).
//
// Page d63fbd4, commit "current rows written straight into staging": each
// layer first copies the current token rows into staging that was zeroed
// beforehand (index_copy_ semantics), then a single gather gives every dense
// slot a whole page, taken from a pointer table that lists the pool arenas
// and then the staging slabs (a prefix slot reads its pool page, a current
// slot reads staging slot i + 1 of its writer's slab).  Page d63fbd4, commit
// "compose_v2": an owner or src of -1 yields a zero page.  Page 0d87bc5,
// commit "fp8 index_copy_ -> uint8 views": rows are raw bytes.
//
// Kernels: k_compose_layer, both steps of a layer in one launch (the
// default; its unit is in layer_unit.h), and k_row_scatter and
// k_compose_gather, the two steps apart (for callers whose scatter and
// gather sit on two sides of a barrier, as on several GPUs).  All are
// HBM-bound copies with no arithmetic to speak of, so the design is about
// the memory system only:
//   - every lane moves 16-byte chunks (buffer_load_dwordx4 /
//     buffer_store_dwordx4), a wave64 moves one contiguous KiB per
//     instruction;
//   - the work is cut into many small units (one wave, one KiB per unit by
//     default), walked in address order: on MI355X this measured faster than
//     fewer, larger units (more chunks in flight per lane, 256-lane
//     workgroups), than part-major orders, than XCD-blocked orders and than a
//     persistent grid looping over the units;
//   - pool and current-row loads are non-temporal (each byte is read once
//     per layer); the dense stores carry nt|sc1; the separate scatter's
//     staging stores carry sc1 (their reader is the next kernel), the
//     one-launch layer's staging stores and read-back the plain policy (the
//     reader is the same wave), each measured fastest for its kernel here;
//     the one-launch layer forms the read-back from the staging region's
//     own resource, which L2 then serves for the most part;
//   - raw buffer resources bound every access, so ragged tails, -1 sentinels
//     and bad rows cost no branches;
//   - kernel arguments come in the order a wave reads them, the first 14
//     dwords preloaded into scalar registers at wave launch (the build passes
//     -amdgpu-kernarg-preload-count), the pointer table last: a wave's first
//     loads then wait on no argument-segment read, which shortened every
//     launch by 0.3-0.5 us here.
// The unit shape and cache-policy bits can be overridden at build time
// (-DGPB_GATHER_CPT=..., etc.) for tuning; the defaults are the measured best.
#include <algorithm>
#include <cstdio>

#include "buffer_io.h"
#include "gpb_common.h"
#include "layer_unit.h"

#ifndef GPB_GATHER_BLOCK
#define GPB_GATHER_BLOCK 64    // lanes per gather workgroup (one wave64)
#endif
#ifndef GPB_GATHER_CPT
#define GPB_GATHER_CPT 1       // 16-byte chunks per lane per unit
#endif
#ifndef GPB_SCATTER_BLOCK
#define GPB_SCATTER_BLOCK 64   // lanes per scatter workgroup
#endif
#ifndef GPB_SCATTER_CPT
#define GPB_SCATTER_CPT 1      // 16-byte chunks per lane
#endif

namespace gpb {
namespace {


typedef ArenaTable<GPB_MAX_SOURCES> SrcTable;

// How a gather workgroup finds its page: dense slot k (owner[k], src[k]),
// the k-th entry of a slot list (slots[k], then owner/src of that slot), or
// the k-th (slot, owner, src, 0) record, one 16-byte scalar load.
enum GatherMode { kAllSlots = 0, kSlotList = 1, kRecords = 2 };

// One workgroup per unit of a slot's page, units of a page consecutive.  The
// slot's descriptor is uniform across the workgroup: owner/src are scalar
// loads and both buffer resources live in scalar registers.  Lane l moves
// chunks l, l + B, ... of the unit.  An invalid or -1 descriptor gets a
// source range of 0 bytes: every load returns zeros.
template <int B, int CPT, int MODE>
__global__ __launch_bounds__(B) void k_compose_gather(
    const int32_t *__restrict__ list, const int32_t *__restrict__ owner,
    const int32_t *__restrict__ src, int32_t n_slots, int32_t parts, int32_t page_bytes,
    uint8_t *__restrict__ dense, int32_t *status, SrcTable tbl) {
  const int k_unit = blockIdx.x / parts;
  const int part = blockIdx.x - k_unit * parts;
  int slot = k_unit, e, p;
  if (MODE == kRecords) {
    const i32x4 rec = reinterpret_cast<const i32x4 *>(list)[k_unit];
    slot = rec.x;
    e = rec.y;
    p = rec.z;
  } else if (MODE == kSlotList) {
    slot = list[k_unit];
  }
  if (MODE != kAllSlots && (slot < 0 || slot >= n_slots)) {
    if (status && part == 0 && threadIdx.x == 0) atomicOr(status, GPB_STATUS_BAD_DESCRIPTOR);
    return;
  }
  if (MODE != kRecords) {
    e = owner[slot];
    p = src[slot];
  }
  const bool sentinel = (e < 0) || (p < 0);
  const bool in_table = !sentinel && e < tbl.n && p < tbl.e[e].n_pages;
  const uint8_t *from = in_table ? tbl.e[e].base + static_cast<int64_t>(p) * page_bytes : dense;
  const __amdgpu_buffer_rsrc_t rs = rsrc(from, in_table ? page_bytes : 0);
  const __amdgpu_buffer_rsrc_t rd =
      rsrc(dense + static_cast<int64_t>(slot) * page_bytes, page_bytes);
  const uint32_t first = (static_cast<uint32_t>(part) * (B * CPT) + threadIdx.x) * 16u;
  u32x4 v[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) v[k] = ld16(rs, first + k * (B * 16));
#pragma unroll
  for (int k = 0; k < CPT; ++k) st16_dense(v[k], rd, first + k * (B * 16));
  if (!sentinel && !in_table && status && part == 0 && threadIdx.x == 0)
    atomicOr(status, GPB_STATUS_BAD_DESCRIPTOR);
}

// One launch for a whole layer (layer_unit.h): the current pages' units
// first, then the prefix pages' units.  Prefix pages go to dense_pre, current
// pages to dense: the same buffer for one layer, or the next layer's dense
// buffer for the prefix pages when the launch is layer l's consume together
// with layer l + 1's prefetch (the table then lists layer l + 1's pool
// entries and layer l's staging slabs).
//
// Arguments every wave reads first come first (14 dwords, preloaded into
// scalar registers at wave launch), then those of the current units, then
// the table.  The fused fill is a kernel of its own: with the pool's
// arguments in this one, the plain layer measured 0.2-0.4 us slower per
// launch on MI355X.
template <int B, bool SROWS>
__global__ __launch_bounds__(B) void k_compose_layer(
    const int32_t *__restrict__ pre_desc, const int32_t *__restrict__ cur_desc,
    int32_t n_cur_units, int32_t parts, uint8_t *dense, uint8_t *dense_pre, int32_t *status,
    int32_t n_slots, int32_t page_bytes, const int32_t *__restrict__ tok0,
    const int32_t *__restrict__ ntok, uint8_t *staging, int32_t staging_bytes,
    int32_t n_staging_rows, const int32_t *__restrict__ rows, const uint8_t *__restrict__ cur,
    int32_t n_rows, int32_t row_chunks, SrcTable tbl) {
  const bool is_cur = static_cast<int>(blockIdx.x) < n_cur_units;
  const int u = is_cur ? blockIdx.x : blockIdx.x - n_cur_units;
  const int k = u / parts;
  layer_unit<B, SROWS, false>(tbl, dense, dense_pre, is_cur, k, u - k * parts, pre_desc,
                              cur_desc, tok0, ntok, staging, staging_bytes, n_staging_rows,
                              rows, cur, n_rows, row_chunks, n_slots, page_bytes, nullptr, 0,
                              nullptr, status);
}

// The same with the fused fill: current units also store each current-row
// chunk to the token's pool row.
template <int B, bool SROWS>
__global__ __launch_bounds__(B) void k_compose_layer_fill(
    const int32_t *__restrict__ pre_desc, const int32_t *__restrict__ cur_desc,
    int32_t n_cur_units, int32_t parts, uint8_t *dense, uint8_t *dense_pre, int32_t *status,
    int32_t n_slots, int32_t page_bytes, const int32_t *__restrict__ tok0,
    const int32_t *__restrict__ ntok, uint8_t *staging, int32_t staging_bytes,
    int32_t n_staging_rows, const int32_t *__restrict__ rows, const uint8_t *__restrict__ cur,
    int32_t n_rows, int32_t row_chunks, u32x4 *pool, int64_t n_pool_rows,
    const int32_t *__restrict__ pool_locs, SrcTable tbl) {
  const bool is_cur = static_cast<int>(blockIdx.x) < n_cur_units;
  const int u = is_cur ? blockIdx.x : blockIdx.x - n_cur_units;
  const int k = u / parts;
  layer_unit<B, SROWS, true>(tbl, dense, dense_pre, is_cur, k, u - k * parts, pre_desc,
                             cur_desc, tok0, ntok, staging, staging_bytes, n_staging_rows,
                             rows, cur, n_rows, row_chunks, n_slots, page_bytes, pool,
                             n_pool_rows, pool_locs, status);
}

// Flat over (row, chunk) of the current rows: lane g of the grid handles
// chunks g, g + B, ... of its workgroup's range; the (row, offset) pair
// advances by the precomputed (B div row_chunks, B mod row_chunks), so a lane
// divides once.  Consecutive lanes read consecutive source chunks; the
// destination row of each chunk comes from staging_rows.  Chunks past the
// last row read zeros and their stores go to kDropOffset (dropped), as do
// rows whose staging row is out of range.  With FILL, each chunk is also
// written to its row of the pool (pool_locs), with a 64-bit address since a
// pool may exceed one buffer range.
//
// With SROWS (rows of at least 21 chunks for one-wave, one-chunk units), a
// workgroup spans at most kScalarRows rows: their staging rows are fetched
// once with uniform scalar loads and each lane picks its own, instead of one
// vector load of an index per lane (2% faster on the traced workload).
template <int B, int CPT, bool FILL, bool SROWS>
__global__ __launch_bounds__(B) void k_row_scatter(
    const int32_t *__restrict__ rows, const uint8_t *__restrict__ cur,
    uint8_t *__restrict__ staging, int32_t n_rows, int32_t row_chunks, int32_t staging_bytes,
    int32_t n_staging_rows, int32_t step_rows, int32_t step_off, int32_t *status,
    u32x4 *__restrict__ pool, int64_t n_pool_rows, const int32_t *__restrict__ pool_locs) {
  const __amdgpu_buffer_rsrc_t rs = rsrc(cur, n_rows * row_chunks * 16);
  const __amdgpu_buffer_rsrc_t rd = rsrc(staging, staging_bytes);
  const int g = blockIdx.x * (B * CPT) + threadIdx.x;
  int row = g / row_chunks;
  int off = g - row * row_chunks;
  int srow[kScalarRows];
  const int row0 = static_cast<int>(blockIdx.x) * (B * CPT) / row_chunks;  // uniform
  if (SROWS) {
#pragma unroll
    for (int q = 0; q < kScalarRows; ++q) srow[q] = rows[min(row0 + q, n_rows - 1)];
  }
  u32x4 v[CPT];
  uint32_t dst[CPT];
  int64_t pdst[CPT];
  bool bad = false;
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const bool live = row < n_rows;
    const int last = live ? row : n_rows - 1;
    int d;
    if (SROWS) {
      const int q = row - row0;  // 0 .. kScalarRows - 1 for every live chunk
      d = srow[kScalarRows - 1];
#pragma unroll
      for (int u = kScalarRows - 2; u >= 0; --u) d = q == u ? srow[u] : d;
    } else {
      d = rows[last];
    }
    const bool ok = live && d >= 0 && d < n_staging_rows;
    bad |= live && !ok;
    v[k] = ld16(rs, static_cast<uint32_t>(row * row_chunks + off) * 16u);
    dst[k] = ok ? static_cast<uint32_t>(d * row_chunks + off) * 16u : kDropOffset;
    if (FILL) {
      const int64_t q = pool_locs[last];
      const bool okp = live && q >= 0 && q < n_pool_rows;
      bad |= live && !okp;
      pdst[k] = okp ? q * row_chunks + off : -1;
    }
    off += step_off;
    row += step_rows;
    if (off >= row_chunks) {
      off -= row_chunks;
      ++row;
    }
  }
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    st16(v[k], rd, dst[k]);
    if (FILL && pdst[k] >= 0) __builtin_nontemporal_store(v[k], pool + pdst[k]);
  }
  if (bad && status) atomicOr(status, GPB_STATUS_BAD_STAGING_ROW);
}

int launch_rows(void *d_staging, int64_t n_staging_rows, const int32_t *d_staging_rows,
                void *d_pool, int64_t n_pool_rows, const int32_t *d_pool_locs,
                const void *d_cur_rows, int32_t n_rows, int32_t row_bytes,
                int32_t *d_status, void *stream, bool fill) {
  constexpr int B = GPB_SCATTER_BLOCK, CPT = GPB_SCATTER_CPT;
  if (n_rows < 0 || n_staging_rows < 0 || row_bytes < 1) return GPB_EINVAL;
  if (fill && n_pool_rows < 0) return GPB_EINVAL;
  if (n_staging_rows > INT32_MAX) return GPB_ERANGE;
  if (row_bytes % 16 != 0) return GPB_EALIGN;
  if (d_status && !aligned(d_status, 4)) return GPB_EALIGN;
  if (n_rows == 0) return GPB_OK;
  if (!d_staging || !d_staging_rows || !d_cur_rows) return GPB_EINVAL;
  if (fill && (!d_pool || !d_pool_locs)) return GPB_EINVAL;
  if (!aligned(d_staging, 16) || !aligned(d_cur_rows, 16) || !aligned(d_staging_rows, 4))
    return GPB_EALIGN;
  if (fill && (!aligned(d_pool, 16) || !aligned(d_pool_locs, 4))) return GPB_EALIGN;
  const int64_t row_chunks = row_bytes / 16;
  // buffer ranges are 32-bit byte counts: both regions must stay below 2 GiB
  const int64_t cur_bytes = static_cast<int64_t>(n_rows) * row_bytes;
  const int64_t staging_bytes = n_staging_rows * row_bytes;
  if (cur_bytes > INT32_MAX || staging_bytes > INT32_MAX) return GPB_ERANGE;
  const int64_t total = static_cast<int64_t>(n_rows) * row_chunks;
  const int64_t grid = ceil_div64(total, static_cast<int64_t>(B) * CPT);
  const dim3 g(static_cast<uint32_t>(grid)), b(B);
  hipStream_t st = as_stream(stream);
  // B * CPT consecutive chunks touch at most 2 + (B * CPT - 2) / row_chunks rows
  const bool srows = 2 + (B * CPT - 2) / row_chunks <= kScalarRows;
  const int32_t rc = static_cast<int32_t>(row_chunks);
  const int32_t sr = static_cast<int32_t>(B / row_chunks), so = static_cast<int32_t>(B % row_chunks);
  const auto kernel = fill ? (srows ? k_row_scatter<B, CPT, true, true>
                                    : k_row_scatter<B, CPT, true, false>)
                           : (srows ? k_row_scatter<B, CPT, false, true>
                                    : k_row_scatter<B, CPT, false, false>);
  return launch(kernel, g, b, st, d_staging_rows, d_cur_rows, d_staging, n_rows, rc,
                staging_bytes, n_staging_rows, sr, so, d_status, fill ? d_pool : nullptr,
                fill ? n_pool_rows : 0, fill ? d_pool_locs : nullptr);
}

// Host checks shared by the two gathers; fills the kernel's table.
int check_gather(const gpb_sources *table, int32_t n_slots, int32_t page_rows,
                 int32_t row_bytes, int32_t *d_status, SrcTable *t, int64_t *page_bytes) {
  if (!table || n_slots < 0 || page_rows < 1 || row_bytes < 1) return GPB_EINVAL;
  if (table->n < 1 || table->n > GPB_MAX_SOURCES) return GPB_EINVAL;
  if (row_bytes % 16 != 0) return GPB_EALIGN;
  if (d_status && !aligned(d_status, 4)) return GPB_EALIGN;
  *page_bytes = static_cast<int64_t>(page_rows) * row_bytes;
  // a page is one buffer range: 32-bit byte count, with room for the last unit
  if (*page_bytes > INT32_MAX - (1 << 20)) return GPB_ERANGE;
  t->n = table->n;
  t->pad = 0;
  for (int e = 0; e < GPB_MAX_SOURCES; ++e) t->e[e] = ArenaEntry{nullptr, 0};
  for (int e = 0; e < table->n; ++e) {
    if (table->n_pages[e] < 0) return GPB_EINVAL;
    if (table->n_pages[e] > 0 && !table->base[e]) return GPB_EINVAL;
    if (!aligned(table->base[e], 16)) return GPB_EALIGN;
    t->e[e] = ArenaEntry{static_cast<const uint8_t *>(table->base[e]), table->n_pages[e]};
  }
  return GPB_OK;
}

}  // namespace
}  // namespace gpb

extern "C" int gpb_current_row_scatter(void *d_staging, int64_t n_staging_rows,
                                       const int32_t *d_staging_rows,
                                       const void *d_cur_rows, int32_t n_rows,
                                       int32_t row_bytes, int32_t *d_status,
                                       void *stream) {
  return gpb::launch_rows(d_staging, n_staging_rows, d_staging_rows, nullptr, 0, nullptr,
                          d_cur_rows, n_rows, row_bytes, d_status, stream, false);
}

extern "C" int gpb_current_row_fill(void *d_staging, int64_t n_staging_rows,
                                    const int32_t *d_staging_rows, void *d_pool,
                                    int64_t n_pool_rows, const int32_t *d_pool_locs,
                                    const void *d_cur_rows, int32_t n_rows,
                                    int32_t row_bytes, int32_t *d_status, void *stream) {
  return gpb::launch_rows(d_staging, n_staging_rows, d_staging_rows, d_pool, n_pool_rows,
                          d_pool_locs, d_cur_rows, n_rows, row_bytes, d_status, stream,
                          true);
}

extern "C" int gpb_compose_gather(void *d_dense, const gpb_sources *table,
                                  const int32_t *d_owner, const int32_t *d_src,
                                  int32_t n_slots, int32_t page_rows,
                                  int32_t row_bytes, int32_t *d_status,
                                  void *stream) {
  using namespace gpb;
  constexpr int B = GPB_GATHER_BLOCK, CPT = GPB_GATHER_CPT;
  SrcTable t;
  int64_t page_bytes = 0;
  int rc = check_gather(table, n_slots, page_rows, row_bytes, d_status, &t, &page_bytes);
  if (rc != GPB_OK) return rc;
  if (n_slots == 0) return GPB_OK;
  if (!d_dense || !d_owner || !d_src) return GPB_EINVAL;
  if (!aligned(d_dense, 16) || !aligned(d_owner, 4) || !aligned(d_src, 4)) return GPB_EALIGN;
  const int64_t parts = ceil_div64(page_bytes / 16, static_cast<int64_t>(B) * CPT);
  const int64_t grid = parts * n_slots;
  if (grid > INT32_MAX) return GPB_ERANGE;
  return launch(k_compose_gather<B, CPT, kAllSlots>, dim3(static_cast<uint32_t>(grid)),
                dim3(B), as_stream(stream), nullptr, d_owner, d_src, n_slots, parts,
                page_bytes, d_dense, d_status, t);
}

extern "C" int gpb_compose_gather_slots(void *d_dense, const gpb_sources *table,
                                        const int32_t *d_slots, int32_t n_list,
                                        const int32_t *d_owner, const int32_t *d_src,
                                        int32_t n_slots, int32_t page_rows,
                                        int32_t row_bytes, int32_t *d_status,
                                        void *stream) {
  using namespace gpb;
  constexpr int B = GPB_GATHER_BLOCK, CPT = GPB_GATHER_CPT;
  SrcTable t;
  int64_t page_bytes = 0;
  int rc = check_gather(table, n_slots, page_rows, row_bytes, d_status, &t, &page_bytes);
  if (rc != GPB_OK) return rc;
  if (n_list < 0) return GPB_EINVAL;
  if (n_list == 0) return GPB_OK;
  if (!d_dense || !d_owner || !d_src || !d_slots || n_slots == 0) return GPB_EINVAL;
  if (!aligned(d_dense, 16) || !aligned(d_owner, 4) || !aligned(d_src, 4) ||
      !aligned(d_slots, 4))
    return GPB_EALIGN;
  const int64_t parts = ceil_div64(page_bytes / 16, static_cast<int64_t>(B) * CPT);
  const int64_t grid = parts * n_list;
  if (grid > INT32_MAX) return GPB_ERANGE;
  return launch(k_compose_gather<B, CPT, kSlotList>, dim3(static_cast<uint32_t>(grid)),
                dim3(B), as_stream(stream), d_slots, d_owner, d_src, n_slots, parts,
                page_bytes, d_dense, d_status, t);
}

extern "C" int gpb_compose_gather_records(void *d_dense, const gpb_sources *table,
                                          const int32_t *d_records, int32_t n_records,
                                          int32_t n_slots, int32_t page_rows,
                                          int32_t row_bytes, int32_t *d_status,
                                          void *stream) {
  using namespace gpb;
  constexpr int B = GPB_GATHER_BLOCK, CPT = GPB_GATHER_CPT;
  SrcTable t;
  int64_t page_bytes = 0;
  int rc = check_gather(table, n_slots, page_rows, row_bytes, d_status, &t, &page_bytes);
  if (rc != GPB_OK) return rc;
  if (n_records < 0) return GPB_EINVAL;
  if (n_records == 0) return GPB_OK;
  if (!d_dense || !d_records || n_slots == 0) return GPB_EINVAL;
  if (!aligned(d_dense, 16) || !aligned(d_records, 16)) return GPB_EALIGN;
  const int64_t parts = ceil_div64(page_bytes / 16, static_cast<int64_t>(B) * CPT);
  const int64_t grid = parts * n_records;
  if (grid > INT32_MAX) return GPB_ERANGE;
  return launch(k_compose_gather<B, CPT, kRecords>, dim3(static_cast<uint32_t>(grid)),
                dim3(B), as_stream(stream), d_records, nullptr, nullptr, n_slots, parts,
                page_bytes, d_dense, d_status, t);
}

namespace gpb {
// The layer in one launch (with_prefix; prefix pages into d_dense_pre) or
// its consume half only: the same kernel over all units, or over the current
// pages' units alone.  With clear_staging, a launch of its own first zeroes
// the whole staging region (all n_staging_rows rows), after every host check
// has passed.
int compose_layer(void *d_dense, void *d_dense_pre, const gpb_sources *table,
                  const gpb_plan *plan, int32_t n_slots, int32_t n_cur_pages,
                  void *d_staging, int64_t n_staging_rows, const void *d_cur_rows,
                  int32_t n_rows, int32_t page_rows, int32_t row_bytes, int32_t *d_status,
                  void *stream, bool with_prefix, void *d_pool, int64_t n_pool_rows,
                  bool clear_staging) {
  const bool fill = n_pool_rows >= 0;
  constexpr int B = 64;
  SrcTable t;
  int64_t page_bytes = 0;
  int rc = check_gather(table, n_slots, page_rows, row_bytes, d_status, &t, &page_bytes);
  if (rc != GPB_OK) return rc;
  if (!plan || n_cur_pages < 0 || n_cur_pages > n_slots || n_rows < 0 || n_staging_rows < 0)
    return GPB_EINVAL;
  // every current page holds at least one current row
  if (n_cur_pages > n_rows) return GPB_EINVAL;
  if (n_staging_rows > INT32_MAX) return GPB_ERANGE;
  if (n_slots == 0) return GPB_OK;
  const int32_t n_prefix = n_slots - n_cur_pages;
  if (!d_dense || (with_prefix && n_prefix > 0 && (!plan->d_prefix_desc || !d_dense_pre)))
    return GPB_EINVAL;
  if (with_prefix && !aligned(d_dense_pre, 16)) return GPB_EALIGN;
  if (n_cur_pages > 0 && (!plan->d_current_desc || !plan->d_cur_page_token0 ||
                          !plan->d_cur_page_ntok || !d_staging ||
                          (n_rows > 0 && (!plan->d_staging_rows || !d_cur_rows))))
    return GPB_EINVAL;
  if (fill && n_cur_pages > 0 && (!d_pool || !plan->d_pool_locs)) return GPB_EINVAL;
  if (!aligned(d_dense, 16) || !aligned(plan->d_prefix_desc, 16) ||
      !aligned(plan->d_current_desc, 16) || !aligned(plan->d_cur_page_token0, 4) ||
      !aligned(plan->d_cur_page_ntok, 4) || !aligned(plan->d_staging_rows, 4) ||
      !aligned(d_staging, 16) || !aligned(d_cur_rows, 16))
    return GPB_EALIGN;
  if (fill && (!aligned(d_pool, 16) || !aligned(plan->d_pool_locs, 4))) return GPB_EALIGN;
  const int64_t row_chunks = row_bytes / 16;
  const int64_t cur_bytes = static_cast<int64_t>(n_rows) * row_bytes;
  const int64_t staging_bytes = n_staging_rows * row_bytes;
  if (cur_bytes > INT32_MAX || staging_bytes > INT32_MAX) return GPB_ERANGE;
  const int64_t parts = ceil_div64(page_bytes / 16, B);
  const int64_t grid = parts * (with_prefix ? n_slots : n_cur_pages);
  if (grid > INT32_MAX) return GPB_ERANGE;
  if (grid == 0) return GPB_OK;
  // a unit of B chunks touches at most 2 + (B - 2) / row_chunks rows
  const bool srows = 2 + (B - 2) / row_chunks <= kScalarRows;
  const dim3 g(static_cast<uint32_t>(grid)), b(B);
  const int32_t cur_units = static_cast<int32_t>(parts * n_cur_pages);
  void *const pre = with_prefix ? d_dense_pre : d_dense;
  const int32_t chunks = static_cast<int32_t>(row_chunks);
  if (clear_staging && n_cur_pages > 0) {
    const int rc_clear = gpb_staging_clear(d_staging, staging_bytes, stream);
    if (rc_clear != GPB_OK) return rc_clear;
  }
  if (fill)
    return launch(srows ? k_compose_layer_fill<B, true> : k_compose_layer_fill<B, false>, g, b,
                  as_stream(stream), plan->d_prefix_desc, plan->d_current_desc, cur_units,
                  parts, d_dense, pre, d_status, n_slots, page_bytes, plan->d_cur_page_token0,
                  plan->d_cur_page_ntok, d_staging, staging_bytes, n_staging_rows,
                  plan->d_staging_rows, d_cur_rows, n_rows, chunks, d_pool, n_pool_rows,
                  plan->d_pool_locs, t);
  return launch(srows ? k_compose_layer<B, true> : k_compose_layer<B, false>, g, b,
                as_stream(stream), plan->d_prefix_desc, plan->d_current_desc, cur_units, parts,
                d_dense, pre, d_status, n_slots, page_bytes, plan->d_cur_page_token0,
                plan->d_cur_page_ntok, d_staging, staging_bytes, n_staging_rows,
                plan->d_staging_rows, d_cur_rows, n_rows, chunks, t);
}
}  // namespace gpb

extern "C" int gpb_compose_layer(void *d_dense, const gpb_sources *table,
                                 const gpb_plan *plan, int32_t n_slots, int32_t n_cur_pages,
                                 void *d_staging, int64_t n_staging_rows,
                                 const void *d_cur_rows, int32_t n_rows, int32_t page_rows,
                                 int32_t row_bytes, int32_t *d_status, void *stream) {
  return gpb::compose_layer(d_dense, d_dense, table, plan, n_slots, n_cur_pages, d_staging,
                            n_staging_rows, d_cur_rows, n_rows, page_rows, row_bytes,
                            d_status, stream, true, nullptr, -1, false);
}

extern "C" int gpb_compose_layer_fill(void *d_dense, const gpb_sources *table,
                                      const gpb_plan *plan, int32_t n_slots,
                                      int32_t n_cur_pages, void *d_staging,
                                      int64_t n_staging_rows, void *d_pool,
                                      int64_t n_pool_rows, const void *d_cur_rows,
                                      int32_t n_rows, int32_t page_rows, int32_t row_bytes,
                                      int32_t *d_status, void *stream) {
  if (n_pool_rows < 0) return GPB_EINVAL;
  return gpb::compose_layer(d_dense, d_dense, table, plan, n_slots, n_cur_pages, d_staging,
                            n_staging_rows, d_cur_rows, n_rows, page_rows, row_bytes,
                            d_status, stream, true, d_pool, n_pool_rows, false);
}

extern "C" int gpb_compose_layer_ahead(void *d_dense, void *d_dense_next,
                                       const gpb_sources *table, const gpb_plan *plan,
                                       int32_t n_slots, int32_t n_cur_pages, void *d_staging,
                                       int64_t n_staging_rows, const void *d_cur_rows,
                                       int32_t n_rows, int32_t page_rows, int32_t row_bytes,
                                       int32_t *d_status, void *stream) {
  return gpb::compose_layer(d_dense, d_dense_next, table, plan, n_slots, n_cur_pages,
                            d_staging, n_staging_rows, d_cur_rows, n_rows, page_rows,
                            row_bytes, d_status, stream, true, nullptr, -1, false);
}

extern "C" int gpb_compose_consume(void *d_dense, const gpb_sources *table,
                                   const gpb_plan *plan, int32_t n_slots,
                                   int32_t n_cur_pages, void *d_staging,
                                   int64_t n_staging_rows, const void *d_cur_rows,
                                   int32_t n_rows, int32_t page_rows, int32_t row_bytes,
                                   int32_t *d_status, void *stream) {
  return gpb::compose_layer(d_dense, nullptr, table, plan, n_slots, n_cur_pages, d_staging,
                            n_staging_rows, d_cur_rows, n_rows, page_rows, row_bytes,
                            d_status, stream, false, nullptr, -1, false);
}

extern "C" int gpb_compose_consume_fill(void *d_dense, const gpb_sources *table,
                                        const gpb_plan *plan, int32_t n_slots,
                                        int32_t n_cur_pages, void *d_staging,
                                        int64_t n_staging_rows, void *d_pool,
                                        int64_t n_pool_rows, const void *d_cur_rows,
                                        int32_t n_rows, int32_t page_rows, int32_t row_bytes,
                                        int32_t *d_status, void *stream) {
  if (n_pool_rows < 0) return GPB_EINVAL;
  return gpb::compose_layer(d_dense, nullptr, table, plan, n_slots, n_cur_pages, d_staging,
                            n_staging_rows, d_cur_rows, n_rows, page_rows, row_bytes,
                            d_status, stream, false, d_pool, n_pool_rows, false);
}

extern "C" int gpb_compose_layer_ahead_fill(void *d_dense, void *d_dense_next,
                                            const gpb_sources *table, const gpb_plan *plan,
                                            int32_t n_slots, int32_t n_cur_pages,
                                            void *d_staging, int64_t n_staging_rows,
                                            void *d_pool, int64_t n_pool_rows,
                                            const void *d_cur_rows, int32_t n_rows,
                                            int32_t page_rows, int32_t row_bytes,
                                            int32_t *d_status, void *stream) {
  if (n_pool_rows < 0) return GPB_EINVAL;
  return gpb::compose_layer(d_dense, d_dense_next, table, plan, n_slots, n_cur_pages,
                            d_staging, n_staging_rows, d_cur_rows, n_rows, page_rows,
                            row_bytes, d_status, stream, true, d_pool, n_pool_rows, false);
}

namespace gpb {
namespace {
thread_local char hip_error_text[160] = "HIP launch failed";
}  // namespace

void note_hip_error(hipError_t e) {
  snprintf(hip_error_text, sizeof(hip_error_text), "HIP launch failed: %s (%d)",
           hipGetErrorString(e), static_cast<int>(e));
}
}  // namespace gpb

extern "C" const char *gpb_strerror(int status) {
  switch (status) {
    case GPB_OK: return "ok";
    case GPB_EINVAL: return "invalid argument";
    case GPB_EALIGN: return "misaligned row size or pointer";
    case GPB_EPAGE: return "page id is the dummy page 0, out of range, or repeated";
    case GPB_ECAPACITY: return "staging capacity exceeded (slot 0 plus current pages)";
    case GPB_ERANGE: return "index or size does not fit in int32";
    case GPB_EHIP: return gpb::hip_error_text;
    case GPB_ESCRATCH: return "staging would exceed the library's static scratch array";
    default: return "unknown gpb status";
  }
}
