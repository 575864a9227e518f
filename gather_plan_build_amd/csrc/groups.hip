// groups.hip -- the per-layer scatter and gather for several row formats of
// one plan in one launch each (gfx950).
//
// Page 0d87bc5, commit "prefetch staging exchange": the indexer-key fill is
// pointed at the token plan's staging page inverse, and the index twin of the
// compose runs beside the token-KV compose.  No plan array depends on the
// row size, so every format shares staging_rows, owner and src; each has its
// own staging, current rows, dense buffer, pointer table and row size.
//
// The launch is the single-format kernel's unit grid for each group, laid end
// to end (group-major, each group in address order): a workgroup finds its
// group with at most GPB_MAX_GROUPS - 1 scalar compares.  Short formats (the
// 144-byte indexer rows) then share one launch ramp with the token rows
// instead of paying their own.
#include "buffer_io.h"
#include "gpb_common.h"
#include "layer_unit.h"

namespace gpb {
namespace {

constexpr int kUnitLanes = 64;  // one wave64 per unit, one 16-byte chunk per lane

struct GatherGroupArgs {
  uint8_t *dense;
  ArenaTable<GPB_MAX_GROUP_SOURCES> tbl;
  int32_t page_bytes, parts, unit_begin;
};
struct GatherGroupsArgs {
  GatherGroupArgs g[GPB_MAX_GROUPS];
  int32_t n;
};

struct RowGroupArgs {
  uint8_t *staging;
  const uint8_t *cur;
  int32_t staging_bytes, n_staging_rows, row_chunks, step_rows, step_off, unit_begin;
};
struct RowGroupsArgs {
  RowGroupArgs g[GPB_MAX_GROUPS];
  int32_t n;
};

// A group's table from the caller's (n already checked against the group
// capacity); unused entries stay zero.
int fill_table(const gpb_sources &s, ArenaTable<GPB_MAX_GROUP_SOURCES> *t) {
  for (int e = 0; e < s.n; ++e) {
    if (s.n_pages[e] < 0) return GPB_EINVAL;
    if (s.n_pages[e] > 0 && !s.base[e]) return GPB_EINVAL;
    if (!aligned(s.base[e], 16)) return GPB_EALIGN;
  }
  t->n = s.n;
  t->pad = 0;
  for (int e = 0; e < GPB_MAX_GROUP_SOURCES; ++e)
    t->e[e] = e < s.n ? ArenaEntry{static_cast<const uint8_t *>(s.base[e]), s.n_pages[e]}
                      : ArenaEntry{nullptr, 0};
  return GPB_OK;
}

template <typename Groups>
__device__ __forceinline__ int group_of(const Groups &G, int unit) {
  int gi = 0;
#pragma unroll
  for (int k = 1; k < GPB_MAX_GROUPS; ++k)
    if (k < G.n && unit >= G.g[k].unit_begin) gi = k;
  return gi;
}

// The gather of k_compose_gather, one 1 KiB unit per workgroup, for the
// group the unit falls in.
__global__ __launch_bounds__(kUnitLanes) void k_gather_groups(
    const int32_t *__restrict__ owner, const int32_t *__restrict__ src, int32_t *status,
    GatherGroupsArgs G) {
  const int unit = blockIdx.x;
  const GatherGroupArgs &gr = G.g[group_of(G, unit)];
  const int u = unit - gr.unit_begin;
  const int slot = u / gr.parts;
  const int part = u - slot * gr.parts;
  const int e = owner[slot];
  const int p = src[slot];
  const bool sentinel = (e < 0) || (p < 0);
  const bool in_table = !sentinel && e < gr.tbl.n && p < gr.tbl.e[e].n_pages;
  const uint8_t *from =
      in_table ? gr.tbl.e[e].base + static_cast<int64_t>(p) * gr.page_bytes : gr.dense;
  const __amdgpu_buffer_rsrc_t rs = rsrc(from, in_table ? gr.page_bytes : 0);
  const __amdgpu_buffer_rsrc_t rd =
      rsrc(gr.dense + static_cast<int64_t>(slot) * gr.page_bytes, gr.page_bytes);
  const uint32_t off = (static_cast<uint32_t>(part) * kUnitLanes + threadIdx.x) * 16u;
  st16_dense(ld16(rs, off), rd, off);
  if (!sentinel && !in_table && status && part == 0 && threadIdx.x == 0)
    atomicOr(status, GPB_STATUS_BAD_DESCRIPTOR);
}

// The scatter of k_row_scatter (one chunk per lane) for the group the
// workgroup falls in.
__global__ __launch_bounds__(kUnitLanes) void k_scatter_groups(
    const int32_t *__restrict__ rows, int32_t n_rows, int32_t *status, RowGroupsArgs G) {
  const int unit = blockIdx.x;
  const RowGroupArgs &gr = G.g[group_of(G, unit)];
  const int rc = gr.row_chunks;
  const int g = (unit - gr.unit_begin) * kUnitLanes + threadIdx.x;
  const int row = g / rc;
  const int off = g - row * rc;
  const bool live = row < n_rows;
  const int d = rows[live ? row : n_rows - 1];
  const bool ok = live && d >= 0 && d < gr.n_staging_rows;
  const __amdgpu_buffer_rsrc_t rs = rsrc(gr.cur, n_rows * rc * 16);
  const __amdgpu_buffer_rsrc_t rd = rsrc(gr.staging, gr.staging_bytes);
  const u32x4 v = ld16(rs, static_cast<uint32_t>(row * rc + off) * 16u);
  st16(v, rd, ok ? static_cast<uint32_t>(d * rc + off) * 16u : kDropOffset);
  if (live && !ok && status) atomicOr(status, GPB_STATUS_BAD_STAGING_ROW);
}

// The one-launch layer (layer_unit.h) for every group: first the current
// pages' units of all groups, then their prefix pages' units, each group's
// units consecutive.  The groups share the plan's records, token ranges and
// staging rows; each has its own dense buffer, staging, current rows, table
// and row size.
struct LayerGroupArgs {
  uint8_t *dense, *staging;
  const uint8_t *cur;
  ArenaTable<GPB_MAX_GROUP_SOURCES> tbl;
  int32_t staging_bytes, n_staging_rows, row_chunks, page_bytes, parts;
  int32_t srows;                 // staging rows fetched as scalars
  int32_t cur_begin, pre_begin;  // first unit of the group's current / prefix units
};
struct LayerGroupsArgs {
  LayerGroupArgs g[GPB_MAX_GROUPS];
  int32_t n;
  int32_t n_cur_units;  // units of every group's current pages, which come first
};

__global__ __launch_bounds__(kUnitLanes) void k_layer_groups(
    const int32_t *__restrict__ pre_desc, const int32_t *__restrict__ cur_desc,
    const int32_t *__restrict__ tok0, const int32_t *__restrict__ ntok, int32_t *status,
    int32_t n_slots, int32_t n_rows, const int32_t *__restrict__ rows, LayerGroupsArgs G) {
  const int unit = blockIdx.x;
  const bool is_cur = unit < G.n_cur_units;
  int gi = 0;
#pragma unroll
  for (int k = 1; k < GPB_MAX_GROUPS; ++k)
    if (k < G.n && unit >= (is_cur ? G.g[k].cur_begin : G.g[k].pre_begin)) gi = k;
  const LayerGroupArgs &gr = G.g[gi];
  const int u = unit - (is_cur ? gr.cur_begin : gr.pre_begin);
  const int k = u / gr.parts;
  if (gr.srows)
    layer_unit<kUnitLanes, true, false>(gr.tbl, gr.dense, gr.dense, is_cur, k,
                                        u - k * gr.parts, pre_desc, cur_desc, tok0, ntok,
                                        gr.staging, gr.staging_bytes, gr.n_staging_rows, rows,
                                        gr.cur, n_rows, gr.row_chunks, n_slots, gr.page_bytes,
                                        nullptr, 0, nullptr, status);
  else
    layer_unit<kUnitLanes, false, false>(gr.tbl, gr.dense, gr.dense, is_cur, k,
                                         u - k * gr.parts, pre_desc, cur_desc, tok0, ntok,
                                         gr.staging, gr.staging_bytes, gr.n_staging_rows, rows,
                                         gr.cur, n_rows, gr.row_chunks, n_slots, gr.page_bytes,
                                         nullptr, 0, nullptr, status);
}

}  // namespace
}  // namespace gpb

extern "C" int gpb_compose_layer_groups(const gpb_layer_group *groups, int32_t n_groups,
                                        const gpb_plan *plan, int32_t n_slots,
                                        int32_t n_cur_pages, int32_t n_rows, int32_t page_rows,
                                        int32_t *d_status, void *stream) {
  using namespace gpb;
  if (!groups || !plan || n_groups < 1 || n_groups > GPB_MAX_GROUPS || n_slots < 0 ||
      page_rows < 1 || n_cur_pages < 0 || n_cur_pages > n_slots || n_rows < 0 ||
      n_cur_pages > n_rows)
    return GPB_EINVAL;
  if (d_status && !aligned(d_status, 4)) return GPB_EALIGN;
  const int32_t n_prefix = n_slots - n_cur_pages;
  LayerGroupsArgs G;
  G.n = n_groups;
  for (int k = 0; k < GPB_MAX_GROUPS; ++k) G.g[k] = LayerGroupArgs{};
  int64_t units = 0;
  // first pass: each group's geometry and its current units; second: prefix
  for (int k = 0; k < n_groups; ++k) {
    const gpb_layer_group &q = groups[k];
    if (!q.table || q.table->n < 1 || q.table->n > GPB_MAX_GROUP_SOURCES || q.row_bytes < 1 ||
        q.n_staging_rows < 0)
      return GPB_EINVAL;
    if (q.row_bytes % 16 != 0) return GPB_EALIGN;
    if (q.n_staging_rows > INT32_MAX) return GPB_ERANGE;
    const int64_t page_bytes = static_cast<int64_t>(page_rows) * q.row_bytes;
    if (page_bytes > INT32_MAX - (1 << 20)) return GPB_ERANGE;
    LayerGroupArgs &a = G.g[k];
    if (int rc = fill_table(*q.table, &a.tbl)) return rc;
    const int64_t row_chunks = q.row_bytes / 16;
    const int64_t cur_bytes = static_cast<int64_t>(n_rows) * q.row_bytes;
    const int64_t staging_bytes = q.n_staging_rows * q.row_bytes;
    if (cur_bytes > INT32_MAX || staging_bytes > INT32_MAX) return GPB_ERANGE;
    if (n_slots == 0) continue;
    if (!q.d_dense || (n_cur_pages > 0 && (!q.d_staging || !q.d_cur_rows))) return GPB_EINVAL;
    if (!aligned(q.d_dense, 16) || !aligned(q.d_staging, 16) || !aligned(q.d_cur_rows, 16))
      return GPB_EALIGN;
    a.dense = static_cast<uint8_t *>(q.d_dense);
    a.staging = static_cast<uint8_t *>(q.d_staging);
    a.cur = static_cast<const uint8_t *>(q.d_cur_rows);
    a.staging_bytes = static_cast<int32_t>(staging_bytes);
    a.n_staging_rows = static_cast<int32_t>(q.n_staging_rows);
    a.row_chunks = static_cast<int32_t>(row_chunks);
    a.page_bytes = static_cast<int32_t>(page_bytes);
    a.parts = static_cast<int32_t>(ceil_div64(page_bytes / 16, kUnitLanes));
    // a unit of kUnitLanes chunks touches at most 2 + (kUnitLanes - 2) / row_chunks rows
    a.srows = 2 + (kUnitLanes - 2) / row_chunks <= kScalarRows;
    a.cur_begin = static_cast<int32_t>(units);
    units += static_cast<int64_t>(a.parts) * n_cur_pages;
    if (units > INT32_MAX) return GPB_ERANGE;
  }
  if (n_slots == 0) return GPB_OK;
  G.n_cur_units = static_cast<int32_t>(units);
  for (int k = 0; k < n_groups; ++k) {
    G.g[k].pre_begin = static_cast<int32_t>(units);
    units += static_cast<int64_t>(G.g[k].parts) * n_prefix;
    if (units > INT32_MAX) return GPB_ERANGE;
  }
  if ((n_prefix > 0 && !plan->d_prefix_desc) ||
      (n_cur_pages > 0 && (!plan->d_current_desc || !plan->d_cur_page_token0 ||
                           !plan->d_cur_page_ntok || !plan->d_staging_rows)))
    return GPB_EINVAL;
  if (!aligned(plan->d_prefix_desc, 16) || !aligned(plan->d_current_desc, 16) ||
      !aligned(plan->d_cur_page_token0, 4) || !aligned(plan->d_cur_page_ntok, 4) ||
      !aligned(plan->d_staging_rows, 4))
    return GPB_EALIGN;
  if (units == 0) return GPB_OK;
  return launch(k_layer_groups, dim3(static_cast<uint32_t>(units)), dim3(kUnitLanes),
                as_stream(stream), plan->d_prefix_desc, plan->d_current_desc,
                plan->d_cur_page_token0, plan->d_cur_page_ntok, d_status, n_slots, n_rows,
                plan->d_staging_rows, G);
}

extern "C" int gpb_current_row_scatter_groups(const gpb_row_group *groups, int32_t n_groups,
                                              const int32_t *d_staging_rows, int32_t n_rows,
                                              int32_t *d_status, void *stream) {
  using namespace gpb;
  if (!groups || n_groups < 1 || n_groups > GPB_MAX_GROUPS || n_rows < 0) return GPB_EINVAL;
  if (d_status && !aligned(d_status, 4)) return GPB_EALIGN;
  RowGroupsArgs G;
  G.n = n_groups;
  int64_t units = 0;
  for (int k = 0; k < GPB_MAX_GROUPS; ++k) G.g[k] = RowGroupArgs{};
  for (int k = 0; k < n_groups; ++k) {
    const gpb_row_group &q = groups[k];
    if (q.n_staging_rows < 0 || q.row_bytes < 1) return GPB_EINVAL;
    if (q.n_staging_rows > INT32_MAX) return GPB_ERANGE;
    if (q.row_bytes % 16 != 0) return GPB_EALIGN;
    if (n_rows == 0) continue;
    if (!q.d_staging || !q.d_cur_rows) return GPB_EINVAL;
    if (!aligned(q.d_staging, 16) || !aligned(q.d_cur_rows, 16)) return GPB_EALIGN;
    const int64_t rc = q.row_bytes / 16;
    const int64_t cur_bytes = static_cast<int64_t>(n_rows) * q.row_bytes;
    const int64_t staging_bytes = q.n_staging_rows * q.row_bytes;
    if (cur_bytes > INT32_MAX || staging_bytes > INT32_MAX) return GPB_ERANGE;
    RowGroupArgs &a = G.g[k];
    a.staging = static_cast<uint8_t *>(q.d_staging);
    a.cur = static_cast<const uint8_t *>(q.d_cur_rows);
    a.staging_bytes = static_cast<int32_t>(staging_bytes);
    a.n_staging_rows = static_cast<int32_t>(q.n_staging_rows);
    a.row_chunks = static_cast<int32_t>(rc);
    a.unit_begin = static_cast<int32_t>(units);
    units += ceil_div64(static_cast<int64_t>(n_rows) * rc, kUnitLanes);
    if (units > INT32_MAX) return GPB_ERANGE;
  }
  if (n_rows == 0) return GPB_OK;
  if (!d_staging_rows) return GPB_EINVAL;
  if (!aligned(d_staging_rows, 4)) return GPB_EALIGN;
  return launch(k_scatter_groups, dim3(static_cast<uint32_t>(units)), dim3(kUnitLanes),
                as_stream(stream), d_staging_rows, n_rows, d_status, G);
}

extern "C" int gpb_compose_gather_groups(const gpb_gather_group *groups, int32_t n_groups,
                                         const int32_t *d_owner, const int32_t *d_src,
                                         int32_t n_slots, int32_t page_rows,
                                         int32_t *d_status, void *stream) {
  using namespace gpb;
  if (!groups || n_groups < 1 || n_groups > GPB_MAX_GROUPS || n_slots < 0 || page_rows < 1)
    return GPB_EINVAL;
  if (d_status && !aligned(d_status, 4)) return GPB_EALIGN;
  GatherGroupsArgs G;
  G.n = n_groups;
  int64_t units = 0;
  for (int k = 0; k < GPB_MAX_GROUPS; ++k) G.g[k] = GatherGroupArgs{};
  for (int k = 0; k < n_groups; ++k) {
    const gpb_gather_group &q = groups[k];
    if (!q.table || q.table->n < 1 || q.table->n > GPB_MAX_GROUP_SOURCES || q.row_bytes < 1)
      return GPB_EINVAL;
    if (q.row_bytes % 16 != 0) return GPB_EALIGN;
    const int64_t page_bytes = static_cast<int64_t>(page_rows) * q.row_bytes;
    if (page_bytes > INT32_MAX - (1 << 20)) return GPB_ERANGE;
    GatherGroupArgs &a = G.g[k];
    if (int rc = fill_table(*q.table, &a.tbl)) return rc;
    if (n_slots == 0) continue;
    if (!q.d_dense) return GPB_EINVAL;
    if (!aligned(q.d_dense, 16)) return GPB_EALIGN;
    a.dense = static_cast<uint8_t *>(q.d_dense);
    a.page_bytes = static_cast<int32_t>(page_bytes);
    a.parts = static_cast<int32_t>(ceil_div64(page_bytes / 16, kUnitLanes));
    a.unit_begin = static_cast<int32_t>(units);
    units += static_cast<int64_t>(a.parts) * n_slots;
    if (units > INT32_MAX) return GPB_ERANGE;
  }
  if (n_slots == 0) return GPB_OK;
  if (!d_owner || !d_src) return GPB_EINVAL;
  if (!aligned(d_owner, 4) || !aligned(d_src, 4)) return GPB_EALIGN;
  return launch(k_gather_groups, dim3(static_cast<uint32_t>(units)), dim3(kUnitLanes),
                as_stream(stream), d_owner, d_src, d_status, G);
}
