// The unit of the one-launch layer: 1 KiB of one dense page, one wave, for
// the single-format kernel (compose.hip) and the grouped one (groups.hip).
#pragma once

#include "buffer_io.h"
#include "gpb_common.h"

namespace gpb {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kScalarRows = 4;  // staging rows a workgroup may fetch as scalars

// Source arenas of a pointer table, passed by value as the last kernel
// argument: entry e (of n) starts at e[e].base and holds e[e].n_pages whole
// pages.  The count and each entry's two fields sit side by side, so a unit
// reads its entry from one line of the argument segment.
struct ArenaEntry {
  const uint8_t *base;
  int64_t n_pages;
};
template <int N>
struct ArenaTable {
  int32_t n;
  int32_t pad;
  ArenaEntry e[N];
};

// One unit of the layer's scatter and gather (page d63fbd4, commit "current
// rows written straight into staging": the current rows go into cleared
// staging, then every dense slot is gathered from the table of pool entries
// and staging slabs).  The unit serves record k of the current records
// (is_cur: a current page, tokens tok0[k] .. tok0[k] + ntok[k] - 1 on it) or
// of the prefix records, and chunk `part * B + lane` of its page.
//
// A current unit first copies the current-row chunks that fall in its KiB
// of the page into staging (the scatter: token t to staging row rows[t]),
// then reads its KiB back from staging through its gather record and stores
// it into the dense page, as the gather does.  Through a valid plan the
// chunk a lane reads back is the chunk that lane wrote, so the lane's own
// program order orders the read after the write; rows past the page's
// tokens read the zeros the per-batch clear left.  `staging` is deliberately
// not __restrict__: the table's staging entries alias it, and the read-back
// must stay behind the write.  The staging stores and the read-back carry
// the plain cache policy: the store completes in L2 instead of writing
// through to memory, so the read-back does not wait on a trip to memory.  The two-launch path's scatter
// writes through instead, since its reader is another kernel.  A lane that
// wrote a current row's chunk also checks that its read-back addressed that
// chunk (GPB_STATUS_LAYER_MISMATCH otherwise: a table or plan that breaks
// the layout); the unit's status bits are ORed in once, after its stores.
//
// A prefix unit copies its KiB of a pool page into dense_pre; a current unit
// stores into dense.  With SROWS (rows of at least 21 chunks) a unit spans
// at most kScalarRows rows, whose staging rows are fetched once with scalar
// loads.  With FILL a current unit also writes each current-row chunk to the
// token's pool row pool_locs[t] (the fused fill: the KV-cache store and the
// staging fill in one pass), with a 64-bit address since a pool may exceed
// one buffer range; the pool rows of current tokens are never pages the
// gather reads.
template <int B, bool SROWS, bool FILL, typename Table>
__device__ __forceinline__ void layer_unit(
    const Table &tbl, uint8_t *dense, uint8_t *dense_pre, bool is_cur, int k, int part,
    const int32_t *__restrict__ pre_desc, const int32_t *__restrict__ cur_desc,
    const int32_t *__restrict__ tok0, const int32_t *__restrict__ ntok, uint8_t *staging,
    int32_t staging_bytes, int32_t n_staging_rows, const int32_t *__restrict__ rows,
    const uint8_t *__restrict__ cur, int32_t n_rows, int32_t row_chunks, int32_t n_slots,
    int32_t page_bytes, u32x4 *pool, int64_t n_pool_rows,
    const int32_t *__restrict__ pool_locs, int32_t *status) {
  const i32x4 rec = reinterpret_cast<const i32x4 *>(is_cur ? cur_desc : pre_desc)[k];
  const int slot = rec.x, e = rec.y, p = rec.z;
  if (slot < 0 || slot >= n_slots) {
    if (status && part == 0 && threadIdx.x == 0) atomicOr(status, GPB_STATUS_BAD_DESCRIPTOR);
    return;
  }
  const int c = part * B + threadIdx.x;  // 16-byte chunk of the page
  const uint32_t off = static_cast<uint32_t>(c) * 16u;
  int flags = 0;
  const uint8_t *wrote = nullptr;  // staging byte this lane wrote (current rows)
  if (is_cur) {
    const int t0 = tok0[k], nt = ntok[k];
    const int j = c / row_chunks;  // row of the page
    const int oc = c - j * row_chunks;
    const int t = t0 + j;
    const bool live = j < nt && off < static_cast<uint32_t>(page_bytes);
    const bool in_rows = live && t >= 0 && t < n_rows;
    int d;
    if (SROWS) {
      const int j0 = part * B / row_chunks;  // first row of the unit (uniform)
      int srow[kScalarRows];
#pragma unroll
      for (int q = 0; q < kScalarRows; ++q)
        srow[q] = rows[min(max(t0 + j0 + q, 0), n_rows - 1)];
      d = srow[kScalarRows - 1];
#pragma unroll
      for (int q = kScalarRows - 2; q >= 0; --q) d = j - j0 == q ? srow[q] : d;
    } else {
      d = rows[in_rows ? t : 0];
    }
    const bool ok = in_rows && d >= 0 && d < n_staging_rows;
    const __amdgpu_buffer_rsrc_t rc = rsrc(cur, n_rows * row_chunks * 16);
    const __amdgpu_buffer_rsrc_t rst = rsrc(staging, staging_bytes);
    const uint32_t to = static_cast<uint32_t>(d * row_chunks + oc) * 16u;
    const u32x4 v = ld16(rc, in_rows ? static_cast<uint32_t>(t * row_chunks + oc) * 16u
                                     : kDropOffset);
    st16_staged(v, rst, ok ? to : kDropOffset);
    bool bad = live && !ok;
    if (FILL) {
      const int64_t q = pool_locs[in_rows ? t : 0];
      const bool okp = in_rows && q >= 0 && q < n_pool_rows;
      bad |= in_rows && !okp;
      if (okp) __builtin_nontemporal_store(v, pool + q * row_chunks + oc);
    }
    if (bad) flags |= GPB_STATUS_BAD_STAGING_ROW;
    if (ok) wrote = staging + to;
  }
  const bool sentinel = (e < 0) || (p < 0);
  const bool in_table = !sentinel && e < tbl.n && p < tbl.e[e].n_pages;
  const uint8_t *from = in_table ? tbl.e[e].base + static_cast<int64_t>(p) * page_bytes : dense;
  const __amdgpu_buffer_rsrc_t rs = rsrc(from, in_table ? page_bytes : 0);
  const __amdgpu_buffer_rsrc_t rd =
      rsrc((is_cur ? dense : dense_pre) + static_cast<int64_t>(slot) * page_bytes, page_bytes);
  // Pool pages are streamed.  A current page's bytes were just written by
  // this very wave: they are read back through the cache at the address the
  // table gives (from + off), formed from the staging region's own buffer
  // resource, the one the scatter's stores used, whenever the unit's KiB
  // lies inside the staging region (always, under the layout
  // gpb_plan_build assumes); otherwise through the table entry's resource.
  // The test is on the unit's whole KiB, so it is one scalar branch.
  // The bytes read are the same either way.  The resource and offset are
  // chosen before the load, so no temporary shares a register with a load
  // in flight and the read-back does not wait for the staging store.  Against
  // the table entry's resource this measured 83.4 instead of 87.2 us per
  // traced layer on MI355X (the consume launch alone 26.3 instead of 30.6 us),
  // with more of the read-back served by L2.
  __amdgpu_buffer_rsrc_t rb = rs;
  uint32_t ob = off;
  if (is_cur && in_table) {
    // where the unit's KiB of the page starts and ends within the staging
    // region (uniform across the wave)
    const int64_t rel0 = from - staging;
    const int64_t end = rel0 + static_cast<int64_t>(part * B + B) * 16;
    if (rel0 >= 0 && end <= staging_bytes) {
      rb = rsrc(staging, staging_bytes);
      ob = static_cast<uint32_t>(rel0) + off;
    }
  }
  const u32x4 back = is_cur ? ld16_staged(rb, ob) : ld16(rb, ob);
  st16_dense(back, rd, off);
  if (wrote && in_table && from + off != wrote) flags |= GPB_STATUS_LAYER_MISMATCH;
  if (!sentinel && !in_table && part == 0 && threadIdx.x == 0)
    flags |= GPB_STATUS_BAD_DESCRIPTOR;
  if (flags && status) atomicOr(status, flags);
}

}  // namespace gpb
