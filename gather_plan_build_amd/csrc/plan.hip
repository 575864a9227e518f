// plan.hip -- per-batch plan build for the KV compose (gfx950).
//
// Page d63fbd4, commit "current rows written straight into staging": the
// plan carries a staging-remapped page inverse that retargets the fill, and
// mixed_locs and the staging row indices, which no layer changes, come from
// one pass per batch.  Page d63fbd4, commit "cut per-layer CPU on the
// prefill launch path": the ragged int32 descriptors and slot spans come
// from batch metadata only, with no device synchronisation.  Page 0d87bc5, commit
// "prefetch staging exchange": page 0 is the dummy page and the staging slot
// of current page i is i + 1.
//
// Three launches on the caller's stream, each a plain function of the
// previous one's outputs:
//   1. k_plan_scan_fill: workgroup 0 runs wave-level exclusive scans over the
//      per-request counts (slots n, tokens c, current pages C) and writes the
//      spans and ragged descriptors, then the first entry of every writer's
//      scatter list; the next workgroups fill both page inverses with -1 and
//      the rest, when the caller passes a staging region, zero it (the
//      per-batch clear rides in the same launch).
//   2. k_plan_slots: one lane per dense slot -> slot page, page inverse,
//      gather descriptor, writer, staging page inverse, the slot's place in
//      the prefix or current slot list and its gather record, a current
//      page's token range and its first entry in its writer's list.
//   3. k_plan_tokens: one lane per current token -> staging row through the
//      staging page inverse, mixed_locs, the per-token expansions (request
//      row id, top-k offset), the token's pool row and its entry in its
//      writer's list.
// Request lookups in 2 and 3 are binary searches over the scanned bases,
// staged in LDS.  A current page's first entry in its writer's list sums the
// shortfalls of earlier requests' last pages on the same writer: a loop over
// the earlier requests, from LDS, per current page.
#include <algorithm>
#include <vector>

#include "buffer_io.h"
#include "gpb_common.h"

namespace gpb {
namespace {

constexpr int kLdsRequests = 1024;  // requests whose bases fit the LDS stage

struct PlanArgs {
  int32_t bs, ps, np, w, cap, n_pool_pages, n_slots, n_rows, n_cur_pages;
  const int32_t *P, *c, *req_pages;
  int32_t *slot_base, *prefix_span, *current_span;
  int32_t *q_lens, *kv_lens, *q_starts, *k_bases, *q_bases, *current_bases;
  int32_t *slot_pages, *owner, *src, *page_inverse, *staging_page_inverse;
  int32_t *writer, *staging_rows, *mixed_locs;
  int32_t *token_req, *topk_offsets, *segments;
  int32_t *prefix_slots, *current_slots, *pool_locs;
  int32_t *cur_page_token0, *cur_page_ntok;
  int32_t *prefix_desc, *current_desc;
  int32_t *writer_offsets, *writer_tokens, *writer_rows, *writer_page_row0;
  uint8_t *clear;        // staging region zeroed by the fill workgroups
  int64_t clear_bytes;
  int32_t fill_blocks;   // workgroups 1 .. fill_blocks fill the inverses
  int32_t *status;
};

// The kernels index by values read from the device copies of the metadata.
// The host validated its own copies; if the device copies differ, every
// indexed write is still kept inside its array and the fault is reported.
__device__ __forceinline__ bool within(int x, int n) { return x >= 0 && x < n; }
__device__ __forceinline__ void flag_bad_input(const PlanArgs &a) {
  if (a.status) atomicOr(a.status, GPB_STATUS_BAD_PLAN_INPUT);
}

// Inclusive scan across one wave64 (Hillis-Steele over lane shuffles).
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

constexpr int kWriterChunk = 1024;  // writers whose token counts fit the LDS pass

// Tokens of every writer (page d63fbd4, commit "counting barrier + CUDA-IPC
// gather": each current page has one writer; writer of batch page i is
// i mod W) and their exclusive sums, the first entry of each writer's list.
// Writer w holds n_w = ceil((NCP - w) / W) pages; all of them are full
// except the last page of a request, which lacks C_r * PS - c_r tokens and
// belongs to writer (first current page of r + C_r - 1) mod W.  The
// shortfalls are summed per writer in LDS, a chunk of writers at a time.
__device__ void writer_offsets(const PlanArgs &a, int ncp) {
  __shared__ int short_by[kWriterChunk];
  __shared__ int chunk_carry;
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid == 0) chunk_carry = 0;
  for (int w0 = 0; w0 < a.w; w0 += kWriterChunk) {
    for (int k = tid; k < kWriterChunk; k += kBlock) short_by[k] = 0;
    __syncthreads();
    for (int r = tid; r < a.bs; r += kBlock) {
      const int c = a.c[r];
      const int C = (c + a.ps - 1) / a.ps;
      if (C == 0 || C * a.ps == c) continue;
      const int last = a.q_bases[r] / a.ps + C - 1;
      const int w = last % a.w - w0;
      if (w >= 0 && w < kWriterChunk) atomicAdd(&short_by[w], C * a.ps - c);
    }
    __syncthreads();
    // exclusive sum over the chunk's writers, one wave, 64 writers a pass
    if (tid < 64) {
      int carry = chunk_carry;
      const int n = min(kWriterChunk, a.w - w0);
      for (int b = 0; b < n; b += 64) {
        const int w = w0 + b + lane;
        int tok = 0;
        if (b + lane < n) {
          const int pages = ncp > w ? (ncp - 1 - w) / a.w + 1 : 0;
          tok = pages * a.ps - short_by[b + lane];
        }
        const int inc = wave_inclusive_scan(tok, lane);
        if (b + lane < n) a.writer_offsets[w] = carry + inc - tok;
        carry += __shfl(inc, 63, 64);
      }
      if (lane == 0) chunk_carry = carry;
    }
    __syncthreads();
  }
  if (tid == 0) a.writer_offsets[a.w] = chunk_carry;
}

__device__ void scan_requests(const PlanArgs &a) {
  __shared__ int wave_tot[3][kBlock / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry_n = 0, carry_c = 0, carry_C = 0;
  for (int base = 0; base < a.bs; base += kBlock) {
    const int r = base + tid;
    int P = 0, c = 0;
    if (r < a.bs) {
      P = a.P[r];
      c = a.c[r];
    }
    const int C = (c + a.ps - 1) / a.ps;
    const int n = P + C;
    const int in_n = wave_inclusive_scan(n, lane);
    const int in_c = wave_inclusive_scan(c, lane);
    const int in_C = wave_inclusive_scan(C, lane);
    if (lane == 63) {
      wave_tot[0][wave] = in_n;
      wave_tot[1][wave] = in_c;
      wave_tot[2][wave] = in_C;
    }
    __syncthreads();
    int pre_n = carry_n, pre_c = carry_c, pre_C = carry_C;
    int all_n = carry_n, all_c = carry_c, all_C = carry_C;
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) {
      if (w < wave) {
        pre_n += wave_tot[0][w];
        pre_c += wave_tot[1][w];
        pre_C += wave_tot[2][w];
      }
      all_n += wave_tot[0][w];
      all_c += wave_tot[1][w];
      all_C += wave_tot[2][w];
    }
    if (r < a.bs) {
      const int ex_n = pre_n + in_n - n;  // exclusive sums
      const int ex_c = pre_c + in_c - c;
      const int ex_C = pre_C + in_C - C;
      a.slot_base[r] = ex_n;
      a.prefix_span[2 * r] = ex_n;
      a.prefix_span[2 * r + 1] = ex_n + P;
      a.current_span[2 * r] = ex_n + P;
      a.current_span[2 * r + 1] = ex_n + n;
      a.q_lens[r] = c;
      a.kv_lens[r] = a.ps * P + c;
      a.q_starts[r] = ex_c;
      a.k_bases[r] = a.ps * ex_n;
      a.current_bases[r] = a.ps * (ex_n + P);
      a.q_bases[r] = a.ps * ex_C;
      a.segments[4 * r] = ex_c;
      a.segments[4 * r + 1] = c;
      a.segments[4 * r + 2] = a.ps * ex_n;
      a.segments[4 * r + 3] = a.ps * P + c;
    }
    carry_n = all_n;
    carry_c = all_c;
    carry_C = all_C;
    __syncthreads();  // wave_tot is reused by the next tile
  }
  // q_bases written above by this workgroup are read back after the
  // workgroup barrier that opens writer_offsets
  writer_offsets(a, carry_C);
}

constexpr int kClearBytes = kBlock * 16;  // staging bytes per clear workgroup

// Workgroup 0 scans the requests; workgroups 1 .. fill_blocks fill both page
// inverses with -1; the workgroups after them zero the staging region, 4 KiB
// each (the per-batch clear, page d63fbd4, commit "current rows written
// straight into staging": the scatter writes into zeroed staging).  The
// clear's last workgroup gets a buffer range that ends with the region.
__global__ __launch_bounds__(kBlock) void k_plan_scan_fill(PlanArgs a) {
  if (blockIdx.x == 0) {
    scan_requests(a);
    return;
  }
  if (static_cast<int>(blockIdx.x) > a.fill_blocks) {
    const int64_t base = static_cast<int64_t>(blockIdx.x - 1 - a.fill_blocks) * kClearBytes;
    const int64_t left = a.clear_bytes - base;
    const int32_t range = left < kClearBytes ? static_cast<int32_t>(left) : kClearBytes;
    st16(u32x4{0, 0, 0, 0}, rsrc(a.clear + base, range), threadIdx.x * 16u);
    return;
  }
  const int stride = a.fill_blocks * kBlock;
  for (int p = (blockIdx.x - 1) * kBlock + threadIdx.x; p < a.n_pool_pages; p += stride) {
    a.page_inverse[p] = -1;
    a.staging_page_inverse[p] = -1;
  }
}

// Largest r in [0, bs) with base[r] <= x, given base[0] == 0 <= x and base
// non-decreasing.  Requests with no entries share the next request's base and
// are skipped because the search keeps the last equal base.
__device__ __forceinline__ int find_request(const int32_t *base, int bs, int x) {
  int lo = 0, hi = bs;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (base[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Writer of request r's last current page and the tokens that page lacks
// (0 when the page is full or r has no current page), from global memory.
__device__ __forceinline__ void last_page_shortfall(const PlanArgs &a, int r, int *w,
                                                    int *lack) {
  const int c = a.c[r];
  const int C = (c + a.ps - 1) / a.ps;
  *lack = C * a.ps - c;
  *w = C > 0 ? (a.q_bases[r] / a.ps + C - 1) % a.w : -1;
}

__global__ __launch_bounds__(kBlock) void k_plan_slots(PlanArgs a) {
  __shared__ int32_t s_base[kLdsRequests], s_P[kLdsRequests], s_qb[kLdsRequests],
      s_qs[kLdsRequests], s_c[kLdsRequests], s_lw[kLdsRequests], s_lack[kLdsRequests];
  const bool lds = a.bs <= kLdsRequests;
  if (lds) {
    for (int r = threadIdx.x; r < a.bs; r += kBlock) {
      s_base[r] = a.slot_base[r];
      s_P[r] = a.P[r];
      s_qb[r] = a.q_bases[r];
      s_qs[r] = a.q_starts[r];
      s_c[r] = a.c[r];
      last_page_shortfall(a, r, &s_lw[r], &s_lack[r]);
    }
    __syncthreads();
  }
  const int32_t *base = lds ? s_base : a.slot_base;
  const int32_t *Pv = lds ? s_P : a.P;
  const int32_t *qb = lds ? s_qb : a.q_bases;
  const int32_t *qs = lds ? s_qs : a.q_starts;
  const int32_t *cv = lds ? s_c : a.c;
  const int s = blockIdx.x * kBlock + threadIdx.x;
  if (s >= a.n_slots) return;
  const int r = find_request(base, a.bs, s);
  const int j = s - base[r];
  const int P = Pv[r];
  const int page = a.req_pages[s];
  a.slot_pages[s] = page;
  if (!within(page, a.n_pool_pages)) {
    flag_bad_input(a);
    return;
  }
  a.page_inverse[page] = s;
  const int cur_before = qb[r] / a.ps;  // current pages of earlier requests
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  if (j < P) {  // prefix slot: modulo-owned pool entry, the page itself
    const int e = page % a.np;
    a.owner[s] = e;
    a.src[s] = page;
    const int u = s - cur_before;
    if (within(u, a.n_slots - a.n_cur_pages)) {
      a.prefix_slots[u] = s;
      reinterpret_cast<i32x4 *>(a.prefix_desc)[u] = i32x4{s, e, page, 0};
    } else {
      flag_bad_input(a);
    }
  } else {      // current page i of the batch
    const int i = cur_before + (j - P);
    const int w = i % a.w;
    a.owner[s] = a.np + w;
    a.src[s] = i + 1;
    a.staging_page_inverse[page] = w * a.cap + i + 1;
    if (within(i, a.n_cur_pages)) {
      const int k = j - P;  // page k of the request's current pages
      a.writer[i] = w;
      a.current_slots[i] = s;
      a.cur_page_token0[i] = qs[r] + k * a.ps;
      a.cur_page_ntok[i] = min(a.ps, cv[r] - k * a.ps);
      reinterpret_cast<i32x4 *>(a.current_desc)[i] = i32x4{s, a.np + w, i + 1, 0};
      // first entry of page i in writer w's list: the i div W earlier pages
      // of w, all full but for the last pages of earlier requests
      int lack = 0;
      for (int q = 0; q < r; ++q) {
        int lw, lk;
        if (lds) {
          lw = s_lw[q];
          lk = s_lack[q];
        } else {
          last_page_shortfall(a, q, &lw, &lk);
        }
        lack += lw == w ? lk : 0;
      }
      a.writer_page_row0[i] = (i / a.w) * a.ps - lack;
    } else {
      flag_bad_input(a);
    }
  }
}

__global__ __launch_bounds__(kBlock) void k_plan_tokens(PlanArgs a) {
  __shared__ int32_t s_qs[kLdsRequests], s_base[kLdsRequests], s_P[kLdsRequests],
      s_cb[kLdsRequests], s_kb[kLdsRequests], s_qb[kLdsRequests];
  const bool lds = a.bs <= kLdsRequests;
  if (lds) {
    for (int r = threadIdx.x; r < a.bs; r += kBlock) {
      s_qs[r] = a.q_starts[r];
      s_base[r] = a.slot_base[r];
      s_P[r] = a.P[r];
      s_cb[r] = a.current_bases[r];
      s_kb[r] = a.k_bases[r];
      s_qb[r] = a.q_bases[r];
    }
    __syncthreads();
  }
  const int32_t *qs = lds ? s_qs : a.q_starts;
  const int32_t *base = lds ? s_base : a.slot_base;
  const int32_t *Pv = lds ? s_P : a.P;
  const int32_t *cb = lds ? s_cb : a.current_bases;
  const int32_t *kb = lds ? s_kb : a.k_bases;
  const int32_t *qb = lds ? s_qb : a.q_bases;
  const int t = blockIdx.x * kBlock + threadIdx.x;
  if (t >= a.n_rows) return;
  const int r = find_request(qs, a.bs, t);
  const int j = t - qs[r];
  const int s = base[r] + Pv[r] + j / a.ps;
  const int page = within(s, a.n_slots) ? a.slot_pages[s] : -1;
  if (!within(page, a.n_pool_pages)) {
    flag_bad_input(a);
    return;
  }
  const int loc = page * a.ps + j % a.ps;  // the token's pool row
  const int spage = a.staging_page_inverse[loc / a.ps];
  const int row = spage * a.ps + loc % a.ps;
  a.staging_rows[t] = row;
  a.mixed_locs[t] = cb[r] + j;
  a.token_req[t] = r;
  a.topk_offsets[t] = kb[r];
  a.pool_locs[t] = loc;
  // the token's entry in its page writer's scatter list, with its row inside
  // that writer's slab
  const int i = qb[r] / a.ps + j / a.ps;
  const int w = i % a.w;
  const int e = within(i, a.n_cur_pages)
                    ? a.writer_offsets[w] + a.writer_page_row0[i] + j % a.ps : -1;
  if (!within(e, a.n_rows)) {
    flag_bad_input(a);
    return;
  }
  a.writer_tokens[e] = t;
  a.writer_rows[e] = row - w * a.cap * a.ps;
}

// Host-side validation of a batch; the rules and their order match the
// header: shape, then sizes, then staging capacity, then page ids.
int validate_batch(const gpb_batch *b, int32_t *S_out, int32_t *T_out,
                   int32_t *NCP_out) {
  if (!b) return GPB_EINVAL;
  if (b->bs < 0 || b->page_size < 1 || b->n_pool_pages < 1 ||
      b->n_pool_entries < 1 || b->n_writers < 1 || b->staging_cap_pages < 1 ||
      b->row_bytes < 1)
    return GPB_EINVAL;
  if (b->row_bytes % 16 != 0) return GPB_EALIGN;
  if (b->bs > 0 && (!b->h_prefix_pages || !b->h_cur_tokens)) return GPB_EINVAL;
  int64_t S = 0, T = 0, NCP = 0;
  for (int32_t r = 0; r < b->bs; ++r) {
    const int64_t P = b->h_prefix_pages[r], c = b->h_cur_tokens[r];
    if (P < 0 || c < 0) return GPB_EINVAL;
    const int64_t C = ceil_div64(c, b->page_size);
    S += P + C;
    T += c;
    NCP += C;
  }
  if (S * b->page_size > INT32_MAX || T > INT32_MAX ||
      static_cast<int64_t>(b->n_pool_pages) * b->page_size > INT32_MAX ||
      static_cast<int64_t>(b->n_writers) * b->staging_cap_pages * b->page_size > INT32_MAX)
    return GPB_ERANGE;
  if (1 + NCP > b->staging_cap_pages) return GPB_ECAPACITY;
  if (S > 0 && !b->h_req_pages) return GPB_EINVAL;
  std::vector<uint8_t> seen(static_cast<size_t>(b->n_pool_pages), 0);
  for (int64_t k = 0; k < S; ++k) {
    const int32_t p = b->h_req_pages[k];
    if (p < 1 || p >= b->n_pool_pages || seen[p]) return GPB_EPAGE;
    seen[p] = 1;
  }
  if (S_out) *S_out = static_cast<int32_t>(S);
  if (T_out) *T_out = static_cast<int32_t>(T);
  if (NCP_out) *NCP_out = static_cast<int32_t>(NCP);
  return GPB_OK;
}

bool ok_array(const void *p, int64_t n, uintptr_t align = 4) {
  return n == 0 || (p && aligned(p, align));
}

// Host-side counts of the per-writer scatter lists: writer w holds the
// current pages i with i mod W == w, each with its request's tokens on it.
void writer_counts(const gpb_batch *b, int32_t *counts) {
  for (int32_t w = 0; w < b->n_writers; ++w) counts[w] = 0;
  int64_t i = 0;
  for (int32_t r = 0; r < b->bs; ++r) {
    const int64_t c = b->h_cur_tokens[r];
    for (int64_t k = 0; k * b->page_size < c; ++k, ++i)
      counts[i % b->n_writers] +=
          static_cast<int32_t>(std::min<int64_t>(b->page_size, c - k * b->page_size));
  }
}

int plan_build(const gpb_batch *b, const gpb_plan *o, void *d_clear, int64_t clear_bytes,
               void *stream) {
  int32_t S = 0, T = 0, NCP = 0;
  int rc = validate_batch(b, &S, &T, &NCP);
  if (rc != GPB_OK) return rc;
  if (!o) return GPB_EINVAL;
  if (clear_bytes < 0 || (clear_bytes > 0 && !d_clear)) return GPB_EINVAL;
  if (clear_bytes % 16 != 0 || (clear_bytes > 0 && !aligned(d_clear, 16))) return GPB_EALIGN;
  const int64_t bs = b->bs, npp = b->n_pool_pages, W = b->n_writers;
  struct Need { const void *p; int64_t n; uintptr_t align; };
  const Need need[] = {
      {b->d_prefix_pages, bs, 4}, {b->d_cur_tokens, bs, 4}, {b->d_req_pages, S, 4},
      {o->d_slot_base, bs, 4}, {o->d_prefix_span, 2 * bs, 4}, {o->d_current_span, 2 * bs, 4},
      {o->d_q_lens, bs, 4}, {o->d_kv_lens, bs, 4}, {o->d_q_starts, bs, 4},
      {o->d_k_bases, bs, 4}, {o->d_q_bases, bs, 4}, {o->d_current_bases, bs, 4},
      {o->d_slot_pages, S, 4}, {o->d_owner, S, 4}, {o->d_src, S, 4},
      {o->d_page_inverse, npp, 4}, {o->d_staging_page_inverse, npp, 4},
      {o->d_writer, NCP, 4}, {o->d_staging_rows, T, 4}, {o->d_mixed_locs, T, 4},
      {o->d_token_req, T, 4}, {o->d_topk_offsets, T, 4}, {o->d_segments, 4 * bs, 4},
      {o->d_prefix_slots, S - NCP, 4}, {o->d_current_slots, NCP, 4},
      {o->d_pool_locs, T, 4}, {o->d_cur_page_token0, NCP, 4},
      {o->d_cur_page_ntok, NCP, 4}, {o->d_prefix_desc, S - NCP, 16},
      {o->d_current_desc, NCP, 16}, {o->d_writer_offsets, W + 1, 4},
      {o->d_writer_tokens, T, 4}, {o->d_writer_rows, T, 4},
      {o->d_writer_page_row0, NCP, 4}};
  for (const Need &e : need) {
    if (e.n > 0 && !e.p) return GPB_EINVAL;
    if (!ok_array(e.p, e.n, e.align)) return GPB_EALIGN;
  }
  if (o->d_status && !aligned(o->d_status, 4)) return GPB_EALIGN;
  const int64_t fill_blocks = std::min<int64_t>(256, ceil_div64(npp, kBlock * 4));
  const int64_t clear_blocks = ceil_div64(clear_bytes, kClearBytes);
  if (1 + fill_blocks + clear_blocks > INT32_MAX) return GPB_ERANGE;
  PlanArgs a;
  a.bs = b->bs; a.ps = b->page_size; a.np = b->n_pool_entries; a.w = b->n_writers;
  a.cap = b->staging_cap_pages; a.n_pool_pages = b->n_pool_pages;
  a.n_slots = S; a.n_rows = T; a.n_cur_pages = NCP;
  a.P = b->d_prefix_pages; a.c = b->d_cur_tokens; a.req_pages = b->d_req_pages;
  a.slot_base = o->d_slot_base; a.prefix_span = o->d_prefix_span;
  a.current_span = o->d_current_span; a.q_lens = o->d_q_lens; a.kv_lens = o->d_kv_lens;
  a.q_starts = o->d_q_starts; a.k_bases = o->d_k_bases; a.q_bases = o->d_q_bases;
  a.current_bases = o->d_current_bases; a.slot_pages = o->d_slot_pages;
  a.owner = o->d_owner; a.src = o->d_src; a.page_inverse = o->d_page_inverse;
  a.staging_page_inverse = o->d_staging_page_inverse; a.writer = o->d_writer;
  a.staging_rows = o->d_staging_rows; a.mixed_locs = o->d_mixed_locs;
  a.token_req = o->d_token_req; a.topk_offsets = o->d_topk_offsets;
  a.segments = o->d_segments;
  a.prefix_slots = o->d_prefix_slots; a.current_slots = o->d_current_slots;
  a.pool_locs = o->d_pool_locs;
  a.cur_page_token0 = o->d_cur_page_token0; a.cur_page_ntok = o->d_cur_page_ntok;
  a.prefix_desc = o->d_prefix_desc; a.current_desc = o->d_current_desc;
  a.writer_offsets = o->d_writer_offsets; a.writer_tokens = o->d_writer_tokens;
  a.writer_rows = o->d_writer_rows; a.writer_page_row0 = o->d_writer_page_row0;
  a.clear = static_cast<uint8_t *>(d_clear);
  a.clear_bytes = clear_bytes;
  a.fill_blocks = static_cast<int32_t>(fill_blocks);
  a.status = o->d_status;

  hipStream_t st = as_stream(stream);
  rc = launch(k_plan_scan_fill, dim3(static_cast<uint32_t>(1 + fill_blocks + clear_blocks)),
              dim3(kBlock), st, a);
  if (rc == GPB_OK && S > 0)
    rc = launch(k_plan_slots, dim3(ceil_div64(S, kBlock)), dim3(kBlock), st, a);
  if (rc == GPB_OK && T > 0)
    rc = launch(k_plan_tokens, dim3(ceil_div64(T, kBlock)), dim3(kBlock), st, a);
  return rc;
}

}  // namespace
}  // namespace gpb

extern "C" int gpb_plan_sizes(const gpb_batch *batch, int32_t *n_slots,
                              int32_t *n_rows, int32_t *n_cur_pages) {
  return gpb::validate_batch(batch, n_slots, n_rows, n_cur_pages);
}

extern "C" int gpb_plan_build(const gpb_batch *b, const gpb_plan *o, void *stream) {
  return gpb::plan_build(b, o, nullptr, 0, stream);
}

extern "C" int gpb_plan_build_clear(const gpb_batch *b, const gpb_plan *o, void *d_staging,
                                    int64_t staging_bytes, void *stream) {
  return gpb::plan_build(b, o, d_staging, staging_bytes, stream);
}

extern "C" int gpb_writer_counts(const gpb_batch *b, int32_t *h_counts) {
  const int rc = gpb::validate_batch(b, nullptr, nullptr, nullptr);
  if (rc != GPB_OK) return rc;
  if (!h_counts) return GPB_EINVAL;
  gpb::writer_counts(b, h_counts);
  return GPB_OK;
}
