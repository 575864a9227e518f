/*
 * gpb.h -- C ABI of libgpb.so: the KV-compose hot path on one MI355X (gfx950).
 *
 * Per batch, gpb_plan_build turns host batch metadata into the layer-invariant
 * plan: slot spans, the page inverse and its staging-remapped twin, gather
 * descriptors (owner, src), per-token staging rows and mixed_locs, and the
 * ragged int32 descriptors (gpb_plan_build_clear also zeroes the staging
 * region in the same launches).  Per layer, gpb_current_row_scatter writes
 * the current token rows into staging cleared once per batch, gpb_compose_gather
 * fills the slot-dense KV buffer one page per slot from a pointer table of
 * source arenas [pool entries || staging slabs]; gpb_compose_layer does both
 * in one launch.  The layer-ahead split gathers a layer's prefix pages
 * early (gpb_compose_gather_records) and its current pages at consume time
 * (gpb_compose_consume), or layer l's consume together with layer l + 1's
 * prefix pages (gpb_compose_layer_ahead); the _fill variants also store the
 * current rows in the KV cache.
 *
 * Where the method comes from (commit pages of the sglang fork, cited by the
 * page's commit hash and the commit's subject):
 *   page d63fbd4, commit "current rows written straight into staging": the
 *     fill kernels find their destinations through a page inverse, so one
 *     extra inverse built per batch points them at staging instead of the
 *     pool; each layer's fill is then a single index_copy_ of the current
 *     rows into staging that was zeroed beforehand; a single gather then
 *     fills every dense slot from a table that lists the pool arenas first
 *     and the staging slabs after them (a current slot's owner is the number
 *     of pool entries plus its writer, its src is its staging slot).
 *     mixed_locs and the staging row of every current token do not change
 *     from layer to layer, so they are computed once per batch.
 *   page d63fbd4, commit "touched-pages-proportional staging": staging is
 *     sized for the current pages of one batch only; current page i of the
 *     batch (requests in batch order, pages in sequence order) owns the same
 *     staging slot on every rank; running out of staging is an error.
 *   page d63fbd4, commit "compose_v2": an owner or src of -1 means a page of
 *     zeros.
 *   page d63fbd4, commit "cut per-layer CPU on the prefill launch path": the
 *     slot spans and the int32 ragged descriptors (kv_lens, q_starts, q_lens,
 *     k_bases, q_bases, current_bases) come from the batch metadata once per
 *     batch, with no wait on the device.
 *   page 0d87bc5, commit "prefetch staging exchange": pool page 0 is a dummy;
 *     staging slot 0 is left unused, so current page i sits in slot i + 1.
 *   page 0d87bc5, commit "canonical prefix/current slot spans": the spans
 *     alone describe where each request's prefix and current pages sit; an
 *     empty span is fine, a missing one is an error.
 *   page 0d87bc5, commit "fp8 index_copy_ -> uint8 views": a row is moved as
 *     raw bytes, whatever element type it holds.
 *
 * How this ABI differs from the plainest signature of the three calls
 * (plan_build; a scatter taking staging, rows, current rows and a count; a
 * gather taking a device array of source pointers and its length):
 *   - gpb_compose_gather takes its pointer table as a host struct
 *     (gpb_sources, at most GPB_MAX_SOURCES = 64 entries) that the library
 *     copies into the kernel arguments, not a device array of pointers: a
 *     workgroup then reads its slot's arena base and page count from the
 *     argument segment with scalar loads, and no device table has to be
 *     built or kept coherent with the arenas.  The table also carries each
 *     arena's size in pages, so a descriptor outside its arena is caught;
 *   - gpb_current_row_scatter takes the staging region's size in rows
 *     (n_staging_rows), so a row index outside it is skipped, not written;
 *   - every per-layer call takes an optional device status word (d_status)
 *     that kernels OR GPB_STATUS_* bits into, since a kernel cannot return
 *     an error code;
 *   - gpb_batch carries device copies of the three metadata arrays beside
 *     the host copies: the host validates its copy, the kernels read theirs,
 *     and nothing is copied or synchronised inside the call.
 *
 * Conventions for every call:
 *   - Returns GPB_OK (0) or a negative gpb_status.  Arguments are checked on
 *     the host before anything is launched; a rejected call launches nothing
 *     and leaves every output untouched.
 *   - d_* pointers are device memory owned by the caller (for instance torch
 *     tensors); h_* pointers are host memory read during the call only.  The
 *     library allocates no device memory and never synchronises: every launch
 *     is asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 *     (gpb_compose_layer_noalloc works in a static array of the library's
 *     own, described with it.)
 *     Order between calls is stream order; the caller keeps buffers alive
 *     until the work is done.
 *   - Row payloads are opaque bytes; row_bytes is a multiple of 16 and every
 *     row-carrying pointer is 16-byte aligned.  Index arrays are int32 and
 *     4-byte aligned; byte offsets are computed in 64 bits.
 *   - Empty work (bs = 0, no slots, no rows) is valid and launches nothing
 *     beyond what is needed to fill outputs that are not empty.
 */
#ifndef GPB_H
#define GPB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gpb_status {
  GPB_OK = 0,
  GPB_EINVAL = -1,     /* null pointer where data is needed, negative size,
                          geometry out of range, table with no entries      */
  GPB_EALIGN = -2,     /* row_bytes % 16 != 0, or a pointer misaligned       */
  GPB_EPAGE = -3,      /* a page id is 0 (dummy), >= n_pool_pages, or repeated
                          within the batch                                   */
  GPB_ECAPACITY = -4,  /* 1 + current pages > staging_cap_pages              */
  GPB_ERANGE = -5,     /* a row or element index would not fit in int32     */
  GPB_EHIP = -6,       /* the HIP runtime refused a launch                   */
  GPB_ESCRATCH = -7    /* gpb_compose_layer_noalloc: the staging region would
                          exceed GPB_SCRATCH_BYTES                           */
} gpb_status;

/* Bits the kernels OR into the optional device status word (int32). */
#define GPB_STATUS_BAD_DESCRIPTOR 1  /* gather: owner >= table entries or src
                                        >= that arena's pages; slot zeroed  */
#define GPB_STATUS_BAD_STAGING_ROW 2 /* scatter: staging row < 0 or beyond
                                        the staging region; row skipped      */
#define GPB_STATUS_BAD_PLAN_INPUT 4  /* plan: the device metadata differs from
                                        the validated host copy (a page id or
                                        index out of range); the entry is not
                                        written                              */
#define GPB_STATUS_LAYER_MISMATCH 8  /* one-launch layer: a current row's
                                        staging row is not where its page's
                                        descriptor reads the page back (a
                                        table whose staging entries are not
                                        the slabs of d_staging, or a plan of
                                        another batch); that page's dense
                                        bytes are not reliable               */

#define GPB_MAX_SOURCES 64           /* pointer-table entries per gather    */

/* Batch metadata for gpb_plan_build (page d63fbd4, commits "current rows
 * written straight into staging" and "cut per-layer CPU on the prefill launch
 * path").  Request r has prefix_pages[r] whole prefix pages (prefix lengths
 * are page-aligned) and cur_tokens[r] current tokens, which occupy
 * ceil(cur_tokens[r] / page_size) current pages.  req_pages lists, request by
 * request, the pool page ids of its prefix pages then of its current pages;
 * its length is sum over r of prefix_pages[r] + ceil(cur_tokens[r]/page_size).
 * Every id is in [1, n_pool_pages) and distinct.  The host arrays are
 * validated; the device arrays must hold the same values (the kernels read
 * them, the host never reads device memory). */
typedef struct gpb_batch {
  int32_t bs;                   /* requests, >= 0                              */
  int32_t page_size;            /* token rows per page, >= 1 (64)             */
  int32_t row_bytes;            /* bytes per token row, multiple of 16        */
  int32_t n_pool_pages;         /* pages per pool arena; page 0 = dummy       */
  int32_t n_pool_entries;       /* NP: pool entries in the pointer table, >= 1 */
  int32_t n_writers;            /* W: staging slabs, >= 1                     */
  int32_t staging_cap_pages;    /* CAP: pages per slab, slot 0 included       */
  const int32_t *h_prefix_pages;   /* host   [bs]                             */
  const int32_t *h_cur_tokens;     /* host   [bs]                             */
  const int32_t *h_req_pages;      /* host   [n_slots]                        */
  const int32_t *d_prefix_pages;   /* device [bs], same values                */
  const int32_t *d_cur_tokens;     /* device [bs], same values                */
  const int32_t *d_req_pages;      /* device [n_slots], same values           */
} gpb_batch;

/* Caller-allocated plan outputs (int32, device).  Sizes from gpb_plan_sizes:
 * S = n_slots, T = n_rows, NCP = n_cur_pages.  A pointer may be NULL only
 * when its size is 0.  Definitions, for request r (C_r current pages,
 * n_r = P_r + C_r slots; "exclusive sum" = sum over earlier requests):
 *   slot_base[r]          exclusive sum of n                          [bs]
 *   prefix_span[2r..2r+1] [slot_base, slot_base + P_r)                [2bs]
 *   current_span[2r..]    [slot_base + P_r, slot_base + n_r)          [2bs]
 *   q_lens[r]             c_r                                         [bs]
 *   kv_lens[r]            page_size * P_r + c_r                       [bs]
 *   q_starts[r]           exclusive sum of c (token-packed base)      [bs]
 *   k_bases[r]            page_size * slot_base[r] (dense row base)   [bs]
 *   current_bases[r]      k_bases[r] + page_size * P_r                [bs]
 *   q_bases[r]            page_size * exclusive sum of C (page-padded
 *                         current base)                               [bs]
 *   slot_pages[s]         pool page held by dense slot s              [S]
 *   owner[s], src[s]      gather descriptor: prefix slot -> pool entry
 *                         (page mod NP), page; current page i (batch
 *                         order) -> entry NP + writer(i), slot i + 1  [S]
 *   page_inverse[p]       dense slot of pool page p, else -1   [n_pool_pages]
 *   staging_page_inverse[p] carved staging page of current page p:
 *                         writer*CAP + i + 1, else -1          [n_pool_pages]
 *   writer[i]             i mod W (page-aligned round robin)          [NCP]
 *   staging_rows[t]       staging row of current token t, found through
 *                         staging_page_inverse                        [T]
 *   mixed_locs[t]         dense row of current token t                [T]
 * Per-token ragged expansions (page d63fbd4, commit "cut per-layer CPU on the
 * prefill launch path": the O(total-q-tokens) top-k offset list and segment
 * records of the ragged index plan; page 0d87bc5, commit "flattened request
 * row ids": the row ids come from the plan, computed a single time for the
 * batch, where a repeat_interleave per layer made them before):
 *   token_req[t]          request of current token t (flattened row id)  [T]
 *   topk_offsets[t]       k_bases of that request: a request-relative KV
 *                         position plus this offset is a dense row       [T]
 *   segments[4r..4r+3]    (q_starts, q_lens, k_bases, kv_lens) of r     [4bs]
 * Layer-ahead prefetch split (page 0d87bc5, commit "prefetch staging
 * exchange": the prefix of the dense buffer is filled a layer ahead, the
 * consume step fills current rows into staging and gathers all current
 * pages from it):
 *   prefix_slots[u]       dense slots of prefix pages, ascending  [S - NCP]
 *   current_slots[i]      dense slot of current page i            [NCP]
 *   pool_locs[t]          pool row (KV-cache location) of current token t:
 *                         slot_pages[its slot] * page_size + j mod page_size
 *                                                                       [T]
 *   cur_page_token0[i]    first current token held by current page i   [NCP]
 *   cur_page_ntok[i]      current tokens it holds (1..page_size)       [NCP]
 *   prefix_desc[4u..4u+3] gather record of prefix_slots[u]: (slot, owner,
 *                         src, 0); 16-byte aligned           [4 * (S - NCP)]
 *   current_desc[4i..]    gather record of current_slots[i]   [4 * NCP]
 * Per-writer scatter lists (page d63fbd4, commit "counting barrier +
 * CUDA-IPC gather": one writer per current page, writers fixed per batch;
 * page 0d87bc5, commit "prefetch staging exchange": each rank fills its own
 * current rows into its own staging).  List w holds, in token order, the
 * tokens on the current pages of writer w; the lists are stored one after
 * another:
 *   writer_offsets[w]     first entry of list w; [W] = T               [W+1]
 *   writer_tokens[k]      batch token of entry k                        [T]
 *   writer_rows[k]        its staging row inside slab w: the batch
 *                         staging row less w * CAP * page_size          [T]
 *   writer_page_row0[i]   entry of current page i's first token within
 *                         its writer's list                           [NCP]
 * A writer holding the rows of its list's tokens, in list order, fills its
 * own slab with gpb_current_row_scatter(slab, CAP * page_size,
 * writer_rows + writer_offsets[w], rows, count, ...). */
typedef struct gpb_plan {
  int32_t *d_slot_base, *d_prefix_span, *d_current_span;
  int32_t *d_q_lens, *d_kv_lens, *d_q_starts;
  int32_t *d_k_bases, *d_q_bases, *d_current_bases;
  int32_t *d_slot_pages, *d_owner, *d_src;
  int32_t *d_page_inverse, *d_staging_page_inverse;
  int32_t *d_writer;
  int32_t *d_staging_rows, *d_mixed_locs;
  int32_t *d_token_req, *d_topk_offsets, *d_segments;
  int32_t *d_prefix_slots, *d_current_slots, *d_pool_locs;
  int32_t *d_cur_page_token0, *d_cur_page_ntok;
  int32_t *d_prefix_desc, *d_current_desc;
  int32_t *d_writer_offsets, *d_writer_tokens, *d_writer_rows, *d_writer_page_row0;
  int32_t *d_status;  /* optional (NULL): GPB_STATUS_* bits the kernels OR in */
} gpb_plan;

/* Pointer table of source arenas for one gather (page d63fbd4, commit
 * "current rows written straight into staging": [pool entries || staging
 * entries]).  Host struct; the library passes it to the kernel by value.
 * base[e] is the device address of arena e (16-byte aligned), n_pages[e] the
 * number of whole pages addressable from it.  On one GPU every pool entry is
 * the layer's pool arena; staging entry w is slab w of the carved staging
 * region, at d_staging + w * CAP * page_size * row_bytes. */
typedef struct gpb_sources {
  int32_t n;                                /* 1 .. GPB_MAX_SOURCES */
  const void *base[GPB_MAX_SOURCES];
  int64_t n_pages[GPB_MAX_SOURCES];
} gpb_sources;

/* Host only: validate the batch (every rule of gpb_plan_build) and return
 * S (dense slots), T (current rows) and NCP (current pages).  Any of the
 * output pointers may be NULL.  Reads only the h_* arrays. */
int gpb_plan_sizes(const gpb_batch *batch, int32_t *n_slots, int32_t *n_rows,
                   int32_t *n_cur_pages);

/* Validate on the host, then launch the plan kernels on `stream`: a scan
 * kernel (wave-level exclusive scans of the per-request counts and the
 * writer list offsets; its other workgroups fill both page inverses with
 * -1), a per-slot kernel (slot pages, page inverse, descriptors, records,
 * writers, staging inverse) and a per-token kernel (staging rows through the
 * staging inverse, mixed_locs, writer lists).  The plan is layer-invariant:
 * build it once per batch.  Errors: GPB_EINVAL, GPB_EPAGE, GPB_ECAPACITY,
 * GPB_ERANGE (S*page_size, T, n_pool_pages*page_size or W*CAP*page_size
 * beyond INT32_MAX), GPB_EALIGN (int32 arrays not 4-byte aligned, the two
 * record arrays not 16-byte aligned), GPB_EHIP. */
int gpb_plan_build(const gpb_batch *batch, const gpb_plan *plan, void *stream);

/* gpb_plan_build plus the per-batch staging clear in the same three launches:
 * the first launch's spare workgroups also zero staging_bytes bytes at
 * d_staging (the whole staging region, both parity halves if the caller
 * keeps two), which gpb_staging_clear would otherwise do in a launch of its
 * own.  staging_bytes = 0 clears nothing.  Errors as gpb_plan_build, plus
 * GPB_EINVAL (staging_bytes < 0, or d_staging NULL with staging_bytes > 0)
 * and GPB_EALIGN (staging_bytes % 16 != 0 or d_staging not 16-byte
 * aligned). */
int gpb_plan_build_clear(const gpb_batch *batch, const gpb_plan *plan, void *d_staging,
                         int64_t staging_bytes, void *stream);

/* Host only: validate the batch and write, for every writer w < n_writers,
 * the number of entries of its scatter list (tokens on the current pages
 * i with i mod n_writers == w) to h_counts[w].  These are the sizes of the
 * per-writer scatters; they equal the differences of the plan's
 * writer_offsets, without reading device memory.  Errors as gpb_plan_sizes,
 * plus GPB_EINVAL for h_counts NULL. */
int gpb_writer_counts(const gpb_batch *batch, int32_t *h_counts);

/* Zero `n_bytes` bytes at d_ptr (n_bytes a multiple of 16, d_ptr 16-byte
 * aligned): the per-batch clear of the staging region, so the rows of a last
 * current page past its request's tokens read back as zero (page d63fbd4,
 * commit "current rows written straight into staging": the rows land in
 * staging that holds zeros wherever no row is written).  The staging rows a batch writes are the same in
 * every layer, so one clear per batch serves all its layers.  A kernel, not a
 * memset node, so the call can be captured in a HIP graph.  Errors:
 * GPB_EINVAL (n_bytes < 0, or d_ptr NULL with n_bytes > 0), GPB_EALIGN,
 * GPB_ERANGE (more than 2^31 workgroups of 4 KiB), GPB_EHIP. */
int gpb_staging_clear(void *d_ptr, int64_t n_bytes, void *stream);

/* Per layer: staging row d_staging_rows[t] <- current row t, for t < n_rows,
 * whole rows of row_bytes bytes (index_copy_ semantics on byte views: page
 * d63fbd4, commit "current rows written straight into staging"; page
 * 0d87bc5, commit "fp8 index_copy_ -> uint8 views").  d_cur_rows holds n_rows
 * contiguous rows; d_staging holds n_staging_rows rows.  A staging row
 * outside [0, n_staging_rows) is skipped and GPB_STATUS_BAD_STAGING_ROW is
 * ORed into *d_status when d_status is not NULL (page 0d87bc5: index_copy_
 * cannot leave out an index of -1, so a valid plan holds none).
 * Rows must not repeat (the plan's rows are distinct), and the staging region
 * must not overlap the current rows.  Errors: GPB_EINVAL (negative sizes,
 * row_bytes < 1, a NULL pointer with n_rows > 0), GPB_EALIGN, GPB_ERANGE (the
 * current rows or the staging region reach 2 GiB: each is one 32-bit buffer
 * range), GPB_EHIP. */
int gpb_current_row_scatter(void *d_staging, int64_t n_staging_rows,
                            const int32_t *d_staging_rows,
                            const void *d_cur_rows, int32_t n_rows,
                            int32_t row_bytes, int32_t *d_status,
                            void *stream);

/* Per layer: for every slot s < n_slots, dense page s (page_rows * row_bytes
 * bytes at d_dense + s * page_rows * row_bytes) <- page d_src[s] of arena
 * table->base[d_owner[s]]; a slot with d_owner[s] < 0 or d_src[s] < 0 is
 * zero-filled (page d63fbd4, commit "compose_v2").  A descriptor with owner
 * >= table->n or src >= table->n_pages[owner] is zero-filled as well and
 * GPB_STATUS_BAD_DESCRIPTOR is ORed into *d_status when d_status is not NULL.
 * The dense buffer must not overlap any source page it reads.  Errors:
 * GPB_EINVAL (table NULL, table->n outside 1..GPB_MAX_SOURCES, a negative
 * n_pages, a NULL base with pages, n_slots < 0, page_rows < 1, a NULL
 * pointer with n_slots > 0), GPB_EALIGN, GPB_ERANGE (a page of 2 GiB - 1 MiB
 * or more: each page is one 32-bit buffer range), GPB_EHIP. */
int gpb_compose_gather(void *d_dense, const gpb_sources *table,
                       const int32_t *d_owner, const int32_t *d_src,
                       int32_t n_slots, int32_t page_rows, int32_t row_bytes,
                       int32_t *d_status, void *stream);

/* Per layer, the two halves of the layer-ahead prefetch split: as
 * gpb_compose_gather, but only for the n_list dense slots d_slots[k] (for
 * instance the plan's prefix_slots a layer ahead, then its current_slots
 * after the scatter); other slots of d_dense are not touched.  n_slots is the
 * number of slots d_dense, d_owner and d_src hold: a listed slot outside
 * [0, n_slots) is skipped and GPB_STATUS_BAD_DESCRIPTOR is ORed into
 * *d_status.  A slot must not be listed twice.  Errors as gpb_compose_gather,
 * plus GPB_EINVAL for n_list < 0. */
int gpb_compose_gather_slots(void *d_dense, const gpb_sources *table,
                             const int32_t *d_slots, int32_t n_list,
                             const int32_t *d_owner, const int32_t *d_src,
                             int32_t n_slots, int32_t page_rows, int32_t row_bytes,
                             int32_t *d_status, void *stream);

/* Per layer, the fused current fill: each current row t goes, in one pass
 * over the rows, to staging row d_staging_rows[t] (the scatter above) and to
 * pool row d_pool_locs[t] of d_pool (its KV-cache location), whole rows of
 * row_bytes.  A destination outside [0, n_staging_rows) or [0, n_pool_rows)
 * is skipped there and GPB_STATUS_BAD_STAGING_ROW is ORed into *d_status.
 * The staging region is below 2 GiB; the pool may be any size.  Errors as
 * gpb_current_row_scatter, plus GPB_EINVAL for n_pool_rows < 0 or a NULL pool
 * or pool_locs with n_rows > 0. */
int gpb_current_row_fill(void *d_staging, int64_t n_staging_rows,
                         const int32_t *d_staging_rows, void *d_pool,
                         int64_t n_pool_rows, const int32_t *d_pool_locs,
                         const void *d_cur_rows, int32_t n_rows, int32_t row_bytes,
                         int32_t *d_status, void *stream);

/* Per layer, the layer-ahead split's halves through the plan's records: as
 * gpb_compose_gather_slots, but record k (four int32: slot, owner, src, 0;
 * the plan's prefix_desc or current_desc, 16-byte aligned) names both the
 * dense slot and its page, so a workgroup reads one 16-byte record instead
 * of a slot and then that slot's descriptor.  A record whose slot is outside
 * [0, n_slots) is skipped and GPB_STATUS_BAD_DESCRIPTOR is ORed into
 * *d_status.  Errors as gpb_compose_gather_slots. */
int gpb_compose_gather_records(void *d_dense, const gpb_sources *table,
                               const int32_t *d_records, int32_t n_records,
                               int32_t n_slots, int32_t page_rows, int32_t row_bytes,
                               int32_t *d_status, void *stream);

/* Per layer, in one launch: the current-row scatter of gpb_current_row_scatter
 * (rows d_cur_rows, destinations plan->d_staging_rows, into d_staging of
 * n_staging_rows rows) and the gather of all n_slots dense slots of
 * gpb_compose_gather, with the same result as the two calls in order.  The
 * plan gives the records (prefix_desc, current_desc), the tokens of each
 * current page (cur_page_token0, cur_page_ntok) and the staging rows;
 * n_cur_pages is its NCP.  The workgroups that gather a current page first
 * write that page's current rows into staging and then read the page back
 * through the table, so the table's staging entries must be the slabs the
 * staging rows address (the layout gpb_plan_build assumes: slab w at
 * d_staging + w * CAP * page_rows * row_bytes), and the staging rows a batch
 * does not write must hold zeros (gpb_staging_clear or gpb_plan_build_clear
 * once per batch).  Rows must not repeat (the plan's do not).  Every lane
 * that writes a current row's chunk checks that its read-back addresses
 * that same chunk; when the table or plan breaks the layout it ORs
 * GPB_STATUS_LAYER_MISMATCH into *d_status (if not NULL).  Errors as the
 * two calls, plus GPB_EINVAL for plan NULL or n_cur_pages outside
 * [0, min(n_slots, n_rows)]. */
int gpb_compose_layer(void *d_dense, const gpb_sources *table, const gpb_plan *plan,
                      int32_t n_slots, int32_t n_cur_pages, void *d_staging,
                      int64_t n_staging_rows, const void *d_cur_rows, int32_t n_rows,
                      int32_t page_rows, int32_t row_bytes, int32_t *d_status,
                      void *stream);

/* Per layer, gpb_compose_layer with the fused current fill (the fill of
 * gpb_current_row_fill: each current row also goes to its pool row
 * plan->d_pool_locs[t] of d_pool, a pool of n_pool_rows rows, whatever its
 * size): the KV-cache store of the current rows, their staging fill and the
 * whole gather in one launch.  The pool rows written are the current
 * tokens' own, never pages the gather reads.  A pool row outside
 * [0, n_pool_rows) is skipped there and GPB_STATUS_BAD_STAGING_ROW is ORed
 * into *d_status.  Errors as gpb_compose_layer, plus GPB_EINVAL for
 * n_pool_rows < 0 or a NULL pool or pool_locs with current pages, and
 * GPB_EALIGN for a pool not 16-byte aligned. */
int gpb_compose_layer_fill(void *d_dense, const gpb_sources *table, const gpb_plan *plan,
                           int32_t n_slots, int32_t n_cur_pages, void *d_staging,
                           int64_t n_staging_rows, void *d_pool, int64_t n_pool_rows,
                           const void *d_cur_rows, int32_t n_rows, int32_t page_rows,
                           int32_t row_bytes, int32_t *d_status, void *stream);

/* Per layer, the consume half of the layer-ahead split in one launch (page
 * 0d87bc5, commit "prefetch staging exchange": the consume step fills the
 * current rows into staging and gathers every current page from it into
 * the dense buffer whose prefix pages were gathered ahead): gpb_compose_layer
 * for the current pages only; prefix slots of d_dense are not touched.
 * Arguments, requirements and errors as gpb_compose_layer. */
int gpb_compose_consume(void *d_dense, const gpb_sources *table, const gpb_plan *plan,
                        int32_t n_slots, int32_t n_cur_pages, void *d_staging,
                        int64_t n_staging_rows, const void *d_cur_rows, int32_t n_rows,
                        int32_t page_rows, int32_t row_bytes, int32_t *d_status,
                        void *stream);

/* Per layer, the layer-ahead split in one launch per layer (page 0d87bc5,
 * commit "prefetch staging exchange": the prefix of the next layer's dense
 * buffer is gathered a layer ahead while this layer is consumed): this
 * layer's consume (gpb_compose_consume into d_dense) and the next layer's
 * prefix pages (the plan's prefix_desc records gathered into d_dense_next),
 * in one launch.  The table lists the next layer's pool entries followed by
 * this layer's staging slabs.  Equivalent to gpb_compose_consume(d_dense,
 * ...) followed by gpb_compose_gather_records(d_dense_next, table,
 * prefix_desc, ...); d_dense and d_dense_next must not overlap.  A batch of
 * L layers runs as the prefix records of layer 0, then this call for layers
 * 0 .. L - 2, then gpb_compose_consume for layer L - 1.  Requirements and
 * errors as gpb_compose_layer, plus GPB_EINVAL for d_dense_next NULL (with
 * prefix pages) and GPB_EALIGN for it misaligned. */
int gpb_compose_layer_ahead(void *d_dense, void *d_dense_next, const gpb_sources *table,
                            const gpb_plan *plan, int32_t n_slots, int32_t n_cur_pages,
                            void *d_staging, int64_t n_staging_rows, const void *d_cur_rows,
                            int32_t n_rows, int32_t page_rows, int32_t row_bytes,
                            int32_t *d_status, void *stream);

/* The consume and layer-ahead launches with the fused fill (page 0d87bc5,
 * commit "prefetch staging exchange": the consume step fills the current
 * rows; page d63fbd4, commit "current rows written straight into staging":
 * the fill goes to the KV cache and to staging in one pass): as
 * gpb_compose_consume and gpb_compose_layer_ahead, with each current row
 * also written to its pool row plan->d_pool_locs[t] of d_pool (this layer's
 * pool, n_pool_rows rows), as gpb_compose_layer_fill does.  In the
 * layer-ahead call the table's pool entries are the next layer's pools and
 * d_pool is this layer's; the pool rows written are current tokens' own,
 * never pages a gather reads.  Errors as gpb_compose_consume /
 * gpb_compose_layer_ahead, plus those gpb_compose_layer_fill adds for the
 * pool. */
int gpb_compose_consume_fill(void *d_dense, const gpb_sources *table, const gpb_plan *plan,
                             int32_t n_slots, int32_t n_cur_pages, void *d_staging,
                             int64_t n_staging_rows, void *d_pool, int64_t n_pool_rows,
                             const void *d_cur_rows, int32_t n_rows, int32_t page_rows,
                             int32_t row_bytes, int32_t *d_status, void *stream);

int gpb_compose_layer_ahead_fill(void *d_dense, void *d_dense_next, const gpb_sources *table,
                                 const gpb_plan *plan, int32_t n_slots, int32_t n_cur_pages,
                                 void *d_staging, int64_t n_staging_rows, void *d_pool,
                                 int64_t n_pool_rows, const void *d_cur_rows, int32_t n_rows,
                                 int32_t page_rows, int32_t row_bytes, int32_t *d_status,
                                 void *stream);

/* Several row formats composed on one plan in one launch each (page 0d87bc5,
 * commit "prefetch staging exchange": the indexer-key fill reuses the token
 * plan's staging page inverse; the index twin of the compose runs beside the
 * token-KV compose).  Every group has its own arenas and row size and shares
 * the plan's staging_rows / owner / src; the result is the one the
 * single-format calls give per group.  Up to GPB_MAX_GROUPS groups; a group's
 * table holds at most GPB_MAX_GROUP_SOURCES entries. */
#define GPB_MAX_GROUPS 4
#define GPB_MAX_GROUP_SOURCES 16

typedef struct gpb_row_group {      /* one format's current-row scatter */
  void *d_staging;                  /* n_staging_rows rows of row_bytes  */
  int64_t n_staging_rows;
  const void *d_cur_rows;           /* n_rows rows of row_bytes           */
  int32_t row_bytes;                /* multiple of 16                     */
} gpb_row_group;

typedef struct gpb_gather_group {   /* one format's slot-dense gather      */
  void *d_dense;                    /* n_slots pages of page_rows*row_bytes */
  const gpb_sources *table;         /* n <= GPB_MAX_GROUP_SOURCES          */
  int32_t row_bytes;                /* multiple of 16                     */
} gpb_gather_group;

/* gpb_current_row_scatter for every group, one launch.  Errors as
 * gpb_current_row_scatter for any group, plus GPB_EINVAL for n_groups outside
 * 1..GPB_MAX_GROUPS and GPB_ERANGE past 2^31 workgroups in total. */
int gpb_current_row_scatter_groups(const gpb_row_group *groups, int32_t n_groups,
                                   const int32_t *d_staging_rows, int32_t n_rows,
                                   int32_t *d_status, void *stream);

/* gpb_compose_gather for every group (same descriptors and page_rows), one
 * launch.  Errors as gpb_compose_gather for any group (a group's table holds
 * at most GPB_MAX_GROUP_SOURCES entries), plus GPB_EINVAL for n_groups outside
 * 1..GPB_MAX_GROUPS and GPB_ERANGE past 2^31 workgroups in total. */
int gpb_compose_gather_groups(const gpb_gather_group *groups, int32_t n_groups,
                              const int32_t *d_owner, const int32_t *d_src,
                              int32_t n_slots, int32_t page_rows, int32_t *d_status,
                              void *stream);

typedef struct gpb_layer_group {    /* one format's one-launch layer        */
  void *d_dense;                    /* n_slots pages of page_rows*row_bytes */
  const gpb_sources *table;         /* n <= GPB_MAX_GROUP_SOURCES: pool
                                       entries, then the slabs carved from
                                       d_staging                           */
  void *d_staging;                  /* n_staging_rows rows, zero where the
                                       plan writes no row                  */
  int64_t n_staging_rows;
  const void *d_cur_rows;           /* n_rows rows of row_bytes            */
  int32_t row_bytes;                /* multiple of 16                      */
} gpb_layer_group;

/* gpb_compose_layer for every group (same plan, n_slots, n_cur_pages,
 * n_rows and page_rows), one launch: the current pages of every group first,
 * then their prefix pages, so the formats share one launch's ramp.  The
 * result is the one gpb_compose_layer gives per group; the requirements are
 * its requirements, per group.  Errors as gpb_compose_layer for any group,
 * plus GPB_EINVAL for n_groups outside 1..GPB_MAX_GROUPS or a table of more
 * than GPB_MAX_GROUP_SOURCES entries, and GPB_ERANGE past 2^31 workgroups in
 * total. */
int gpb_compose_layer_groups(const gpb_layer_group *groups, int32_t n_groups,
                             const gpb_plan *plan, int32_t n_slots, int32_t n_cur_pages,
                             int32_t n_rows, int32_t page_rows, int32_t *d_status,
                             void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the layer
 * of gpb_compose_layer with its staging region taken from a static array of
 * the library's own, GPB_SCRATCH_BYTES on each GPU (held from the first
 * call on that GPU until the process ends), instead of a caller buffer.
 * pools lists the NP pool entries only (1 <= NP <= GPB_MAX_SOURCES -
 * n_writers); the library appends n_writers slabs of staging_cap_pages
 * pages, carved from the array as gpb_plan_build assumes, and plan is a
 * plan built for that geometry (n_writers, staging_cap_pages, page_rows).
 * Each call zeroes the W * CAP * page_rows * row_bytes bytes it uses, in a
 * launch of its own before the layer's (the array keeps the last call's
 * rows), so the staging clear of gpb_plan_build_clear is not needed.  The
 * work runs on the calling thread's current device, which `stream` must
 * belong to.  Calls that overlap on one GPU share its array and race;
 * calls in stream order do not.  Calls no allocating routine; the first
 * call on a device looks the array's address up once, so make it before
 * capturing a graph; later calls can be captured (two kernel nodes).  Errors as
 * gpb_compose_layer, plus GPB_ESCRATCH (n_writers * staging_cap_pages *
 * page_rows * row_bytes > GPB_SCRATCH_BYTES), GPB_EINVAL (pools NULL, NP or
 * n_writers out of range, staging_cap_pages < 1, a stream of another
 * device) and GPB_EHIP (no device, or the address lookup failed). */
#define GPB_SCRATCH_BYTES (64LL * 1024 * 1024)

int gpb_compose_layer_noalloc(void *d_dense, const gpb_sources *pools, int32_t n_writers,
                              int32_t staging_cap_pages, const gpb_plan *plan,
                              int32_t n_slots, int32_t n_cur_pages, const void *d_cur_rows,
                              int32_t n_rows, int32_t page_rows, int32_t row_bytes,
                              int32_t *d_status, void *stream);

/* Static, human-readable name of a gpb_status value. */
const char *gpb_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* GPB_H */
