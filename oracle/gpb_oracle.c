/*
 * gpb_oracle.c -- plain, slow, obviously correct CPU oracle for the KV-compose
 * plan build and the per-layer current-row scatter + slot-dense page gather.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or helper with the HIP path under gather_plan_build_amd/.
 *
 * Sources (commit pages of the sglang fork; cited by page and commit):
 *   [SD]  page d63fbd4, commit "current rows written straight into staging,
 *         one slot-dense gather over a 2*cp pointer table"
 *   [TP]  page d63fbd4, commit "touched-pages-proportional staging"
 *   [CG]  page d63fbd4 (and page f74f0a5), commit "cut per-layer CPU on the
 *         prefill launch path" (ragged plan, slot spans)
 *   [V2]  page d63fbd4, commit "compose_v2" (-1 sentinels zero-fill)
 *   [SS]  page 0d87bc5, commit "canonical prefix/current slot spans"
 *   [PS]  page 0d87bc5, commit "prefetch staging exchange" (page 0 is the
 *         dummy page; staging slot of current page i is i + 1)
 *   [F8]  page 0d87bc5, commit "fp8 index_copy_ -> uint8 views"
 *
 * Every value is an integer; rows are opaque byte strings.  All loops are
 * the plainest form of the step they implement; nothing is fused, blocked
 * or reordered.
 *
 * Parity status (the pins live in tests/):
 *   gpbo_validate, gpbo_counts, gpbo_plan's spans, slot pages, page inverse,
 *   staging page inverse, owner/src, writer, staging rows and mixed_locs,
 *   gpbo_layer, gpbo_gather_slots, gpbo_fill, gpbo_prefetch_lists,
 *   gpbo_page_records, gpbo_gather_records, gpbo_writer_lists and the
 *   token_req of gpbo_token_expansions: pinned (brute force on tagged rows,
 *   the closed form, torch index_copy_ / index_select and numpy take and
 *   repeat, a hand-derived worked example).
 *   q_lens, kv_lens, q_starts, k_bases, current_bases, q_bases, and the
 *   topk_offsets and segments of gpbo_token_expansions: the pages give only
 *   their names, so they are pinned only to their stated definitions through
 *   the dense and staging geometry they must agree with -- parity unpinned as
 *   far as the pages themselves go.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Reasons a batch is rejected (fail fast, never fall back: [TP], [SS]). */
enum {
  GPBO_OK = 0,
  GPBO_BAD_SHAPE = 1,    /* negative or zero geometry / counts          */
  GPBO_BAD_PAGE = 2,     /* page id 0 (dummy), out of range, or repeated */
  GPBO_CAPACITY = 3,     /* 1 + current pages > staging pages per slab   */
  GPBO_TOO_LARGE = 4     /* a row index would not fit in int32           */
};

/* ceil(a / b) for a >= 0, b > 0 */
static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/*
 * O1: validate the batch.  Page ids live in [1, n_pool_pages) because page 0
 * is the dummy page [PS]; every page of the batch is distinct, so the page
 * inverse is a true inverse.  Staging must hold slot 0 plus every current
 * page of the batch [PS], [TP].
 */
int gpbo_validate(int32_t bs, int32_t page_size, int32_t row_bytes,
                  int32_t n_pool_pages, int32_t n_pool_entries,
                  int32_t n_writers, int32_t staging_cap_pages,
                  const int32_t *prefix_pages, const int32_t *cur_tokens,
                  const int32_t *req_pages) {
  if (bs < 0 || page_size < 1 || row_bytes < 16 || row_bytes % 16 != 0 ||
      n_pool_pages < 1 || n_pool_entries < 1 || n_writers < 1 ||
      staging_cap_pages < 1)
    return GPBO_BAD_SHAPE;
  int64_t total_pages = 0, total_tokens = 0, total_cur_pages = 0;
  for (int32_t r = 0; r < bs; r++) {
    if (prefix_pages[r] < 0 || cur_tokens[r] < 0) return GPBO_BAD_SHAPE;
    int64_t cp = ceil_div(cur_tokens[r], page_size);
    total_pages += prefix_pages[r] + cp;
    total_tokens += cur_tokens[r];
    total_cur_pages += cp;
  }
  if (total_pages * page_size > INT32_MAX || total_tokens > INT32_MAX ||
      (int64_t)n_pool_pages * page_size > INT32_MAX ||
      (int64_t)n_writers * staging_cap_pages * page_size > INT32_MAX)
    return GPBO_TOO_LARGE;
  if (1 + total_cur_pages > staging_cap_pages) return GPBO_CAPACITY;
  char *seen = (char *)calloc((size_t)n_pool_pages, 1);
  if (!seen) return GPBO_TOO_LARGE;
  int rc = GPBO_OK;
  for (int64_t k = 0; k < total_pages; k++) {
    int32_t p = req_pages[k];
    if (p < 1 || p >= n_pool_pages || seen[p]) { rc = GPBO_BAD_PAGE; break; }
    seen[p] = 1;
  }
  free(seen);
  return rc;
}

/* O2: S (dense slots), T (current rows), NCP (current pages). */
void gpbo_counts(int32_t bs, int32_t page_size, const int32_t *prefix_pages,
                 const int32_t *cur_tokens, int64_t out[3]) {
  int64_t S = 0, T = 0, NCP = 0;
  for (int32_t r = 0; r < bs; r++) {
    int64_t C = ceil_div(cur_tokens[r], page_size);
    S += prefix_pages[r] + C;
    T += cur_tokens[r];
    NCP += C;
  }
  out[0] = S; out[1] = T; out[2] = NCP;
}

/*
 * O3..O9: the per-batch plan.  Output arrays are caller-allocated:
 *   slot_base[bs], prefix_span[2bs], current_span[2bs],
 *   q_lens, kv_lens, q_starts, k_bases, q_bases, current_bases [bs each],
 *   slot_pages, owner, src [S], page_inverse, staging_page_inverse
 *   [n_pool_pages], writer [NCP], staging_rows, mixed_locs [T].
 * Returns the validation code; on failure no output is written.
 */
int gpbo_plan(int32_t bs, int32_t page_size, int32_t row_bytes,
              int32_t n_pool_pages, int32_t n_pool_entries, int32_t n_writers,
              int32_t staging_cap_pages, const int32_t *prefix_pages,
              const int32_t *cur_tokens, const int32_t *req_pages,
              int32_t *slot_base, int32_t *prefix_span, int32_t *current_span,
              int32_t *q_lens, int32_t *kv_lens, int32_t *q_starts,
              int32_t *k_bases, int32_t *q_bases, int32_t *current_bases,
              int32_t *slot_pages, int32_t *owner, int32_t *src,
              int32_t *page_inverse, int32_t *staging_page_inverse,
              int32_t *writer, int32_t *staging_rows, int32_t *mixed_locs) {
  int rc = gpbo_validate(bs, page_size, row_bytes, n_pool_pages,
                         n_pool_entries, n_writers, staging_cap_pages,
                         prefix_pages, cur_tokens, req_pages);
  if (rc != GPBO_OK) return rc;
  const int32_t PS = page_size, NP = n_pool_entries, W = n_writers;
  const int32_t CAP = staging_cap_pages;

  /* O2/O3: per-request current pages C_r and slots n_r = P_r + C_r; the slot
   * base of request r is the count of slots of all earlier requests.  The
   * prefix span comes first, the current span abuts it [SS], [CG]. */
  int32_t running_slots = 0;
  for (int32_t r = 0; r < bs; r++) {
    int32_t C = (int32_t)ceil_div(cur_tokens[r], PS);
    int32_t n = prefix_pages[r] + C;
    slot_base[r] = running_slots;
    prefix_span[2 * r + 0] = running_slots;
    prefix_span[2 * r + 1] = running_slots + prefix_pages[r];
    current_span[2 * r + 0] = running_slots + prefix_pages[r];
    current_span[2 * r + 1] = running_slots + n;
    running_slots += n;
  }
  const int32_t S = running_slots;

  /* O8: ragged int32 descriptors [CG]; each base is an exclusive running
   * sum over the earlier requests. */
  int32_t run_tokens = 0, run_slots = 0, run_cur_pages = 0;
  for (int32_t r = 0; r < bs; r++) {
    int32_t C = (int32_t)ceil_div(cur_tokens[r], PS);
    q_lens[r] = cur_tokens[r];
    kv_lens[r] = PS * prefix_pages[r] + cur_tokens[r];
    q_starts[r] = run_tokens;
    k_bases[r] = PS * run_slots;
    current_bases[r] = PS * run_slots + PS * prefix_pages[r];
    q_bases[r] = PS * run_cur_pages;
    run_tokens += cur_tokens[r];
    run_slots += prefix_pages[r] + C;
    run_cur_pages += C;
  }

  /* O4: the page of every dense slot, request by request, prefix pages
   * then current pages, in the order the request lists them. */
  for (int32_t s = 0; s < S; s++) slot_pages[s] = req_pages[s];

  /* O5: page -> dense slot, -1 where the page is not in the batch. */
  for (int32_t p = 0; p < n_pool_pages; p++) page_inverse[p] = -1;
  for (int32_t s = 0; s < S; s++) page_inverse[slot_pages[s]] = s;

  /* O6: current page i (batch order: requests in order, pages in sequence
   * order [TP]) has writer i mod W and sits in staging slot i + 1 of slab w
   * (slot 0 reserved [PS]).  The slabs are carved one after another, CAP
   * pages each, so its page in the carved region is w*CAP + i + 1. */
  for (int32_t p = 0; p < n_pool_pages; p++) staging_page_inverse[p] = -1;
  int32_t i = 0;
  for (int32_t r = 0; r < bs; r++) {
    int32_t C = (int32_t)ceil_div(cur_tokens[r], PS);
    for (int32_t k = 0; k < C; k++, i++) {
      int32_t s = slot_base[r] + prefix_pages[r] + k;
      int32_t w = i % W;
      writer[i] = w;
      staging_page_inverse[slot_pages[s]] = w * CAP + i + 1;
    }
  }

  /* O7: gather descriptors into the [pool entries || staging entries]
   * pointer table [SD]: prefix slots read pool entry (page mod NP) at the
   * page itself; current slots read staging entry NP + writer at staging
   * slot i + 1. */
  i = 0;
  for (int32_t r = 0; r < bs; r++) {
    for (int32_t k = 0; k < prefix_pages[r]; k++) {
      int32_t s = slot_base[r] + k;
      owner[s] = slot_pages[s] % NP;
      src[s] = slot_pages[s];
    }
    int32_t C = (int32_t)ceil_div(cur_tokens[r], PS);
    for (int32_t k = 0; k < C; k++, i++) {
      int32_t s = slot_base[r] + prefix_pages[r] + k;
      owner[s] = NP + writer[i];
      src[s] = i + 1;
    }
  }

  /* O9: per current token, its pool location (loc) and the staging row the
   * fill writes, found through the staging-remapped page inverse, the same
   * route by which the pages' fill reaches its destinations [SD];
   * mixed_locs is the token's row in the dense buffer. */
  for (int32_t r = 0; r < bs; r++) {
    for (int32_t j = 0; j < cur_tokens[r]; j++) {
      int32_t t = q_starts[r] + j;
      int32_t s = slot_base[r] + prefix_pages[r] + j / PS;
      int32_t loc = slot_pages[s] * PS + j % PS;
      staging_rows[t] = staging_page_inverse[loc / PS] * PS + loc % PS;
      mixed_locs[t] = current_bases[r] + j;
    }
  }
  return GPBO_OK;
}

/*
 * O10: one layer of the compose.
 *  1. the staging region (n_staging_rows rows) is zeroed;
 *  2. staging[staging_rows[t]] = cur[t] for every current row, as whole
 *     byte rows (index_copy_ on uint8 views [F8], [SD]);
 *  3. every dense slot receives one page: the page src of table entry
 *     owner, or zeros when owner or src is -1 [V2], [SD].
 * table[e] is the base of arena e; table_pages[e] its size in pages.  A
 * descriptor outside its arena, or a staging row outside the region, is an
 * error (returns 1) after the rest of the layer has been done; such a page
 * is zeroed and such a row is skipped.
 */
int gpbo_layer(const uint8_t *const *table, const int64_t *table_pages,
               int32_t n_src, uint8_t *staging, int64_t n_staging_rows,
               const uint8_t *cur, int32_t n_rows, const int32_t *staging_rows,
               const int32_t *owner, const int32_t *src, int32_t n_slots,
               int32_t page_size, int32_t row_bytes, uint8_t *dense) {
  int bad = 0;
  const int64_t RB = row_bytes;
  const int64_t page_bytes = (int64_t)page_size * RB;
  memset(staging, 0, (size_t)(n_staging_rows * RB));
  for (int32_t t = 0; t < n_rows; t++) {
    int64_t row = staging_rows[t];
    if (row < 0 || row >= n_staging_rows) { bad = 1; continue; }
    memcpy(staging + row * RB, cur + (int64_t)t * RB, (size_t)RB);
  }
  for (int32_t s = 0; s < n_slots; s++) {
    uint8_t *out = dense + (int64_t)s * page_bytes;
    int32_t e = owner[s], p = src[s];
    if (e < 0 || p < 0) { memset(out, 0, (size_t)page_bytes); continue; }
    if (e >= n_src || p >= table_pages[e]) {
      bad = 1;
      memset(out, 0, (size_t)page_bytes);
      continue;
    }
    memcpy(out, table[e] + (int64_t)p * page_bytes, (size_t)page_bytes);
  }
  return bad;
}

/*
 * O12: per-token ragged expansions, one set per batch ([CG]: the
 * O(total-q-tokens) top-k offset list and the segment records of the ragged
 * index plan; page 0d87bc5, commit "flattened request row ids": row ids that
 * the pages built with repeat_interleave over per-request lengths).  For every
 * current token t (token-packed, request order):
 *   token_req[t]     the request it belongs to;
 *   topk_offsets[t]  the dense row where that request's KV starts, so a
 *                    request-relative KV position (a top-k index) plus the
 *                    offset is a row of the composed dense buffer.
 * For every request r one segment record of four int32:
 *   (first token, tokens, first dense row, KV rows = PS * P_r + c_r).
 */
void gpbo_token_expansions(int32_t bs, int32_t page_size,
                           const int32_t *prefix_pages, const int32_t *cur_tokens,
                           int32_t *token_req, int32_t *topk_offsets,
                           int32_t *segments) {
  int32_t token = 0, dense_row = 0;
  for (int32_t r = 0; r < bs; r++) {
    int32_t pages = prefix_pages[r] + (int32_t)ceil_div(cur_tokens[r], page_size);
    for (int32_t j = 0; j < cur_tokens[r]; j++) {
      token_req[token + j] = r;
      topk_offsets[token + j] = dense_row;
    }
    segments[4 * r + 0] = token;
    segments[4 * r + 1] = cur_tokens[r];
    segments[4 * r + 2] = dense_row;
    segments[4 * r + 3] = page_size * prefix_pages[r] + cur_tokens[r];
    token += cur_tokens[r];
    dense_row += page_size * pages;
  }
}

/*
 * O13: lists for the layer-ahead prefetch (page 0d87bc5, commit "prefetch
 * staging exchange": the prefetcher fills the dense buffer's prefix a layer
 * ahead; the consume step fills the current rows into staging and gathers
 * ALL current pages from the staging).  From the batch metadata alone:
 *   prefix_slots[u]   dense slot of the u-th prefix page of the batch
 *                     (requests in order, pages in order)   [S - NCP]
 *   current_slots[i]  dense slot of current page i           [NCP]
 *   pool_locs[t]      pool row of current token t: its page is the request's
 *                     listed current page j / PS, row j mod PS   [T]
 *   cur_page_token0[i], cur_page_ntok[i]  the current tokens page i holds:
 *                     first token index and count (1..PS)       [NCP]
 */
void gpbo_prefetch_lists(int32_t bs, int32_t page_size,
                         const int32_t *prefix_pages, const int32_t *cur_tokens,
                         const int32_t *req_pages, int32_t *prefix_slots,
                         int32_t *current_slots, int32_t *pool_locs,
                         int32_t *cur_page_token0, int32_t *cur_page_ntok) {
  int32_t slot = 0, u = 0, i = 0, token = 0;
  for (int32_t r = 0; r < bs; r++) {
    for (int32_t k = 0; k < prefix_pages[r]; k++) prefix_slots[u++] = slot++;
    int32_t first_cur = slot;
    int32_t pages = (int32_t)ceil_div(cur_tokens[r], page_size);
    for (int32_t k = 0; k < pages; k++) {
      /* current page i holds tokens [token + k*PS, token + min(c, (k+1)*PS)) */
      cur_page_token0[i] = token + k * page_size;
      cur_page_ntok[i] = cur_tokens[r] - k * page_size < page_size
                             ? cur_tokens[r] - k * page_size : page_size;
      current_slots[i++] = slot++;
    }
    for (int32_t j = 0; j < cur_tokens[r]; j++)
      pool_locs[token++] = req_pages[first_cur + j / page_size] * page_size + j % page_size;
  }
}

/*
 * O14: gather only the listed dense slots (the prefetch half or the current
 * half of a layer's gather); every other slot of `dense` is left as it is.
 * Same descriptor rules as O10.  Returns 1 if a descriptor was out of range.
 */
int gpbo_gather_slots(const uint8_t *const *table, const int64_t *table_pages,
                      int32_t n_src, const int32_t *slots, int32_t n,
                      const int32_t *owner, const int32_t *src, int32_t page_size,
                      int32_t row_bytes, uint8_t *dense) {
  int bad = 0;
  const int64_t page_bytes = (int64_t)page_size * row_bytes;
  for (int32_t k = 0; k < n; k++) {
    int32_t s = slots[k];
    uint8_t *out = dense + (int64_t)s * page_bytes;
    int32_t e = owner[s], p = src[s];
    if (e < 0 || p < 0) { memset(out, 0, (size_t)page_bytes); continue; }
    if (e >= n_src || p >= table_pages[e]) {
      bad = 1;
      memset(out, 0, (size_t)page_bytes);
      continue;
    }
    memcpy(out, table[e] + (int64_t)p * page_bytes, (size_t)page_bytes);
  }
  return bad;
}

/*
 * O15: the fused current fill: every current row goes to its staging row
 * (as the scatter) and to its pool row (its KV-cache location), whole rows
 * of bytes.  Rows whose destination is out of range are skipped there and
 * reported (returns 1).  Nothing is zeroed here.
 */
int gpbo_fill(uint8_t *staging, int64_t n_staging_rows, const int32_t *staging_rows,
              uint8_t *pool, int64_t n_pool_rows, const int32_t *pool_locs,
              const uint8_t *cur, int32_t n_rows, int32_t row_bytes) {
  int bad = 0;
  const int64_t RB = row_bytes;
  for (int32_t t = 0; t < n_rows; t++) {
    const uint8_t *row = cur + (int64_t)t * RB;
    int64_t d = staging_rows[t];
    if (d < 0 || d >= n_staging_rows) bad = 1;
    else memcpy(staging + d * RB, row, (size_t)RB);
    int64_t q = pool_locs[t];
    if (q < 0 || q >= n_pool_rows) bad = 1;
    else memcpy(pool + q * RB, row, (size_t)RB);
  }
  return bad;
}

/*
 * O16: gather records for a list of dense slots (the two halves of the
 * layer-ahead split, page 0d87bc5, commit "prefetch staging exchange"):
 * record k is four int32 (slot, owner[slot], src[slot], 0), so a gather over
 * the list finds everything about a page in one record.
 */
void gpbo_page_records(const int32_t *slots, int32_t n, const int32_t *owner,
                       const int32_t *src, int32_t *records) {
  for (int32_t k = 0; k < n; k++) {
    int32_t s = slots[k];
    records[4 * k + 0] = s;
    records[4 * k + 1] = owner[s];
    records[4 * k + 2] = src[s];
    records[4 * k + 3] = 0;
  }
}

/*
 * O17: gather the pages the records name: dense page records[4k] receives
 * page records[4k+2] of table entry records[4k+1]; descriptor rules as O10.
 * Returns 1 if a descriptor was out of range.
 */
int gpbo_gather_records(const uint8_t *const *table, const int64_t *table_pages,
                        int32_t n_src, const int32_t *records, int32_t n,
                        int32_t page_size, int32_t row_bytes, uint8_t *dense) {
  int bad = 0;
  const int64_t page_bytes = (int64_t)page_size * row_bytes;
  for (int32_t k = 0; k < n; k++) {
    int32_t s = records[4 * k + 0], e = records[4 * k + 1], p = records[4 * k + 2];
    uint8_t *out = dense + (int64_t)s * page_bytes;
    if (e < 0 || p < 0) { memset(out, 0, (size_t)page_bytes); continue; }
    if (e >= n_src || p >= table_pages[e]) {
      bad = 1;
      memset(out, 0, (size_t)page_bytes);
      continue;
    }
    memcpy(out, table[e] + (int64_t)p * page_bytes, (size_t)page_bytes);
  }
  return bad;
}

/*
 * O18: what each writer scatters (page d63fbd4, commit "counting barrier +
 * CUDA-IPC gather": a current page has exactly one writer under the
 * page-aligned split, and the writers are fixed per batch; page 0d87bc5,
 * commit "prefetch staging exchange": each rank fills its own current rows
 * into its own staging).  Writer w owns the current pages i with writer
 * i mod W; its tokens, in token order, form list w, and list w is stored
 * after lists 0..w-1:
 *   writer_offsets[w]   first entry of list w; writer_offsets[W] = T  [W+1]
 *   writer_tokens[k]    batch token of entry k                         [T]
 *   writer_rows[k]      that token's staging row inside slab w (the
 *                       batch staging row less w * CAP * PS)           [T]
 *   writer_page_row0[i] entry of current page i's first token, counted
 *                       from the start of its writer's list           [NCP]
 * A writer holding its tokens' rows in list order scatters row k of its
 * list to writer_rows[k] of its own slab.
 */
void gpbo_writer_lists(int32_t bs, int32_t page_size, int32_t n_writers,
                       int32_t staging_cap_pages, const int32_t *prefix_pages,
                       const int32_t *cur_tokens, const int32_t *staging_rows,
                       int32_t *writer_offsets, int32_t *writer_tokens,
                       int32_t *writer_rows, int32_t *writer_page_row0) {
  const int32_t PS = page_size, W = n_writers;
  const int64_t slab_rows = (int64_t)staging_cap_pages * PS;
  (void)prefix_pages;
  int32_t k = 0;
  for (int32_t w = 0; w < W; w++) {
    writer_offsets[w] = k;
    int32_t i = 0, token = 0;
    for (int32_t r = 0; r < bs; r++) {
      int32_t C = (int32_t)ceil_div(cur_tokens[r], PS);
      for (int32_t q = 0; q < C; q++, i++) {
        if (i % W != w) continue;
        writer_page_row0[i] = k - writer_offsets[w];
        int32_t end = (q + 1) * PS < cur_tokens[r] ? (q + 1) * PS : cur_tokens[r];
        for (int32_t j = q * PS; j < end; j++) {
          int32_t t = token + j;
          writer_tokens[k] = t;
          writer_rows[k] = (int32_t)(staging_rows[t] - w * slab_rows);
          k++;
        }
      }
      token += cur_tokens[r];
    }
  }
  writer_offsets[W] = k;
}
