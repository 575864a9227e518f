/*
 * A plain C consumer of include/gpb.h: no torch, no C++.  Device memory comes
 * from the HIP runtime API directly.
 *
 *   consumer check            host-only: error paths and plan sizes
 *   consumer run <in> <out>   read a batch (binary, see below), build the plan,
 *                             clear staging, scatter and gather one layer on
 *                             the GPU, write the plan arrays, staging and
 *                             dense buffer to <out>
 *
 * Input file (int32 little endian unless noted): bs, page_size, row_bytes,
 * n_pool_pages, n_pool_entries, n_writers, staging_cap_pages, then P[bs],
 * c[bs], n_req, req_pages[n_req], then the pool bytes
 * (n_pool_pages*page_size*row_bytes) and the current rows (T*row_bytes).
 * Output: S, T, NCP, the plan arrays in the header's order, staging bytes,
 * dense bytes.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "gpb.h"

#define CHECK(x) do { int rc_ = (x); if (rc_ != GPB_OK) { \
  fprintf(stderr, "%s:%d %s -> %d (%s)\n", __FILE__, __LINE__, #x, rc_, gpb_strerror(rc_)); \
  return 2; } } while (0)
#define HCHECK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
  fprintf(stderr, "%s:%d %s -> %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
  return 3; } } while (0)

static int expect(int got, int want, const char *what) {
  if (got != want) {
    fprintf(stderr, "%s: got %d want %d\n", what, got, want);
    return 1;
  }
  return 0;
}

static int check(void) {
  int32_t P[2] = {3, 5}, c[2] = {100, 37};
  int32_t pages[11] = {10, 20, 30, 40, 50, 60, 70, 80, 90, 100, 110};
  gpb_batch b;
  memset(&b, 0, sizeof b);
  b.bs = 2; b.page_size = 64; b.row_bytes = 1152; b.n_pool_pages = 256;
  b.n_pool_entries = 1; b.n_writers = 1; b.staging_cap_pages = 6;
  b.h_prefix_pages = P; b.h_cur_tokens = c; b.h_req_pages = pages;
  int32_t S = -1, T = -1, NCP = -1;
  int bad = 0;
  bad |= expect(gpb_plan_sizes(&b, &S, &T, &NCP), GPB_OK, "sizes");
  bad |= expect(S, 11, "S") | expect(T, 137, "T") | expect(NCP, 3, "NCP");
  pages[4] = 0;
  bad |= expect(gpb_plan_sizes(&b, NULL, NULL, NULL), GPB_EPAGE, "dummy page");
  pages[4] = 50;
  b.staging_cap_pages = 3;
  bad |= expect(gpb_plan_sizes(&b, NULL, NULL, NULL), GPB_ECAPACITY, "capacity");
  b.staging_cap_pages = 6;
  b.row_bytes = 1000;
  bad |= expect(gpb_plan_sizes(&b, NULL, NULL, NULL), GPB_EALIGN, "row bytes");
  b.row_bytes = 1152;
  gpb_plan p;
  memset(&p, 0, sizeof p);
  bad |= expect(gpb_plan_build(&b, &p, NULL), GPB_EINVAL, "plan without outputs");
  gpb_sources t;
  memset(&t, 0, sizeof t);
  bad |= expect(gpb_compose_gather(NULL, &t, NULL, NULL, 4, 64, 1152, NULL, NULL),
                GPB_EINVAL, "empty table");
  bad |= expect(gpb_current_row_scatter(NULL, 8, NULL, NULL, 0, 1152, NULL, NULL),
                GPB_OK, "empty scatter");
  bad |= expect(gpb_staging_clear(NULL, 0, NULL), GPB_OK, "empty clear");
  t.n = 1;
  bad |= expect(gpb_compose_layer_noalloc(NULL, &t, 1, (int32_t)(GPB_SCRATCH_BYTES / (64 * 1152)) + 1,
                                          &p, 11, 3, NULL, 137, 64, 1152, NULL, NULL),
                GPB_ESCRATCH, "staging beyond the static array");
  if (!bad) printf("c consumer: host checks ok\n");
  return bad;
}

static int32_t rd32(FILE *f) {
  int32_t v = 0;
  if (fread(&v, 4, 1, f) != 1) { fprintf(stderr, "short input\n"); exit(4); }
  return v;
}

/* Equality of two device regions, compared on the host. */
static int same_device_bytes(const void *a, const void *b, size_t n) {
  if (n == 0) return 1;
  uint8_t *ha = malloc(n), *hb = malloc(n);
  int ok = ha && hb && hipMemcpy(ha, a, n, hipMemcpyDeviceToHost) == hipSuccess &&
           hipMemcpy(hb, b, n, hipMemcpyDeviceToHost) == hipSuccess && memcmp(ha, hb, n) == 0;
  free(ha);
  free(hb);
  return ok;
}

/* The remaining entry points against the layer just composed by the core
 * calls: the prefetch split (prefix slots, then current slots, by slot list
 * and by record) and the grouped gather must reproduce its dense buffer; the
 * grouped scatter, the fused fill and the per-writer scatters must reproduce
 * its staging, and the fill must leave each current row at its pool row and
 * every other pool byte as it was; the one-launch layer and the fused
 * consume must reproduce both; the plan build with clear zeroes staging. */
static int other_entry_points(const gpb_batch *b, const gpb_plan *p, const gpb_sources *t,
                              int32_t S, int32_t T, int32_t NCP, void *d_pool, void *d_cur,
                              void *d_stag, void *d_dense, const uint8_t *h_pool,
                              const uint8_t *h_cur, int32_t *d_status, hipStream_t st) {
  const size_t RB = (size_t)b->row_bytes, PS = (size_t)b->page_size;
  const size_t dense_bytes = (size_t)S * PS * RB;
  const size_t stag_rows = (size_t)b->n_writers * b->staging_cap_pages * PS;
  const size_t pool_bytes = (size_t)b->n_pool_pages * PS * RB;
  void *d_dense2, *d_stag2, *d_pool2;
  HCHECK(hipMalloc(&d_dense2, dense_bytes + 16));
  HCHECK(hipMalloc(&d_stag2, stag_rows * RB));
  HCHECK(hipMalloc(&d_pool2, pool_bytes));

  /* prefetch split: prefix slots a layer ahead, then the current slots */
  HCHECK(hipMemset(d_dense2, 0xEE, dense_bytes + 16));
  CHECK(gpb_compose_gather_slots(d_dense2, t, p->d_prefix_slots, S - NCP, p->d_owner,
                                 p->d_src, S, b->page_size, b->row_bytes, d_status, st));
  CHECK(gpb_compose_gather_slots(d_dense2, t, p->d_current_slots, NCP, p->d_owner,
                                 p->d_src, S, b->page_size, b->row_bytes, d_status, st));
  HCHECK(hipStreamSynchronize(st));
  if (!same_device_bytes(d_dense2, d_dense, dense_bytes)) {
    fprintf(stderr, "prefetch split differs from the one-shot gather\n");
    return 6;
  }

  /* grouped calls with one group each (the table fits a group's limit) */
  if (t->n <= GPB_MAX_GROUP_SOURCES) {
    CHECK(gpb_staging_clear(d_stag2, (int64_t)(stag_rows * RB), st));
    gpb_row_group rg = {d_stag2, (int64_t)stag_rows, d_cur, b->row_bytes};
    CHECK(gpb_current_row_scatter_groups(&rg, 1, p->d_staging_rows, T, d_status, st));
    HCHECK(hipMemsetAsync(d_dense2, 0xEE, dense_bytes + 16, st));
    gpb_gather_group gg = {d_dense2, t, b->row_bytes};
    CHECK(gpb_compose_gather_groups(&gg, 1, p->d_owner, p->d_src, S, b->page_size, d_status,
                                    st));
    HCHECK(hipStreamSynchronize(st));
    if (!same_device_bytes(d_stag2, d_stag, stag_rows * RB) ||
        !same_device_bytes(d_dense2, d_dense, dense_bytes)) {
      fprintf(stderr, "grouped calls differ from the single-format calls\n");
      return 7;
    }
  }

  /* the launches with the fused fill, each into a fresh copy of the pool:
   * the one-launch layer, the prefix records then the consume with fill,
   * and the layer-ahead launch with fill (the "next" layer's prefix pages
   * into the same buffer through a separate pointer).  Same dense and
   * staging as the two-call layer; the same pool as the first of them,
   * which is checked with the separate fill below */
  {
    gpb_sources t3 = *t;
    for (int w = 0; w < b->n_writers; w++)
      t3.base[b->n_pool_entries + w] =
          (uint8_t *)d_stag2 + (size_t)w * b->staging_cap_pages * PS * RB;
    const int64_t pool_rows = (int64_t)b->n_pool_pages * (int64_t)PS;
    void *d_pool3;
    HCHECK(hipMalloc(&d_pool3, pool_bytes));
    for (int pass = 0; pass < 3; pass++) {
      HCHECK(hipMemcpy(d_pool2, d_pool, pool_bytes, hipMemcpyDeviceToDevice));
      CHECK(gpb_staging_clear(d_stag2, (int64_t)(stag_rows * RB), st));
      HCHECK(hipMemsetAsync(d_dense2, 0xEE, dense_bytes + 16, st));
      if (pass == 0) {
        CHECK(gpb_compose_layer_fill(d_dense2, &t3, p, S, NCP, d_stag2, (int64_t)stag_rows,
                                     d_pool2, pool_rows, d_cur, T, b->page_size, b->row_bytes,
                                     d_status, st));
      } else if (pass == 1) {
        CHECK(gpb_compose_gather_records(d_dense2, &t3, p->d_prefix_desc, S - NCP, S,
                                         b->page_size, b->row_bytes, d_status, st));
        CHECK(gpb_compose_consume_fill(d_dense2, &t3, p, S, NCP, d_stag2, (int64_t)stag_rows,
                                       d_pool2, pool_rows, d_cur, T, b->page_size,
                                       b->row_bytes, d_status, st));
      } else {
        CHECK(gpb_compose_layer_ahead_fill(d_dense2, d_dense2, &t3, p, S, NCP, d_stag2,
                                           (int64_t)stag_rows, d_pool2, pool_rows, d_cur, T,
                                           b->page_size, b->row_bytes, d_status, st));
      }
      HCHECK(hipStreamSynchronize(st));
      if (!same_device_bytes(d_stag2, d_stag, stag_rows * RB) ||
          !same_device_bytes(d_dense2, d_dense, dense_bytes)) {
        fprintf(stderr, "%s differs from the two-call layer\n",
                pass == 0 ? "one-launch layer with fill"
                : pass == 1 ? "consume with fill" : "layer ahead with fill");
        return 14;
      }
      if (pass == 0) {
        HCHECK(hipMemcpy(d_pool3, d_pool2, pool_bytes, hipMemcpyDeviceToDevice));
      } else if (!same_device_bytes(d_pool2, d_pool3, pool_bytes)) {
        fprintf(stderr, "%s leaves another pool\n",
                pass == 1 ? "consume with fill" : "layer ahead with fill");
        return 16;
      }
    }
    HCHECK(hipFree(d_pool3));
  }

  /* fused fill into a copy of the pool */
  HCHECK(hipMemcpy(d_pool2, d_pool, pool_bytes, hipMemcpyDeviceToDevice));
  CHECK(gpb_staging_clear(d_stag2, (int64_t)(stag_rows * RB), st));
  CHECK(gpb_current_row_fill(d_stag2, (int64_t)stag_rows, p->d_staging_rows, d_pool2,
                             (int64_t)(b->n_pool_pages * PS), p->d_pool_locs, d_cur, T,
                             b->row_bytes, d_status, st));
  HCHECK(hipStreamSynchronize(st));
  if (!same_device_bytes(d_stag2, d_stag, stag_rows * RB)) {
    fprintf(stderr, "fused fill staging differs from the scatter\n");
    return 8;
  }
  int32_t *locs = malloc(4 * (size_t)T + 4);
  uint8_t *want = malloc(pool_bytes), *got = malloc(pool_bytes);
  HCHECK(hipMemcpy(locs, p->d_pool_locs, 4 * (size_t)T, hipMemcpyDeviceToHost));
  HCHECK(hipMemcpy(got, d_pool2, pool_bytes, hipMemcpyDeviceToHost));
  memcpy(want, h_pool, pool_bytes);
  for (int32_t k = 0; k < T; k++) {
    if (locs[k] < 0 || (size_t)locs[k] >= (size_t)b->n_pool_pages * PS) return 9;
    memcpy(want + (size_t)locs[k] * RB, h_cur + (size_t)k * RB, RB);
  }
  int pool_ok = memcmp(want, got, pool_bytes) == 0;
  free(locs);
  free(want);
  free(got);
  if (!pool_ok) {
    fprintf(stderr, "fused fill pool differs\n");
    return 9;
  }
  /* the split halves through the plan's records */
  HCHECK(hipMemset(d_dense2, 0xEE, dense_bytes + 16));
  CHECK(gpb_compose_gather_records(d_dense2, t, p->d_prefix_desc, S - NCP, S, b->page_size,
                                   b->row_bytes, d_status, st));
  CHECK(gpb_compose_gather_records(d_dense2, t, p->d_current_desc, NCP, S, b->page_size,
                                   b->row_bytes, d_status, st));
  HCHECK(hipStreamSynchronize(st));
  if (!same_device_bytes(d_dense2, d_dense, dense_bytes)) {
    fprintf(stderr, "record gathers differ from the one-shot gather\n");
    return 10;
  }

  /* the layer in one launch, and the consume half in one launch after the
   * prefix records, each into a cleared second staging region (the table's
   * staging entries are that region's slabs) */
  gpb_sources t2 = *t;
  for (int w = 0; w < b->n_writers; w++)
    t2.base[b->n_pool_entries + w] =
        (uint8_t *)d_stag2 + (size_t)w * b->staging_cap_pages * PS * RB;
  for (int pass = 0; pass < 4; pass++) {
    CHECK(gpb_staging_clear(d_stag2, (int64_t)(stag_rows * RB), st));
    HCHECK(hipMemsetAsync(d_dense2, 0xEE, dense_bytes + 16, st));
    if (pass == 0) {
      CHECK(gpb_compose_layer(d_dense2, &t2, p, S, NCP, d_stag2, (int64_t)stag_rows, d_cur, T,
                              b->page_size, b->row_bytes, d_status, st));
    } else if (pass == 3) {
      /* the grouped one-launch layer with a single group */
      gpb_layer_group lg = {d_dense2, &t2, d_stag2, (int64_t)stag_rows, d_cur, b->row_bytes};
      if (t2.n <= GPB_MAX_GROUP_SOURCES)
        CHECK(gpb_compose_layer_groups(&lg, 1, p, S, NCP, T, b->page_size, d_status, st));
      else
        CHECK(gpb_compose_layer(d_dense2, &t2, p, S, NCP, d_stag2, (int64_t)stag_rows, d_cur,
                                T, b->page_size, b->row_bytes, d_status, st));
    } else if (pass == 2) {
      /* this layer's consume and the "next" layer's prefix pages, here into
       * the same buffer's prefix slots through a separate pointer */
      CHECK(gpb_compose_layer_ahead(d_dense2, d_dense2, &t2, p, S, NCP, d_stag2,
                                    (int64_t)stag_rows, d_cur, T, b->page_size, b->row_bytes,
                                    d_status, st));
    } else {
      CHECK(gpb_compose_gather_records(d_dense2, &t2, p->d_prefix_desc, S - NCP, S,
                                       b->page_size, b->row_bytes, d_status, st));
      CHECK(gpb_compose_consume(d_dense2, &t2, p, S, NCP, d_stag2, (int64_t)stag_rows, d_cur,
                                T, b->page_size, b->row_bytes, d_status, st));
    }
    HCHECK(hipStreamSynchronize(st));
    if (!same_device_bytes(d_stag2, d_stag, stag_rows * RB) ||
        !same_device_bytes(d_dense2, d_dense, dense_bytes)) {
      fprintf(stderr, "%s differs from the two-call layer\n",
              pass == 0 ? "one-launch layer" : pass == 1 ? "fused consume"
              : pass == 2 ? "layer ahead" : "grouped one-launch layer");
      return 11;
    }
  }

  /* the one-launch layer with its staging in the library's static array:
   * the pool entries only, the library adds the slabs */
  {
    gpb_sources pools = *t;
    pools.n = b->n_pool_entries;
    HCHECK(hipMemsetAsync(d_dense2, 0xEE, dense_bytes + 16, st));
    CHECK(gpb_compose_layer_noalloc(d_dense2, &pools, b->n_writers, b->staging_cap_pages, p, S,
                                    NCP, d_cur, T, b->page_size, b->row_bytes, d_status, st));
    HCHECK(hipStreamSynchronize(st));
    if (!same_device_bytes(d_dense2, d_dense, dense_bytes)) {
      fprintf(stderr, "layer with static staging differs from the two-call layer\n");
      return 15;
    }
  }

  /* the scatter as one call per writer, each writer's own rows in its list
   * order into its own slab, sized on the host by gpb_writer_counts */
  {
    const int32_t W = b->n_writers;
    int32_t *counts = calloc((size_t)W, 4), *toks = malloc(4 * (size_t)T + 4);
    uint8_t *own = malloc((size_t)T * RB + 16);
    void *d_own;
    HCHECK(hipMalloc(&d_own, (size_t)T * RB + 16));
    CHECK(gpb_writer_counts(b, counts));
    HCHECK(hipMemcpy(toks, p->d_writer_tokens, 4 * (size_t)T, hipMemcpyDeviceToHost));
    for (int32_t k = 0; k < T; k++) {
      if (toks[k] < 0 || toks[k] >= T) return 12;
      memcpy(own + (size_t)k * RB, h_cur + (size_t)toks[k] * RB, RB);
    }
    if (T) HCHECK(hipMemcpy(d_own, own, (size_t)T * RB, hipMemcpyHostToDevice));
    CHECK(gpb_staging_clear(d_stag2, (int64_t)(stag_rows * RB), st));
    const size_t slab_rows = (size_t)b->staging_cap_pages * PS;
    size_t at = 0;
    for (int32_t w = 0; w < W; w++) {
      CHECK(gpb_current_row_scatter((uint8_t *)d_stag2 + (size_t)w * slab_rows * RB,
                                    (int64_t)slab_rows, p->d_writer_rows + at,
                                    (uint8_t *)d_own + at * RB, counts[w], b->row_bytes,
                                    d_status, st));
      at += (size_t)counts[w];
    }
    HCHECK(hipStreamSynchronize(st));
    int ok = at == (size_t)T && same_device_bytes(d_stag2, d_stag, stag_rows * RB);
    HCHECK(hipFree(d_own));
    free(counts);
    free(toks);
    free(own);
    if (!ok) {
      fprintf(stderr, "per-writer scatters differ from the single scatter\n");
      return 12;
    }
  }

  /* the plan build with the staging clear in its first launch: the same
   * plan, and the staging region all zeros */
  HCHECK(hipMemset(d_stag2, 0x5A, stag_rows * RB));
  CHECK(gpb_plan_build_clear(b, p, d_stag2, (int64_t)(stag_rows * RB), st));
  HCHECK(hipStreamSynchronize(st));
  {
    uint8_t *z = calloc(stag_rows * RB + 1, 1), *h = malloc(stag_rows * RB + 1);
    HCHECK(hipMemcpy(h, d_stag2, stag_rows * RB, hipMemcpyDeviceToHost));
    int zero = memcmp(z, h, stag_rows * RB) == 0;
    free(z);
    free(h);
    if (!zero) {
      fprintf(stderr, "plan build with clear left staging bytes set\n");
      return 13;
    }
  }

  int32_t status = -1;
  HCHECK(hipMemcpy(&status, d_status, 4, hipMemcpyDeviceToHost));
  if (status != 0) { fprintf(stderr, "status %d after the other entry points\n", status); return 5; }
  HCHECK(hipFree(d_dense2));
  HCHECK(hipFree(d_stag2));
  HCHECK(hipFree(d_pool2));
  printf("c consumer: slot-list and record gathers, grouped calls, fused fill, one-launch "
         "layer (single, grouped, with fill), fused consume, layer ahead, per-writer scatters and "
         "plan build with clear agree\n");
  return 0;
}

static int run(const char *in, const char *out) {
  FILE *f = fopen(in, "rb");
  if (!f) return 4;
  gpb_batch b;
  memset(&b, 0, sizeof b);
  b.bs = rd32(f); b.page_size = rd32(f); b.row_bytes = rd32(f);
  b.n_pool_pages = rd32(f); b.n_pool_entries = rd32(f); b.n_writers = rd32(f);
  b.staging_cap_pages = rd32(f);
  int32_t *P = calloc((size_t)b.bs + 1, 4), *c = calloc((size_t)b.bs + 1, 4);
  for (int r = 0; r < b.bs; r++) P[r] = rd32(f);
  for (int r = 0; r < b.bs; r++) c[r] = rd32(f);
  int32_t n_req = rd32(f);
  int32_t *req = calloc((size_t)n_req + 1, 4);
  for (int k = 0; k < n_req; k++) req[k] = rd32(f);
  b.h_prefix_pages = P; b.h_cur_tokens = c; b.h_req_pages = req;
  int32_t S, T, NCP;
  CHECK(gpb_plan_sizes(&b, &S, &T, &NCP));
  const size_t RB = (size_t)b.row_bytes, PS = (size_t)b.page_size;
  const size_t pool_bytes = (size_t)b.n_pool_pages * PS * RB;
  const size_t cur_bytes = (size_t)T * RB;
  const size_t stag_rows = (size_t)b.n_writers * b.staging_cap_pages * PS;
  uint8_t *h_pool = malloc(pool_bytes), *h_cur = malloc(cur_bytes + 1);
  if (fread(h_pool, 1, pool_bytes, f) != pool_bytes) return 4;
  if (cur_bytes && fread(h_cur, 1, cur_bytes, f) != cur_bytes) return 4;
  fclose(f);

  /* device copies of the metadata, the arenas and every plan output */
  void *d_P, *d_c, *d_req, *d_pool, *d_cur, *d_stag, *d_dense, *d_status;
  HCHECK(hipMalloc(&d_P, 4 * (size_t)b.bs + 4));
  HCHECK(hipMalloc(&d_c, 4 * (size_t)b.bs + 4));
  HCHECK(hipMalloc(&d_req, 4 * (size_t)n_req + 4));
  HCHECK(hipMalloc(&d_pool, pool_bytes));
  HCHECK(hipMalloc(&d_cur, cur_bytes + 16));
  HCHECK(hipMalloc(&d_stag, stag_rows * RB));
  HCHECK(hipMalloc(&d_dense, (size_t)S * PS * RB + 16));
  HCHECK(hipMalloc(&d_status, 4));
  HCHECK(hipMemcpy(d_P, P, 4 * (size_t)b.bs, hipMemcpyHostToDevice));
  HCHECK(hipMemcpy(d_c, c, 4 * (size_t)b.bs, hipMemcpyHostToDevice));
  HCHECK(hipMemcpy(d_req, req, 4 * (size_t)n_req, hipMemcpyHostToDevice));
  HCHECK(hipMemcpy(d_pool, h_pool, pool_bytes, hipMemcpyHostToDevice));
  if (cur_bytes) HCHECK(hipMemcpy(d_cur, h_cur, cur_bytes, hipMemcpyHostToDevice));
  HCHECK(hipMemset(d_status, 0, 4));
  b.d_prefix_pages = d_P; b.d_cur_tokens = d_c; b.d_req_pages = d_req;

  /* plan outputs in the header's order, with their sizes */
  const int64_t bs = b.bs, npp = b.n_pool_pages;
  const int64_t W = b.n_writers;
  const int64_t sizes[] = {bs, 2 * bs, 2 * bs, bs, bs, bs, bs, bs, bs, S, S, S, npp, npp,
                           NCP, T, T, T, T, 4 * bs, S - NCP, NCP, T, NCP, NCP,
                           4 * (S - NCP), 4 * (int64_t)NCP, W + 1, T, T, NCP};
  enum { NF = sizeof sizes / sizeof sizes[0] };
  int32_t *outs[NF];
  for (int k = 0; k < NF; k++) HCHECK(hipMalloc((void **)&outs[k], 4 * (size_t)sizes[k] + 4));
  gpb_plan p;
  int32_t **fields[NF] = {&p.d_slot_base, &p.d_prefix_span, &p.d_current_span, &p.d_q_lens,
                          &p.d_kv_lens, &p.d_q_starts, &p.d_k_bases, &p.d_q_bases,
                          &p.d_current_bases, &p.d_slot_pages, &p.d_owner, &p.d_src,
                          &p.d_page_inverse, &p.d_staging_page_inverse, &p.d_writer,
                          &p.d_staging_rows, &p.d_mixed_locs, &p.d_token_req,
                          &p.d_topk_offsets, &p.d_segments, &p.d_prefix_slots,
                          &p.d_current_slots, &p.d_pool_locs, &p.d_cur_page_token0,
                          &p.d_cur_page_ntok, &p.d_prefix_desc, &p.d_current_desc,
                          &p.d_writer_offsets, &p.d_writer_tokens, &p.d_writer_rows,
                          &p.d_writer_page_row0};
  for (int k = 0; k < NF; k++) *fields[k] = outs[k];
  p.d_status = d_status;

  hipStream_t st;
  HCHECK(hipStreamCreate(&st));
  CHECK(gpb_plan_build(&b, &p, st));
  CHECK(gpb_staging_clear(d_stag, (int64_t)(stag_rows * RB), st));
  CHECK(gpb_current_row_scatter(d_stag, (int64_t)stag_rows, p.d_staging_rows, d_cur, T,
                                b.row_bytes, d_status, st));
  gpb_sources t;
  memset(&t, 0, sizeof t);
  t.n = b.n_pool_entries + b.n_writers;
  for (int e = 0; e < b.n_pool_entries; e++) {
    t.base[e] = d_pool;
    t.n_pages[e] = b.n_pool_pages;
  }
  for (int w = 0; w < b.n_writers; w++) {
    t.base[b.n_pool_entries + w] = (uint8_t *)d_stag + (size_t)w * b.staging_cap_pages * PS * RB;
    t.n_pages[b.n_pool_entries + w] = b.staging_cap_pages;
  }
  CHECK(gpb_compose_gather(d_dense, &t, p.d_owner, p.d_src, S, b.page_size, b.row_bytes,
                           d_status, st));
  HCHECK(hipStreamSynchronize(st));
  int32_t status = -1;
  HCHECK(hipMemcpy(&status, d_status, 4, hipMemcpyDeviceToHost));
  if (status != 0) { fprintf(stderr, "status %d\n", status); return 5; }
  int rc = other_entry_points(&b, &p, &t, S, T, NCP, d_pool, d_cur, d_stag, d_dense,
                              h_pool, h_cur, d_status, st);
  if (rc) return rc;

  FILE *o = fopen(out, "wb");
  if (!o) return 4;
  int32_t head[3] = {S, T, NCP};
  fwrite(head, 4, 3, o);
  for (int k = 0; k < NF; k++) {
    int32_t *h = malloc(4 * (size_t)sizes[k] + 4);
    HCHECK(hipMemcpy(h, outs[k], 4 * (size_t)sizes[k], hipMemcpyDeviceToHost));
    fwrite(h, 4, (size_t)sizes[k], o);
    free(h);
  }
  uint8_t *h = malloc(stag_rows * RB + (size_t)S * PS * RB + 1);
  HCHECK(hipMemcpy(h, d_stag, stag_rows * RB, hipMemcpyDeviceToHost));
  fwrite(h, 1, stag_rows * RB, o);
  if (S) HCHECK(hipMemcpy(h, d_dense, (size_t)S * PS * RB, hipMemcpyDeviceToHost));
  fwrite(h, 1, (size_t)S * PS * RB, o);
  fclose(o);
  printf("c consumer: ran S=%d T=%d NCP=%d\n", S, T, NCP);
  return 0;
}

int main(int argc, char **argv) {
  if (argc >= 2 && strcmp(argv[1], "check") == 0) return check();
  if (argc >= 4 && strcmp(argv[1], "run") == 0) return run(argv[2], argv[3]);
  fprintf(stderr, "usage: consumer check | consumer run <in> <out>\n");
  return 1;
}
