/*
 * pattern_sanitize.c -- the library's host pattern code (bsa_build_pattern,
 * bsa_transpose_pattern, bsa_pattern_order, bsa_plan_row_split,
 * bsa_status_string, bsa_abi_version) driven over many inputs, built with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitize.py).
 * Out-of-bounds block indices are the failure the log-linear page names
 * first among its troubleshooting cases (section 5.1); this program checks
 * that no input, valid or not, makes the host code read or write outside
 * the caller's arrays, and that every result holds its invariants:
 *
 *  - CSR rows ascend, hold no duplicate and stay in [0, M); nnz agrees;
 *  - log-linear rows hold their own block and respect the O(log M) bound;
 *  - a mask round-trips through the CSR;
 *  - the transpose of the transpose is the pattern again;
 *  - an order is a permutation;
 *  - a row-split plan covers each heavy row's entries once, in order.
 *
 * Arrays are allocated to exactly the documented sizes, so that a write one
 * past their end is a sanitizer error.  Prints "ok <cases>" and exits 0, or
 * names the failing case and exits 1.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "bsa.h"

static int failures = 0;
static long cases = 0;

#define EXPECT(cond, ...)                        \
  do {                                           \
    if (!(cond)) {                               \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);              \
      fprintf(stderr, "\n");                     \
      ++failures;                                \
    }                                            \
  } while (0)

static uint64_t rng_state = 0x243f6a8885a308d3ull;
static uint32_t rnd(void) { /* xorshift64*, a test input source only */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545f4914f6cdd1dull) >> 32);
}

static bsa_pattern_desc base_desc(int32_t kind, int32_t N, int32_t bs) {
  bsa_pattern_desc d;
  memset(&d, 0, sizeof d);
  d.kind = kind;
  d.seq_len = N;
  d.block_size = bs;
  d.local_radius = -1;
  d.k_max = -1;
  d.num_global = -1;
  d.dilation = 1;
  return d;
}

/* Builds a pattern into exactly sized arrays; returns the status, and on
   BSA_OK the CSR (caller frees). */
static bsa_status build(const bsa_pattern_desc* d, int32_t** rp, int32_t** ci, int64_t* nnz) {
  *rp = NULL;
  *ci = NULL;
  int64_t n = -1;
  bsa_status s = bsa_build_pattern(d, NULL, NULL, 0, &n);
  ++cases;
  if (s != BSA_OK) return s;
  const int32_t M = d->seq_len / d->block_size;
  int32_t* r = (int32_t*)malloc(sizeof(int32_t) * (size_t)(M + 1));
  int32_t* c = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  int64_t n2 = -1;
  s = bsa_build_pattern(d, r, c, n, &n2);
  EXPECT(s == BSA_OK && n2 == n, "second build: status %d nnz %lld vs %lld", (int)s,
         (long long)n2, (long long)n);
  if (n > 0) {  /* one entry short: refused, nnz still reported */
    int32_t* small = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    int64_t n3 = -1;
    bsa_status s3 = bsa_build_pattern(d, r, small, n - 1, &n3);
    EXPECT(s3 == BSA_ERR_BUFFER_TOO_SMALL && n3 == n, "short col_cap: status %d", (int)s3);
    free(small);
    /* the first call above may have written row_ptr; rebuild */
    s = bsa_build_pattern(d, r, c, n, &n2);
  }
  *rp = r;
  *ci = c;
  *nnz = n;
  return s;
}

static void check_csr(int32_t M, const int32_t* rp, const int32_t* ci, int64_t nnz,
                      const char* what) {
  EXPECT(rp[0] == 0 && rp[M] == nnz, "%s: row_ptr ends %d %d nnz %lld", what, rp[0], rp[M],
         (long long)nnz);
  for (int32_t i = 0; i < M; ++i) {
    EXPECT(rp[i] <= rp[i + 1], "%s: row_ptr decreases at %d", what, i);
    for (int32_t t = rp[i]; t < rp[i + 1]; ++t) {
      EXPECT(ci[t] >= 0 && ci[t] < M, "%s: entry %d of row %d = %d", what, t, i, ci[t]);
      if (t > rp[i]) EXPECT(ci[t - 1] < ci[t], "%s: row %d not ascending", what, i);
    }
  }
}

static void check_transpose_and_orders(int32_t M, const int32_t* rp, const int32_t* ci,
                                       int64_t nnz, const char* what) {
  int32_t* cp = (int32_t*)malloc(sizeof(int32_t) * (size_t)(M + 1));
  int32_t* ri = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1));
  int32_t* rp2 = (int32_t*)malloc(sizeof(int32_t) * (size_t)(M + 1));
  int32_t* ci2 = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1));
  int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)M);
  int32_t* seen = (int32_t*)calloc((size_t)M, sizeof(int32_t));
  ++cases;
  bsa_status s = bsa_transpose_pattern(M, rp, ci, nnz, cp, ri);
  EXPECT(s == BSA_OK, "%s: transpose status %d", what, (int)s);
  if (s == BSA_OK) {
    check_csr(M, cp, ri, nnz, what);
    s = bsa_transpose_pattern(M, cp, ri, nnz, rp2, ci2);
    EXPECT(s == BSA_OK, "%s: transpose twice status %d", what, (int)s);
    EXPECT(memcmp(rp, rp2, sizeof(int32_t) * (size_t)(M + 1)) == 0 &&
               memcmp(ci, ci2, sizeof(int32_t) * (size_t)nnz) == 0,
           "%s: transpose of the transpose differs", what);
    for (int pass = 0; pass < 2; ++pass) {
      memset(seen, 0, sizeof(int32_t) * (size_t)M);
      s = bsa_pattern_order(M, pass == 0 ? rp : cp, order);
      EXPECT(s == BSA_OK, "%s: order status %d", what, (int)s);
      for (int32_t i = 0; i < M && s == BSA_OK; ++i) {
        EXPECT(order[i] >= 0 && order[i] < M && !seen[order[i]], "%s: order not a permutation",
               what);
        if (order[i] >= 0 && order[i] < M) seen[order[i]] = 1;
      }
    }
  }
  free(cp); free(ri); free(rp2); free(ci2); free(order); free(seen);
}

static void check_split(int32_t M, const int32_t* rp, int64_t nnz, int32_t chunk,
                        const char* what) {
  const int32_t cap = (int32_t)(nnz > 0 ? nnz : 1);
  uint8_t* heavy = (uint8_t*)malloc((size_t)M);
  int32_t* items = (int32_t*)malloc(sizeof(int32_t) * 3 * (size_t)cap);
  int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * 3 * (size_t)M);
  int32_t n_items = -1, n_rows = -1;
  ++cases;
  bsa_status s = bsa_plan_row_split(M, rp, chunk, heavy, items, cap, &n_items, rows, &n_rows);
  EXPECT(s == BSA_OK, "%s: plan status %d (chunk %d)", what, (int)s, chunk);
  if (s == BSA_OK) {
    int32_t heavy_count = 0;
    for (int32_t i = 0; i < M; ++i) heavy_count += heavy[i] != 0;
    EXPECT(heavy_count == n_rows, "%s: %d heavy flags, %d rows", what, heavy_count, n_rows);
    for (int32_t h = 0; h < n_rows; ++h) {
      const int32_t row = rows[3 * h], first = rows[3 * h + 1], count = rows[3 * h + 2];
      EXPECT(row >= 0 && row < M && heavy[row], "%s: heavy row %d", what, row);
      EXPECT(first >= 0 && count >= 1 && first + count <= n_items, "%s: item range", what);
      int32_t expect = rp[row];
      for (int32_t k = first; k < first + count && k < n_items && k >= 0; ++k) {
        EXPECT(items[3 * k] == row && items[3 * k + 1] == expect && items[3 * k + 2] > expect,
               "%s: item %d of row %d", what, k, row);
        expect = items[3 * k + 2];
      }
      EXPECT(expect == rp[row + 1], "%s: row %d not covered", what, row);
    }
    if (n_items > 0) {  /* too little item room: refused */
      int32_t n2 = -1, r2 = -1;
      bsa_status s2 = bsa_plan_row_split(M, rp, chunk, heavy, items, n_items - 1, &n2, rows, &r2);
      EXPECT(s2 == BSA_ERR_BUFFER_TOO_SMALL, "%s: short item room status %d", what, (int)s2);
    }
  }
  free(heavy); free(items); free(rows);
}

static void check_all(const bsa_pattern_desc* d, const char* what) {
  int32_t *rp, *ci;
  int64_t nnz;
  bsa_status s = build(d, &rp, &ci, &nnz);
  EXPECT(s == BSA_OK, "%s: build status %d", what, (int)s);
  if (s == BSA_OK) {
    const int32_t M = d->seq_len / d->block_size;
    check_csr(M, rp, ci, nnz, what);
    if (d->kind == BSA_PATTERN_LOGLINEAR && d->local_radius < 0 && d->k_max < 0 &&
        d->num_global < 0 && !d->causal) {
      int lg = 0;
      while ((1 << lg) < M) ++lg;
      int lbs = 0;
      while ((1 << lbs) < d->block_size) ++lbs;
      const int ns = lg - lbs + 1 > 0 ? lg - lbs + 1 : 0;
      const int bound = 6 + 2 * (ns > 1 ? ns - 1 : 0);
      for (int32_t i = 0; i < M; ++i) {
        int own = 0;
        for (int32_t t = rp[i]; t < rp[i + 1]; ++t) own |= ci[t] == i;
        EXPECT(own, "%s: row %d lacks its own block", what, i);
        EXPECT(rp[i + 1] - rp[i] <= bound, "%s: row %d has %d > %d", what, i, rp[i + 1] - rp[i],
               bound);
      }
    }
    check_transpose_and_orders(M, rp, ci, nnz, what);
    const int32_t chunks[] = {0, 1, 2, 3, 5, 16, 1000};
    for (unsigned k = 0; k < sizeof chunks / sizeof chunks[0]; ++k) check_split(M, rp, nnz, chunks[k], what);
  }
  free(rp);
  free(ci);
}

int main(void) {
  char what[128];
  /* log-linear: every (N, bs) with M up to 4096, defaults and variants */
  const int32_t sizes[] = {1, 2, 3, 4, 5, 7, 8, 16, 31, 64, 127, 128, 512, 1000, 4096};
  const int32_t blocks[] = {1, 16, 32, 64, 128};
  for (unsigned a = 0; a < sizeof sizes / sizeof sizes[0]; ++a)
    for (unsigned b = 0; b < sizeof blocks / sizeof blocks[0]; ++b) {
      bsa_pattern_desc d = base_desc(BSA_PATTERN_LOGLINEAR, sizes[a] * blocks[b], blocks[b]);
      snprintf(what, sizeof what, "loglinear M=%d bs=%d", sizes[a], blocks[b]);
      check_all(&d, what);
      d.causal = 1;
      check_all(&d, what);
      d.causal = 0;
      d.local_radius = (int32_t)(rnd() % 4);
      d.k_max = (int32_t)(rnd() % 14);
      int32_t g[7];
      d.num_global = (int32_t)(rnd() % 8);
      for (int k = 0; k < d.num_global; ++k) g[k] = (int32_t)(rnd() % (uint32_t)sizes[a]);
      d.global_blocks = g;
      check_all(&d, what);
    }
  /* dilated and BigBird */
  for (int rep = 0; rep < 200; ++rep) {
    const int32_t M = 1 + (int32_t)(rnd() % 300), bs = 1 << (rnd() % 7);
    bsa_pattern_desc d = base_desc(BSA_PATTERN_DILATED, M * bs, bs);
    d.window = (int32_t)(rnd() % 6);
    d.dilation = 1 + (int32_t)(rnd() % 5);
    d.causal = (int32_t)(rnd() % 2);
    snprintf(what, sizeof what, "dilated M=%d w=%d dil=%d", M, d.window, d.dilation);
    check_all(&d, what);
    bsa_pattern_desc e = base_desc(BSA_PATTERN_BIGBIRD, M * bs, bs);
    e.local_radius = (int32_t)(rnd() % 3);
    e.num_random = (int32_t)(rnd() % (uint32_t)(M + 5));
    e.seed = ((uint64_t)rnd() << 32) | rnd();
    e.causal = (int32_t)(rnd() % 2);
    int32_t g[2] = {0, M - 1};
    e.num_global = (int32_t)(rnd() % 3);
    e.global_blocks = g;
    snprintf(what, sizeof what, "bigbird M=%d r=%d R=%d", M, e.local_radius, e.num_random);
    check_all(&e, what);
  }
  /* masks: random densities with the diagonal on, and their round trip */
  for (int rep = 0; rep < 200; ++rep) {
    const int32_t M = 1 + (int32_t)(rnd() % 200), bs = 1 << (rnd() % 7);
    uint8_t* mask = (uint8_t*)malloc((size_t)M * (size_t)M);
    const uint32_t p = rnd() % 101;
    for (int32_t i = 0; i < M; ++i)
      for (int32_t j = 0; j < M; ++j) mask[i * M + j] = (uint8_t)(i == j || rnd() % 100 < p ? 1 + rnd() % 255 : 0);
    bsa_pattern_desc d = base_desc(BSA_PATTERN_BLOCK_MASK, M * bs, bs);
    d.mask = mask;
    d.causal = (int32_t)(rnd() % 2);
    snprintf(what, sizeof what, "mask M=%d p=%u", M, p);
    check_all(&d, what);
    int32_t *rp, *ci;
    int64_t nnz;
    d.causal = 0;
    if (build(&d, &rp, &ci, &nnz) == BSA_OK) {
      int64_t pop = 0;
      for (int64_t k = 0; k < (int64_t)M * M; ++k) pop += mask[k] != 0;
      EXPECT(pop == nnz, "%s: nnz %lld popcount %lld", what, (long long)nnz, (long long)pop);
      for (int32_t i = 0; i < M; ++i)
        for (int32_t t = rp[i]; t < rp[i + 1]; ++t) EXPECT(mask[i * M + ci[t]] != 0, "%s", what);
    }
    free(rp);
    free(ci);
    /* an empty row is refused */
    const int32_t row = (int32_t)(rnd() % (uint32_t)M);
    memset(mask + (size_t)row * M, 0, (size_t)M);
    int64_t n = 0;
    ++cases;
    EXPECT(bsa_build_pattern(&d, NULL, NULL, 0, &n) == BSA_ERR_EMPTY_ROW, "%s: empty row", what);
    free(mask);
  }
  /* refused descriptors */
  {
    int64_t n = 0;
    bsa_pattern_desc d = base_desc(BSA_PATTERN_LOGLINEAR, 4096, 32);
    ++cases;
    EXPECT(bsa_build_pattern(NULL, NULL, NULL, 0, &n) == BSA_ERR_NULL_POINTER, "null desc");
    EXPECT(bsa_build_pattern(&d, NULL, NULL, 0, NULL) == BSA_ERR_NULL_POINTER, "null nnz_out");
    bsa_pattern_desc e = d;
    e.seq_len = 4095;
    EXPECT(bsa_build_pattern(&e, NULL, NULL, 0, &n) == BSA_ERR_SHAPE, "indivisible");
    e = d;
    e.block_size = 0;
    EXPECT(bsa_build_pattern(&e, NULL, NULL, 0, &n) == BSA_ERR_SHAPE, "zero block");
    e = d;
    e.seq_len = -64;
    EXPECT(bsa_build_pattern(&e, NULL, NULL, 0, &n) == BSA_ERR_SHAPE, "negative length");
    e = d;
    e.kind = 99;
    EXPECT(bsa_build_pattern(&e, NULL, NULL, 0, &n) == BSA_ERR_INVALID_ARGUMENT, "kind");
    int32_t g[2] = {0, 128};
    e = d;
    e.num_global = 2;
    e.global_blocks = g;
    EXPECT(bsa_build_pattern(&e, NULL, NULL, 0, &n) == BSA_ERR_INDEX_RANGE, "global range");
    e.global_blocks = NULL;
    EXPECT(bsa_build_pattern(&e, NULL, NULL, 0, &n) == BSA_ERR_NULL_POINTER, "null globals");
    e = base_desc(BSA_PATTERN_BLOCK_MASK, 4096, 32);
    EXPECT(bsa_build_pattern(&e, NULL, NULL, 0, &n) == BSA_ERR_NULL_POINTER, "null mask");
    e = base_desc(BSA_PATTERN_DILATED, 4096, 32);
    e.dilation = 0;
    EXPECT(bsa_build_pattern(&e, NULL, NULL, 0, &n) == BSA_ERR_INVALID_ARGUMENT, "dilation");
    e.dilation = 1;
    e.window = -1;
    EXPECT(bsa_build_pattern(&e, NULL, NULL, 0, &n) == BSA_ERR_INVALID_ARGUMENT, "window");
    e = base_desc(BSA_PATTERN_BIGBIRD, 4096, 32);
    e.num_random = -1;
    EXPECT(bsa_build_pattern(&e, NULL, NULL, 0, &n) == BSA_ERR_INVALID_ARGUMENT, "num_random");
  }
  /* refused CSR inputs of the transpose, the orders and the planner */
  {
    int32_t rp[4] = {0, 2, 1, 3}, ci[3] = {0, 1, 2}, cp[4], ri[3], order[3];
    uint8_t heavy[3];
    int32_t items[9], rows[9], ni, nr;
    ++cases;
    EXPECT(bsa_transpose_pattern(3, rp, ci, 3, cp, ri) == BSA_ERR_SHAPE, "decreasing row_ptr");
    int32_t rp_ok[4] = {0, 1, 2, 3}, ci_bad[3] = {0, 3, 1};
    EXPECT(bsa_transpose_pattern(3, rp_ok, ci_bad, 3, cp, ri) == BSA_ERR_INDEX_RANGE, "range");
    int32_t ci_neg[3] = {0, -1, 1};
    EXPECT(bsa_transpose_pattern(3, rp_ok, ci_neg, 3, cp, ri) == BSA_ERR_INDEX_RANGE, "negative");
    EXPECT(bsa_transpose_pattern(3, rp_ok, ci, 2, cp, ri) == BSA_ERR_SHAPE, "nnz mismatch");
    EXPECT(bsa_transpose_pattern(0, rp_ok, ci, 3, cp, ri) == BSA_ERR_SHAPE, "M = 0");
    EXPECT(bsa_transpose_pattern(3, NULL, ci, 3, cp, ri) == BSA_ERR_NULL_POINTER, "null");
    EXPECT(bsa_pattern_order(3, rp, order) != BSA_OK, "order of decreasing row_ptr");
    EXPECT(bsa_pattern_order(3, NULL, order) == BSA_ERR_NULL_POINTER, "order null");
    EXPECT(bsa_plan_row_split(3, rp, 1, heavy, items, 3, &ni, rows, &nr) != BSA_OK,
           "plan of decreasing row_ptr");
    EXPECT(bsa_plan_row_split(3, rp_ok, 1, heavy, items, -1, &ni, rows, &nr) != BSA_OK,
           "negative item room");
  }
  for (int32_t code = -3; code < 12; ++code) {
    const char* t = bsa_status_string(code);
    EXPECT(t != NULL && strncmp(t, "BSA_", 4) == 0, "status string %d", code);
  }
  EXPECT(bsa_abi_version() == BSA_ABI_VERSION, "abi version");
  if (failures) {
    fprintf(stderr, "%d failures in %ld cases\n", failures, cases);
    return 1;
  }
  printf("ok %ld\n", cases);
  return 0;
}
