/*
 * bsa_c_forward.c -- libbsa's C ABI driven from plain C, with no Python in
 * the process: the pattern builder, its transpose and orders, the row-split
 * planner, and one forward launch through the HIP runtime's C API.
 *
 *   bsa_c_forward pattern N BS
 *     Host only.  Builds the log-linear pattern of [P1] section 3.1 with the
 *     built-in defaults (local radius 1, k_max = ceil(log2 M), anchors
 *     {0, M/2, M-1}), its CSC transpose, the long-first order of both, and the
 *     row-split plan with the default chunk, and prints each as one line
 *     "name v0 v1 ..." on stdout.  Then the same for a user block mask
 *     ([P1] section 2.2's local + global form): |i - j| <= 4, with blocks 0
 *     and M - 1 both global columns and dense rows, under the prefix "lg_".
 *
 *   bsa_c_forward forward IN OUT
 *     IN holds int32 B, H, N, d, BS, then float32 Q, K, V, each [B, H, N, d]
 *     row-major.  Builds the same pattern for (N, BS), copies everything to
 *     device 0, runs bsa_forward in float32 on the null stream with the
 *     default scale 1/sqrt(d), and writes float32 O [B, H, N, d] followed by
 *     float32 LSE [B, H, N] to OUT.
 *
 * Exit status 0 on success, 1 on a bad command line or file, 2 when a
 * library or HIP call fails (its name and status string go to stderr).
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "Block Sparse Attention: Log-Linear complexity sparse attention
 *       implementation" (czchanglian.com, news/56740).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "bsa.h"

#define CHECK_BSA(call)                                                              \
  do {                                                                               \
    bsa_status s_ = (call);                                                          \
    if (s_ != BSA_OK) {                                                              \
      fprintf(stderr, "%s failed: %s\n", #call, bsa_status_string((int32_t)s_));   \
      return 2;                                                                      \
    }                                                                                \
  } while (0)

#define CHECK_HIP(call)                                                              \
  do {                                                                               \
    hipError_t e_ = (call);                                                          \
    if (e_ != hipSuccess) {                                                          \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));             \
      return 2;                                                                      \
    }                                                                                \
  } while (0)

/* A CSR pattern in host memory. */
typedef struct pattern {
  int32_t M;
  int64_t nnz;
  int32_t* row_ptr; /* [M + 1] */
  int32_t* col_idx; /* [nnz] */
} pattern;

static void print_ints(const char* name, const int32_t* v, int64_t n) {
  printf("%s", name);
  for (int64_t i = 0; i < n; ++i) printf(" %d", v[i]);
  printf("\n");
}

/* The pattern `desc` selects: first ask for nnz, then fill. */
static int build(const bsa_pattern_desc* desc, pattern* p) {
  CHECK_BSA(bsa_build_pattern(desc, NULL, NULL, 0, &p->nnz)); /* validates the sizes */
  p->M = desc->seq_len / desc->block_size;
  p->row_ptr = (int32_t*)malloc(sizeof(int32_t) * ((size_t)p->M + 1));
  p->col_idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)p->nnz);
  if (!p->row_ptr || !p->col_idx) {
    fprintf(stderr, "out of host memory\n");
    return 2;
  }
  CHECK_BSA(bsa_build_pattern(desc, p->row_ptr, p->col_idx, p->nnz, &p->nnz));
  return 0;
}

/* Log-linear pattern with the built-in defaults. */
static int build_loglinear(int32_t N, int32_t bs, pattern* p) {
  bsa_pattern_desc desc;
  memset(&desc, 0, sizeof desc);
  desc.kind = BSA_PATTERN_LOGLINEAR;
  desc.seq_len = N;
  desc.block_size = bs;
  desc.local_radius = -1;
  desc.k_max = -1;
  desc.num_global = -1;
  return build(&desc, p);
}

/* Local + global block mask: band |i - j| <= 4, blocks 0 and M - 1 global. */
static int build_local_global(int32_t N, int32_t bs, pattern* p) {
  if (bs <= 0 || N <= 0 || N % bs != 0) {
    fprintf(stderr, "bad sizes N=%d bs=%d\n", N, bs);
    return 2;
  }
  const int32_t M = N / bs;
  uint8_t* mask = (uint8_t*)calloc((size_t)M * (size_t)M, 1);
  if (!mask) {
    fprintf(stderr, "out of host memory\n");
    return 2;
  }
  for (int32_t i = 0; i < M; ++i)
    for (int32_t j = 0; j < M; ++j)
      mask[(size_t)i * M + j] = (uint8_t)(abs(i - j) <= 4 || i == 0 || j == 0 || i == M - 1 ||
                                          j == M - 1);
  bsa_pattern_desc desc;
  memset(&desc, 0, sizeof desc);
  desc.kind = BSA_PATTERN_BLOCK_MASK;
  desc.seq_len = N;
  desc.block_size = bs;
  desc.mask = mask;
  const int rc = build(&desc, p);
  free(mask);
  return rc;
}

/* Prints a pattern, its transpose, both orders and its row-split plan, each
 * line's name prefixed by `prefix`. */
static int print_pattern(const char* prefix, const pattern* p) {
  const int32_t M = p->M;
  int32_t* col_ptr = (int32_t*)malloc(sizeof(int32_t) * ((size_t)M + 1));
  int32_t* row_idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)p->nnz);
  int32_t* row_order = (int32_t*)malloc(sizeof(int32_t) * (size_t)M);
  int32_t* col_order = (int32_t*)malloc(sizeof(int32_t) * (size_t)M);
  uint8_t* heavy = (uint8_t*)malloc((size_t)M);
  int32_t* items = (int32_t*)malloc(sizeof(int32_t) * 3 * (size_t)p->nnz);
  int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * 3 * (size_t)M);
  int32_t* heavy_i = (int32_t*)malloc(sizeof(int32_t) * (size_t)M);
  if (!col_ptr || !row_idx || !row_order || !col_order || !heavy || !items || !rows || !heavy_i) {
    fprintf(stderr, "out of host memory\n");
    return 2;
  }
  CHECK_BSA(bsa_transpose_pattern(M, p->row_ptr, p->col_idx, p->nnz, col_ptr, row_idx));
  CHECK_BSA(bsa_pattern_order(M, p->row_ptr, row_order));
  CHECK_BSA(bsa_pattern_order(M, col_ptr, col_order));
  int32_t n_items = 0, n_rows = 0;
  CHECK_BSA(bsa_plan_row_split(M, p->row_ptr, 0, heavy, items, (int32_t)p->nnz, &n_items, rows,
                               &n_rows));
  for (int32_t i = 0; i < M; ++i) heavy_i[i] = heavy[i];

  char name[64];
#define LINE(what, v, n)                                   \
  do {                                                     \
    snprintf(name, sizeof name, "%s%s", prefix, what);     \
    print_ints(name, v, n);                                \
  } while (0)
  printf("%sM %d\n", prefix, M);
  printf("%snnz %lld\n", prefix, (long long)p->nnz);
  LINE("row_ptr", p->row_ptr, (int64_t)M + 1);
  LINE("col_idx", p->col_idx, p->nnz);
  LINE("col_ptr", col_ptr, (int64_t)M + 1);
  LINE("row_idx", row_idx, p->nnz);
  LINE("row_order", row_order, M);
  LINE("col_order", col_order, M);
  LINE("heavy", heavy_i, M);
  LINE("items", items, 3 * (int64_t)n_items);
  LINE("split_rows", rows, 3 * (int64_t)n_rows);
#undef LINE

  free(col_ptr);
  free(row_idx);
  free(row_order);
  free(col_order);
  free(heavy);
  free(items);
  free(rows);
  free(heavy_i);
  return 0;
}

static int run_pattern(int32_t N, int32_t bs) {
  printf("abi %d\n", bsa_abi_version());
  pattern p;
  int rc = build_loglinear(N, bs, &p);
  if (rc) return rc;
  rc = print_pattern("", &p);
  free(p.row_ptr);
  free(p.col_idx);
  if (rc) return rc;
  rc = build_local_global(N, bs, &p);
  if (rc) return rc;
  rc = print_pattern("lg_", &p);
  free(p.row_ptr);
  free(p.col_idx);
  return rc;
}

static int run_forward(const char* in_path, const char* out_path) {
  FILE* f = fopen(in_path, "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", in_path);
    return 1;
  }
  int32_t hdr[5];
  if (fread(hdr, sizeof(int32_t), 5, f) != 5) {
    fprintf(stderr, "short header in %s\n", in_path);
    fclose(f);
    return 1;
  }
  const int32_t B = hdr[0], H = hdr[1], N = hdr[2], d = hdr[3], bs = hdr[4];
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0 || bs <= 0 || N % bs != 0) {
    fprintf(stderr, "bad sizes B=%d H=%d N=%d d=%d bs=%d\n", B, H, N, d, bs);
    fclose(f);
    return 1;
  }
  const size_t n_x = (size_t)B * H * N * d, n_lse = (size_t)B * H * N;
  float* host = (float*)malloc(sizeof(float) * (4 * n_x + n_lse)); /* Q, K, V, O, LSE */
  if (!host) {
    fprintf(stderr, "out of host memory\n");
    fclose(f);
    return 2;
  }
  const size_t got = fread(host, sizeof(float), 3 * n_x, f);
  fclose(f);
  if (got != 3 * n_x) {
    fprintf(stderr, "short data in %s: %zu of %zu floats\n", in_path, got, 3 * n_x);
    return 1;
  }

  pattern p;
  int rc = build_loglinear(N, bs, &p);
  if (rc) return rc;

  void *dq, *dk, *dv, *dout, *dlse, *drp, *dci;
  CHECK_HIP(hipSetDevice(0));
  CHECK_HIP(hipMalloc(&dq, sizeof(float) * n_x));
  CHECK_HIP(hipMalloc(&dk, sizeof(float) * n_x));
  CHECK_HIP(hipMalloc(&dv, sizeof(float) * n_x));
  CHECK_HIP(hipMalloc(&dout, sizeof(float) * n_x));
  CHECK_HIP(hipMalloc(&dlse, sizeof(float) * n_lse));
  CHECK_HIP(hipMalloc(&drp, sizeof(int32_t) * ((size_t)p.M + 1)));
  CHECK_HIP(hipMalloc(&dci, sizeof(int32_t) * (size_t)p.nnz));
  CHECK_HIP(hipMemcpy(dq, host, sizeof(float) * n_x, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dk, host + n_x, sizeof(float) * n_x, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dv, host + 2 * n_x, sizeof(float) * n_x, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(drp, p.row_ptr, sizeof(int32_t) * ((size_t)p.M + 1),
                      hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dci, p.col_idx, sizeof(int32_t) * (size_t)p.nnz, hipMemcpyHostToDevice));

  CHECK_BSA(bsa_forward(dq, dk, dv, dout, (float*)dlse, B, H, N, d, bs, BSA_DTYPE_F32,
                        (const int32_t*)drp, (const int32_t*)dci, p.nnz, 0.0f, NULL));
  CHECK_HIP(hipDeviceSynchronize());
  CHECK_HIP(hipMemcpy(host + 3 * n_x, dout, sizeof(float) * n_x, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(host + 4 * n_x, dlse, sizeof(float) * n_lse, hipMemcpyDeviceToHost));

  FILE* g = fopen(out_path, "wb");
  if (!g) {
    fprintf(stderr, "cannot open %s\n", out_path);
    return 1;
  }
  const size_t put = fwrite(host + 3 * n_x, sizeof(float), n_x + n_lse, g);
  if (fclose(g) != 0 || put != n_x + n_lse) {
    fprintf(stderr, "short write to %s\n", out_path);
    return 1;
  }

  CHECK_HIP(hipFree(dq));
  CHECK_HIP(hipFree(dk));
  CHECK_HIP(hipFree(dv));
  CHECK_HIP(hipFree(dout));
  CHECK_HIP(hipFree(dlse));
  CHECK_HIP(hipFree(drp));
  CHECK_HIP(hipFree(dci));
  free(p.row_ptr);
  free(p.col_idx);
  free(host);
  printf("forward B=%d H=%d N=%d d=%d bs=%d nnz=%lld ok\n", B, H, N, d, bs, (long long)p.nnz);
  return 0;
}

int main(int argc, char** argv) {
  if (argc == 4 && strcmp(argv[1], "pattern") == 0)
    return run_pattern((int32_t)atoi(argv[2]), (int32_t)atoi(argv[3]));
  if (argc == 4 && strcmp(argv[1], "forward") == 0) return run_forward(argv[2], argv[3]);
  fprintf(stderr, "usage: %s pattern N BS | %s forward IN OUT\n", argv[0], argv[0]);
  return 1;
}
