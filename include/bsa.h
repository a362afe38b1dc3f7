/*
 * bsa.h -- block-sparse attention forward for AMD Instinct MI355X (gfx950).
 *
 * Plain C ABI.  All pointers are raw host or device pointers (stated per
 * argument); no framework types cross this boundary.  Every entry point
 * returns a bsa_status; none aborts or throws.
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "Block Sparse Attention: Log-Linear complexity sparse attention
 *       implementation" (czchanglian.com, news/56740).
 *  [P2] "How to implement efficient sparse attention for the 4090: from
 *       principle to engineering practice" (qqiyuan.cn).
 *  [P3] Ascend CANN SparseFlashAttention article (hwcomputing.csdn.net).
 */
#ifndef BSA_H_
#define BSA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Values are stable. */
typedef enum bsa_status {
  BSA_OK = 0,
  BSA_ERR_NULL_POINTER = 1,     /* a required pointer is NULL */
  BSA_ERR_INVALID_ARGUMENT = 2, /* unknown kind/dtype, unsupported block or head size */
  BSA_ERR_SHAPE = 3,            /* sizes <= 0, seq_len % block_size != 0, nnz inconsistent,
                                   or a size that overflows the index types */
  BSA_ERR_EMPTY_ROW = 4,        /* a query block selects no K block */
  BSA_ERR_INDEX_RANGE = 5,      /* a global block outside [0, M) */
  BSA_ERR_BUFFER_TOO_SMALL = 6, /* col_cap < nnz; *nnz_out still holds nnz */
  BSA_ERR_HIP = 7               /* the HIP runtime reported an error at launch */
} bsa_status;

typedef enum bsa_pattern_kind {
  BSA_PATTERN_LOGLINEAR = 0,  /* built-in log-linear rule, [P1] section 3.1 */
  BSA_PATTERN_BLOCK_MASK = 1, /* user [M, M] block mask, [P2] item 1, [P3] "Block-Sparse" */
  BSA_PATTERN_DILATED = 2,    /* dilated sliding window, [P3] pattern configuration examples */
  BSA_PATTERN_BIGBIRD = 3     /* local + global + random blocks, [P1] section 2.2, [P3] same */
} bsa_pattern_kind;

typedef enum bsa_dtype {
  BSA_DTYPE_F32 = 0,  /* IEEE binary32 Q/K/V/O */
  BSA_DTYPE_BF16 = 1  /* bfloat16 Q/K/V/O, float32 accumulation */
} bsa_dtype;

/*
 * Pattern descriptor (host memory, read only during the call).
 *
 * Notation of [P1] section 3.1: N = seq_len, bs = block_size, M = N / bs,
 * query block i ("row_i").  Every kind keeps only blocks in [0, M).
 *
 * BSA_PATTERN_LOGLINEAR selects, for every query block i,
 *   local      {i - r, ..., i + r}                 r = local_radius
 *   log-stride {i - floor(2^k / bs), i + floor(2^k / bs)}  k = 1 .. k_max
 *   global     the global blocks (default {0, M/2, M-1})
 * [P1] section 3.1 prints r = 1, k_max = ceil(log2 M) and the anchors
 * {0, M/2, M-1} (worked example N = 4096, bs = 32, M = 128, k = 1..7, anchors
 * {0, 64, 127}); the anchors are added as columns of every row, and anchor
 * rows are not made dense.  [P1] section 6.1's seven anchors are a
 * seven-entry global_blocks list.
 *
 * BSA_PATTERN_BLOCK_MASK selects block j for query block i iff
 * mask[i * M + j] != 0.
 *
 * BSA_PATTERN_DILATED selects {i + dilation * t : t = -window .. window} and
 * the global blocks (default: none).
 *
 * BSA_PATTERN_BIGBIRD selects the local blocks {i - r .. i + r}, the global
 * blocks (default: none) and num_random further blocks drawn for row i:
 * candidate c = 0, 1, 2, ... is block x_c mod M, where x_c is output number
 * (i * 2^32 + c + 1) of SplitMix64 started at state `seed` (state advances by
 * 0x9e3779b97f4a7c15; output mixes with the shifts 30, 27, 31 and the
 * multipliers 0xbf58476d1ce4e5b9, 0x94d049bb133111eb); candidates already in
 * the row are skipped, and the draw stops after num_random new blocks, when
 * the row holds all M blocks, or after 64 M + 1024 candidates.  Global
 * blocks are columns only.
 *
 * causal != 0 then drops every block j > i from row i (the diagonal block
 * stays; inside it the causal forward masks the later keys).
 */
typedef struct bsa_pattern_desc {
  int32_t kind;                 /* bsa_pattern_kind */
  int32_t seq_len;              /* N > 0, multiple of block_size */
  int32_t block_size;           /* bs > 0 */
  int32_t local_radius;         /* LOGLINEAR, BIGBIRD: r >= 0; < 0 selects the default 1 */
  int32_t k_max;                /* LOGLINEAR: >= 0; < 0 selects ceil(log2 M) */
  int32_t num_global;           /* < 0 selects the kind's default global blocks;
                                   >= 0 uses global_blocks[0 .. num_global) */
  const int32_t* global_blocks; /* host array, each in [0, M) */
  const uint8_t* mask;          /* BLOCK_MASK: host array, M * M bytes, row-major */
  int32_t causal;               /* != 0: keep only blocks j <= i */
  int32_t window;               /* DILATED: window >= 0 (in steps of `dilation`) */
  int32_t dilation;             /* DILATED: dilation >= 1 */
  int32_t num_random;           /* BIGBIRD: random blocks per row, >= 0 */
  uint64_t seed;                /* BIGBIRD: generator seed */
} bsa_pattern_desc;

/*
 * bsa_build_pattern -- selected K blocks of every query block, as CSR.
 *
 * The per-query-block index table of [P1] section 3.2 (built on the CPU
 * before launch), encoded as CSR because rows differ in length:
 *   row_ptr[0] = 0, row_ptr[i + 1] = row_ptr[i] + |S(i)|,
 *   col_idx[row_ptr[i] .. row_ptr[i + 1]) = S(i) in ascending order, unique.
 *
 * desc     host; required.
 * row_ptr  host, caller-owned int32[M + 1]; may be NULL (not written).
 * col_idx  host, caller-owned int32[col_cap]; may be NULL to query nnz only.
 * col_cap  capacity of col_idx in elements (ignored when col_idx is NULL).
 * nnz_out  host; required; receives nnz = sum_i |S(i)| on BSA_OK and on
 *          BSA_ERR_BUFFER_TOO_SMALL.
 *
 * Errors: BSA_ERR_NULL_POINTER (desc, nnz_out, or mask for BLOCK_MASK, or
 * global_blocks when num_global > 0), BSA_ERR_INVALID_ARGUMENT (unknown kind,
 * window < 0, dilation < 1, num_random < 0),
 * BSA_ERR_SHAPE (sizes, divisibility, nnz > INT32_MAX), BSA_ERR_INDEX_RANGE
 * (global block outside [0, M)), BSA_ERR_EMPTY_ROW (a mask row with no block;
 * [P1] section 5.1 traces NaN outputs to such rows), BSA_ERR_BUFFER_TOO_SMALL.
 * On error nothing is guaranteed about row_ptr / col_idx contents.
 *
 * Host only, synchronous, deterministic, thread-safe (no global state).
 */
bsa_status bsa_build_pattern(const bsa_pattern_desc* desc, int32_t* row_ptr, int32_t* col_idx,
                             int64_t col_cap, int64_t* nnz_out);

/*
 * bsa_forward -- block-sparse attention forward, one fused kernel launch.
 *
 * For every batch b, head h and query block qb, over the key positions of the
 * K blocks S(qb) = col_idx[row_ptr[qb] .. row_ptr[qb + 1]):
 *   O[b,h,r,:] = sum_j softmax_j(scale * Q[b,h,r,:] . K[b,h,j,:]) V[b,h,j,:]
 *   LSE[b,h,r] = ln sum_j exp(scale * Q[b,h,r,:] . K[b,h,j,:])
 * with the softmax normalised over exactly the selected positions
 * ([P3] "the O(N^2) bottleneck of long sequences" for the formula, [P1]
 * section 3.3 for the normalisation over the connected blocks only).
 * Every block of S(qb) is attended in full (non-causal).
 *
 * q, k, v  device, caller-owned, contiguous [batch, heads, seq_len, head_dim]
 *          of `dtype`, 16-byte aligned.
 * o        device, caller-owned, same shape and dtype; written.
 * lse      device, caller-owned float32 [batch, heads, seq_len]; written.
 *          May be NULL when the log-sum-exp is not wanted.
 * row_ptr, col_idx  device copies of bsa_build_pattern's output for
 *          (seq_len, block_size); one pattern serves every batch and head.
 *          col_idx entries outside [0, M) are skipped by the kernel.
 * nnz      row_ptr[M] (host copy); must satisfy M <= nnz <= M * M.
 * scale    > 0 multiplies the scores; <= 0 selects 1 / sqrt(head_dim)
 *          ([P3] "full call flow").
 * stream   a hipStream_t, or NULL for the null stream.  The launch is
 *          enqueued and the call returns without synchronising.
 *
 * Supported: dtype BF16 or F32; block_size 32 or 64; head_dim 64 or 128.
 * All arguments are validated on the host before any HIP call; errors are
 * BSA_ERR_NULL_POINTER, BSA_ERR_INVALID_ARGUMENT, BSA_ERR_SHAPE, and
 * BSA_ERR_HIP when the launch itself fails.  NaN/Inf inputs propagate.
 */
bsa_status bsa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
                       int32_t batch, int32_t heads, int32_t seq_len, int32_t head_dim,
                       int32_t block_size, int32_t dtype, const int32_t* row_ptr,
                       const int32_t* col_idx, int64_t nnz, float scale, void* stream);

/* Flags of bsa_forward_ex. */
typedef enum bsa_forward_flags {
  /* Causal: query row r sees only keys at positions <= r.  Pattern blocks
   * j > i are skipped, the diagonal block is masked inside.  Every row must
   * reach its own block (bsa_build_pattern with causal set keeps it whenever
   * the row selects it).  A row with no visible key gets O = 0 and
   * LSE = -inf. */
  BSA_FORWARD_CAUSAL = 1,
  /* One pattern per head: row_ptr holds heads * (M + 1) entries, head h's
   * rows at row_ptr[h * (M + 1) ..], each an offset into the one col_idx
   * array (nnz entries in all); every batch uses the same per-head patterns. */
  BSA_FORWARD_PATTERN_PER_HEAD = 2
} bsa_forward_flags;

/*
 * bsa_forward_ex -- bsa_forward with flags and an explicit workgroup shape.
 *
 * Same computation, arguments and errors as bsa_forward, plus:
 * flags      a bitwise OR of bsa_forward_flags (0: exactly bsa_forward);
 * group      query blocks sharing one workgroup's K/V tiles: 1, 2 or 4;
 * key_split  wave sets that split each query block's CSR row (>= 1), merged
 *            through LDS before the store;
 * group == key_split == 0 selects the shape bsa_forward would use.  A shape
 * needing more than 8 waves (block_size / 32 * group * key_split) or more
 * LDS than a workgroup may use returns BSA_ERR_INVALID_ARGUMENT, as do
 * unknown flags.  With BSA_FORWARD_PATTERN_PER_HEAD, nnz is the total over
 * the heads and must satisfy heads * M <= nnz <= heads * M * M.  Every shape
 * computes the same result up to floating-point summation order.
 */
bsa_status bsa_forward_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                          int32_t batch, int32_t heads, int32_t seq_len, int32_t head_dim,
                          int32_t block_size, int32_t dtype, const int32_t* row_ptr,
                          const int32_t* col_idx, int64_t nnz, float scale, int32_t flags,
                          int32_t group, int32_t key_split, void* stream);

/*
 * bsa_plan_row_split -- a plan that splits the long rows of a CSR pattern
 * across workgroups.  A banded pattern's global rows ([P3] local+global:
 * the first and last query blocks select every block) are ten times longer
 * than the others; walked by one workgroup each they end up alone at the end
 * of the grid.  A row is heavy when it has more than 2 * chunk entries; its
 * entries are cut, in order, into ceil(n / chunk) items of at most `chunk`.
 *
 * M         blocks (> 0).
 * row_ptr   host int32[M + 1]: row_ptr of bsa_build_pattern (non-decreasing
 *           from 0).
 * chunk     entries per item (> 0), or <= 0 for about one ordinary row: the
 *           mean row length rounded up to a multiple of 8, at least 8.
 * heavy     host, caller-owned uint8[M]; written: 1 for a heavy row, else 0.
 * items     host, caller-owned int32[3 * item_cap]; written: (row, first
 *           entry, end entry) per item, entries as offsets into col_idx.
 * item_cap  items' capacity in items (>= 0; nnz always suffices).
 * n_items   host; required; receives the number of items (also when it
 *           exceeds item_cap, with BSA_ERR_BUFFER_TOO_SMALL).
 * rows      host, caller-owned int32[3 * M]; written: (row, first item, item
 *           count) per heavy row.
 * n_rows    host; required; receives the number of heavy rows.
 * Errors: BSA_ERR_NULL_POINTER, BSA_ERR_SHAPE (M <= 0, row_ptr not
 * non-decreasing from 0, item_cap < 0), BSA_ERR_BUFFER_TOO_SMALL.  Host only,
 * synchronous.
 */
bsa_status bsa_plan_row_split(int32_t M, const int32_t* row_ptr, int32_t chunk, uint8_t* heavy,
                              int32_t* items, int32_t item_cap, int32_t* n_items, int32_t* rows,
                              int32_t* n_rows);

/* Bytes of device workspace bsa_forward_split needs for n_items items: one
 * float32 partial (O, m, l) per (batch, head, item, 32-row wave).  -1 for
 * invalid arguments. */
int64_t bsa_row_split_workspace_bytes(int32_t batch, int32_t heads, int32_t block_size,
                                      int32_t head_dim, int32_t n_items);

/*
 * bsa_forward_split -- bsa_forward_ex (automatic shape) with the heavy rows of
 * a bsa_plan_row_split plan spread over workgroups.  Same result as
 * bsa_forward_ex up to floating-point summation order.  Three launches on
 * `stream`: the forward over every other row; the plan's items, one
 * one-block workgroup each, writing partial states to `workspace`; and a
 * merge that combines each heavy row's partials as the online softmax
 * combines two key ranges, then writes its O and LSE.  The
 * call enqueues and returns without synchronising.
 *
 * Arguments as bsa_forward_ex (flags: BSA_FORWARD_CAUSAL only; one pattern
 * for every head), plus device copies of the plan:
 * heavy     device uint8[M]; items device int32[3 * n_items]; rows device
 *           int32[3 * n_rows] -- from bsa_plan_row_split of the same row_ptr
 *           (the kernels read them as given).  n_items == 0 runs bsa_forward.
 * workspace device, caller-owned, 16-byte aligned, at least
 *           bsa_row_split_workspace_bytes(batch, heads, block_size,
 *           head_dim, n_items) bytes; its contents on entry do not matter.
 * Errors: those of bsa_forward_ex; BSA_ERR_INVALID_ARGUMENT for the per-head
 * flag; BSA_ERR_SHAPE for inconsistent counts; BSA_ERR_BUFFER_TOO_SMALL for
 * a short workspace.  Calls that share a workspace must not overlap.
 */
bsa_status bsa_forward_split(const void* q, const void* k, const void* v, void* o, float* lse,
                             int32_t batch, int32_t heads, int32_t seq_len, int32_t head_dim,
                             int32_t block_size, int32_t dtype, const int32_t* row_ptr,
                             const int32_t* col_idx, int64_t nnz, float scale, int32_t flags,
                             const uint8_t* heavy, const int32_t* items, int32_t n_items,
                             const int32_t* rows, int32_t n_rows, void* workspace,
                             int64_t workspace_bytes, void* stream);

/*
 * bsa_transpose_pattern -- the CSC (column-major) form of a CSR pattern.
 *
 * For every K block j, the query blocks whose rows select it, ascending:
 *   col_ptr[0] = 0, col_ptr[j + 1] = col_ptr[j] + |{i : j in S(i)}|,
 *   row_idx[col_ptr[j] .. col_ptr[j + 1]) = those i.
 * The backward's dK/dV kernel walks these columns.
 *
 * M        blocks per sequence (> 0).
 * row_ptr  host int32[M + 1], col_idx host int32[nnz]: a pattern as
 *          bsa_build_pattern returns it (entries in [0, M)).
 * col_ptr  host, caller-owned int32[M + 1]; row_idx host int32[nnz].
 * Errors: BSA_ERR_NULL_POINTER, BSA_ERR_SHAPE (M <= 0, nnz != row_ptr[M],
 * row_ptr not non-decreasing from 0), BSA_ERR_INDEX_RANGE (an entry outside
 * [0, M)).  Host only, synchronous.
 */
bsa_status bsa_transpose_pattern(int32_t M, const int32_t* row_ptr, const int32_t* col_idx,
                                 int64_t nnz, int32_t* col_ptr, int32_t* row_idx);

/*
 * bsa_backward -- gradients of bsa_forward: dQ, dK, dV.
 *
 * With P the softmax of bsa_forward (recomputed from its LSE), O its output
 * and dO the gradient of a loss with respect to O:
 *   dV = P^T dO,  dP = dO V^T,  D_r = dO_r . O_r,  dS = P * (dP - D),
 *   dQ = scale dS K,  dK = scale dS^T Q.
 * (The log-linear page's section 5.3 backward without its gradient
 * compensation heuristic.)
 *
 * q, k, v, o, dout  device, [batch, heads, seq_len, head_dim] of `dtype`,
 *          16-byte aligned: the forward's inputs, its output and dO.
 * lse      device float32 [batch, heads, seq_len]: the forward's LSE.
 * dq, dk, dv  device, caller-owned, same shape and dtype; written.
 * delta    device, caller-owned float32 [batch, heads, seq_len]: workspace
 *          (receives D).
 * row_ptr, col_idx  device copies of the forward's CSR pattern;
 * col_ptr, row_idx  device copies of its bsa_transpose_pattern.  With
 *          BSA_FORWARD_PATTERN_PER_HEAD both are [heads, M + 1] offsets into
 *          one index array each (head h's CSC the transpose of head h's CSR).
 * row_order, col_order  device int32[M] or NULL: bsa_pattern_order of the
 *          CSR (row_ptr) and of the CSC (col_ptr).  With them each kernel
 *          starts its long blocks first (the anchors' columns and dense rows
 *          hold every block; started last they would run alone at the end);
 *          NULL takes blocks in ascending order.  The result is the same
 *          either way.  An order must be a permutation of 0 .. M-1 (the
 *          kernels read it as given).  Both NULL with one pattern per head.
 * nnz      the pattern's entry count (host).
 * scale    as for bsa_forward (<= 0: 1 / sqrt(head_dim)).
 * flags    0, BSA_FORWARD_CAUSAL (the forward's causal masking) and/or
 *          BSA_FORWARD_PATTERN_PER_HEAD (one pattern per head, as for
 *          bsa_forward_ex).
 * stream   a hipStream_t or NULL; two launches are enqueued (dQ and D,
 *          then dK and dV), without synchronising.
 *
 * Supported: dtype BF16 or F32, block_size 32 or 64, head_dim 64 or 128.
 * Errors as for bsa_forward; unknown flags, and orders with
 * BSA_FORWARD_PATTERN_PER_HEAD, are BSA_ERR_INVALID_ARGUMENT.
 */
bsa_status bsa_backward(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        float* delta, int32_t batch, int32_t heads, int32_t seq_len,
                        int32_t head_dim, int32_t block_size, int32_t dtype,
                        const int32_t* row_ptr, const int32_t* col_idx, const int32_t* col_ptr,
                        const int32_t* row_idx, const int32_t* row_order,
                        const int32_t* col_order, int64_t nnz, float scale, int32_t flags,
                        void* stream);

/*
 * bsa_pattern_order -- a work order for the blocks of a CSR (or CSC)
 * pattern: order[0 .. M) is a permutation of 0 .. M-1 that lists first the
 * blocks whose entry count ptr[i + 1] - ptr[i] exceeds twice the mean
 * (ptr[M] / M), by descending count (equal counts in ascending i), then all
 * other blocks in ascending i.  The work-ordering input of bsa_backward: the
 * few long blocks (anchors' columns, dense rows) start first, while the rest
 * keep the order in which neighbours share their data.
 *
 * M      blocks (> 0).
 * ptr    host int32[M + 1]: row_ptr of bsa_build_pattern or col_ptr of
 *        bsa_transpose_pattern (non-decreasing from 0).
 * order  host, caller-owned int32[M]; written.
 * Errors: BSA_ERR_NULL_POINTER, BSA_ERR_SHAPE (M <= 0, ptr[0] != 0, ptr
 * decreasing).  Host only, synchronous.
 */
bsa_status bsa_pattern_order(int32_t M, const int32_t* ptr, int32_t* order);

/*
 * bsa_forward_int8kv -- bsa_forward on int8 K and V with one scale per block.
 *
 * The log-linear page's section 6.3 keeps K and V in int8 with one scale per
 * block and computes attention in 16-bit floating point.  This is the
 * forward of bsa_forward_ex with K_p = k_codes[p] * k_scales[p / bs] and
 * V_p = v_codes[p] * v_scales[p / bs] (per batch and head), as
 * bsa_quantize_kv writes them.  The codes convert exactly to bf16 on the way
 * into the matrix cores; the K scale multiplies the scores and the V scale
 * the softmax weights of its block, so the arithmetic is that of the bf16
 * forward on the dequantised values.  K and V move half the bytes of bf16.
 *
 * q, o, lse  as for bsa_forward, bf16 (q and o) only.
 * k_codes, v_codes    device int8 [batch, heads, seq_len, head_dim],
 *            16-byte aligned.
 * k_scales, v_scales  device float32 [batch, heads, seq_len / block_size].
 * row_ptr, col_idx, nnz, scale  as for bsa_forward.
 * flags      0, BSA_FORWARD_CAUSAL and/or BSA_FORWARD_PATTERN_PER_HEAD.
 * group, key_split   0, 0 (the library chooses) or a workgroup shape, as for
 *            bsa_forward_ex.
 * Errors as for bsa_forward_ex; NULL scales: BSA_ERR_NULL_POINTER.
 */
bsa_status bsa_forward_int8kv(const void* q, const int8_t* k_codes, const float* k_scales,
                              const int8_t* v_codes, const float* v_scales, void* o, float* lse,
                              int32_t batch, int32_t heads, int32_t seq_len, int32_t head_dim,
                              int32_t block_size, const int32_t* row_ptr, const int32_t* col_idx,
                              int64_t nnz, float scale, int32_t flags, int32_t group,
                              int32_t key_split, void* stream);

/*
 * bsa_backward_noalloc -- bsa_backward without the caller's delta workspace,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, computation and results as bsa_backward, minus `delta`:
 * D (one float per query row, batch * heads * seq_len of them) goes to a
 * scratch array the library's code object holds in device memory, 16 MiB
 * per GPU (bsa_backward_noalloc_max_rows() = 4194304 rows), kept until the
 * process ends.  The call allocates nothing: no hipMalloc, no hipFree.  Its
 * first call on a device looks up that device's scratch address once.
 * Every call on one GPU shares that GPU's scratch, so calls that overlap on
 * one GPU (other streams, other host threads) race and must be ordered by
 * the caller; D is written in full before it is read, so nothing needs
 * clearing between calls.
 * Errors: as bsa_backward, plus BSA_ERR_BUFFER_TOO_SMALL when
 * batch * heads * seq_len exceeds the scratch, and BSA_ERR_HIP when the
 * scratch address cannot be looked up.
 */
bsa_status bsa_backward_noalloc(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                int32_t batch, int32_t heads, int32_t seq_len, int32_t head_dim,
                                int32_t block_size, int32_t dtype, const int32_t* row_ptr,
                                const int32_t* col_idx, const int32_t* col_ptr,
                                const int32_t* row_idx, const int32_t* row_order,
                                const int32_t* col_order, int64_t nnz, float scale, int32_t flags,
                                void* stream);

/* Query rows (batch * heads * seq_len) the scratch of bsa_backward_noalloc holds. */
int64_t bsa_backward_noalloc_max_rows(void);

/*
 * bsa_decode -- one new token per sequence against a block-aligned KV cache.
 *
 * The KV cache of sequence b holds L_b = seqlens[b] tokens; the new token is
 * the last of them, at position t = L_b - 1 in query block i = t / block_size
 * (its K and V are already in the cache).  Its output is row t of the causal
 * bsa_forward: softmax(scale q . K_p) V_p over the cached positions p <= t
 * whose block the pattern row S(i) selects (the log-linear page, section 3.3:
 * the softmax runs over the connected blocks only; its section 1 puts the
 * method's gains at inference, in the KV cache and in latency).
 *
 * q        device, [batch, heads, head_dim] of `dtype`, 16-byte aligned.
 * k_cache, v_cache  device, [batch, heads, cache_len, head_dim] of `dtype`,
 *          16-byte aligned; positions >= L_b are never read into the result
 *          (they may hold anything).
 * o        device, caller-owned [batch, heads, head_dim] of `dtype`; written.
 * lse      device float32 [batch, heads] (natural-log log-sum-exp of the
 *          scaled visible scores), or NULL.
 * cache_len  capacity N_cap of the cache, a multiple of block_size; the
 *          pattern has M = cache_len / block_size rows.
 * seqlens  device int32[batch].  A length outside [1, cache_len] (which the
 *          host cannot check without synchronising) gives O = 0 and
 *          LSE = -inf for that sequence, as does a token that sees no
 *          position (its block selects neither itself nor an earlier block).
 * row_ptr, col_idx, nnz  a pattern of M rows as for bsa_forward (entries
 *          j > i are skipped: decoding is causal).
 * scale    <= 0 selects 1 / sqrt(head_dim).
 * flags    0 or BSA_FORWARD_PATTERN_PER_HEAD (row_ptr [heads, M + 1]).
 * stream   a hipStream_t or NULL; one launch, not synchronised.
 *
 * Supported: dtype BF16 or F32, block_size 32 or 64, head_dim 64 or 128.
 * Errors as for bsa_forward; unknown flags are BSA_ERR_INVALID_ARGUMENT.
 */
bsa_status bsa_decode(const void* q, const void* k_cache, const void* v_cache, void* o,
                      float* lse, int32_t batch, int32_t heads, int32_t cache_len,
                      int32_t head_dim, int32_t block_size, int32_t dtype,
                      const int32_t* seqlens, const int32_t* row_ptr, const int32_t* col_idx,
                      int64_t nnz, float scale, int32_t flags, void* stream);

/*
 * bsa_quantize_kv -- int8 codes and one scale per block of a K or V tensor.
 *
 * The log-linear page's section 6.3 keeps the KV cache in int8 with one
 * scale per block and computes attention in 16-bit floating point.  The
 * quantiser here is symmetric, per (batch, head, block of block_size
 * positions) over all head_dim features, every decision in float32:
 *   scale = max|x| / 127,  code = clamp(rint(x / scale), -127, 127)
 * (correctly rounded divisions, ties to even; an all-zero block gets scale 0
 * and codes 0).  Values are code * scale.
 *
 * x       device [batch, heads, seq_len, head_dim] of `dtype`, finite,
 *         16-byte aligned.
 * codes   device, caller-owned int8 [batch, heads, seq_len, head_dim],
 *         16-byte aligned; written.
 * scales  device, caller-owned float32 [batch, heads, seq_len / block_size];
 *         written.
 * Supported: dtype BF16 or F32, block_size 32 or 64, head_dim 64 or 128.
 * One launch on `stream`, not synchronised.  Errors as for bsa_forward.
 */
bsa_status bsa_quantize_kv(const void* x, int8_t* codes, float* scales, int32_t batch,
                           int32_t heads, int32_t seq_len, int32_t head_dim, int32_t block_size,
                           int32_t dtype, void* stream);

/*
 * bsa_decode_int8kv -- bsa_decode on an int8 KV cache with per-block scales.
 *
 * Same computation as bsa_decode with K_p = k_codes[p] * k_scales[p / bs]
 * and V_p = v_codes[p] * v_scales[p / bs] (per batch and head), as written by
 * bsa_quantize_kv.  The codes convert exactly; the K scale multiplies the
 * scores and the V scale the softmax weights (section 6.3 of the log-linear
 * page: int8 storage, floating-point attention).
 *
 * q, o, lse, seqlens, row_ptr, col_idx, nnz, scale, flags, stream: as for
 *          bsa_decode (`dtype` is q's and o's type).
 * k_codes, v_codes    device int8 [batch, heads, cache_len, head_dim],
 *          16-byte aligned.
 * k_scales, v_scales  device float32 [batch, heads, cache_len / block_size].
 * Errors as for bsa_decode (NULL scales: BSA_ERR_NULL_POINTER).
 */
bsa_status bsa_decode_int8kv(const void* q, const int8_t* k_codes, const float* k_scales,
                             const int8_t* v_codes, const float* v_scales, void* o, float* lse,
                             int32_t batch, int32_t heads, int32_t cache_len, int32_t head_dim,
                             int32_t block_size, int32_t dtype, const int32_t* seqlens,
                             const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                             float scale, int32_t flags, void* stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char* bsa_status_string(int32_t status);

/* ABI version of this header: bump on any incompatible change. */
#define BSA_ABI_VERSION 4
int32_t bsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H_ */
