// Host-side pattern builder: block-selection rule or user mask -> CSR.
//
// The rule is that of "Block Sparse Attention: Log-Linear complexity sparse
// attention implementation" (czchanglian.com), section 3.1: for query block
// i, the local blocks i-1..i+1, the log-stride blocks i +- floor(2^k / bs) for
// k = 1..ceil(log2 M), and the global anchors {0, M/2, M-1}, all inside
// [0, M).  Section 3.2 of the same page precomputes this table on the CPU
// before the launch; it is stored here as CSR (row_ptr / col_idx) because the
// number of selected blocks differs from row to row.
//
// Further kinds: a dilated sliding window and BigBird's local + global +
// random blocks (the pattern configuration examples of the Ascend CANN
// SparseFlashAttention article; BigBird also in section 2.2 of the log-linear
// page).  The random blocks come from SplitMix64 used as a counter-based
// generator (output n of the sequence started at `seed` is mix(seed + n * g),
// g = 0x9e3779b97f4a7c15), so any row can be drawn on its own.  With
// `causal`, blocks after the query block are dropped.
//
// Each row is assembled as a short candidate list (O(log M) entries for the
// rule), sorted and deduplicated; a mask row is scanned in order.

#include "bsa.h"

#include <algorithm>
#include <cstdint>
#include <vector>

namespace {

int ceil_log2_int(int64_t m) {
  int e = 0;
  while ((int64_t{1} << e) < m) ++e;
  return e;
}

struct Rule {
  int32_t kind = BSA_PATTERN_LOGLINEAR;
  int32_t M = 0;
  int32_t bs = 0;
  int32_t radius = 1;
  int32_t k_max = 0;
  int32_t window = 0;
  int32_t dilation = 1;
  int32_t num_random = 0;
  uint64_t seed = 0;
  std::vector<int32_t> globals;
};

// Output n (n >= 1) of SplitMix64 started at state `seed`.
uint64_t splitmix64_at(uint64_t seed, uint64_t n) {
  uint64_t z = seed + n * 0x9e3779b97f4a7c15ull;
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

void sort_unique(std::vector<int32_t>& row) {
  std::sort(row.begin(), row.end());
  row.erase(std::unique(row.begin(), row.end()), row.end());
}

// Dilated window: {i + dilation * t, |t| <= window} and the globals.
void dilated_row(const Rule& r, int32_t i, std::vector<int32_t>& row) {
  row.clear();
  for (int64_t t = -int64_t{r.window}; t <= r.window; ++t) {
    const int64_t j = int64_t{i} + t * r.dilation;
    if (j >= 0 && j < r.M) row.push_back(static_cast<int32_t>(j));
  }
  for (int32_t g : r.globals) row.push_back(g);
  sort_unique(row);
}

// BigBird: local {i - r .. i + r}, the globals, then num_random new blocks:
// candidate c is splitmix64_at(seed, i * 2^32 + c + 1) mod M, skipping blocks
// already in the row, until num_random are added, the row is full or
// 64 M + 1024 candidates have been drawn.
void bigbird_row(const Rule& r, int32_t i, std::vector<int32_t>& row) {
  row.clear();
  for (int64_t j = int64_t{i} - r.radius; j <= int64_t{i} + r.radius; ++j)
    if (j >= 0 && j < r.M) row.push_back(static_cast<int32_t>(j));
  for (int32_t g : r.globals) row.push_back(g);
  sort_unique(row);
  std::vector<char> in(static_cast<size_t>(r.M), 0);
  for (int32_t j : row) in[static_cast<size_t>(j)] = 1;
  int32_t added = 0;
  int64_t have = static_cast<int64_t>(row.size());
  // At most 64 M + 1024 candidates (a bound the draw never reaches in practice:
  // it keeps the loop finite whatever the generator's residues).
  const uint64_t cap = 64 * static_cast<uint64_t>(r.M) + 1024;
  for (uint64_t c = 0; added < r.num_random && have < r.M && c < cap; ++c) {
    const uint64_t n = (static_cast<uint64_t>(i) << 32) + c + 1;
    const int32_t j = static_cast<int32_t>(splitmix64_at(r.seed, n) % static_cast<uint64_t>(r.M));
    if (in[static_cast<size_t>(j)]) continue;
    in[static_cast<size_t>(j)] = 1;
    row.push_back(j);
    ++added;
    ++have;
  }
  sort_unique(row);
}

// Candidate blocks of one query block under the log-linear rule, ascending
// and unique, written into `row` (cleared first).
void loglinear_row(const Rule& r, int32_t i, std::vector<int32_t>& row) {
  row.clear();
  auto add = [&](int64_t j) {
    if (j >= 0 && j < r.M) row.push_back(static_cast<int32_t>(j));
  };
  for (int64_t j = int64_t{i} - r.radius; j <= int64_t{i} + r.radius; ++j) add(j);
  for (int k = 1; k <= r.k_max; ++k) {
    // 2^k is a token distance; floor(2^k / bs) is the block distance.  Once
    // the block distance reaches M every further k lands outside [0, M).
    const int64_t stride = (k >= 62) ? INT64_MAX : ((int64_t{1} << k) / r.bs);
    if (stride >= r.M) break;
    add(int64_t{i} - stride);
    add(int64_t{i} + stride);
  }
  for (int32_t g : r.globals) add(g);
  sort_unique(row);
}

}  // namespace

extern "C" bsa_status bsa_build_pattern(const bsa_pattern_desc* desc, int32_t* row_ptr,
                                        int32_t* col_idx, int64_t col_cap, int64_t* nnz_out) {
  if (desc == nullptr || nnz_out == nullptr) return BSA_ERR_NULL_POINTER;
  if (desc->kind != BSA_PATTERN_LOGLINEAR && desc->kind != BSA_PATTERN_BLOCK_MASK &&
      desc->kind != BSA_PATTERN_DILATED && desc->kind != BSA_PATTERN_BIGBIRD)
    return BSA_ERR_INVALID_ARGUMENT;
  if (desc->seq_len <= 0 || desc->block_size <= 0 || desc->seq_len % desc->block_size != 0)
    return BSA_ERR_SHAPE;
  const int32_t M = desc->seq_len / desc->block_size;

  Rule rule;
  rule.kind = desc->kind;
  rule.M = M;
  rule.bs = desc->block_size;
  if (desc->kind == BSA_PATTERN_BLOCK_MASK) {
    if (desc->mask == nullptr) return BSA_ERR_NULL_POINTER;
  } else {
    rule.radius = desc->local_radius < 0 ? 1 : desc->local_radius;
    rule.k_max = desc->k_max < 0 ? ceil_log2_int(M) : desc->k_max;
    if (desc->kind == BSA_PATTERN_DILATED) {
      if (desc->window < 0 || desc->dilation < 1) return BSA_ERR_INVALID_ARGUMENT;
      rule.window = desc->window;
      rule.dilation = desc->dilation;
    }
    if (desc->kind == BSA_PATTERN_BIGBIRD) {
      if (desc->num_random < 0) return BSA_ERR_INVALID_ARGUMENT;
      rule.num_random = desc->num_random;
      rule.seed = desc->seed;
    }
    if (desc->num_global < 0) {
      if (desc->kind == BSA_PATTERN_LOGLINEAR) rule.globals = {0, M / 2, M - 1};
    } else {
      if (desc->num_global > 0 && desc->global_blocks == nullptr) return BSA_ERR_NULL_POINTER;
      rule.globals.assign(desc->global_blocks, desc->global_blocks + desc->num_global);
    }
    for (int32_t g : rule.globals)
      if (g < 0 || g >= M) return BSA_ERR_INDEX_RANGE;
  }

  // Pass 1 counts, pass 2 (when col_idx is given and large enough) fills.
  std::vector<int32_t> row;
  int64_t nnz = 0;
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
      *nnz_out = nnz;
      if (col_idx == nullptr) return BSA_OK;
      if (col_cap < nnz) return BSA_ERR_BUFFER_TOO_SMALL;
    }
    int64_t pos = 0;
    if (pass == 0 && row_ptr != nullptr) row_ptr[0] = 0;
    for (int32_t i = 0; i < M; ++i) {
      if (desc->kind == BSA_PATTERN_LOGLINEAR) {
        loglinear_row(rule, i, row);
      } else if (desc->kind == BSA_PATTERN_DILATED) {
        dilated_row(rule, i, row);
      } else if (desc->kind == BSA_PATTERN_BIGBIRD) {
        bigbird_row(rule, i, row);
      } else {
        row.clear();
        const uint8_t* mrow = desc->mask + static_cast<int64_t>(i) * M;
        for (int32_t j = 0; j < M; ++j)
          if (mrow[j] != 0) row.push_back(j);
      }
      if (desc->causal != 0)
        row.erase(std::upper_bound(row.begin(), row.end(), i), row.end());
      if (row.empty()) return BSA_ERR_EMPTY_ROW;
      if (pass == 1) std::copy(row.begin(), row.end(), col_idx + pos);
      pos += static_cast<int64_t>(row.size());
      if (pos > INT32_MAX) return BSA_ERR_SHAPE;
      if (pass == 0 && row_ptr != nullptr) row_ptr[i + 1] = static_cast<int32_t>(pos);
    }
    nnz = pos;
  }
  return BSA_OK;
}

extern "C" bsa_status bsa_transpose_pattern(int32_t M, const int32_t* row_ptr,
                                            const int32_t* col_idx, int64_t nnz,
                                            int32_t* col_ptr, int32_t* row_idx) {
  if (row_ptr == nullptr || col_ptr == nullptr || (nnz > 0 && (col_idx == nullptr ||
                                                                row_idx == nullptr)))
    return BSA_ERR_NULL_POINTER;
  if (M <= 0 || row_ptr[0] != 0 || row_ptr[M] != nnz) return BSA_ERR_SHAPE;
  for (int32_t i = 0; i < M; ++i)
    if (row_ptr[i + 1] < row_ptr[i]) return BSA_ERR_SHAPE;
  std::vector<int64_t> count(static_cast<size_t>(M) + 1, 0);
  for (int64_t t = 0; t < nnz; ++t) {
    const int32_t j = col_idx[t];
    if (j < 0 || j >= M) return BSA_ERR_INDEX_RANGE;
    ++count[static_cast<size_t>(j) + 1];
  }
  for (int32_t j = 0; j < M; ++j) count[j + 1] += count[j];
  for (int32_t j = 0; j <= M; ++j) col_ptr[j] = static_cast<int32_t>(count[j]);
  // Rows are visited in ascending order, so every column comes out ascending.
  for (int32_t i = 0; i < M; ++i)
    for (int32_t t = row_ptr[i]; t < row_ptr[i + 1]; ++t)
      row_idx[count[static_cast<size_t>(col_idx[t])]++] = i;
  return BSA_OK;
}

extern "C" bsa_status bsa_pattern_order(int32_t M, const int32_t* ptr, int32_t* order) {
  if (ptr == nullptr || order == nullptr) return BSA_ERR_NULL_POINTER;
  if (M <= 0 || ptr[0] != 0) return BSA_ERR_SHAPE;
  for (int32_t i = 0; i < M; ++i)
    if (ptr[i + 1] < ptr[i]) return BSA_ERR_SHAPE;
  // Blocks with more than twice the mean count go first, longest first; the
  // rest keep ascending order, so that neighbouring blocks (which share data)
  // still run close together.
  const int64_t total = ptr[M];
  std::vector<int32_t> longer, rest;
  for (int32_t i = 0; i < M; ++i) {
    const int64_t n = ptr[i + 1] - ptr[i];
    (n * M > 2 * total ? longer : rest).push_back(i);
  }
  std::stable_sort(longer.begin(), longer.end(), [ptr](int32_t a, int32_t b) {
    return ptr[a + 1] - ptr[a] > ptr[b + 1] - ptr[b];
  });
  int32_t k = 0;
  for (const int32_t i : longer) order[k++] = i;
  for (const int32_t i : rest) order[k++] = i;
  return BSA_OK;
}

extern "C" bsa_status bsa_plan_row_split(int32_t M, const int32_t* row_ptr, int32_t chunk,
                                         uint8_t* heavy, int32_t* items, int32_t item_cap,
                                         int32_t* n_items, int32_t* rows, int32_t* n_rows) {
  if (row_ptr == nullptr || heavy == nullptr || n_items == nullptr || rows == nullptr ||
      n_rows == nullptr || (items == nullptr && item_cap > 0))
    return BSA_ERR_NULL_POINTER;
  if (M <= 0 || row_ptr[0] != 0 || item_cap < 0) return BSA_ERR_SHAPE;
  for (int32_t i = 0; i < M; ++i)
    if (row_ptr[i + 1] < row_ptr[i]) return BSA_ERR_SHAPE;
  if (chunk <= 0) {  // about one ordinary row: the mean length, rounded up to 8
    const int64_t mean = (static_cast<int64_t>(row_ptr[M]) + M - 1) / M;
    chunk = static_cast<int32_t>(std::max<int64_t>(8, (mean + 7) / 8 * 8));
  }
  int64_t k = 0;
  int32_t h = 0;
  for (int32_t r = 0; r < M; ++r) {
    const int32_t n = row_ptr[r + 1] - row_ptr[r];
    heavy[r] = n > 2 * static_cast<int64_t>(chunk) ? 1 : 0;
    if (!heavy[r]) continue;
    const int32_t pieces = (n + chunk - 1) / chunk;
    rows[3 * h] = r;
    rows[3 * h + 1] = static_cast<int32_t>(k);
    rows[3 * h + 2] = pieces;
    ++h;
    for (int32_t i = 0; i < pieces; ++i, ++k) {
      if (k >= item_cap) continue;
      const int32_t e0 = row_ptr[r] + i * chunk;
      items[3 * k] = r;
      items[3 * k + 1] = e0;
      items[3 * k + 2] = std::min(e0 + chunk, row_ptr[r + 1]);
    }
  }
  if (k > INT32_MAX) return BSA_ERR_SHAPE;
  *n_items = static_cast<int32_t>(k);
  *n_rows = h;
  return k > item_cap ? BSA_ERR_BUFFER_TOO_SMALL : BSA_OK;
}

extern "C" const char* bsa_status_string(int32_t status) {
  switch (status) {
    case BSA_OK: return "BSA_OK";
    case BSA_ERR_NULL_POINTER: return "BSA_ERR_NULL_POINTER: a required pointer is NULL";
    case BSA_ERR_INVALID_ARGUMENT:
      return "BSA_ERR_INVALID_ARGUMENT: unknown kind/dtype or unsupported block/head size";
    case BSA_ERR_SHAPE: return "BSA_ERR_SHAPE: inconsistent or out-of-range sizes";
    case BSA_ERR_EMPTY_ROW: return "BSA_ERR_EMPTY_ROW: a query block selects no K block";
    case BSA_ERR_INDEX_RANGE: return "BSA_ERR_INDEX_RANGE: a block index outside [0, M)";
    case BSA_ERR_BUFFER_TOO_SMALL: return "BSA_ERR_BUFFER_TOO_SMALL: col_cap < nnz";
    case BSA_ERR_HIP: return "BSA_ERR_HIP: the HIP runtime reported an error";
    default: return "BSA_ERR_UNKNOWN";
  }
}

extern "C" int32_t bsa_abi_version(void) { return BSA_ABI_VERSION; }
