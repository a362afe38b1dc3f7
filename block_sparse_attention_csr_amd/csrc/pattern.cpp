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
  int32_t M = 0;
  int32_t bs = 0;
  int32_t radius = 1;
  int32_t k_max = 0;
  std::vector<int32_t> globals;
};

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
  std::sort(row.begin(), row.end());
  row.erase(std::unique(row.begin(), row.end()), row.end());
}

}  // namespace

extern "C" bsa_status bsa_build_pattern(const bsa_pattern_desc* desc, int32_t* row_ptr,
                                        int32_t* col_idx, int64_t col_cap, int64_t* nnz_out) {
  if (desc == nullptr || nnz_out == nullptr) return BSA_ERR_NULL_POINTER;
  if (desc->kind != BSA_PATTERN_LOGLINEAR && desc->kind != BSA_PATTERN_BLOCK_MASK)
    return BSA_ERR_INVALID_ARGUMENT;
  if (desc->seq_len <= 0 || desc->block_size <= 0 || desc->seq_len % desc->block_size != 0)
    return BSA_ERR_SHAPE;
  const int32_t M = desc->seq_len / desc->block_size;

  Rule rule;
  if (desc->kind == BSA_PATTERN_LOGLINEAR) {
    rule.M = M;
    rule.bs = desc->block_size;
    rule.radius = desc->local_radius < 0 ? 1 : desc->local_radius;
    rule.k_max = desc->k_max < 0 ? ceil_log2_int(M) : desc->k_max;
    if (desc->num_global < 0) {
      rule.globals = {0, M / 2, M - 1};
    } else {
      if (desc->num_global > 0 && desc->global_blocks == nullptr) return BSA_ERR_NULL_POINTER;
      rule.globals.assign(desc->global_blocks, desc->global_blocks + desc->num_global);
    }
    for (int32_t g : rule.globals)
      if (g < 0 || g >= M) return BSA_ERR_INDEX_RANGE;
  } else if (desc->mask == nullptr) {
    return BSA_ERR_NULL_POINTER;
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
      } else {
        row.clear();
        const uint8_t* mrow = desc->mask + static_cast<int64_t>(i) * M;
        for (int32_t j = 0; j < M; ++j)
          if (mrow[j] != 0) row.push_back(j);
      }
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
