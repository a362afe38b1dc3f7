// Block-sparse attention backward for gfx950 (MI355X): dQ, dK, dV.
//
// The gradient of the forward in forward.hip: softmax(scale Q K^T) V over the
// selected blocks (Ascend CANN SparseFlashAttention article,
// hwcomputing.csdn.net, "the O(N^2) bottleneck of long sequences"), with the
// normalisation over the connected blocks only ("Block Sparse Attention:
// Log-Linear complexity sparse attention implementation", czchanglian.com,
// section 3.3).  That page's section 5.3 takes the backward as its next
// step; its gradient-compensation heuristic is not applied here.  With P recomputed from the saved log-sum-exp,
//   dV = P^T dO,  dP = dO V^T,  D_r = dO_r . O_r,  dS = P * (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// Two kernels with 32 rows per wave, both streaming tiles through an LDS ring
// with direct-to-LDS copies:
//  * bsa_bwd_dq: per query block (or per group of four at block 32 on a large
//    grid), walks its CSR row (the K blocks it selects); K and V tiles in the
//    ring.  It also writes D for its rows.
//    S^T = K Q^T and dP^T = V dO^T keep one query per lane, so P and dS are
//    per-lane arithmetic; dQ^T += K^T dS^T reads K transposed from LDS.
//  * bsa_bwd_dkv: per key block, walks its CSC column (the query blocks that
//    select it); Q, dO, LSE and D tiles in the ring.  S = Q K^T and
//    dP = dO V^T keep one key per lane; dV^T += dO^T P and dK^T += Q^T dS read
//    dO and Q transposed from LDS.
// Each output element is written once; no atomics.
//
// Work per block is uneven (the log-linear anchors' columns, and dense rows
// of banded masks, hold every block), so with an order array the long blocks
// of each XCD's heads are taken first (largest processing time first): a
// long block then never starts near the end of the grid.

#include <hip/hip_runtime.h>

#include <atomic>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "bsa.h"
#include "mfma_tiles.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // D = rowsum(dO * O), written by bsa_bwd_dq, read by bsa_bwd_dkv
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const int32_t* col_ptr;
  const int32_t* row_idx;
  const int32_t* row_order;  // query blocks, most entries first (or NULL: ascending)
  const int32_t* col_order;  // key blocks, most entries first (or NULL: ascending)
  int32_t M;
  int32_t N;
  int32_t num_wg;  // workgroups of the launch: batch * heads * ceil(M / blocks per workgroup)
  int32_t heads;
  int32_t ptr_stride;  // row_ptr / col_ptr entries per head: M + 1 (one pattern per head) or 0
  float scale;
  float scale_log2;
};

// (batch*head, group) of a workgroup: group k holds the G blocks
// order[kG .. kG + G) (or kG .. kG + G without an order array; blocks past M
// are absent).  Workgroup ids run XCD by XCD (each XCD one contiguous range
// of HX heads, so one head's blocks share an L2).  With an order array
// (bsa_pattern_order: the long blocks -- more than twice the mean entry
// count -- first, then the rest ascending), a range starts with the groups
// that hold long blocks, for all its heads, then takes the rest head by head.
__device__ __forceinline__ void group_of(int wg, int M, int G, int num_wg, const int32_t* order,
                                         const int32_t* ptr, int& bh, int& grp) {
  const int NG = (M + G - 1) / G;
  if (order == nullptr) {
    grp = wg % NG;
    bh = wg / NG;
    return;
  }
  // Number of long blocks: the leading entries of `order` whose count exceeds
  // twice the mean (the same test the host applies).  The lanes test 64
  // entries at once (two dependent loads, where a bisection took two per
  // step); the first chunk that holds a short block ends the prefix.
  const int64_t total = ptr[M];
  const int lane = threadIdx.x & (kWave - 1);
  int lo = 0;
  for (int k0 = 0; k0 < M; k0 += kWave) {
    const int k = k0 + lane;
    bool is_long = false;
    if (k < M) {
      const int b = order[k];
      is_long = (int64_t)(ptr[b + 1] - ptr[b]) * M > 2 * total;
    }
    const uint64_t longs = __builtin_amdgcn_ballot_w64(is_long);
    lo += __builtin_popcountll(longs);
    if (longs != ~0ull) break;
  }
  const int nlong = (lo + G - 1) / G;  // groups holding a long block
  const int bhs = num_wg / NG;
  const int hx = (bhs + kNumXcd - 1) / kNumXcd;
  const int gidx = wg / (hx * NG);
  const int r = wg % (hx * NG);
  const int nh = bhs - gidx * hx < hx ? bhs - gidx * hx : hx;
  if (r < nlong * nh) {  // long groups, rank by rank over the range's heads
    bh = gidx * hx + r % nh;
    grp = r / nh;
  } else {               // the rest, head by head
    const int rr = r - nlong * nh;
    bh = gidx * hx + rr / (NG - nlong);
    grp = nlong + rr % (NG - nlong);
  }
}

// Block g of group grp, or -1 past the last block.
__device__ __forceinline__ int group_block(int grp, int g, int G, int M, const int32_t* order) {
  const int k = grp * G + g;
  return k >= M ? -1 : order != nullptr ? order[k] : k;
}

// The union of a workgroup's G lists (G > 1), ascending, built in LDS:
// bitmap[0, MW) marks the union and bitmap[(1 + g) MW, ...) block g's own
// list (with the causal bound applied: dir < 0 keeps j <= blk, dir > 0 keeps
// j >= blk).  The block's `loader` wave marks its entries; wave 0 then writes
// the union into `list`.  Returns the union's size.  `first` is idx[s + lane]
// (for s + lane < e), which the loader read before its operand loads: the
// vector-memory counter drains in order, so a load issued after them would
// wait for all of them.
template <int G>
__device__ int build_union(const int32_t* idx, int s, int e, int first, bool loader, int g,
                           int blk, int dir, int M, int32_t* list, uint32_t* bitmap,
                           int32_t* size, int lane, int wave) {
  const int MW = (M + 31) / 32;
  for (int i = threadIdx.x; i < (G + 1) * MW; i += blockDim.x) bitmap[i] = 0;
  __syncthreads();
  if (loader) {
    for (int t = s + lane; t < e; t += kWave) {
      const int j = t < s + kWave ? first : idx[t];
      if (j >= 0 && j < M && (dir == 0 || (dir < 0 ? j <= blk : j >= blk))) {
        atomicOr(&bitmap[j >> 5], 1u << (j & 31));
        atomicOr(&bitmap[(1 + g) * MW + (j >> 5)], 1u << (j & 31));
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    int base = 0;
    for (int w0 = 0; w0 < MW; w0 += kWave) {
      const int w = w0 + lane;
      uint32_t bits = w < MW ? bitmap[w] : 0u;
      const int cnt = __builtin_popcount(bits);
      int incl = cnt;
      for (int off = 1; off < kWave; off <<= 1) {
        const int t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
      }
      int pos = base + incl - cnt;
      while (bits != 0u) {
        list[pos++] = w * 32 + __builtin_ctz(bits);
        bits &= bits - 1;
      }
      base += __shfl(incl, kWave - 1);
    }
    if (lane == 0) *size = base;
  }
  __syncthreads();
  return uniform(*size);
}

// Dynamic LDS of a G-block workgroup: the union list (M ints) and G + 1
// bitmaps; none for one block.
inline size_t union_lds_bytes(int G, int M) {
  return G == 1 ? 0 : 4 * ((size_t)M + (size_t)(G + 1) * ((M + 31) / 32));
}

// Ring depth and copy split of a backward kernel whose stage holds two tiles
// of BS rows (plus `extra` bytes), for G blocks per workgroup.  One wave per
// workgroup (block 32, G = 1) keeps a two-stage ring: half the LDS of three
// stages lets more of those one-wave workgroups share a CU (5% faster at the
// worked example's B = 32).  Otherwise three stages within 48 KB, else two
// (four stages measured 3% slower at B = 32: the steps are not waiting on
// their copies).
template <typename T, int BS, int D, int kExtraBytes, int G = 1>
struct BwdCfg {
  using L = TileLayout<T, BS, D>;
  static constexpr int QW = BS / kQRows;  // waves per block
  static constexpr int W = G * QW;
  static constexpr int kStage = L::kEntryBytes + kExtraBytes;
  static constexpr int NB = W == 1 ? 2 : 3 * kStage <= 48 * 1024 ? 3 : 2;
  static_assert(NB <= 4, "the kernels handle rings of up to four stages");
  static_assert(L::kCopies % W == 0, "stage copies must split evenly over the waves");
  static constexpr int kParts = L::kCopies / W;
  // the epilogue stages each wave's 32 rows (D features) through the ring
  static constexpr int kRowsStage = kQRows * D * (int)sizeof(T);
  static constexpr int kPerBuf = kStage / kRowsStage;
  static_assert(kPerBuf >= 1 && W <= NB * kPerBuf, "output stages fit the ring");
};

// Per-lane dot product of two row operands (the lane's features of one row);
// halves_sum completes the row.
template <typename T, int D>
__device__ __forceinline__ float operand_dot(const typename Ops<T>::template QOperand<D>& a,
                                             const typename Ops<T>::template QOperand<D>& b) {
  float s = 0.f;
  if constexpr (std::is_same<T, __bf16>::value) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = a.r[c][w], y = b.r[c][w];
        s = fmaf(__uint_as_float(x << 16), __uint_as_float(y << 16), s);
        s = fmaf(__uint_as_float(x & 0xffff0000u), __uint_as_float(y & 0xffff0000u), s);
      }
  } else {
#pragma unroll
    for (int c = 0; c < D / 8; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) s = fmaf(a.r[c][e], b.r[c][e], s);
  }
  return s;
}

// The two score tiles of a step, a from the stage's first tile with operand
// qa and b from its second tile with qb: interleaved MFMA chains for bf16
// with block 64 or d = 128 (backward of the long workload 11% faster; at
// block 32 and d = 64 the plain order measured 1% faster).
template <typename T, int BS, int D>
__device__ __forceinline__ void score_pair(const typename Ops<T>::template QOperand<D>& qa,
                                           const typename Ops<T>::template QOperand<D>& qb,
                                           const typename Ops<T>::template Offsets<BS, D>& off,
                                           LDS_PTR(unsigned char) tile, int st, f32x16_t& a,
                                           f32x16_t& b) {
  using L = TileLayout<T, BS, D>;
  if constexpr (std::is_same<T, __bf16>::value && (BS == 64 || D == 128)) {
    Ops<T>::template scores_pair<BS, D>(qa, qb, off, tile, 0, L::kTileBytes, st, a, b);
  } else {
    a = Ops<T>::template scores<BS, D>(qa, off, tile, 0, st);
    b = Ops<T>::template scores<BS, D>(qb, off, tile, L::kTileBytes, st);
  }
}

// A workgroup's list (CSR row or CSC column): each wave reads it from the
// index array itself, 64 entries at a time, one per lane.  The first 64 are
// loaded before the operand loads: the vector-memory counter drains in
// order, so loaded after the operands the first copies would wait for all of
// them.  Later chunks (lists longer than 64 entries) are loaded when reached.
struct ListHead {
  int start, n, first;
};
__device__ __forceinline__ ListHead list_head(const int32_t* idx, int start, int end, int lane) {
  ListHead h{start, end - start, -1};
  if (lane < h.n) h.first = idx[start + lane];
  return h;
}

// ---------------------------------------------------------------- dQ (and D)
// G query blocks per workgroup (G > 1): they share each K/V stage of the
// union of their rows; a wave computes the entries its own row selects.
// bf16, block 32, d = 64, four blocks per workgroup: held to 128 VGPRs (from
// 130), so four waves per SIMD instead of three (the B = 32 worked example's
// dQ kernel 12% faster).
template <typename T, int BS, int D, int G, bool CAUSAL>
__global__ __launch_bounds__((kWave * BwdCfg<T, BS, D, 0, G>::W))
__attribute__((amdgpu_waves_per_eu(std::is_same<T, __bf16>::value && BS == 32 && D == 64 && G == 4 ? 4 : 1)))
void bsa_bwd_dq(BwdParams p) {
  using C = BwdCfg<T, BS, D, 0, G>;
  using L = typename C::L;
  using O = Ops<T>;
  constexpr int NB = C::NB;
  constexpr int KSTEPS = BS / kKeyStep;

  __shared__ __attribute__((aligned(16))) unsigned char buf0[C::kStage];
  __shared__ __attribute__((aligned(16))) unsigned char buf1[C::kStage];
  __shared__ __attribute__((aligned(16))) unsigned char buf2[NB >= 3 ? C::kStage : 16];
  __shared__ __attribute__((aligned(16))) unsigned char buf3[NB >= 4 ? C::kStage : 16];
  extern __shared__ __attribute__((aligned(16))) int32_t dyn[];  // (G > 1) union list | bitmaps
  __shared__ int32_t union_size;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(threadIdx.x / kWave);
  const int qg = wave % C::QW;  // 32-row query group of the block
  const int g = wave / C::QW;   // block of the workgroup
  const int M = p.M;
  int bh, grp;
  group_of(xcd_remap(blockIdx.x, p.num_wg), M, G, p.num_wg, p.row_order, p.row_ptr, bh, grp);
  const int blk = group_block(grp, g, G, M, p.row_order);
  const bool has = blk >= 0;
  const int qb = has ? blk : 0;
  const int32_t* const row_ptr = p.row_ptr + (size_t)(bh % p.heads) * p.ptr_stride;
  const size_t head = (size_t)bh * p.N * D;
  const T* K = static_cast<const T*>(p.k) + head;
  const T* V = static_cast<const T*>(p.v) + head;
  const int q0 = qb * BS + qg * kQRows;
  const int row = q0 + (lane & 31);

  ListHead lh{0, 0, -1};
  int U;
  const uint32_t* my_bits = reinterpret_cast<const uint32_t*>(dyn + M) + (1 + g) * ((M + 31) / 32);
  // The list's first entries, then the operand loads, whose latency the
  // union build and the first copies overlap.
  const int rs = has ? row_ptr[qb] : 0, re = has ? row_ptr[qb + 1] : 0;
  int first = -1;
  if constexpr (G == 1) {
    lh = list_head(p.col_idx, rs, re, lane);
    U = lh.n;
  } else {
    if (has && qg == 0 && lane < re - rs) first = p.col_idx[rs + lane];
  }
  typename O::template QOperand<D> qop, dop, oop;
  O::template load_q<D>(qop, static_cast<const T*>(p.q) + head + (size_t)q0 * D, lane);
  O::template load_q<D>(dop, static_cast<const T*>(p.dout) + head + (size_t)q0 * D, lane);
  O::template load_q<D>(oop, static_cast<const T*>(p.o) + head + (size_t)q0 * D, lane);
  const float lse_raw = p.lse[(size_t)bh * p.N + row];
  if constexpr (G > 1)
    U = build_union<G>(p.col_idx, rs, re, first, has && qg == 0, g, qb, CAUSAL ? -1 : 0, M, dyn,
                       reinterpret_cast<uint32_t*>(dyn + M), &union_size, lane, wave);
  float lse2 = 0.f, dsum = 0.f;  // set once the operand loads have landed

  int chunk_base = -kWave, chunk = -1;
  uint64_t chunk_sel = 0;
  auto entry_at = [&](int t, bool& use) -> int {
    if (t >= U) {
      use = false;
      return -1;
    }
    if ((t & ~(kWave - 1)) != chunk_base) {
      chunk_base = t & ~(kWave - 1);
      const int idx = chunk_base + lane;
      bool sel;
      if constexpr (G == 1) {
        chunk = chunk_base == 0 ? lh.first : idx < U ? p.col_idx[lh.start + idx] : -1;
        sel = chunk >= 0 && chunk < M && (!CAUSAL || chunk <= qb);
      } else {  // the union holds only selected, in-range blocks
        chunk = idx < U ? dyn[idx] : -1;
        const int cj = chunk < 0 ? 0 : chunk;
        sel = has && chunk >= 0 && ((my_bits[cj >> 5] >> (cj & 31)) & 1u) != 0;
      }
      chunk_sel = __builtin_amdgcn_ballot_w64(sel);
    }
    use = ((chunk_sel >> (t - chunk_base)) & 1ull) != 0;
    return __builtin_amdgcn_readlane(chunk, t - chunk_base);
  };

  constexpr int kPartsPerTile = L::kCopies / 2;
  // One-wave workgroups copy every part of a stage, in runs of kRun behind
  // one M0 write (within one tile; dma_off carries the run's immediate offset
  // taken off).  Several waves interleave their parts: wave w copies parts
  // w, w + W, ..., one copy per M0 write (at block 64 and d = 128, the long
  // workload's backward ran 3.7% slower with each wave copying a whole tile).
  constexpr int kRun = C::W == 1 ? dma_run(C::kParts, kPartsPerTile) : 1;
  auto part_of = [&](int c) { return C::W == 1 ? c : wave + c * C::W; };
  uint32_t dma_off[C::kParts];
#pragma unroll
  for (int c = 0; c < C::kParts; ++c) {
    const int part = part_of(c) % kPartsPerTile;
    const int slot = part * kWave + lane;
    const int r = slot / L::kChunksPerRow;
    dma_off[c] = (uint32_t)(r * L::kRowBytes + (((slot % L::kChunksPerRow) ^ L::swz(r)) << 4) -
                            (c % kRun) * kWave * 16);
  }
  auto issue = [&](int j, unsigned char* buf) {
    const size_t key0 = (size_t)((uint32_t)j < (uint32_t)M ? (uint32_t)j : 0u) * BS;
    const uint32_t dst = (uint32_t)(uintptr_t)(LDS_PTR(unsigned char))buf;
#pragma unroll
    for (int r = 0; r < C::kParts / kRun; ++r) {
      const int part = part_of(r * kRun);
      uint32_t v[kRun];
#pragma unroll
      for (int k = 0; k < kRun; ++k) v[k] = dma_off[r * kRun + k];
      lds_dma16_run<kRun>((part < kPartsPerTile ? K : V) + key0 * D, v, dst + part * kWave * 16);
    }
  };

  typename O::template Offsets<BS, D> off;
  off.init(lane, 0);
  f32x16_t dq[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dq[dt] = f32x16_t{};
  const float c2 = p.scale_log2;

  auto compute = [&](unsigned char* buf, bool diag) {
    LDS_PTR(unsigned char) tile = (LDS_PTR(unsigned char))buf;
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) {
      if (diag && st > qg) continue;
      f32x16_t s, dp;  // S^T = K Q^T and dP^T = V dO^T, lane = query
      score_pair<T, BS, D>(qop, dop, off, tile, st, s, dp);
      if (diag && st == qg) {
        const int h = lane >> 5;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r / 4) + 4 * h + (r % 4) > (lane & 31)) s[r] = -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = fast_exp2(fmaf(s[r], c2, -lse2));  // P^T
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = s[r] * (dp[r] - dsum);  // dS^T
      (void)O::template accumulate<BS, D>(dq, s, off, tile, -L::kTileBytes, st);  // K^T dS^T
    }
  };

  int jq[NB];
  bool mq[NB];
#pragma unroll
  for (int e = 0; e < NB; ++e) jq[e] = entry_at(e, mq[e]);
  auto buffer = [&](auto b_c) -> unsigned char* {
    constexpr int b = decltype(b_c)::value;
    if constexpr (b == 0) return buf0;
    else if constexpr (b == 1) return buf1;
    else if constexpr (b == 2) return buf2;
    else return buf3;
  };
  // The first NB - 1 copies, for the entries there are (none for an empty
  // list), go out while the operand loads are still in flight; then
  // everything issued so far is waited for (the compiler does not count the
  // copies, so a later wait of its own for the operands would be a full one).
  if (U > 0) issue(jq[0], buf0);
  if (NB >= 3 && U > 1) issue(jq[1], buf1);
  if (NB >= 4 && U > 2) issue(jq[2], buf2);
  wait_vm_lgkm0<0>();
  lse2 = lse_raw * kLog2e;
  // D for this lane's row; the lane half h = 0 stores it for bsa_bwd_dkv.
  dsum = halves_sum(operand_dot<T, D>(dop, oop));
  if (has && (lane >> 5) == 0) p.delta[(size_t)bh * p.N + row] = dsum;
  auto step = [&](int i, auto b_c) {
    constexpr int b = decltype(b_c)::value;
    // this wave's copies of entry i have landed; those of the min(NB - 2,
    // U - 1 - i) later entries already issued may stay in flight
    const int ahead = U - 1 - i;
    if (NB >= 4 && ahead >= 2) wait_vm_lgkm0<(NB >= 4 ? 2 : 0) * C::kParts>();
    else if (NB >= 3 && ahead >= 1) wait_vm_lgkm0<(NB >= 3 ? 1 : 0) * C::kParts>();
    else wait_vm_lgkm0<0>();
    raw_barrier();
    const bool use = mq[0];
    const bool diag = CAUSAL && jq[0] == qb;
#pragma unroll
    for (int e = 0; e + 1 < NB; ++e) {
      jq[e] = jq[e + 1];
      mq[e] = mq[e + 1];
    }
    jq[NB - 1] = entry_at(i + NB, mq[NB - 1]);
    if (i + NB - 1 < U) issue(jq[NB - 2], buffer(std::integral_constant<int, (b + NB - 1) % NB>{}));
    if (use) compute(buffer(b_c), diag);
  };
  for (int i = 0; i < U; i += NB) {
    step(i, std::integral_constant<int, 0>{});
    if (i + 1 < U) step(i + 1, std::integral_constant<int, 1>{});
    if constexpr (NB >= 3)
      if (i + 2 < U) step(i + 2, std::integral_constant<int, 2>{});
    if constexpr (NB >= 4)
      if (i + 3 < U) step(i + 3, std::integral_constant<int, 3>{});
  }

  // dQ leaves through this wave's part of the idle ring (whole 16-byte stores).
  wait_vm_lgkm0<0>();  // no copy is still landing (the compiler does not track them)
  __syncthreads();     // every wave is done with the ring
  if (!has) return;
  unsigned char* const stage_buf = wave < C::kPerBuf       ? buf0
                                  : wave < 2 * C::kPerBuf ? buf1
                                  : wave < 3 * C::kPerBuf ? buf2
                                                          : buf3;
  store_rows_lds<T, D>(static_cast<T*>(p.dq) + head + (size_t)q0 * D, dq, p.scale, lane,
                       (LDS_PTR(unsigned char))stage_buf + (wave % C::kPerBuf) * C::kRowsStage);
}

// ---------------------------------------------------------------- dK, dV
// One key block per workgroup.  (Four blocks sharing the stages of the union
// of their columns, as bsa_bwd_dq does at block 32, measured slower here:
// the log-linear columns of neighbouring key blocks share few query blocks,
// so each wave idled through about 40% of the union's steps.)
template <typename T, int BS, int D, bool CAUSAL>
__global__ __launch_bounds__((kWave * BwdCfg<T, BS, D, 8 * BS>::W)) void bsa_bwd_dkv(
    BwdParams p) {
  using C = BwdCfg<T, BS, D, 8 * BS>;  // Q tile, dO tile, then LSE[BS] and D[BS] floats
  using L = typename C::L;
  using O = Ops<T>;
  constexpr int NB = C::NB;
  static_assert(NB <= 3, "one key block per workgroup keeps a ring of up to three stages");
  constexpr int QSTEPS = BS / kQRows;
  constexpr int kVecOff = L::kEntryBytes;          // LSE floats, then D floats

  __shared__ __attribute__((aligned(16))) unsigned char buf0[C::kStage];
  __shared__ __attribute__((aligned(16))) unsigned char buf1[C::kStage];
  __shared__ __attribute__((aligned(16))) unsigned char buf2[NB >= 3 ? C::kStage : 16];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(threadIdx.x / kWave);
  const int kg = wave;  // 32-key group of the block
  // dword copies per stage by this wave: LSE by wave 0, D by wave 1 (or
  // both by the one wave of a one-wave workgroup)
  const int n_vec = C::W == 1 ? 2 : wave < 2 ? 1 : 0;
  const int M = p.M;
  int bh, kb;
  group_of(xcd_remap(blockIdx.x, p.num_wg), M, 1, p.num_wg, p.col_order, p.col_ptr, bh, kb);
  kb = group_block(kb, 0, 1, M, p.col_order);
  const int32_t* const col_ptr = p.col_ptr + (size_t)(bh % p.heads) * p.ptr_stride;
  const size_t head = (size_t)bh * p.N * D;
  const T* Qh = static_cast<const T*>(p.q) + head;
  const T* dOh = static_cast<const T*>(p.dout) + head;
  const float* lse_h = p.lse + (size_t)bh * p.N;
  const float* del_h = p.delta + (size_t)bh * p.N;
  const int k0 = kb * BS + kg * kQRows;

  // The column's first entries, then the K and V loads, whose latency the
  // first copies overlap.
  const ListHead lh = list_head(p.row_idx, col_ptr[kb], col_ptr[kb + 1], lane);
  const int U = lh.n;
  typename O::template QOperand<D> kop, vop;
  O::template load_q<D>(kop, static_cast<const T*>(p.k) + head + (size_t)k0 * D, lane);
  O::template load_q<D>(vop, static_cast<const T*>(p.v) + head + (size_t)k0 * D, lane);

  int chunk_base = -kWave, chunk = -1;
  uint64_t chunk_sel = 0;
  auto entry_at = [&](int t, bool& use) -> int {
    if (t >= U) {
      use = false;
      return -1;
    }
    if ((t & ~(kWave - 1)) != chunk_base) {
      chunk_base = t & ~(kWave - 1);
      const int idx = chunk_base + lane;
      chunk = chunk_base == 0 ? lh.first : idx < U ? p.row_idx[lh.start + idx] : -1;
      const bool sel = chunk >= 0 && chunk < M && (!CAUSAL || chunk >= kb);
      chunk_sel = __builtin_amdgcn_ballot_w64(sel);
    }
    use = ((chunk_sel >> (t - chunk_base)) & 1ull) != 0;
    return __builtin_amdgcn_readlane(chunk, t - chunk_base);
  };

  constexpr int kPartsPerTile = L::kCopies / 2;
  // One-wave workgroups copy every part of a stage, in runs of kRun behind
  // one M0 write (within one tile; dma_off carries the run's immediate offset
  // taken off).  Several waves interleave their parts: wave w copies parts
  // w, w + W, ..., one copy per M0 write (at block 64 and d = 128, the long
  // workload's backward ran 3.7% slower with each wave copying a whole tile).
  constexpr int kRun = C::W == 1 ? dma_run(C::kParts, kPartsPerTile) : 1;
  auto part_of = [&](int c) { return C::W == 1 ? c : wave + c * C::W; };
  uint32_t dma_off[C::kParts];
#pragma unroll
  for (int c = 0; c < C::kParts; ++c) {
    const int part = part_of(c) % kPartsPerTile;
    const int slot = part * kWave + lane;
    const int r = slot / L::kChunksPerRow;
    dma_off[c] = (uint32_t)(r * L::kRowBytes + (((slot % L::kChunksPerRow) ^ L::swz(r)) << 4) -
                            (c % kRun) * kWave * 16);
  }
  auto issue = [&](int i, unsigned char* buf) {
    const int q0 = (int)((uint32_t)i < (uint32_t)M ? (uint32_t)i : 0u) * BS;
    const uint32_t dst = (uint32_t)(uintptr_t)(LDS_PTR(unsigned char))buf;
#pragma unroll
    for (int r = 0; r < C::kParts / kRun; ++r) {
      const int part = part_of(r * kRun);
      uint32_t v[kRun];
#pragma unroll
      for (int k = 0; k < kRun; ++k) v[k] = dma_off[r * kRun + k];
      lds_dma16_run<kRun>((part < kPartsPerTile ? Qh : dOh) + (size_t)q0 * D, v,
                          dst + part * kWave * 16);
    }
    // LSE and D of the block's rows (BS floats each): waves 0 and 1 copy
    // one vector each, or the one wave both.
    if (lane < BS) {
      if (C::W == 1 || wave == 0) lds_dma4(lse_h + q0, (uint32_t)lane * 4, dst + kVecOff);
      if (C::W == 1 || wave == 1) lds_dma4(del_h + q0, (uint32_t)lane * 4, dst + kVecOff + 4 * BS);
    }
  };

  typename O::template Offsets<BS, D> off;
  off.init(lane, 0);
  f32x16_t dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    dk[dt] = f32x16_t{};
    dv[dt] = f32x16_t{};
  }
  const float c2 = p.scale_log2;
  const int h = lane >> 5;

  auto compute = [&](unsigned char* buf, bool diag) {
    LDS_PTR(unsigned char) tile = (LDS_PTR(unsigned char))buf;
    LDS_PTR(const f32x4_t) vec = (LDS_PTR(const f32x4_t))(tile + kVecOff);
#pragma unroll
    for (int sq = 0; sq < QSTEPS; ++sq) {
      if (diag && sq < kg) continue;  // those queries precede every key of the wave
      f32x16_t s, dp;  // S = Q K^T and dP = dO V^T, lane = key
      score_pair<T, BS, D>(kop, vop, off, tile, sq, s, dp);
      if (diag && sq == kg) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if ((lane & 31) > 8 * (r / 4) + 4 * h + (r % 4)) s[r] = -INFINITY;
      }
      // Register r of the lane half h holds query 32 sq + 8 (r / 4) + 4 h + r % 4;
      // its LSE, then its D, are read from the stage four at a time.
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4_t l4 = vec[(32 * sq + 8 * g + 4 * h) / 4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s[4 * g + e] = fast_exp2(fmaf(s[4 * g + e], c2, -l4[e] * kLog2e));
      }
      (void)O::template accumulate<BS, D>(dv, s, off, tile, 0, sq);  // dO^T P
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4_t d4 = vec[(BS + 32 * sq + 8 * g + 4 * h) / 4];
#pragma unroll
        for (int e = 0; e < 4; ++e) s[4 * g + e] = s[4 * g + e] * (dp[4 * g + e] - d4[e]);  // dS
      }
      (void)O::template accumulate<BS, D>(dk, s, off, tile, -L::kTileBytes, sq);  // Q^T dS
    }
  };

  int jq[NB];
  bool mq[NB];
#pragma unroll
  for (int e = 0; e < NB; ++e) jq[e] = entry_at(e, mq[e]);
  auto buffer = [&](auto b_c) -> unsigned char* {
    constexpr int b = decltype(b_c)::value;
    if constexpr (b == 0) return buf0;
    else if constexpr (b == 1) return buf1;
    else return buf2;
  };
  // The first NB - 1 copies, for the entries there are (none for an empty
  // list), go out while the K and V loads are still in flight; then
  // everything issued so far is waited for.
  if (U > 0) issue(jq[0], buf0);
  if (NB >= 3 && U > 1) issue(jq[1], buf1);
  wait_vm_lgkm0<0>();
  // Waits for this wave's copies of the current entry, leaving those of `k`
  // later entries in flight (a stage is kParts tile copies plus n_vec).
  auto wait_leaving = [&](auto k_c) {
    constexpr int k = decltype(k_c)::value;
    if (n_vec == 2) wait_vm_lgkm0<k * (C::kParts + 2)>();
    else if (n_vec == 1) wait_vm_lgkm0<k * (C::kParts + 1)>();
    else wait_vm_lgkm0<k * C::kParts>();
  };
  auto step = [&](int i, auto b_c) {
    constexpr int b = decltype(b_c)::value;
    // the min(NB - 2, U - 1 - i) later entries already issued may stay in flight
    const int ahead = U - 1 - i;
    if (NB >= 3 && ahead >= 1) wait_leaving(std::integral_constant<int, NB >= 3 ? 1 : 0>{});
    else wait_vm_lgkm0<0>();
    raw_barrier();
    const bool use = mq[0];
    const bool diag = CAUSAL && jq[0] == kb;
#pragma unroll
    for (int e = 0; e + 1 < NB; ++e) {
      jq[e] = jq[e + 1];
      mq[e] = mq[e + 1];
    }
    jq[NB - 1] = entry_at(i + NB, mq[NB - 1]);
    if (i + NB - 1 < U) issue(jq[NB - 2], buffer(std::integral_constant<int, (b + NB - 1) % NB>{}));
    if (use) compute(buffer(b_c), diag);
  };
  for (int i = 0; i < U; i += NB) {
    step(i, std::integral_constant<int, 0>{});
    if (i + 1 < U) step(i + 1, std::integral_constant<int, 1>{});
    if constexpr (NB >= 3)
      if (i + 2 < U) step(i + 2, std::integral_constant<int, 2>{});
  }

  // dK then dV leave through this wave's part of the idle ring.
  wait_vm_lgkm0<0>();  // no copy is still landing (the compiler does not track them)
  __syncthreads();     // every wave is done with the ring
  unsigned char* const stage_buf = wave < C::kPerBuf ? buf0 : wave < 2 * C::kPerBuf ? buf1 : buf2;
  LDS_PTR(unsigned char) region =
      (LDS_PTR(unsigned char))stage_buf + (wave % C::kPerBuf) * C::kRowsStage;
  store_rows_lds<T, D>(static_cast<T*>(p.dk) + head + (size_t)k0 * D, dk, p.scale, lane, region);
  store_rows_lds<T, D>(static_cast<T*>(p.dv) + head + (size_t)k0 * D, dv, 1.0f, lane, region);
}

// ---------------------------------------------------------------- host

constexpr size_t kMaxLds = 160 * 1024;

template <typename T, int BS, int D, int G, bool CAUSAL>
bsa_status launch_bwd(const BwdParams& p, hipStream_t stream) {
  // dQ: G blocks per workgroup; dK/dV: one
  const size_t dyn = union_lds_bytes(G, p.M);
  BwdParams pk = p;
  pk.num_wg = p.num_wg / ((p.M + G - 1) / G) * p.M;
  // Shapes with more than 64 KB of LDS need the per-kernel limit raised, once
  // per device.
  static std::atomic<uint64_t> raised{0};
  uint64_t bit;
  const void* kernels[2] = {reinterpret_cast<const void*>(&bsa_bwd_dq<T, BS, D, G, CAUSAL>),
                            reinterpret_cast<const void*>(&bsa_bwd_dkv<T, BS, D, CAUSAL>)};
  const size_t dyns[2] = {dyn, 0};
  for (int i = 0; i < 2; ++i) {
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, kernels[i]) != hipSuccess) return BSA_ERR_HIP;
    if (attr.sharedSizeBytes + dyns[i] > kMaxLds) return BSA_ERR_INVALID_ARGUMENT;
  }
  if (due_on_device(raised, &bit)) {
    for (const void* f : kernels) {
      hipFuncAttributes attr;
      if (hipFuncGetAttributes(&attr, f) != hipSuccess) return BSA_ERR_HIP;
      if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(kMaxLds - attr.sharedSizeBytes)) != hipSuccess)
        return BSA_ERR_HIP;
    }
    mark_done(raised, bit);
  }
  hipLaunchKernelGGL((bsa_bwd_dq<T, BS, D, G, CAUSAL>), dim3(p.num_wg),
                     dim3(kWave * BwdCfg<T, BS, D, 0, G>::W), dyn, stream, p);
  if (hipGetLastError() != hipSuccess) return BSA_ERR_HIP;
  hipLaunchKernelGGL((bsa_bwd_dkv<T, BS, D, CAUSAL>), dim3(pk.num_wg),
                     dim3(kWave * BwdCfg<T, BS, D, 8 * BS>::W), 0, stream, pk);
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

template <typename T, int BS, int D>
bsa_status launch_group(const BwdParams& p, int group, bool causal, hipStream_t stream) {
  if (group == 1)
    return causal ? launch_bwd<T, BS, D, 1, true>(p, stream) : launch_bwd<T, BS, D, 1, false>(p, stream);
  if constexpr (BS == 32) {
    if (group == 4)
      return causal ? launch_bwd<T, BS, D, 4, true>(p, stream)
                    : launch_bwd<T, BS, D, 4, false>(p, stream);
  }
  return BSA_ERR_INVALID_ARGUMENT;
}

template <typename T>
bsa_status dispatch_bwd(const BwdParams& p, int bs, int d, int group, bool causal,
                        hipStream_t stream) {
  if (bs == 32 && d == 64) return launch_group<T, 32, 64>(p, group, causal, stream);
  if (bs == 32 && d == 128) return launch_group<T, 32, 128>(p, group, causal, stream);
  if (bs == 64 && d == 64) return launch_group<T, 64, 64>(p, group, causal, stream);
  if (bs == 64 && d == 128) return launch_group<T, 64, 128>(p, group, causal, stream);
  return BSA_ERR_INVALID_ARGUMENT;
}

// Compute units of the current device (cached per device; 256 if the query
// fails).
int64_t device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = -1;
  if (dev >= 0) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) !=
          hipSuccess ||
      n <= 0)
    n = 256;
  if (dev >= 0) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Query blocks per dQ workgroup.  Block 32 on a large grid (eight one-wave
// blocks per SIMD or more): four blocks share each stage of the union of
// their rows, so a K/V tile is copied once for four waves instead of once per
// wave.  Otherwise (block 64 holds two waves already; small grids want every
// block's own short chain) one block.  The union list and its bitmaps must
// fit beside the ring (M up to a few thousand blocks).  The dK/dV kernel
// always takes one key block per workgroup.
int choose_group(int64_t bhm, int bs, int M) {
  if (bs != 32 || bhm < 8 * 4 * device_cus()) return 1;
  if (union_lds_bytes(4, M) > 32 * 1024) return 1;
  return 4;
}

}  // namespace

// Scratch of the allocation-free backward: D (one float per query row), in
// device memory the code object itself holds.  Every GPU the library runs
// on keeps its own copy until the process ends.
constexpr int64_t kScratchRows = int64_t{1} << 22;  // 16 MiB of float
static __device__ __align__(256) float scratch[kScratchRows];

namespace {

bsa_status backward_impl(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv,
                         float* delta, int32_t batch, int32_t heads, int32_t seq_len,
                         int32_t head_dim, int32_t block_size, int32_t dtype,
                         const int32_t* row_ptr, const int32_t* col_idx, const int32_t* col_ptr,
                         const int32_t* row_idx, const int32_t* row_order,
                         const int32_t* col_order, int64_t nnz, float scale, int32_t flags,
                         void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr ||
      dout == nullptr || dq == nullptr || dk == nullptr || dv == nullptr || delta == nullptr ||
      row_ptr == nullptr || col_idx == nullptr || col_ptr == nullptr || row_idx == nullptr)
    return BSA_ERR_NULL_POINTER;
  if (dtype != BSA_DTYPE_F32 && dtype != BSA_DTYPE_BF16) return BSA_ERR_INVALID_ARGUMENT;
  if (block_size != 32 && block_size != 64) return BSA_ERR_INVALID_ARGUMENT;
  if (head_dim != 64 && head_dim != 128) return BSA_ERR_INVALID_ARGUMENT;
  if ((flags & ~(BSA_FORWARD_CAUSAL | BSA_FORWARD_PATTERN_PER_HEAD)) != 0)
    return BSA_ERR_INVALID_ARGUMENT;
  const bool per_head = (flags & BSA_FORWARD_PATTERN_PER_HEAD) != 0;
  // one pattern per head: the work orders are of one shared pattern
  if (per_head && (row_order != nullptr || col_order != nullptr)) return BSA_ERR_INVALID_ARGUMENT;
  if (batch <= 0 || heads <= 0 || seq_len <= 0 || seq_len % block_size != 0) return BSA_ERR_SHAPE;
  if (!(scale == scale) || std::isinf(scale)) return BSA_ERR_INVALID_ARGUMENT;
  const int64_t M = seq_len / block_size;
  const int64_t patterns = per_head ? heads : 1;
  if (nnz < patterns * M || nnz > patterns * M * M) return BSA_ERR_SHAPE;
  const int group = choose_group((int64_t)batch * heads * M, block_size, (int)M);
  const int64_t num_wg = (int64_t)batch * heads * ((M + group - 1) / group);
  if ((int64_t)batch * heads * seq_len > INT32_MAX || num_wg > INT32_MAX) return BSA_ERR_SHAPE;
  const uintptr_t align = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                          reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o) |
                          reinterpret_cast<uintptr_t>(dout) | reinterpret_cast<uintptr_t>(dq) |
                          reinterpret_cast<uintptr_t>(dk) | reinterpret_cast<uintptr_t>(dv);
  if (align % 16 != 0 || reinterpret_cast<uintptr_t>(lse) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(delta) % 4 != 0)
    return BSA_ERR_INVALID_ARGUMENT;

  BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.delta = delta;
  p.row_ptr = row_ptr;
  p.col_idx = col_idx;
  p.col_ptr = col_ptr;
  p.row_idx = row_idx;
  p.row_order = row_order;
  p.col_order = col_order;
  p.M = static_cast<int32_t>(M);
  p.N = seq_len;
  p.num_wg = static_cast<int32_t>(num_wg);
  p.heads = heads;
  p.ptr_stride = per_head ? static_cast<int32_t>(M + 1) : 0;
  p.scale = scale > 0.f ? scale : 1.0f / std::sqrt(static_cast<float>(head_dim));
  p.scale_log2 = p.scale * kLog2e;
  const bool causal = (flags & BSA_FORWARD_CAUSAL) != 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (dtype == BSA_DTYPE_F32)
    return dispatch_bwd<float>(p, block_size, head_dim, group, causal, st);
  return dispatch_bwd<__bf16>(p, block_size, head_dim, group, causal, st);
}

// The device address of `scratch` on each device (looked up once per device,
// with that device current).  In host code the array's name is only a
// host-side stand-in, never a device address.
std::atomic<void*> scratch_ptr[64];

bsa_status scratch_on_current_device(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return BSA_ERR_HIP;
  if (dev < 0 || dev >= 64) return BSA_ERR_INVALID_ARGUMENT;
  void* ptr = scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return BSA_ERR_HIP;
    }
    scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  *out = static_cast<float*>(ptr);
  return BSA_OK;
}

}  // namespace

extern "C" bsa_status bsa_backward(const void* q, const void* k, const void* v, const void* o,
                                   const float* lse, const void* dout, void* dq, void* dk,
                                   void* dv, float* delta, int32_t batch, int32_t heads,
                                   int32_t seq_len, int32_t head_dim, int32_t block_size,
                                   int32_t dtype, const int32_t* row_ptr, const int32_t* col_idx,
                                   const int32_t* col_ptr, const int32_t* row_idx,
                                   const int32_t* row_order, const int32_t* col_order,
                                   int64_t nnz, float scale, int32_t flags, void* stream) {
  return backward_impl(q, k, v, o, lse, dout, dq, dk, dv, delta, batch, heads, seq_len, head_dim,
                       block_size, dtype, row_ptr, col_idx, col_ptr, row_idx, row_order,
                       col_order, nnz, scale, flags, stream);
}

extern "C" int64_t bsa_backward_noalloc_max_rows(void) { return kScratchRows; }

extern "C" bsa_status bsa_backward_noalloc(const void* q, const void* k, const void* v,
                                           const void* o, const float* lse, const void* dout,
                                           void* dq, void* dk, void* dv, int32_t batch,
                                           int32_t heads, int32_t seq_len, int32_t head_dim,
                                           int32_t block_size, int32_t dtype,
                                           const int32_t* row_ptr, const int32_t* col_idx,
                                           const int32_t* col_ptr, const int32_t* row_idx,
                                           const int32_t* row_order, const int32_t* col_order,
                                           int64_t nnz, float scale, int32_t flags,
                                           void* stream) {
  if (batch > 0 && heads > 0 && seq_len > 0 &&
      (int64_t)batch * heads * seq_len > kScratchRows)
    return BSA_ERR_BUFFER_TOO_SMALL;
  float* delta = nullptr;
  const bsa_status st = scratch_on_current_device(&delta);
  if (st != BSA_OK) return st;
  return backward_impl(q, k, v, o, lse, dout, dq, dk, dv, delta, batch, heads, seq_len, head_dim,
                       block_size, dtype, row_ptr, col_idx, col_ptr, row_idx, row_order,
                       col_order, nnz, scale, flags, stream);
}
