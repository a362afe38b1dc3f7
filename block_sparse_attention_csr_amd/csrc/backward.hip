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
// Two kernels, both one workgroup per (batch, head, block) with 32 rows per
// wave, both streaming tiles through an LDS ring with direct-to-LDS copies:
//  * bsa_bwd_dq: per query block, walks its CSR row (the K blocks it
//    selects); K and V tiles in the ring.  It also writes D for its rows.
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
  int32_t num_wg;  // batch * heads * M
  float scale;
  float scale_log2;
};

// (batch*head, block) of a workgroup.  Workgroup ids run XCD by XCD (each XCD
// one contiguous range of HX heads, so one head's blocks share an L2).  With
// an order array (bsa_pattern_order: the long blocks -- more than twice the
// mean entry count -- first, then the rest ascending), a range starts with
// the long blocks of all its heads, then takes the rest head by head.
__device__ __forceinline__ void block_of(int wg, int M, int num_wg, const int32_t* order,
                                         const int32_t* ptr, int& bh, int& blk) {
  if (order == nullptr) {
    blk = wg % M;
    bh = wg / M;
    return;
  }
  // Number of long blocks: the leading entries of `order` whose count exceeds
  // twice the mean (the same test the host applies), by bisection.
  const int64_t total = ptr[M];
  auto is_long = [&](int k) {
    const int b = order[k];
    return (int64_t)(ptr[b + 1] - ptr[b]) * M > 2 * total;
  };
  int lo = 0, hi = M;  // is_long holds on [0, lo) and fails on [hi, M)
  while (lo < hi) {
    const int mid = (lo + hi) / 2;
    if (is_long(mid)) lo = mid + 1;
    else hi = mid;
  }
  const int nlong = lo;
  const int bhs = num_wg / M;
  const int hx = (bhs + kNumXcd - 1) / kNumXcd;
  const int gidx = wg / (hx * M);
  const int r = wg % (hx * M);
  const int nh = bhs - gidx * hx < hx ? bhs - gidx * hx : hx;
  if (r < nlong * nh) {  // long blocks, rank by rank over the range's heads
    bh = gidx * hx + r % nh;
    blk = order[r / nh];
  } else {               // the rest, head by head
    const int rr = r - nlong * nh;
    bh = gidx * hx + rr / (M - nlong);
    blk = order[nlong + rr % (M - nlong)];
  }
}

// Ring depth and copy split of a backward kernel whose stage holds two tiles
// of BS rows (plus `extra` bytes).
template <typename T, int BS, int D, int kExtraBytes>
struct BwdCfg {
  using L = TileLayout<T, BS, D>;
  static constexpr int W = BS / kQRows;
  static constexpr int kStage = L::kEntryBytes + kExtraBytes;
  static constexpr int NB = 3 * kStage <= 48 * 1024 ? 3 : 2;
  static_assert(L::kCopies % W == 0, "stage copies must split evenly over the waves");
  static constexpr int kParts = L::kCopies / W;
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

// A workgroup's list (CSR row or CSC column) in LDS, written by wave 0;
// `list_store` returns its length and the caller synchronises.  The first 64
// entries are loaded (`list_head`, one per lane) before the operand loads and
// written after them: the vector-memory counter drains in order, so loaded
// after the operands the list would wait for all of them first.
struct ListHead {
  int start, n, first;
};
__device__ __forceinline__ ListHead list_head(const int32_t* idx, int start, int end, int wave,
                                              int lane) {
  ListHead h{start, end - start, -1};
  if (wave == 0 && lane < h.n) h.first = idx[start + lane];
  return h;
}
__device__ __forceinline__ int list_store(int32_t* list, const int32_t* idx, const ListHead& h,
                                          int wave, int lane) {
  if (wave == 0) {
    if (lane < h.n) list[lane] = h.first;
    for (int t = kWave + lane; t < h.n; t += kWave) list[t] = idx[h.start + t];
  }
  return h.n;
}

// ---------------------------------------------------------------- dQ (and D)
template <typename T, int BS, int D, bool CAUSAL>
__global__ __launch_bounds__((kWave * BwdCfg<T, BS, D, 0>::W)) void bsa_bwd_dq(BwdParams p) {
  using C = BwdCfg<T, BS, D, 0>;
  using L = typename C::L;
  using O = Ops<T>;
  constexpr int NB = C::NB;
  constexpr int KSTEPS = BS / kKeyStep;

  __shared__ __attribute__((aligned(16))) unsigned char buf0[C::kStage];
  __shared__ __attribute__((aligned(16))) unsigned char buf1[C::kStage];
  __shared__ __attribute__((aligned(16))) unsigned char buf2[NB == 3 ? C::kStage : 16];
  extern __shared__ __attribute__((aligned(16))) int32_t list[];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(threadIdx.x / kWave);  // 32-row query group
  const int M = p.M;
  int bh, qb;
  block_of(xcd_remap(blockIdx.x, p.num_wg), M, p.num_wg, p.row_order, p.row_ptr, bh, qb);
  const size_t head = (size_t)bh * p.N * D;
  const T* K = static_cast<const T*>(p.k) + head;
  const T* V = static_cast<const T*>(p.v) + head;
  const int q0 = qb * BS + wave * kQRows;
  const int row = q0 + (lane & 31);

  const ListHead lh = list_head(p.col_idx, p.row_ptr[qb], p.row_ptr[qb + 1], wave, lane);
  typename O::template QOperand<D> qop, dop, oop;
  O::template load_q<D>(qop, static_cast<const T*>(p.q) + head + (size_t)q0 * D, lane);
  O::template load_q<D>(dop, static_cast<const T*>(p.dout) + head + (size_t)q0 * D, lane);
  O::template load_q<D>(oop, static_cast<const T*>(p.o) + head + (size_t)q0 * D, lane);
  const float lse2 = p.lse[(size_t)bh * p.N + row] * kLog2e;

  const int U = list_store(list, p.col_idx, lh, wave, lane);
  __syncthreads();

  // D for this lane's row; the lane half h = 0 stores it for bsa_bwd_dkv.
  const float dsum = halves_sum(operand_dot<T, D>(dop, oop));
  if ((lane >> 5) == 0) p.delta[(size_t)bh * p.N + row] = dsum;

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
      chunk = idx < U ? list[idx] : -1;
      chunk_sel = __builtin_amdgcn_ballot_w64(chunk >= 0 && chunk < M && (!CAUSAL || chunk <= qb));
    }
    use = ((chunk_sel >> (t - chunk_base)) & 1ull) != 0;
    return __builtin_amdgcn_readlane(chunk, t - chunk_base);
  };

  constexpr int kPartsPerTile = L::kCopies / 2;
  int dma_off[C::kParts];
#pragma unroll
  for (int c = 0; c < C::kParts; ++c) {
    const int part = (wave + c * C::W) % kPartsPerTile;
    const int slot = part * kWave + lane;
    const int r = slot / L::kChunksPerRow;
    dma_off[c] = r * L::kRowBytes + (((slot % L::kChunksPerRow) ^ L::swz(r)) << 4);
  }
  auto issue = [&](int j, unsigned char* buf) {
    const int key0 = (j < 0 || j >= M ? 0 : j) * BS;
    const uint32_t dst = (uint32_t)(uintptr_t)(LDS_PTR(unsigned char))buf;
#pragma unroll
    for (int c = 0; c < C::kParts; ++c) {
      const int part = wave + c * C::W;
      const T* base = (part < kPartsPerTile ? K : V) + (size_t)key0 * D;
      lds_dma16(base, (uint32_t)dma_off[c], dst + part * kWave * 16);
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
      if (diag && st > wave) continue;
      f32x16_t s = O::template scores<BS, D>(qop, off, tile, 0, st);  // S^T, lane = query
      if (diag && st == wave) {
        const int h = lane >> 5;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r / 4) + 4 * h + (r % 4) > (lane & 31)) s[r] = -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = fast_exp2(fmaf(s[r], c2, -lse2));  // P^T
      const f32x16_t dp = O::template scores<BS, D>(dop, off, tile, L::kTileBytes, st);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = s[r] * (dp[r] - dsum);  // dS^T
      (void)O::template accumulate<BS, D>(dq, s, off, tile, -L::kTileBytes, st);  // K^T dS^T
    }
  };

  int jq[NB];
  bool mq[NB];
#pragma unroll
  for (int e = 0; e < NB; ++e) jq[e] = entry_at(e, mq[e]);
  wait_vm_lgkm0<0>();  // Q, dO, O, LSE loads and the list are complete
  // The first copies, for the entries there are (none for an empty list).
  if (U > 0) issue(jq[0], buf0);
  if (NB == 3 && U > 1) issue(jq[1], buf1);
  auto buffer = [&](auto b_c) -> unsigned char* {
    constexpr int b = decltype(b_c)::value;
    if constexpr (b == 0) return buf0;
    else if constexpr (b == 1) return buf1;
    else return buf2;
  };
  auto step = [&](int i, auto b_c) {
    constexpr int b = decltype(b_c)::value;
    if (NB == 3 && i + 1 < U) wait_vm_lgkm0<C::kParts>();
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
    if constexpr (NB == 3)
      if (i + 2 < U) step(i + 2, std::integral_constant<int, 2>{});
  }

  // dQ leaves through this wave's part of the idle ring (whole 16-byte stores).
  wait_vm_lgkm0<0>();  // no copy is still landing (the compiler does not track them)
  __syncthreads();     // every wave is done with the ring
  store_rows_lds<T, D>(static_cast<T*>(p.dq) + head + (size_t)q0 * D, dq, p.scale, lane,
                       (LDS_PTR(unsigned char))buf0 + wave * (kQRows * D * (int)sizeof(T)));
}

// ---------------------------------------------------------------- dK, dV
template <typename T, int BS, int D, bool CAUSAL>
__global__ __launch_bounds__((kWave * BwdCfg<T, BS, D, 8 * BS>::W)) void bsa_bwd_dkv(BwdParams p) {
  using C = BwdCfg<T, BS, D, 8 * BS>;  // Q tile, dO tile, then LSE[BS] and D[BS] floats
  using L = typename C::L;
  using O = Ops<T>;
  constexpr int NB = C::NB;
  constexpr int QSTEPS = BS / kQRows;
  constexpr int kVecOff = L::kEntryBytes;          // LSE floats, then D floats
  constexpr int kExtra = C::W == 1 ? 2 : 1;        // dword copies per wave per stage

  __shared__ __attribute__((aligned(16))) unsigned char buf0[C::kStage];
  __shared__ __attribute__((aligned(16))) unsigned char buf1[C::kStage];
  __shared__ __attribute__((aligned(16))) unsigned char buf2[NB == 3 ? C::kStage : 16];
  extern __shared__ __attribute__((aligned(16))) int32_t list[];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(threadIdx.x / kWave);  // 32-key group
  const int M = p.M;
  int bh, kb;
  block_of(xcd_remap(blockIdx.x, p.num_wg), M, p.num_wg, p.col_order, p.col_ptr, bh, kb);
  const size_t head = (size_t)bh * p.N * D;
  const T* Qh = static_cast<const T*>(p.q) + head;
  const T* dOh = static_cast<const T*>(p.dout) + head;
  const float* lse_h = p.lse + (size_t)bh * p.N;
  const float* del_h = p.delta + (size_t)bh * p.N;
  const int k0 = kb * BS + wave * kQRows;

  const ListHead lh = list_head(p.row_idx, p.col_ptr[kb], p.col_ptr[kb + 1], wave, lane);
  typename O::template QOperand<D> kop, vop;
  O::template load_q<D>(kop, static_cast<const T*>(p.k) + head + (size_t)k0 * D, lane);
  O::template load_q<D>(vop, static_cast<const T*>(p.v) + head + (size_t)k0 * D, lane);

  const int U = list_store(list, p.row_idx, lh, wave, lane);
  __syncthreads();

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
      chunk = idx < U ? list[idx] : -1;
      chunk_sel = __builtin_amdgcn_ballot_w64(chunk >= 0 && chunk < M && (!CAUSAL || chunk >= kb));
    }
    use = ((chunk_sel >> (t - chunk_base)) & 1ull) != 0;
    return __builtin_amdgcn_readlane(chunk, t - chunk_base);
  };

  constexpr int kPartsPerTile = L::kCopies / 2;
  int dma_off[C::kParts];
#pragma unroll
  for (int c = 0; c < C::kParts; ++c) {
    const int part = (wave + c * C::W) % kPartsPerTile;
    const int slot = part * kWave + lane;
    const int r = slot / L::kChunksPerRow;
    dma_off[c] = r * L::kRowBytes + (((slot % L::kChunksPerRow) ^ L::swz(r)) << 4);
  }
  auto issue = [&](int i, unsigned char* buf) {
    const int q0 = (i < 0 || i >= M ? 0 : i) * BS;
    const uint32_t dst = (uint32_t)(uintptr_t)(LDS_PTR(unsigned char))buf;
#pragma unroll
    for (int c = 0; c < C::kParts; ++c) {
      const int part = wave + c * C::W;
      const T* base = (part < kPartsPerTile ? Qh : dOh) + (size_t)q0 * D;
      lds_dma16(base, (uint32_t)dma_off[c], dst + part * kWave * 16);
    }
    // LSE and D of the block's rows (BS floats each): one wave copies each
    // vector, or wave 0 both.
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
      if (diag && sq < wave) continue;  // those queries precede every key of the wave
      f32x16_t s = O::template scores<BS, D>(kop, off, tile, 0, sq);  // S, lane = key
      if (diag && sq == wave) {
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
      const f32x16_t dp = O::template scores<BS, D>(vop, off, tile, L::kTileBytes, sq);
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
  wait_vm_lgkm0<0>();  // K, V loads and the list are complete
  // The first copies, for the entries there are (none for an empty list).
  if (U > 0) issue(jq[0], buf0);
  if (NB == 3 && U > 1) issue(jq[1], buf1);
  auto buffer = [&](auto b_c) -> unsigned char* {
    constexpr int b = decltype(b_c)::value;
    if constexpr (b == 0) return buf0;
    else if constexpr (b == 1) return buf1;
    else return buf2;
  };
  constexpr int kPerStage = C::kParts + kExtra;
  auto step = [&](int i, auto b_c) {
    constexpr int b = decltype(b_c)::value;
    if (NB == 3 && i + 1 < U) wait_vm_lgkm0<kPerStage>();
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
    if constexpr (NB == 3)
      if (i + 2 < U) step(i + 2, std::integral_constant<int, 2>{});
  }

  // dK then dV leave through this wave's part of the idle ring.
  wait_vm_lgkm0<0>();  // no copy is still landing (the compiler does not track them)
  __syncthreads();     // every wave is done with the ring
  LDS_PTR(unsigned char) region =
      (LDS_PTR(unsigned char))buf0 + wave * (kQRows * D * (int)sizeof(T));
  store_rows_lds<T, D>(static_cast<T*>(p.dk) + head + (size_t)k0 * D, dk, p.scale, lane, region);
  store_rows_lds<T, D>(static_cast<T*>(p.dv) + head + (size_t)k0 * D, dv, 1.0f, lane, region);
}

// ---------------------------------------------------------------- host

template <typename T, int BS, int D, bool CAUSAL>
bsa_status launch_bwd(const BwdParams& p, hipStream_t stream) {
  const size_t list_bytes = 4 * (size_t)p.M;
  const dim3 grid(p.num_wg);
  const dim3 block(kWave * (BS / kQRows));
  if (list_bytes > 16 * 1024) return BSA_ERR_SHAPE;  // M > 4096 blocks: list does not fit
  // Shapes with more than 64 KB of LDS need the per-kernel limit raised, once
  // per device.
  static std::atomic<uint64_t> raised{0};
  uint64_t bit;
  if (due_on_device(raised, &bit)) {
    const void* kernels[2] = {reinterpret_cast<const void*>(&bsa_bwd_dq<T, BS, D, CAUSAL>),
                              reinterpret_cast<const void*>(&bsa_bwd_dkv<T, BS, D, CAUSAL>)};
    for (const void* f : kernels) {
      hipFuncAttributes attr;
      if (hipFuncGetAttributes(&attr, f) != hipSuccess) return BSA_ERR_HIP;
      if (attr.sharedSizeBytes + 16 * 1024 > 64 * 1024 &&
          hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(160 * 1024 - attr.sharedSizeBytes)) != hipSuccess)
        return BSA_ERR_HIP;
    }
    mark_done(raised, bit);
  }
  hipLaunchKernelGGL((bsa_bwd_dq<T, BS, D, CAUSAL>), grid, block, list_bytes, stream, p);
  if (hipGetLastError() != hipSuccess) return BSA_ERR_HIP;
  hipLaunchKernelGGL((bsa_bwd_dkv<T, BS, D, CAUSAL>), grid, block, list_bytes, stream, p);
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

template <typename T>
bsa_status dispatch_bwd(const BwdParams& p, int bs, int d, bool causal, hipStream_t stream) {
  if (bs == 32 && d == 64) return causal ? launch_bwd<T, 32, 64, true>(p, stream) : launch_bwd<T, 32, 64, false>(p, stream);
  if (bs == 32 && d == 128) return causal ? launch_bwd<T, 32, 128, true>(p, stream) : launch_bwd<T, 32, 128, false>(p, stream);
  if (bs == 64 && d == 64) return causal ? launch_bwd<T, 64, 64, true>(p, stream) : launch_bwd<T, 64, 64, false>(p, stream);
  if (bs == 64 && d == 128) return causal ? launch_bwd<T, 64, 128, true>(p, stream) : launch_bwd<T, 64, 128, false>(p, stream);
  return BSA_ERR_INVALID_ARGUMENT;
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
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr ||
      dout == nullptr || dq == nullptr || dk == nullptr || dv == nullptr || delta == nullptr ||
      row_ptr == nullptr || col_idx == nullptr || col_ptr == nullptr || row_idx == nullptr)
    return BSA_ERR_NULL_POINTER;
  if (dtype != BSA_DTYPE_F32 && dtype != BSA_DTYPE_BF16) return BSA_ERR_INVALID_ARGUMENT;
  if (block_size != 32 && block_size != 64) return BSA_ERR_INVALID_ARGUMENT;
  if (head_dim != 64 && head_dim != 128) return BSA_ERR_INVALID_ARGUMENT;
  if ((flags & ~BSA_FORWARD_CAUSAL) != 0) return BSA_ERR_INVALID_ARGUMENT;
  if (batch <= 0 || heads <= 0 || seq_len <= 0 || seq_len % block_size != 0) return BSA_ERR_SHAPE;
  if (!(scale == scale) || std::isinf(scale)) return BSA_ERR_INVALID_ARGUMENT;
  const int64_t M = seq_len / block_size;
  if (nnz < M || nnz > M * M || M > 4096) return BSA_ERR_SHAPE;
  const int64_t num_wg = (int64_t)batch * heads * M;
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
  p.scale = scale > 0.f ? scale : 1.0f / std::sqrt(static_cast<float>(head_dim));
  p.scale_log2 = p.scale * kLog2e;
  const bool causal = (flags & BSA_FORWARD_CAUSAL) != 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (dtype == BSA_DTYPE_F32) return dispatch_bwd<float>(p, block_size, head_dim, causal, st);
  return dispatch_bwd<__bf16>(p, block_size, head_dim, causal, st);
}
