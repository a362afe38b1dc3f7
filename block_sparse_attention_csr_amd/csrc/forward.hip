// Block-sparse attention forward for gfx950 (MI355X): one fused kernel.
//
// What is computed: for every (batch, head, query block qb) and every query
// row r of that block, softmax(scale * Q_r . K_j) V_j over exactly the key
// positions j of the K blocks the CSR row of qb lists ("Block Sparse
// Attention: Log-Linear complexity sparse attention implementation",
// czchanglian.com, section 3.3: the denominator sums exp(score) over the
// connected blocks only; Ascend CANN SparseFlashAttention article,
// hwcomputing.csdn.net, "the O(N^2) bottleneck of long sequences", for
// softmax(QK^T / sqrt(d)) V).  The per-row log-sum-exp is written as well.
//
// Mapping onto CDNA4 (gfx950):
//  * A workgroup owns G consecutive query blocks of one (batch, head), each
//    block BS/32 waves of 32 query rows, times KS key-slice wave sets (small
//    grids only).  The K/V blocks of the UNION of the G CSR rows are copied
//    once into LDS and shared: neighbouring query blocks of the log-linear
//    and banded patterns select mostly the same K blocks, so the tile traffic
//    out of L2 drops by the reuse factor.  Every wave computes only the
//    blocks its own row selects (a bit test on its row bitmap).
//  * K/V tiles are software-pipelined through registers: while union entry u
//    computes, entry u+1 is written from registers into the other LDS
//    buffer and entry u+2 is loaded from global memory (16-byte loads).
//    16-byte chunks are XOR-swizzled per row pair to spread LDS banks.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys = MFMA rows, queries =
//    MFMA columns): each lane holds the scores of ONE query, so row max and
//    row sum are in-lane plus one v_permlane32_swap between the lane halves.
//  * P stays in registers: the S^T accumulator layout is the B operand layout
//    of O^T = V^T P^T with the key order permuted consistently in V; the V
//    operand comes from row-major LDS through ds_read_b64_tr_b16.
//  * Online softmax in the log2 domain with lazy rescaling: the running max
//    used for exponentiation only moves when a block raises a row's max by
//    more than 2^8, so O is rarely rescaled; row sums use v_dot2 on the
//    bf16-rounded probabilities (the weights the P.V product actually uses).
//  * Workgroup ids are remapped so that the query blocks of one (b, h) run
//    on one XCD and share that XCD's L2.
// The fp32 variant uses v_mfma_f32_32x32x2_f32 with the same layouts.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "bsa.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define LDS_PTR(T) __attribute__((address_space(3))) T*

constexpr int kWave = 64;
constexpr int kQRows = 32;        // query rows per wave
constexpr int kKeyStep = 32;      // keys per MFMA step
constexpr int kNumXcd = 8;
constexpr int kMaxWaves = 8;      // waves per workgroup
constexpr float kLazyRescale = 8.0f;  // log2 headroom before the running max moves

#ifndef BSA_MAX_LDS
#define BSA_MAX_LDS (160 * 1024)
#endif
constexpr size_t kMaxLds = BSA_MAX_LDS;  // dynamic LDS per workgroup (gfx950: 160 KB)


struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int32_t M;          // blocks per sequence
  int32_t N;          // sequence length
  int32_t num_wg;     // batch * heads * ceil(M / group)
  int32_t group;      // G: query blocks per workgroup
  int32_t key_split;  // KS: key-slice wave sets per workgroup
  int32_t nbuf;       // LDS entry buffers per key slice (1 or 2)
  float scale_log2;   // scale * log2(e)
};

// Workgroups are dispatched round-robin over the XCDs.  Give each XCD a
// contiguous range of workgroups so that the query blocks of one head
// (which read overlapping K/V blocks) share one L2.
__device__ __forceinline__ int xcd_remap(int x, int G) {
  const int per = (G + kNumXcd - 1) / kNumXcd;
  int tall = G % kNumXcd;
  if (tall == 0) tall = kNumXcd;
  const int xcd = x % kNumXcd;
  const int local = x / kNumXcd;
  if (xcd < tall) return xcd * per + local;
  return tall * per + (xcd - tall) * (per - 1) + local;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Max (or sum) of a per-lane value with the lane 32 apart.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t f = {lo, hi};
  bf16x2_t b = __builtin_convertvector(f, bf16x2_t);  // round to nearest even
  return __builtin_bit_cast(uint32_t, b);
}

// ---------------------------------------------------------------- tile layout
// A K or V tile is BS rows of D elements, row-major in LDS, in 16-byte
// chunks; chunk c of row r sits at position c ^ swz(r).
template <typename T, int BS, int D>
struct TileLayout {
  static constexpr int kRowBytes = D * (int)sizeof(T);
  static constexpr int kChunksPerRow = kRowBytes / 16;
  static constexpr int kTileBytes = BS * kRowBytes;
  static constexpr int kEntryBytes = 2 * kTileBytes;  // K tile then V tile
  static constexpr int kCopies = kEntryBytes / (kWave * 16);  // 1 KB parts per entry

  static __device__ __forceinline__ int swz(int r) { return (r >> 1) & (kChunksPerRow - 1); }
  static __device__ __forceinline__ int chunk_offset(int r, int c) {
    return r * kRowBytes + ((c ^ swz(r)) << 4);
  }
};

// Register staging of one entry (K tile then V tile of key block `key0`).
// The entry is cut into 1 KB parts; part c is staged by wave (c % SW) of the
// key slice, lane i holding the 16-byte chunk that LDS slot 64 c + i gets
// under the swizzle.
template <typename T, int BS, int D, int SW>
struct Stage {
  using L = TileLayout<T, BS, D>;
  static_assert(L::kCopies % SW == 0, "entry parts must split evenly over the slice waves");
  static constexpr int kParts = L::kCopies / SW;  // parts per wave
  u32x4_t r[kParts];

  __device__ __forceinline__ void load(const T* K, const T* V, int key0, int ws, int lane) {
    constexpr int kSlotsPerTile = L::kTileBytes / 16;
#pragma unroll
    for (int c = 0; c < kParts; ++c) {
      const int slot = (ws + c * SW) * kWave + lane;
      const bool is_v = slot >= kSlotsPerTile;
      const int s = is_v ? slot - kSlotsPerTile : slot;
      const int row = s / L::kChunksPerRow;
      const int chunk = (s % L::kChunksPerRow) ^ L::swz(row);
      const T* src = (is_v ? V : K) + (size_t)(key0 + row) * D + chunk * (16 / (int)sizeof(T));
      r[c] = *reinterpret_cast<const u32x4_t*>(src);
    }
  }
  __device__ __forceinline__ void store(unsigned char* entry, int ws, int lane) const {
#pragma unroll
    for (int c = 0; c < kParts; ++c)
      *reinterpret_cast<u32x4_t*>(entry + ((ws + c * SW) * kWave + lane) * 16) = r[c];
  }
};

template <typename T>
struct Ops;

// ---------------------------------------------------------------- bf16
template <>
struct Ops<__bf16> {
  template <int D>
  struct QOperand { u32x4_t r[D / 16]; };

  // Lane (query = lane % 32, half h = lane / 32) holds Q[query][16c + 8h .. +8].
  template <int D>
  static __device__ __forceinline__ void load_q(QOperand<D>& q, const __bf16* Q, int lane) {
    const __bf16* p = Q + (size_t)(lane & 31) * D + (lane >> 5) * 8;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) q.r[c] = *reinterpret_cast<const u32x4_t*>(p + 16 * c);
  }

  // S^T for 32-key step st: A operand (lane = key, half h) = K[key][16c + 8h .. +8].
  template <int BS, int D>
  static __device__ __forceinline__ f32x16_t scores(const QOperand<D>& q,
                                                    const unsigned char* ktile, int st,
                                                    int lane) {
    using L = TileLayout<__bf16, BS, D>;
    const int key = st * kKeyStep + (lane & 31);
    const int h = lane >> 5;
    f32x16_t s = {};
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const u32x4_t k =
          *reinterpret_cast<const u32x4_t*>(ktile + L::chunk_offset(key, 2 * c + h));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, k),
                                                  __builtin_bit_cast(bf16x8_t, q.r[c]), s, 0, 0,
                                                  0);
    }
    return s;
  }

  // V^T operand of step st, 16-key sub-step sc, feature tile dt: lane
  // (feature = 32 dt + lane % 32, half h) holds V[key][feature] for keys
  // kappa(h, j) = 32 st + 16 sc + 8 (j / 4) + 4 h + j % 4, j = 0..7, read with
  // two transpose loads.  In each 16-lane group, lane 4k + q addresses the 4
  // features (feature0 + 4q ..) of key row k; the hardware returns to lane i
  // feature0 + i of rows k = 0..3.
  template <int BS, int D>
  static __device__ __forceinline__ u32x4_t v_operand(const unsigned char* vtile, int st, int sc,
                                                      int dt, int lane) {
    using L = TileLayout<__bf16, BS, D>;
    const int g4 = lane >> 4;
    const int h = g4 >> 1;
    const int i = lane & 15;
    const int row = st * kKeyStep + 16 * sc + 4 * h + (i >> 2);
    const int feature = dt * 32 + 16 * (g4 & 1) + 4 * (i & 3);
    const int chunk = feature >> 3;
    const int half = (feature & 7) * 2;
    const u32x2_t lo = __builtin_bit_cast(
        u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                     (LDS_PTR(s16x4_t))(vtile + L::chunk_offset(row, chunk) + half)));
    const u32x2_t hi = __builtin_bit_cast(
        u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                     (LDS_PTR(s16x4_t))(vtile + L::chunk_offset(row + 8, chunk) + half)));
    return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
  }

  // O^T += V^T P^T over one block; returns the sum of the bf16-rounded P.
  template <int BS, int D>
  static __device__ __forceinline__ float accumulate(f32x16_t (&o)[D / 32],
                                                     const f32x16_t (&p)[BS / kKeyStep],
                                                     const unsigned char* vtile, int lane) {
    float sum = 0.f;
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int st = 0; st < BS / kKeyStep; ++st) {
#pragma unroll
      for (int sc = 0; sc < 2; ++sc) {
        // The four packed words are built as separate scalars: reading dot2
        // operands out of a 128-bit vector miscompiles (every v_dot2c read
        // the first word).
        uint32_t w4[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          w4[w] = pack_bf16x2(p[st][8 * sc + 2 * w], p[st][8 * sc + 2 * w + 1]);
          sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w4[w]), ones, sum,
                                                false);
        }
        const u32x4_t pb = {w4[0], w4[1], w4[2], w4[3]};
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const u32x4_t va = v_operand<BS, D>(vtile, st, sc, dt, lane);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, va),
                                                          __builtin_bit_cast(bf16x8_t, pb),
                                                          o[dt], 0, 0, 0);
        }
      }
    }
    return sum;
  }

  // Lane holds O^T[d = 32 dt + 8 g + 4 h + e][query], e = 0..3.
  static __device__ __forceinline__ void store_o4(__bf16* dst, float a, float b, float c,
                                                  float d) {
    u32x2_t w = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
    *reinterpret_cast<u32x2_t*>(dst) = w;
  }
};

// ---------------------------------------------------------------- fp32
template <>
struct Ops<float> {
  template <int D>
  struct QOperand { f32x4_t r[D / 8]; };

  // v_mfma_f32_32x32x2_f32 contracts 2 features per instruction, one per lane
  // half.  Lane (query, h) holds Q[query][(D/2) h + c], c = 0 .. D/2-1.
  template <int D>
  static __device__ __forceinline__ void load_q(QOperand<D>& q, const float* Q, int lane) {
    const float* p = Q + (size_t)(lane & 31) * D + (lane >> 5) * (D / 2);
#pragma unroll
    for (int c = 0; c < D / 8; ++c) q.r[c] = *reinterpret_cast<const f32x4_t*>(p + 4 * c);
  }

  template <int BS, int D>
  static __device__ __forceinline__ f32x16_t scores(const QOperand<D>& q,
                                                    const unsigned char* ktile, int st,
                                                    int lane) {
    using L = TileLayout<float, BS, D>;
    const int key = st * kKeyStep + (lane & 31);
    const int h = lane >> 5;
    f32x16_t s = {};
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const f32x4_t k =
          *reinterpret_cast<const f32x4_t*>(ktile + L::chunk_offset(key, (D / 8) * h + c));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(k[e], q.r[c][e], s, 0, 0, 0);
    }
    return s;
  }

  // Instruction i of a 32-key step contracts the keys held in accumulator
  // register i: key 8 (i / 4) + 4 h + i % 4 for lane half h.
  template <int BS, int D>
  static __device__ __forceinline__ float accumulate(f32x16_t (&o)[D / 32],
                                                     const f32x16_t (&p)[BS / kKeyStep],
                                                     const unsigned char* vtile, int lane) {
    using L = TileLayout<float, BS, D>;
    const int h = lane >> 5;
    float sum = 0.f;
#pragma unroll
    for (int st = 0; st < BS / kKeyStep; ++st) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sum += p[st][i];
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int feature = dt * 32 + (lane & 31);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = st * kKeyStep + 8 * (i / 4) + 4 * h + (i % 4);
          const float va = *reinterpret_cast<const float*>(
              vtile + L::chunk_offset(row, feature >> 2) + (feature & 3) * 4);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(va, p[st][i], o[dt], 0, 0, 0);
        }
      }
    }
    return sum;
  }

  static __device__ __forceinline__ void store_o4(float* dst, float a, float b, float c,
                                                  float d) {
    f32x4_t w = {a, b, c, d};
    *reinterpret_cast<f32x4_t*>(dst) = w;
  }
};

// Partial state of a key-slice wave, stored for the merge: O^T in accumulator
// order [reg][lane], then m and l per lane.
template <int D>
constexpr int partial_bytes() {
  return (D / 32) * 16 * kWave * 4 + 2 * kWave * 4;
}

template <typename T, int BS, int D>
size_t lds_bytes(int group, int key_split, int nbuf, int M) {
  using L = TileLayout<T, BS, D>;
  constexpr int QW = BS / kQRows;
  const size_t tiles = (size_t)nbuf * key_split * L::kEntryBytes;
  const size_t merge = (size_t)QW * group * (key_split - 1) * partial_bytes<D>();
  const size_t words = (size_t)(group + 1) * ((M + 31) / 32);
  return (tiles > merge ? tiles : merge) + 4 * words;
}

// Iterator over the set bits of the union bitmap, in ascending block order.
struct BitIter {
  const uint32_t* words;
  int nwords;
  int w;
  uint32_t bits;
  __device__ __forceinline__ int next() {
    while (bits == 0) {
      if (++w >= nwords) return -1;
      bits = (uint32_t)uniform((int)words[w]);
    }
    const int j = w * 32 + __builtin_ctz(bits);
    bits &= bits - 1;
    return j;
  }
};

template <typename T, int BS, int D, int G>
__global__ __launch_bounds__(kWave* kMaxWaves) void bsa_fwd_kernel(FwdParams p) {
  using L = TileLayout<T, BS, D>;
  using O = Ops<T>;
  constexpr int QW = BS / kQRows;
  constexpr int KSTEPS = BS / kKeyStep;
  constexpr int SW = QW * G;  // waves per key slice
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(threadIdx.x / kWave);
  const int KS = p.key_split;
  const int qg = wave % QW;          // 32-row query group within the block
  const int g = (wave / QW) % G;     // query block within the workgroup
  const int ks = wave / SW;          // key slice
  const int slice_waves = SW;
  const int ws = wave % SW;          // wave index within its key slice

  const int M = p.M;
  const int ngroups = (M + G - 1) / G;
  const int wg = xcd_remap(blockIdx.x, p.num_wg);
  const int grp = wg % ngroups;
  const int bh = wg / ngroups;
  const int qb = grp * G + g;
  const bool has_rows = qb < M;
  const size_t head = (size_t)bh * p.N * D;
  const T* Q = static_cast<const T*>(p.q) + head;
  const T* K = static_cast<const T*>(p.k) + head;
  const T* V = static_cast<const T*>(p.v) + head;

  // ---- LDS: tile buffers [KS][kNumBuf][entry] | union bitmap | row bitmaps [G]
  const int MW = (M + 31) / 32;
  const int NB = p.nbuf;
  size_t tiles = (size_t)NB * KS * L::kEntryBytes;
  const size_t merge = (size_t)slice_waves * (KS - 1) * partial_bytes<D>();
  if (merge > tiles) tiles = merge;
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(lds + tiles);
  for (int i = threadIdx.x; i < (G + 1) * MW; i += blockDim.x) bitmap[i] = 0;
  __syncthreads();
  if (has_rows && qg == 0 && ks == 0) {
    const int rs = p.row_ptr[qb];
    const int re = p.row_ptr[qb + 1];
    for (int t = rs + lane; t < re; t += kWave) {
      const int j = p.col_idx[t];
      if (j >= 0 && j < M) {
        atomicOr(&bitmap[j >> 5], 1u << (j & 31));
        atomicOr(&bitmap[(1 + g) * MW + (j >> 5)], 1u << (j & 31));
      }
    }
  }

  // Q operand in registers while the bitmaps settle.
  typename O::template QOperand<D> qop;
  const int q0 = (has_rows ? qb : 0) * BS + qg * kQRows;
  O::template load_q<D>(qop, Q + (size_t)q0 * D, lane);
  __syncthreads();

  int U = 0;  // union size
  for (int w = lane; w < MW; w += kWave) U += __builtin_popcount(bitmap[w]);
  for (int off = 32; off > 0; off >>= 1) U += __shfl_xor(U, off);
  U = uniform(U);
  const int niter = (U + KS - 1) / KS;  // same trip count for every wave

  // This slice's entries are union entries ks, ks + KS, ...
  BitIter it{bitmap, MW, -1, 0};
  auto next_entry = [&]() -> int {  // next column of this slice, or -1
    int j = -1;
    for (int s = 0; s < KS; ++s) {
      const int x = it.next();
      if (s == ks) j = x;
    }
    return j;
  };
  unsigned char* slice_buf = lds + (size_t)ks * NB * L::kEntryBytes;
  Stage<T, BS, D, SW> stage;
  auto stage_load = [&](int j) {  // a missing entry stages block 0 (never used)
    stage.load(K, V, (j < 0 ? 0 : j) * BS, ws, lane);
  };

  f32x16_t o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16_t{};
  float m2 = -INFINITY;  // exponent offset (log2 domain) for this lane's query
  float lsum = 0.f;      // sum of exponentials over this lane half's keys
  const float c2 = p.scale_log2;
  const uint32_t* my_row = bitmap + (1 + g) * MW;
  // Pipeline (two buffers): entry i computes from LDS buffer i % 2 while
  // entry i+1 goes registers -> LDS buffer (i+1) % 2 and entry i+2 goes
  // global -> registers.  With one buffer, entry i+1 is written to LDS after a
  // second barrier that ends entry i's reads.
  int j_cur = next_entry();
  int j_next = next_entry();
  stage_load(j_cur);
  stage.store(slice_buf, ws, lane);
  if (niter > 1) stage_load(j_next);
  auto advance = [&](int i, unsigned char* dst) {
    if (i + 1 < niter) stage.store(dst, ws, lane);
    j_cur = j_next;
    j_next = next_entry();
    if (i + 2 < niter) stage_load(j_next);
  };
  for (int i = 0; i < niter; ++i) {
    const int j = j_cur;
    __syncthreads();  // entry i is in LDS; with two buffers nobody reads entry i-1 any more
    if (NB == 2) advance(i, slice_buf + ((i + 1) & 1) * L::kEntryBytes);
    const bool mine = j >= 0 && has_rows &&
                      ((((uint32_t)uniform((int)my_row[j >> 5])) >> (j & 31)) & 1u) != 0;
    if (mine) {
      const unsigned char* ktile = slice_buf + (NB == 2 ? (i & 1) : 0) * L::kEntryBytes;
      const unsigned char* vtile = ktile + L::kTileBytes;
      f32x16_t s[KSTEPS];
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st)
        s[st] = O::template scores<BS, D>(qop, ktile, st, lane);

      float mx = s[0][0];
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[st][r]);
      mx = halves_max(mx) * c2;
      if (__builtin_amdgcn_ballot_w64(mx > m2 + kLazyRescale) != 0) {
        const float m_new = fmaxf(m2, mx);
        const float alpha = fast_exp2(m2 - m_new);
        m2 = m_new;
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
      }
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[st][r] = fast_exp2(fmaf(s[st][r], c2, -m2));
      lsum += O::template accumulate<BS, D>(o, s, vtile, lane);
    }
    if (NB == 1) {
      __syncthreads();  // entry i is no longer read
      advance(i, slice_buf);
    }
  }

  // ---- merge the key slices: slices 1..KS-1 publish (O, m, l); slice 0 merges
  if (KS > 1) {
    __syncthreads();  // tile buffers are free
    float* part = reinterpret_cast<float*>(lds);
    constexpr int kPartFloats = partial_bytes<D>() / 4;
    if (ks > 0) {
      float* mine = part + (size_t)((ks - 1) * slice_waves + ws) * kPartFloats;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mine[(dt * 16 + r) * kWave + lane] = o[dt][r];
      mine[(D / 32) * 16 * kWave + lane] = m2;
      mine[(D / 32) * 16 * kWave + kWave + lane] = lsum;
    }
    __syncthreads();
    if (ks > 0) return;
    for (int w = 1; w < KS; ++w) {
      const float* other = part + (size_t)((w - 1) * slice_waves + ws) * kPartFloats;
      const float mo = other[(D / 32) * 16 * kWave + lane];
      const float lo = other[(D / 32) * 16 * kWave + kWave + lane];
      const float m_new = fmaxf(m2, mo);
      if (m_new == -INFINITY) continue;  // neither side has seen a key yet
      const float a_self = fast_exp2(m2 - m_new);
      const float a_other = fast_exp2(mo - m_new);
      lsum = lsum * a_self + lo * a_other;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          o[dt][r] = o[dt][r] * a_self + other[(dt * 16 + r) * kWave + lane] * a_other;
      m2 = m_new;
    }
  }
  if (!has_rows) return;

  // ---- epilogue: total row sum over both lane halves, normalise, store
  const float l_all = halves_sum(lsum);
  const float inv = l_all > 0.f ? 1.f / l_all : 0.f;
  const int h = lane >> 5;
  const int row = q0 + (lane & 31);
  T* Out = static_cast<T*>(p.o) + head + (size_t)row * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int gg = 0; gg < 4; ++gg)
      O::store_o4(Out + dt * 32 + 8 * gg + 4 * h, o[dt][4 * gg] * inv, o[dt][4 * gg + 1] * inv,
                  o[dt][4 * gg + 2] * inv, o[dt][4 * gg + 3] * inv);
  if (p.lse != nullptr && h == 0) {
    const float lse2 = l_all > 0.f ? m2 + log2f(l_all) : -INFINITY;
    p.lse[(size_t)bh * p.N + row] = lse2 * 0.69314718055994530942f;
  }
}

template <typename T, int BS, int D, int G>
bsa_status launch(const FwdParams& p, hipStream_t stream) {
  constexpr int QW = BS / kQRows;
  const size_t lds = lds_bytes<T, BS, D>(G, p.key_split, p.nbuf, p.M);
  if (lds > 64 * 1024) {
    static bool raised = false;  // one attribute call per instantiation
    if (!raised) {
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(&bsa_fwd_kernel<T, BS, D, G>),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(kMaxLds)) != hipSuccess)
        return BSA_ERR_HIP;
      raised = true;
    }
  }
  const dim3 block(kWave * QW * G * p.key_split);
  const dim3 grid(p.num_wg);
  hipLaunchKernelGGL((bsa_fwd_kernel<T, BS, D, G>), grid, block, lds, stream, p);
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

template <typename T, int BS, int D>
bsa_status launch_group(const FwdParams& p, hipStream_t stream) {
  switch (p.group) {
    case 1: return launch<T, BS, D, 1>(p, stream);
    case 2: return launch<T, BS, D, 2>(p, stream);
    case 4: return launch<T, BS, D, 4>(p, stream);
    default: return BSA_ERR_INVALID_ARGUMENT;
  }
}

template <typename T>
bsa_status dispatch(const FwdParams& p, int bs, int d, hipStream_t stream) {
  if (bs == 32 && d == 64) return launch_group<T, 32, 64>(p, stream);
  if (bs == 32 && d == 128) return launch_group<T, 32, 128>(p, stream);
  if (bs == 64 && d == 64) return launch_group<T, 64, 64>(p, stream);
  if (bs == 64 && d == 128) return launch_group<T, 64, 128>(p, stream);
  return BSA_ERR_INVALID_ARGUMENT;
}

size_t lds_for(int dtype, int bs, int d, int group, int ks, int nbuf, int M) {
  if (dtype == BSA_DTYPE_F32) {
    if (bs == 32) return d == 64 ? lds_bytes<float, 32, 64>(group, ks, nbuf, M)
                                 : lds_bytes<float, 32, 128>(group, ks, nbuf, M);
    return d == 64 ? lds_bytes<float, 64, 64>(group, ks, nbuf, M)
                   : lds_bytes<float, 64, 128>(group, ks, nbuf, M);
  }
  if (bs == 32) return d == 64 ? lds_bytes<__bf16, 32, 64>(group, ks, nbuf, M)
                               : lds_bytes<__bf16, 32, 128>(group, ks, nbuf, M);
  return d == 64 ? lds_bytes<__bf16, 64, 64>(group, ks, nbuf, M)
                 : lds_bytes<__bf16, 64, 128>(group, ks, nbuf, M);
}

// Workgroup shape.  Large grids: G query blocks per workgroup share their K/V
// tiles (4 blocks of 32 rows, or 2 of 64).  Grids too small to give every
// SIMD ~4 waves: one query block per workgroup and the CSR row split over KS
// key-slice wave sets instead.  Two LDS entry buffers when they fit in
// kMaxLds, else one.
void choose_shape(int64_t bhm, int bs, int d, int dtype, int M, int* group, int* key_split,
                  int* nbuf) {
  constexpr int64_t kTargetWaves = 4 * 4 * 256;
  const int qw = bs / kQRows;
  auto fits = [&](int g, int ks, int nb) { return lds_for(dtype, bs, d, g, ks, nb, M) <= kMaxLds; };
  int g = 1, ks = 1;
  if (bhm * qw >= 2 * kTargetWaves) {
    g = bs == 32 ? 4 : 2;
  } else {
    while (qw * ks * 2 <= kMaxWaves && bhm * qw * ks < kTargetWaves && fits(1, ks * 2, 2))
      ks *= 2;
  }
  *group = g;
  *key_split = ks;
  *nbuf = fits(g, ks, 2) ? 2 : 1;
}

}  // namespace

namespace {

bsa_status forward_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                        int32_t batch, int32_t heads, int32_t seq_len, int32_t head_dim,
                        int32_t block_size, int32_t dtype, const int32_t* row_ptr,
                        const int32_t* col_idx, int64_t nnz, float scale, int32_t group,
                        int32_t key_split, void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || row_ptr == nullptr ||
      col_idx == nullptr)
    return BSA_ERR_NULL_POINTER;
  if (dtype != BSA_DTYPE_F32 && dtype != BSA_DTYPE_BF16) return BSA_ERR_INVALID_ARGUMENT;
  if (block_size != 32 && block_size != 64) return BSA_ERR_INVALID_ARGUMENT;
  if (head_dim != 64 && head_dim != 128) return BSA_ERR_INVALID_ARGUMENT;
  if (batch <= 0 || heads <= 0 || seq_len <= 0 || seq_len % block_size != 0) return BSA_ERR_SHAPE;
  if (!(scale == scale) || std::isinf(scale)) return BSA_ERR_INVALID_ARGUMENT;
  const int64_t M = seq_len / block_size;
  if (nnz < M || nnz > M * M) return BSA_ERR_SHAPE;
  if ((int64_t)batch * heads * seq_len > INT32_MAX) return BSA_ERR_SHAPE;  // LSE/row indices
  const uintptr_t align = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                          reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o);
  if (align % 16 != 0) return BSA_ERR_INVALID_ARGUMENT;

  FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.row_ptr = row_ptr;
  p.col_idx = col_idx;
  p.M = static_cast<int32_t>(M);
  p.N = seq_len;
  if (group == 0 && key_split == 0) {
    choose_shape((int64_t)batch * heads * M, block_size, head_dim, dtype, (int)M, &p.group,
                 &p.key_split, &p.nbuf);
  } else {
    const int qw = block_size / kQRows;
    if ((group != 1 && group != 2 && group != 4) || key_split < 1 ||
        qw * group * key_split > kMaxWaves)
      return BSA_ERR_INVALID_ARGUMENT;
    p.group = group;
    p.key_split = key_split;
    p.nbuf = lds_for(dtype, block_size, head_dim, group, key_split, 2, (int)M) <= kMaxLds ? 2 : 1;
  }
  if (lds_for(dtype, block_size, head_dim, p.group, p.key_split, p.nbuf, (int)M) > kMaxLds)
    return BSA_ERR_INVALID_ARGUMENT;
  const int64_t ngroups = (M + p.group - 1) / p.group;
  const int64_t num_wg = (int64_t)batch * heads * ngroups;
  if (num_wg > INT32_MAX) return BSA_ERR_SHAPE;
  p.num_wg = static_cast<int32_t>(num_wg);
  const float s = scale > 0.f ? scale : 1.0f / std::sqrt(static_cast<float>(head_dim));
  p.scale_log2 = s * 1.4426950408889634f;

  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale, non-sticky error from earlier calls
  if (dtype == BSA_DTYPE_F32) return dispatch<float>(p, block_size, head_dim, st);
  return dispatch<__bf16>(p, block_size, head_dim, st);
}

}  // namespace

extern "C" bsa_status bsa_forward(const void* q, const void* k, const void* v, void* o,
                                  float* lse, int32_t batch, int32_t heads, int32_t seq_len,
                                  int32_t head_dim, int32_t block_size, int32_t dtype,
                                  const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                                  float scale, void* stream) {
  return forward_impl(q, k, v, o, lse, batch, heads, seq_len, head_dim, block_size, dtype,
                      row_ptr, col_idx, nnz, scale, 0, 0, stream);
}

extern "C" bsa_status bsa_forward_ex(const void* q, const void* k, const void* v, void* o,
                                     float* lse, int32_t batch, int32_t heads, int32_t seq_len,
                                     int32_t head_dim, int32_t block_size, int32_t dtype,
                                     const int32_t* row_ptr, const int32_t* col_idx,
                                     int64_t nnz, float scale, int32_t group,
                                     int32_t key_split, void* stream) {
  return forward_impl(q, k, v, o, lse, batch, heads, seq_len, head_dim, block_size, dtype,
                      row_ptr, col_idx, nnz, scale, group, key_split, stream);
}
