// Shared device code of the forward and backward kernels for gfx950:
// vector types, the LDS tile layout of K/V (or Q/dO) blocks, the MFMA
// operand loaders and products on those tiles, and the copy/barrier
// primitives of the LDS pipelines.
//
// MFMA layouts (v_mfma_f32_32x32x16_bf16): accumulator lane l, register i
// holds row 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32.  A product
// X^T = R C^T keeps the rows R of a tile (keys, or queries) as MFMA rows read
// from LDS and the 32 rows C a wave owns in registers as the B operand, so
// every lane holds one column (one query, or one key).  A product
// Y^T = T^T X packs X's accumulator (bf16) as the B operand directly, with the
// matching key order kappa(h, j) = 16 sc + 8 (j / 4) + 4 h + j % 4 taken on
// the A side through transposing LDS reads of tile T.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <type_traits>

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
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

  // XOR key of row r: a bit-reversed row index, chosen so that (a) 16 rows
  // read at the same chunk hit 16 different 16-byte bank groups and (b) the
  // transpose reads (4 consecutive rows x 4 consecutive chunks) do too.  It
  // depends on r mod 16 only, so per-lane offsets computed for rows 0..15
  // hold for every row at a multiple of 16 further on.
  static __device__ __forceinline__ int swz(int r) {
    if constexpr (kChunksPerRow == 8) {  // 128-byte rows: two rows per 256-byte bank line
      const int t = (r >> 1) & 7;
      return ((t & 1) << 2) | (t & 2) | ((t >> 2) & 1);
    } else {
      const int t = r & 15;
      const int rev = ((t & 1) << 3) | ((t & 2) << 1) | ((t & 4) >> 1) | ((t & 8) >> 3);
      return rev & (kChunksPerRow - 1);
    }
  }
  static __device__ __forceinline__ int chunk_offset(int r, int c) {
    return r * kRowBytes + ((c ^ swz(r)) << 4);
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

  // Per-lane LDS byte offsets of the operand reads, relative to the LDS base
  // of the slice's buffer 0 (plus that base).  Valid for every 32-key step
  // and 16-key sub-step: those move by multiples of 16 rows.
  template <int BS, int D>
  struct Offsets {
    int k[D / 16];     // K chunk 2c + h of key row lane % 32
    int v[2][D / 32];  // transpose-read address, rows +0 / +8, feature tile dt
    __device__ __forceinline__ void init(int lane, int base) {
      using L = TileLayout<__bf16, BS, D>;
      const int h = lane >> 5;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) k[c] = base + L::chunk_offset(lane & 31, 2 * c + h);
      // In each 16-lane group, lane 4k + q addresses the 4 features
      // (feature0 + 4q ..) of key row k; the hardware returns to lane i
      // feature0 + i of rows k = 0..3.
      const int g4 = lane >> 4;
      const int i = lane & 15;
      const int row = 4 * (g4 >> 1) + (i >> 2);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int feature = dt * 32 + 16 * (g4 & 1) + 4 * (i & 3);
        const int half = (feature & 7) * 2;
        v[0][dt] = base + L::kTileBytes + L::chunk_offset(row, feature >> 3) + half;
        v[1][dt] = base + L::kTileBytes + L::chunk_offset(row + 8, feature >> 3) + half;
      }
    }
  };

  // S^T for 32-key step st of the entry at byte `entry` (a constant) past
  // the offsets' base: A operand (lane = key, half h) = K[key][16c + 8h .. +8].
  template <int BS, int D>
  static __device__ __forceinline__ f32x16_t scores(const QOperand<D>& q,
                                                    const Offsets<BS, D>& off,
                                                    LDS_PTR(unsigned char) lds, int entry,
                                                    int st) {
    using L = TileLayout<__bf16, BS, D>;
    f32x16_t s = {};
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const u32x4_t k = *(LDS_PTR(const u32x4_t))(lds + off.k[c] + entry +
                                                  st * kKeyStep * L::kRowBytes);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, k),
                                                  __builtin_bit_cast(bf16x8_t, q.r[c]), s, 0, 0,
                                                  0);
    }
    return s;
  }

  // S^T of all NS 32-key steps of the entry with the steps' chains
  // interleaved: feature chunk c of every step, then chunk c + 1, so that
  // independent accumulators alternate and each K read has more MFMAs ahead
  // of its use to land.
  template <int BS, int D, int NS>
  static __device__ __forceinline__ void scores_steps(const QOperand<D>& q,
                                                      const Offsets<BS, D>& off,
                                                      LDS_PTR(unsigned char) lds, int entry,
                                                      f32x16_t (&s)[NS]) {
    using L = TileLayout<__bf16, BS, D>;
#pragma unroll
    for (int st = 0; st < NS; ++st) s[st] = f32x16_t{};
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const u32x4_t k = *(LDS_PTR(const u32x4_t))(lds + off.k[c] + entry +
                                                    st * kKeyStep * L::kRowBytes);
        s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, k),
                                                        __builtin_bit_cast(bf16x8_t, q.r[c]),
                                                        s[st], 0, 0, 0);
      }
  }

  // Two score tiles of step st from one stage: a = A-tile . qa^T (the tile at
  // byte `ea`) and b = B-tile . qb^T (at `eb`), their MFMA chains
  // interleaved so that each has the other's work between its dependent
  // steps.
  template <int BS, int D>
  static __device__ __forceinline__ void scores_pair(const QOperand<D>& qa,
                                                     const QOperand<D>& qb,
                                                     const Offsets<BS, D>& off,
                                                     LDS_PTR(unsigned char) lds, int ea, int eb,
                                                     int st, f32x16_t& a, f32x16_t& b) {
    using L = TileLayout<__bf16, BS, D>;
    a = f32x16_t{};
    b = f32x16_t{};
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const int rows = st * kKeyStep * L::kRowBytes;
      const u32x4_t ka = *(LDS_PTR(const u32x4_t))(lds + off.k[c] + ea + rows);
      const u32x4_t kb = *(LDS_PTR(const u32x4_t))(lds + off.k[c] + eb + rows);
      a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ka),
                                                  __builtin_bit_cast(bf16x8_t, qa.r[c]), a, 0, 0,
                                                  0);
      b = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kb),
                                                  __builtin_bit_cast(bf16x8_t, qb.r[c]), b, 0, 0,
                                                  0);
    }
  }

  // V^T operand of step st, 16-key sub-step sc, feature tile dt: lane
  // (feature = 32 dt + lane % 32, half h) holds V[key][feature] for keys
  // kappa(h, j) = 32 st + 16 sc + 8 (j / 4) + 4 h + j % 4, j = 0..7: two
  // transpose loads, rows +0 and +8.
  template <int BS, int D>
  static __device__ __forceinline__ u32x4_t v_operand(const Offsets<BS, D>& off,
                                                      LDS_PTR(unsigned char) lds, int entry,
                                                      int st, int sc, int dt) {
    using L = TileLayout<__bf16, BS, D>;
    const int rows = (st * kKeyStep + 16 * sc) * L::kRowBytes;
    const u32x2_t lo = __builtin_bit_cast(
        u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                     (LDS_PTR(s16x4_t))(lds + off.v[0][dt] + entry + rows)));
    const u32x2_t hi = __builtin_bit_cast(
        u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                     (LDS_PTR(s16x4_t))(lds + off.v[1][dt] + entry + rows)));
    return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
  }

  // O^T += V^T P^T over 32-key step st of the entry; returns the sum of the
  // bf16-rounded P (the weights the product uses).
  template <int BS, int D>
  static __device__ __forceinline__ float accumulate(f32x16_t (&o)[D / 32], const f32x16_t& p,
                                                     const Offsets<BS, D>& off,
                                                     LDS_PTR(unsigned char) lds, int entry,
                                                     int st) {
    float sum = 0.f;
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int sc = 0; sc < 2; ++sc) {
      // The four packed words are built as separate scalars: reading dot2
      // operands out of a 128-bit vector miscompiles (every v_dot2c read
      // the first word).
      uint32_t w4[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        w4[w] = pack_bf16x2(p[8 * sc + 2 * w], p[8 * sc + 2 * w + 1]);
        sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w4[w]), ones, sum,
                                              false);
      }
      const u32x4_t pb = {w4[0], w4[1], w4[2], w4[3]};
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const u32x4_t va = v_operand<BS, D>(off, lds, entry, st, sc, dt);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, va),
                                                        __builtin_bit_cast(bf16x8_t, pb), o[dt],
                                                        0, 0, 0);
      }
    }
    return sum;
  }

  // O^T += V^T P^T over 32-key step st, with P given as its eight packed
  // bf16 words (w[4 sc + k] holds P[8 sc + 2k], P[8 sc + 2k + 1]).
  template <int BS, int D>
  static __device__ __forceinline__ void accumulate_words(f32x16_t (&o)[D / 32],
                                                          const uint32_t (&w)[8],
                                                          const Offsets<BS, D>& off,
                                                          LDS_PTR(unsigned char) lds, int entry,
                                                          int st) {
#pragma unroll
    for (int sc = 0; sc < 2; ++sc) {
      const u32x4_t pb = {w[4 * sc], w[4 * sc + 1], w[4 * sc + 2], w[4 * sc + 3]};
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const u32x4_t va = v_operand<BS, D>(off, lds, entry, st, sc, dt);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, va),
                                                        __builtin_bit_cast(bf16x8_t, pb), o[dt],
                                                        0, 0, 0);
      }
    }
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
  struct Offsets {
    int lane;
    int base;
    __device__ __forceinline__ void init(int l, int b) {
      lane = l;
      base = b;
    }
  };

  template <int BS, int D>
  static __device__ __forceinline__ f32x16_t scores(const QOperand<D>& q,
                                                    const Offsets<BS, D>& off,
                                                    LDS_PTR(unsigned char) lds, int entry,
                                                    int st) {
    using L = TileLayout<float, BS, D>;
    const int key = st * kKeyStep + (off.lane & 31);
    const int h = off.lane >> 5;
    f32x16_t s = {};
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const f32x4_t k = *(LDS_PTR(const f32x4_t))(lds + off.base + entry +
                                                   L::chunk_offset(key, (D / 8) * h + c));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(k[e], q.r[c][e], s, 0, 0, 0);
    }
    return s;
  }

  // Instruction i of a 32-key step contracts the keys held in accumulator
  // register i: key 8 (i / 4) + 4 h + i % 4 for lane half h.
  template <int BS, int D>
  static __device__ __forceinline__ float accumulate(f32x16_t (&o)[D / 32], const f32x16_t& p,
                                                     const Offsets<BS, D>& off,
                                                     LDS_PTR(unsigned char) lds, int entry,
                                                     int st) {
    using L = TileLayout<float, BS, D>;
    const int h = off.lane >> 5;
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += p[i];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int feature = dt * 32 + (off.lane & 31);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = st * kKeyStep + 8 * (i / 4) + 4 * h + (i % 4);
        const float va = *(LDS_PTR(const float))(lds + off.base + entry + L::kTileBytes +
                                                 L::chunk_offset(row, feature >> 2) +
                                                 (feature & 3) * 4);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(va, p[i], o[dt], 0, 0, 0);
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

// Stores a wave's 32 rows x D of an accumulator in the O^T layout (lane =
// row, register 4 g + e of tile dt = element 32 dt + 8 g + 4 h + e), scaled
// by `mul` and rounded to T, through the wave's LDS region `st` (32 D
// sizeof(T) bytes): written row-major with 16-byte chunks XOR-swizzled by row
// (8 bank groups), read back as 16-byte chunks of consecutive rows and
// stored to rows dst0 + r D.  Each lane then issues whole 16-byte stores
// instead of 8-byte pieces, non-temporal (they fill whole lines and are not
// read back, so they do not push the K/V tiles out of L2).
template <typename T, int D>
__device__ __forceinline__ void store_rows_lds(T* dst0, const f32x16_t (&x)[D / 32], float mul,
                                               int lane, LDS_PTR(unsigned char) st) {
  constexpr int kRowB = D * (int)sizeof(T);
  constexpr int kCpr = kRowB / 16;
  const int h = lane >> 5;
  const int r = lane & 31;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int byte = (32 * dt + 8 * g + 4 * h) * (int)sizeof(T);
      LDS_PTR(unsigned char) dst = st + r * kRowB + (((byte >> 4) ^ (r & 7)) << 4) + (byte & 15);
      const float a0 = x[dt][4 * g] * mul, a1 = x[dt][4 * g + 1] * mul;
      const float a2 = x[dt][4 * g + 2] * mul, a3 = x[dt][4 * g + 3] * mul;
      if constexpr (std::is_same<T, __bf16>::value)
        *(LDS_PTR(u32x2_t))dst = u32x2_t{pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)};
      else
        *(LDS_PTR(f32x4_t))dst = f32x4_t{a0, a1, a2, a3};
    }
#pragma unroll
  for (int i = 0; i < 32 * kCpr / kWave; ++i) {
    const int k = lane + kWave * i;
    const int rr = k / kCpr, c = k % kCpr;
    const u32x4_t v = *(LDS_PTR(const u32x4_t))(st + rr * kRowB + ((c ^ (rr & 7)) << 4));
    // non-temporal: the output is not read again here, and whole 16-byte
    // chunks of consecutive rows fill whole lines, so it need not occupy L2
    __builtin_nontemporal_store(
        v, reinterpret_cast<u32x4_t*>(reinterpret_cast<unsigned char*>(dst0) +
                                      (size_t)rr * kRowB + c * 16));
  }
}

// As store_rows_lds, for the NT tiles T0 .. T0 + NT - 1 of the accumulator
// only (columns 32 T0 .. 32 (T0 + NT) - 1 of each row): the rows are staged
// NT * 32 sizeof(T) bytes wide, and the stores go to dst0 + r D + 32 T0.
template <typename T, int D, int T0, int NT>
__device__ __forceinline__ void store_cols_lds(T* dst0, const f32x16_t (&x)[D / 32], float mul,
                                               int lane, LDS_PTR(unsigned char) st) {
  constexpr int kRowB = D * (int)sizeof(T);        // global row stride
  constexpr int kPartB = NT * 32 * (int)sizeof(T);  // staged row
  constexpr int kCpr = kPartB / 16;
  constexpr int kSwz = kCpr < 8 ? kCpr - 1 : 7;
  static_assert(T0 + NT <= D / 32 && (32 * kCpr) % kWave == 0, "column tiles");
  const int h = lane >> 5;
  const int r = lane & 31;
#pragma unroll
  for (int dt = 0; dt < NT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int byte = (32 * dt + 8 * g + 4 * h) * (int)sizeof(T);
      LDS_PTR(unsigned char) dst = st + r * kPartB + (((byte >> 4) ^ (r & kSwz)) << 4) + (byte & 15);
      const float a0 = x[T0 + dt][4 * g] * mul, a1 = x[T0 + dt][4 * g + 1] * mul;
      const float a2 = x[T0 + dt][4 * g + 2] * mul, a3 = x[T0 + dt][4 * g + 3] * mul;
      if constexpr (std::is_same<T, __bf16>::value)
        *(LDS_PTR(u32x2_t))dst = u32x2_t{pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)};
      else
        *(LDS_PTR(f32x4_t))dst = f32x4_t{a0, a1, a2, a3};
    }
  unsigned char* const base = reinterpret_cast<unsigned char*>(dst0) + T0 * 32 * (int)sizeof(T);
#pragma unroll
  for (int i = 0; i < 32 * kCpr / kWave; ++i) {
    const int k = lane + kWave * i;
    const int rr = k / kCpr, c = k % kCpr;
    const u32x4_t v = *(LDS_PTR(const u32x4_t))(st + rr * kPartB + ((c ^ (rr & kSwz)) << 4));
    u32x4_t* const out = reinterpret_cast<u32x4_t*>(base + (size_t)rr * kRowB + c * 16);
    // rows narrower than a 128-byte line leave the other part of the line to
    // another wave: those stores go through L2, which merges the two halves
    if constexpr (kPartB >= 128) __builtin_nontemporal_store(v, out);
    else *out = v;
  }
}

// s_waitcnt: vector-memory count <= n and LDS/scalar count == 0.
template <int n>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  // gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  __builtin_amdgcn_s_waitcnt((n & 0xF) | (0x7 << 4) | (0x0 << 8) | ((n >> 4) << 14));
}

// s_waitcnt: LDS/scalar count == 0, vector-memory count left as it is.
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
}

// Direct-to-LDS copy of 16 bytes per lane: lane i reads sbase + voff (its
// own offset) and the data lands at LDS byte address m0 + 16 i.  Written as
// asm so that the compiler does not add waits for these copies in front of
// LDS reads of other buffers; the kernel waits for them itself (s_waitcnt
// vmcnt before the barrier that publishes a buffer).  The asm has no register
// outputs.  It sets M0, which nothing else in these kernels uses.
// The base and M0 must be wave-uniform; readfirstlane states that to the
// compiler, which then keeps them in SGPRs (a no-op when they already are).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t b = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  return reinterpret_cast<const void*>(lo | (hi << 32));
}

__device__ __forceinline__ void lds_dma16(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(uniform_ptr(sbase)),
                 "s"((uint32_t)__builtin_amdgcn_readfirstlane((int)m0))
               : "memory", "m0");
}

// N (1, 2 or 4) such copies behind one M0 write.  Copy c reads
// sbase + voff[c] + c KB and lands at m0 + c KB + 16 i: the instruction's
// immediate offset is added to both the global and the LDS address, so the
// caller passes voff[c] = (its global offset) - c KB.  The offsets stay
// within the signed 13-bit field (at most 3 KB).
template <int N>
__device__ __forceinline__ void lds_dma16_run(const void* sbase, const uint32_t (&voff)[N],
                                              uint32_t m0) {
  static_assert(N == 1 || N == 2 || N == 4, "runs of 1, 2 or 4 copies");
  const void* b = uniform_ptr(sbase);
  const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)m0);
  if constexpr (N == 1) {
    lds_dma16(b, voff[0], m);
  } else if constexpr (N == 2) {
    asm volatile(
        "s_mov_b32 m0, %3\n\t"
        "global_load_lds_dwordx4 %0, %2\n\t"
        "global_load_lds_dwordx4 %1, %2 offset:1024"
        :
        : "v"(voff[0]), "v"(voff[1]), "s"(b), "s"(m)
        : "memory", "m0");
  } else {
    asm volatile(
        "s_mov_b32 m0, %5\n\t"
        "global_load_lds_dwordx4 %0, %4\n\t"
        "global_load_lds_dwordx4 %1, %4 offset:1024\n\t"
        "global_load_lds_dwordx4 %2, %4 offset:2048\n\t"
        "global_load_lds_dwordx4 %3, %4 offset:3072"
        :
        : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(b), "s"(m)
        : "memory", "m0");
  }
}

// Longest run length (4, 2 or 1) that divides both n and m.
constexpr int dma_run(int n, int m) {
  return n % 4 == 0 && m % 4 == 0 ? 4 : n % 2 == 0 && m % 2 == 0 ? 2 : 1;
}

// Workgroup barrier without a memory fence: the caller has already waited for
// the memory operations the barrier publishes.  The empty asm statements keep
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


// Direct-to-LDS copy of 4 bytes per lane (same rules as lds_dma16): lane i's
// dword lands at LDS byte address m0 + 4 i.
__device__ __forceinline__ void lds_dma4(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(uniform_ptr(sbase)),
                 "s"((uint32_t)__builtin_amdgcn_readfirstlane((int)m0))
               : "memory", "m0");
}

// Host: whether a once-per-device action (raising a kernel's dynamic LDS
// limit, which is a per-device attribute) is still due on the current
// device.  `done` holds one bit per device (devices past 63: always due);
// mark_done sets it after the action succeeded.
inline bool due_on_device(const std::atomic<uint64_t>& done, uint64_t* bit) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 64;
  *bit = dev >= 0 && dev < 64 ? (1ull << dev) : 0;
  return *bit == 0 || (done.load(std::memory_order_acquire) & *bit) == 0;
}
inline void mark_done(std::atomic<uint64_t>& done, uint64_t bit) {
  done.fetch_or(bit, std::memory_order_acq_rel);
}

}  // namespace
