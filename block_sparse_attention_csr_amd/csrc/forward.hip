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
// Mapping onto CDNA4:
//  * one workgroup per (b, h, qb); a wave owns 32 query rows (block 64 -> 2
//    query waves) and, when the grid is small, the CSR row is split across
//    KS key-slice waves whose partial results are merged through LDS;
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys = MFMA rows, queries =
//    MFMA columns), so each lane holds 16 scores of ONE query: the row max
//    and row sum are in-lane plus one exchange between the two lane halves;
//  * P stays in registers: the S^T accumulator layout is exactly the B
//    operand layout of O^T = V^T P^T (key order permuted consistently in V);
//  * Q lives in VGPRs for the whole row; K tiles go straight from global
//    memory to MFMA operand registers (each lane reads 16 contiguous bytes of
//    one key row); V tiles are staged transposed in wave-private LDS so that
//    each lane can read 8 consecutive keys of one feature column;
//  * online softmax in the log2 domain (exp2 with scale * log2(e) folded in);
//  * workgroup ids are remapped so that the query blocks of one (b, h) run on
//    one XCD and share that XCD's L2.
// The fp32 variant uses v_mfma_f32_32x32x2_f32 with the same layouts.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "bsa.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kQRows = 32;     // query rows per wave
constexpr int kKeyStep = 32;   // keys per inner step
constexpr int kNumXcd = 8;
constexpr int kMaxKeySplit = 4;
constexpr int kVtPad = 4;      // LDS row padding (elements) of the transposed V tile

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int32_t M;          // query/key blocks per sequence
  int32_t N;          // sequence length
  int32_t num_units;  // batch * heads * M
  int32_t key_split;  // KS: waves sharing one CSR row
  float scale_log2;   // scale * log2(e)
};

// Workgroups are dispatched round-robin over the XCDs.  Give each XCD a
// contiguous range of (b, h, qb) units so that the query blocks of one head
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

__device__ __forceinline__ void wave_lds_fence() {
  // LDS traffic of one wave is processed in order; this only stops the
  // compiler from moving LDS accesses across the staging boundary.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t f = {lo, hi};
  bf16x2_t b = __builtin_convertvector(f, bf16x2_t);  // round to nearest even
  return __builtin_bit_cast(uint32_t, b);
}

template <typename T>
struct Tile;

// ---------------------------------------------------------------- bf16 tiles
template <>
struct Tile<__bf16> {
  // LDS: transposed V step, vt[d][key], key-contiguous, padded rows.
  template <int D>
  static constexpr int vt_elems() { return D * (kKeyStep + kVtPad); }
  static constexpr int elem_bytes = 2;

  template <int D>
  struct QOperand { u32x4_t r[D / 16]; };

  // Lane (query = lane % 32, half h = lane / 32) holds Q[query][16c + 8h .. +8].
  template <int D>
  static __device__ __forceinline__ void load_q(QOperand<D>& q, const __bf16* Q, int lane) {
    const __bf16* p = Q + (size_t)(lane & 31) * D + (lane >> 5) * 8;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) q.r[c] = *reinterpret_cast<const u32x4_t*>(p + 16 * c);
  }

  // K operand of one 32-key step (lane = key, half h): K[key][16c + 8h .. +8],
  // read straight from global memory into MFMA operand registers.
  template <int D>
  struct KRegs { u32x4_t r[D / 16]; };

  template <int D>
  static __device__ __forceinline__ void load_k(KRegs<D>& k, const __bf16* Kstep, int lane) {
    const __bf16* p = Kstep + (size_t)(lane & 31) * D + (lane >> 5) * 8;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) k.r[c] = *reinterpret_cast<const u32x4_t*>(p + 16 * c);
  }

  // S^T[key][query] = sum over features of K[key][f] Q[query][f].
  template <int D>
  static __device__ __forceinline__ f32x16_t scores(const QOperand<D>& q, const KRegs<D>& k) {
    f32x16_t s = {};
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, k.r[c]),
                                                  __builtin_bit_cast(bf16x8_t, q.r[c]), s, 0, 0,
                                                  0);
    return s;
  }

  // V rows of one 32-key step in registers.  Lane handles key pairs
  // (2r, 2r+1), r = lane % 16, and 8-feature pieces (lane / 16) + 4u.
  template <int D>
  struct VRegs { u32x4_t a[D / 32], b[D / 32]; };

  template <int D>
  static __device__ __forceinline__ void load_v(VRegs<D>& v, const __bf16* Vstep, int lane) {
    const int r = lane & 15;
#pragma unroll
    for (int u = 0; u < D / 32; ++u) {
      const int piece = (lane >> 4) + 4 * u;
      const __bf16* src = Vstep + (size_t)(2 * r) * D + piece * 8;
      v.a[u] = *reinterpret_cast<const u32x4_t*>(src);
      v.b[u] = *reinterpret_cast<const u32x4_t*>(src + D);
    }
  }

  // Store the step transposed into vt[D][32 + pad]: each 32-bit LDS word
  // holds one feature of the two adjacent keys (2r, 2r+1).
  template <int D>
  static __device__ __forceinline__ void store_vt(uint16_t* vt, const VRegs<D>& v, int lane) {
    constexpr int kStride = kKeyStep + kVtPad;
    const int r = lane & 15;
#pragma unroll
    for (int u = 0; u < D / 32; ++u) {
      const int piece = (lane >> 4) + 4 * u;
      uint16_t* dst = vt + (piece * 8) * kStride + 2 * r;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // feature 2w: low halves of a[w], b[w]; feature 2w+1: high halves.
        const uint32_t lo = __builtin_amdgcn_perm(v.b[u][w], v.a[u][w], 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(v.b[u][w], v.a[u][w], 0x07060302u);
        *reinterpret_cast<uint32_t*>(dst + (2 * w) * kStride) = lo;
        *reinterpret_cast<uint32_t*>(dst + (2 * w + 1) * kStride) = hi;
      }
    }
  }

  // O^T += V^T P^T for one 32-key step.  P (fp32, S^T accumulator layout) is
  // packed to bf16 in place as the B operand; key kappa(h, j, sc) =
  // 16 sc + 8 (j / 4) + 4 h + j % 4 for element j of 16-key sub-step sc.
  template <int D>
  static __device__ __forceinline__ void accumulate(f32x16_t (&o)[D / 32], const f32x16_t& p,
                                                    const uint16_t* vt, int lane) {
    constexpr int kStride = kKeyStep + kVtPad;
    const int h = lane >> 5;
#pragma unroll
    for (int sc = 0; sc < 2; ++sc) {
      u32x4_t pb;
      pb[0] = pack_bf16x2(p[8 * sc + 0], p[8 * sc + 1]);
      pb[1] = pack_bf16x2(p[8 * sc + 2], p[8 * sc + 3]);
      pb[2] = pack_bf16x2(p[8 * sc + 4], p[8 * sc + 5]);
      pb[3] = pack_bf16x2(p[8 * sc + 6], p[8 * sc + 7]);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const uint16_t* row = vt + (dt * 32 + (lane & 31)) * kStride + 16 * sc + 4 * h;
        const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(row);
        const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(row + 8);
        const u32x4_t va = {lo[0], lo[1], hi[0], hi[1]};
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, va),
                                                        __builtin_bit_cast(bf16x8_t, pb), o[dt],
                                                        0, 0, 0);
      }
    }
  }

  // Lane holds O^T[d = 32 dt + 8 g + 4 h + e][query], e = 0..3: 4 consecutive
  // features of one output row.
  static __device__ __forceinline__ void store_o4(__bf16* dst, float a, float b, float c,
                                                  float d) {
    u32x2_t w = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
    *reinterpret_cast<u32x2_t*>(dst) = w;
  }
};

// ---------------------------------------------------------------- fp32 tiles
template <>
struct Tile<float> {
  template <int D>
  static constexpr int vt_elems() { return D * (kKeyStep + kVtPad); }
  static constexpr int elem_bytes = 4;

  template <int D>
  struct QOperand { f32x4_t r[D / 8]; };

  // v_mfma_f32_32x32x2_f32 contracts 2 features per instruction, one per lane
  // half.  Lane (query, h) holds Q[query][(D/2) h + c] for c = 0 .. D/2-1.
  template <int D>
  static __device__ __forceinline__ void load_q(QOperand<D>& q, const float* Q, int lane) {
    const float* p = Q + (size_t)(lane & 31) * D + (lane >> 5) * (D / 2);
#pragma unroll
    for (int c = 0; c < D / 8; ++c) q.r[c] = *reinterpret_cast<const f32x4_t*>(p + 4 * c);
  }

  template <int D>
  struct KRegs { f32x4_t r[D / 8]; };

  // Lane (key, h) holds K[key][(D/2) h + c], c = 0 .. D/2-1.
  template <int D>
  static __device__ __forceinline__ void load_k(KRegs<D>& k, const float* Kstep, int lane) {
    const float* p = Kstep + (size_t)(lane & 31) * D + (lane >> 5) * (D / 2);
#pragma unroll
    for (int c = 0; c < D / 8; ++c) k.r[c] = *reinterpret_cast<const f32x4_t*>(p + 4 * c);
  }

  template <int D>
  static __device__ __forceinline__ f32x16_t scores(const QOperand<D>& q, const KRegs<D>& k) {
    f32x16_t s = {};
#pragma unroll
    for (int c = 0; c < D / 8; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(k.r[c][e], q.r[c][e], s, 0, 0, 0);
    return s;
  }

  // Lane handles key lane % 32 and 4-feature pieces (lane / 32) + 2u.
  template <int D>
  struct VRegs { f32x4_t a[D / 8]; };

  template <int D>
  static __device__ __forceinline__ void load_v(VRegs<D>& v, const float* Vstep, int lane) {
    const int key = lane & 31;
#pragma unroll
    for (int u = 0; u < D / 8; ++u) {
      const int piece = (lane >> 5) + 2 * u;
      v.a[u] = *reinterpret_cast<const f32x4_t*>(Vstep + (size_t)key * D + piece * 4);
    }
  }

  template <int D>
  static __device__ __forceinline__ void store_vt(float* vt, const VRegs<D>& v, int lane) {
    constexpr int kStride = kKeyStep + kVtPad;
    const int key = lane & 31;
#pragma unroll
    for (int u = 0; u < D / 8; ++u) {
      const int piece = (lane >> 5) + 2 * u;
#pragma unroll
      for (int e = 0; e < 4; ++e) vt[(piece * 4 + e) * kStride + key] = v.a[u][e];
    }
  }

  // Instruction i of a 32-key step contracts the keys held in accumulator
  // register i: key 8 (i / 4) + 4 h + i % 4 for lane half h.
  template <int D>
  static __device__ __forceinline__ void accumulate(f32x16_t (&o)[D / 32], const f32x16_t& p,
                                                    const float* vt, int lane) {
    constexpr int kStride = kKeyStep + kVtPad;
    const int h = lane >> 5;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const float* row = vt + (dt * 32 + (lane & 31)) * kStride + 4 * h;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4_t va = *reinterpret_cast<const f32x4_t*>(row + 8 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(va[e], p[4 * g + e], o[dt], 0, 0, 0);
      }
    }
  }

  static __device__ __forceinline__ void store_o4(float* dst, float a, float b, float c,
                                                  float d) {
    f32x4_t w = {a, b, c, d};
    *reinterpret_cast<f32x4_t*>(dst) = w;
  }
};

template <typename T, int BS, int D>
constexpr int vt_bytes_per_wave() {
  return Tile<T>::template vt_elems<D>() * Tile<T>::elem_bytes;
}

// Partial state of a key-slice wave, stored for the merge: O^T in accumulator
// order [reg][lane], then m and l per lane.
template <int D>
constexpr int partial_bytes() {
  return (D / 32) * 16 * kWave * 4 + 2 * kWave * 4;
}

template <typename T, int BS, int D>
size_t lds_bytes(int key_split) {
  constexpr int QW = BS / kQRows;
  const size_t stage = (size_t)QW * key_split * vt_bytes_per_wave<T, BS, D>();
  const size_t merge = (size_t)QW * (key_split - 1) * partial_bytes<D>();
  return stage > merge ? stage : merge;
}

template <typename T, int BS, int D>
__global__ __launch_bounds__(kWave * (BS / kQRows) * kMaxKeySplit) void bsa_fwd_kernel(
    FwdParams p) {
  using Ops = Tile<T>;
  using VtElem = typename std::conditional<std::is_same<T, float>::value, float, uint16_t>::type;
  constexpr int QW = BS / kQRows;
  constexpr int kSteps = BS / kKeyStep;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int qg = wave % QW;
  const int ks = wave / QW;
  const int KS = p.key_split;

  const int unit = xcd_remap(blockIdx.x, p.num_units);
  const int qb = unit % p.M;
  const int bh = unit / p.M;
  const size_t head = (size_t)bh * p.N * D;
  const T* Q = static_cast<const T*>(p.q) + head;
  const T* K = static_cast<const T*>(p.k) + head;
  const T* V = static_cast<const T*>(p.v) + head;
  const int q0 = qb * BS + qg * kQRows;

  VtElem* vt = reinterpret_cast<VtElem*>(lds) + (size_t)wave * Ops::template vt_elems<D>();

  typename Ops::template QOperand<D> qop;
  Ops::template load_q<D>(qop, Q + (size_t)q0 * D, lane);

  f32x16_t o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16_t{};
  float m2 = -INFINITY;  // running max of scale*log2(e)*score for this lane's query
  float lsum = 0.f;      // running sum over this lane half's keys
  const float c2 = p.scale_log2;

  // This wave's blocks are CSR entries rs + ks, rs + ks + KS, ...; each block
  // is BS / 32 steps of 32 keys.  Software pipeline: the K and V registers of
  // step s+1 are loaded while step s computes, and col_idx is read two blocks
  // ahead into scalar registers.
  const int rs = p.row_ptr[qb];
  const int re = p.row_ptr[qb + 1];
  const int nblk = (re - rs > ks) ? (re - rs - ks + KS - 1) / KS : 0;
  auto block_col = [&](int b) -> int { return p.col_idx[rs + ks + KS * b]; };
  auto key_of = [&](int j) -> int {  // first key row of block j, or -1 if out of range
    return (j >= 0 && j < p.M) ? j * BS : -1;
  };
  typename Ops::template KRegs<D> kn;
  typename Ops::template VRegs<D> vn;
  int key_next = nblk > 0 ? key_of(block_col(0)) : -1;  // block b
  int col_next2 = nblk > 1 ? block_col(1) : -1;         // block b + 1 (raw column)
  if (nblk > 0) {
    const size_t k0 = (size_t)(key_next < 0 ? 0 : key_next) * D;
    Ops::template load_k<D>(kn, K + k0, lane);
    Ops::template load_v<D>(vn, V + k0, lane);
  }

  for (int b = 0; b < nblk; ++b) {
    const int key_cur = key_next;
    key_next = key_of(col_next2);
    col_next2 = (b + 2 < nblk) ? block_col(b + 2) : -1;
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const typename Ops::template KRegs<D> kc = kn;
      const typename Ops::template VRegs<D> vc = vn;
      // prefetch the next step: the rest of this block, else the next block
      int pre = -1;
      if (st + 1 < kSteps) pre = key_cur < 0 ? 0 : key_cur + (st + 1) * kKeyStep;
      else if (b + 1 < nblk) pre = key_next < 0 ? 0 : key_next;
      if (pre >= 0) {
        Ops::template load_k<D>(kn, K + (size_t)pre * D, lane);
        Ops::template load_v<D>(vn, V + (size_t)pre * D, lane);
      }
      if (key_cur < 0) continue;

      f32x16_t s = Ops::template scores<D>(qop, kc);
      wave_lds_fence();
      Ops::template store_vt<D>(vt, vc, lane);

      float mx = s[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m2, mx * c2);
      const float alpha = fast_exp2(m2 - m_new);
      m2 = m_new;
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = fast_exp2(fmaf(s[i], c2, -m_new));
        ps += s[i];
      }
      lsum = lsum * alpha + ps;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;

      wave_lds_fence();
      Ops::template accumulate<D>(o, s, vt, lane);
    }
  }

  // Merge the key slices: slice waves 1..KS-1 publish (O, m, l); slice 0 merges.
  if (KS > 1) {
    __syncthreads();  // every wave is done with its V staging area
    float* part = reinterpret_cast<float*>(lds);
    constexpr int kPartFloats = partial_bytes<D>() / 4;
    if (ks > 0) {
      float* mine = part + (size_t)((ks - 1) * QW + qg) * kPartFloats;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mine[(dt * 16 + i) * kWave + lane] = o[dt][i];
      mine[(D / 32) * 16 * kWave + lane] = m2;
      mine[(D / 32) * 16 * kWave + kWave + lane] = lsum;
    }
    __syncthreads();
    if (ks > 0) return;
    for (int w = 1; w < KS; ++w) {
      const float* other = part + (size_t)((w - 1) * QW + qg) * kPartFloats;
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
        for (int i = 0; i < 16; ++i)
          o[dt][i] = o[dt][i] * a_self + other[(dt * 16 + i) * kWave + lane] * a_other;
      m2 = m_new;
    }
  }

  // Epilogue: total row sum over both lane halves, normalise, store.
  const float l_all = lsum + __shfl_xor(lsum, 32);
  const float inv = l_all > 0.f ? 1.f / l_all : 0.f;
  const int h = lane >> 5;
  const int row = q0 + (lane & 31);
  T* O = static_cast<T*>(p.o) + head + (size_t)row * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      Ops::store_o4(O + dt * 32 + 8 * g + 4 * h, o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv,
                    o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv);
  if (p.lse != nullptr && h == 0) {
    const float lse2 = l_all > 0.f ? m2 + log2f(l_all) : -INFINITY;
    p.lse[(size_t)bh * p.N + row] = lse2 * 0.69314718055994530942f;
  }
}

template <typename T, int BS, int D>
bsa_status launch(const FwdParams& p, hipStream_t stream) {
  constexpr int QW = BS / kQRows;
  const size_t lds = lds_bytes<T, BS, D>(p.key_split);
  const dim3 block(kWave * QW * p.key_split);
  const dim3 grid(p.num_units);
  hipLaunchKernelGGL((bsa_fwd_kernel<T, BS, D>), grid, block, lds, stream, p);
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

template <typename T>
bsa_status dispatch(const FwdParams& p, int bs, int d, hipStream_t stream) {
  if (bs == 32 && d == 64) return launch<T, 32, 64>(p, stream);
  if (bs == 32 && d == 128) return launch<T, 32, 128>(p, stream);
  if (bs == 64 && d == 64) return launch<T, 64, 64>(p, stream);
  if (bs == 64 && d == 128) return launch<T, 64, 128>(p, stream);
  return BSA_ERR_INVALID_ARGUMENT;
}

template <typename T>
size_t lds_for(int bs, int d, int ks) {
  if (bs == 32 && d == 64) return lds_bytes<T, 32, 64>(ks);
  if (bs == 32 && d == 128) return lds_bytes<T, 32, 128>(ks);
  if (bs == 64 && d == 64) return lds_bytes<T, 64, 64>(ks);
  return lds_bytes<T, 64, 128>(ks);
}

// Key-slice waves per CSR row: split only while the grid would leave SIMDs
// idle (fewer than ~4 waves per SIMD over 256 CUs), and only within 64 KB LDS.
int choose_key_split(int64_t units, int qw, int dtype, int bs, int d) {
  constexpr int64_t kTargetWaves = 4 * 4 * 256;
  int ks = 1;
  while (ks < kMaxKeySplit && units * qw * ks < kTargetWaves) {
    const int next = ks * 2;
    const size_t lds = dtype == BSA_DTYPE_F32 ? lds_for<float>(bs, d, next)
                                              : lds_for<__bf16>(bs, d, next);
    if (lds > 64 * 1024) break;
    ks = next;
  }
  return ks;
}

}  // namespace

extern "C" bsa_status bsa_forward(const void* q, const void* k, const void* v, void* o,
                                  float* lse, int32_t batch, int32_t heads, int32_t seq_len,
                                  int32_t head_dim, int32_t block_size, int32_t dtype,
                                  const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                                  float scale, void* stream) {
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
  const int64_t units = (int64_t)batch * heads * M;
  if (units > INT32_MAX) return BSA_ERR_SHAPE;
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
  p.num_units = static_cast<int32_t>(units);
  const float s = scale > 0.f ? scale : 1.0f / std::sqrt(static_cast<float>(head_dim));
  p.scale_log2 = s * 1.4426950408889634f;
  p.key_split = choose_key_split(units, block_size / kQRows, dtype, block_size, head_dim);

  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale, non-sticky error from earlier calls
  if (dtype == BSA_DTYPE_F32) return dispatch<float>(p, block_size, head_dim, st);
  return dispatch<__bf16>(p, block_size, head_dim, st);
}
