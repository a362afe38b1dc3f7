// Block-sparse attention decode for gfx950 (MI355X): one new token per
// sequence against a block-aligned KV cache.
//
// What is computed: the KV cache of sequence b holds L_b tokens and the new
// token is the last, at position t = L_b - 1 in block i = t / BS.  Its output
// is row t of the causal forward: softmax(scale q . K_p) V_p over the cached
// positions p <= t whose block the pattern row S(i) selects ("Block Sparse
// Attention: Log-Linear complexity sparse attention implementation",
// czchanglian.com, section 3.3 for the normalisation over the connected
// blocks; section 1 motivates the KV-cache use).  The log-sum-exp is written
// as well.
//
// Mapping: one workgroup of W waves per (batch, head).  The work is
// memory-bound (each cached K/V element is used once, by two multiply-adds),
// so it runs on the VALU, not on MFMA:
//  * The selected blocks are cut into units of KU keys, four 16-byte loads
//    per lane for K and four for V; lane l holds 16-byte chunk l % LPK of
//    the keys l / LPK + KPI n (n = 0..3), so every load instruction reads
//    one contiguous 1 KB run of the cache.
//  * Units are dealt round-robin to the waves; each wave loads its next unit
//    while it computes the current one, with an exact online softmax.
//  * A score is the chunk's partial dot product summed over the LPK lanes of
//    its key; the unit max over the key groups.  The cross-lane steps are
//    VALU lane moves (DPP within rows of 16 lanes, permlane swaps across
//    rows), with no LDS round trip in the loop.
//  * bf16 cache and query: the dot products run two elements per
//    instruction (v_dot2 on bf16 pairs); P V pairs two keys per element,
//    with P rounded to bf16 as the MFMA forward rounds it.  float32 data
//    keeps one fused multiply-add per element.
//  * Keys after the token only occur in the unit that holds it; there the
//    V chunks of those keys are zeroed (the cache beyond L_b may hold
//    anything, NaN included) and their scores set to -inf, so the other
//    units carry no per-element selection.
//  * At the end each wave sums its O over the key groups and the W waves
//    merge (O, m, l) through LDS.
//
// int8 caches (the log-linear page, section 6.3: KV cache in int8, attention
// in 16-bit floating point, one scale per block): codes convert exactly to
// float, each as (code + 128) from one unsigned-byte conversion, the 128
// taken off once per sum (q's chunk sum for the scores, the weight sum for
// O); a unit lies in one block, so its K scale multiplies the unit's scores
// and its V scale the unit's weights (the exponential sum uses the unscaled
// weights).  With a bf16 query and d = 128, the int8 products also run two
// per instruction: q is scaled by a power of two (exactly) into float16
// range, and byte permutes turn two biased codes into the f16 values
// 1024 + code + 128, exact (for the scores two elements of one key, for P V
// one element of two keys, against the two weights in f16); the 1152 offset
// is taken off once per chunk, or once at the end for O.  The same file holds the quantiser that writes such a
// cache: per (batch, head, block), scale = max|x| / 127 and
// code = rint(x / scale) clamped to [-127, 127], both in float32.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "bsa.h"
#include "mfma_tiles.h"

namespace {

constexpr int kDecodeWaves = 4;

struct DecParams {
  const void* q;
  const void* k;        // cache: q's type, or int8 codes
  const void* v;
  const float* k_scale;  // int8 caches: [batch, heads, M] per-block scales
  const float* v_scale;
  void* o;
  float* lse;
  const int32_t* seqlens;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int32_t heads;
  int32_t n_cap;       // cache capacity in tokens (multiple of the block size)
  int32_t M;           // n_cap / block size
  int32_t row_stride;  // row_ptr entries per head: M + 1 (one pattern per head) or 0
  float scale_log2;    // scale * log2(e)
};

template <typename TC, int BS, int D>
struct DecCfg {
  static constexpr int E = 16 / (int)sizeof(TC);  // cache elements per 16-byte chunk
  static constexpr int LPK = D / E;              // lanes per key
  static constexpr int KPI = kWave / LPK;        // keys per load instruction
  static constexpr int NI = BS / KPI < 4 ? BS / KPI : 4;  // loads per unit (K, and again V)
  static constexpr int KU = NI * KPI;            // keys per unit
  static constexpr int SUB = BS / KU;            // units per block
  static_assert(LPK <= 32 && SUB >= 1 && BS % KU == 0, "decode unit shape");
};

// A lane's value moved by a DPP pattern within each row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // lane i of 8 <- lane 7 - i
constexpr int kDppMirror = 0x140;      // lane i of 16 <- lane 15 - i
template <int R>
constexpr int dpp_ror() {  // lane i of 16 <- lane (i + R) mod 16
  return 0x120 + R;
}

// Sum (or max) of a lane's value with the lane 16 apart within its half of
// the wave (one v_permlane16_swap).
__device__ __forceinline__ float sum_rows16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_rows16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum (or max) over each aligned group of N lanes (N a power of two, 1 ..
// 64); every lane of the group receives it.  Steps below FROM are skipped:
// the value must then already be equal across each aligned group of FROM
// lanes.  Steps 4 and 8 pair the two halves of a group by mirroring, which
// needs exactly that equality (it holds after the steps before them).
template <int FROM, int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (FROM <= 1 && N >= 2) x += dpp_move<kDppXor1>(x);
  if constexpr (FROM <= 2 && N >= 4) x += dpp_move<kDppXor2>(x);
  if constexpr (FROM <= 4 && N >= 8) x += dpp_move<kDppHalfMirror>(x);
  if constexpr (FROM <= 8 && N >= 16) x += dpp_move<kDppMirror>(x);
  if constexpr (FROM <= 16 && N >= 32) x = sum_rows16(x);
  if constexpr (N >= 64) x = halves_sum(x);
  return x;
}
template <int FROM, int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (FROM <= 1 && N >= 2) x = __builtin_elementwise_maximum(x, dpp_move<kDppXor1>(x));
  if constexpr (FROM <= 2 && N >= 4) x = __builtin_elementwise_maximum(x, dpp_move<kDppXor2>(x));
  if constexpr (FROM <= 4 && N >= 8)
    x = __builtin_elementwise_maximum(x, dpp_move<kDppHalfMirror>(x));
  if constexpr (FROM <= 8 && N >= 16) x = __builtin_elementwise_maximum(x, dpp_move<kDppMirror>(x));
  if constexpr (FROM <= 16 && N >= 32) x = max_rows16(x);
  if constexpr (N >= 64) x = halves_max(x);
  return x;
}

// Sum over the lanes with the same lane % S (S a power of two, 1 .. 32): the
// 64 / S lanes of one residue class, each receiving it.  Any values.
template <int S>
__device__ __forceinline__ float stride_sum(float x) {
  if constexpr (S <= 1) x += dpp_move<kDppXor1>(x);
  if constexpr (S <= 2) x += dpp_move<dpp_ror<2>()>(x);
  if constexpr (S <= 4) x += dpp_move<dpp_ror<4>()>(x);
  if constexpr (S <= 8) x += dpp_move<dpp_ror<8>()>(x);
  if constexpr (S <= 16) x = sum_rows16(x);
  return halves_sum(x);
}

// The elements of a 16-byte chunk as floats (exact for every type).
template <typename T>
__device__ __forceinline__ void chunk_to_float(const u32x4_t& c, float* f) {
  if constexpr (std::is_same<T, int8_t>::value) {
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int b = 0; b < 4; ++b) f[4 * w + b] = (float)(int8_t)(c[w] >> (8 * b));
  } else if constexpr (std::is_same<T, __bf16>::value) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      f[2 * w] = __uint_as_float(c[w] << 16);
      f[2 * w + 1] = __uint_as_float(c[w] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) f[w] = __uint_as_float(c[w]);
  }
}

// int8 codes as floats plus 128 (one unsigned-byte conversion each; the
// caller takes the 128 off once per sum instead of once per element).
__device__ __forceinline__ void codes_to_float_biased(const u32x4_t& c, float* f) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t u = c[w] ^ 0x80808080u;
#pragma unroll
    for (int b = 0; b < 4; ++b) f[4 * w + b] = (float)((u >> (8 * b)) & 0xFFu);
  }
}

// Two biased int8 codes (bytes B0 and B0 + 1 of u, each code + 128) as the
// f16 pair (1024 + byte, 1024 + byte), exact: each byte under an 0x64
// exponent byte.
template <int B0>
__device__ __forceinline__ uint32_t biased_pair_f16(uint32_t u) {
  constexpr uint32_t sel = 0x04000400u | ((uint32_t)(B0 + 1) << 16) | (uint32_t)B0;
  return __builtin_amdgcn_perm(0x64646464u, u, sel);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c,
                                false);
}

template <typename T>
__device__ __forceinline__ void store_elem(T* dst, float x) {
  if constexpr (std::is_same<T, __bf16>::value) *dst = (__bf16)x;  // round to nearest even
  else *dst = x;
}

// E elements of q (type T) starting at `src`, as floats.
template <typename T, int E>
__device__ __forceinline__ void load_floats(const T* src, float* f) {
  constexpr int per = 16 / (int)sizeof(T);
#pragma unroll
  for (int c = 0; c < E / per; ++c)
    chunk_to_float<T>(*reinterpret_cast<const u32x4_t*>(src + c * per), f + c * per);
}

template <typename T, typename TC, int BS, int D>
__global__ __launch_bounds__(kWave * kDecodeWaves) void bsa_decode_kernel(DecParams p) {
  using C = DecCfg<TC, BS, D>;
  constexpr bool kInt8 = std::is_same<TC, int8_t>::value;
  constexpr bool kBf16Q = std::is_same<T, __bf16>::value;
  constexpr bool kDotBf16 = kBf16Q && std::is_same<TC, __bf16>::value;  // dot2 on bf16 pairs
  // dot2 on f16 pairs: at d = 128 (at d = 64 a sequence's units are too few
  // for it to repay the query's conversion, which lies on their critical path)
  constexpr bool kDotF16 = kBf16Q && kInt8 && D == 128;
  constexpr int W = kDecodeWaves;
  constexpr int E = C::E;
  constexpr int LPK = C::LPK;
  constexpr int KPI = C::KPI;
  constexpr int SUB = C::SUB;

  __shared__ float part[W][D + 2];  // per wave: O (unnormalised), m, l

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(threadIdx.x / kWave);
  const int bh = blockIdx.x;
  const int b = bh / p.heads;
  const int h = bh % p.heads;
  const int chunk = lane % LPK;  // 16-byte chunk of a key this lane holds
  const int kq = lane / LPK;     // key within a load instruction's group

  const int L = p.seqlens[b];
  const bool valid_len = L >= 1 && L <= p.n_cap;
  const int t = valid_len ? L - 1 : 0;
  const int qb = t / BS;
  const int32_t* row_ptr = p.row_ptr + (size_t)h * p.row_stride;
  const int rs = valid_len ? row_ptr[qb] : 0;
  const int re = valid_len ? row_ptr[qb + 1] : 0;
  const int nslots = (re - rs) * SUB;

  const size_t head = (size_t)bh * p.n_cap * D;
  const TC* K = static_cast<const TC*>(p.k) + head;
  const TC* V = static_cast<const TC*>(p.v) + head;

  // The lane's q elements: as floats (float32 data), as the raw bf16 pairs
  // (bf16 cache), or scaled by 2^-qexp into f16 pairs (int8 cache, bf16 q).
  float qf[E];
  load_floats<T, E>(static_cast<const T*>(p.q) + (size_t)bh * D + chunk * E, qf);
  uint32_t qw[E / 2];
  float qsum = 0.f;    // int8: sum of the lane's q elements (for the code offset)
  float qmul = 1.f;    // int8 with f16 q: 2^qexp, the scores' factor
  if constexpr (kDotBf16) {
#pragma unroll
    for (int w = 0; w < E / 2; ++w) qw[w] = pack_bf16x2(qf[2 * w], qf[2 * w + 1]);  // exact
  } else if constexpr (kDotF16) {
    // max|q| over the whole row (the LPK lanes of a key group hold all of it)
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(qf[e]));
    amax = group_max<1, LPK>(amax);
    // scale so that max|q| lands in [2^14, 2^15): every bf16 element then
    // converts to f16 exactly (bar those below 2^-28 max|q|, which the
    // float32 sum cannot see either)
    const int qexp = (amax > 0.f && amax < INFINITY) ? ilogbf(amax) - 14 : 0;
    qmul = ldexpf(1.f, qexp);
#pragma unroll
    for (int w = 0; w < E / 2; ++w) {
      const auto h2 = __builtin_amdgcn_cvt_pkrtz(ldexpf(qf[2 * w], -qexp),
                                                    ldexpf(qf[2 * w + 1], -qexp));
      qw[w] = __builtin_bit_cast(uint32_t, h2);
      qsum += (float)h2[0] + (float)h2[1];
    }
  } else if constexpr (kInt8) {
#pragma unroll
    for (int e = 0; e < E; ++e) qsum += qf[e];
  }

  // The row's entries, 64 at a time in one VGPR (lane l: entry base + l).
  int ent_base = -kWave;
  int ent = -1;
  auto entry = [&](int e) -> int {  // col_idx[rs + e], wave-uniform
    const int base = e & ~(kWave - 1);
    if (base != ent_base) {
      ent_base = base;
      const int idx = rs + base + lane;
      ent = idx < re ? p.col_idx[idx] : -1;
    }
    return __builtin_amdgcn_readlane(ent, e - base);
  };
  // First key of slot s (entry s / SUB, unit s % SUB), or -1 when the slot
  // holds no visible key: a block after the token's block, a unit after the
  // token, or an entry outside [0, M).
  auto slot_key = [&](int s) -> int {
    const int j = entry(s / SUB);
    if (j < 0 || j > qb) return -1;
    const int key0 = j * BS + (s % SUB) * C::KU;
    return key0 <= t ? key0 : -1;
  };
  auto next_slot = [&](int s, int& key0) -> int {
    for (; s < nslots; s += W) {
      key0 = slot_key(s);
      if (key0 >= 0) return s;
    }
    return nslots;
  };
  // A unit's loads: its K and V chunks and, for int8, its block's two scales
  // (so that no load is left for the compute to wait on).
  auto load = [&](int key0, u32x4_t (&kr)[C::NI], u32x4_t (&vr)[C::NI], f32x2_t& sc2) {
#pragma unroll
    for (int n = 0; n < C::NI; ++n) {
      const size_t off = (size_t)(key0 + n * KPI + kq) * D + chunk * E;
      kr[n] = *reinterpret_cast<const u32x4_t*>(K + off);
      vr[n] = *reinterpret_cast<const u32x4_t*>(V + off);
    }
    if constexpr (kInt8) {
      const size_t blk = (size_t)bh * p.M + key0 / BS;
      sc2 = f32x2_t{p.k_scale[blk], p.v_scale[blk]};
    }
  };

  const float c2 = p.scale_log2;
  float m2 = -INFINITY;  // running max of the scaled scores (log2 domain)
  float l = 0.f;         // this lane's share of the exponential sum
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  float pvsum = 0.f;  // int8: sum of the lane's V weights (for the code offset)

  // One unit: its keys' scores, the online-softmax update, and P V.
  auto unit = [&](int key0, u32x4_t (&kr)[C::NI], u32x4_t (&vr)[C::NI], const f32x2_t& scv) {
    // scores of the lane's keys key0 + KPI n + kq (scaled, log2 domain)
    // int8: the unit's block scales (the scores' and the weights' factors)
    const float ks = scv[0] * c2 * qmul;
    const float vs = scv[1];
    float sc[C::NI];
    float mx = -INFINITY;
#pragma unroll
    for (int n = 0; n < C::NI; ++n) {
      float d = 0.f;
      if constexpr (kDotBf16) {
#pragma unroll
        for (int w = 0; w < 4; ++w) d = dot2_bf16(kr[n][w], qw[w], d);
      } else if constexpr (kDotF16) {
        d = -1152.f * qsum;  // the pairs carry code + 1152
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t u = kr[n][w] ^ 0x80808080u;  // code + 128 per byte
          d = dot2_f16(biased_pair_f16<0>(u), qw[2 * w], d);
          d = dot2_f16(biased_pair_f16<2>(u), qw[2 * w + 1], d);
        }
      } else {
        float kf[E];
        if constexpr (kInt8) {
          codes_to_float_biased(kr[n], kf);  // code + 128
          d = -128.f * qsum;
        } else {
          chunk_to_float<TC>(kr[n], kf);
        }
#pragma unroll
        for (int e = 0; e < E; ++e) d = fmaf(qf[e], kf[e], d);
      }
      d = group_sum<1, LPK>(d) * ks;
      sc[n] = key0 + n * KPI + kq <= t ? d : -INFINITY;
      mx = __builtin_elementwise_maximum(mx, sc[n]);
    }
    mx = group_max<LPK, kWave>(mx);  // finite: the unit's first key is visible
    const float m_new = fmaxf(m2, mx);
    const float alpha = fast_exp2(m2 - m_new);  // 0 on the first unit (m2 = -inf)
    m2 = m_new;
    l *= alpha;
    pvsum *= alpha;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] *= alpha;
    // The unit that holds the token: the V chunks of the keys after it are
    // zeroed (their weights are 0 already), so that no value there, NaN
    // included, reaches O.
    if (key0 + C::KU - 1 > t) {
#pragma unroll
      for (int n = 0; n < C::NI; ++n) {
        const bool visible = key0 + n * KPI + kq <= t;
#pragma unroll
        for (int w = 0; w < 4; ++w) vr[n][w] = visible ? vr[n][w] : 0u;
      }
    }
    float pw[C::NI];  // the keys' weights (0 after the token)
#pragma unroll
    for (int n = 0; n < C::NI; ++n) {
      pw[n] = fast_exp2(sc[n] - m_new);
      l += pw[n];
      if constexpr (kInt8 && !kDotF16) pw[n] *= vs;  // (the f16 form scales per unit)
    }
    if constexpr (kDotBf16) {
      static_assert(C::NI % 2 == 0, "keys pair up for v_dot2");
#pragma unroll
      for (int n = 0; n < C::NI; n += 2) {
        const uint32_t pp = pack_bf16x2(pw[n], pw[n + 1]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // element 2w (low halves) and 2w + 1 (high halves) of the two keys
          const uint32_t lo = __builtin_amdgcn_perm(vr[n + 1][w], vr[n][w], 0x05040100u);
          const uint32_t hi = __builtin_amdgcn_perm(vr[n + 1][w], vr[n][w], 0x07060302u);
          o[2 * w] = dot2_bf16(lo, pp, o[2 * w]);
          o[2 * w + 1] = dot2_bf16(hi, pp, o[2 * w + 1]);
        }
      }
    } else if constexpr (kDotF16) {
      // Two keys' codes per element as the f16 pair (1024 + code + 128) of
      // each, weighted by the two weights in f16; the unit's V scale then
      // multiplies the unit's sums once.
      static_assert(C::NI % 2 == 0, "keys pair up for v_dot2");
      float oc[E];
      float psum = 0.f;
#pragma unroll
      for (int n = 0; n < C::NI; n += 2) {
        const auto ph = __builtin_amdgcn_cvt_pkrtz(pw[n], pw[n + 1]);  // weights in [0, 1]
        const uint32_t pp = __builtin_bit_cast(uint32_t, ph);
        psum += (float)ph[0] + (float)ph[1];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // bytes k of both keys side by side: lo holds elements 4w, 4w + 1,
          // hi elements 4w + 2, 4w + 3
          const uint32_t lo = __builtin_amdgcn_perm(vr[n + 1][w], vr[n][w], 0x05010400u) ^ 0x80808080u;
          const uint32_t hi = __builtin_amdgcn_perm(vr[n + 1][w], vr[n][w], 0x07030602u) ^ 0x80808080u;
          const float c0 = n == 0 ? 0.f : oc[4 * w], c1 = n == 0 ? 0.f : oc[4 * w + 1];
          const float c2v = n == 0 ? 0.f : oc[4 * w + 2], c3 = n == 0 ? 0.f : oc[4 * w + 3];
          oc[4 * w] = dot2_f16(biased_pair_f16<0>(lo), pp, c0);
          oc[4 * w + 1] = dot2_f16(biased_pair_f16<2>(lo), pp, c1);
          oc[4 * w + 2] = dot2_f16(biased_pair_f16<0>(hi), pp, c2v);
          oc[4 * w + 3] = dot2_f16(biased_pair_f16<2>(hi), pp, c3);
        }
      }
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = fmaf(vs, oc[e], o[e]);
      pvsum = fmaf(vs, psum, pvsum);
    } else {
#pragma unroll
      for (int n = 0; n < C::NI; ++n) {
        float vf[E];
        if constexpr (kInt8) {
          codes_to_float_biased(vr[n], vf);  // code + 128
          pvsum += pw[n];
        } else {
          chunk_to_float<TC>(vr[n], vf);
        }
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = fmaf(pw[n], vf[e], o[e]);
      }
    }
  };

  // Two register sets take turns: while one unit is computed, the next
  // one's loads are in flight into the other set (no copies between them).
  u32x4_t ka[C::NI], va[C::NI], kb[C::NI], vb[C::NI];
  f32x2_t sa = {1.f, 1.f}, sb = {1.f, 1.f};
  int key_a = -1, key_b = -1;
  int s = next_slot(wave, key_a);
  if (s < nslots) load(key_a, ka, va, sa);
  while (s < nslots) {
    s = next_slot(s + W, key_b);
    if (s < nslots) load(key_b, kb, vb, sb);
    unit(key_a, ka, va, sa);
    if (s >= nslots) break;
    s = next_slot(s + W, key_a);
    if (s < nslots) load(key_a, ka, va, sa);
    unit(key_b, kb, vb, sb);
  }

  if constexpr (kInt8) {  // take off the offset the biased V codes carried
    constexpr float kOffset = kDotF16 ? -1152.f : -128.f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = fmaf(kOffset, pvsum, o[e]);
  }
  // Sum over the key groups: every lane of chunk c then holds the wave's
  // O[c E .. c E + E) and l (each key's weight counted once per group).
  l = stride_sum<LPK>(l);
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = stride_sum<LPK>(o[e]);
  if (kq == 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) part[wave][chunk * E + e] = o[e];
  }
  if (lane == 0) {
    part[wave][D] = m2;
    part[wave][D + 1] = l;
  }
  __syncthreads();

  // Merge the waves: thread x < D finishes output element x.
  const int x = threadIdx.x;
  if (x < D) {
    float m_all = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) m_all = fmaxf(m_all, part[w][D]);
    float l_all = 0.f, acc = 0.f;
    if (m_all != -INFINITY) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float a = fast_exp2(part[w][D] - m_all);  // 0 for a wave with no unit
        l_all = fmaf(part[w][D + 1], a, l_all);
        acc = fmaf(part[w][x], a, acc);
      }
    }
    const float inv = l_all > 0.f ? 1.f / l_all : 0.f;
    store_elem<T>(static_cast<T*>(p.o) + (size_t)bh * D + x, acc * inv);
    if (x == 0 && p.lse != nullptr)
      p.lse[bh] = l_all > 0.f ? (m_all + log2f(l_all)) * 0.69314718055994530942f : -INFINITY;
  }
}

template <typename T, typename TC, int BS, int D>
bsa_status launch_decode(const DecParams& p, int num_wg, hipStream_t stream) {
  hipLaunchKernelGGL((bsa_decode_kernel<T, TC, BS, D>), dim3(num_wg), dim3(kWave * kDecodeWaves),
                     0, stream, p);
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

template <typename T, typename TC>
bsa_status dispatch_decode(const DecParams& p, int num_wg, int bs, int d, hipStream_t stream) {
  if (bs == 32 && d == 64) return launch_decode<T, TC, 32, 64>(p, num_wg, stream);
  if (bs == 32 && d == 128) return launch_decode<T, TC, 32, 128>(p, num_wg, stream);
  if (bs == 64 && d == 64) return launch_decode<T, TC, 64, 64>(p, num_wg, stream);
  if (bs == 64 && d == 128) return launch_decode<T, TC, 64, 128>(p, num_wg, stream);
  return BSA_ERR_INVALID_ARGUMENT;
}

bsa_status decode_impl(const void* q, const void* k_cache, const float* k_scale,
                       const void* v_cache, const float* v_scale, bool int8_cache, void* o,
                       float* lse, int32_t batch, int32_t heads, int32_t cache_len,
                       int32_t head_dim, int32_t block_size, int32_t dtype,
                       const int32_t* seqlens, const int32_t* row_ptr, const int32_t* col_idx,
                       int64_t nnz, float scale, int32_t flags, void* stream) {
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || o == nullptr ||
      seqlens == nullptr || row_ptr == nullptr || col_idx == nullptr)
    return BSA_ERR_NULL_POINTER;
  if (int8_cache && (k_scale == nullptr || v_scale == nullptr)) return BSA_ERR_NULL_POINTER;
  if (dtype != BSA_DTYPE_F32 && dtype != BSA_DTYPE_BF16) return BSA_ERR_INVALID_ARGUMENT;
  if (block_size != 32 && block_size != 64) return BSA_ERR_INVALID_ARGUMENT;
  if (head_dim != 64 && head_dim != 128) return BSA_ERR_INVALID_ARGUMENT;
  if (batch <= 0 || heads <= 0 || cache_len <= 0 || cache_len % block_size != 0)
    return BSA_ERR_SHAPE;
  if (!(scale == scale) || std::isinf(scale)) return BSA_ERR_INVALID_ARGUMENT;
  if ((flags & ~BSA_FORWARD_PATTERN_PER_HEAD) != 0) return BSA_ERR_INVALID_ARGUMENT;
  const bool per_head = (flags & BSA_FORWARD_PATTERN_PER_HEAD) != 0;
  const int64_t M = cache_len / block_size;
  const int64_t patterns = per_head ? heads : 1;
  if (nnz < patterns * M || nnz > patterns * M * M) return BSA_ERR_SHAPE;
  if ((int64_t)batch * heads > INT32_MAX) return BSA_ERR_SHAPE;
  const uintptr_t align = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
                          reinterpret_cast<uintptr_t>(v_cache);
  if (align % 16 != 0) return BSA_ERR_INVALID_ARGUMENT;

  DecParams p;
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.o = o;
  p.lse = lse;
  p.seqlens = seqlens;
  p.row_ptr = row_ptr;
  p.col_idx = col_idx;
  p.heads = heads;
  p.n_cap = cache_len;
  p.M = static_cast<int32_t>(M);
  p.row_stride = per_head ? static_cast<int32_t>(M + 1) : 0;
  const float s = scale > 0.f ? scale : 1.0f / std::sqrt(static_cast<float>(head_dim));
  p.scale_log2 = s * 1.4426950408889634f;

  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int num_wg = batch * heads;
  if (dtype == BSA_DTYPE_F32)
    return int8_cache ? dispatch_decode<float, int8_t>(p, num_wg, block_size, head_dim, st)
                      : dispatch_decode<float, float>(p, num_wg, block_size, head_dim, st);
  return int8_cache ? dispatch_decode<__bf16, int8_t>(p, num_wg, block_size, head_dim, st)
                    : dispatch_decode<__bf16, __bf16>(p, num_wg, block_size, head_dim, st);
}

// ---------------------------------------------------------------- quantiser
// One workgroup per (batch, head, block): the block's BS x D values are read
// once into registers (16-byte chunks), reduced to max|x|, then coded.
constexpr int kQuantThreads = 256;

template <typename T, int BS, int D>
__global__ __launch_bounds__(kQuantThreads) void bsa_quantize_kernel(const T* __restrict__ x,
                                                                    int8_t* __restrict__ codes,
                                                                    float* __restrict__ scales) {
  constexpr int per = 16 / (int)sizeof(T);      // elements per 16-byte chunk
  constexpr int kChunks = BS * D / per;
  constexpr int kPerThread = kChunks / kQuantThreads;
  static_assert(kChunks % kQuantThreads == 0 && per % 4 == 0, "quantiser shape");
  __shared__ float wave_max[kQuantThreads / kWave];

  const size_t base = (size_t)blockIdx.x * BS * D;
  float f[kPerThread][per];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int c = i * kQuantThreads + threadIdx.x;
    chunk_to_float<T>(*reinterpret_cast<const u32x4_t*>(x + base + (size_t)c * per), f[i]);
#pragma unroll
    for (int e = 0; e < per; ++e) amax = fmaxf(amax, fabsf(f[i][e]));
  }
  amax = group_max<1, kWave>(amax);
  if ((threadIdx.x & (kWave - 1)) == 0) wave_max[threadIdx.x / kWave] = amax;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kQuantThreads / kWave; ++w) amax = fmaxf(amax, wave_max[w]);
  const float scale = amax / 127.0f;  // correctly rounded float32 division
  if (threadIdx.x == 0) scales[blockIdx.x] = scale;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int c = i * kQuantThreads + threadIdx.x;
    uint32_t w[per / 4];
#pragma unroll
    for (int k = 0; k < per / 4; ++k) {
      uint32_t word = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        float qv = scale > 0.f ? rintf(f[i][4 * k + b] / scale) : 0.f;
        qv = fminf(fmaxf(qv, -127.f), 127.f);
        word |= ((uint32_t)(int32_t)qv & 0xFFu) << (8 * b);
      }
      w[k] = word;
    }
    int8_t* dst = codes + base + (size_t)c * per;
    if constexpr (per == 8) {
      *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{w[0], w[1]};
    } else {
      *reinterpret_cast<uint32_t*>(dst) = w[0];
    }
  }
}

template <typename T, int BS, int D>
bsa_status launch_quantize(const void* x, int8_t* codes, float* scales, int64_t blocks,
                           hipStream_t stream) {
  hipLaunchKernelGGL((bsa_quantize_kernel<T, BS, D>), dim3((uint32_t)blocks),
                     dim3(kQuantThreads), 0, stream, static_cast<const T*>(x), codes, scales);
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

template <typename T>
bsa_status dispatch_quantize(const void* x, int8_t* codes, float* scales, int64_t blocks, int bs,
                             int d, hipStream_t stream) {
  if (bs == 32 && d == 64) return launch_quantize<T, 32, 64>(x, codes, scales, blocks, stream);
  if (bs == 32 && d == 128) return launch_quantize<T, 32, 128>(x, codes, scales, blocks, stream);
  if (bs == 64 && d == 64) return launch_quantize<T, 64, 64>(x, codes, scales, blocks, stream);
  if (bs == 64 && d == 128) return launch_quantize<T, 64, 128>(x, codes, scales, blocks, stream);
  return BSA_ERR_INVALID_ARGUMENT;
}

}  // namespace

extern "C" bsa_status bsa_decode(const void* q, const void* k_cache, const void* v_cache, void* o,
                                 float* lse, int32_t batch, int32_t heads, int32_t cache_len,
                                 int32_t head_dim, int32_t block_size, int32_t dtype,
                                 const int32_t* seqlens, const int32_t* row_ptr,
                                 const int32_t* col_idx, int64_t nnz, float scale, int32_t flags,
                                 void* stream) {
  return decode_impl(q, k_cache, nullptr, v_cache, nullptr, false, o, lse, batch, heads,
                     cache_len, head_dim, block_size, dtype, seqlens, row_ptr, col_idx, nnz,
                     scale, flags, stream);
}

extern "C" bsa_status bsa_decode_int8kv(const void* q, const int8_t* k_codes,
                                        const float* k_scales, const int8_t* v_codes,
                                        const float* v_scales, void* o, float* lse,
                                        int32_t batch, int32_t heads, int32_t cache_len,
                                        int32_t head_dim, int32_t block_size, int32_t dtype,
                                        const int32_t* seqlens, const int32_t* row_ptr,
                                        const int32_t* col_idx, int64_t nnz, float scale,
                                        int32_t flags, void* stream) {
  return decode_impl(q, k_codes, k_scales, v_codes, v_scales, true, o, lse, batch, heads,
                     cache_len, head_dim, block_size, dtype, seqlens, row_ptr, col_idx, nnz,
                     scale, flags, stream);
}

extern "C" bsa_status bsa_quantize_kv(const void* x, int8_t* codes, float* scales, int32_t batch,
                                      int32_t heads, int32_t seq_len, int32_t head_dim,
                                      int32_t block_size, int32_t dtype, void* stream) {
  if (x == nullptr || codes == nullptr || scales == nullptr) return BSA_ERR_NULL_POINTER;
  if (dtype != BSA_DTYPE_F32 && dtype != BSA_DTYPE_BF16) return BSA_ERR_INVALID_ARGUMENT;
  if (block_size != 32 && block_size != 64) return BSA_ERR_INVALID_ARGUMENT;
  if (head_dim != 64 && head_dim != 128) return BSA_ERR_INVALID_ARGUMENT;
  if (batch <= 0 || heads <= 0 || seq_len <= 0 || seq_len % block_size != 0) return BSA_ERR_SHAPE;
  const uintptr_t align = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(codes);
  if (align % 16 != 0) return BSA_ERR_INVALID_ARGUMENT;
  const int64_t blocks = (int64_t)batch * heads * (seq_len / block_size);
  if (blocks > INT32_MAX) return BSA_ERR_SHAPE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (dtype == BSA_DTYPE_F32)
    return dispatch_quantize<float>(x, codes, scales, blocks, block_size, head_dim, st);
  return dispatch_quantize<__bf16>(x, codes, scales, blocks, block_size, head_dim, st);
}
