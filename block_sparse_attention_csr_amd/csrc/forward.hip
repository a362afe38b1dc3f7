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
//  * The union's K/V blocks stream through a ring of NB LDS buffers with
//    direct-to-LDS copies (global_load_lds_dwordx4), NB - 1 entries ahead of
//    the compute.  16-byte chunks are XOR-swizzled per row to spread LDS
//    banks.  bf16 at block 64 with one query block per workgroup holds one
//    K slot and one V slot instead (each copy lands while the other half of
//    the step runs), so that two waves per SIMD fit without pairing rows.
//  * Rows far longer than the mean can be cut into items (a row-split plan):
//    each item's workgroup writes a partial (O, m, l) that a merge combines.
//    With several query blocks per workgroup the items run in the same
//    launch as the query groups.
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
//  * O leaves through LDS: each wave writes its normalised rows row-major
//    into the idle ring and stores whole 16-byte chunks of consecutive rows
//    (the accumulator layout alone would give 8-byte pieces, one query per
//    lane).
// The fp32 variant uses v_mfma_f32_32x32x2_f32 with the same layouts.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "bsa.h"
#include "mfma_tiles.h"

namespace {

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
  int32_t heads;      // H
  int32_t causal;     // hide keys after each query position
  int32_t row_stride; // row_ptr entries per head: M + 1 (one pattern per head) or 0
  float scale_log2;   // scale * log2(e)
  // Rows split across workgroups (bsa_plan_row_split).  Main pass: heavy[r]
  // != 0 marks a row this pass leaves out.  Split pass (G = KS = 1 only):
  // split holds (row, first entry, end entry) per item, and each workgroup
  // writes its item's partial (O, m, l) to partial.
  const uint8_t* heavy;
  const int32_t* split;
  int32_t n_items;
  float* partial;
  // One launch for both (G > 1): per (batch * head), the first n_tuples
  // workgroups take the items, item t + g n_tuples as block g; the query
  // groups follow.
  int32_t n_tuples;
  // int8 K/V (bsa_forward_int8kv): k and v hold int8 codes, and these one
  // float32 scale per (batch * head, block); NULL for bf16 / float32 K/V.
  const float* k_scale;
  const float* v_scale;
};

// Sixteen int8 codes (four words) as sixteen bf16 values, in order, in two
// 16-byte groups.  A code is an integer in [-128, 127]: its float32 value
// has at most 8 significant bits, so its upper half is its exact bf16.
__device__ __forceinline__ void codes_to_bf16(const u32x4_t& w, u32x4_t& lo, u32x4_t& hi) {
  uint32_t b[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float f[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) f[k] = (float)(int)(int8_t)(w[i] >> (8 * k));
    b[2 * i] = __builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
    b[2 * i + 1] =
        __builtin_amdgcn_perm(__float_as_uint(f[3]), __float_as_uint(f[2]), 0x07060302u);
  }
  lo = u32x4_t{b[0], b[1], b[2], b[3]};
  hi = u32x4_t{b[4], b[5], b[6], b[7]};
}

// Partial state of a key-slice wave, stored for the merge: O^T in accumulator
// order [reg][lane], then m and l per lane.
template <int D>
constexpr int partial_bytes() {
  return (D / 32) * 16 * kWave * 4 + 2 * kWave * 4;
}
// Two key slices split the finish by columns: each publishes the half of its
// (O, m, l) the other finishes.
template <int D>
constexpr int half_partial_bytes() {
  return (D / 64) * 16 * kWave * 4 + 2 * kWave * 4;
}

// Compile-time shape of one kernel instantiation.  KV8: K and V are int8
// codes; each entry lands as int8 in one of NB8 slots (copies NB8 - 1
// entries ahead) and is converted to bf16 into the one tile buffer the math
// reads.  RING: a one-block, one-slice shape keeps the two-entry ring (the
// row-split pass: few workgroups, each with a long run of entries).
template <typename T, int BS, int D, int G, int KS, bool KV8 = false, bool RING = false>
struct Cfg {
  using L = TileLayout<T, BS, D>;
  static constexpr int QW = BS / kQRows;  // query waves per query block
  static constexpr int SW = QW * G;       // waves per key slice
  static constexpr int W = SW * KS;       // waves per workgroup
  static constexpr int kEntry = L::kEntryBytes;
  // bf16 at block 64 with one query block and one key slice: one K slot and
  // one V slot (a tile each), not two whole entries (see the kernel's loop).
  static constexpr bool kSingle =
      std::is_same<T, __bf16>::value && !KV8 && !RING && BS == 64 && G == 1 && KS == 1;
  static constexpr int kSliceBytes = kSingle ? L::kTileBytes : KS * kEntry;  // per buffer
  static_assert(L::kCopies % SW == 0, "entry parts must split evenly over a slice's waves");
  static constexpr int kParts = L::kCopies / SW;  // 1 KB copies per wave per entry
  static constexpr int kEntry8 = kEntry / 2;       // int8 K then V of one entry
  static constexpr int kSlice8 = KS * kEntry8;
  static constexpr int kPartsTile8 = BS * D / (kWave * 16);  // 1 KB parts of an int8 tile
  static_assert(!KV8 || (2 * kPartsTile8) % SW == 0, "int8 entry parts split evenly");
  static constexpr int kParts8 = 2 * kPartsTile8 / SW;       // per wave per entry
  static constexpr int NB8 = KS == 1 && 2 * kSliceBytes + kSlice8 <= 40 * 1024 ? 3 : 2;
  // Three tile buffers (prefetch distance 2) while they leave room for four
  // workgroups per CU, else two (prefetch distance 1): at block 64 and d = 64
  // three 16 KB buffers (48 KB, three workgroups per CU) made the random mask
  // 6.5% slower than two (four per CU).  Key-split shapes keep two: their
  // slices already run KS entries ahead together, and the smaller footprint
  // keeps a whole small grid resident at once.
  // KV8: buf0 is the bf16 tile buffer, buf1 int8 slots 0 and 1, buf2 slot 2.
  static constexpr int NB = KV8 || kSingle ? 2 : (KS == 1 && 3 * kSliceBytes <= 40 * 1024 ? 3 : 2);
  static constexpr int kBuf2 = KV8 ? (NB8 == 3 ? kSlice8 : 16) : (NB == 3 ? kSliceBytes : 16);
  static constexpr int kLdsBytes = 2 * kSliceBytes + kBuf2;
  // Shapes whose buffers do not fit a workgroup's LDS are not instantiated.
  static constexpr bool kValid = (!KV8 || std::is_same<T, __bf16>::value) &&
                                 kLdsBytes + 1024 <= 160 * 1024 &&
                                 (KS - 1) * SW * partial_bytes<D>() <= kSliceBytes &&
                                 (KS != 2 || 2 * SW * half_partial_bytes<D>() <= kSliceBytes);
};

template <typename T, int BS, int D, int G, int KS, bool CAUSAL, bool KV8 = false,
          bool RING = false>
__global__ __launch_bounds__((kWave * Cfg<T, BS, D, G, KS, KV8, RING>::W)) void bsa_fwd_kernel(
    FwdParams p) {
  using C = Cfg<T, BS, D, G, KS, KV8, RING>;
  using L = typename C::L;
  using O = Ops<T>;
  constexpr int QW = C::QW;
  constexpr int SW = C::SW;
  constexpr int NB = C::NB;
  constexpr int KSTEPS = BS / kKeyStep;

  // K/V tile buffers: separate LDS objects so that the compiler can tell a
  // copy in flight into one buffer from the reads of another.
  __shared__ __attribute__((aligned(16))) unsigned char buf0[C::kSliceBytes];
  __shared__ __attribute__((aligned(16))) unsigned char buf1[C::kSliceBytes];
  __shared__ __attribute__((aligned(16))) unsigned char buf2[C::kBuf2];
  extern __shared__ __attribute__((aligned(16))) int32_t dyn[];  // entry list | bitmaps
  __shared__ int32_t union_size;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = uniform(threadIdx.x / kWave);
  const int qg = wave % QW;        // 32-row query group within the block
  const int g = (wave / QW) % G;   // query block within the workgroup
  const int ks = wave / SW;        // key slice
  const int ws = wave % SW;        // wave index within its key slice

  const int M = p.M;
  const int ngroups = (M + G - 1) / G;
  const int wg = xcd_remap(blockIdx.x, p.num_wg);
  // A head's last group runs first, then groups 0, 1, 2, ...: the first and
  // last query blocks are the ones a banded pattern's global rows make dense,
  // and started last the last one would run alone at the end.  The rest keep
  // their order, so neighbouring groups (which share K/V blocks) stay close
  // in time.
  int grp, bh, item = -1;
  bool item_wg = false;  // a workgroup of items (all its waves)
  if (G == 1 && KS == 1 && p.split != nullptr) {  // split pass: one item of a heavy row
    item = wg % p.n_items;
    bh = wg / p.n_items;
    grp = p.split[3 * item];
  } else if (G > 1 && KS == 1 && p.split != nullptr) {
    // items and groups in one launch: a head's items first (each is as long
    // as an ordinary row or longer), then its groups in the order below
    const int per_head = p.n_tuples + ngroups;
    const int r = wg % per_head;
    bh = wg / per_head;
    if (r < p.n_tuples) {
      item_wg = true;
      const int t = r + g * p.n_tuples;
      item = t < p.n_items ? t : -1;
      grp = 0;
    } else {
      const int rank = r - p.n_tuples;
      grp = rank == 0 ? ngroups - 1 : rank - 1;
    }
  } else {
    const int rank = wg % ngroups;
    grp = rank == 0 ? ngroups - 1 : rank - 1;
    bh = wg / ngroups;
  }
  // (block g of an item workgroup: its item's row, or none past the last item)
  const int qb = !item_wg ? grp * G + g : item >= 0 ? p.split[3 * item] : M;
  // (a row the split pass takes is left out of this pass: no entry, no store)
  const bool has_rows = qb < M && (item >= 0 || p.heavy == nullptr || p.heavy[qb] == 0);
  constexpr bool causal = CAUSAL;
  const int32_t* const row_ptr = p.row_ptr + (size_t)(bh % p.heads) * p.row_stride;
  const size_t head = (size_t)bh * p.N * D;
  const T* Q = static_cast<const T*>(p.q) + head;
  const T* K = static_cast<const T*>(p.k) + head;
  const T* V = static_cast<const T*>(p.v) + head;
  const int8_t* K8 = static_cast<const int8_t*>(p.k) + head;  // (KV8)
  const int8_t* V8 = static_cast<const int8_t*>(p.v) + head;
  const float* const ksc = KV8 ? p.k_scale + (size_t)bh * M : nullptr;  // (KV8) per block
  const float* const vsc = KV8 ? p.v_scale + (size_t)bh * M : nullptr;

  // Several query blocks per workgroup: the loading wave of each block reads
  // the first 64 entries of its CSR row (one per lane) before any Q load.
  // The union is built from them, and the vector-memory counter drains in
  // order, so issued after Q they would wait for all of Q first.
  const bool loads_row = G > 1 && has_rows && qg == 0 && ks == 0;
  int row_s = 0, row_e = 0, row_first = -1;
  if (loads_row) {
    row_s = item >= 0 ? p.split[3 * item + 1] : row_ptr[qb];
    row_e = item >= 0 ? p.split[3 * item + 2] : row_ptr[qb + 1];
    if (row_s + lane < row_e) row_first = p.col_idx[row_s + lane];
  }

  // One query block per workgroup: the row's bounds, read before the Q
  // copies below.  Read after them, these uniform loads could not go through
  // the scalar cache (the copies' asm may write memory), and each vector load
  // would wait for the Q copies as well (the counter drains in order).
  int rs = 0;     // G == 1: the row's first entry in col_idx
  int row_n = 0;  // G == 1: its entry count
  if constexpr (G == 1) {
    if (item >= 0) {  // the item's entries of its row
      rs = p.split[3 * item + 1];
      row_n = p.split[3 * item + 2] - rs;
    } else {
      rs = row_ptr[grp];
      row_n = has_rows ? row_ptr[grp + 1] - rs : 0;
    }
  }

  typename O::template QOperand<D> qop;
  const int q0 = (has_rows ? qb : 0) * BS + qg * kQRows;
  // bf16, one query block per workgroup: the wave's 32 Q rows come in as
  // whole 1 KB runs (direct-to-LDS, swizzled like the K/V tiles) into its part
  // of the ring's last buffer, which no K/V copy touches before the first
  // step's barrier; the operand is read from there once they land.  (The
  // operand layout read straight from memory takes 16 bytes from each of 32
  // rows per load: it cost 5% of the latency-bound small-grid forward.)
  using QL = TileLayout<T, kQRows, D>;
  constexpr bool kStageQ = G == 1 && std::is_same<T, __bf16>::value &&
                           C::W * QL::kTileBytes <= C::kSliceBytes;
  unsigned char* const q_stage =
      (KV8 ? buf0 : NB == 3 ? buf2 : buf1) + (ks * QW + qg) * QL::kTileBytes;
  if constexpr (kStageQ) {
    const uint32_t dst = (uint32_t)(uintptr_t)(LDS_PTR(unsigned char))q_stage;
    constexpr int kQParts = QL::kTileBytes / (kWave * 16);
    constexpr int kQRun = dma_run(kQParts, kQParts);
#pragma unroll
    for (int r = 0; r < kQParts / kQRun; ++r) {
      uint32_t v[kQRun];
#pragma unroll
      for (int k = 0; k < kQRun; ++k) {
        const int slot = (r * kQRun + k) * kWave + lane;
        const int row = slot / QL::kChunksPerRow;
        const int chunk = (slot % QL::kChunksPerRow) ^ QL::swz(row);
        v[k] = (uint32_t)(row * QL::kRowBytes + chunk * 16 - k * kWave * 16);
      }
      lds_dma16_run<kQRun>(Q + (size_t)q0 * D, v, dst + r * kQRun * kWave * 16);
    }
  } else {
    O::template load_q<D>(qop, Q + (size_t)q0 * D, lane);
  }

  // ---- entry list: the workgroup's CSR row (G == 1, read from col_idx) or
  // the sorted union of its G rows (G > 1, built in LDS, with per-row bitmaps
  // that say which entries a wave uses).
  const int MW = (M + 31) / 32;
  int32_t* list = dyn;                                        // [M]
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(dyn + M);    // [(G + 1) * MW] (G > 1)
  const uint32_t* my_row = bitmap + (1 + g) * MW;
  int U;
  if constexpr (G == 1) {
    // Every wave reads the row from col_idx itself (64 entries at a time, in
    // entry_at): no LDS list and no barrier before the first copy.
    U = row_n;
  } else {
    for (int i = threadIdx.x; i < (G + 1) * MW; i += blockDim.x) bitmap[i] = 0;
    __syncthreads();
    if (loads_row) {
      auto mark = [&](int j) {
        if (j >= 0 && j < M && (!causal || j <= qb)) {
          atomicOr(&bitmap[j >> 5], 1u << (j & 31));
          atomicOr(&bitmap[(1 + g) * MW + (j >> 5)], 1u << (j & 31));
        }
      };
      if (row_s + lane < row_e) mark(row_first);
      // entries past the first 64 (long rows only: no load, and no wait on
      // the Q loads, for the others)
      for (int t = row_s + kWave + lane; t < row_e; t += kWave) mark(p.col_idx[t]);
    }
    __syncthreads();
    if (wave == 0) {  // ascending list of the union's blocks
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
      if (lane == 0) union_size = base;
    }
    __syncthreads();
    U = uniform(union_size);
  }
  // Slice ks takes list entries ks, ks + KS, ...; every wave runs niter steps.
  const int niter = (U + KS - 1) / KS;
  // The list is read 64 entries at a time into one VGPR (lane l holds entry
  // base + l) with a ballot of which of them this wave's row selects, so a
  // step needs one v_readlane and a scalar bit test, not an LDS round trip.
  int chunk_base = -64;
  int chunk = -1;
  uint64_t chunk_mine = 0;
  float chunk_ks = 0.f, chunk_vs = 0.f;  // (KV8) the entries' K and V scales
  auto entry_at = [&](int step, bool& mine, float* sk = nullptr,
                      float* sv = nullptr) -> int {  // block of this slice's step, or -1
    const int t = step * KS + ks;
    if (t >= U) {
      mine = false;
      return -1;
    }
    if ((t & ~(kWave - 1)) != chunk_base) {
      chunk_base = t & ~(kWave - 1);
      const int idx = chunk_base + lane;
      if constexpr (G == 1) chunk = idx < U ? p.col_idx[rs + idx] : -1;
      else chunk = idx < U ? list[idx] : -1;
      bool sel = chunk >= 0 && chunk < M && has_rows && (!causal || chunk <= qb);
      if constexpr (G > 1)
        sel = sel && ((my_row[chunk >> 5] >> (chunk & 31)) & 1u) != 0;
      chunk_mine = __builtin_amdgcn_ballot_w64(sel);
      if constexpr (KV8) {
        const bool in_range = chunk >= 0 && chunk < M;
        chunk_ks = in_range ? ksc[chunk] : 0.f;
        chunk_vs = in_range ? vsc[chunk] : 0.f;
      }
    }
    const int l = t - chunk_base;
    mine = ((chunk_mine >> l) & 1ull) != 0;
    if constexpr (KV8) {
      *sk = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, chunk_ks), l));
      *sv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, chunk_vs), l));
    }
    return __builtin_amdgcn_readlane(chunk, l);
  };

  // ---- direct-to-LDS copies.  An entry is 1 KB parts (part p: slots
  // 64 p .. 64 p + 63); lane i fetches the 16-byte global chunk the swizzle
  // places in its slot.  Wave ws copies parts ws kParts .. ws kParts +
  // kParts - 1, in runs of kRun consecutive parts behind one M0 write (a run
  // lies in the K tile or in the V tile, never both); dma_off carries the
  // run's immediate offset taken off.
  constexpr int kPartsPerTile = L::kCopies / 2;
  constexpr int kRun = dma_run(C::kParts, kPartsPerTile);
  uint32_t dma_off[C::kParts];
#pragma unroll
  for (int c = 0; c < C::kParts; ++c) {
    const int part = (ws * C::kParts + c) % kPartsPerTile;
    const int slot = part * kWave + lane;
    const int row = slot / L::kChunksPerRow;
    const int chunk = (slot % L::kChunksPerRow) ^ L::swz(row);
    dma_off[c] = (uint32_t)(row * L::kRowBytes + chunk * 16 - (c % kRun) * kWave * 16);
  }
  auto issue = [&](int j, unsigned char* buf) {
    // a missing entry copies block 0 (unused)
    const size_t key0 = (size_t)((uint32_t)j < (uint32_t)M ? (uint32_t)j : 0u) * BS;
    const uint32_t dst = (uint32_t)(uintptr_t)(LDS_PTR(unsigned char))buf + ks * C::kEntry +
                         ws * C::kParts * kWave * 16;
#pragma unroll
    for (int r = 0; r < C::kParts / kRun; ++r) {
      const int part = ws * C::kParts + r * kRun;
      uint32_t v[kRun];
#pragma unroll
      for (int k = 0; k < kRun; ++k) v[k] = dma_off[r * kRun + k];
      lds_dma16_run<kRun>((part < kPartsPerTile ? K : V) + key0 * D, v,
                          dst + r * kRun * kWave * 16);
    }
  };
  // (KV8) copies of an entry's int8 codes as they are: part c of this wave
  // is part ws + c SW of the entry (1 KB; K tile parts first).
  auto issue8 = [&](int j, uint32_t slot) {  // slot: LDS byte address
    const int key0 = (j < 0 || j >= M ? 0 : j) * BS;
    const uint32_t dst = slot + ks * C::kEntry8;
#pragma unroll
    for (int c = 0; c < C::kParts8; ++c) {
      const int part = ws + c * SW;
      const int8_t* base = (part < C::kPartsTile8 ? K8 : V8) + (size_t)key0 * D;
      lds_dma16(base, (uint32_t)((part % C::kPartsTile8) * kWave * 16 + lane * 16),
                dst + part * kWave * 16);
    }
  };
  // (KV8) this wave's parts of the entry in `slot`, converted to bf16 into
  // the tile buffer buf0 in the bf16 layout: lane i holds codes 16 i .. of
  // its part, sixteen consecutive features of one row.
  auto convert = [&](uint32_t slot) {
#pragma unroll
    for (int c = 0; c < C::kParts8; ++c) {
      const int part = ws + c * SW;
      const int e0 = (part % C::kPartsTile8) * kWave * 16 + lane * 16;  // element of the tile
      const int row = e0 / D, f0 = e0 % D;
      const u32x4_t w = *(LDS_PTR(const u32x4_t))(uintptr_t)(slot + ks * C::kEntry8 +
                                                             part * kWave * 16 + lane * 16);
      u32x4_t lo, hi;
      codes_to_bf16(w, lo, hi);
      LDS_PTR(unsigned char) dst = (LDS_PTR(unsigned char))buf0 + ks * C::kEntry +
                                   (part < C::kPartsTile8 ? 0 : L::kTileBytes);
      *(LDS_PTR(u32x4_t))(dst + L::chunk_offset(row, f0 / 8)) = lo;
      *(LDS_PTR(u32x4_t))(dst + L::chunk_offset(row, f0 / 8 + 1)) = hi;
    }
  };

  typename O::template Offsets<BS, D> off;
  off.init(lane, ks * C::kEntry);

  f32x16_t o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16_t{};
  float m2 = -INFINITY;  // exponent offset (log2 domain) for this lane's query
  float lsum = 0.f;      // sum of exponentials over this lane half's keys
  bool first = true;     // no block computed yet by this wave
  const float c2 = p.scale_log2;

  // One entry: all S^T tiles are issued first (the steps' MFMA chains
  // interleaved); then one running-max update for the whole entry, and each
  // 32-key step's exponentials (VALU) run beside the previous step's P.V.
  // `diag`: the entry is this wave's own query block under causal masking.
  // Its 32-key steps after the wave's 32 rows are skipped, the step level
  // with them is masked above the diagonal (the keys after each query).
  // KV8: the tile holds the codes, so the scores are sk (q . code): sk folds
  // into the score factor; and the product runs on P sv, sv folded into the
  // exponent, while the row sum takes P = (P sv) / sv.  A zero scale (an
  // all-zero block, codes 0) may take any value: 1.
  // The scores of an entry whose K tile sits at byte `kpos` of `ktile`.
  auto scores_of = [&](unsigned char* ktile, int kpos, f32x16_t (&sc)[KSTEPS]) {
    LDS_PTR(unsigned char) tile = (LDS_PTR(unsigned char))ktile;
    if constexpr (std::is_same<T, __bf16>::value) {
      O::template scores_steps<BS, D, KSTEPS>(qop, off, tile, kpos, sc);
    } else {
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st) sc[st] = O::template scores<BS, D>(qop, off, tile, kpos, st);
    }
  };
  // Softmax and P.V of an entry from its scores; its V tile sits at byte
  // `vpos` + (a tile) of `vtile` (as in a K-then-V entry at `vpos`).
  auto softmax_pv = [&](f32x16_t (&sc)[KSTEPS], unsigned char* vtile, int vpos, bool diag,
                        float sk, float sv) {
    LDS_PTR(unsigned char) tile = (LDS_PTR(unsigned char))vtile;
    const float c2k = KV8 ? c2 * (sk > 0.f ? sk : 1.f) : c2;
    float lsv = 0.f, isv = 1.f;
    if constexpr (KV8) {
      const float sve = sv > 0.f ? sv : 1.f;
      lsv = __builtin_amdgcn_logf(sve);
      isv = __builtin_amdgcn_rcpf(sve);
    }
    if (diag) {  // keys after each query of the diagonal step are masked
      const int qrow = lane & 31;
      const int h = lane >> 5;
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st)
        if (st == qg)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (8 * (r / 4) + 4 * h + (r % 4) > qrow) sc[st][r] = -INFINITY;
    }
    // The row max (log2 domain) over the entry's steps, on both lane halves.
    auto entry_max = [&]() {
      float mx = sc[0][0];
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st)
        if (st == 0 || !diag || st <= qg)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, sc[st][r]);
      return halves_max(mx) * c2k;
    };
    if constexpr (!std::is_same<T, __bf16>::value || D != 64) {
      // One running-max update per entry, over all of its 32-key steps: one
      // ballot and one (rarely taken) rescale branch per entry, and the
      // steps' exponentials and P.V products in one straight run of code.
      const float mx = entry_max();
      if (first) {  // O and l are still zero: no rescale
        m2 = mx;
        first = false;
      } else if (__builtin_amdgcn_ballot_w64(mx > m2 + kLazyRescale) != 0) {
        const float m_new = fmaxf(m2, mx);
        const float alpha = fast_exp2(m2 - m_new);
        m2 = m_new;
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
      }
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st) {
        if (diag && st > qg) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[st][r] = fast_exp2(fmaf(sc[st][r], c2k, KV8 ? lsv - m2 : -m2));
        const float ps = O::template accumulate<BS, D>(o, sc[st], off, tile, vpos, st);
        lsum = KV8 ? fmaf(ps, isv, lsum) : lsum + ps;
      }
    } else {
      // bf16 at d = 64, where the VALU rather than the matrix cores is the
      // busier unit: no row max per entry.  The first entry sets the running
      // max; after that a step's weights are taken with it as it stands, and
      // only a step whose weights sum past 2^64 (scores risen by about 60 in
      // the log2 domain, or a NaN) takes the max and rescales O and l before
      // taking them again.  The check rides on the row sum already formed.
      if (first) {  // O and l are still zero: no rescale
        m2 = entry_max();
        first = false;
      }
      const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st) {
        if (diag && st > qg) continue;
        uint32_t w[8];  // the weights as packed bf16 pairs (separate scalars)
        float ps = 0.f;
        auto weights = [&]() {
          const float bias = KV8 ? lsv - m2 : -m2;
          ps = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float t0 = fast_exp2(fmaf(sc[st][2 * i], c2k, bias));
            const float t1 = fast_exp2(fmaf(sc[st][2 * i + 1], c2k, bias));
            w[i] = pack_bf16x2(t0, t1);
            ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[i]), ones, ps,
                                                 false);
          }
        };
        weights();
        const float pchk = KV8 ? ps * isv : ps;
        if (__builtin_amdgcn_ballot_w64(!(pchk <= 0x1p64f)) != 0) {
          float mx = sc[st][0];
#pragma unroll
          for (int r = 1; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, sc[st][r]);
          mx = halves_max(mx) * c2k;
          const float m_new = fmaxf(m2, mx);
          const float alpha =
              m2 == -INFINITY || m_new == -INFINITY ? 1.f : fast_exp2(m2 - m_new);
          m2 = m_new;
          lsum *= alpha;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
          weights();
        }
        lsum = KV8 ? fmaf(ps, isv, lsum) : lsum + ps;
        O::template accumulate_words<BS, D>(o, w, off, tile, vpos, st);
      }
    }
  };
  auto compute = [&](unsigned char* buf, bool diag, float sk = 1.f, float sv = 1.f) {
    f32x16_t sc[KSTEPS];
    scores_of(buf, 0, sc);
    softmax_pv(sc, buf, 0, diag, sk, sv);
  };

  // ---- pipeline: entry i computes from buffer i % NB while the copies of
  // entries up to i + NB - 1 are in flight.  Before the barrier that starts
  // entry i each wave waits for its own copies of entry i (the later entries'
  // copies may stay in flight) and for its LDS reads of entry i-1; after it,
  // every wave's copies of entry i have landed and buffer (i-1) % NB is free.
  // One query block per workgroup with one wave per key slice: a slice copies
  // and reads only its own part of each buffer, so its own waits suffice and
  // only entry 0's barrier stays (every wave has read its Q rows before entry
  // 1's copies land over them).  Uncoupled, the slices no longer wait for
  // each other at every entry (worked example 1-2% faster, graph-timed).
  constexpr bool kSliceBarrier = G > 1 || SW > 1;
  if constexpr (C::kSingle) {
    // One K slot (buf0) and one V slot (buf1), each a tile.  Step i: every
    // wave waits for its copies of K[i] and its reads of V[i-1]; a barrier;
    // the copies of V[i]; the scores of entry i (K slot); every wave waits
    // for its copies of V[i] and its K reads; a barrier; the copies of
    // K[i+1]; softmax and P.V of entry i (V slot).  Each copy lands while
    // the other half of the step runs.  Half the LDS of a two-entry ring lets
    // twice the workgroups share a CU, so one query block per workgroup
    // (no wave idles on another row's entries) keeps two waves per SIMD.
    constexpr int kTile = L::kTileBytes;
    constexpr int kPartsT = kPartsPerTile / SW;  // 1 KB copies per wave per tile
    constexpr int kRunT = dma_run(kPartsT, kPartsT);
    uint32_t toff[kPartsT];  // wave ws: parts ws kPartsT .. + kPartsT - 1 of a tile
#pragma unroll
    for (int c = 0; c < kPartsT; ++c) {
      const int slot = (ws * kPartsT + c) * kWave + lane;
      const int row = slot / L::kChunksPerRow;
      toff[c] = (uint32_t)(row * L::kRowBytes +
                           (((slot % L::kChunksPerRow) ^ L::swz(row)) << 4) -
                           (c % kRunT) * kWave * 16);
    }
    const uint32_t kslot = (uint32_t)(uintptr_t)(LDS_PTR(unsigned char))buf0;
    const uint32_t vslot = (uint32_t)(uintptr_t)(LDS_PTR(unsigned char))buf1;
    auto issue_tile = [&](const T* src, int j, uint32_t dst) {
      // a missing entry copies block 0 (unused)
      const size_t key0 = (size_t)((uint32_t)j < (uint32_t)M ? (uint32_t)j : 0u) * BS;
#pragma unroll
      for (int r = 0; r < kPartsT / kRunT; ++r) {
        uint32_t v[kRunT];
#pragma unroll
        for (int k = 0; k < kRunT; ++k) v[k] = toff[r * kRunT + k];
        lds_dma16_run<kRunT>(src + key0 * D, v,
                             dst + (ws * kPartsT + r * kRunT) * kWave * 16);
      }
    };
    bool m0, m1;
    int j0 = entry_at(0, m0);
    wait_vm_lgkm0<0>();  // the Q loads (see the ring below)
    if (niter > 0) issue_tile(K, j0, kslot);
    if constexpr (kStageQ) {  // Q sits in the V slot: read before step 0's barrier
      LDS_PTR(const unsigned char) qs = (LDS_PTR(const unsigned char))q_stage;
#pragma unroll
      for (int c = 0; c < D / 16; ++c)
        qop.r[c] = *(LDS_PTR(const u32x4_t))(qs + QL::chunk_offset(lane & 31, 2 * c + (lane >> 5)));
    }
    for (int i = 0; i < niter; ++i) {
      const int j1 = entry_at(i + 1, m1);
      wait_vm_lgkm0<0>();
      raw_barrier();
      issue_tile(V, j0, vslot);
      f32x16_t sc[KSTEPS];
      if (m0) scores_of(buf0, 0, sc);
      wait_vm_lgkm0<0>();
      raw_barrier();
      if (i + 1 < niter) issue_tile(K, j1, kslot);
      if (m0) softmax_pv(sc, buf1, -kTile, causal && j0 == qb, 1.f, 1.f);
      j0 = j1;
      m0 = m1;
    }
  } else if constexpr (!KV8) {
    int jq[NB];   // blocks of steps i .. i + NB - 1
    bool mq[NB];  // whether this wave computes them
  #pragma unroll
    for (int e = 0; e < NB; ++e) jq[e] = entry_at(e, mq[e]);
    // The Q loads were issued long ago; waiting for them here, before the first
    // copy, tells the compiler they are complete (it does not see the copies
    // and would otherwise wait on the vector-memory counter inside the loop).
    wait_vm_lgkm0<0>();
    if constexpr (kStageQ) {  // lane (query r, half h) takes chunks 2c + h of row r
      LDS_PTR(const unsigned char) qs = (LDS_PTR(const unsigned char))q_stage;
  #pragma unroll
      for (int c = 0; c < D / 16; ++c)
        qop.r[c] = *(LDS_PTR(const u32x4_t))(qs + QL::chunk_offset(lane & 31, 2 * c + (lane >> 5)));
    }
    // The first copies, for the steps there are (none for a row with no entry).
    if (niter > 0) issue(jq[0], buf0);
    if (NB == 3 && niter > 1) issue(jq[1], buf1);
    auto buffer = [&](auto b_c) -> unsigned char* {
      constexpr int b = decltype(b_c)::value;
      if constexpr (b == 0) return buf0;
      else if constexpr (b == 1) return buf1;
      else return buf2;
    };
    auto step = [&](int i, auto b_c) {
      constexpr int b = decltype(b_c)::value;
      if (NB == 3 && i + 1 < niter) wait_vm_lgkm0<C::kParts>();
      else wait_vm_lgkm0<0>();
      if (kSliceBarrier || i == 0) raw_barrier();
      const bool mine = mq[0];
      const bool diag = causal && jq[0] == qb;
  #pragma unroll
      for (int e = 0; e + 1 < NB; ++e) {
        jq[e] = jq[e + 1];
        mq[e] = mq[e + 1];
      }
      jq[NB - 1] = entry_at(i + NB, mq[NB - 1]);
      if (i + NB - 1 < niter) issue(jq[NB - 2], buffer(std::integral_constant<int, (b + NB - 1) % NB>{}));
      if (mine) compute(buffer(b_c), diag);
    };
    for (int i = 0; i < niter; i += NB) {
      step(i, std::integral_constant<int, 0>{});
      if (i + 1 < niter) step(i + 1, std::integral_constant<int, 1>{});
      if constexpr (NB == 3)
        if (i + 2 < niter) step(i + 2, std::integral_constant<int, 2>{});
    }
  } else {
    // int8 entries land in NB8 slots, copies NB8 - 1 entries ahead.  Step i:
    // every wave waits for its own copies of entry i; a barrier (entry i has
    // landed, every wave is done with the tile buffer); the copies of entry
    // i + NB8 - 1 go into the slot entry i - 1 was converted from; entry i is
    // converted into the tile buffer; a barrier; the math.  One-wave slices
    // convert and read only their own parts: their own waits suffice.
    constexpr int NB8 = C::NB8;
    int jq[NB8];
    bool mq[NB8];
    float skq[NB8], svq[NB8];
#pragma unroll
    for (int e = 0; e < NB8; ++e) jq[e] = entry_at(e, mq[e], &skq[e], &svq[e]);
    wait_vm_lgkm0<0>();
    if constexpr (kStageQ) {
      LDS_PTR(const unsigned char) qs = (LDS_PTR(const unsigned char))q_stage;
#pragma unroll
      for (int c = 0; c < D / 16; ++c)
        qop.r[c] = *(LDS_PTR(const u32x4_t))(qs + QL::chunk_offset(lane & 31, 2 * c + (lane >> 5)));
    }
    const uint32_t slots01 = (uint32_t)(uintptr_t)(LDS_PTR(unsigned char))buf1;
    const uint32_t slot2 = (uint32_t)(uintptr_t)(LDS_PTR(unsigned char))buf2;
    auto slot = [&](auto b_c) -> uint32_t {  // LDS byte address of int8 slot b
      constexpr int b = decltype(b_c)::value;
      if constexpr (b < 2) return slots01 + b * C::kSlice8;
      else return slot2;
    };
    if (niter > 0) issue8(jq[0], slot(std::integral_constant<int, 0>{}));
    if (NB8 == 3 && niter > 1) issue8(jq[1], slot(std::integral_constant<int, 1>{}));
    auto step8 = [&](int i, auto b_c) {
      constexpr int b = decltype(b_c)::value;
      if (NB8 == 3 && i + 1 < niter) wait_vm_lgkm0<C::kParts8>();
      else wait_vm_lgkm0<0>();
      if (kSliceBarrier || i == 0) raw_barrier();
      const bool mine = mq[0];
      const bool diag = causal && jq[0] == qb;
      const float sk = skq[0], sv = svq[0];
#pragma unroll
      for (int e = 0; e + 1 < NB8; ++e) {
        jq[e] = jq[e + 1];
        mq[e] = mq[e + 1];
        skq[e] = skq[e + 1];
        svq[e] = svq[e + 1];
      }
      jq[NB8 - 1] = entry_at(i + NB8, mq[NB8 - 1], &skq[NB8 - 1], &svq[NB8 - 1]);
      if (i + NB8 - 1 < niter)
        issue8(jq[NB8 - 2], slot(std::integral_constant<int, (b + NB8 - 1) % NB8>{}));
      convert(slot(b_c));
      if constexpr (kSliceBarrier) {
        wait_lgkm0();
        raw_barrier();
      }
      if (mine) compute(buf0, diag, sk, sv);
    };
    for (int i = 0; i < niter; i += NB8) {
      step8(i, std::integral_constant<int, 0>{});
      if (i + 1 < niter) step8(i + 1, std::integral_constant<int, 1>{});
      if constexpr (NB8 == 3)
        if (i + 2 < niter) step8(i + 2, std::integral_constant<int, 2>{});
    }
  }

  // No copy may still be landing in the ring once it is reused below (the
  // copies are not tracked by the compiler's own waits).
  wait_vm_lgkm0<0>();
  // ---- split pass: the item's partial state, unnormalised, in accumulator
  // order [register][lane], then m and l per lane (the merge reads the same)
  if constexpr (KS == 1) {
    if (G == 1 ? item >= 0 : item_wg) {
      if (item < 0) return;  // (a block past the last item)
      float* dst = p.partial + ((size_t)bh * p.n_items + item) * QW * (partial_bytes<D>() / 4) +
                   (size_t)qg * (partial_bytes<D>() / 4);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[(dt * 16 + r) * kWave + lane] = o[dt][r];
      dst[(D / 32) * 16 * kWave + lane] = m2;
      dst[(D / 32) * 16 * kWave + kWave + lane] = lsum;
      return;
    }
  }
  // ---- two key slices: each finishes half of the columns.  Slice s keeps
  // the d-tiles [s H, (s + 1) H), H = D / 64, publishes its other tiles with
  // its (m, l), merges the other slice's copy of its own tiles and stores them.
  if constexpr (KS == 2) {
    constexpr int H = D / 64;
    constexpr int kPF = half_partial_bytes<D>() / 4;
    __syncthreads();  // every read of the tile buffers is over
    float* part = reinterpret_cast<float*>(buf0);
    auto publish = [&](auto s_c) {
      constexpr int S = decltype(s_c)::value;
      float* mine = part + (size_t)(S * SW + ws) * kPF;
#pragma unroll
      for (int t = 0; t < H; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mine[(t * 16 + r) * kWave + lane] = o[(1 - S) * H + t][r];
      mine[H * 16 * kWave + lane] = m2;
      mine[H * 16 * kWave + kWave + lane] = lsum;
    };
    if (ks == 0) publish(std::integral_constant<int, 0>{});
    else publish(std::integral_constant<int, 1>{});
    __syncthreads();
    auto finish = [&](auto s_c) {
      constexpr int S = decltype(s_c)::value;
      const float* other = part + (size_t)((1 - S) * SW + ws) * kPF;
      const float mo = other[H * 16 * kWave + lane];
      const float lo = other[H * 16 * kWave + kWave + lane];
      const float m_new = fmaxf(m2, mo);
      if (m_new != -INFINITY) {  // else neither slice has seen a key
        const float a_self = fast_exp2(m2 - m_new);
        const float a_other = fast_exp2(mo - m_new);
        lsum = lsum * a_self + lo * a_other;
#pragma unroll
        for (int t = 0; t < H; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            o[S * H + t][r] = o[S * H + t][r] * a_self + other[(t * 16 + r) * kWave + lane] * a_other;
        m2 = m_new;
      }
      if (!has_rows) return;
      const float l_all = halves_sum(lsum);
      const float inv = l_all > 0.f ? 1.f / l_all : 0.f;
      // staged through buf1 (idle now): 32 rows of 32 H columns per wave
      constexpr int kStageB = kQRows * H * 32 * (int)sizeof(T);
      static_assert(2 * SW * kStageB <= C::kSliceBytes, "column stages fit one ring buffer");
      LDS_PTR(unsigned char) region = (LDS_PTR(unsigned char))buf1 + (S * SW + ws) * kStageB;
      store_cols_lds<T, D, S * H, H>(static_cast<T*>(p.o) + head + (size_t)q0 * D, o, inv, lane,
                                     region);
      if (S == 0 && p.lse != nullptr && (lane >> 5) == 0) {
        const float lse2 = l_all > 0.f ? m2 + log2f(l_all) : -INFINITY;
        p.lse[(size_t)bh * p.N + q0 + (lane & 31)] = lse2 * 0.69314718055994530942f;
      }
    };
    if (ks == 0) finish(std::integral_constant<int, 0>{});
    else finish(std::integral_constant<int, 1>{});
    return;
  }
  // ---- merge the key slices: slices 1..KS-1 publish (O, m, l); slice 0 merges
  if constexpr (KS > 1) {
    __syncthreads();  // every copy and read of the tile buffers is over
    float* part = reinterpret_cast<float*>(buf0);
    constexpr int kPartFloats = partial_bytes<D>() / 4;
    if (ks > 0) {
      float* mine = part + (size_t)((ks - 1) * SW + ws) * kPartFloats;
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
      const float* other = part + (size_t)((w - 1) * SW + ws) * kPartFloats;
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
  // ---- epilogue: total row sum over both lane halves, normalise, store.
  // O^T sits one query per lane; it goes row-major through this wave's own
  // LDS region (the ring is idle now), so that the global stores are whole
  // 16-byte chunks of consecutive rows.
  constexpr int kRowB = D * (int)sizeof(T);      // bytes per output row
  constexpr int kStage = kQRows * kRowB;          // a wave's 32 rows
  constexpr int kPerBuf = C::kSliceBytes / kStage;
  constexpr int kStoreWaves = KS > 1 ? SW : C::W;
  // (staged through buf1, then buf2 for a three-buffer ring, or buf0 for int8 K/V)
  constexpr bool kStaged = kPerBuf >= 1 && kStoreWaves <= (KV8 || NB == 3 ? 2 : 1) * kPerBuf;
  if constexpr (kStaged && KS == 1) __syncthreads();  // every wave is done with the ring
  if (!has_rows) return;
  const float l_all = halves_sum(lsum);
  const float inv = l_all > 0.f ? 1.f / l_all : 0.f;
  const int h = lane >> 5;
  const int row = q0 + (lane & 31);
  if constexpr (kStaged) {
    const int wv = KS > 1 ? ws : wave;  // index among the storing waves
    unsigned char* region =
        (wv < kPerBuf ? buf1 : KV8 ? buf0 : buf2) + (wv % kPerBuf) * kStage;
    store_rows_lds<T, D>(static_cast<T*>(p.o) + head + (size_t)q0 * D, o, inv, lane,
                         (LDS_PTR(unsigned char))region);
  } else {
    T* Out = static_cast<T*>(p.o) + head + (size_t)row * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
        O::store_o4(Out + dt * 32 + 8 * gg + 4 * h, o[dt][4 * gg] * inv, o[dt][4 * gg + 1] * inv,
                    o[dt][4 * gg + 2] * inv, o[dt][4 * gg + 3] * inv);
  }
  if (p.lse != nullptr && h == 0) {
    const float lse2 = l_all > 0.f ? m2 + log2f(l_all) : -INFINITY;
    p.lse[(size_t)bh * p.N + row] = lse2 * 0.69314718055994530942f;
  }
}

// Finishes the rows split across workgroups: one workgroup per (batch*head,
// heavy row, 32-column tile of O), one wave per 32 query rows.  rows holds
// (row, first item, item count) per heavy row.  Each lane first reads every
// item's (m, l) and takes their maximum, then sums the items' tile of O with
// weights exp2(m_item - m_max): independent loads, not a chain of merges.
template <typename T, int BS, int D>
__global__ __launch_bounds__(kWave * (BS / kQRows)) void bsa_fwd_merge_kernel(
    FwdParams p, const int32_t* rows, int32_t n_rows) {
  constexpr int QW = BS / kQRows;
  constexpr int kPF = partial_bytes<D>() / 4;
  constexpr int kTiles = D / 32;
  __shared__ __attribute__((aligned(16))) unsigned char stage[QW][kQRows * 32 * sizeof(T)];
  const int lane = threadIdx.x & (kWave - 1);
  const int qg = uniform(threadIdx.x / kWave);
  const int dt = blockIdx.x % kTiles;
  const int hr = (blockIdx.x / kTiles) % n_rows;
  const int bh = blockIdx.x / (kTiles * n_rows);
  const int row = rows[3 * hr], first = rows[3 * hr + 1], count = rows[3 * hr + 2];
  const float* base = p.partial + ((size_t)bh * p.n_items + first) * QW * kPF + (size_t)qg * kPF;
  const size_t item_stride = (size_t)QW * kPF;
  float m_max = -INFINITY;
  for (int c = 0; c < count; ++c)
    m_max = fmaxf(m_max, base[c * item_stride + kTiles * 16 * kWave + lane]);
  f32x16_t o[kTiles];  // only tile dt is summed; the others stay zero
#pragma unroll
  for (int t = 0; t < kTiles; ++t) o[t] = f32x16_t{};
  float lsum = 0.f;
  if (m_max != -INFINITY) {  // else no item has seen a key: O = 0, LSE = -inf
    f32x16_t acc = f32x16_t{};
#pragma unroll 4
    for (int c = 0; c < count; ++c) {
      const float* src = base + c * item_stride;
      const float w = fast_exp2(src[kTiles * 16 * kWave + lane] - m_max);
      lsum = fmaf(w, src[kTiles * 16 * kWave + kWave + lane], lsum);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = fmaf(w, src[(dt * 16 + r) * kWave + lane], acc[r]);
    }
#pragma unroll
    for (int t = 0; t < kTiles; ++t)
      if (t == dt) o[t] = acc;
  }
  const float l_all = halves_sum(lsum);
  const float inv = l_all > 0.f ? 1.f / l_all : 0.f;
  const int q0 = row * BS + qg * kQRows;
  T* const dst = static_cast<T*>(p.o) + (size_t)bh * p.N * D + (size_t)q0 * D;
  LDS_PTR(unsigned char) st = (LDS_PTR(unsigned char))stage[qg];
  if (dt == 0) store_cols_lds<T, D, 0, 1>(dst, o, inv, lane, st);
  if constexpr (kTiles > 1) if (dt == 1) store_cols_lds<T, D, 1, 1>(dst, o, inv, lane, st);
  if constexpr (kTiles > 2) if (dt == 2) store_cols_lds<T, D, 2, 1>(dst, o, inv, lane, st);
  if constexpr (kTiles > 3) if (dt == 3) store_cols_lds<T, D, 3, 1>(dst, o, inv, lane, st);
  if (dt == 0 && p.lse != nullptr && (lane >> 5) == 0) {
    const float lse2 = l_all > 0.f ? m_max + log2f(l_all) : -INFINITY;
    p.lse[(size_t)bh * p.N + q0 + (lane & 31)] = lse2 * 0.69314718055994530942f;
  }
}

// Dynamic LDS (G > 1): the union's entry list (M ints) and G + 1 bitmaps.
size_t dynamic_lds_bytes(int group, int M) {
  if (group == 1) return 0;  // the row is read from col_idx directly
  const size_t words = (size_t)(group + 1) * ((M + 31) / 32);
  return 4 * ((size_t)M + words);
}

template <typename T, int BS, int D, int G, int KS, bool KV8 = false, bool RING = false>
constexpr size_t static_lds_bytes() {  // 0 for a shape that is not instantiated
  using C = Cfg<T, BS, D, G, KS, KV8, RING>;
  return C::kValid ? (size_t)C::kLdsBytes + 16 : 0;
}

template <typename T, int BS, int D, int G, int KS, bool CAUSAL, bool KV8, bool RING = false>
bsa_status launch_kernel(const FwdParams& p, hipStream_t stream) {
  using C = Cfg<T, BS, D, G, KS, KV8, RING>;
  if constexpr (!C::kValid) {
    return BSA_ERR_INVALID_ARGUMENT;
  } else {
  constexpr size_t kStatic = static_lds_bytes<T, BS, D, G, KS, KV8, RING>();
  const size_t dyn = dynamic_lds_bytes(G, p.M);
  if (dyn + kStatic > kMaxLds) return BSA_ERR_INVALID_ARGUMENT;
  if (dyn + kStatic > 64 * 1024) {
    static std::atomic<uint64_t> raised{0};  // per instantiation, one bit per device
    uint64_t bit;
    if (due_on_device(raised, &bit)) {
      if (hipFuncSetAttribute(
              reinterpret_cast<const void*>(&bsa_fwd_kernel<T, BS, D, G, KS, CAUSAL, KV8, RING>),
              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kMaxLds - kStatic)) !=
          hipSuccess)
        return BSA_ERR_HIP;
      mark_done(raised, bit);
    }
  }
  const dim3 block(kWave * C::W);
  const dim3 grid(p.num_wg);
  hipLaunchKernelGGL((bsa_fwd_kernel<T, BS, D, G, KS, CAUSAL, KV8, RING>), grid, block, dyn, stream,
                     p);
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_ERR_HIP;
  }
}

template <typename T, int BS, int D, int G, int KS>
bsa_status launch(const FwdParams& p, hipStream_t stream) {
  if (p.k_scale != nullptr) {  // int8 K/V: bf16 only
    if constexpr (std::is_same<T, __bf16>::value)
      return p.causal != 0 ? launch_kernel<T, BS, D, G, KS, true, true>(p, stream)
                           : launch_kernel<T, BS, D, G, KS, false, true>(p, stream);
    else
      return BSA_ERR_INVALID_ARGUMENT;
  }
  if constexpr (Cfg<T, BS, D, G, KS>::kSingle) {
    if (p.split != nullptr)  // the row-split pass keeps the two-entry ring
      return p.causal != 0 ? launch_kernel<T, BS, D, G, KS, true, false, true>(p, stream)
                           : launch_kernel<T, BS, D, G, KS, false, false, true>(p, stream);
  }
  return p.causal != 0 ? launch_kernel<T, BS, D, G, KS, true, false>(p, stream)
                       : launch_kernel<T, BS, D, G, KS, false, false>(p, stream);
}

// Static LDS of a shape, or 0 when the shape is not instantiated.
template <typename T, int BS, int D, bool KV8>
size_t shape_lds_kv(int group, int key_split) {
  if (group == 1 && key_split == 1) return static_lds_bytes<T, BS, D, 1, 1, KV8>();
  if (group == 1 && key_split == 2) return static_lds_bytes<T, BS, D, 1, 2, KV8>();
  if (group == 1 && key_split == 4) return static_lds_bytes<T, BS, D, 1, 4, KV8>();
  if (group == 2 && key_split == 1) return static_lds_bytes<T, BS, D, 2, 1, KV8>();
  if (group == 4 && key_split == 1) return static_lds_bytes<T, BS, D, 4, 1, KV8>();
  return 0;
}
template <typename T, int BS, int D>
size_t shape_lds(int group, int key_split, bool kv8) {
  return kv8 ? shape_lds_kv<T, BS, D, true>(group, key_split)
             : shape_lds_kv<T, BS, D, false>(group, key_split);
}

template <typename T, int BS, int D>
bsa_status launch_shape(const FwdParams& p, hipStream_t stream) {
  if (p.group == 1 && p.key_split == 1) return launch<T, BS, D, 1, 1>(p, stream);
  if (p.group == 1 && p.key_split == 2) return launch<T, BS, D, 1, 2>(p, stream);
  if (p.group == 1 && p.key_split == 4) return launch<T, BS, D, 1, 4>(p, stream);
  if (p.group == 2 && p.key_split == 1) return launch<T, BS, D, 2, 1>(p, stream);
  if (p.group == 4 && p.key_split == 1) return launch<T, BS, D, 4, 1>(p, stream);
  return BSA_ERR_INVALID_ARGUMENT;
}

template <typename T>
bsa_status dispatch(const FwdParams& p, int bs, int d, hipStream_t stream) {
  if (bs == 32 && d == 64) return launch_shape<T, 32, 64>(p, stream);
  if (bs == 32 && d == 128) return launch_shape<T, 32, 128>(p, stream);
  if (bs == 64 && d == 64) return launch_shape<T, 64, 64>(p, stream);
  if (bs == 64 && d == 128) return launch_shape<T, 64, 128>(p, stream);
  return BSA_ERR_INVALID_ARGUMENT;
}

template <typename T, int BS, int D>
bsa_status launch_merge(const FwdParams& p, const int32_t* rows, int32_t n_rows, int64_t grid,
                        hipStream_t stream) {
  hipLaunchKernelGGL((bsa_fwd_merge_kernel<T, BS, D>), dim3((uint32_t)grid),
                     dim3(kWave * (BS / kQRows)), 0, stream, p, rows, n_rows);
  return hipGetLastError() == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}

template <typename T>
bsa_status dispatch_merge(const FwdParams& p, int bs, int d, const int32_t* rows, int32_t n_rows,
                          int64_t grid, hipStream_t stream) {
  if (bs == 32 && d == 64) return launch_merge<T, 32, 64>(p, rows, n_rows, grid, stream);
  if (bs == 32 && d == 128) return launch_merge<T, 32, 128>(p, rows, n_rows, grid, stream);
  if (bs == 64 && d == 64) return launch_merge<T, 64, 64>(p, rows, n_rows, grid, stream);
  if (bs == 64 && d == 128) return launch_merge<T, 64, 128>(p, rows, n_rows, grid, stream);
  return BSA_ERR_INVALID_ARGUMENT;
}

// Bytes of split-pass partials: per (batch*head, item), one partial state
// per 32-row wave of the query block.
int64_t split_workspace_bytes(int64_t bh, int bs, int d, int64_t n_items) {
  const int64_t per_wave = d == 64 ? partial_bytes<64>() : partial_bytes<128>();
  return bh * n_items * (bs / kQRows) * per_wave;
}

// Total LDS of a shape for (dtype, bs, d, int8 K/V), or 0 when it is not
// instantiated.
size_t lds_for(int dtype, int bs, int d, int group, int ks, int M, bool kv8 = false) {
  size_t st = 0;
  if (dtype == BSA_DTYPE_F32) {
    if (kv8) return 0;
    if (bs == 32) st = d == 64 ? shape_lds<float, 32, 64>(group, ks, false) : shape_lds<float, 32, 128>(group, ks, false);
    else st = d == 64 ? shape_lds<float, 64, 64>(group, ks, false) : shape_lds<float, 64, 128>(group, ks, false);
  } else {
    if (bs == 32) st = d == 64 ? shape_lds<__bf16, 32, 64>(group, ks, kv8) : shape_lds<__bf16, 32, 128>(group, ks, kv8);
    else st = d == 64 ? shape_lds<__bf16, 64, 64>(group, ks, kv8) : shape_lds<__bf16, 64, 128>(group, ks, kv8);
  }
  return st == 0 ? 0 : st + dynamic_lds_bytes(group, M);
}

// Compute units of the current device (read once per device; 256 on an
// MI355X, the figure used if the query fails).
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

// Workgroup shape.  Large grids: G query blocks per workgroup share their K/V
// tiles (4 blocks of 32 rows, or 2 of 64).  Smaller grids: one query block
// per workgroup, which has the shortest critical path, with each CSR row split
// over KS key-slice wave sets while the grid stays within two waves per SIMD
// (the worked example, 1024 query blocks of one wave, runs 9.2 us with KS = 2
// against 9.8 us with KS = 1).
void choose_shape(int64_t bhm, int bs, int d, int dtype, int M, int* group, int* key_split,
                  bool kv8 = false, bool banded = false) {
  const int64_t kCus = device_cus();
  const int64_t kLargeGrid = 8 * 4 * kCus;  // 8 query waves per SIMD
  const int qw = bs / kQRows;
  auto fits = [&](int g, int ks) {
    const size_t b = lds_for(dtype, bs, d, g, ks, M, kv8);
    return b != 0 && b <= kMaxLds;
  };
  int g = 1, ks = 1;
  if (bhm * qw >= kLargeGrid) {
    // bf16 at block 64 keeps one query block per workgroup: its one-tile K
    // and V slots already hold two waves per SIMD, while two rows per
    // workgroup make each wave idle through the entries only the other row
    // selects (29% of the steps of the log-linear pattern at M = 512, 42% of
    // a Bernoulli(0.3) mask's at M = 32).  A banded pattern (dense rows taken
    // by a row split) is the exception: neighbouring rows share nearly every
    // block, and two rows per workgroup halve its copies.
    g = bs == 32 ? 4 : (dtype == BSA_DTYPE_BF16 && !kv8 && !banded ? 1 : 2);
    if (!fits(g, 1)) g = 1;
  } else {
    while (ks < 4 && qw * ks * 2 <= kMaxWaves && bhm * qw * ks * 2 <= 2 * 4 * kCus &&
           fits(1, ks * 2))
      ks *= 2;
  }
  *group = g;
  *key_split = ks;
}

}  // namespace

namespace {

// Rows split across workgroups (bsa_forward_split).
struct SplitPlan {
  const uint8_t* heavy;
  const int32_t* items;
  int32_t n_items;
  const int32_t* rows;
  int32_t n_rows;
  void* workspace;
  int64_t workspace_bytes;
};

bsa_status forward_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                        int32_t batch, int32_t heads, int32_t seq_len, int32_t head_dim,
                        int32_t block_size, int32_t dtype, const int32_t* row_ptr,
                        const int32_t* col_idx, int64_t nnz, float scale, int32_t flags,
                        int32_t group, int32_t key_split, void* stream,
                        const SplitPlan* plan = nullptr, const float* k_scale = nullptr,
                        const float* v_scale = nullptr) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || row_ptr == nullptr ||
      col_idx == nullptr)
    return BSA_ERR_NULL_POINTER;
  if (dtype != BSA_DTYPE_F32 && dtype != BSA_DTYPE_BF16) return BSA_ERR_INVALID_ARGUMENT;
  if (block_size != 32 && block_size != 64) return BSA_ERR_INVALID_ARGUMENT;
  if (head_dim != 64 && head_dim != 128) return BSA_ERR_INVALID_ARGUMENT;
  if (batch <= 0 || heads <= 0 || seq_len <= 0 || seq_len % block_size != 0) return BSA_ERR_SHAPE;
  if (!(scale == scale) || std::isinf(scale)) return BSA_ERR_INVALID_ARGUMENT;
  if ((flags & ~(BSA_FORWARD_CAUSAL | BSA_FORWARD_PATTERN_PER_HEAD)) != 0)
    return BSA_ERR_INVALID_ARGUMENT;
  const bool per_head = (flags & BSA_FORWARD_PATTERN_PER_HEAD) != 0;
  const int64_t M = seq_len / block_size;
  const int64_t patterns = per_head ? heads : 1;
  if (nnz < patterns * M || nnz > patterns * M * M) return BSA_ERR_SHAPE;
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
  p.heads = heads;
  p.causal = (flags & BSA_FORWARD_CAUSAL) != 0 ? 1 : 0;
  p.row_stride = per_head ? static_cast<int32_t>(M + 1) : 0;
  p.heavy = nullptr;
  p.split = nullptr;
  p.n_items = 0;
  p.partial = nullptr;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  const bool kv8 = k_scale != nullptr;
  if (kv8 && (v_scale == nullptr || dtype != BSA_DTYPE_BF16 || plan != nullptr))
    return BSA_ERR_INVALID_ARGUMENT;
  const bool split = plan != nullptr && plan->n_items > 0;
  if (plan != nullptr) {
    if (per_head) return BSA_ERR_INVALID_ARGUMENT;  // the plan is of one shared pattern
    if (plan->n_items < 0 || plan->n_rows < 0 || (plan->n_items > 0) != (plan->n_rows > 0) ||
        plan->n_rows > M || plan->n_items > nnz)
      return BSA_ERR_SHAPE;
    if (split && (plan->heavy == nullptr || plan->items == nullptr || plan->rows == nullptr ||
                  plan->workspace == nullptr))
      return BSA_ERR_NULL_POINTER;
    if (split) {
      if ((int64_t)batch * heads * plan->n_items > INT32_MAX) return BSA_ERR_SHAPE;
      if (reinterpret_cast<uintptr_t>(plan->workspace) % 16 != 0) return BSA_ERR_INVALID_ARGUMENT;
      if (plan->workspace_bytes <
          split_workspace_bytes((int64_t)batch * heads, block_size, head_dim, plan->n_items))
        return BSA_ERR_BUFFER_TOO_SMALL;
      if (lds_for(dtype, block_size, head_dim, 1, 1, (int)M) == 0) return BSA_ERR_INVALID_ARGUMENT;
      p.heavy = plan->heavy;
    }
  }
  if (group == 0 && key_split == 0) {
    choose_shape((int64_t)batch * heads * M, block_size, head_dim, dtype, (int)M, &p.group,
                 &p.key_split, kv8, split);
  } else {
    const int qw = block_size / kQRows;
    if (qw * group * key_split > kMaxWaves) return BSA_ERR_INVALID_ARGUMENT;
    p.group = group;
    p.key_split = key_split;
  }
  const size_t lds = lds_for(dtype, block_size, head_dim, p.group, p.key_split, (int)M, kv8);
  if (lds == 0 || lds > kMaxLds) return BSA_ERR_INVALID_ARGUMENT;
  const int64_t ngroups = (M + p.group - 1) / p.group;
  // Several query blocks per workgroup and one key slice: the heavy rows'
  // items run in the same launch as the groups, G per workgroup (the split
  // pass's own launch is left out).
  const bool fused = split && p.group > 1 && p.key_split == 1;
  p.split = nullptr;
  p.n_items = 0;
  p.n_tuples = 0;
  if (fused) {
    p.split = plan->items;
    p.n_items = plan->n_items;
    p.partial = static_cast<float*>(plan->workspace);
    p.n_tuples = (plan->n_items + p.group - 1) / p.group;
  }
  const int64_t num_wg = (int64_t)batch * heads * (ngroups + p.n_tuples);
  if (num_wg > INT32_MAX) return BSA_ERR_SHAPE;
  p.num_wg = static_cast<int32_t>(num_wg);
  const float s = scale > 0.f ? scale : 1.0f / std::sqrt(static_cast<float>(head_dim));
  p.scale_log2 = s * 1.4426950408889634f;

  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale, non-sticky error from earlier calls
  bsa_status r = dtype == BSA_DTYPE_F32 ? dispatch<float>(p, block_size, head_dim, st)
                                        : dispatch<__bf16>(p, block_size, head_dim, st);
  if (r != BSA_OK || !split) return r;
  // The heavy rows: their items (in their own launch of one-block workgroups
  // unless they ran beside the groups), then the merge.  (Forking the item
  // launch onto a second stream to overlap the main pass was measured:
  // within a few percent either way.)
  FwdParams ps = p;
  ps.heavy = nullptr;
  ps.split = plan->items;
  ps.n_items = plan->n_items;
  ps.partial = static_cast<float*>(plan->workspace);
  if (!fused) {
    ps.group = 1;
    ps.key_split = 1;
    ps.n_tuples = 0;
    ps.num_wg = batch * heads * plan->n_items;
    r = dtype == BSA_DTYPE_F32 ? dispatch<float>(ps, block_size, head_dim, st)
                               : dispatch<__bf16>(ps, block_size, head_dim, st);
    if (r != BSA_OK) return r;
  }
  const int64_t grid = (int64_t)batch * heads * plan->n_rows * (head_dim / 32);
  return dtype == BSA_DTYPE_F32
             ? dispatch_merge<float>(ps, block_size, head_dim, plan->rows, plan->n_rows, grid, st)
             : dispatch_merge<__bf16>(ps, block_size, head_dim, plan->rows, plan->n_rows, grid, st);
}

}  // namespace

extern "C" bsa_status bsa_forward(const void* q, const void* k, const void* v, void* o,
                                  float* lse, int32_t batch, int32_t heads, int32_t seq_len,
                                  int32_t head_dim, int32_t block_size, int32_t dtype,
                                  const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                                  float scale, void* stream) {
  return forward_impl(q, k, v, o, lse, batch, heads, seq_len, head_dim, block_size, dtype,
                      row_ptr, col_idx, nnz, scale, 0, 0, 0, stream);
}

extern "C" bsa_status bsa_forward_ex(const void* q, const void* k, const void* v, void* o,
                                     float* lse, int32_t batch, int32_t heads, int32_t seq_len,
                                     int32_t head_dim, int32_t block_size, int32_t dtype,
                                     const int32_t* row_ptr, const int32_t* col_idx,
                                     int64_t nnz, float scale, int32_t flags, int32_t group,
                                     int32_t key_split, void* stream) {
  return forward_impl(q, k, v, o, lse, batch, heads, seq_len, head_dim, block_size, dtype,
                      row_ptr, col_idx, nnz, scale, flags, group, key_split, stream);
}

extern "C" int64_t bsa_row_split_workspace_bytes(int32_t batch, int32_t heads, int32_t block_size,
                                                 int32_t head_dim, int32_t n_items) {
  if (batch <= 0 || heads <= 0 || n_items < 0 || (block_size != 32 && block_size != 64) ||
      (head_dim != 64 && head_dim != 128))
    return -1;
  return split_workspace_bytes((int64_t)batch * heads, block_size, head_dim, n_items);
}

extern "C" bsa_status bsa_forward_split(const void* q, const void* k, const void* v, void* o,
                                        float* lse, int32_t batch, int32_t heads,
                                        int32_t seq_len, int32_t head_dim, int32_t block_size,
                                        int32_t dtype, const int32_t* row_ptr,
                                        const int32_t* col_idx, int64_t nnz, float scale,
                                        int32_t flags, const uint8_t* heavy,
                                        const int32_t* items, int32_t n_items,
                                        const int32_t* rows, int32_t n_rows, void* workspace,
                                        int64_t workspace_bytes, void* stream) {
  const SplitPlan plan{heavy, items, n_items, rows, n_rows, workspace, workspace_bytes};
  return forward_impl(q, k, v, o, lse, batch, heads, seq_len, head_dim, block_size, dtype,
                      row_ptr, col_idx, nnz, scale, flags, 0, 0, stream, &plan);
}

extern "C" bsa_status bsa_forward_int8kv(const void* q, const int8_t* k_codes,
                                         const float* k_scales, const int8_t* v_codes,
                                         const float* v_scales, void* o, float* lse,
                                         int32_t batch, int32_t heads, int32_t seq_len,
                                         int32_t head_dim, int32_t block_size,
                                         const int32_t* row_ptr, const int32_t* col_idx,
                                         int64_t nnz, float scale, int32_t flags, int32_t group,
                                         int32_t key_split, void* stream) {
  if (k_scales == nullptr || v_scales == nullptr) return BSA_ERR_NULL_POINTER;
  return forward_impl(q, k_codes, v_codes, o, lse, batch, heads, seq_len, head_dim, block_size,
                      BSA_DTYPE_BF16, row_ptr, col_idx, nnz, scale, flags, group, key_split,
                      stream, nullptr, k_scales, v_scales);
}
