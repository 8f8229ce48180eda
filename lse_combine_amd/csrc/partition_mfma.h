// Split-K pass 1 on the matrix cores for bf16 (or fp8) caches and a GQA group of up to 16
// (query, head) columns per kv head (FA4Config: fused GQA tiles, BM_eff). The depths are a
// template shape (MShape): Dqk = Dv = 128, and the wider pairs with rotary columns
// (FA4Config, rope_depth: the q.K depth minus the nope depth, which may differ from the V
// depth), optionally stored apart in bf16 (FA4Config, rope_dtype). Shapes are instantiated
// by the translation units that include this header.
//
// Work decomposition. A workgroup covers one partition p of one sequence b for HG
// kv heads, with KS waves per kv head splitting the partition's keys (NW = HG * KS
// <= 8 waves). Wave w serves kv head kg*HG + w % HG and takes the 32-key tiles
// ks, ks + KS, ... (ks = w / HG). With HG = 8 the waves of a workgroup read the
// eight 256-byte kv-head slices of the same tokens, i.e. whole 2 KB token rows of
// the paged cache; HG shrinks when that would leave too few workgroups for the chip.
// Under the equal-share schedule a workgroup runs the pieces of its share one by one.
//
// Per tile, with v_mfma_f32_16x16x32_bf16:
//   S^T[key][col] = K[key][:] . q[col][:]      A = K rows: read from the wave's LDS K tile
//                                              (bf16, depth 128) or loaded straight into
//                                              the A-operand layout (wider depths, fp8),
//                                              B = q (16 columns, see below)
//   p = exp2((x - m_new) * c)                  online softmax in fp32; a lane owns one
//                                              column and 8 keys, so the tile max needs
//                                              two cross-lane steps
//   O^T[d][col] += V^T[d][key] . P^T[key][col] A = V^T read from LDS with the gfx950
//                                              transposing read ds_read_b64_tr_b16,
//                                              B = P^T straight from the S^T registers
//
// P must not be rounded to bf16 before P.V (the fp32 O must stay within 1e-5), so it
// is split as p = hi + lo, hi = bf16(p), lo = bf16(p - hi) (about 16 significant
// bits). When g <= 8 the 16 MFMA columns hold the g heads twice: columns 0-7 carry hi
// and 8-15 carry lo (their scores are equal), so hi and lo cost one MFMA and the two
// column halves of O^T are added at the end. For 8 < g <= 16 a second MFMA per depth
// block adds the lo part.
//
// Addressing: tiles are 32 keys and partitions start on multiples of 32, so with a
// contiguous cache or pages of a power of two >= 32 keys a tile is 32 consecutive cache
// rows, and with pages of 16 keys each 16-key half of it is: every load covers one half, its
// base is a scalar and every lane adds a fixed 32-bit offset. Other page sizes take a
// per-key page lookup: every lane finds its own row. The page
// indices of the partition are staged in LDS once, so no dependent page-table load
// sits between consecutive prefetches. Loads run one tile ahead: the next tile's K is
// requested once the current tile's scores are done and its V once the current P.V is
// done (bf16); fp8 caches, half the bytes per tile, keep two tiles in flight.
//
// Epilogue: with KS = 1 every wave stores its own normalised partial and (m, l)
// (fa4_splitk_combine_write, second paragraph), or the finished bf16 row when the
// sequence has a single partition. With KS > 1 the waves of a kv head first merge
// their (m, l, O) through LDS with the log-sum-exp weights (fa4_lse_combine_write:
// fragments merged with per-row scales).
#pragma once

#include "da_device.h"

namespace da {
namespace mfma {

constexpr int kTile = 32;
constexpr int kMaxWaves = 8;
constexpr int kMaxLdsPages = 512;             // page indices of one segment staged in LDS
constexpr int kLdsBytes = 160 * 1024;         // LDS of one compute unit (gfx950)

// Depths of one instantiation. DR > 0: the last DR columns of every K row are stored apart
// (bf16, k_rope); the K cache holds the first DK = DQK - DR.
template <int DQK_, int DV_, int DR_>
struct MShape {
  static constexpr int DQK = DQK_;             // q.K depth
  static constexpr int DV = DV_;               // V / output depth
  static constexpr int DR = DR_;               // rotary columns stored apart (0: none)
  static constexpr int DK = DQK - DR;          // columns held by the K cache
  static constexpr int NJ = DQK / 32;          // 32-deep MFMA steps of the scores
  static constexpr int NJK = DK / 32;          //   ... over the K cache columns
  static constexpr int NR = DR / 32;           //   ... over the rotary columns
  static constexpr int DB = DV / 16;           // 16-deep blocks of O
  static constexpr int kVRow = DV * 2;         // bytes of one bf16 V row in LDS
  static constexpr int kVXm = DV >= 128 ? 15 : DV / 8 - 1;   // chunk swizzle mask of a V row
  static constexpr int kVBytes = kTile * kVRow;       // one wave's V tile in LDS
  // fp8 caches stage V codes (32 x DV bytes per tile) beside a half-depth bf16 tile; at
  // V depth 128 the region has room for two staged tiles (two tiles in flight)
  static constexpr int kV8Tiles = DV == 128 ? 2 : 1;
  // bf16 caches at depth 128/128 and 64/64 also stage the K tile (32 rows like V's) in the
  // region
  static constexpr bool kKLds = DQK == DV && (DV == 128 || DV == 64) && DR == 0;
  static constexpr int kRegionBytes = kKLds ? 2 * kVBytes : (kV8Tiles == 2 ? 3 * kTile * DV : kVBytes);
  static_assert(!kKLds || 3 * kTile * DV <= 2 * kVBytes, "the fp8 staging fits the region");
  static_assert(kRegionBytes >= kVBytes, "the region holds a bf16 V tile");
  static constexpr int kWaveBytes = kRegionBytes + 256;   // + merge (m, l) for up to 16 columns
  static_assert(DK % 64 == 0 && DR % 32 == 0 && (DV == 64 || DV == 128 || DV == 256), "unsupported depths");
};

typedef short s16x8 __attribute__((ext_vector_type(8)));


__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kLoadNT));
}

// K rows of one tile in registers: [16-key half][16-byte load]; bf16 loads hold 8 values,
// fp8 loads 16. The rotary columns (bf16) stored apart have loads of their own.
template <class S, bool F8>
struct KTile {
  static constexpr int NL = F8 ? S::DK / 64 : S::DK / 32;
  u32x4 k[2][NL];
  u32x4 r[2][S::NR > 0 ? S::NR : 1];
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Grid. Equal shares: (W workers, head groups). Fixed chunks: (partitions x head groups,
// sequences) with the head groups fastest, so that the workgroups of all kv heads of one
// key range are dispatched together and read neighbouring parts of the same token rows at
// about the same time (gqa 29.8 -> 28.7 us, long 55 -> 53.3 us against partitions fastest).
__device__ __forceinline__ int groups_of(const PartArgs& a, int HG) {
  return a.workers > 0 ? (int)gridDim.y : (a.Hkv + HG - 1) / HG;
}
__device__ __forceinline__ int grp_of(const PartArgs& a, int HG) {
  return a.workers > 0 ? (int)blockIdx.y : (int)blockIdx.x % groups_of(a, HG);
}
__device__ __forceinline__ int fixed_part_of(const PartArgs& a, int HG) { return (int)blockIdx.x / groups_of(a, HG); }
__device__ __forceinline__ int fixed_seq_of() { return (int)blockIdx.y; }

template <int V>
struct IntC {
  static constexpr int value = V;
};


// max over the four lanes n, n+16, n+32, n+48 (the four key groups of a column).
// (v_permlane32_swap / v_permlane16_swap would do this on the VALU, but this compiler
// folds the two results of a swap of a value with itself into one, losing half the
// lanes; the LDS permute is used instead.)
__device__ __forceinline__ float max_over_key_groups(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}

// Zero a wave's V tile once per launch: direct-to-LDS loads outside the buffer range
// leave their rows untouched, and those rows must hold finite values (they meet p = 0).
template <class S>
__device__ __forceinline__ void zero_v_tile(char* vt, int lane) {
#pragma unroll
  for (int i = 0; i < S::kRegionBytes / 1024; ++i) *(u32x4*)(vt + (i * 64 + lane) * 16) = u32x4{0u, 0u, 0u, 0u};
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the zeros are in place before any load lands
}

// Per-wave constants of a workgroup: its place in the (kv head, key split) grid and the
// lane's MFMA coordinates.
struct WaveInfo {
  int HG, KS, NW, w, ks, kvh, lane, n, qd, hc;
  int qi, hh;   // the (query, head-in-group) pair of this lane's MFMA column
  bool wave_active, col_valid, is_lo;
};

// KS > 1: merge the key splits of each kv head through LDS (each wave reuses its own V
// region; waves that saw no tile hold m = -inf, l = 0, O = 0 and get weight 0), with the
// log-sum-exp weights of the two-fragment combine (fa4_lse_combine_write).
template <bool HL, class S>
__device__ __forceinline__ OwnPartial merge_key_splits(const PartArgs& a, const WaveInfo& wv, char* smem, int b,
                                                       int p, bool direct, const f32x4* o, float m_run,
                                                       float l_run) {
  const int tid = threadIdx.x, NW = wv.NW, HG = wv.HG, KS = wv.KS, kg = grp_of(a, HG);
  const int hc = wv.hc, qd = wv.qd, g = a.g;
  const bool col_valid = wv.col_valid, is_lo = wv.is_lo;
  const float c = a.c;
  constexpr int DV = S::DV;
  char* vt = smem + wv.w * S::kWaveBytes;
  float* mo = (float*)vt;                      // [16][DV] O of this wave
  float* mml = (float*)(vt + S::kRegionBytes);   // m[16], l[16]
  __syncthreads();
  if (col_valid && !is_lo) {
#pragma unroll
    for (int db = 0; db < S::DB; ++db) *(f32x4*)(mo + hc * DV + 16 * db + 4 * qd) = o[db];
    if (qd == 0) {
      mml[hc] = m_run;
      mml[16 + hc] = l_run;
    }
  }
  __syncthreads();
  constexpr int kUnits = DV / 4;
  const int cols = a.q_len * g;   // (query, head) columns per kv head
  const int units = HG * cols * kUnits;
  OwnPartial own;
  for (int u = tid; u < units; u += NW * 64) {
    const int mem = u / (cols * kUnits);
    const int h = (u / kUnits) % cols, d0 = (u % kUnits) * 4;
    const int kv2 = kg * HG + mem;
    if (kv2 >= a.Hkv) continue;
    // (a split that saw no key of this column holds l = 0 and weighs nothing)
    float M = -INFINITY;
    for (int s2 = 0; s2 < KS; ++s2) {
      const float* ml = (const float*)(smem + (s2 * HG + mem) * S::kWaveBytes + S::kRegionBytes);
      if (ml[16 + h] > 0.f) M = fmaxf(M, ml[h]);
    }
    float Ls = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s2 = 0; s2 < KS; ++s2) {
      const char* reg = smem + (s2 * HG + mem) * S::kWaveBytes;
      const float* ml = (const float*)(reg + S::kRegionBytes);
      if (ml[16 + h] > 0.f) {
        const float e = exp2_fast((ml[h] - M) * c);
        Ls = fmaf(ml[16 + h], e, Ls);
        acc += e * *(const f32x4*)((const float*)reg + h * DV + d0);
      }
    }
    const int row = (h / g) * a.Hq1 + kv2 * g + h % g;
    const f32x4 on = acc * (Ls > 0.f ? 1.f / Ls : 0.f);
    if (u == tid) {
      // (the fused combine's fold takes the units in this order; with one unit per thread the
      // thread keeps the partial it stores)
      own.idx = p;
      own.ml = make_float2(M, Ls);
      own.o = on;
    }
    store_unit(a, b, row, p, direct, d0, on, M, Ls, d0 == 0);
  }
  // the merge read other waves' V tiles: the next piece may refill them only after this
  __syncthreads();
  return units <= NW * 64 ? own : OwnPartial();
}

// Last-arriving-workgroup combine (fa4_splitk_combine_write, fourth paragraph: the writer
// that completes the set combines all). After storing its partial, every workgroup of a
// (sequence, kv-head group) publishes it device-wide and counts itself in; the one that
// brings the count to the number of partitions reads the others' partials and writes the
// final bf16 rows, LSE and fp32 O of the group's heads, then returns the counter to zero for
// the next call. The counters (one int per (sequence, group)) must be zero before the first
// call.
// Publication without cache-wide fences: in fused mode every partial is stored with cache
// policy SC1 (store_unit), i.e. written through the XCD's L2, and such a store counts as
// complete only once it is visible to every XCD. Every wave waits until its own partial
// stores are complete (vmcnt(0)) before the workgroup barrier, and only after that barrier
// does one thread increment the counter (an agent-scope atomic). The workgroup that
// completes the count therefore sees every partial of the set already visible device-wide;
// its waves read them, after a second barrier, with SC1 loads, which never return a stale
// line of their own XCD's L2 (that L2 may hold lines of these addresses from an earlier
// call). The usual agent-scope release/acquire pair would instead write back and invalidate
// the whole L2 of the XCD in every workgroup; the SC1 stores and loads cost the same
// number of instructions as plain ones.
// The fold uses every thread of the workgroup: NT / S (row, 4-wide slice) units at a time,
// S threads per unit splitting the partitions (merged through LDS like the combine launch).
template <class S>
__device__ __forceinline__ void fused_combine(const PartArgs& a, const WaveInfo& wv, char* smem, int* flag_s, int b,
                                              int count, int first_slot, OwnPartial own) {
  const int tid = threadIdx.x, HG = wv.HG, kg = grp_of(a, HG), g = a.g;
  wait_vm<0>();   // this wave's partial stores are complete
  __syncthreads();
  int* cnt = a.counters + (int64_t)b * groups_of(a, HG) + kg;
  if (tid == 0) {
    const int last = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == count - 1;
    *flag_s = last ? 1 : 0;
  }
  __syncthreads();
  if (!__builtin_amdgcn_readfirstlane(*flag_s)) return;
  const int kv_end = min((kg + 1) * HG, a.Hkv);
  const int cols = a.q_len * g, ncol = (kv_end - kg * HG) * cols;
  constexpr int DV = S::DV;
  constexpr int kUnits = DV / 4;
  const int NT = wv.NW * 64;
  const int total = ncol * kUnits;
  // (S threads per unit: 1 up to 16 partitions, 4 up to 64, else 16)
  const int SUB = count <= 16 ? 1 : (count <= 64 ? 4 : 16);
  const int UNITS = NT / SUB;
  const int sub = tid / UNITS, ui = tid % UNITS;
  // the thread's own partial (stored by merge_key_splits for unit tid) stays in registers when
  // the fold gives every unit to one thread in a single round: index among the row's partials
  if (SUB == 1 && total <= UNITS && own.idx >= 0) {
    if (first_slot >= 0) own.idx -= first_slot;
  } else {
    own.idx = -1;
  }
  // (the merge's LDS: the waves' tile regions, free by now)
  float* sM = (float*)smem;                          // [SUB][UNITS]
  float* sL = sM + SUB * UNITS;
  f32x4* sO = (f32x4*)(sL + SUB * UNITS);
  for (int u0 = 0; u0 < total; u0 += UNITS) {
    const int u = u0 + ui;
    const bool valid = u < total && sub < SUB;
    int64_t row = 0, first = 0, stride = 1;
    int d0 = 0;
    if (valid) {
      const int cc = u / kUnits;
      d0 = (u % kUnits) * 4;
      const int kv = kg * HG + cc / cols, col = cc % cols;
      const int h = (col / g) * a.Hq1 + kv * g + col % g;   // row within the sequence
      row = (int64_t)b * a.Hq + h;
      // partial rows of this head: equal shares [slot][Hq], fixed chunks [B][Hq][max_splits]
      first = first_slot >= 0 ? (int64_t)first_slot * a.Hq + h : row * a.max_splits;
      stride = first_slot >= 0 ? a.Hq : 1;
    }
    float M = -INFINITY, Ls = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (valid)
      fold_partials<DV, 8, true>((const float2*)a.part_ml + first, a.part_o + first * DV + d0, stride, count, sub,
                                 SUB, a.c, M, Ls, acc, a.part_ml, a.part_o, own);
    if (SUB > 1) {
      if (sub < SUB) {
        sM[sub * UNITS + ui] = M;
        sL[sub * UNITS + ui] = Ls;
        sO[sub * UNITS + ui] = acc;
      }
      __syncthreads();
      if (valid && sub == 0) {
        float G = -INFINITY;
        for (int t = 0; t < SUB; ++t)
          if (sL[t * UNITS + ui] > 0.f) G = fmaxf(G, sM[t * UNITS + ui]);
        Ls = 0.f;
        acc = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int t = 0; t < SUB; ++t) {
          if (sL[t * UNITS + ui] > 0.f) {
            const float e = exp2_fast((sM[t * UNITS + ui] - G) * a.c);
            Ls += sL[t * UNITS + ui] * e;
            acc += e * sO[t * UNITS + ui];
          }
        }
        M = G;
      }
      __syncthreads();   // (the LDS is reused by the next units)
    }
    if (valid && sub == 0) write_row_unit(a.out, a.o32, a.lse, row, DV, d0, M, Ls, acc, a.scale);
  }
  if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One piece of work: keys [start, end) of sequence b for this workgroup's kv heads.
// Writes the normalised partial and (m, l) of partition / slot p, or the finished bf16
// row when `direct` (the sequence has a single partition).
template <bool HL, int PM, bool F8, class S>
__device__ __forceinline__ void run_piece(const PartArgs& a, const WaveInfo& wv, char* smem, int* pages_s,
                                          int* flag_s, int b, int start, int end, int p, int count,
                                          int first_slot) {
  // (count = partitions of sequence b; first_slot = its first slot under equal shares, or -1)
  constexpr int DQK = S::DQK, DK = S::DK, DR = S::DR, DB = S::DB, NJ = S::NJ, NJK = S::NJK;
  typedef KTile<S, F8> KT;
  const bool direct = a.direct_single && count == 1;
  const int lane = wv.lane, n = wv.n, qd = wv.qd, kvh = wv.kvh, ks = wv.ks, KS = wv.KS;
  const int g = a.g;
  const bool wave_active = wv.wave_active, col_valid = wv.col_valid, is_lo = wv.is_lo;
  const float lo_mask = is_lo ? 1.f : 0.f;
  char* vt = smem + wv.w * S::kWaveBytes;
  int first_page = 0;   // page index held by pages_s[0] in the current segment
  // keys this lane's column attends: query qi of q_len sees keys t < L - q_len + 1 + qi
  const int L_seq = __builtin_amdgcn_readfirstlane(attended_len(a, b, PM == kContiguous));
  const int col_end = min(end, L_seq - a.q_len + 1 + wv.qi);

  // q as the B operand of S^T = K q^T: column n; MFMA step j covers depth 32j + 8qd .. +8
  // (bf16 caches) or, matching the 16-value fp8 loads of K, depth 64(j/2) + 16qd + 8(j%2)
  // .. +8 (the order of the depth sum is free as long as q and K agree). Steps past the
  // K cache columns take the rotary columns stored apart, 32 per step as for bf16.
  bf16x8 qf[NJ];
  {
    const int kv_safe = wave_active ? kvh : 0;
    const uint16_t* qrow = (const uint16_t*)a.q +
                           ((int64_t)b * a.Hq + (int64_t)wv.qi * a.Hq1 + (int64_t)kv_safe * g + wv.hh) * DQK;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int d0 = j >= NJK ? DK + 32 * (j - NJK) + 8 * qd
                              : (F8 ? 64 * (j >> 1) + 16 * qd + 8 * (j & 1) : 32 * j + 8 * qd);
      u32x4 v = *(const u32x4*)(qrow + d0);
      if (!col_valid) v = u32x4{0u, 0u, 0u, 0u};
      qf[j] = as_bf16x8(v);
    }
  }

  const char* kc = (const char*)a.k;
  const char* kr = (const char*)a.k_rope;
  const char* vc = (const char*)a.v;
  constexpr uint32_t es = F8 ? 1 : 2;                              // bytes per cache element
  // (a.Hkv counts virtual kv heads, a.kv_div of them per cached kv head)
  const int kv_heads = a.Hkv / a.kv_div;                          // kv heads in the cache rows
  const int kvc = (wave_active ? kvh : 0) / a.kv_div;             // this wave's cached kv head
  const uint32_t krow_bytes = (uint32_t)kv_heads * DK * es;       // bytes between tokens (K)
  const uint32_t rrow_bytes = (uint32_t)kv_heads * DR * 2;        // ... (rotary columns, bf16)
  const uint32_t vrow_bytes = (uint32_t)kv_heads * a.v_row_len * es; // ... (V)
  const uint32_t kslice = (uint32_t)kvc * DK * es;
  const uint32_t rslice = (uint32_t)kvc * DR * 2;
  const uint32_t vslice = (uint32_t)kvc * a.v_row_len * es;
  const float c = a.c;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int tid = threadIdx.x, NW = wv.NW;
  // first cache row of the tile starting at t0 (contiguous / aligned pages: the tile
  // is 32 consecutive rows; pages of 16 keys: the 16-key run starting at t0), and the row
  // of key t in the general paged case
  auto tile_row0 = [&](int t0) -> int64_t {
    if constexpr (PM == kContiguous) {
      return (int64_t)b * a.kv_capacity + t0;
    } else {
      const int pi = t0 >> a.page_shift;   // pages are a power of two >= 16 keys
      // an LDS value read at a uniform address: tell the compiler it is uniform; index and
      // value are clamped so that no cache address can leave the page pool
      const int slot = min(max(pi - first_page, 0), kMaxLdsPages - 1);
      // (clamped before readfirstlane: a clamp after it may be done in vector registers,
      // which makes the descriptor divergent and every load a waterfall loop)
      const int page = __builtin_amdgcn_readfirstlane(min(max(pages_s[slot], 0), a.num_pages - 1));
      return ((int64_t)page << a.page_shift) + (t0 & (a.page_size - 1));
    }
  };
  // first cache row of 16-key half h of the tile at t0, given row0 = tile_row0(t0): every
  // half is 16 consecutive cache rows (with pages of 16 keys each half is a page of its own)
  auto half_row0 = [&](int t0, int64_t row0, int h) -> int64_t {
    if constexpr (PM == kPagedHalf) return h == 0 ? row0 : tile_row0(t0 + 16);
    else return row0 + 16 * h;
  };
  // (general case: the page of key t and its slot in that page)
  auto general_page = [&](int t, int& off) -> int {
    t = max(t, 0);
    const int pi = t / a.page_size;
    const int slot = min(max(pi - first_page, 0), kMaxLdsPages - 1);
    off = t - pi * a.page_size;
    return min(max(pages_s[slot], 0), a.num_pages - 1);
  };
  auto general_row = [&](int t) -> int64_t {
    int off;
    const int page = general_page(t, off);
    return (int64_t)page * a.page_size + off;
  };

  // Per-lane byte offsets inside a 16-row half tile: key n, 16-byte depth chunk qd
  // (+64 bytes per load, an immediate).
  const uint32_t koff = (uint32_t)n * krow_bytes + 16 * qd;
  const uint32_t roff = (uint32_t)n * rrow_bytes + 16 * qd;

  // K of the tile at t0 into registers (A operand of the score MFMAs).
  // (valid = false: the loads are issued with an empty buffer range, i.e. they return
  // zeros without touching memory; loops that always issue the same loads use this)
  auto load_k = [&](KT& T, int t0, bool valid = true) {
    const int last = valid ? min(kTile - 1, end - 1 - t0) : -1;
    if constexpr (PM != kPagedGeneral) {
      // The tile is 32 consecutive cache rows: a scalar base per 16-row half. Each half's
      // buffer range covers only its valid rows, so on a ragged last tile the loads of
      // missing keys return zeros without touching memory (their scores are masked).
      const int64_t row0 = tile_row0(t0);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // (the clamp is selected as a vector op; readfirstlane keeps the descriptor scalar)
        const int rows = __builtin_amdgcn_readfirstlane(min(max(last + 1 - 16 * h, 0), 16));
        const int64_t rowh = half_row0(t0, row0, h);
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(kc + rowh * krow_bytes + kslice), 0, rows * krow_bytes, kRsrcWord3);
        // bf16: 8 values per load, depth 32l + 8qd; fp8: 16 values, depth 64l + 16qd
#pragma unroll
        for (int l = 0; l < KT::NL; ++l) T.k[h][l] = buf_load16(rk, koff + 64 * l, 0);
        if constexpr (S::NR > 0) {
          const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
              (void*)(kr + rowh * rrow_bytes + rslice), 0, rows * rrow_bytes, kRsrcWord3);
#pragma unroll
          for (int l = 0; l < S::NR; ++l) T.r[h][l] = buf_load16(rr, roff + 64 * l, 0);
        }
      }
    } else {
      // per-key page lookup: each lane reads its own key's row (keys past the end of a ragged
      // tile repeat the last one; their scores are masked)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int64_t row = general_row(t0 + min(n + 16 * blk, last));
        const char* kp = kc + row * krow_bytes + kslice + 16 * qd;
#pragma unroll
        for (int l = 0; l < KT::NL; ++l) T.k[blk][l] = __builtin_nontemporal_load((const u32x4*)(kp + 64 * l));
        if constexpr (S::NR > 0) {
          const char* rp = kr + row * rrow_bytes + rslice + 16 * qd;
#pragma unroll
          for (int l = 0; l < S::NR; ++l) T.r[blk][l] = __builtin_nontemporal_load((const u32x4*)(rp + 64 * l));
        }
      }
    }
  };

  // V of the tile at t0 straight into this wave's LDS tile with direct-to-LDS 16-byte loads
  // of 1 KB each: a load fills kRpi consecutive rows of kCpr 16-byte chunks, lane l writing
  // row l / kCpr, chunk slot l % kCpr with the swizzled source chunk slot ^ (row & kVXm). Rows
  // past the end of a ragged tile are outside the buffer range and deliver zeros.
  constexpr int kCpr = S::DV / 8, kRpi = 64 / kCpr, kLoadsPerHalf = 16 / kRpi;
  const int v_row = lane / kCpr, v_slot = lane % kCpr;
  auto load_v = [&](int t0) {
    const int last = min(kTile - 1, end - 1 - t0);
    if constexpr (PM != kPagedGeneral) {
      const int64_t row0 = tile_row0(t0);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int rows = __builtin_amdgcn_readfirstlane(min(max(last + 1 - 16 * h, 0), 16));
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(vc + half_row0(t0, row0, h) * vrow_bytes + vslice), 0, rows * vrow_bytes, kRsrcWord3);
#pragma unroll
        for (int i = 0; i < kLoadsPerHalf; ++i) {
          const int r = kRpi * i + v_row;   // row within the half; the swizzle repeats per half
          const uint32_t voff = (uint32_t)r * vrow_bytes + 16 * (v_slot ^ (r & S::kVXm));
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (DA_LDS void*)(vt + (kLoadsPerHalf * h + i) * 1024), 16,
                                                   voff, 0, 0, kLoadNT);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 2 * kLoadsPerHalf; ++i) {
        const int r = kRpi * i + v_row;
        const char* vp = vc + general_row(t0 + min(r, last)) * vrow_bytes + vslice + 16 * (v_slot ^ (r & S::kVXm));
        __builtin_amdgcn_global_load_lds((const void*)vp, (DA_LDS void*)(vt + i * 1024), 16, 0, 0);
      }
    }
  };

  // phase A: S^T = K q^T for keys 0-15 and 16-31; afterwards the K registers are free.
  // With an fp8 cache and rotary columns stored apart, the rotary part of the scores is
  // summed on its own (sr): the K scales multiply the nope part only.
  auto score = [&](const KT& T, f32x4* s, f32x4* sr) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      s[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NJK; ++j) {
        // fp8 K: the 8 values of step j are dwords 2(j%2), 2(j%2)+1 of load j/2, widened
        // exactly to bf16 (every E4M3 value is a bf16 value)
        const bf16x8 kf = F8 ? fp8x8_to_bf16x8(T.k[blk][j >> 1][2 * (j & 1)], T.k[blk][j >> 1][2 * (j & 1) + 1])
                             : as_bf16x8(T.k[blk][j]);
        s[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[j], s[blk], 0, 0, 0);
      }
      if constexpr (S::NR > 0) {
        if constexpr (F8) {
          sr[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int l = 0; l < S::NR; ++l)
            sr[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(T.r[blk][l]), qf[NJK + l], sr[blk], 0, 0, 0);
        } else {
#pragma unroll
          for (int l = 0; l < S::NR; ++l)
            s[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(T.r[blk][l]), qf[NJK + l], s[blk], 0, 0, 0);
        }
      }
    }
  };

  // per-token scales of the tile's keys that this lane holds (fp8 caches): keys
  // 4qd .. 4qd+3 and 16+4qd .. 16+4qd+3, 16 contiguous bytes each in the tokens-innermost
  // scale layout (key by key with the per-key page lookup); missing keys of a ragged tile
  // read 0 (their scores are masked anyway)
  auto load_sc = [&](f32x4* ksc, f32x4* vsc, int t0, bool valid = true) {
    const int last = valid ? min(kTile - 1, end - 1 - t0) : -1;
    // scale index of the first key of the run of consecutive keys starting at t
    auto sc_base = [&](int t) -> int64_t {
      if constexpr (PM == kContiguous) {
        return ((int64_t)b * kv_heads + kvc) * a.kv_capacity + t;
      } else {
        const int slot = min(max((t >> a.page_shift) - first_page, 0), kMaxLdsPages - 1);
        const int page = __builtin_amdgcn_readfirstlane(min(max(pages_s[slot], 0), a.num_pages - 1));
        return ((int64_t)page * kv_heads + kvc) * a.page_size + (t & (a.page_size - 1));
      }
    };
    const int nk = __builtin_amdgcn_readfirstlane(max(last + 1, 0));
    const float* vs = a.v_scale ? a.v_scale : a.k_scale;
    // (the V scales are loaded in every case, from the K scales when there are none, then
    // replaced by 1 where they are used: the same loads on every path)
    if constexpr (PM == kPagedGeneral) {
      // per-key page lookup: one 4-byte load per key (keys past the end repeat the last one)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int off;
          const int page = general_page(t0 + min(16 * blk + 4 * qd + i, max(last, 0)), off);
          const int64_t idx = ((int64_t)page * kv_heads + kvc) * a.page_size + off;
          ksc[blk][i] = __builtin_nontemporal_load(a.k_scale + idx);
          vsc[blk][i] = __builtin_nontemporal_load(vs + idx);
        }
    } else if constexpr (PM == kPagedHalf) {
      // each 16-key half of the tile is a page of its own
      const int64_t base0 = sc_base(t0), base1 = sc_base(t0 + 16);
      const int n0 = min(nk, 16), n1 = max(nk - 16, 0);
      const __amdgpu_buffer_rsrc_t rk0 = __builtin_amdgcn_make_buffer_rsrc((void*)(a.k_scale + base0), 0, n0 * 4, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rk1 = __builtin_amdgcn_make_buffer_rsrc((void*)(a.k_scale + base1), 0, n1 * 4, kRsrcWord3);
      ksc[0] = __builtin_bit_cast(f32x4, buf_load16(rk0, 16 * qd, 0));
      ksc[1] = __builtin_bit_cast(f32x4, buf_load16(rk1, 16 * qd, 0));
      const __amdgpu_buffer_rsrc_t rv0 = __builtin_amdgcn_make_buffer_rsrc((void*)(vs + base0), 0, n0 * 4, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rv1 = __builtin_amdgcn_make_buffer_rsrc((void*)(vs + base1), 0, n1 * 4, kRsrcWord3);
      vsc[0] = __builtin_bit_cast(f32x4, buf_load16(rv0, 16 * qd, 0));
      vsc[1] = __builtin_bit_cast(f32x4, buf_load16(rv1, 16 * qd, 0));
    } else {
      const int64_t base = sc_base(t0);
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc((void*)(a.k_scale + base), 0, nk * 4, kRsrcWord3);
      ksc[0] = __builtin_bit_cast(f32x4, buf_load16(rk, 16 * qd, 0));
      ksc[1] = __builtin_bit_cast(f32x4, buf_load16(rk, 64 + 16 * qd, 0));
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vs + base), 0, nk * 4, kRsrcWord3);
      vsc[0] = __builtin_bit_cast(f32x4, buf_load16(rv, 16 * qd, 0));
      vsc[1] = __builtin_bit_cast(f32x4, buf_load16(rv, 64 + 16 * qd, 0));
    }
  };
  const bool has_vscale = a.v_scale != nullptr;

  // phase B: online softmax, giving P^T as the B operand of P.V. On a ragged tile the
  // scores of missing keys are set to -inf first; exp2(-inf) = 0 then removes them from
  // the sums. With fp8 caches the scores take the K scales of their keys first, and the
  // V scales multiply p in the P.V operand only (l sums the unscaled p).
  auto softmax_p = [&](f32x4* s, const f32x4* sr, int t0, bf16x8& pb_hi, bf16x8& pb_lo, const f32x4* ksc,
                       const f32x4* vsc) {
    if constexpr (F8) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        if constexpr (S::NR > 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) s[blk][i] = fmaf(s[blk][i], ksc[blk][i], sr[blk][i]);
        } else {
          s[blk] *= ksc[blk];
        }
      }
    }
    const int nvalid = col_end - t0;   // this column's keys in the tile (may be <= 0)
    if (__ballot(nvalid < kTile)) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * blk + 4 * qd + i >= nvalid) s[blk][i] = -INFINITY;
    }
    // online softmax: this lane holds keys 16*blk + 4*qd + i of column n
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = max_over_key_groups(mx);
    const float mn = fmaxf(m_run, mx);
    // (a column that has seen no key yet keeps m = -inf; its p and l stay 0)
    const float mref = mn == -INFINITY ? 0.f : mn;
    const float alpha = exp2_fast((m_run - mref) * c);
    const float mc = mref * c;
    float pr[2][4];
    float psum = 0.f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[blk][i] = exp2_fast(fmaf(s[blk][i], c, -mc));
        psum += pr[blk][i];
      }
    l_run = fmaf(l_run, alpha, psum);
    m_run = mn;
    // the running max rarely moves once a few tiles are in: skip the rescale then
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }

    // P^T as the B operand: k-slots 0-3 = keys 4qd..+3, 4-7 = keys 16+4qd..+3.
    // hi columns take bf16(p); lo columns take bf16(p - float(bf16(p))).
    uint32_t pw[4], lw[4];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const int blk = s2 >> 1, i0 = (s2 & 1) * 2;
      const float p0 = F8 ? pr[blk][i0] * (has_vscale ? vsc[blk][i0] : 1.f) : pr[blk][i0];
      const float p1 = F8 ? pr[blk][i0 + 1] * (has_vscale ? vsc[blk][i0 + 1] : 1.f) : pr[blk][i0 + 1];
      const uint32_t h = pack_bf16x2(p0, p1);
      if constexpr (HL) {
        pw[s2] = pack_bf16x2(fmaf(-lo_mask, bf16lo(h), p0), fmaf(-lo_mask, bf16hi(h), p1));
      } else {
        pw[s2] = h;
        lw[s2] = pack_bf16x2(p0 - bf16lo(h), p1 - bf16hi(h));
      }
    }
    pb_hi = as_bf16x8(u32x4{pw[0], pw[1], pw[2], pw[3]});
    if constexpr (!HL) pb_lo = as_bf16x8(u32x4{lw[0], lw[1], lw[2], lw[3]});
  };

  // phase C: O^T += V^T P^T, V^T read transposed from the LDS tile
  // (O blocks DB0 .. DB0 + NB - 1 from a bf16 tile of rows of ROW bytes whose 16-byte chunk c
  // of row r sits at slot c ^ (r & XM))
  auto pv_tile = [&](auto db0_c, auto nb_c, auto row_c, auto xm_c, const char* tile, const bf16x8& pb_hi,
                     const bf16x8& pb_lo) {
    constexpr int DB0 = decltype(db0_c)::value, NB = decltype(nb_c)::value;
    constexpr int ROW = decltype(row_c)::value, XM = decltype(xm_c)::value;
    // V^T A operand: lane (n, qd) gets depth 16db + n of keys 4qd..+3 and 16+4qd..+3
    const int r0 = 4 * qd + (n >> 2);
#pragma unroll
    for (int db = 0; db < NB; ++db) {
      const int ch = 2 * db + ((n & 3) >> 1);
      const int sub = (n & 1) * 8;
      const int ra = r0, rb = r0 + 16;
      const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (s16x4 DA_LDS*)(tile + ra * ROW + ((ch ^ (ra & XM)) << 4) + sub));
      const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (s16x4 DA_LDS*)(tile + rb * ROW + ((ch ^ (rb & XM)) << 4) + sub));
      s16x8 v8;
      v8[0] = va[0]; v8[1] = va[1]; v8[2] = va[2]; v8[3] = va[3];
      v8[4] = vb[0]; v8[5] = vb[1]; v8[6] = vb[2]; v8[7] = vb[3];
      const bf16x8 vf = __builtin_bit_cast(bf16x8, v8);
      o[DB0 + db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb_hi, o[DB0 + db], 0, 0, 0);
      if constexpr (!HL) o[DB0 + db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb_lo, o[DB0 + db], 0, 0, 0);
    }
  };
  auto pv = [&](const bf16x8& pb_hi, const bf16x8& pb_lo) {
    pv_tile(IntC<0>{}, IntC<DB>{}, IntC<S::kVRow>{}, IntC<S::kVXm>{}, vt, pb_hi, pb_lo);
  };

  // fp8 V through LDS: the tile's 32 rows of DV codes land, direct-to-LDS and
  // unswizzled, in the upper half of the wave's region; each depth half is then widened to
  // a 32 x DV/2 bf16 tile in the lower half (the swizzled layout of the transposing reads)
  // and consumed by P.V before the other half is widened. No registers hold V in flight.
  // staging tile(s) of 32 x DV codes after the half-depth bf16 tile (32 x DV bytes)
  char* const v8_stage = vt + kTile * S::DV;
  constexpr int kV8Chunks = S::DV / 16;             // 16-byte chunks per fp8 row
  constexpr int kV8Rows = 64 / kV8Chunks;           // rows per 1 KB direct-to-LDS load
  constexpr int kV8PerHalf = 16 / kV8Rows;          // loads per 16-row half tile
  constexpr int kHalfXm = S::DV / 16 - 1 < 15 ? S::DV / 16 - 1 : 15;   // swizzle of the half-depth tile
  // (the same loads through lds_dma16, for loops whose waits are all explicit)
  auto load_v8_lds_asm = [&](char* stage, int t0, bool valid) {
    const int last = valid ? min(kTile - 1, end - 1 - t0) : -1;
    // (no LDS wait is needed here: the staging tile's reads fed the widening arithmetic,
    // so they have completed before this point)
    const int rr = lane / kV8Chunks, cc = lane % kV8Chunks;
    if constexpr (PM == kPagedGeneral) {
      // per-key page lookup: each lane loads from its own row (rows past the end of a ragged
      // tile repeat the last key, finite codes that meet p = 0; past the last tile the data
      // lands in a staging tile that is never read)
#pragma unroll
      for (int i = 0; i < 2 * kV8PerHalf; ++i) {
        const int r = kV8Rows * (i % kV8PerHalf) + 16 * (i / kV8PerHalf) + rr;
        lds_dma16_ptr(vc + general_row(t0 + min(r, last)) * vrow_bytes + vslice + 16 * cc,
                      __builtin_amdgcn_readfirstlane(lds_addr(stage + i * 1024)));
      }
      return;
    }
    const int64_t row0 = tile_row0(t0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rows = __builtin_amdgcn_readfirstlane(min(max(last + 1 - 16 * h, 0), 16));
      const u32x4 rv = rsrc_words(vc + half_row0(t0, row0, h) * vrow_bytes + vslice, (uint32_t)rows * vrow_bytes);
#pragma unroll
      for (int i = 0; i < kV8PerHalf; ++i) {
        const int r = kV8Rows * i + rr;
        lds_dma16(rv, (uint32_t)r * vrow_bytes + 16 * cc,
                  __builtin_amdgcn_readfirstlane(lds_addr(stage + (kV8PerHalf * h + i) * 1024)));
      }
    }
  };
  auto load_v8_lds = [&](char* stage, int t0, bool valid = true) {
    const int last = valid ? min(kTile - 1, end - 1 - t0) : -1;
    const int rr = lane / kV8Chunks, cc = lane % kV8Chunks;
    if constexpr (PM == kPagedGeneral) {
      // per-key page lookup, as above
#pragma unroll
      for (int i = 0; i < 2 * kV8PerHalf; ++i) {
        const int r = kV8Rows * (i % kV8PerHalf) + 16 * (i / kV8PerHalf) + rr;
        __builtin_amdgcn_global_load_lds((const void*)(vc + general_row(t0 + min(r, last)) * vrow_bytes + vslice +
                                                       16 * cc),
                                         (DA_LDS void*)(stage + i * 1024), 16, 0, 0);
      }
      return;
    }
    const int64_t row0 = tile_row0(t0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rows = __builtin_amdgcn_readfirstlane(min(max(last + 1 - 16 * h, 0), 16));
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(vc + half_row0(t0, row0, h) * vrow_bytes + vslice), 0, rows * vrow_bytes, kRsrcWord3);
#pragma unroll
      for (int i = 0; i < kV8PerHalf; ++i) {
        const int r = kV8Rows * i + rr;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (DA_LDS void*)(stage + (kV8PerHalf * h + i) * 1024), 16,
                                                 (uint32_t)r * vrow_bytes + 16 * cc, 0, 0, kLoadNT);
      }
    }
  };
  auto widen_half = [&](char* work, const char* stage, int hd) {
    constexpr int kCph = S::DV / 32;                // 16-value fp8 chunks per half row
#pragma unroll
    for (int k = 0; k < 32 * kCph / 64; ++k) {
      const int u = lane + 64 * k;
      const int r = u / kCph, c8 = u % kCph;
      const u32x4 w = *(const u32x4*)(stage + r * S::DV + hd * (S::DV / 2) + 16 * c8);
      *(bf16x8*)(work + r * S::DV + (((2 * c8) ^ (r & kHalfXm)) << 4)) = fp8x8_to_bf16x8(w[0], w[1]);
      *(bf16x8*)(work + r * S::DV + (((2 * c8 + 1) ^ (r & kHalfXm)) << 4)) = fp8x8_to_bf16x8(w[2], w[3]);
    }
  };

  // Segments: the page indices of up to kMaxLdsPages pages are staged in LDS at a time
  // (one segment for every page size >= 32 with chunks up to 16K keys, >= 16 up to 8K).
  int seg_len = end - start;
  if constexpr (PM != kContiguous) {
    const int cap = ((kMaxLdsPages - 1) * a.page_size) / kTile * kTile;
    seg_len = min(seg_len, cap);
  }
  for (int s0 = start; s0 < end; s0 += seg_len) {
    const int s1 = min(s0 + seg_len, end);
    if constexpr (PM != kContiguous) {
      __syncthreads();
      first_page = s0 / a.page_size;
      const int n_pages = (s1 - 1) / a.page_size - first_page + 1;
      const int32_t* pt = a.page_table + (int64_t)b * a.pt_stride + first_page;
      for (int i = tid; i < n_pages; i += NW * 64) {
        const int page = pt[i];
        pages_s[i] = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
      }
      __syncthreads();
    }
    const int n_tiles = (s1 - s0 + kTile - 1) / kTile;
    if (wave_active && ks < n_tiles) {
      // One tile buffer: the next tile's K and V are requested as soon as the current tile
      // has been moved to LDS and into the score MFMAs, and stay in flight through the
      // softmax and P.V of the current tile.
      KT T;
      if constexpr (F8 && S::kV8Tiles == 2) {
        // fp8 at V depth 128, two tiles in flight (a tile is half the bytes of bf16, so one
        // tile per wave leaves too few bytes in flight to cover the memory latency). Tiles
        // alternate between (T, ksc0, vsc0, stage 0) and (T1, ksc1, vsc1, stage 1); the
        // loads of tile j are issued in the order K, scales, V, two tiles ahead: K after
        // the scores of tile j - 2, the scales after its softmax, V after its staged codes
        // were consumed. At the wait for tile j's V, the loads issued after it are those of
        // tile j + 1 and the K and scales of tile j + 2.
        // (scales: four 16-byte loads per tile, or 16 single ones with the per-key page lookup)
        constexpr int kK = 2 * (KT::NL + S::NR), kSc = PM == kPagedGeneral ? 16 : 4, kV = 2 * kV8PerHalf;
        KT T1;
        f32x4 ksc0[2], vsc0[2], ksc1[2], vsc1[2];
        // the wave's region: the half-depth bf16 tile, then the two staging tiles (their
        // loads are issued as inline assembly: the compiler adds no waits for them, and the
        // explicit wait below is the only one)
        char* const work = vt;
        char* const stage0 = vt + kTile * S::DV;
        char* const stage1 = vt + 2 * kTile * S::DV;
        auto issue = [&](KT& TT, f32x4* ksc, f32x4* vsc, char* stage, int t0, bool valid) {
          load_k(TT, t0, valid);
          load_sc(ksc, vsc, t0, valid);
          load_v8_lds_asm(stage, t0, valid);
        };
        // Every step issues the same loads (those past the last tile with an empty range), so
        // that a single count holds at the wait and the compiler sees one straight path.
        auto step = [&](KT& TT, f32x4* ksc, f32x4* vsc, char* stage, int it) {
          const bool has2 = it + 2 * KS < n_tiles;
          const int t2 = s0 + (it + 2 * KS) * kTile;
          f32x4 s[2], sr[2];
          score(TT, s, sr);
          load_k(TT, t2, has2);
          bf16x8 pb_hi, pb_lo;
          softmax_p(s, sr, s0 + it * kTile, pb_hi, pb_lo, ksc, vsc);
          load_sc(ksc, vsc, t2, has2);
          wait_vm<2 * kK + 2 * kSc + kV>();
          widen_half(work, stage, 0);
          pv_tile(IntC<0>{}, IntC<DB / 2>{}, IntC<S::DV>{}, IntC<kHalfXm>{}, work, pb_hi, pb_lo);
          widen_half(work, stage, 1);
          pv_tile(IntC<DB / 2>{}, IntC<DB / 2>{}, IntC<S::DV>{}, IntC<kHalfXm>{}, work, pb_hi, pb_lo);
          // this stage has been read: tile j + 2 may land there
          load_v8_lds_asm(stage, t2, has2);
        };
        // (earlier LDS writes of this wave to the staging tiles, e.g. the zero fill, are
        // complete before the first loads land there)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        issue(T, ksc0, vsc0, stage0, s0 + ks * kTile, true);
        issue(T1, ksc1, vsc1, stage1, s0 + (ks + KS) * kTile, ks + KS < n_tiles);
        // (pairs of tiles with no branch inside, so that the compiler's own waits for the K
        // registers see the same loads in flight on every path; an odd last tile after)
        int it = ks;
        for (; it + KS < n_tiles; it += 2 * KS) {
          step(T, ksc0, vsc0, stage0, it);
          step(T1, ksc1, vsc1, stage1, it + KS);
        }
        if (it < n_tiles) step(T, ksc0, vsc0, stage0, it);
        wait_vm<0>();   // the empty-range loads past the last tile have retired
      } else if constexpr (F8) {
        // fp8 (wide V): K and the scales of the next tile in flight in registers, its V
        // codes in LDS. (V widened in registers and then written to LDS needed more
        // registers than two waves per SIMD have at V depth 256.)
        constexpr int kKLoads = 2 * (KT::NL + S::NR);
        f32x4 ksc[2], vsc[2];
        load_k(T, s0 + ks * kTile);
        load_v8_lds(v8_stage, s0 + ks * kTile);
        load_sc(ksc, vsc, s0 + ks * kTile);
        for (int it = ks; it < n_tiles; it += KS) {
          const bool has_next = it + KS < n_tiles;
          const int tn = s0 + (it + KS) * kTile;
          f32x4 s[2], sr[2];
          score(T, s, sr);
          if (has_next) load_k(T, tn);
          bf16x8 pb_hi, pb_lo;
          softmax_p(s, sr, s0 + it * kTile, pb_hi, pb_lo, ksc, vsc);
          // this tile's V codes are in LDS: they were requested before the next tile's K
          if (has_next) wait_vm<kKLoads>();
          else wait_vm<0>();
          widen_half(vt, v8_stage, 0);
          pv_tile(IntC<0>{}, IntC<DB / 2>{}, IntC<S::DV>{}, IntC<kHalfXm>{}, vt, pb_hi, pb_lo);
          widen_half(vt, v8_stage, 1);
          // the staging area has been read: the next tile's V may land there
          if (has_next) {
            load_v8_lds(v8_stage, tn);
            load_sc(ksc, vsc, tn);
          }
          pv_tile(IntC<DB / 2>{}, IntC<DB / 2>{}, IntC<S::DV>{}, IntC<kHalfXm>{}, vt, pb_hi, pb_lo);
        }
      } else if constexpr (S::kKLds && PM != kPagedGeneral) {
        // K through LDS as well: both tiles arrive by direct-to-LDS loads of 4 rows x 256
        // bytes per instruction (16 rows x 64 bytes, the register layout of the A operand,
        // streams markedly slower), issued as inline assembly with explicit waits. The K tile
        // sits after the V tile in the wave's region, rows swizzled like V.
        char* const kt = vt + S::kVBytes;
        constexpr int kKD = 2 * kLoadsPerHalf, kVD = 2 * kLoadsPerHalf;   // loads per tile
        auto load_tile_asm = [&](char* dst, const char* cache, uint32_t row_bytes, uint32_t slice, int t0) {
          const int last = min(kTile - 1, end - 1 - t0);
          const int64_t row0 = tile_row0(t0);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int rows = __builtin_amdgcn_readfirstlane(min(max(last + 1 - 16 * h, 0), 16));
            const u32x4 rs = rsrc_words(cache + half_row0(t0, row0, h) * row_bytes + slice, (uint32_t)rows * row_bytes);
#pragma unroll
            for (int i = 0; i < kLoadsPerHalf; ++i) {
              const int r = kRpi * i + v_row;
              lds_dma16(rs, (uint32_t)r * row_bytes + 16 * (v_slot ^ (r & S::kVXm)),
                        __builtin_amdgcn_readfirstlane(lds_addr(dst + (kLoadsPerHalf * h + i) * 1024)));
            }
          }
        };
        // S^T = K q^T with the K rows read from the LDS tile (chunk 4j + qd of row n + 16 blk)
        auto score_lds = [&](f32x4* s) {
#pragma unroll
          for (int blk = 0; blk < 2; ++blk) {
            s[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int r = n + 16 * blk;
#pragma unroll
            for (int j = 0; j < NJK; ++j) {
              const bf16x8 kf =
                  as_bf16x8(*(const u32x4*)(kt + r * S::kVRow + (((4 * j + qd) ^ (r & S::kVXm)) << 4)));
              s[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[j], s[blk], 0, 0, 0);
            }
          }
        };
        auto lds_quiet = [&] {   // this wave's LDS reads are complete (before a tile is refilled)
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          __builtin_amdgcn_s_waitcnt(0xC07F);
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
        };
        lds_quiet();
        load_tile_asm(kt, kc, krow_bytes, kslice, s0 + ks * kTile);
        load_tile_asm(vt, vc, vrow_bytes, vslice, s0 + ks * kTile);
        for (int it = ks; it < n_tiles; it += KS) {
          const bool has_next = it + KS < n_tiles;
          const int tn = s0 + (it + KS) * kTile;
          // this tile's K has landed (its V, requested after it, may still be in flight)
          wait_vm<kVD>();
          f32x4 s[2];
          score_lds(s);
          if (has_next) {
            lds_quiet();
            load_tile_asm(kt, kc, krow_bytes, kslice, tn);
          }
          bf16x8 pb_hi, pb_lo;
          softmax_p(s, nullptr, s0 + it * kTile, pb_hi, pb_lo, nullptr, nullptr);
          // this tile's V has landed (the next tile's K may stay in flight)
          if (has_next) wait_vm<kKD>();
          else wait_vm<0>();
          pv(pb_hi, pb_lo);
          if (has_next) {
            lds_quiet();
            load_tile_asm(vt, vc, vrow_bytes, vslice, tn);
          }
        }
        wait_vm<0>();
      } else {
        // loads issued per tile: K (and rotary) first, then V; V of the current tile must
        // be in LDS before P.V while the next tile's K loads may stay in flight
        constexpr int kKLoads = 2 * (KT::NL + S::NR);
        load_k(T, s0 + ks * kTile);
        load_v(s0 + ks * kTile);
        for (int it = ks; it < n_tiles; it += KS) {
          const bool has_next = it + KS < n_tiles;
          f32x4 s[2], sr[2];
          score(T, s, sr);
          if (has_next) load_k(T, s0 + (it + KS) * kTile);
          bf16x8 pb_hi, pb_lo;
          softmax_p(s, sr, s0 + it * kTile, pb_hi, pb_lo, nullptr, nullptr);
          // V of this tile must have landed in LDS: it was requested before the K loads
          // of the next tile, which may stay in flight
          if (has_next) wait_vm<kKLoads>();
          else wait_vm<0>();
          pv(pb_hi, pb_lo);
          // the transposing reads of this tile are complete (their data fed the MFMAs):
          // the LDS tile can take the next V
          if (has_next) load_v(s0 + (it + KS) * kTile);
        }
      }
    }
  }

  // this wave's totals: sum l over the four key groups; fold the lo columns into hi
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if constexpr (HL) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[db][i] += __shfl_xor(o[db][i], 8);
  }

  OwnPartial own;   // (KS == 1 stores in the MFMA layout, not the fold's: nothing kept)
  if (KS == 1) {
    // one wave per kv head: store straight from registers
    if (wave_active && col_valid && !is_lo) {
      const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
      const int row = wv.qi * a.Hq1 + kvh * g + wv.hh;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        store_unit(a, b, row, p, direct, 16 * db + 4 * qd, o[db] * inv, m_run, l_run, db == 0 && qd == 0);
    }
  } else {
    own = merge_key_splits<HL, S>(a, wv, smem, b, p, direct, o, m_run, l_run);
  }
  if (a.counters && !direct) fused_combine<S>(a, wv, smem, flag_s, b, count, first_slot, own);
}

// A piece of work as wave 0 of a workgroup publishes it to the other waves.
struct Piece {
  int b, start, end, slot;
  int first_slot, count;   // the sequence's first slot and number of partitions
};
struct PieceTable {
  Piece row[64];      // indexed by lane = sequence within the current chunk of 64
  uint32_t mask_lo, mask_hi;
  int done;
  // scan state, kept here rather than in registers across the pieces (wave 0 only)
  int c0, slot_base;
  int64_t U, Wact, ts, te, tile_base;
};

template <bool HL, int PM, bool F8, class S>
// one 8-wave workgroup per CU (two waves per SIMD): the tile loop needs about 160 VGPRs,
// and eight waves per CU already keep the memory system busy under the equal-share schedule
__global__ __launch_bounds__(kMaxWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void partition_gqa_kernel(PartArgs a, int HG, int KS) {
  extern __shared__ __attribute__((aligned(16))) char smem[];   // NW * S::kWaveBytes (launch size)

  __shared__ int pages_s[kMaxLdsPages];
  __shared__ PieceTable table;
  __shared__ int fuse_flag;
  // everything a workgroup of kMaxWaves waves holds must fit the compute unit's LDS
  static_assert(kMaxWaves * S::kWaveBytes + sizeof(pages_s) + sizeof(PieceTable) + sizeof(int) <= kLdsBytes,
                "LDS budget");
  WaveInfo wv;
  wv.HG = HG;
  wv.KS = KS;
  wv.NW = HG * KS;
  wv.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index, uniform
  wv.ks = wv.w / HG;
  wv.kvh = grp_of(a, HG) * HG + wv.w % HG;
  wv.wave_active = wv.kvh < a.Hkv;
  wv.lane = threadIdx.x & 63;
  wv.n = wv.lane & 15;
  wv.qd = wv.lane >> 4;
  wv.hc = HL ? (wv.n & 7) : wv.n;          // (query, head) column of this lane
  wv.col_valid = wv.hc < a.q_len * a.g;
  wv.qi = wv.col_valid ? wv.hc / a.g : 0;
  wv.hh = wv.col_valid ? wv.hc % a.g : 0;
  wv.is_lo = HL && wv.n >= 8;
  const int lane = wv.lane;

  if (a.workers == 0) {
    // fixed chunks: partition fixed_part_of() of sequence fixed_seq_of() (sequence length
    // loaded by a vector load: state that it is uniform)
    const int L = __builtin_amdgcn_readfirstlane(attended_len(a, fixed_seq_of(), PM == kContiguous));
    // (with the fused combine there is no combine launch to write the rows of an empty
    // sequence: its first workgroup writes them, as a piece without keys)
    const bool empty_rows = L == 0 && fixed_part_of(a, HG) == 0 && a.counters && a.direct_single;
    if (fixed_part_of(a, HG) * a.chunk >= L && !empty_rows) return;
  }
  zero_v_tile<S>(smem + wv.w * S::kWaveBytes, lane);


  // Equal shares: worker wid = blockIdx.x takes tiles [ts, te) of the U 32-key tiles of
  // all sequences concatenated in batch order (at least kMinShareTiles per worker, so
  // fewer workers than launched may be active). Each sequence the share meets is one
  // piece, stored in slot (first slot of the sequence) + (wid - first worker of the
  // sequence). Wave 0 scans seq_lens 64 sequences at a time and publishes the pieces of
  // each chunk in LDS; every wave then runs them in order.
  const int wid = blockIdx.x;
  uint64_t pending = 0;
  bool fixed_taken = false;
  if (a.workers > 0 && wv.w == 0) {
    int64_t U = 0;
    for (int c = 0; c < a.B; c += 64) {
      const int bb = c + lane;
      const int64_t nt = bb < a.B ? (attended_len(a, bb, PM == kContiguous) + kTile - 1) / kTile : 0;
      U += wave_sum_i64(nt);
    }
    U = lane_value(U, 0);
    int64_t Wact = U / kMinShareTiles;
    Wact = Wact < 1 ? 1 : (Wact > a.workers ? a.workers : Wact);
    if (lane == 0) {
      table.U = U;
      table.Wact = Wact;
      table.ts = (int64_t)wid * U / Wact;
      table.te = (int64_t)(wid + 1) * U / Wact;
      table.tile_base = 0;   // tiles of the sequences before the current chunk
      table.slot_base = 0;   // slots of the sequences before the current chunk
      table.c0 = -64;
    }
  }

  for (;;) {
    int b, start, end, p, count, first_slot;
    if (a.workers == 0) {
      if (fixed_taken) break;
      fixed_taken = true;
      b = fixed_seq_of();
      p = fixed_part_of(a, HG);
      const int L = __builtin_amdgcn_readfirstlane(attended_len(a, b, PM == kContiguous));
      start = p * a.chunk;
      end = min(start + a.chunk, L);
      count = min((L + a.chunk - 1) / a.chunk, a.max_splits);
      if (L == 0) count = 1;   // the empty rows of the fused combine: finished in place
      first_slot = -1;
    } else {
      while (pending == 0) {
        __syncthreads();   // every wave is done with the previous table
        if (wv.w == 0) {
          const int64_t U = table.U, Wact = table.Wact, ts = table.ts, te = table.te;
          int64_t tile_base = table.tile_base;
          int slot_base = table.slot_base;
          const int c0 = table.c0 + 64;
          // past the end of this share nothing is left, except for the last worker, which
          // also writes the (first slot, count) of empty sequences at the very end
          const bool done = wid >= Wact || c0 >= a.B || (tile_base >= te && wid != Wact - 1);
          uint64_t mask = 0;
          if (!done) {
            const int bb = c0 + lane;
            const int len = bb < a.B ? attended_len(a, bb, PM == kContiguous) : 0;
            const int64_t nt = (len + kTile - 1) / kTile;
            const int64_t incl = wave_incl_scan(nt);
            const int64_t pre = tile_base + incl - nt;   // first tile of sequence bb
            int64_t first = 0;                           // worker holding that tile
            int count = 0;                               // partitions of sequence bb
            if (nt > 0) {
              first = share_owner(pre, U, Wact);
              count = (int)(share_owner(pre + nt - 1, U, Wact) - first + 1);
            }
            const int sincl = wave_incl_scan(count);
            const int slot = slot_base + sincl - count;
            // (first slot, count) of each sequence for the combine, written by exactly one
            // worker: the one whose share holds the sequence's first tile (the last one
            // for trailing empty sequences)
            const int64_t writer = pre < U ? share_owner(pre, U, Wact) : Wact - 1;
            if (grp_of(a, HG) == 0 && bb < a.B && writer == wid) {
              a.meta[2 * bb] = slot;
              a.meta[2 * bb + 1] = count;
            }
            // With the fused combine no combine launch writes the rows of an empty sequence:
            // the same worker takes them as a piece without keys, finished in place.
            const bool empty_rows = bb < a.B && nt == 0 && writer == wid && a.counters && a.direct_single;
            const bool mine = (bb < a.B && nt > 0 && pre < te && pre + nt > ts) || empty_rows;
            mask = __ballot(mine);
            if (mine) {
              Piece pc;
              pc.b = bb;
              if (nt == 0) {
                pc.start = pc.end = 0;
                pc.slot = slot;
                pc.first_slot = slot;
                pc.count = 1;
              } else {
                const int64_t lo = (ts > pre ? ts : pre) - pre;
                const int64_t hi = (te < pre + nt ? te : pre + nt) - pre;
                pc.start = (int)lo * kTile;
                pc.end = min((int)hi * kTile, len);
                pc.slot = slot + (int)(wid - first);
                pc.first_slot = slot;
                pc.count = count;
              }
              table.row[lane] = pc;
            }
            tile_base += lane_value(incl, 63);
            slot_base += lane_value(sincl, 63);
          }
          if (lane == 0) {
            table.mask_lo = (uint32_t)mask;
            table.mask_hi = (uint32_t)(mask >> 32);
            table.done = done ? 1 : 0;
            table.c0 = c0;
            table.tile_base = tile_base;
            table.slot_base = slot_base;
          }
        }
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(table.done)) break;
        pending = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)table.mask_hi) << 32) |
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)table.mask_lo);
      }
      if (pending == 0) break;
      const int j = __builtin_ctzll(pending);
      pending &= pending - 1;
      b = __builtin_amdgcn_readfirstlane(table.row[j].b);
      start = __builtin_amdgcn_readfirstlane(table.row[j].start);
      end = __builtin_amdgcn_readfirstlane(table.row[j].end);
      p = __builtin_amdgcn_readfirstlane(table.row[j].slot);
      first_slot = __builtin_amdgcn_readfirstlane(table.row[j].first_slot);
      count = __builtin_amdgcn_readfirstlane(table.row[j].count);
    }
    run_piece<HL, PM, F8, S>(a, wv, smem, pages_s, &fuse_flag, b, start, end, p, count, first_slot);
  }
}

template <bool HL, class S>
hipError_t launch_hl(const PartArgs& a, int pm, int HG, int KS, hipStream_t s) {
  const unsigned groups = (unsigned)((a.Hkv + HG - 1) / HG);
  if (a.workers == 0 && (int64_t)a.max_splits * groups > INT32_MAX) return hipErrorInvalidConfiguration;
  const dim3 grid = a.workers > 0 ? dim3((unsigned)a.workers, groups) : dim3((unsigned)a.max_splits * groups, (unsigned)a.B);
  const dim3 block(HG * KS * 64);
  const size_t lds = (size_t)HG * KS * S::kWaveBytes;
  if (a.kv_fp8) {
    // fp8 caches
    switch (pm) {
      case kContiguous:
        hipLaunchKernelGGL((partition_gqa_kernel<HL, kContiguous, true, S>), grid, block, lds, s, a, HG, KS);
        break;
      case kPagedAligned:
        hipLaunchKernelGGL((partition_gqa_kernel<HL, kPagedAligned, true, S>), grid, block, lds, s, a, HG, KS);
        break;
      case kPagedHalf:
        hipLaunchKernelGGL((partition_gqa_kernel<HL, kPagedHalf, true, S>), grid, block, lds, s, a, HG, KS);
        break;
      default:
        hipLaunchKernelGGL((partition_gqa_kernel<HL, kPagedGeneral, true, S>), grid, block, lds, s, a, HG, KS);
        break;
    }
    return hipGetLastError();
  }
  switch (pm) {
    case kContiguous:
      hipLaunchKernelGGL((partition_gqa_kernel<HL, kContiguous, false, S>), grid, block, lds, s, a, HG, KS);
      break;
    case kPagedAligned:
      hipLaunchKernelGGL((partition_gqa_kernel<HL, kPagedAligned, false, S>), grid, block, lds, s, a, HG, KS);
      break;
    case kPagedHalf:
      hipLaunchKernelGGL((partition_gqa_kernel<HL, kPagedHalf, false, S>), grid, block, lds, s, a, HG, KS);
      break;
    default:
      // per-key page lookup (any page size)
      hipLaunchKernelGGL((partition_gqa_kernel<HL, kPagedGeneral, false, S>), grid, block, lds, s, a, HG, KS);
      break;
  }
  return hipGetLastError();
}

// Launch of one depth shape: HG kv heads per workgroup, KS key splits per kv head
// (HG * KS <= 8). Instantiated by the translation unit that owns the shape.
template <class S>
hipError_t launch_shape(const PartArgs& a, int page_mode, int HG, int KS, hipStream_t s) {
  if (HG < 1 || KS < 1 || HG * KS > kMaxWaves) return hipErrorInvalidValue;
  return a.q_len * a.g <= 8 ? launch_hl<true, S>(a, page_mode, HG, KS, s) : launch_hl<false, S>(a, page_mode, HG, KS, s);
}

typedef MShape<64, 64, 0> Shape64;
typedef MShape<128, 128, 0> Shape128;
typedef MShape<192, 128, 0> Shape192;        // nope 128 + 64 rotary, V 128 (nope == V)
typedef MShape<192, 128, 64> Shape192R;      //   ... rotary columns stored apart
typedef MShape<256, 256, 0> Shape256;        // nope 192 + 64 rotary, V 256 (nope != V)
typedef MShape<256, 256, 64> Shape256R;      //   ... rotary columns stored apart

}  // namespace mfma
}  // namespace da
