// Device-side helpers shared by the partition and combine kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "da_internal.h"

namespace da {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define DA_LDS __attribute__((address_space(3)))

template <int V>
struct IntK {
  static constexpr int value = V;
};

// Buffer-resource dword 3 for raw (untyped) dword loads on gfx9-family parts.
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy of the K/V loads: non-temporal (each byte is read once per step).
constexpr int kLoadNT = 2;

// Wait until at most N vector-memory operations of this wave are outstanding
// (s_waitcnt vmcnt(N), other counters untouched; gfx9 encoding: vmcnt bits 3:0 and 15:14,
// expcnt 6:4 and lgkmcnt 11:8 at their no-wait maxima). The compiler fences keep the LDS
// reads that depend on a direct-to-LDS load after the wait.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Buffer resource of `bytes` bytes at `base` (raw, stride 0), as four scalar words.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t addr = (uint64_t)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)addr);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = kRsrcWord3;
  return r;
}

// Direct-to-LDS 16-byte buffer load (the 64 lanes fill 1 KB at LDS address lds_base, lane
// l at 16 l; a lane outside the buffer range reads nothing and writes zeros there, as an
// out-of-range buffer load returns zeros), non-temporal, written as
// inline assembly: the compiler does not see an LDS write, so it adds no wait of its own
// before later LDS reads (it would wait for the most recent such load, whatever it
// fills). Every consumer waits explicitly (wait_vm). M0, which holds the LDS base of the
// instruction, is saved and restored around it.
__device__ __forceinline__ void lds_dma16(u32x4 rsrc, uint32_t voff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen nt lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(lds_base)
      : "memory");
}

// The same from a per-lane 64-bit address (global_load_lds_dwordx4: lane l fills 16 bytes
// at lds_base + 16 l), for rows found key by key.
__device__ __forceinline__ void lds_dma16_ptr(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_base)
      : "memory");
}

// The buffer form with 4 bytes per lane (the 64 lanes fill 256 bytes, lane l at 4 l).
__device__ __forceinline__ void lds_dma4(u32x4 rsrc, uint32_t voff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen nt lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(lds_base)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const DA_LDS char*)p;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16 bits, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Four E4M3 codes (one dword, byte 0 first) as two packed bf16 pairs, through the gfx950
// scaled conversion with scale 1 (one instruction per pair; OCP E4M3, exact, since every
// E4M3 value is a bf16 value; checked on all 256 codes on the GPU).
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
  u32x2 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  return r;
}

__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  const u32x2 a = fp8x4_to_bf16x4(w0), b = fp8x4_to_bf16x4(w1);
  return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Sequence length actually attended: negative -> 0, clamped to the grid's bound and,
// for a contiguous cache, to its capacity.
__device__ __forceinline__ int attended_len(const PartArgs& a, int b, bool contiguous) {
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : L;
  L = L > a.max_seq_len ? a.max_seq_len : L;
  if (contiguous && L > a.kv_capacity) L = a.kv_capacity;
  return L;
}

// Cache row (token slot) of key t of sequence b.
template <int PM>
__device__ __forceinline__ int64_t key_row(const PartArgs& a, int b, int t) {
  if (PM == kContiguous) return (int64_t)b * a.kv_capacity + t;
  const int pi = t / a.page_size;
  int page = a.page_table[(int64_t)b * a.pt_stride + pi];
  page = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
  return (int64_t)page * a.page_size + (t - pi * a.page_size);
}

__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}

// Value of lane j (j uniform) as a wave-uniform value.
__device__ __forceinline__ int lane_value(int v, int j) { return __builtin_amdgcn_readlane(v, j); }
__device__ __forceinline__ int64_t lane_value(int64_t v, int j) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, j);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), j);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Equal-share schedule. The 32-key tiles of all sequences, concatenated in batch order,
// number U; worker w of W takes tiles [floor(w U / W), floor((w + 1) U / W)). This is
// the worker whose share holds tile t (0 <= t < U, 1 <= W <= U).
__device__ __forceinline__ int64_t share_owner(int64_t t, int64_t U, int64_t W) {
  return ((t + 1) * W + U - 1) / U - 1;
}

// Device-coherent accesses for the fused combine's partials: 16- and 8-byte buffer accesses
// with cache policy SC1 (the code this chip's agent-scope atomics use): a store is written
// through the XCD's L2 and counts as complete once every XCD can see it; a load is served
// coherently, never from a stale line of the reading XCD's L2. Offsets are bytes from the
// start of the partial array (the fused path is used while the arrays stay below 4 GB).
constexpr int kCpolSC1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t whole_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, kRsrcWord3);
}
// Folds partials j = j0, j0 + step, ... (< P) of one (row, 4-wide depth slice) unit into a
// running (M, Ls, acc) with the combine's weights l_j exp2((m_j - M) c); when a batch
// raises the running max, what was summed so far is rescaled (fa4_splitk_combine_write,
// first paragraph). ml / po point at partial 0 of the row; partials are `stride` partial
// rows apart; loads are issued kBatch at a time. Partials with l_j == 0 weigh nothing.
// DEV: the partials were published by device-coherent stores, and ml_base / po_base are the
// starts of their arrays.
// The calling thread's own partial, when it is one of them, can stay in registers
// (fa4_splitk_combine_write, second paragraph: the writer's own band is not read back):
// partial `own` is then taken as (own_ml, own_o) instead of being loaded, in its place in the
// order, so that the result does not depend on which workgroup folds.
struct OwnPartial {
  int idx = -1;   // index of the partial among the row's P, -1: none
  float2 ml;
  f32x4 o;
};
template <int DV, int kBatch = 8, bool DEV = false>
__device__ __forceinline__ void fold_partials(const float2* ml, const float* po, int64_t stride, int P, int j0,
                                              int step, float c, float& M, float& Ls, f32x4& acc,
                                              const float* ml_base = nullptr, const float* po_base = nullptr,
                                              const OwnPartial& own = OwnPartial()) {
  __amdgpu_buffer_rsrc_t rml, ro;
  if constexpr (DEV) rml = whole_rsrc(ml_base), ro = whole_rsrc(po_base);
  for (int p0 = j0; p0 < P; p0 += step * kBatch) {
    float2 v[kBatch];
    f32x4 o[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int p = p0 + i * step;
      const bool in = p < P;
      if (p == own.idx) {
        v[i] = own.ml;
        o[i] = own.o;
      } else if constexpr (DEV) {
        // (partials published by the fused combine's device-coherent stores)
        const uint32_t mo = (uint32_t)((const char*)(ml + p * stride) - (const char*)ml_base);
        const uint32_t oo = (uint32_t)((const char*)(po + p * stride * DV) - (const char*)po_base);
        v[i] = in ? __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rml, mo, 0, kCpolSC1))
                  : make_float2(-INFINITY, 0.f);
        o[i] = in ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, oo, 0, kCpolSC1))
                  : f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
        v[i] = in ? ml[p * stride] : make_float2(-INFINITY, 0.f);
        o[i] = in ? *(const f32x4*)(po + p * stride * DV) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    float mb = M;
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (v[i].y > 0.f) mb = fmaxf(mb, v[i].x);
    if (mb > M) {
      const float r = Ls > 0.f ? exp2_fast((M - mb) * c) : 0.f;
      Ls *= r;
      acc *= r;
      M = mb;
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (v[i].y > 0.f) {
        const float e = v[i].y * exp2_fast((v[i].x - M) * c);
        Ls += e;
        acc += e * o[i];
      }
    }
  }
}

// Final outputs of one (row, 4-wide slice) unit from its merged (M, Ls, acc): O = acc / Ls
// as bf16 (round to nearest even) and optionally fp32, LSE = scale M + ln Ls (written by
// the slice at depth 0). A row without keys gets O = 0 and LSE = -inf.
__device__ __forceinline__ void write_row_unit(uint16_t* out, float* o32, float* lse, int64_t row, int Dv, int d0,
                                               float M, float Ls, f32x4 acc, float scale) {
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  float l = -INFINITY;
  if (Ls > 0.f) {
    o = acc * (1.f / Ls);
    l = scale * M + logf(Ls);
  }
  u32x2 pk;
  pk[0] = pack_bf16x2(o[0], o[1]);
  pk[1] = pack_bf16x2(o[2], o[3]);
  *(u32x2*)(out + row * Dv + d0) = pk;
  if (o32) *(f32x4*)(o32 + row * Dv + d0) = o;
  if (lse && d0 == 0) lse[row] = l;
}

// Store one float4 of a finished (head, depth) unit: either the final outputs of a
// single-partition row or the normalised partial of partition p.
__device__ __forceinline__ void store_unit(const PartArgs& a, int b, int hq, int p, bool direct,
                                           int d0, f32x4 o, float M, float Lsum, bool write_ml) {
  const int64_t row = (int64_t)b * a.Hq + hq;
  if (direct) {
    u32x2 pk;
    pk[0] = pack_bf16x2(o[0], o[1]);
    pk[1] = pack_bf16x2(o[2], o[3]);
    *(u32x2*)(a.out + row * a.Dv + d0) = pk;
    if (a.o32) *(f32x4*)(a.o32 + row * a.Dv + d0) = o;
    if (write_ml && a.lse) a.lse[row] = a.scale * M + logf(Lsum);
  } else {
    // fixed chunks: p is the partition of sequence b; equal shares: p is the slot
    const int64_t pr = a.workers ? (int64_t)p * a.Hq + hq : row * a.max_splits + p;
    if (a.counters) {
      // fused combine: the partial is read by whichever workgroup completes the count
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), whole_rsrc(a.part_o),
                                             (uint32_t)((pr * a.Dv + d0) * 4), 0, kCpolSC1);
      if (write_ml)
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, make_float2(M, Lsum)), whole_rsrc(a.part_ml),
                                              (uint32_t)(pr * 8), 0, kCpolSC1);
      return;
    }
    *(f32x4*)(a.part_o + pr * a.Dv + d0) = o;
    if (write_ml) {
      float2 ml;
      ml.x = M;
      ml.y = Lsum;
      *(float2*)(a.part_ml + pr * 2) = ml;
    }
  }
}

// LDS a block of the combine needs to merge its S thread subsets (none for S = 1).
template <int DV, int S, int NT>
struct CombineLds {
  static constexpr int kUnits = NT / S;
  static constexpr int kBytes = S > 1 ? S * kUnits * (2 * 4 + 16) : 16;
};

// One block of the LSE combine (fa4_splitk_combine_write, first paragraph): NT threads own
// (row, 4-wide depth slice) units, S threads per unit; block `blk` covers rows
// blk * RPB .. +RPB-1. Thread subset s takes partitions s, s + S, ... of its row and keeps a
// running (max, sum, O) for them (the same exp2 weights, rescaled when the running max
// grows); the S results are merged through `lds` (CombineLds bytes) with the combine
// formula. With S = 1 this is the plain per-thread combine; S > 1 shortens the dependent
// load chain of rows with many partitions by a factor S. Every thread of the block calls it
// (it holds a barrier when S > 1).
// BANDS > 1 (rows with many partitions, few rows): block blk takes depth band blk % BANDS of
// row blk / BANDS, so that the row's partials are read by BANDS compute units.
template <int DV, int S, int NT, int BANDS = 1>
__device__ __forceinline__ void combine_rows(const CombineArgs& a, int64_t blk, int tid, char* lds) {
  constexpr int TPR = DV / 4 / BANDS;               // threads (units) per row in a block
  constexpr int UNITS = NT / S;                     // units per block
  constexpr int RPB = UNITS / TPR;                  // rows per block
  static_assert(RPB >= 1 && UNITS % TPR == 0 && (BANDS == 1 || RPB == 1), "block shape");
  float* sM = (float*)lds;                          // [S][UNITS]
  float* sL = sM + S * UNITS;                       // [S][UNITS]
  f32x4* sO = (f32x4*)(sL + S * UNITS);             // [S][UNITS]

  const int sub = tid / UNITS, u = tid % UNITS;
  const int r_in = u / TPR, ch = (int)(blk % BANDS) * TPR + u % TPR;
  const int64_t row = (blk / BANDS) * RPB + r_in;
  const bool row_ok = row < (int64_t)a.B * a.Hq;
  const int b = row_ok ? (int)(row / a.Hq) : 0;
  // partials of this row: P_b of them, `stride` partial rows apart, from partial row `first`
  int P_b = 0;
  int64_t first = 0, stride = 1;
  if (row_ok) {
    if (a.meta) {
      // equal-share schedule: slots first .. first + P_b - 1 hold all heads of sequence b
      // (clamped to the slots that exist, so a stale table cannot send loads astray)
      const int s0 = min(max(a.meta[2 * b], 0), a.slots - 1);
      P_b = min(max(a.meta[2 * b + 1], 0), a.slots - s0);
      first = (int64_t)s0 * a.Hq + (row - (int64_t)b * a.Hq);
      stride = a.Hq;
    } else {
      int L = a.seq_lens[b];
      L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
      if (a.kv_cap_clamp > 0 && L > a.kv_cap_clamp) L = a.kv_cap_clamp;
      P_b = min((L + a.chunk - 1) / a.chunk, a.max_splits);
      first = row * a.max_splits;
    }
  }
  // rows that pass 1 finished itself (single partition) are left alone; their threads
  // still take part in the barrier below
  const bool active = row_ok && !(a.skip_single && P_b == 1);

  const float2* ml = (const float2*)a.part_ml + first;
  const float* po = a.part_o + first * DV + ch * 4;
  float M = -INFINITY, Ls = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (active) fold_partials<DV>(ml, po, stride, P_b, sub, S, a.c, M, Ls, acc);
  if constexpr (S > 1) {
    sM[sub * UNITS + u] = M;
    sL[sub * UNITS + u] = Ls;
    sO[sub * UNITS + u] = acc;
    __syncthreads();
    if (sub == 0) {
      float G = -INFINITY;
#pragma unroll
      for (int t = 0; t < S; ++t)
        if (sL[t * UNITS + u] > 0.f) G = fmaxf(G, sM[t * UNITS + u]);
      Ls = 0.f;
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < S; ++t) {
        if (sL[t * UNITS + u] > 0.f) {
          const float e = exp2_fast((sM[t * UNITS + u] - G) * a.c);
          Ls += sL[t * UNITS + u] * e;
          acc += e * sO[t * UNITS + u];
        }
      }
      M = G;
    }
  }
  if (active && sub == 0) write_row_unit(a.out, a.o32, a.lse, row, DV, ch * 4, M, Ls, acc, a.scale);
}

}  // namespace da
