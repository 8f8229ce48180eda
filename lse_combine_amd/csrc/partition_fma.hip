// Split-K pass 1 on the vector ALU: one workgroup per (kv head, partition, sequence).
//
// Used for fp32 caches (and for bf16 when asked for explicitly), where q.K and P.V do not
// run on the matrix cores. Four waves split the partition's keys in 64-key tiles (tile i
// goes to wave i % 4). Within a tile:
//   K        coalesced 16-byte direct-to-LDS loads (consecutive lanes on consecutive
//            16-byte chunks of a row, 1 KB per instruction, every load of the tile in
//            flight at once) into the wave's LDS tile; the chunks of row r are rotated by r
//            so that the reads below hit distinct banks;
//   scores   lane = key: x[h] = q[h] . K[key] for the g heads of the kv head (fused GQA
//            tile, FA4Config BM_eff), K from the LDS tile, q broadcast from LDS;
//   softmax  online: running max m, per-lane running sum, O rescaled by
//            exp2((m_old - m_new) * c) (FA4Config, num_correction_cols);
//   P.V      lane = 16-byte depth slice of one key, V read straight from the cache into
//            registers (a row per LPR consecutive lanes: coalesced), issued with the K
//            loads so that both arrive in one round trip: O[h][d] += p[h][key] V[key][d].
// A tile's cache rows come from one page-table read per tile when tiles cannot straddle a
// page, else from one read per lane (key = lane) handed to the lanes that load them by
// readlane; either way the read is made one tile ahead. q is loaded before the first tile
// and written to LDS after that tile's loads are issued.
// The four waves then merge their (m, l, O) through LDS with the same log-sum-exp weights
// as the split-K combine (fa4_lse_combine_write: two O fragments merged with per-row
// scales), and the workgroup stores the normalised partial and (m, l) of its partition
// (fa4_splitk_combine_write, second paragraph), or the final bf16 row when the sequence has
// one partition. With the fused combine the last workgroup of a (sequence, kv head) to store
// its partial combines them (fa4_splitk_combine_write, fourth paragraph).
#include "da_device.h"

namespace da {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kTile = 64;   // keys per tile (one per lane in the scores)

template <typename T>
struct Vec16;
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static void unpack(u32x4 v, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u = v[i];   // (a vector element is not addressable: copy it out first)
      out[i] = __builtin_bit_cast(float, u);
    }
  }
};
template <>
struct Vec16<uint16_t> {
  static constexpr int N = 8;
  __device__ static void unpack(u32x4 v, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = bf16lo(v[i]);
      out[2 * i + 1] = bf16hi(v[i]);
    }
  }
};

// LDS sizes of one workgroup (64-key tiles). fp32 holds one workgroup per CU, bf16 two.
template <typename T, int GMAX>
struct FmaLds {
  static constexpr int kMinWaves = sizeof(T) == 2 && GMAX <= 4 ? 2 : 1;   // waves per SIMD aimed at
  static constexpr int kRowBytes = kD * (int)sizeof(T);
  static constexpr int kPBytes = kWaves * kTile * GMAX * 4;        // p during the key loop
  static constexpr int kCBytes = kWaves * GMAX * (kD + 2) * 4;        // (m, l, O) for the merge
  static constexpr int kTileBytes = kWaves * kTile * kRowBytes;   // one buffer of K tiles
  static constexpr int kKtBytes = kTileBytes > kCBytes ? kTileBytes : kCBytes;
  static constexpr int kBytes = kKtBytes + kPBytes + GMAX * kD * 4 + 16;
};

// AFF: every tile lies within one page (contiguous cache, or pages and chunks in multiples
// of the tile), so its rows are consecutive.
template <typename T, int GMAX, int PM, bool AFF>
__global__ __launch_bounds__(kWaves * 64, (FmaLds<T, GMAX>::kMinWaves)) void partition_fma_kernel(PartArgs a) {
  typedef FmaLds<T, GMAX> Lds;
  static_assert(Lds::kBytes <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) char kt_s[Lds::kKtBytes];   // K tiles, then the merge arrays
  __shared__ __attribute__((aligned(16))) float p_s[kWaves][kTile][GMAX];
  __shared__ __attribute__((aligned(16))) float q_s[GMAX][kD];
  __shared__ int last_s;                                                // fused combine: 1 = last
  constexpr int VEC = Vec16<T>::N;      // elements per 16-byte chunk
  constexpr int RB = Lds::kRowBytes;   // bytes of one K / V row of a kv head
  constexpr int CPR = RB / 16;          // chunks per row
  constexpr int RPI = 64 / CPR;         // rows per 1 KB load instruction
  constexpr int NLD = kTile / RPI;      // load instructions per K tile
  constexpr int LPR = CPR;              // lanes covering one V row in the P.V phase
  constexpr int TPI = 64 / LPR;         // keys per P.V load instruction
  constexpr int NV = kTile / TPI;       // P.V load instructions per tile

  // kv heads fastest in the grid: the workgroups of all heads of one key range run together,
  // so the rows of neighbouring heads (adjacent in the cache) are read at about the same time
  const int kvh = blockIdx.x % a.Hkv, p = blockIdx.x / a.Hkv, b = blockIdx.y;
  const int L = attended_len(a, b, PM == kContiguous);
  const int start = p * a.chunk;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // (uniform: tile indices and page lookups stay scalar)
  const int g = a.g;
  constexpr int kUnits = kD / 4;   // 4-wide depth slices of an output row
  if (start >= L) {
    // fused combine: the rows of a sequence without keys (O = 0, LSE = -inf) come from
    // its first workgroup
    if (a.counters && p == 0 && L == 0)
      for (int u = tid; u < g * kUnits; u += kWaves * 64)
        write_row_unit(a.out, a.o32, a.lse, (int64_t)b * a.Hq + kvh * g + u / kUnits, kD, (u % kUnits) * 4,
                       -INFINITY, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}, a.scale);
    return;
  }
  const int end = min(start + a.chunk, L);
  const int P_b = min((L + a.chunk - 1) / a.chunk, a.max_splits);
  const bool direct = a.direct_single && P_b == 1;

  // q of the g heads: loads issued now, written to LDS once the first tile's loads are out
  constexpr int kQPer = (GMAX * kD + kWaves * 64 - 1) / (kWaves * 64);
  const T* q = (const T*)a.q + ((int64_t)b * a.Hq + (int64_t)kvh * g) * kD;
  float qv[kQPer];
#pragma unroll
  for (int j = 0; j < kQPer; ++j) {
    const int i = tid + j * kWaves * 64, h = i / kD;
    qv[j] = 0.f;
    if (i < GMAX * kD && h < g) {
      if constexpr (sizeof(T) == 4) qv[j] = ((const float*)q)[i];
      else qv[j] = bf16lo((uint32_t)((const uint16_t*)q)[i]);
    }
  }

  // (kvh and a.Hkv count virtual kv heads, a.kv_div of them per cached kv head)
  const int kvc = kvh / a.kv_div, kv_heads = a.Hkv / a.kv_div;
  const char* kc = (const char*)a.k + (int64_t)kvc * RB;
  const char* vc = (const char*)a.v + (int64_t)kvc * a.v_row_len * (int64_t)sizeof(T);
  const int64_t kstride = (int64_t)kv_heads * RB;                                  // bytes between K rows
  const int64_t vstride = (int64_t)kv_heads * a.v_row_len * (int64_t)sizeof(T);   // bytes between V rows

  float m[GMAX], lsum[GMAX], o[GMAX][VEC];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[h][e] = 0.f;
  }
  const int col0 = (lane % LPR) * VEC;
  const int tsub = lane / LPR;
  const int n_tiles = (end - start + kTile - 1) / kTile;

  // Loads of tile `it` into K buffer `buf` and the registers vr.
  //   K: load i, lane l fills tile row rr = RPI i + l / CPR at chunk slot l % CPR with that
  //      row's chunk (slot - rr) mod CPR (rotation by the row), 1 KB per instruction;
  //   V: load i, lane l reads the 16-byte slice col0 of key tsub + i TPI into vr[i].
  // Keys past the end repeat the last key (masked in the softmax). With AFF the tile's rows
  // are consecutive from the row of its first key; otherwise every lane finds the row of key
  // t0 + lane and the rows a lane loads are taken from their owners by readlane. The
  // page-table entries of a tile are read one tile ahead of its loads (page_entry), and
  // turned into rows only when the tile is issued (row_of), so that the read is not waited
  // for in front of the loads.
  auto key_of = [&](int it) {
    const int t0 = start + it * kTile;
    return AFF ? t0 : min(t0 + lane, end - 1);
  };
  auto page_entry = [&](int t) -> int {
    if constexpr (PM == kContiguous) {
      return 0;
    } else if constexpr (AFF) {
      // one entry per tile, at a wave-uniform address: read through the scalar cache (the
      // table is not written during the kernel), so that it is not waited for with the
      // vector loads
      typedef const __attribute__((address_space(4))) int32_t* ConstPtr;
      return ((ConstPtr)a.page_table)[(int64_t)b * a.pt_stride + t / a.page_size];
    } else {
      return a.page_table[(int64_t)b * a.pt_stride + t / a.page_size];
    }
  };
  auto row_of = [&](int t, int page) -> int64_t {
    if constexpr (PM == kContiguous) return (int64_t)b * a.kv_capacity + t;
    page = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
    return (int64_t)page * a.page_size + (t - (t / a.page_size) * a.page_size);
  };
  auto issue = [&](int it, u32x4(&vr)[NV], int64_t row) {
    const int t0 = start + it * kTile;
    const int last = end - 1 - t0;
    char* ktb = kt_s + w * kTile * RB;
    if constexpr (AFF) {
      const int64_t r0 = row;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int rr = RPI * i + lane / CPR;
        const int c = ((lane % CPR) - rr) & (CPR - 1);
        const char* src = kc + (r0 + min(rr, last)) * kstride + 16 * c;
        __builtin_amdgcn_global_load_lds((const void*)src, (DA_LDS void*)(ktb + i * 1024), 16, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < NV; ++i)
        vr[i] = *(const u32x4*)(vc + (r0 + min(tsub + i * TPI, last)) * vstride + col0 * (int)sizeof(T));
      return;
    }
    const int64_t ko = row * kstride, vo = row * vstride;
    auto from = [&](int64_t v, int src) {
      return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), src) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, src));
    };
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      int64_t off = from(ko, RPI * i);
#pragma unroll
      for (int r = 1; r < RPI; ++r) {
        const int64_t alt = from(ko, RPI * i + r);
        off = lane / CPR == r ? alt : off;
      }
      const int rr = RPI * i + lane / CPR;
      const int c = ((lane % CPR) - rr) & (CPR - 1);
      __builtin_amdgcn_global_load_lds((const void*)(kc + off + 16 * c), (DA_LDS void*)(ktb + i * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int64_t off = from(vo, i * TPI);
#pragma unroll
      for (int r = 1; r < TPI; ++r) {
        const int64_t alt = from(vo, i * TPI + r);
        off = tsub == r ? alt : off;
      }
      vr[i] = *(const u32x4*)(vc + off + col0 * (int)sizeof(T));
    }
  };

  // One tile's math, its K tile in LDS (the caller waited for it); the V registers are
  // waited for by the compiler at their first use.
  auto compute = [&](int it, const u32x4(&vr)[NV]) {
    const bool valid = start + it * kTile + lane < end;
    // scores, lane = key: chunk c of row r sits at slot (c + r) mod CPR
    float x[GMAX];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) x[h] = 0.f;
    const char* myrow = kt_s + (w * kTile + lane) * RB;
#pragma unroll 8
    for (int c = 0; c < CPR; ++c) {
      float kv[VEC];
      Vec16<T>::unpack(*(const u32x4*)(myrow + 16 * ((c + lane) & (CPR - 1))), kv);
#pragma unroll
      for (int h = 0; h < GMAX; ++h)
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[h] = fmaf(q_s[h][c * VEC + e], kv[e], x[h]);
    }

    // online softmax per head
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      const float mx = wave_max(valid ? x[h] : -INFINITY);
      const float mn = fmaxf(m[h], mx);
      const float alpha = exp2_fast((m[h] - mn) * a.c);
      const float pv = valid ? exp2_fast(fmaf(x[h], a.c, -mn * a.c)) : 0.f;
      lsum[h] = fmaf(lsum[h], alpha, pv);
      m[h] = mn;
      p_s[w][lane][h] = pv;
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[h][e] *= alpha;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // P.V: O[h][d] += p[h][key] V[key][d]
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j = tsub + i * TPI;
      float vv[VEC];
      Vec16<T>::unpack(vr[i], vv);
#pragma unroll
      for (int h = 0; h < GMAX; ++h) {
        const float pj = p_s[w][j][h];
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[h][e] = fmaf(pj, vv[e], o[h][e]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  u32x4 va[NV];
  int page_next = 0;
  if (w < n_tiles) {
    const int t = key_of(w), e = page_entry(t);
    if (w + kWaves < n_tiles) page_next = page_entry(key_of(w + kWaves));
    issue(w, va, row_of(t, e));
  }
#pragma unroll
  for (int j = 0; j < kQPer; ++j) {
    const int i = tid + j * kWaves * 64;
    if (i < GMAX * kD) q_s[i / kD][i % kD] = qv[j];
  }
  __syncthreads();   // (waits for the first tile's loads too: q, K and V arrive in one round trip)

  for (int it = w; it < n_tiles; it += kWaves) {
    if (it != w) {
      const int e = page_next;
      if (it + kWaves < n_tiles) page_next = page_entry(key_of(it + kWaves));
      issue(it, va, row_of(key_of(it), e));
    }
    wait_vm<NV>();   // the K tile is in LDS (its loads were issued before the V loads)
    compute(it, va);
  }

  // finish this wave's (m, l, O)
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    lsum[h] = wave_sum(lsum[h]);
#pragma unroll
    for (int e = 0; e < VEC; ++e)
#pragma unroll
      for (int s = LPR; s < 64; s <<= 1) o[h][e] += __shfl_xor(o[h][e], s);
  }
  __syncthreads();   // (the K tiles are free: the merge arrays take their place)
  float* cm = (float*)kt_s;                         // [kWaves][GMAX] max
  float* cl = cm + kWaves * GMAX;                    // [kWaves][GMAX] sum
  float* co = cl + kWaves * GMAX;                    // [kWaves][GMAX][kD] O
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      cm[w * GMAX + h] = m[h];
      cl[w * GMAX + h] = lsum[h];
    }
  }
  if (tsub == 0) {
#pragma unroll
    for (int h = 0; h < GMAX; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e) co[(w * GMAX + h) * kD + col0 + e] = o[h][e];
  }
  __syncthreads();

  // merge the waves (same LSE weights as the split-K combine) and store; the fused combine's
  // fold below takes the same units in the same order, so each thread keeps what it stored
  constexpr int kOwn = (GMAX * kUnits + kWaves * 64 - 1) / (kWaves * 64);
  OwnPartial own[kOwn];
#pragma unroll
  for (int k = 0; k < kOwn; ++k) {
    const int u = tid + k * kWaves * 64;
    if (u >= g * kUnits) break;
    const int h = u / kUnits, d0 = (u % kUnits) * 4;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, cm[ww * GMAX + h]);
    float Ls = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float e = exp2_fast((cm[ww * GMAX + h] - M) * a.c);
      Ls = fmaf(cl[ww * GMAX + h], e, Ls);
      const f32x4 ov = *(const f32x4*)(co + (ww * GMAX + h) * kD + d0);
      acc += e * ov;
    }
    const float inv = 1.f / Ls;
    own[k].idx = p;
    own[k].ml = make_float2(M, Ls);
    own[k].o = acc * inv;
    store_unit(a, b, kvh * g + h, p, direct, d0, own[k].o, M, Ls, d0 == 0);
  }

  if (!a.counters || direct) return;
  // Fused combine, published as in the matrix-core kernel: the partial stores (device-
  // coherent, cache policy SC1) of every wave complete before the barrier, then one count on
  // the (sequence, kv head) counter; the workgroup that completes the count reads the
  // others' partials with SC1 loads and writes the g final rows.
  wait_vm<0>();
  __syncthreads();
  int* cnt = a.counters + (int64_t)b * a.Hkv + kvh;
  if (tid == 0) {
    const int last = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == P_b - 1;
    last_s = last ? 1 : 0;
  }
  __syncthreads();
  if (!__builtin_amdgcn_readfirstlane(last_s)) return;
#pragma unroll
  for (int k = 0; k < kOwn; ++k) {
    const int u = tid + k * kWaves * 64;
    if (u >= g * kUnits) break;
    const int h = u / kUnits, d0 = (u % kUnits) * 4;
    const int64_t row = (int64_t)b * a.Hq + kvh * g + h;
    float M = -INFINITY, Ls = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    fold_partials<kD, 8, true>((const float2*)a.part_ml + row * a.max_splits,
                               a.part_o + row * a.max_splits * kD + d0, 1, P_b, 0, 1, a.c, M, Ls, acc, a.part_ml,
                               a.part_o, own[k]);
    write_row_unit(a.out, a.o32, a.lse, row, kD, d0, M, Ls, acc, a.scale);
  }
  if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T, int GMAX>
hipError_t launch_t(const PartArgs& a, int pm, hipStream_t s) {
  if ((int64_t)a.max_splits * a.Hkv > INT32_MAX || a.B > 65535) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)(a.max_splits * a.Hkv), a.B), block(kWaves * 64);
  if (pm == kContiguous)
    hipLaunchKernelGGL((partition_fma_kernel<T, GMAX, kContiguous, true>), grid, block, 0, s, a);
  else if (a.page_size % kTile == 0 && a.chunk % kTile == 0)
    hipLaunchKernelGGL((partition_fma_kernel<T, GMAX, kPagedGeneral, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((partition_fma_kernel<T, GMAX, kPagedGeneral, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_g(const PartArgs& a, int pm, hipStream_t s) {
  if (a.g <= 1) return launch_t<T, 1>(a, pm, s);
  if (a.g <= 2) return launch_t<T, 2>(a, pm, s);
  if (a.g <= 4) return launch_t<T, 4>(a, pm, s);
  if (a.g <= 8) return launch_t<T, 8>(a, pm, s);
  return launch_t<T, 16>(a, pm, s);
}

}  // namespace

hipError_t launch_partition_fma(const PartArgs& a, int dtype, int page_mode, hipStream_t s) {
  if (dtype == 0) return launch_g<float>(a, page_mode, s);
  return launch_g<uint16_t>(a, page_mode, s);
}

}  // namespace da
