// Split-K pass 1 on the vector ALU: one workgroup per (partition, kv head, sequence).
//
// Used for fp32 caches and for single-head groups, where q.K and P.V are not
// dense enough to feed the matrix cores. Four waves split the partition's keys
// in 64-key tiles (tile i goes to wave i % 4). Within a tile:
//   scores   lane = key: x[h] = q[h] . K[key] for the g heads of the kv head
//            (fused GQA tile, FA4Config BM_eff), q broadcast from LDS;
//   softmax  online: running max m, per-lane running sum, O rescaled by
//            exp2((m_old - m_new) * c) (FA4Config, num_correction_cols);
//   P.V      lane = 16-byte depth slice of one key: O[h][d] += p[h][key] V[key][d].
// The four waves then merge their (m, l, O) through LDS with the same
// log-sum-exp weights as the split-K combine (fa4_lse_combine_write: two O
// fragments merged with per-row scales), and the workgroup stores the
// normalised partial and (m, l) of its partition (fa4_splitk_combine_write,
// second paragraph), or the final bf16 row when the sequence has one partition.
#include "da_device.h"

namespace da {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;

template <typename T>
struct Vec16;
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* out) {
    f32x4 v = *(const f32x4*)p;
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
  }
};
template <>
struct Vec16<uint16_t> {
  static constexpr int N = 8;
  __device__ static void load(const uint16_t* p, float* out) {
    u32x4 v = *(const u32x4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = bf16lo(v[i]);
      out[2 * i + 1] = bf16hi(v[i]);
    }
  }
};

template <typename T, int GMAX, int PM>
__global__ __launch_bounds__(kWaves * 64) void partition_fma_kernel(PartArgs a) {
  constexpr int VEC = Vec16<T>::N;      // elements per 16-byte load
  constexpr int LPR = kD / VEC;         // lanes covering one row in the P.V phase
  constexpr int TPI = 64 / LPR;         // keys per P.V load instruction
  constexpr int kTile = 64;

  const int p = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int L = attended_len(a, b, PM == kContiguous);
  const int start = p * a.chunk;
  if (start >= L) return;
  const int end = min(start + a.chunk, L);
  const int P_b = min((L + a.chunk - 1) / a.chunk, a.max_splits);
  const bool direct = a.direct_single && P_b == 1;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = a.g;

  __shared__ float q_s[GMAX][kD];
  __shared__ int64_t rows_s[kWaves][kTile];
  // p_s during the key loop, then the per-wave (m, l, O) for the merge.
  constexpr int kPBytes = kWaves * kTile * GMAX * 4;
  constexpr int kCBytes = kWaves * GMAX * (kD + 2) * 4;
  __shared__ __attribute__((aligned(16))) char scratch[kPBytes > kCBytes ? kPBytes : kCBytes];
  float(*p_s)[kTile][GMAX] = (float(*)[kTile][GMAX])scratch;

  const T* q = (const T*)a.q + ((int64_t)b * a.Hq + (int64_t)kvh * g) * kD;
  for (int i = tid; i < GMAX * kD; i += kWaves * 64) {
    const int h = i / kD, d = i % kD;
    float val = 0.f;
    if (h < g) {
      if constexpr (sizeof(T) == 4) val = ((const float*)q)[h * kD + d];
      else val = bf16lo((uint32_t)((const uint16_t*)q)[h * kD + d]);
    }
    q_s[h][d] = val;
  }
  __syncthreads();

  const T* kc = (const T*)a.k;
  const T* vc = (const T*)a.v;
  const int64_t kstride = (int64_t)a.Hkv * a.Dqk;
  const int64_t vstride = (int64_t)a.Hkv * a.v_row_len;

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
  for (int it = w; it < n_tiles; it += kWaves) {
    const int t0 = start + it * kTile;
    const int t = t0 + lane;
    const bool valid = t < end;
    const int64_t row = key_row<PM>(a, b, valid ? t : end - 1);
    rows_s[w][lane] = row;

    // scores, lane = key
    float x[GMAX];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) x[h] = 0.f;
    const T* krow = kc + row * kstride + (int64_t)kvh * a.Dqk;
#pragma unroll 4
    for (int c = 0; c < LPR; ++c) {
      float kv[VEC];
      Vec16<T>::load(krow + c * VEC, kv);
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

    // P.V, lane = (key subset, 16-byte depth slice)
#pragma unroll 4
    for (int j = tsub; j < kTile; j += TPI) {
      const int64_t r = rows_s[w][j];
      float vv[VEC];
      Vec16<T>::load(vc + r * vstride + (int64_t)kvh * a.v_row_len + col0, vv);
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
  __syncthreads();
  float* cm = (float*)scratch;                       // [kWaves][GMAX] max
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

  // merge the waves (same LSE weights as the split-K combine) and store
  constexpr int kUnits = kD / 4;
  for (int u = tid; u < g * kUnits; u += kWaves * 64) {
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
    store_unit(a, b, kvh * g + h, p, direct, d0, acc * inv, M, Ls, d0 == 0);
  }
}

template <typename T, int GMAX>
hipError_t launch_t(const PartArgs& a, int pm, hipStream_t s) {
  dim3 grid(a.max_splits, a.Hkv, a.B), block(kWaves * 64);
  switch (pm) {
    case kContiguous:
      hipLaunchKernelGGL((partition_fma_kernel<T, GMAX, kContiguous>), grid, block, 0, s, a);
      break;
    default:
      hipLaunchKernelGGL((partition_fma_kernel<T, GMAX, kPagedGeneral>), grid, block, 0, s, a);
      break;
  }
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
