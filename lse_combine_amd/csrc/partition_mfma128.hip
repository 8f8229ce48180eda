// Split-K pass 1 on the matrix cores for bf16 caches with Dqk = Dv = 128 and a GQA
// group of up to 16 q heads per kv head (FA4Config: fused GQA tiles, BM_eff).
//
// One workgroup per (partition, kv head, sequence); NW waves split the
// partition's keys in 32-key tiles (tile i goes to wave i % NW) and each keeps
// its own online-softmax state. Per tile, with v_mfma_f32_16x16x32_bf16:
//
//   S^T[key][col] = K[key][:] . q[col][:]      A = K rows straight from HBM (16-byte
//                                              loads already in the A-operand layout),
//                                              B = q (16 columns, see below)
//   p = exp2((x - m_new) * c)                  online softmax in fp32; every lane owns
//                                              one column and 8 keys, so the row max
//                                              needs two cross-lane steps
//   O^T[d][col] += V^T[d][key] . P^T[key][col] A = V^T read from LDS with the gfx950
//                                              transposing read ds_read_b64_tr_b16,
//                                              B = P^T taken from the S^T registers as is
//
// P must not be rounded to bf16 before P.V (the fp32 O must stay within 1e-5), so
// P is split as p = hi + lo with hi = bf16(p), lo = bf16(p - hi) (about 16
// significant bits). When g <= 8 the 16 MFMA columns hold the g heads twice:
// columns 0-7 carry hi, columns 8-15 carry lo (the scores of both copies are the
// same), so hi and lo cost one MFMA; the two halves of O^T are summed at the end.
// For 8 < g <= 16 a second MFMA per depth block adds the lo part.
//
// After the key loop the waves merge their (m, l, O) through LDS with the
// log-sum-exp weights (fa4_lse_combine_write: fragments merged with per-row
// scales) and the workgroup stores the normalised partial and (m, l)
// (fa4_splitk_combine_write, second paragraph), or the finished bf16 row when the
// sequence has a single partition.
//
// Loads are software-pipelined: the next tile's K and V (16 KB per wave) are in
// flight while the current tile is computed.
#include "da_device.h"

namespace da {
namespace {

constexpr int kD = 128;
constexpr int kTile = 32;
constexpr int kVBytes = kTile * kD * 2;       // one wave's V tile in LDS
constexpr int kWaveBytes = kVBytes + 256;     // + merge (m, l) for up to 16 heads

typedef short s16x8 __attribute__((ext_vector_type(8)));

struct Tile {
  u32x4 k[2][4];  // K rows: [key block][depth step], 8 bf16 each
  u32x4 v[8];     // V: 8 x 16 bytes, stored to LDS as loaded
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int NW, bool HL, int PM>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void partition_mfma128_kernel(PartArgs a) {
  const int p = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int L = attended_len(a, b, PM == kContiguous);
  const int start = p * a.chunk;
  if (start >= L) return;
  const int end = min(start + a.chunk, L);
  const int P_b = min((L + a.chunk - 1) / a.chunk, a.max_splits);
  const bool direct = a.direct_single && P_b == 1;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, qd = lane >> 4;
  const int g = a.g;
  const int hc = HL ? (n & 7) : n;          // head index of this lane's MFMA column
  const bool col_valid = hc < g;
  const bool is_lo = HL && n >= 8;

  __shared__ __attribute__((aligned(16))) char smem[NW * kWaveBytes];
  char* vt = smem + w * kWaveBytes;

  // q as the B operand of S^T = K q^T: column n, depth 32j + 8qd .. +8.
  bf16x8 qf[4];
  {
    const uint16_t* qrow =
        (const uint16_t*)a.q + ((int64_t)b * a.Hq + (int64_t)kvh * g + (col_valid ? hc : 0)) * kD;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 v = *(const u32x4*)(qrow + 32 * j + 8 * qd);
      if (!col_valid) v = u32x4{0u, 0u, 0u, 0u};
      qf[j] = as_bf16x8(v);
    }
  }

  const uint16_t* kc = (const uint16_t*)a.k;
  const uint16_t* vc = (const uint16_t*)a.v;
  const int64_t kstride = (int64_t)a.Hkv * kD;
  const int64_t vstride = (int64_t)a.Hkv * a.v_row_len;
  const int64_t koff = (int64_t)kvh * kD;
  const int64_t voff = (int64_t)kvh * a.v_row_len;
  const float c = a.c;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // cache row of key kk (0..31) of the tile starting at t0; keys past the end are
  // clamped to the last valid key (loaded but given p = 0)
  auto row_of = [&](int t0, int kk) -> int64_t {
    const int last = end - 1 - t0;
    kk = kk < last ? kk : last;
    if constexpr (PM == kContiguous) {
      return (int64_t)b * a.kv_capacity + t0 + kk;
    } else if constexpr (PM == kPagedAligned) {
      const int pi = t0 / a.page_size;    // the whole tile sits in this page
      int page = a.page_table[(int64_t)b * a.pt_stride + pi];
      page = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
      return (int64_t)page * a.page_size + (t0 - pi * a.page_size) + kk;
    } else {
      return key_row<PM>(a, b, t0 + kk);
    }
  };

  auto load_tile = [&](Tile& T, int it) {
    const int t0 = start + it * kTile;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const uint16_t* kp = kc + row_of(t0, n + 16 * blk) * kstride + koff + 8 * qd;
#pragma unroll
      for (int j = 0; j < 4; ++j) T.k[blk][j] = __builtin_nontemporal_load((const u32x4*)(kp + 32 * j));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + qd;             // tile row this lane stages
      const int chunk = n ^ (r & 15);       // XOR swizzle of 16-byte chunks within the row
      const uint16_t* vp = vc + row_of(t0, r) * vstride + voff + 8 * chunk;
      T.v[i] = __builtin_nontemporal_load((const u32x4*)vp);
    }
  };

  auto compute = [&](const Tile& T, int it) {
    const int t0 = start + it * kTile;
    const int nvalid = min(kTile, end - t0);
    // stage V (row-major, swizzled) for the transposing reads
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u32x4*)(vt + (i * 64 + lane) * 16) = T.v[i];

    // S^T = K q^T for keys 0-15 and 16-31
    f32x4 s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      s[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        s[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(T.k[blk][j]), qf[j], s[blk], 0, 0, 0);
    }

    // online softmax: this lane holds keys 16*blk + 4*qd + i of column n
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (16 * blk + 4 * qd + i < nvalid) mx = fmaxf(mx, s[blk][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m_run, mx);
    const float alpha = exp2_fast((m_run - mn) * c);
    const float mc = mn * c;
    float pr[2][4];
    float psum = 0.f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = 16 * blk + 4 * qd + i < nvalid;
        pr[blk][i] = ok ? exp2_fast(fmaf(s[blk][i], c, -mc)) : 0.f;
        psum += pr[blk][i];
      }
    l_run = fmaf(l_run, alpha, psum);
    m_run = mn;
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db] *= alpha;

    // P^T as the B operand: k-slots 0-3 = keys 4qd..+3, 4-7 = keys 16+4qd..+3
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const int blk = s2 >> 1, i0 = (s2 & 1) * 2;
      const float p0 = pr[blk][i0], p1 = pr[blk][i0 + 1];
      const uint32_t h = pack_bf16x2(p0, p1);
      hw[s2] = h;
      lw[s2] = pack_bf16x2(p0 - bf16lo(h), p1 - bf16hi(h));
    }
    bf16x8 pb_hi, pb_lo;
    if constexpr (HL) {
      u32x4 sel = is_lo ? u32x4{lw[0], lw[1], lw[2], lw[3]} : u32x4{hw[0], hw[1], hw[2], hw[3]};
      pb_hi = as_bf16x8(sel);
    } else {
      pb_hi = as_bf16x8(u32x4{hw[0], hw[1], hw[2], hw[3]});
      pb_lo = as_bf16x8(u32x4{lw[0], lw[1], lw[2], lw[3]});
    }

    // V^T A operand: lane (n, qd) gets depth 16db + n of keys 4qd..+3 and 16+4qd..+3
    const int r0 = 4 * qd + (n >> 2);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int ch = 2 * db + ((n & 3) >> 1);
      const int sub = (n & 1) * 8;
      const int ra = r0, rb = r0 + 16;
      const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (s16x4 DA_LDS*)(vt + ra * 256 + ((ch ^ (ra & 15)) << 4) + sub));
      const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (s16x4 DA_LDS*)(vt + rb * 256 + ((ch ^ (rb & 15)) << 4) + sub));
      s16x8 v8;
      v8[0] = va[0]; v8[1] = va[1]; v8[2] = va[2]; v8[3] = va[3];
      v8[4] = vb[0]; v8[5] = vb[1]; v8[6] = vb[2]; v8[7] = vb[3];
      const bf16x8 vf = __builtin_bit_cast(bf16x8, v8);
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb_hi, o[db], 0, 0, 0);
      if constexpr (!HL) o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb_lo, o[db], 0, 0, 0);
    }
  };

  const int n_tiles = (end - start + kTile - 1) / kTile;
  int it = w;
  if (it < n_tiles) {
    Tile A, B;
    load_tile(A, it);
    while (true) {
      load_tile(B, min(it + NW, n_tiles - 1));
      compute(A, it);
      it += NW;
      if (it >= n_tiles) break;
      load_tile(A, min(it + NW, n_tiles - 1));
      compute(B, it);
      it += NW;
      if (it >= n_tiles) break;
    }
  }

  // this wave's totals: sum l over the four key groups; fold the lo columns into hi
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if constexpr (HL) {
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[db][i] += __shfl_xor(o[db][i], 8);
  }

  // merge the waves through LDS (each wave reuses its own V region)
  float* mo = (float*)vt;                      // [16][128] O of this wave
  float* mml = (float*)(vt + kVBytes);         // m[16], l[16]
  if (col_valid && !is_lo) {
#pragma unroll
    for (int db = 0; db < 8; ++db) *(f32x4*)(mo + hc * kD + 16 * db + 4 * qd) = o[db];
    if (qd == 0) {
      mml[hc] = m_run;
      mml[16 + hc] = l_run;
    }
  }
  __syncthreads();
  constexpr int kUnits = kD / 4;
  for (int u = tid; u < g * kUnits; u += NW * 64) {
    const int h = u / kUnits, d0 = (u % kUnits) * 4;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, ((const float*)(smem + ww * kWaveBytes + kVBytes))[h]);
    float Ls = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float* ml = (const float*)(smem + ww * kWaveBytes + kVBytes);
      const float e = exp2_fast((ml[h] - M) * c);
      Ls = fmaf(ml[16 + h], e, Ls);
      acc += e * *(const f32x4*)((const float*)(smem + ww * kWaveBytes) + h * kD + d0);
    }
    store_unit(a, b, kvh * g + h, p, direct, d0, acc * (1.f / Ls), M, Ls, d0 == 0);
  }
}

template <int NW, bool HL>
hipError_t launch_nw(const PartArgs& a, int pm, hipStream_t s) {
  dim3 grid(a.max_splits, a.Hkv, a.B), block(NW * 64);
  switch (pm) {
    case kContiguous:
      hipLaunchKernelGGL((partition_mfma128_kernel<NW, HL, kContiguous>), grid, block, 0, s, a);
      break;
    case kPagedAligned:
      hipLaunchKernelGGL((partition_mfma128_kernel<NW, HL, kPagedAligned>), grid, block, 0, s, a);
      break;
    default:
      hipLaunchKernelGGL((partition_mfma128_kernel<NW, HL, kPagedGeneral>), grid, block, 0, s, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_partition_mfma128(const PartArgs& a, int page_mode, int waves, hipStream_t s) {
  const bool hl = a.g <= 8;
  if (waves >= 8) return hl ? launch_nw<8, true>(a, page_mode, s) : launch_nw<8, false>(a, page_mode, s);
  return hl ? launch_nw<4, true>(a, page_mode, s) : launch_nw<4, false>(a, page_mode, s);
}

}  // namespace da
