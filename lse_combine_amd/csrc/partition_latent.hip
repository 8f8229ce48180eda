// Split-K pass 1 for the latent-shared layout: one kv head whose K rows hold 576 values
// (512 non-rotary followed by 64 rotary ones, FA4Config rope_depth) and V = the first
// 512 values of each K row (FA4Config shared_kv_cols: K_nope and V share one buffer).
// Every q head of a sequence attends the same rows, so q.K and P.V are dense
// contractions (about 240 flop per byte of KV) and run on v_mfma_f32_16x16x32_bf16.
//
// Workgroup = (partition p, block of 64 q heads, sequence b); four waves, each owning
// 16 heads (one MFMA column block) and their full 512-wide output:
//   S^T[key][head] = K[key][0:576] . q[head][0:576]   A = K from the LDS tile,
//                                                      B = q from LDS (18 k-steps)
//   O^T[d][head]  += V^T[d][key] . P^T[key][head]       A = V^T read transposed from the
//                                                      same LDS tile (ds_read_b64_tr_b16),
//                                                      B = P^T from the S^T registers
// P is split hi/lo in bf16 (two MFMAs per depth block) so that the fp32 O keeps ~16
// significant bits of the weights. The K tile (32 keys x 1152 B, 16-byte chunks XOR
// swizzled within groups of 8) is double-buffered in LDS: the next tile's global loads
// are in flight while the current tile is computed. The two head blocks of a
// (sequence, partition) get workgroup ids 8 apart, so they run on the same XCD and the
// second read of each K tile is an L2 hit.
// Epilogue as in the GQA kernel: normalised partial + (m, l) per head, or the finished
// bf16 row when the sequence has a single partition (fa4_splitk_combine_write, second
// paragraph; fa4_scale_write_output for the single-partition case).
#include "da_device.h"

namespace da {
namespace {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kTile = 32;
constexpr int kChunks = kDqk / 8;               // 16-byte chunks per K row (72)
constexpr int kRowBytes = kDqk * 2;             // 1152
constexpr int kTileBytes = kTile * kRowBytes;   // 36 KB
constexpr int kHeadsPerWave = 16;
constexpr int kWaves = 4;
constexpr int kHeadsPerWG = kHeadsPerWave * kWaves;   // 64
constexpr int kQBytes = kHeadsPerWG * kRowBytes;      // 72 KB
constexpr int kThreads = kWaves * 64;
constexpr int kStage = (kTile * kChunks) / kThreads;  // 16-byte chunks per thread per tile (9)
constexpr int kMaxLdsPages = 256;

typedef short s16x8 __attribute__((ext_vector_type(8)));

// byte offset of 16-byte chunk c of row r in a swizzled LDS row block
__device__ __forceinline__ int swz(int r, int c) { return r * kRowBytes + ((c ^ (r & 7)) << 4); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int PM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
void partition_latent_kernel(PartArgs a) {
  const int p = blockIdx.x, hb = blockIdx.y, b = blockIdx.z;
  const int L = __builtin_amdgcn_readfirstlane(attended_len(a, b, PM == kContiguous));
  const int start = p * a.chunk;
  if (start >= L) return;
  const int end = min(start + a.chunk, L);
  const int P_b = min((L + a.chunk - 1) / a.chunk, a.max_splits);
  const bool direct = a.direct_single && P_b == 1;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, qd = lane >> 4;
  const int g = a.g;
  const int head0 = hb * kHeadsPerWG + w * kHeadsPerWave;   // first q head of this wave
  const bool wave_active = head0 < g;
  const float c = a.c;

  extern __shared__ __attribute__((aligned(16))) char smem[];   // 2 K tiles + q block
  auto ktile = [&](int i) -> char* { return smem + (i & 1) * kTileBytes; };
  char* qs = smem + 2 * kTileBytes;
  __shared__ int pages_s[kMaxLdsPages];

  // q block -> LDS (rows beyond the group are zero)
  {
    const uint16_t* qb = (const uint16_t*)a.q + ((int64_t)b * a.Hq + (int64_t)hb * kHeadsPerWG) * kDqk;
    for (int cid = tid; cid < kHeadsPerWG * kChunks; cid += kThreads) {
      const int h = cid / kChunks, ch = cid % kChunks;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (hb * kHeadsPerWG + h < g) v = *(const u32x4*)(qb + (int64_t)h * kDqk + ch * 8);
      *(u32x4*)(qs + swz(h, ch)) = v;
    }
  }

  // page indices of the partition (one segment: chunks of at most (kMaxLdsPages-1)*page keys)
  int first_page = 0;
  if constexpr (PM != kContiguous) {
    first_page = start / a.page_size;
    const int n_pages = (end - 1) / a.page_size - first_page + 1;
    const int32_t* pt = a.page_table + (int64_t)b * a.pt_stride + first_page;
    for (int i = tid; i < n_pages && i < kMaxLdsPages; i += kThreads) {
      const int page = pt[i];
      pages_s[i] = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
    }
  }
  __syncthreads();

  auto key_row = [&](int t) -> int64_t {   // cache row of key t (t < end)
    if constexpr (PM == kContiguous) {
      return (int64_t)b * a.kv_capacity + t;
    } else {
      const int pi = t / a.page_size;
      const int slot = min(max(pi - first_page, 0), kMaxLdsPages - 1);
      const int page = min(max(pages_s[slot], 0), a.num_pages - 1);
      return (int64_t)page * a.page_size + (t - pi * a.page_size);
    }
  };

  // global -> registers for the tile at t0 (thread covers chunks tid + i*256; rows past
  // the end reuse the last valid key, their scores are masked)
  const uint16_t* kc = (const uint16_t*)a.k;
  const int64_t krow = (int64_t)a.Hkv * kDqk;   // elements between cache rows (Hkv == 1)
  auto fetch = [&](u32x4* st, int t0) {
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
      const int cid = tid + i * kThreads;
      const int r = cid / kChunks, ch = cid % kChunks;
      const int t = min(t0 + r, end - 1);
      st[i] = __builtin_nontemporal_load((const u32x4*)(kc + key_row(t) * krow + ch * 8));
    }
  };
  auto stage = [&](const u32x4* st, char* dst) {
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
      const int cid = tid + i * kThreads;
      const int r = cid / kChunks, ch = cid % kChunks;
      *(u32x4*)(dst + swz(r, ch)) = st[i];
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[kDv / 16];
#pragma unroll
  for (int db = 0; db < kDv / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int n_tiles = (end - start + kTile - 1) / kTile;
  u32x4 st[kStage];
  fetch(st, start);
  stage(st, ktile(0));
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    const int t0 = start + it * kTile;
    const bool has_next = it + 1 < n_tiles;
    if (has_next) fetch(st, t0 + kTile);
    const char* K = ktile(it);

    if (wave_active) {
      // S^T = K q^T: keys 16*blk + (4qd..+3) of column (head) n
      f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll 6
      for (int j = 0; j < kChunks / 4; ++j) {
        const bf16x8 qf = as_bf16x8(*(const u32x4*)(qs + swz(w * kHeadsPerWave + n, 4 * j + qd)));
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          const bf16x8 kf = as_bf16x8(*(const u32x4*)(K + swz(n + 16 * blk, 4 * j + qd)));
          s[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf, s[blk], 0, 0, 0);
        }
      }
      // online softmax (missing keys of a ragged tile get -inf, i.e. p = 0)
      const int nvalid = end - t0;
      if (nvalid < kTile) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * blk + 4 * qd + i >= nvalid) s[blk][i] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                       fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
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
          pr[blk][i] = exp2_fast(fmaf(s[blk][i], c, -mc));
          psum += pr[blk][i];
        }
      l_run = fmaf(l_run, alpha, psum);
      m_run = mn;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < kDv / 16; ++db) o[db] *= alpha;
      }
      // P^T (B operand), hi and lo parts
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const int blk = s2 >> 1, i0 = (s2 & 1) * 2;
        const float p0 = pr[blk][i0], p1 = pr[blk][i0 + 1];
        const uint32_t h = pack_bf16x2(p0, p1);
        hw[s2] = h;
        lw[s2] = pack_bf16x2(p0 - bf16lo(h), p1 - bf16hi(h));
      }
      const bf16x8 pb_hi = as_bf16x8(u32x4{hw[0], hw[1], hw[2], hw[3]});
      const bf16x8 pb_lo = as_bf16x8(u32x4{lw[0], lw[1], lw[2], lw[3]});
      // O^T += V^T P^T; V^T A operand: depth 16db + n of keys 4qd..+3 and 16+4qd..+3
      const int ra = 4 * qd + (n >> 2), rb = ra + 16;
      const int sub = (n & 1) * 8;
#pragma unroll
      for (int db = 0; db < kDv / 16; ++db) {
        const int ch = 2 * db + ((n & 3) >> 1);
        const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 DA_LDS*)(K + swz(ra, ch) + sub));
        const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 DA_LDS*)(K + swz(rb, ch) + sub));
        s16x8 v8;
        v8[0] = va[0]; v8[1] = va[1]; v8[2] = va[2]; v8[3] = va[3];
        v8[4] = vb[0]; v8[5] = vb[1]; v8[6] = vb[2]; v8[7] = vb[3];
        const bf16x8 vf = __builtin_bit_cast(bf16x8, v8);
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb_hi, o[db], 0, 0, 0);
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb_lo, o[db], 0, 0, 0);
      }
    }
    if (has_next) stage(st, ktile(it + 1));
    __syncthreads();
  }

  // totals over the four key groups of each column, then store
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  const int hq = head0 + n;   // q head of this lane's column (within the kv head's group)
  if (wave_active && hq < g) {
    const float inv = 1.f / l_run;
#pragma unroll
    for (int db = 0; db < kDv / 16; ++db)
      store_unit(a, b, hq, p, direct, 16 * db + 4 * qd, o[db] * inv, m_run, l_run, db == 0 && qd == 0);
  }
}

}  // namespace

hipError_t launch_partition_latent(const PartArgs& a, int page_mode, hipStream_t s) {
  if (a.Dqk != kDqk || a.Dv != kDv || a.Hkv != 1 || a.g % kHeadsPerWave) return hipErrorInvalidValue;
  // x = partition, y = 64-head block, z = sequence: with 8 partitions the two head blocks
  // of a (sequence, partition) are 8 workgroup ids apart (same XCD under round-robin dispatch)
  dim3 grid(a.max_splits, (a.g + kHeadsPerWG - 1) / kHeadsPerWG, a.B), block(kThreads);
  const size_t lds = 2 * kTileBytes + kQBytes;
  if (page_mode == kContiguous) {
    hipLaunchKernelGGL(partition_latent_kernel<kContiguous>, grid, block, lds, s, a);
  } else {
    hipLaunchKernelGGL(partition_latent_kernel<kPagedGeneral>, grid, block, lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace da
