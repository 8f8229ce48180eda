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

// max over the four lanes n, n+16, n+32, n+48 on the VALU (v_permlane16/32_swap), without
// the LDS permute unit that the tile's operand reads keep busy. Written out because the
// compiler folds the two results of a swap of a value with itself into one; the s_nop
// gives the two wait states a VALU write needs before a permlane reads it (the compiler
// cannot see into the asm to insert them).
__device__ __forceinline__ float max_over_key_groups(float v) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  v = fmaxf(a, b);
  a = v;
  b = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Fixed reference max: the exponentials are taken relative to the first tile's max
// m_ref and the 128 accumulator registers are never rescaled inside the key loop. That
// holds while every score stays within kHeadroomLog2 powers of two of m_ref (p <= 2^64,
// far from fp32 overflow, and keys far below the max underflow harmlessly). A score
// beyond that (rare; adversarial or huge logits) makes the workgroup run the partition
// once more with m_ref = the partition's exact max. The exact max is tracked on the side.
constexpr float kHeadroomLog2 = 64.f;

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

  // Two K tiles as two distinct LDS arrays: the compiler then sees that reads of one tile
  // do not depend on the direct-to-LDS loads still filling the other, and waits for
  // those loads only where a tile is consumed.
  __shared__ __attribute__((aligned(16))) char kt0[kTileBytes];
  __shared__ __attribute__((aligned(16))) char kt1[kTileBytes];
  extern __shared__ __attribute__((aligned(16))) char qs[];   // q block, kQBytes
  __shared__ int pages_s[kMaxLdsPages];

  // Rows that a ragged tile does not load keep what the buffer held: zero both tiles
  // once so that such rows are finite (their scores are masked, their V meets p = 0).
  for (int i = tid; i < kTileBytes / 16; i += kThreads) {
    *(u32x4*)(kt0 + i * 16) = u32x4{0u, 0u, 0u, 0u};
    *(u32x4*)(kt1 + i * 16) = u32x4{0u, 0u, 0u, 0u};
  }
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

  // The K tile of keys t0 .. t0+31 lands in LDS by direct-to-LDS 16-byte loads: wave w
  // fills the 1 KB blocks w, w+4, ..., so lane l of block j writes tile byte j*1024 + 16l,
  // i.e. row r and chunk slot s of the swizzled layout, and loads the cache chunk
  // s ^ (r & 7) of row r there (the XOR swizzle is its own inverse).
  const char* kc = (const char*)a.k;
  auto lane_chunk = [&](int i, int& r, int& gchunk) {
    const int pos = (w + kWaves * i) * 1024 + lane * 16;
    r = pos / kRowBytes;
    const int slot = (pos - r * kRowBytes) >> 4;
    gchunk = slot ^ (r & 7);
  };
  auto issue = [&](char* dst, int t0) {
    const int last = min(kTile - 1, end - 1 - t0);   // rows 0..last hold keys
    if constexpr (PM != kPagedGeneral) {
      // 32 consecutive cache rows: one scalar base; the buffer range ends at the last
      // valid row, so a ragged tile's missing rows are not read
      int64_t row0;
      if constexpr (PM == kContiguous) {
        row0 = (int64_t)b * a.kv_capacity + t0;
      } else {
        const int slot = min(max((t0 >> a.page_shift) - first_page, 0), kMaxLdsPages - 1);
        // (clamped before readfirstlane: a clamp after it may be done in vector registers,
        // which makes the descriptor divergent and every load a waterfall loop)
        const int page = __builtin_amdgcn_readfirstlane(min(max(pages_s[slot], 0), a.num_pages - 1));
        row0 = ((int64_t)page << a.page_shift) + (t0 & (a.page_size - 1));
      }
      const int rows = __builtin_amdgcn_readfirstlane(last + 1);
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc((void*)(kc + row0 * kRowBytes), 0, rows * kRowBytes, kRsrcWord3);
#pragma unroll
      for (int i = 0; i < kStage; ++i) {
        int r, gc;
        lane_chunk(i, r, gc);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (DA_LDS void*)(dst + (w + kWaves * i) * 1024), 16,
                                                 (uint32_t)(r * kRowBytes + gc * 16), 0, 0, kLoadNT);
      }
    } else {
      // any page size: every lane looks up its own row (rows past the end repeat the
      // last key; their scores are masked)
#pragma unroll
      for (int i = 0; i < kStage; ++i) {
        int r, gc;
        lane_chunk(i, r, gc);
        const int t = t0 + min(r, last);
        const int pi = t / a.page_size;
        const int slot = min(max(pi - first_page, 0), kMaxLdsPages - 1);
        const int page = min(max(pages_s[slot], 0), a.num_pages - 1);
        const int64_t row = (int64_t)page * a.page_size + (t - pi * a.page_size);
        __builtin_amdgcn_global_load_lds((const void*)(kc + row * kRowBytes + gc * 16),
                                         (DA_LDS void*)(dst + (w + kWaves * i) * 1024), 16, 0, 0);
      }
    }
  };

  float m_ref = -INFINITY;   // reference max of the exponentials (raw units)
  float m_true = -INFINITY;  // exact running max
  float l_run = 0.f;
  bool beyond = false;       // a score exceeded m_ref by more than the headroom
  f32x4 o[kDv / 16];

  auto compute = [&](const char* K, int t0) {
    if (!wave_active) return;
    // S^T = K q^T: keys 16*blk + (4qd..+3) of column (head) n
    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
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
    mx = max_over_key_groups(mx);
    m_true = fmaxf(m_true, mx);
    m_ref = m_ref == -INFINITY ? mx : m_ref;   // first tile of the pass: O and l are still 0
    beyond = beyond || (mx - m_ref) * c > kHeadroomLog2;
    const float mc = m_ref * c;
    float pr[2][4];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[blk][i] = exp2_fast(fmaf(s[blk][i], c, -mc));
        l_run += pr[blk][i];
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
  };

  // Double buffer: tile it+1 is requested right after the barrier that retires tile it-1
  // from the other buffer, and lands while tile it is computed. A second pass runs only
  // if some score left the headroom of m_ref (then m_ref = the exact max: no second miss).
  const int n_tiles = (end - start + kTile - 1) / kTile;
  for (int pass = 0; pass < 2; ++pass) {
    l_run = 0.f;
#pragma unroll
    for (int db = 0; db < kDv / 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    issue(kt0, start);
    for (int it = 0; it < n_tiles; it += 2) {
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's part of tile it is in LDS
      __syncthreads();                      // ... and every wave's; tile it-1 is retired
      if (it + 1 < n_tiles) issue(kt1, start + (it + 1) * kTile);
      compute(kt0, start + it * kTile);
      if (it + 1 >= n_tiles) break;
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      if (it + 2 < n_tiles) issue(kt0, start + (it + 2) * kTile);
      compute(kt1, start + (it + 1) * kTile);
    }
    // every wave is past its last LDS read before a second pass refills the tiles
    if (!__syncthreads_or(beyond)) break;
    m_ref = m_true;
    beyond = false;
  }

  // O and l are relative to m_ref; the partial reports the exact max, so its sum is
  // rescaled once (the normalised O does not change).
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  const int hq = head0 + n;   // q head of this lane's column (within the kv head's group)
  if (wave_active && hq < g) {
    const float inv = 1.f / l_run;
    const float l_true = l_run * exp2_fast((m_ref - m_true) * c);
#pragma unroll
    for (int db = 0; db < kDv / 16; ++db)
      store_unit(a, b, hq, p, direct, 16 * db + 4 * qd, o[db] * inv, m_true, l_true, db == 0 && qd == 0);
  }
}

}  // namespace

hipError_t launch_partition_latent(const PartArgs& a, int page_mode, hipStream_t s) {
  if (a.Dqk != kDqk || a.Dv != kDv || a.Hkv != 1 || a.g % kHeadsPerWave) return hipErrorInvalidValue;
  // x = partition, y = 64-head block, z = sequence: with 8 partitions the two head blocks
  // of a (sequence, partition) are 8 workgroup ids apart (same XCD under round-robin dispatch)
  dim3 grid(a.max_splits, (a.g + kHeadsPerWG - 1) / kHeadsPerWG, a.B), block(kThreads);
  const size_t lds = kQBytes;   // (the two K tiles are static)
  switch (page_mode) {
    case kContiguous:
      hipLaunchKernelGGL(partition_latent_kernel<kContiguous>, grid, block, lds, s, a);
      break;
    case kPagedAligned:
      hipLaunchKernelGGL(partition_latent_kernel<kPagedAligned>, grid, block, lds, s, a);
      break;
    default:
      hipLaunchKernelGGL(partition_latent_kernel<kPagedGeneral>, grid, block, lds, s, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace da
