// Split-K pass 1 for the latent-shared layout: one kv head whose K rows hold 576 values
// (512 non-rotary followed by 64 rotary ones, FA4Config rope_depth) and V = the first
// 512 values of each K row (FA4Config shared_kv_cols: K_nope and V share one buffer).
// Every q head of a sequence attends the same rows, so q.K and P.V are dense
// contractions (about 240 flop per byte of KV) and run on v_mfma_f32_16x16x32_bf16.
//
// Workgroup = (partition p, block of 64 q heads, sequence b); eight waves, two per SIMD.
// Wave w owns the 16 heads of head block w/2 (one MFMA column block) and depth half w%2
// of both products:
//   S^T[key][head] partial = K[key][288h : 288h+288] . q[head][288h : 288h+288]
//       A = K from the LDS tile, B = q held in registers (9 k-steps); the two waves of a
//       pair add their partials through a 2 KB-per-wave LDS exchange, so both hold the
//       full scores and take the same softmax
//   O^T[d][head] += V^T[d][key] . P^T[key][head]   for d in depth half w%2 of V (256)
//       A = V^T read transposed from the same LDS tile (ds_read_b64_tr_b16); B = P^T from
//       the score registers
// Splitting both products by depth halves the fp32 accumulators a wave holds (64
// registers for 16 heads x 256 columns), so that two waves fit on each SIMD and hide each
// other's LDS operand latency; with one wave per SIMD the operand reads, not the matrix
// cores, set the pace.
// P is split hi/lo in bf16 (two MFMAs per depth block) so that the fp32 O keeps ~16
// significant bits of the weights. The K tile (32 keys x 1152 B, 16-byte chunks XOR
// swizzled within groups of 8) is double-buffered in LDS: the next tile's direct-to-LDS
// loads are in flight while the current tile is computed (a third buffer, two tiles in
// flight, measured slower). The two head blocks of a
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
// MFMA column blocks (16 heads) per wave: each K / V operand read serves all of them, at
// 64 accumulator registers each. Two blocks leave room for one wave per SIMD only, and
// measured no faster.
constexpr int kCB = 1;
constexpr int kHeadsPerWave = 16 * kCB;
constexpr int kWaves = 8;                             // 4 head blocks x 2 depth halves
constexpr int kHeadsPerWG = kHeadsPerWave * kWaves / 2;   // 64
constexpr int kQkSteps = kDqk / 2 / 32;               // k-steps of 32 per depth half of q.K (9)
constexpr int kDvBlocks = kDv / 2 / 16;               // 16-wide depth blocks per half of V (16)
constexpr int kThreads = kWaves * 64;
constexpr int kTileBlocks = kTileBytes / 1024;         // 1 KB direct-to-LDS loads per tile (36)
constexpr int kStage = (kTileBlocks + kWaves - 1) / kWaves;   // ... per wave, at most (5)
constexpr int kMaxLdsPages = 256;
constexpr int kRing = 2;   // K tiles in LDS: one in flight while the other is computed

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
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void partition_latent_kernel(PartArgs a) {
  const int p = blockIdx.x, hblk = blockIdx.y, b = blockIdx.z;
  const int L = __builtin_amdgcn_readfirstlane(attended_len(a, b, PM == kContiguous));
  const int start = p * a.chunk;
  if (start >= L) return;
  const int end = min(start + a.chunk, L);
  const int P_b = min((L + a.chunk - 1) / a.chunk, a.max_splits);
  const bool direct = a.direct_single && P_b == 1;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int dh = w & 1;                      // depth half of q.K and of V
  const int n = lane & 15, qd = lane >> 4;
  const int g = a.g;
  const int head0 = hblk * kHeadsPerWG + (w >> 1) * kHeadsPerWave;   // first q head of this wave
  const float c = a.c;

  // Two K tiles. Their direct-to-LDS loads are inline assembly (lds_dma16): the compiler
  // sees no LDS write and adds no wait of its own before the LDS reads of the other tile;
  // a tile is read only after the explicit wait and barrier at the top of its step.
  __shared__ __attribute__((aligned(16))) char ktile[kRing][kTileBytes];
  // partial scores of each wave, lane-major (8 floats per lane and column block), read by
  // its partner
  __shared__ __attribute__((aligned(16))) f32x4 xchg[kWaves][2 * kCB][64];
  __shared__ int pages_s[kMaxLdsPages];

  // Rows that a ragged tile does not load keep what the buffer held: zero both tiles
  // once so that such rows are finite (their scores are masked, their V meets p = 0).
  for (int i = tid; i < kRing * kTileBytes / 16; i += kThreads) *(u32x4*)(&ktile[0][0] + i * 16) = u32x4{0u, 0u, 0u, 0u};
  // q as the B operand of S^T = K q^T, in registers for the wave's whole piece: column
  // block cb, k-step j holds depth 288 dh + 32 j + 8 qd .. +8 of head head0 + 16 cb + n
  // (zero past the group)
  bf16x8 qf[kCB][kQkSteps];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    const int h = head0 + 16 * cb + n;
    const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)b * a.Hq + (h < g ? h : 0)) * kDqk + 288 * dh + 8 * qd;
#pragma unroll
    for (int j = 0; j < kQkSteps; ++j) {
      u32x4 v = *(const u32x4*)(qrow + 32 * j);
      if (h >= g) v = u32x4{0u, 0u, 0u, 0u};
      qf[cb][j] = as_bf16x8(v);
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
  // fills the 1 KB blocks w, w+8, ..., so lane l of block j writes tile byte j*1024 + 16l,
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
      const u32x4 rk = rsrc_words(kc + row0 * kRowBytes, (uint32_t)(rows * kRowBytes));
      const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_addr(dst) + w * 1024);
#pragma unroll
      for (int i = 0; i < kStage; ++i) {
        if (w + kWaves * i >= kTileBlocks) break;   // (uniform: the tile has 36 blocks of 1 KB)
        int r, gc;
        lane_chunk(i, r, gc);
        lds_dma16(rk, (uint32_t)(r * kRowBytes + gc * 16), lb + kWaves * 1024 * i);
      }
    } else {
      // any page size: every lane looks up its own row (rows past the end repeat the
      // last key; their scores are masked)
#pragma unroll
      for (int i = 0; i < kStage; ++i) {
        if (w + kWaves * i >= kTileBlocks) break;
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

  // per column block cb: reference max of the exponentials (raw units), exact running
  // max, running sum (this lane's keys)
  float m_ref[kCB], m_true[kCB], l_run[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    m_ref[cb] = -INFINITY;
    m_true[cb] = -INFINITY;
    l_run[cb] = 0.f;
  }
  bool beyond = false;       // a score exceeded m_ref by more than the headroom
  f32x4 o[kCB][kDvBlocks];

  auto compute = [&](const char* K, int t0) {
    // S^T partial over this wave's depth half: keys 16 blk + (4qd..+3) of column n of
    // column block cb; each K operand serves every column block
    // (k-step j of depth half dh is chunk 4 jj + qd, jj = 9 dh + j, of row r; under the
    // swizzle that is byte 128 (jj >> 1) + 16 ((4 (jj & 1) + qd) ^ (r & 7)) of the row, so
    // two per-lane bases per row, one per parity of jj, and constant offsets cover all
    // k-steps)
    f32x4 s[kCB][2];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) s[cb][blk] = f32x4{0.f, 0.f, 0.f, 0.f};
    const DA_LDS char* KL = (const DA_LDS char*)K;
    // k-step j = 2m (even) of depth half dh reads from pe + 128 m, j = 2m + 1 from po + 128 m
    const int kr = n * kRowBytes;   // row n of key block 0; block 1 is 16 rows on
    const DA_LDS char* pe = KL + kr + 16 * ((4 * dh + qd) ^ (n & 7)) + 512 * dh;
    const DA_LDS char* po = KL + kr + 16 * ((4 * (1 - dh) + qd) ^ (n & 7)) + 640 * dh;
    bf16x8 kf[kQkSteps][2];
#pragma unroll
    for (int j = 0; j < kQkSteps; ++j)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
        kf[j][blk] = as_bf16x8(*(const DA_LDS u32x4*)((j & 1 ? po : pe) + 128 * (j >> 1) + 16 * blk * kRowBytes));
    // (all 18 operand reads are issued before the first product)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kQkSteps; ++j)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb)
          s[cb][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[j][blk], qf[cb][j], s[cb][blk], 0, 0, 0);
    // the partner wave (other depth half, same heads) adds its partial: both waves then
    // hold the full scores. A wave rewrites its slot only after the next tile's barrier,
    // which its partner passes after reading it.
#pragma unroll
    for (int k = 0; k < 2 * kCB; ++k) xchg[w][k][lane] = s[k >> 1][k & 1];
    __syncthreads();
    f32x4 sp[2 * kCB];
#pragma unroll
    for (int k = 0; k < 2 * kCB; ++k) sp[k] = xchg[w ^ 1][k][lane];
    // O^T += V^T P^T over this wave's depth half; V^T A operand: depth 16 db + n of keys
    // 4qd..+3 and 16+4qd..+3, shared by every column block. Depth block d = 16 dh + db is
    // chunk 2d + ((n & 3) >> 1) of rows ra and rb = ra + 16; under the swizzle that is byte
    // 128 (d >> 2) + 16 ((2 (d & 3) + ((n & 3) >> 1)) ^ (ra & 7)) of the row (rb & 7 =
    // ra & 7): four per-lane bases and constant offsets
    const int ra = 4 * qd + (n >> 2);
    const int sub = (n & 1) * 8;
    const DA_LDS char* vbase[4];
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4)
      vbase[v4] = KL + ra * kRowBytes + 16 * ((2 * v4 + ((n & 3) >> 1)) ^ (ra & 7)) + sub + 128 * 4 * dh;
    auto load_v = [&](int db) {
      const DA_LDS char* pa = vbase[db & 3] + 128 * (db >> 2);
      const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 DA_LDS*)pa);
      const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 DA_LDS*)(pa + 16 * kRowBytes));
      s16x8 v8;
      v8[0] = va[0]; v8[1] = va[1]; v8[2] = va[2]; v8[3] = va[3];
      v8[4] = vb[0]; v8[5] = vb[1]; v8[6] = vb[2]; v8[7] = vb[3];
      return __builtin_bit_cast(bf16x8, v8);
    };
    // the first V^T operands are requested before the softmax, the rest kAhead depth
    // blocks ahead of their products (the scheduling barriers keep that order)
    constexpr int kAhead = 6;
    bf16x8 vf[kDvBlocks];
#pragma unroll
    for (int db = 0; db < kAhead; ++db) vf[db] = load_v(db);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 2 * kCB; ++k) s[k >> 1][k & 1] += sp[k];
    // online softmax (missing keys of a ragged tile get -inf, i.e. p = 0)
    const int nvalid = end - t0;
    if (nvalid < kTile) {
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * blk + 4 * qd + i >= nvalid) s[cb][blk][i] = -INFINITY;
    }
    bf16x8 pb_hi[kCB], pb_lo[kCB];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const f32x4* sc = s[cb];
      float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                       fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
      mx = max_over_key_groups(mx);
      m_true[cb] = fmaxf(m_true[cb], mx);
      m_ref[cb] = m_ref[cb] == -INFINITY ? mx : m_ref[cb];   // first tile of the pass: O and l are still 0
      beyond = beyond || (mx - m_ref[cb]) * c > kHeadroomLog2;
      const float mc = m_ref[cb] * c;
      float pr[2][4];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[blk][i] = exp2_fast(fmaf(sc[blk][i], c, -mc));
          l_run[cb] += pr[blk][i];
        }
      // P^T (B operand), hi and lo parts
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const int blk = s2 >> 1, i0 = (s2 & 1) * 2;
        const float p0 = pr[blk][i0], p1 = pr[blk][i0 + 1];
        const uint32_t hv = pack_bf16x2(p0, p1);
        hw[s2] = hv;
        lw[s2] = pack_bf16x2(p0 - bf16lo(hv), p1 - bf16hi(hv));
      }
      pb_hi[cb] = as_bf16x8(u32x4{hw[0], hw[1], hw[2], hw[3]});
      pb_lo[cb] = as_bf16x8(u32x4{lw[0], lw[1], lw[2], lw[3]});
    }
#pragma unroll
    for (int db = 0; db < kDvBlocks; ++db) {
      if (db + kAhead < kDvBlocks) vf[db + kAhead] = load_v(db + kAhead);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        o[cb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], pb_hi[cb], o[cb][db], 0, 0, 0);
        o[cb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], pb_lo[cb], o[cb][db], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Double buffer: tile it+1 is requested right after the barrier that retires tile it-1
  // from the other buffer, and lands while tile it is computed. A second pass runs only
  // if some score left the headroom of m_ref (then m_ref = the exact max: no second miss).
  const int n_tiles = (end - start + kTile - 1) / kTile;
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      l_run[cb] = 0.f;
#pragma unroll
      for (int db = 0; db < kDvBlocks; ++db) o[cb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    issue(ktile[0], start);
    for (int it = 0; it < n_tiles; ++it) {
      wait_vm<0>();      // this wave's part of tile it is in LDS
      __syncthreads();   // ... and every wave's; tile it-1 is retired (its reads have returned)
      if (it + 1 < n_tiles) issue(ktile[(it + 1) & 1], start + (it + 1) * kTile);
      compute(ktile[it & 1], start + it * kTile);
    }
    // every wave is past its last LDS read before a second pass refills the tiles
    if (!__syncthreads_or(beyond)) break;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) m_ref[cb] = m_true[cb];
    beyond = false;
  }

  // O and l are relative to m_ref; the partial reports the exact max, so its sum is
  // rescaled once (the normalised O does not change). Both waves of a pair hold the
  // same (m, l): the depth-half-0 wave writes them.
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    float l = l_run[cb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int hq = head0 + 16 * cb + n;   // q head of this lane's column (within the kv head's group)
    if (hq < g) {
      const float inv = 1.f / l;
      const float l_true = l * exp2_fast((m_ref[cb] - m_true[cb]) * c);
#pragma unroll
      for (int db = 0; db < kDvBlocks; ++db)
        store_unit(a, b, hq, p, direct, 256 * dh + 16 * db + 4 * qd, o[cb][db] * inv, m_true[cb], l_true,
                   db == 0 && qd == 0 && dh == 0);
    }
  }
}

}  // namespace

hipError_t launch_partition_latent(const PartArgs& a, int page_mode, hipStream_t s) {
  if (a.Dqk != kDqk || a.Dv != kDv || a.Hkv != 1 || a.g % 16) return hipErrorInvalidValue;
  // x = partition, y = 64-head block, z = sequence: with 8 partitions the two head blocks
  // of a (sequence, partition) are 8 workgroup ids apart (same XCD under round-robin dispatch)
  dim3 grid(a.max_splits, (a.g + kHeadsPerWG - 1) / kHeadsPerWG, a.B), block(kThreads);
  const size_t lds = 0;   // (the K tiles and the exchange are static)
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
