// Split-K pass 1 for the latent-shared layout: one kv head whose K rows hold 576 values
// (512 non-rotary followed by 64 rotary ones, FA4Config rope_depth) and V = the first
// 512 values of each K row (FA4Config shared_kv_cols: K_nope and V share one buffer).
// Every q head of a sequence attends the same rows, so q.K and P.V are dense
// contractions (about 240 flop per byte of KV) and run on v_mfma_f32_16x16x32_bf16.
//
// Workgroup = (partition p, block of 64 q heads, sequence b); eight waves, two per SIMD.
// Each wave has two roles, one per product:
//   q.K: wave w takes the 16 heads of head block w/2 (one MFMA column block) and the 16
//       keys of key half w%2 of each 32-key tile, over the full 576-column depth:
//         S^T[key][head] = K[key][:] . q[head][:]
//       A = K from the LDS tile, B = q held in registers (18 k-steps). Its softmax needs
//       nothing from other waves: the exponentials are taken against a fixed reference
//       max (below), and the running max and sum are reduced once at the end.
//   P.V: wave w takes the 64 columns 64 w .. 64 w + 63 of V for all 64 heads:
//         O^T[d][head] += V^T[d][key] . P^T[key][head]
//       A = V^T read transposed from the same LDS tile (ds_read_b64_tr_b16); B = P^T, which
//       every wave writes to an 8 KB LDS buffer in the B-operand layout after its softmax
//       and reads back for all four head blocks after one barrier.
// Each V element is then read from LDS once per tile and workgroup, not once per head
// block, and each K element once per head block. Both roles keep a wave's fp32
// accumulators at 64 registers (16 x 256 fp32 in total per product), so two waves fit on
// each SIMD and hide each other's LDS operand latency.
// P is split hi/lo in bf16 (two MFMAs per depth block) so that the fp32 O keeps ~16
// significant bits of the weights. K tiles (32 keys x 1152 B, 16-byte chunks XOR swizzled
// within groups of 8) pass through three LDS slots: in the step for tile t, tile t - 1
// feeds P.V, tile t feeds q.K and tile t + 1 is in flight, so one barrier per tile
// suffices (P of tile t - 1 is written before it, P of tile t after it), and the first K
// operands of q.K are read while the P.V products run. (Two tiles in flight measured
// slower.) The two 64-head workgroups of a (sequence, partition) get workgroup ids 8
// apart, so they run on the same XCD and the second read of each K tile is an L2 hit.
// Epilogue as in the GQA kernel: normalised partial + (m, l) per head, or the finished
// bf16 row when the sequence has a single partition (fa4_splitk_combine_write, second
// paragraph; fa4_scale_write_output for the single-partition case).
#include "da_device.h"

namespace da {
namespace {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kTile = 32;
constexpr int kRowBytes = kDqk * 2;             // 1152
constexpr int kTileBytes = kTile * kRowBytes;   // 36 KB
constexpr int kWaves = 8;
constexpr int kHeadsPerWG = 64;                        // 4 head blocks of 16 (MFMA columns)
constexpr int kQkSteps = kDqk / 32;                    // k-steps of 32 over the q.K depth (18)
constexpr int kDvBlocks = kDv / kWaves / 16;           // 16-wide depth blocks of a wave's V slice (4)
constexpr int kThreads = kWaves * 64;
constexpr int kTileBlocks = kTileBytes / 1024;         // 1 KB direct-to-LDS loads per tile (36)
constexpr int kStage = (kTileBlocks + kWaves - 1) / kWaves;   // ... per wave, at most (5)
constexpr int kMaxLdsPages = 256;
constexpr int kRing = 3;   // K tiles in LDS: one feeds P.V, one q.K, one is in flight

typedef short s16x8 __attribute__((ext_vector_type(8)));

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
// m_ref and the accumulators are never rescaled inside the key loop. That
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
  const int kh = w & 1, hb = w >> 1;        // q.K role: key half kh of head block hb
  const int n = lane & 15, qd = lane >> 4;
  const int g = a.g;
  const int head0 = hblk * kHeadsPerWG + 16 * hb;   // first q head of the q.K role
  const float c = a.c;

  // Three K tiles. Their direct-to-LDS loads are inline assembly (lds_dma16): the compiler
  // sees no LDS write and adds no wait of its own before the LDS reads of the other tile;
  // a tile is read only after the explicit wait and barrier at the top of its step.
  __shared__ __attribute__((aligned(16))) char ktile[kRing][kTileBytes];
  // P of a tile for P.V (two buffers: tile t uses buffer t & 1), hi and lo bf16 parts per
  // head block, lane-major in the B-operand layout: lane (n, qd) reads 16 bytes, the k-slots
  // 8 qd .. 8 qd + 7 of head n, whose first 8 bytes the wave of key half 0 writes (keys
  // 4 qd .. +3) and whose last 8 the wave of key half 1 (keys 16 + 4 qd .. +3)
  __shared__ __attribute__((aligned(16))) char pbuf[2][4][2][64][16];
  // per wave and head: first-tile maxima, then the final (max, sum, reference)
  __shared__ float xm[kWaves][16], xl[kWaves][16], xr[kWaves][16];
  __shared__ int pages_s[kMaxLdsPages];

  // Rows that a ragged tile does not load keep what the slot held: zero the three slots
  // once so that such rows are finite (their scores are masked, their V meets p = 0).
  for (int i = tid; i < kRing * kTileBytes / 16; i += kThreads) *(u32x4*)(&ktile[0][0] + i * 16) = u32x4{0u, 0u, 0u, 0u};
  // q as the B operand of S^T = K q^T over the full depth, in registers for the whole
  // piece: k-step j holds depth 32 j + 8 qd .. +8 of head head0 + n (zero past the group)
  bf16x8 qf[kQkSteps];
  {
    const int h = head0 + n;
    const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)b * a.Hq + (h < g ? h : 0)) * kDqk + 8 * qd;
#pragma unroll
    for (int j = 0; j < kQkSteps; ++j) {
      u32x4 v = *(const u32x4*)(qrow + 32 * j);
      if (h >= g) v = u32x4{0u, 0u, 0u, 0u};
      qf[j] = as_bf16x8(v);
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

  // q.K role (head head0 + n, this lane's keys): reference max of the exponentials (raw
  // units), exact running max and running sum
  float m_ref = -INFINITY, m_lane = -INFINITY, l_lane = 0.f;
  bool beyond = false;       // a score exceeded m_ref by more than the headroom
  // P.V role: O^T of depth block db of this wave's 64 columns and head block hb2
  f32x4 o[kDvBlocks][4];

  // q.K operands: the A operand of k-step j is chunk 4 j + qd of row r = 16 kh + n; under
  // the swizzle that is byte 128 (j >> 1) + 16 ((4 (j & 1) + qd) ^ (r & 7)) of the row
  // (r & 7 = n & 7): two per-lane offsets, one per parity of j, and constant offsets
  const int kr = (16 * kh + n) * kRowBytes;
  const int k_even = kr + 16 * (qd ^ (n & 7)), k_odd = kr + 16 * ((4 + qd) ^ (n & 7));
  auto load_k = [&](const DA_LDS char* KL, int j) {
    return as_bf16x8(*(const DA_LDS u32x4*)(KL + (j & 1 ? k_odd : k_even) + 128 * (j >> 1)));
  };
  // P.V operands: the V^T A operand of depth 16 d + n holds keys 4 qd .. +3 and 16 + 4 qd ..
  // +3 (the k-slot order of the P buffer); depth block d = 4 w + db is chunk 2 d + ((n & 3)
  // >> 1) of rows ra and ra + 16, under the swizzle byte 128 (d >> 2) + 16 ((2 (d & 3) +
  // ((n & 3) >> 1)) ^ (ra & 7)) of the row (d >> 2 = w, d & 3 = db)
  const int ra = 4 * qd + (n >> 2);
  const int v_off = ra * kRowBytes + (n & 1) * 8 + 128 * w;
  auto load_v = [&](const DA_LDS char* KL, int db) {
    const DA_LDS char* pa = KL + v_off + 16 * ((2 * db + ((n & 3) >> 1)) ^ (ra & 7));
    const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 DA_LDS*)pa);
    const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 DA_LDS*)(pa + 16 * kRowBytes));
    s16x8 v8;
    v8[0] = va[0]; v8[1] = va[1]; v8[2] = va[2]; v8[3] = va[3];
    v8[4] = vb[0]; v8[5] = vb[1]; v8[6] = vb[2]; v8[7] = vb[3];
    return __builtin_bit_cast(bf16x8, v8);
  };
  // K operands of q.K issued ahead of their products; the first kEarly of them go out
  // during the P.V products of the tile before, so that their latency hides behind those
  // (not with per-lane page lookups: that form, for page sizes that are not a power of two
  // >= 32 keys, already spills about 10 registers)
  constexpr int kEarly = PM == kPagedGeneral ? 0 : 4;
  constexpr int kQkAhead = 8;

  const int n_tiles = (end - start + kTile - 1) / kTile;
  // Step it: P.V of tile it - 1 (its P is in buffer (it - 1) & 1 since the barrier before),
  // then q.K and the softmax of tile it, whose P goes to buffer it & 1.
  auto step = [&](int it, bool first) {
    const bool has_pv = it >= 1, has_qk = it < n_tiles;
    const DA_LDS char* KQ = (const DA_LDS char*)ktile[it % kRing];
    const DA_LDS char* KV = (const DA_LDS char*)ktile[(it + kRing - 1) % kRing];
    bf16x8 kf[kQkSteps];
    if (has_pv) {
      bf16x8 vf[kDvBlocks], ph[4], pl[4];
#pragma unroll
      for (int db = 0; db < kDvBlocks; ++db) vf[db] = load_v(KV, db);
#pragma unroll
      for (int hb2 = 0; hb2 < 4; ++hb2) {
        ph[hb2] = as_bf16x8(*(const u32x4*)&pbuf[(it - 1) & 1][hb2][0][lane][0]);
        pl[hb2] = as_bf16x8(*(const u32x4*)&pbuf[(it - 1) & 1][hb2][1][lane][0]);
      }
      if (has_qk) {
#pragma unroll
        for (int j = 0; j < kEarly; ++j) kf[j] = load_k(KQ, j);
      }
      __builtin_amdgcn_sched_barrier(0);
      // the wave's issue priority is raised for its products, so that where the two waves of
      // a SIMD are in different phases the one with matrix-core work issues first
      __builtin_amdgcn_s_setprio(1);
      // O^T += V^T P^T for the wave's 4 depth blocks and all 4 head blocks: head block by
      // head block, the hi products of the 4 depth blocks, then their lo products, so that
      // no product waits for the one just before it
#pragma unroll
      for (int hb2 = 0; hb2 < 4; ++hb2) {
#pragma unroll
        for (int db = 0; db < kDvBlocks; ++db)
          o[db][hb2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], ph[hb2], o[db][hb2], 0, 0, 0);
#pragma unroll
        for (int db = 0; db < kDvBlocks; ++db)
          o[db][hb2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], pl[hb2], o[db][hb2], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
    } else {
#pragma unroll
      for (int j = 0; j < kEarly; ++j) kf[j] = load_k(KQ, j);
    }
    if (!has_qk) return;
    // S^T over the full q.K depth for keys 16 kh + 4 qd + i of head n; even and odd k-steps
    // accumulate apart, two independent chains of products
    const int t0 = start + it * kTile;
#pragma unroll
    for (int j = kEarly; j < kQkAhead; ++j) kf[j] = load_k(KQ, j);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kQkSteps; j += 2) {
      if (j + kQkAhead < kQkSteps) kf[j + kQkAhead] = load_k(KQ, j + kQkAhead);
      if (j + 1 + kQkAhead < kQkSteps) kf[j + 1 + kQkAhead] = load_k(KQ, j + 1 + kQkAhead);
      __builtin_amdgcn_sched_barrier(0);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[j], qf[j], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[j + 1], qf[j + 1], s1, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    f32x4 sc = s0 + s1;
    // keys past the end of a ragged tile get -inf (p = 0)
    if (end - t0 < kTile) {
      const int nvalid = end - t0 - 16 * kh - 4 * qd;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i >= nvalid) sc[i] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    m_lane = fmaxf(m_lane, mx);
    if (first) {
      // the reference of the first pass: the first tile's max over both key halves (O and
      // l are still 0); one exchange per pass, the other tiles need no cross-lane step
      mx = max_over_key_groups(mx);
      if (qd == 0) xm[w][n] = mx;
      __syncthreads();
      m_ref = fmaxf(mx, xm[w ^ 1][n]);
    }
    beyond = beyond || (mx - m_ref) * c > kHeadroomLog2;
    const float mc = m_ref * c;
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = exp2_fast(fmaf(sc[i], c, -mc));
      l_lane += pr[i];
    }
    // hi and lo parts of P into the buffer (8 bytes each per lane)
    const uint32_t h0 = pack_bf16x2(pr[0], pr[1]), h1 = pack_bf16x2(pr[2], pr[3]);
    const uint32_t l0 = pack_bf16x2(pr[0] - bf16lo(h0), pr[1] - bf16hi(h0));
    const uint32_t l1 = pack_bf16x2(pr[2] - bf16lo(h1), pr[3] - bf16hi(h1));
    *(u32x2*)&pbuf[it & 1][hb][0][lane][8 * kh] = u32x2{h0, h1};
    *(u32x2*)&pbuf[it & 1][hb][1][lane][8 * kh] = u32x2{l0, l1};
  };

  // Three K tiles: during step it, tile it - 1 feeds P.V, tile it feeds q.K and tile it + 1
  // is in flight (requested right after the barrier that retires tile it - 2). One barrier
  // per tile. A second pass runs only if some score left the headroom of m_ref (then
  // m_ref = the exact max: no second miss).
  for (int pass = 0; pass < 2; ++pass) {
    l_lane = 0.f;
#pragma unroll
    for (int db = 0; db < kDvBlocks; ++db)
#pragma unroll
      for (int hb2 = 0; hb2 < 4; ++hb2) o[db][hb2] = f32x4{0.f, 0.f, 0.f, 0.f};
    issue(ktile[0], start);
    for (int it = 0; it <= n_tiles; ++it) {
      wait_vm<0>();      // this wave's part of tile it is in LDS (none is in flight at the end)
      __syncthreads();   // ... and every wave's; P of tile it - 1 is written; tile it - 2 and
                         // the P buffer of tile it - 2 are retired
      if (it + 1 < n_tiles) issue(ktile[(it + 1) % kRing], start + (it + 1) * kTile);
      step(it, pass == 0 && it == 0);
    }
    // every wave is past its last LDS read before a second pass refills the tiles
    if (!__syncthreads_or(beyond)) break;
    // second pass: the reference is each head's exact max over the partition
    const float mt = max_over_key_groups(m_lane);
    if (qd == 0) xm[w][n] = mt;
    __syncthreads();
    m_ref = fmaxf(mt, xm[w ^ 1][n]);
    beyond = false;
    __syncthreads();   // (xm is written again before it is next read)
  }

  // (max, sum) per head: the q.K role reduces this wave's over its key groups and publishes
  // it; the P.V role reads those of the heads it holds. O and l are relative to m_ref; the
  // partial reports the exact max, so its sum is rescaled once (the normalised O does not
  // change).
  {
    const float mt = max_over_key_groups(m_lane);
    float l = l_lane;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (qd == 0) {
      xm[w][n] = mt;
      xl[w][n] = l;
      xr[w][n] = m_ref;
    }
  }
  __syncthreads();
#pragma unroll
  for (int hb2 = 0; hb2 < 4; ++hb2) {
    const int hq = hblk * kHeadsPerWG + 16 * hb2 + n;   // q head of this lane's column
    if (hq < g) {
      const float M = fmaxf(xm[2 * hb2][n], xm[2 * hb2 + 1][n]);
      const float L = xl[2 * hb2][n] + xl[2 * hb2 + 1][n];   // both halves share m_ref
      const float inv = 1.f / L;
      const float l_true = L * exp2_fast((xr[2 * hb2][n] - M) * c);
#pragma unroll
      for (int db = 0; db < kDvBlocks; ++db)
        store_unit(a, b, hq, p, direct, 64 * w + 16 * db + 4 * qd, o[db][hb2] * inv, M, l_true,
                   w == 0 && db == 0 && qd == 0);
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
