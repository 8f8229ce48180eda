// Split-K pass 1 when one kv head serves every q head of a sequence (FA4Config,
// use_shared_kv / shared_kv_cols: MLA-style latent attention, where V is the first ov_depth
// columns of each K row, and one-kv-head attention with a V of its own whose depth need not
// equal the nope depth, as FA4Config's with_splitk keeps for GLM-style configs, or, at
// depth 128, multi-query attention). Every q head reads the same K and V rows, so q.K and
// P.V are dense contractions (about 200 flop per byte of KV for the latent form) and run on
// v_mfma_f32_16x16x32_bf16.
//
// A K row is [nope columns | rotary columns] (FA4Config, rope_depth = q.K depth minus the
// nope depth); the rotary columns sit in the K rows or in a tensor of their own (bf16,
// FA4Config rope_dtype). The kernel only sees two column ranges with their own base and row
// stride, so both forms run the same code (a shape without rotary columns has an empty
// second range).
//
// Workgroup = (partition p, block of 64 (query, head) columns, sequence b): eight waves,
// two per SIMD, with one role each:
//   waves 0-3, q.K and the softmax: wave w takes the 32 columns 32 (w/2) .. +31 (two MFMA
//       column blocks, q in registers over the full q.K depth) and the 16 keys of key half
//       w%2 of each 32-key tile. Every K operand read from LDS feeds two products. Its
//       softmax needs nothing from other waves: the exponentials are taken against a fixed
//       reference max (below). The probabilities go to LDS, split hi/lo in bf16, in the
//       B-operand layout of P.V.
//   waves 4-7, P.V: wave 4+v takes the V columns DV/4 v .. +DV/4-1 for all 64 columns
//       (O^T in registers), reading V^T transposed from the LDS tile (ds_read_b64_tr_b16)
//       and P from LDS.
// Each SIMD thus holds one wave of each role: the softmax arithmetic of the one runs beside
// the matrix-core products of the other instead of both waves stalling in the same phase.
// Per 32-key tile and workgroup the LDS carries the tile once (direct-to-LDS loads), K
// twice (two column pairs), V once, and P (8 KB) four times.
//
// Tiles pass through a ring of four LDS slots: in step s the q.K waves work on tile s, the
// P.V waves on tile s - 1, and tiles s + 1 and s + 2 are in flight (their loads issued by
// the q.K waves, so that the P.V waves keep to their products); one barrier per step. P
// is double-buffered. (Four slots of the latent tile and the two P buffers fill the 160 KB
// of LDS exactly: the page indices live in registers and the exchange arrays in a P buffer.
// With one tile in flight a step waits for its whole tile, and a load-only copy streams at
// about 2.8 TB/s.)
//
// P must not be rounded to bf16 before P.V (the fp32 O must stay within 1e-5), so it is
// split as p = hi + lo, hi = bf16(p), lo = bf16(p - hi), and P.V runs both halves.
//
// Fixed reference max: the exponentials are taken relative to a per-column reference m_ref
// (the first tile's max) and O is never rescaled inside the key loop. That holds while every
// score stays within kHeadroomLog2 powers of two of m_ref; a score beyond that (adversarial
// logits) makes the workgroup run its partition once more with m_ref = the partition's exact
// max, which the q.K waves track on the side.
//
// Epilogue as in the GQA kernel: normalised partial + (m, l) per column, or the finished
// bf16 row when the sequence has a single partition (fa4_splitk_combine_write, second
// paragraph).
#include "da_device.h"

namespace da {
namespace {

constexpr int kTile = 32;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kCols = 64;                 // (query, head) columns of a workgroup: 4 MFMA blocks of 16
constexpr int kMaxLdsPages = 256;
constexpr int kLdsBytes = 160 * 1024;
constexpr float kHeadroomLog2 = 64.f;

typedef short s16x8 __attribute__((ext_vector_type(8)));

// Depths of one instantiation: DN nope columns and DR rotary columns make the q.K depth; V
// has DV columns and is either the first DV nope columns (SHARED) or a cache of its own.
// F8: the nope columns (and a V of its own) are E4M3 codes with per-token scales; the rotary
// columns stay bf16, stored apart, or (RF8) are codes in the K rows, scaled with them. A V that
// is a prefix of the nope columns is read as code x the token's K scale, a V of its own as
// code x its V scale.
template <int DN_, int DR_, int DV_, bool SHARED_, bool F8_ = false, bool RF8_ = false>
struct SShape {
  static constexpr int DN = DN_, DR = DR_, DV = DV_;
  static constexpr bool SHARED = SHARED_, F8 = F8_, RF8 = RF8_;
  static constexpr int DQK = DN + DR;
  static constexpr int NJ = DQK / 32;            // 32-deep k-steps of q.K
  static constexpr int NJN = DN / 32;            // ... over the nope columns
  static constexpr int kElt = F8 ? 1 : 2;        // bytes per cached nope / V element
  static constexpr int kNRow = DN * kElt;        // LDS bytes of one row, per region
  static constexpr int kRRow = DR * (RF8 ? 1 : 2);
  static constexpr int kVSrcRow = DV * kElt;     // ... of the V region (a V of its own)
  static constexpr int kVCols = DV / 4;          // V columns of one P.V wave
  static constexpr int kDB = kVCols / 16;        // its 16-deep O blocks
  // rows of the tile that the transposing V reads see: the nope rows (bf16, SHARED), the V
  // rows of its own, or (F8) the wave's own bf16 copy of its V columns
  static constexpr int kVRow = F8 ? kVCols * 2 : (SHARED ? DN * 2 : DV * 2);
  static constexpr int kNBytes = kTile * kNRow;  // region offsets inside a slot
  static constexpr int kRBytes = kTile * kRRow;
  static constexpr int kVOff = SHARED ? 0 : kNBytes + kRBytes;
  static constexpr int kVReadOff = F8 ? 0 : kVOff;   // the V rows the transposing reads see
  static constexpr int kScOff = kNBytes + kRBytes + (SHARED ? 0 : kTile * kVSrcRow);   // F8: K scales
  static constexpr int kVScOff = kScOff + 1024;                                         // F8, own V: V scales
  static constexpr int kSlot = kScOff + (F8 ? (SHARED ? 1024 : 2048) : 0);
  static constexpr int kBlocks = kSlot / 1024;   // 1 KB direct-to-LDS loads per tile
  // the tile's loads are issued by the four q.K waves (the P.V waves, with the most
  // matrix-core work per tile, only consume): 61.0 against 63.5 us on the latent workload
  static constexpr int kDmaWaves = 4;
  static constexpr int kPerWave = (kBlocks + kDmaWaves - 1) / kDmaWaves;
  static_assert(NJ % 2 == 0 && DN % 64 == 0 && DR % 64 == 0 && DV % 64 == 0, "depths");
  static_assert(kNBytes % 1024 == 0 && kRBytes % 1024 == 0 && kSlot % 1024 == 0, "1 KB load blocks");
  static_assert((16 * kNRow) % 1024 == 0 && (16 * kRRow) % 1024 == 0 && (16 * kVSrcRow) % 1024 == 0,
                "16 rows of a region are whole load blocks");
  static_assert(!SHARED || DV <= DN, "a shared V is a prefix of the nope columns");
  static_assert(!RF8 || F8, "rotary codes come with an fp8 cache");
  static_assert(!F8 || (SHARED && DN == 512) || (!SHARED && DN == 192 && DV == 256),
                "fp8: the latent form, or nope 192 with a V of 256 of its own");
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// max over the four lanes n, n+16, n+32, n+48 on the VALU (v_permlane16/32_swap), keeping
// the LDS permute unit free for the tile's operands. Written out because the compiler folds
// the two results of a swap of a value with itself into one; the s_nop gives the two wait
// states a VALU write needs before a permlane reads it.
__device__ __forceinline__ float max_over_key_groups(float v) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  v = fmaxf(a, b);
  a = v;
  b = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}

constexpr int kPBytes = 4 * 2 * 64 * 16;   // P of one tile: 4 column blocks x (hi, lo) x 64 lanes x 16 B

// Per q.K wave, column block of its pair and column: maxima, sums, reference maxima; and one
// flag per wave for the block-wide "any". They live in P buffer 1 whenever no P is live there.
struct XArrays {
  float xm[4][2][16], xl[4][2][16], xr[4][2][16];
  int any[kWaves];
};
static_assert(sizeof(XArrays) <= kPBytes, "exchange arrays fit a P buffer");

// XOR swizzle of the 16-byte chunks of a tile row, chosen per region from its row stride so
// that the operand reads hit 16 different 16-byte bank groups (the LDS serves 256 bytes per
// clock: 64 banks of 4 bytes). Physical chunk = logical chunk ^ swz(row), its own inverse.
//  - rows of a multiple of 256 bytes (latent nope 1024, V 512): the K reads take one chunk
//    of 16 consecutive rows, the transposing V reads two adjacent chunks of 8 rows, so
//    swz(r) = 2 (r & 7) + ((r >> 3) & 1) (16 distinct values over 16 rows, whose halves are
//    distinct over 8 rows); the XOR spans 16-chunk groups.
//  - rows of 128 bytes mod 256 (rotary 128, GLM nope 384): consecutive rows alternate bank
//    halves, so swz(r) = (r >> 1) & 7; the XOR stays within 8-chunk groups.
//  - rows of 192 bytes (GLM nope as fp8 codes): not swizzled. The stride is 48 banks, so
//    16 rows fall on 4 bank phases: their 8-byte operand reads conflict four ways (six such
//    reads per tile and wave, a few dozen clocks). Rows of 64 bytes (rotary columns as fp8
//    codes in the K rows) likewise: a four-way conflict on two reads per tile and wave.
template <int RB>
__device__ __forceinline__ int swz(int r) {
  if constexpr (RB == 192 || RB == 64) return 0;
  static_assert(RB == 192 || RB == 64 || RB % 256 == 0 || RB % 256 == 128,
                "row strides of 128 + 256 k, 256 k, 192 or 64 bytes");
  if constexpr (RB % 256 == 0) return ((r & 7) << 1) | ((r >> 3) & 1);
  else return (r >> 1) & 7;
}

template <class S, int R>
struct SmemBase {
  char tile[R][S::kSlot];
  // P of a tile for P.V (tile s uses buffer s & 1): hi and lo bf16 parts per column block in
  // the B-operand layout, [4 column blocks][hi, lo][key half][64 lanes][8 bytes]. Lane (n, qd)
  // reads the k-slots 8 qd .. 8 qd + 7 of column n: the 8 bytes of key half 0 (keys 4 qd .. +3)
  // and the 8 bytes of key half 1 (keys 16 + 4 qd .. +3), one ds_read2_b64; each key half's
  // wave writes its 8 bytes per lane contiguously (no bank conflicts either way).
  char pbuf[2][kPBytes];
};
// F8: each P.V wave's bf16 copy of its V columns of the tile it consumes (32 rows of
// kVRow bytes, chunks swizzled for the transposing reads)
template <class S, bool F8 = S::F8>
struct VPriv {};
template <class S>
struct VPriv<S, true> {
  char vpriv[4][kTile * S::kVRow];
};
template <class S, int R, bool LDS_PAGES>
struct SharedSmem : SmemBase<S, R>, VPriv<S> {};
template <class S, int R>
struct SharedSmem<S, R, true> : SmemBase<S, R>, VPriv<S> {
  int pages[kMaxLdsPages];   // page indices of the partition (per-key page lookup)
};

// Ring depth: R tiles in LDS, of which R - 2 are in flight (one feeds q.K, one P.V). With a
// power-of-two page size or a contiguous cache the page indices live in registers and four
// slots fit (two tiles in flight); the per-key page lookup keeps its indices in LDS and
// three slots.
template <int PM>
constexpr int ring_of() { return PM == kPagedGeneral ? 3 : 4; }

template <class S, int PM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void partition_shared_kernel(PartArgs a, const char* rope_base, uint32_t rope_row_bytes) {
  constexpr int R = ring_of<PM>();
  constexpr int A = R - 2;                      // tiles in flight
  constexpr bool kLdsPages = PM == kPagedGeneral;
  typedef SharedSmem<S, R, kLdsPages> Smem;
  static_assert(sizeof(Smem) <= kLdsBytes, "LDS budget");
  __shared__ __attribute__((aligned(16))) Smem sm;
  XArrays& xa = *(XArrays*)sm.pbuf[1];

  const int p = blockIdx.x, cblk = blockIdx.y, b = blockIdx.z;
  const int L = __builtin_amdgcn_readfirstlane(attended_len(a, b, PM == kContiguous));
  const int start = p * a.chunk;
  if (start >= L) {
    // fused combine: the rows of a sequence without keys (O = 0, LSE = -inf) come from its
    // first workgroup of each column block
    if (a.counters && p == 0 && L == 0) {
      constexpr int kUnits = S::DV / 4;
      const int nrow = min(kCols, a.Hq - cblk * kCols);
      for (int u = threadIdx.x; u < nrow * kUnits; u += kThreads)
        write_row_unit(a.out, a.o32, a.lse, (int64_t)b * a.Hq + cblk * kCols + u / kUnits, S::DV, (u % kUnits) * 4,
                       -INFINITY, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}, a.scale);
    }
    return;
  }
  const int end = min(start + a.chunk, L);
  const int P_b = min((L + a.chunk - 1) / a.chunk, a.max_splits);
  const bool direct = a.direct_single && P_b == 1;
  const int ncols = a.Hq;                      // rows of the sequence = (query, head) columns
  const int col0 = cblk * kCols;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, qd = lane >> 4;
  const float c = a.c;
  const int n_tiles = (end - start + kTile - 1) / kTile;

  // A ragged tile's rows past the end are not loaded and keep what the slot held; they
  // must be finite (their scores are masked, their V meets p = 0). A slot that a partition
  // of more than R tiles reuses holds an earlier full tile; shorter partitions zero the
  // slots first.
  if (n_tiles <= R)
    for (int i = tid; i < R * S::kSlot / 16; i += kThreads) *(u32x4*)(&sm.tile[0][0] + i * 16) = u32x4{0u, 0u, 0u, 0u};
  int first_page = 0;
  // page indices of the partition (at most kMaxLdsPages): in LDS for the per-key lookup, else
  // lane l of register k holds page first_page + 64 k + l
  int pg[kMaxLdsPages / 64];
  if constexpr (PM != kContiguous) {
    first_page = start / a.page_size;
    const int n_pages = (end - 1) / a.page_size - first_page + 1;
    const int32_t* pt = a.page_table + (int64_t)b * a.pt_stride + first_page;
    if constexpr (kLdsPages) {
      for (int i = tid; i < n_pages && i < kMaxLdsPages; i += kThreads) {
        const int page = pt[i];
        sm.pages[i] = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
      }
    } else {
#pragma unroll
      for (int k = 0; k < kMaxLdsPages / 64; ++k) {
        const int i = 64 * k + lane;
        const int page = i < n_pages ? pt[i] : 0;
        pg[k] = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
      }
    }
  }
  __syncthreads();

  // The tile of keys t0 .. t0 + 31 lands in LDS by direct-to-LDS 16-byte loads: 1 KB block j
  // of the slot is loaded by q.K wave j % 4 (its load i = j / 4). Within a region of rows of RB
  // bytes, lane l of a block writes slot byte pos = 1024 j + 16 l - (region offset), i.e. row
  // pos / RB and chunk slot (pos % RB) / 16, and loads the cache chunk slot ^ swz(row) of
  // that row there.
  // A wave issues its loads of a tile (kPerWave or kPerWave - 1 of them) on every step, past
  // the last tile too, with an empty buffer range: such a load reads nothing and writes zeros
  // into its LDS block, here a block of the retired slot being refilled. The wave's count is
  // the same at every wait. (A lane outside the buffer range of a direct-to-LDS load writes
  // zeros, so a wave's surplus block is skipped rather than loaded empty: it would land in a
  // live block.)
  const char* kc = (const char*)a.k;
  const char* vc = (const char*)a.v;
  const uint32_t krow = (uint32_t)a.Dk * (S::F8 ? 1 : 2);   // bytes between tokens in k_cache
  const uint32_t vrow = (uint32_t)a.v_row_len * S::kElt;   // ... in v_cache
  // per load i of this wave: region base and row stride (uniform), lane offset
  const char* lbase[S::kPerWave];
  uint32_t lstride[S::kPerWave], loff[S::kPerWave];
  bool lvalid[S::kPerWave];
  // pages of 16 keys (each 16-key half of a tile is a page): the block's rows lie in the
  // second half (row offsets then count from that half), or the block holds scales
  bool lhalf[S::kPerWave], lsc[S::kPerWave];
  const int dw = w;                 // index among the waves that load
  const bool dma_wave = w < S::kDmaWaves;
#pragma unroll
  for (int i = 0; i < S::kPerWave; ++i) {
    const int j = dw + S::kDmaWaves * i;
    lvalid[i] = dma_wave && j < S::kBlocks;
    // (the region follows from the block alone: regions are whole 1 KB blocks)
    const int jb = (lvalid[i] ? j : 0) * 1024;
    int q2, r, cs, gc;
    if (jb < S::kNBytes) {
      q2 = jb + lane * 16, lbase[i] = kc, lstride[i] = krow;
      r = q2 / S::kNRow, cs = (q2 - r * S::kNRow) >> 4, gc = cs ^ swz<S::kNRow>(r);
    } else if (jb < S::kNBytes + S::kRBytes) {
      constexpr int kRR = S::kRRow > 0 ? S::kRRow : 1;   // (no rotary region without rotary columns)
      q2 = jb - S::kNBytes + lane * 16, lbase[i] = rope_base, lstride[i] = rope_row_bytes;
      r = q2 / kRR, cs = (q2 - r * kRR) >> 4, gc = cs ^ swz<S::kRRow>(r);
    } else if (S::F8 && jb >= S::kScOff) {
      // the tile's 32 K (then V) scales (4 bytes per token, tokens innermost): lanes 0-7 load
      // them, the rest fall outside the buffer range. Without V scales the V block repeats the
      // K scales and is not used.
      const bool vsc = jb >= S::kVScOff && a.v_scale;
      q2 = 0, lbase[i] = (const char*)(vsc ? a.v_scale : a.k_scale), lstride[i] = 4u;
      r = 4 * lane, cs = 0, gc = 0;
    } else {
      q2 = jb - S::kNBytes - S::kRBytes + lane * 16, lbase[i] = vc, lstride[i] = vrow;
      r = q2 / S::kVSrcRow, cs = (q2 - r * S::kVSrcRow) >> 4, gc = cs ^ swz<S::kVSrcRow>(r);
    }
    loff[i] = (uint32_t)r * lstride[i] + 16u * (uint32_t)gc;
    // (16 rows of every region are whole 1 KB blocks, so all lanes of a block share lane
    // 0's half)
    lsc[i] = S::F8 && jb >= S::kScOff;
    lhalf[i] = !lsc[i] && __builtin_amdgcn_readfirstlane(r) >= 16;
    if (PM == kPagedHalf && lhalf[i]) loff[i] -= 16u * lstride[i];
  }
  // cache row of the first key of the tile at t0 (the tile is 32 consecutive rows; pages of
  // 16 keys: the 16-key run starting at t0)
  auto tile_row0 = [&](int t0) -> int64_t {
    if constexpr (PM == kContiguous) {
      return (int64_t)b * a.kv_capacity + t0;
    } else {
      const int pi = min(max((t0 >> a.page_shift) - first_page, 0), kMaxLdsPages - 1);
      const int sel = pi >> 6;
      const int v = sel == 0 ? pg[0] : sel == 1 ? pg[1] : sel == 2 ? pg[2] : pg[3];
      const int page = __builtin_amdgcn_readlane(v, pi & 63);
      return ((int64_t)page << a.page_shift) + (t0 & (a.page_size - 1));
    }
  };
  auto issue = [&](int ti) {
    char* dst = sm.tile[ti % R];
    const int t0 = start + ti * kTile;
    if constexpr (PM == kPagedHalf) {
      // pages of 16 keys: a scalar base per region and half; the scales (4 bytes per token)
      // come one token per lane from the whole scale tensor, lanes past the last valid key
      // (and lanes 32-63) outside the buffer range, so they read nothing and write zeros
      const bool live = ti < n_tiles;
      const int64_t row0 = live ? tile_row0(t0) : 0, row1 = live ? tile_row0(t0 + 16) : 0;
      const int rows = live ? __builtin_amdgcn_readfirstlane(min(kTile, end - t0)) : 0;
      const uint32_t rows0 = (uint32_t)min(rows, 16), rows1 = (uint32_t)max(rows - 16, 0);
      const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_addr(dst));
      const uint32_t sc_bytes = (uint32_t)a.num_pages * 16u * 4u;
#pragma unroll
      for (int i = 0; i < S::kPerWave; ++i) {
        if (!lvalid[i]) break;
        const uint32_t ldst = lb + (dw + S::kDmaWaves * i) * 1024;
        if (S::F8 && lsc[i]) {
          const uint32_t off = lane < rows ? (uint32_t)(((lane < 16 ? row0 : row1) + (lane & 15)) * 4) : sc_bytes;
          lds_dma4(rsrc_words(lbase[i], sc_bytes), off, ldst);
        } else {
          const u32x4 rs = lhalf[i] ? rsrc_words(lbase[i] + row1 * lstride[i], rows1 * lstride[i])
                                    : rsrc_words(lbase[i] + row0 * lstride[i], rows0 * lstride[i]);
          lds_dma16(rs, loff[i], ldst);
        }
      }
    } else if constexpr (PM != kPagedGeneral) {
      // 32 consecutive cache rows: one scalar base per region; the buffer range ends at the
      // last valid row, so a ragged tile's missing rows are not read (and past the last tile
      // nothing is)
      const bool live = ti < n_tiles;
      const int64_t row0 = live ? tile_row0(t0) : 0;
      const uint32_t rows = live ? (uint32_t)__builtin_amdgcn_readfirstlane(min(kTile, end - t0)) : 0u;
      const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_addr(dst));
#pragma unroll
      for (int i = 0; i < S::kPerWave; ++i) {
        if (!lvalid[i]) break;   // (uniform; only the last load of a wave can be surplus)
        const u32x4 rs = rsrc_words(lbase[i] + row0 * lstride[i], rows * lstride[i]);
        lds_dma16(rs, loff[i], lb + (dw + S::kDmaWaves * i) * 1024);
      }
    } else {
      if (ti >= n_tiles) return;
      // any page size: every lane looks up its own row (rows past the end repeat the last
      // key; their scores are masked); the fp8 scales come one token per lane (4 bytes)
      const int last = min(kTile - 1, end - 1 - t0);
#pragma unroll
      for (int i = 0; i < S::kPerWave; ++i) {
        if (!lvalid[i]) continue;
        const int j = dw + S::kDmaWaves * i;
        if (S::F8 && lsc[i]) {
          const int t = t0 + min(lane, last);
          const int pi = t / a.page_size;
          const int slot = min(max(pi - first_page, 0), kMaxLdsPages - 1);
          const int page = min(max(sm.pages[slot], 0), a.num_pages - 1);
          const int64_t row = (int64_t)page * a.page_size + (t - pi * a.page_size);
          __builtin_amdgcn_global_load_lds((const void*)(lbase[i] + row * 4), (DA_LDS void*)(dst + j * 1024), 4, 0, 0);
          continue;
        }
        const int r = (int)(loff[i] / lstride[i]);
        const int t = t0 + min(r, last);
        const int pi = t / a.page_size;
        const int slot = min(max(pi - first_page, 0), kMaxLdsPages - 1);
        const int page = min(max(sm.pages[slot], 0), a.num_pages - 1);
        const int64_t row = (int64_t)page * a.page_size + (t - pi * a.page_size);
        __builtin_amdgcn_global_load_lds((const void*)(lbase[i] + row * lstride[i] + (loff[i] - r * lstride[i])),
                                         (DA_LDS void*)(dst + j * 1024), 16, 0, 0);
      }
    }
  };
  // tile s has landed (this wave's loads): the loads of the A - 1 tiles after it may stay in
  // flight
  // (blocks are dealt round-robin, so a loading wave has kPerWave or kPerWave - 1 of them;
  // the P.V waves have none and wait for nothing here)
  const bool full_share = lvalid[S::kPerWave - 1];
  auto wait_tile = [&] {
    if constexpr (A == 2) {
      if (full_share) wait_vm<S::kPerWave>();
      else wait_vm<S::kPerWave - 1>();
    } else {
      wait_vm<0>();
    }
  };
  // block-wide "any" (every wave calls it; two barriers, flags in P buffer 1)
  auto block_any = [&](bool f) {
    __syncthreads();
    if (lane == 0) xa.any[w] = f ? 1 : 0;
    __syncthreads();
    int r = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) r |= xa.any[i];
    return r != 0;
  };

  if (w < 4) {
    // ------------------------------------------------------------------ q.K and softmax
    const int cp = w >> 1, kh = w & 1;
    // q as the B operand of S^T = K q^T: column block bi of the pair, k-step j holds depth
    // 32 j + 8 qd .. +8 of column col0 + 32 cp + 16 bi + n (zero past the last column)
    bf16x8 qf[2][S::NJ];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      const int col = col0 + 32 * cp + 16 * bi + n;
      const uint16_t* qrow = (const uint16_t*)a.q + ((int64_t)b * ncols + (col < ncols ? col : 0)) * S::DQK + 8 * qd;
#pragma unroll
      for (int j = 0; j < S::NJ; ++j) {
        u32x4 v = *(const u32x4*)(qrow + 32 * j);
        if (col >= ncols) v = u32x4{0u, 0u, 0u, 0u};
        qf[bi][j] = as_bf16x8(v);
      }
    }
    // keys this lane's columns attend (query qi of q_len sees keys t < L - q_len + 1 + qi)
    int col_end[2];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      const int col = col0 + 32 * cp + 16 * bi + n;
      const int qi = col < ncols ? col / a.g : 0;
      col_end[bi] = min(end, L - a.q_len + 1 + qi);
    }
    // K operands: k-step j reads logical chunk 4 j + qd of row r = 16 kh + n. The swizzle
    // only changes the low 4 (wide rows) or 3 (narrow rows) bits of the chunk, so the offset
    // is a per-lane part for j mod 4 (resp. mod 2) plus a constant.
    const int r = 16 * kh + n;
    constexpr bool kNW = S::kNRow % 256 == 0;
    const int fn = swz<S::kNRow>(r), fr = swz<S::kRRow>(r);
    int kn[4], kr[2];
#pragma unroll
    for (int u = 0; u < 4; ++u) kn[u] = r * S::kNRow + 16 * (((4 * u + qd) ^ fn) & (kNW ? 15 : 7));
#pragma unroll
    for (int u = 0; u < 2; ++u) kr[u] = S::kNBytes + r * S::kRRow + 16 * ((4 * u + qd) ^ fr);
    // F8 nope operands: k-step j reads the 8 codes of depth 32 j + 8 qd .. +7, i.e. half
    // qd & 1 of logical chunk 2 j + qd / 2 of row r (rows of 512 codes, the wide-row swizzle);
    // the per-lane part repeats every 8 steps
    int kn8[8];
    if constexpr (S::F8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) kn8[u] = r * S::kNRow + 16 * ((2 * u + (qd >> 1)) ^ fn) + 8 * (qd & 1);
    }
    auto load_k8 = [&](const DA_LDS char* KL, int j) {
      return *(const DA_LDS u32x2*)(KL + kn8[j & 7] + 256 * (j >> 3));
    };
    auto load_k = [&](const DA_LDS char* KL, int j) {
      int off;
      if (j < S::NJN) off = kNW ? kn[j & 3] + 256 * (j >> 2) : kn[j & 1] + 128 * (j >> 1);
      else off = kr[(j - S::NJN) & 1] + 128 * ((j - S::NJN) >> 1);
      return as_bf16x8(*(const DA_LDS u32x4*)(KL + off));
    };
    // K operands in flight ahead of their products (q takes 4 NJ registers per column block)
    constexpr int kAhead = S::NJ < 12 ? S::NJ : 12;

    float m_ref[2], m_lane[2], l_lane[2];
    bool beyond = false;
    // Step s of the key loop: S^T of tile s over the full q.K depth (two chains per column
    // block), then the softmax against m_ref and the P write.
    auto qk_step = [&](int s, bool first) {
      const DA_LDS char* KL = (const DA_LDS char*)sm.tile[s % R];
      f32x4 acc[2][2];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) acc[bi][0] = acc[bi][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 ks = f32x4{1.f, 1.f, 1.f, 1.f};   // F8: K scales of the lane's 4 keys
      f32x4 vs = f32x4{1.f, 1.f, 1.f, 1.f};   // F8: their V scales (the K scales for a shared V)
      if constexpr (S::F8) {
        // all nope codes (2 registers per step) and the rotary operands are requested first;
        // a step's codes are widened to bf16 just before its products. Rotary columns stored
        // apart (bf16) are summed apart: the K scale multiplies the nope part only. Rotary
        // codes in the K rows (RF8: step j reads the 8 codes of depth 32 (j - NJN) + 8 qd of
        // the unswizzled 64-byte rotary row) join the nope sum and take the same scale.
        u32x2 kc[S::NJN];
        bf16x8 krp[S::NJ - S::NJN];
        u32x2 kcr[S::NJ - S::NJN];
#pragma unroll
        for (int j = 0; j < S::NJN; ++j) kc[j] = load_k8(KL, j);
#pragma unroll
        for (int j = S::NJN; j < S::NJ; ++j) {
          if constexpr (S::RF8)
            kcr[j - S::NJN] = *(const DA_LDS u32x2*)(KL + S::kNBytes + r * S::kRRow + 32 * (j - S::NJN) + 8 * qd);
          else
            krp[j - S::NJN] = load_k(KL, j);
        }
        ks = *(const DA_LDS f32x4*)(KL + S::kScOff + 4 * (16 * kh + 4 * qd));
        if constexpr (!S::SHARED) {
          if (a.v_scale) vs = *(const DA_LDS f32x4*)(KL + S::kVScOff + 4 * (16 * kh + 4 * qd));
        } else {
          vs = ks;
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < S::NJN; ++j) {
          const bf16x8 kf = fp8x8_to_bf16x8(kc[j][0], kc[j][1]);
          acc[0][j & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][j], acc[0][j & 1], 0, 0, 0);
          acc[1][j & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[1][j], acc[1][j & 1], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (S::RF8) {
#pragma unroll
          for (int j = S::NJN; j < S::NJ; ++j) {
            const bf16x8 kf = fp8x8_to_bf16x8(kcr[j - S::NJN][0], kcr[j - S::NJN][1]);
            acc[0][j & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][j], acc[0][j & 1], 0, 0, 0);
            acc[1][j & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[1][j], acc[1][j & 1], 0, 0, 0);
          }
        }
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) acc[bi][0] = (acc[bi][0] + acc[bi][1]) * ks;
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) acc[bi][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (!S::RF8) {
#pragma unroll
          for (int j = S::NJN; j < S::NJ; ++j) {
            acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(krp[j - S::NJN], qf[0][j], acc[0][1], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(krp[j - S::NJN], qf[1][j], acc[1][1], 0, 0, 0);
          }
        }
      } else {
        bf16x8 kf[S::NJ];
#pragma unroll
        for (int j = 0; j < kAhead; ++j) kf[j] = load_k(KL, j);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < S::NJ; ++j) {
          acc[0][j & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[j], qf[0][j], acc[0][j & 1], 0, 0, 0);
          acc[1][j & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[j], qf[1][j], acc[1][j & 1], 0, 0, 0);
          if (j + kAhead < S::NJ) kf[j + kAhead] = load_k(KL, j + kAhead);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      const int t0 = start + s * kTile;
      float pr[2][4];
      float mx[2];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) {
        f32x4 sc = acc[bi][0] + acc[bi][1];
        // keys past the end of a ragged tile, or past a query's own position, get -inf
        const int nvalid = col_end[bi] - t0 - 16 * kh - 4 * qd;
        if (__ballot(nvalid < 4)) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i >= nvalid) sc[i] = -INFINITY;
        }
        mx[bi] = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        m_lane[bi] = fmaxf(m_lane[bi], mx[bi]);
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[bi][i] = sc[i];
      }
      if (first) {
        // the reference of the first pass: the first tile's max over both key halves; one
        // exchange per pass, the other tiles need no cross-lane step (P buffer 1 holds no P
        // before step 1)
        float g4[2];
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) {
          g4[bi] = max_over_key_groups(mx[bi]);
          if (qd == 0) xa.xm[w][bi][n] = g4[bi];
        }
        __syncthreads();
#pragma unroll
        for (int bi = 0; bi < 2; ++bi) {
          const float mt = fmaxf(g4[bi], xa.xm[w ^ 1][bi][n]);
          // (a column with no key in this tile: any finite reference; a later key far above
          // it sends the workgroup to the exact second pass)
          m_ref[bi] = mt == -INFINITY ? 0.f : mt;
        }
      }
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) {
        beyond = beyond || (mx[bi] - m_ref[bi]) * c > kHeadroomLog2;
        const float mc = m_ref[bi] * c;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[bi][i] = exp2_fast(fmaf(pr[bi][i], c, -mc));
          l_lane[bi] += pr[bi][i];
          // F8: V is code x the token's V scale (its K scale for a shared V); the scale goes
          // into P.V's operand, l sums the unscaled p
          if constexpr (S::F8) pr[bi][i] *= vs[i];
        }
        // hi and lo parts of P into the buffer (8 bytes each per lane)
        const uint32_t h0 = pack_bf16x2(pr[bi][0], pr[bi][1]), h1 = pack_bf16x2(pr[bi][2], pr[bi][3]);
        const uint32_t l0 = pack_bf16x2(pr[bi][0] - bf16lo(h0), pr[bi][1] - bf16hi(h0));
        const uint32_t l1 = pack_bf16x2(pr[bi][2] - bf16lo(h1), pr[bi][3] - bf16hi(h1));
        char* pb = sm.pbuf[s & 1] + (((2 * cp + bi) * 2 * 2 + kh) * 64 + lane) * 8;
        *(u32x2*)pb = u32x2{h0, h1};
        *(u32x2*)(pb + 2 * 64 * 8) = u32x2{l0, l1};
      }
    };

#pragma unroll
    for (int bi = 0; bi < 2; ++bi) m_lane[bi] = -INFINITY, m_ref[bi] = 0.f;
    wait_vm<0>();   // q is in registers: from here on the only loads in flight are the tiles'
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) l_lane[bi] = 0.f;
#pragma unroll
      for (int i = 0; i < A; ++i) issue(i);
      for (int s = 0; s <= n_tiles; ++s) {
        wait_tile();       // this wave's part of tile s is in LDS
        __syncthreads();   // ... and every wave's; P of tile s - 1 is written; tile s - 2 is retired
        issue(s + A);
        if (s < n_tiles) qk_step(s, pass == 0 && s == 0);
      }
      wait_vm<0>();        // (the empty loads past the last tile)
      if (!block_any(beyond)) break;
      // second pass: the reference is each column's exact max over the partition
      float g4[2];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) {
        g4[bi] = max_over_key_groups(m_lane[bi]);
        if (qd == 0) xa.xm[w][bi][n] = g4[bi];
      }
      __syncthreads();
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) {
        const float mt = fmaxf(g4[bi], xa.xm[w ^ 1][bi][n]);
        m_ref[bi] = mt == -INFINITY ? 0.f : mt;
      }
      beyond = false;
      __syncthreads();   // (xm is written again before it is next read)
    }
    // (max, sum, reference) per column for the P.V waves
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      const float mt = max_over_key_groups(m_lane[bi]);
      float l = l_lane[bi];
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
      if (qd == 0) {
        xa.xm[w][bi][n] = mt;
        xa.xl[w][bi][n] = l;
        xa.xr[w][bi][n] = m_ref[bi];
      }
    }
    __syncthreads();
  } else {
    // ------------------------------------------------------------------ P.V
    const int v = w - 4;
    // V^T A operand of 16-deep block D: lane (n, qd) holds depth 16 D + n of keys 4 qd .. +3
    // and 16 + 4 qd .. +3 (the k-slot order of the P buffer); that is chunk 2 D + ((n & 3) >> 1)
    // of rows ra and ra + 16, ra = 4 qd + (n >> 2), read transposed
    const int ra = 4 * qd + (n >> 2);
    const int v_off = S::kVReadOff + ra * S::kVRow + (n & 1) * 8;
    auto load_v = [&](const DA_LDS char* KL, int db) {
      const int ch = 2 * ((S::F8 ? 0 : v * S::kDB) + db) + ((n & 3) >> 1);
      const DA_LDS char* pa = KL + v_off + 16 * (ch ^ swz<S::kVRow>(ra));
      const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 DA_LDS*)pa);
      const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 DA_LDS*)(pa + 16 * S::kVRow));
      s16x8 v8;
      v8[0] = va[0]; v8[1] = va[1]; v8[2] = va[2]; v8[3] = va[3];
      v8[4] = vb[0]; v8[5] = vb[1]; v8[6] = vb[2]; v8[7] = vb[3];
      return __builtin_bit_cast(bf16x8, v8);
    };
    f32x4 o[S::kDB][4];
    // O^T += V^T P^T for the wave's depth blocks and all four column blocks: every operand is
    // requested first, then column block by column block the hi products of the depth blocks,
    // then their lo products, so that no product waits for the one just before it
    // F8: the wave widens the codes of its V columns of tile s into its bf16 copy (lane:
    // row lane / 2, four of the eight 16-code chunks of the row), which the transposing reads
    // then see like a bf16 tile. Only this wave writes and reads the copy.
    auto widen_v = [&](int s) {
      if constexpr (S::F8) {
        // the wave's kVCols codes of each row: kWC 16-code chunks, half of them per lane
        // (lane: row lane / 2, chunks (lane & 1) kWC / 2 ...); source rows are the nope rows
        // (shared V) or the V region's rows, each with its region's swizzle
        constexpr int kWC = S::kVCols / 16;
        constexpr int kSrcRow = S::SHARED ? S::kNRow : S::kVSrcRow;
        const char* src = sm.tile[s % R] + S::kVOff;
        char* dst = sm.vpriv[v];
        const int r = lane >> 1, h = lane & 1;
        const int fs = swz<kSrcRow>(r), fd = swz<S::kVRow>(r);
        u32x4 cw[kWC / 2];
#pragma unroll
        for (int k = 0; k < kWC / 2; ++k)
          cw[k] = *(const u32x4*)(src + r * kSrcRow + 16 * ((kWC * v + (kWC / 2) * h + k) ^ fs));
#pragma unroll
        for (int k = 0; k < kWC / 2; ++k) {
          const int bc = 2 * ((kWC / 2) * h + k);
          *(bf16x8*)(dst + r * S::kVRow + 16 * (bc ^ fd)) = fp8x8_to_bf16x8(cw[k][0], cw[k][1]);
          *(bf16x8*)(dst + r * S::kVRow + 16 * ((bc + 1) ^ fd)) = fp8x8_to_bf16x8(cw[k][2], cw[k][3]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    };
    auto pv_step = [&](int s) {
      widen_v(s);
      const DA_LDS char* KL;
      if constexpr (S::F8) KL = (const DA_LDS char*)sm.vpriv[v];
      else KL = (const DA_LDS char*)sm.tile[s % R];
      const char* pb = sm.pbuf[s & 1] + lane * 8;
      bf16x8 vf[S::kDB], ph[4], pl[4];
      auto load_p = [&](int cb) {
        const u32x2 h0 = *(const u32x2*)(pb + ((cb * 2 + 0) * 2 + 0) * 64 * 8);
        const u32x2 h1 = *(const u32x2*)(pb + ((cb * 2 + 0) * 2 + 1) * 64 * 8);
        const u32x2 l0 = *(const u32x2*)(pb + ((cb * 2 + 1) * 2 + 0) * 64 * 8);
        const u32x2 l1 = *(const u32x2*)(pb + ((cb * 2 + 1) * 2 + 1) * 64 * 8);
        ph[cb] = as_bf16x8(u32x4{h0[0], h0[1], h1[0], h1[1]});
        pl[cb] = as_bf16x8(u32x4{l0[0], l0[1], l1[0], l1[1]});
      };
      // P of column block 0, then V, then the other blocks' P: the first products wait for
      // their own operands only (latent: 60.3 against 61.2 us with all of V first)
      load_p(0);
#pragma unroll
      for (int db = 0; db < S::kDB; ++db) vf[db] = load_v(KL, db);
#pragma unroll
      for (int cb = 1; cb < 4; ++cb) load_p(cb);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
        for (int db = 0; db < S::kDB; ++db)
          o[db][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], ph[cb], o[db][cb], 0, 0, 0);
#pragma unroll
        for (int db = 0; db < S::kDB; ++db)
          o[db][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], pl[cb], o[db][cb], 0, 0, 0);
      }
    };
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int db = 0; db < S::kDB; ++db)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) o[db][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < A; ++i) issue(i);
      for (int s = 0; s <= n_tiles; ++s) {
        wait_tile();
        __syncthreads();
        issue(s + A);
        if (pass == 0 && s == 0) __syncthreads();   // (the q.K waves' first-tile exchange)
        if (s >= 1) pv_step(s - 1);
      }
      wait_vm<0>();
      if (!block_any(false)) break;
      __syncthreads();   // (the q.K waves' exact-max exchange)
      __syncthreads();
    }
    __syncthreads();   // the q.K waves have published (max, sum, reference)
    // O and l are relative to m_ref; the partial reports the exact max M, so its sum is
    // rescaled once (the normalised O does not change)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int col = col0 + 16 * cb + n;
      if (col >= ncols) continue;
      const int qw = 2 * (cb >> 1), bi = cb & 1;
      const float M = fmaxf(xa.xm[qw][bi][n], xa.xm[qw + 1][bi][n]);
      const float Ls = xa.xl[qw][bi][n] + xa.xl[qw + 1][bi][n];   // both halves share m_ref
      const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
      const float l_true = Ls > 0.f ? Ls * exp2_fast((xa.xr[qw][bi][n] - M) * c) : 0.f;
#pragma unroll
      for (int db = 0; db < S::kDB; ++db)
        store_unit(a, b, col, p, direct, S::kVCols * v + 16 * db + 4 * qd, o[db][cb] * inv, M, l_true,
                   v == 0 && db == 0 && qd == 0);
    }
  }

  if (!a.counters || direct) return;
  // Fused combine (fa4_splitk_combine_write, fourth paragraph), published as in the
  // matrix-core kernel: every wave's partial stores (device-coherent, cache policy SC1)
  // complete before the barrier, then one count on the (sequence, column block) counter; the
  // workgroup that completes the count reads the others' partials with SC1 loads and folds
  // the block's rows with every thread (S threads per (row, 4-wide slice) unit splitting the
  // partitions, merged through LDS as in the combine launch).
  wait_vm<0>();
  __syncthreads();
  int* cnt = a.counters + (int64_t)b * gridDim.y + cblk;
  int* flag_s = (int*)sm.pbuf[0];
  if (tid == 0) {
    const int last = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == P_b - 1;
    *flag_s = last ? 1 : 0;
  }
  __syncthreads();
  if (!__builtin_amdgcn_readfirstlane(*flag_s)) return;
  {
    constexpr int kUnits = S::DV / 4;
    const int nrow = min(kCols, ncols - col0);
    const int total = nrow * kUnits;
    const int SUB = P_b <= 16 ? 1 : (P_b <= 64 ? 4 : 16);
    const int UNITS = kThreads / SUB;
    const int sub = tid / UNITS, ui = tid % UNITS;
    // (the merge's LDS: the tile ring, free by now)
    float* sM = (float*)&sm.tile[0][0];   // [SUB][UNITS]
    float* sL = sM + SUB * UNITS;
    f32x4* sO = (f32x4*)(sL + SUB * UNITS);
    for (int u0 = 0; u0 < total; u0 += UNITS) {
      const int u = u0 + ui;
      const bool valid = u < total;
      const int d0 = valid ? (u % kUnits) * 4 : 0;
      const int64_t row = (int64_t)b * a.Hq + col0 + (valid ? u / kUnits : 0);
      float M = -INFINITY, Ls = 0.f;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (valid)
        fold_partials<S::DV, 8, true>((const float2*)a.part_ml + row * a.max_splits, a.part_o + row * a.max_splits * S::DV + d0,
                             1, P_b, sub, SUB, c, M, Ls, acc,
        a.part_ml, a.part_o);
      if (SUB > 1) {
        sM[sub * UNITS + ui] = M;
        sL[sub * UNITS + ui] = Ls;
        sO[sub * UNITS + ui] = acc;
        __syncthreads();
        if (valid && sub == 0) {
          float G = -INFINITY;
          for (int t = 0; t < SUB; ++t)
            if (sL[t * UNITS + ui] > 0.f) G = fmaxf(G, sM[t * UNITS + ui]);
          Ls = 0.f;
          acc = f32x4{0.f, 0.f, 0.f, 0.f};
          for (int t = 0; t < SUB; ++t) {
            if (sL[t * UNITS + ui] > 0.f) {
              const float e = exp2_fast((sM[t * UNITS + ui] - G) * c);
              Ls += sL[t * UNITS + ui] * e;
              acc += e * sO[t * UNITS + ui];
            }
          }
          M = G;
        }
        __syncthreads();   // (the LDS is reused by the next units)
      }
      if (valid && sub == 0) write_row_unit(a.out, a.o32, a.lse, row, S::DV, d0, M, Ls, acc, a.scale);
    }
  }
  if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class S>
hipError_t launch_shape(const PartArgs& a, int page_mode, hipStream_t s) {
  // rotary columns: stored apart (k_rope rows of DR bf16), or the last DR of each K row
  // (bf16, or codes with an fp8 cache)
  const char* rope = a.k_rope ? (const char*)a.k_rope : (const char*)a.k + S::DN * S::kElt;
  const uint32_t rope_row = a.k_rope ? (uint32_t)S::DR * 2 : (uint32_t)a.Dk * S::kElt;
  // x = partition, y = block of 64 columns, z = sequence: with 8 partitions the column blocks
  // of a (sequence, partition) are 8 workgroup ids apart (same XCD under round-robin
  // dispatch, so the second read of each tile is an L2 hit)
  dim3 grid(a.max_splits, (a.Hq + kCols - 1) / kCols, a.B), block(kThreads);
  switch (page_mode) {
    case kContiguous:
      hipLaunchKernelGGL((partition_shared_kernel<S, kContiguous>), grid, block, 0, s, a, rope, rope_row);
      break;
    case kPagedAligned:
      hipLaunchKernelGGL((partition_shared_kernel<S, kPagedAligned>), grid, block, 0, s, a, rope, rope_row);
      break;
    case kPagedHalf:
      hipLaunchKernelGGL((partition_shared_kernel<S, kPagedHalf>), grid, block, 0, s, a, rope, rope_row);
      break;
    default:
      hipLaunchKernelGGL((partition_shared_kernel<S, kPagedGeneral>), grid, block, 0, s, a, rope, rope_row);
      break;
  }
  return hipGetLastError();
}

}  // namespace

// One kv head for all q heads: MLA-style latent (q.K 576 = 512 nope + 64 rotary, V = the
// first 512 nope columns), one-kv-head GLM-style widths (q.K 256 = 192 nope + 64 rotary,
// V 256 of its own) and multi-query attention at depth 128 (bf16). The rotary columns may be
// in the K rows or stored apart.
hipError_t launch_partition_shared(const PartArgs& a, int page_mode, hipStream_t s) {
  if (a.Hkv != 1) return hipErrorInvalidValue;
  const bool rope_apart = a.k_rope != nullptr;
  if (a.kv_fp8) {
    if (!a.k_scale) return hipErrorInvalidValue;
    // latent over an fp8 cache: nope codes with per-token K scales, the rotary columns bf16
    // apart or codes in the K rows
    if (a.Dqk == 576 && a.Dv == 512 && a.v == a.k && !a.v_scale) {
      if (rope_apart && a.Dk == 512) return launch_shape<SShape<512, 64, 512, true, true>>(a, page_mode, s);
      if (!rope_apart && a.Dk == 576) return launch_shape<SShape<512, 64, 512, true, true, true>>(a, page_mode, s);
    }
    // one kv head with GLM widths: nope 192 and V 256 (its own, optional V scales) as codes
    if (a.Dqk == 256 && a.Dv == 256 && a.v != a.k) {
      if (rope_apart && a.Dk == 192) return launch_shape<SShape<192, 64, 256, false, true>>(a, page_mode, s);
      if (!rope_apart && a.Dk == 256) return launch_shape<SShape<192, 64, 256, false, true, true>>(a, page_mode, s);
    }
    return hipErrorInvalidValue;
  }
  if (a.Dqk == 576 && a.Dv == 512 && a.v == a.k && a.Dk == (rope_apart ? 512 : 576))
    return launch_shape<SShape<512, 64, 512, true>>(a, page_mode, s);
  // multi-query attention at depth 128: no rotary columns of their own, V its own cache
  if (a.Dqk == 128 && a.Dv == 128 && a.v != a.k && a.Dk == 128 && !rope_apart)
    return launch_shape<SShape<128, 0, 128, false>>(a, page_mode, s);
  if (a.Dqk == 256 && a.Dv == 256 && a.v != a.k && a.Dk == (rope_apart ? 192 : 256))
    return launch_shape<SShape<192, 64, 256, false>>(a, page_mode, s);
  return hipErrorInvalidValue;
}

}  // namespace da
