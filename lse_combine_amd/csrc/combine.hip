// Split-K pass 2: the log-sum-exp combine (fa4_splitk_combine_write, first paragraph).
//
// Threads own (row, 16-byte depth slice) units: as on the pages each thread forms the
// per-row weights itself and owns a band of depth columns; the threads of a row together
// cover the whole depth, the analogue of the pages' reduce-scatter band ownership. Rows
// with many partitions give each unit S threads that split the partitions (see
// combine_kernel). Rows are (sequence, q head) pairs; a row reads the
// (m_p, l_p) and normalised O_p of its P_b partitions:
//     Gmax = max_p m_p,   e_p = l_p * exp2((m_p - Gmax) * c),   Gsum = sum_p e_p
//     O = sum_p e_p O_p / Gsum   (= sum_p w_p O_p with w_p = e_p / Gsum)
//     LSE = scale * Gmax + ln Gsum,   out = bf16(O) (round to nearest even)
// Partitions with l_p == 0 are skipped (weight 0); a row with no keys gets O = 0 and
// LSE = -inf. With fixed chunks a row's partials are contiguous ([B][Hq][max_splits]);
// with the equal-share schedule they sit in consecutive slots ([slot][Hq]) named by the
// per-sequence (first slot, count) table that pass 1 wrote.
#include "da_device.h"

namespace da {
namespace {

constexpr int kCombineThreads = 256;
constexpr int kBatch = 8;   // partitions whose loads are in flight together, per thread (fold_partials)

// One (row, 4-wide depth slice) unit per thread and S threads per unit: thread subset s
// takes partitions s, s + S, s + 2S, ... of the row and keeps a running (max, sum, O)
// for them (the same exp2 weights, rescaled when the running max grows); the S
// partial results are then merged through LDS with the combine formula. With S = 1 this
// is the plain per-thread combine; S > 1 shortens the dependent load chain of rows with
// many partitions (64 for the long workload) by a factor S.
template <int DV, int S>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineArgs a) {
  constexpr int TPR = DV / 4;                       // threads (units) per row
  constexpr int UNITS = kCombineThreads / S;        // units per block
  constexpr int RPB = UNITS / TPR;                  // rows per block
  static_assert(RPB >= 1 && UNITS % TPR == 0, "block shape");
  __shared__ float sM[S > 1 ? S : 1][UNITS], sL[S > 1 ? S : 1][UNITS];
  __shared__ f32x4 sO[S > 1 ? S : 1][UNITS];

  const int tid = threadIdx.x;
  const int sub = tid / UNITS, u = tid % UNITS;
  const int r_in = u / TPR, ch = u % TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + r_in;
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
    sM[sub][u] = M;
    sL[sub][u] = Ls;
    sO[sub][u] = acc;
    __syncthreads();
    if (sub != 0) return;
    float G = -INFINITY;
#pragma unroll
    for (int t = 0; t < S; ++t)
      if (sL[t][u] > 0.f) G = fmaxf(G, sM[t][u]);
    Ls = 0.f;
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < S; ++t) {
      if (sL[t][u] > 0.f) {
        const float e = exp2_fast((sM[t][u] - G) * a.c);
        Ls += sL[t][u] * e;
        acc += e * sO[t][u];
      }
    }
    M = G;
  }
  if (!active) return;
  write_row_unit(a.out, a.o32, a.lse, row, DV, ch * 4, M, Ls, acc, a.scale);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.Hq;
  // partitions a row may have: fixed chunks max_splits; equal shares about W / B + 1
  // (a single long sequence can meet every share)
  const int64_t pmax = a.meta ? (a.slots - a.B) / a.B + 1 : a.max_splits;
  int S = 1;
  while (S < 8 && (int64_t)S * kBatch < pmax) S *= 2;
  if (a.Dv == 128) {
    auto go = [&](auto kern, int rpb) {
      hipLaunchKernelGGL(kern, dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(kCombineThreads), 0, s, a);
    };
    switch (S) {
      case 1: go(combine_kernel<128, 1>, 8); break;
      case 2: go(combine_kernel<128, 2>, 4); break;
      case 4: go(combine_kernel<128, 4>, 2); break;
      default: go(combine_kernel<128, 8>, 1); break;
    }
  } else if (a.Dv == 256) {
    auto go = [&](auto kern, int rpb) {
      hipLaunchKernelGGL(kern, dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(kCombineThreads), 0, s, a);
    };
    switch (S) {
      case 1: go(combine_kernel<256, 1>, 4); break;
      case 2: go(combine_kernel<256, 2>, 2); break;
      default: go(combine_kernel<256, 4>, 1); break;
    }
  } else {
    if (S == 1)
      hipLaunchKernelGGL((combine_kernel<512, 1>), dim3((unsigned)((rows + 1) / 2)), dim3(kCombineThreads), 0, s, a);
    else
      hipLaunchKernelGGL((combine_kernel<512, 2>), dim3((unsigned)rows), dim3(kCombineThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace da
