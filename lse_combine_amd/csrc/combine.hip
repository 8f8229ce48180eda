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
constexpr int64_t kFewRows = 128;   // rows below which a many-partition row is split into depth bands
// (the rows each block folds: combine_rows in da_device.h)

template <int DV, int S, int NT = kCombineThreads, int BANDS = 1>
__global__ __launch_bounds__(NT) void combine_kernel(CombineArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[CombineLds<DV, S, NT>::kBytes];
  combine_rows<DV, S, NT, BANDS>(a, blockIdx.x, threadIdx.x, lds);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.Hq;
  // partitions a row may have: fixed chunks max_splits; equal shares about W / B + 1
  // (a single long sequence can meet every share)
  const int64_t pmax = a.meta ? (a.slots - a.B) / a.B + 1 : a.max_splits;
  int S = 1;
  while (S < 32 && (int64_t)S * kBatch < pmax) S *= 2;
  if (a.Dv == 128 && S >= 8 && rows < kFewRows) {
    // few rows with many partitions each: every row's depth is cut into 4 bands, one block
    // each, so that four compute units read a row's partials
    auto go = [&](auto kern, int nt) { hipLaunchKernelGGL(kern, dim3((unsigned)(rows * 4)), dim3(nt), 0, s, a); };
    switch (S) {
      case 8: go(combine_kernel<128, 8, 64, 4>, 64); break;
      case 16: go(combine_kernel<128, 16, 128, 4>, 128); break;
      default: go(combine_kernel<128, 32, 256, 4>, 256); break;
    }
  } else if (a.Dv == 128) {
    auto go = [&](auto kern, int rpb, int nt = kCombineThreads) {
      hipLaunchKernelGGL(kern, dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(nt), 0, s, a);
    };
    switch (S) {
      case 1: go(combine_kernel<128, 1>, 8); break;
      case 2: go(combine_kernel<128, 2>, 4); break;
      case 4: go(combine_kernel<128, 4>, 2); break;
      case 8: go(combine_kernel<128, 8>, 1); break;
      // rows with hundreds of partitions: 16 or 32 thread subsets per unit, one row per block
      case 16: go(combine_kernel<128, 16, 512>, 1, 512); break;
      default: go(combine_kernel<128, 32, 1024>, 1, 1024); break;
    }
  } else if (a.Dv == 64) {
    auto go = [&](auto kern, int rpb, int nt = kCombineThreads) {
      hipLaunchKernelGGL(kern, dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(nt), 0, s, a);
    };
    switch (S) {
      case 1: go(combine_kernel<64, 1>, 16); break;
      case 2: go(combine_kernel<64, 2>, 8); break;
      case 4: go(combine_kernel<64, 4>, 4); break;
      case 8: go(combine_kernel<64, 8>, 2); break;
      case 16: go(combine_kernel<64, 16>, 1); break;
      default: go(combine_kernel<64, 32, 512>, 1, 512); break;
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
