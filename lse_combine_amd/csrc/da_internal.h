// Internal declarations shared by the host API and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_attn.h"

namespace da {

enum PageMode : int {
  kContiguous = 0,   // row of key t in sequence b = b * kv_capacity + t
  kPagedAligned = 1, // paged, page_size a power of two >= 32: a 32-key tile never crosses a page
  kPagedGeneral = 2, // paged, any page_size: per-key page lookup
  kPagedHalf = 3     // paged, page_size 16: each 16-key half of a 32-key tile is one page
};

// Everything the partition kernels need; passed by value as the kernel argument.
struct PartArgs {
  const void* q;            // [B][q_len][heads][Dqk] = [B][Hq][Dqk]
  const void* k;            // cache rows of Dk elements, see key_row()
  const void* k_rope;       // rotary columns stored apart: rows of Dqk - Dk bf16 elements (or NULL)
  const void* v;            // cache rows of v_row_len elements (== k when V is a K prefix)
  const int32_t* page_table;
  const int32_t* seq_lens;
  float* part_o;            // fixed chunks: [B][Hq][max_splits][Dv]; equal shares: [slots][Hq][Dv]
  float* part_ml;           // fixed chunks: [B][Hq][max_splits][2];  equal shares: [slots][Hq][2]
  int32_t* meta;            // equal shares: [B][2] (first slot, partition count) per sequence
  int32_t* counters;        // fused combine: [B][head groups or 64-column blocks] arrival counters (zero between
                            // calls); NULL: the combine is a separate launch
  const float* k_scale;     // fp8 caches: per-token scales, tokens innermost ([B][Hkv][Lcap]
  const float* v_scale;     //   or [pages][Hkv][page]); v_scale may be NULL (1)
  int32_t kv_fp8;           // 1: k / v hold E4M3 codes
  uint16_t* out;            // bf16 [B][Hq][Dv]; written directly by single-partition rows
  float* lse;               // optional
  float* o32;               // optional
  int32_t B, Hq, Hkv, g, Dqk, Dv;   // Hq: rows per sequence (q_len x heads)
  int32_t kv_div;                   // GQA kernels: Hkv and g count virtual kv heads, kv_div per
                                    // cached kv head (1: none); shared-kv-head kernel: 1
  int32_t Dk;                       // K cache columns (Dqk, or the nope part when k_rope)
  int32_t Hq1, q_len;               // heads; queries per sequence (>= 1)
  int32_t v_row_len;        // elements between consecutive (row, kv-head) V vectors / Hkv
  int32_t page_size, pt_stride, num_pages, kv_capacity, max_seq_len;
  int32_t page_shift;       // log2(page_size) when it is a power of two, else -1
  int32_t chunk, max_splits;
  int32_t workers;          // 0: fixed chunks of `chunk` keys; > 0: equal-share schedule over
                            // this many workers (grid.x), slots = workers + B
  int32_t direct_single;    // 1: rows whose sequence has a single partition write out/lse/o32
  float scale;              // softmax scale
  float c;                  // scale * log2(e)
};

struct CombineArgs {
  const float* part_o;
  const float* part_ml;
  const int32_t* meta;      // equal shares: per-sequence (first slot, count); NULL: fixed chunks
  int32_t slots;            // equal shares: number of slots (workers + B)
  const int32_t* seq_lens;
  uint16_t* out;
  float* lse;
  float* o32;
  int32_t B, Hq, Dv;
  int32_t chunk, max_splits, max_seq_len, kv_cap_clamp;  // kv_cap_clamp: 0 = none
  int32_t skip_single;      // 1: rows with one partition were finished by pass 1
  float scale, c;
};

// Equal-share schedule: a workgroup (worker) gets at least this many 32-key tiles
// (when there are that many), so small problems are not cut into slivers.
constexpr int kMinShareTiles = 8;

// Kernel arguments of a partition launch for a validated problem (api.hip).
PartArgs build_part_args(const ::da_problem* p, const void* q, const void* k, const void* v,
                         const int32_t* page_table, const int32_t* seq_lens, float scale, int32_t chunk,
                         int32_t max_splits, int32_t kv_div = 1);

// Launchers (return hipSuccess or the launch error).
hipError_t launch_partition_fma(const PartArgs& a, int dtype, int page_mode, hipStream_t s);
// matrix-core kernel: dispatch over the depth shapes (partition_mfma128.hip), and the
// wider shapes' own translation units
hipError_t launch_partition_mfma(const PartArgs& a, int page_mode, int kv_heads_per_wg, int key_splits,
                                 hipStream_t s);
hipError_t launch_partition_mfma_d64(const PartArgs& a, int page_mode, int kv_heads_per_wg, int key_splits,
                                     hipStream_t s);
hipError_t launch_partition_mfma_d192(const PartArgs& a, int page_mode, int kv_heads_per_wg, int key_splits,
                                      hipStream_t s);
hipError_t launch_partition_mfma_d256(const PartArgs& a, int page_mode, int kv_heads_per_wg, int key_splits,
                                      hipStream_t s);
// one kv head for all q heads (latent 576/512, one-kv-head 256/256): partition_shared.hip
hipError_t launch_partition_shared(const PartArgs& a, int page_mode, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

}  // namespace da
