// C ABI of the split-KV decode-attention library: validation, split selection,
// workspace sizing and the launches of the two passes on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <mutex>

#include "da_internal.h"
#include "decode_attn.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return DA_OK;
}

enum Variant { kVarFma = 0, kVarMfma = 1, kVarShared = 2 };

constexpr int kTileKeys = 32;  // key tile of every partition kernel; chunks are multiples of it

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int q_len_of(const da_problem* p) { return p->q_len <= 0 ? 1 : p->q_len; }

// Output / partial rows per sequence: one per (query, head).
int64_t rows_per_seq(const da_problem* p) { return (int64_t)q_len_of(p) * p->num_q_heads; }

int device_num_cus() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Shape checks shared by every entry point; picks the partition-kernel family.
int check_problem(const da_problem* p, Variant* var) {
  if (!p) return fail(DA_EINVAL, "problem is NULL");
  if (p->batch < 1 || p->batch > 65535) return fail(DA_EINVAL, "batch must be in [1, 65535] (got %d)", p->batch);
  if (p->num_q_heads < 1 || p->num_kv_heads < 1 || p->num_kv_heads > 65535)
    return fail(DA_EINVAL, "num_q_heads and num_kv_heads must be >= 1 (got %d, %d)", p->num_q_heads, p->num_kv_heads);
  if (p->num_q_heads % p->num_kv_heads)
    return fail(DA_EINVAL, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)", p->num_q_heads, p->num_kv_heads);
  if (p->qk_depth < 1 || p->ov_depth < 1) return fail(DA_EINVAL, "depths must be >= 1");
  if (p->dtype != DA_F32 && p->dtype != DA_BF16) return fail(DA_EINVAL, "dtype must be DA_F32 or DA_BF16 (got %d)", p->dtype);
  if (p->page_size < 0) return fail(DA_EINVAL, "page_size must be >= 0");
  if (p->max_seq_len < 0) return fail(DA_EINVAL, "max_seq_len must be >= 0");
  if (p->page_size > 0) {
    if (p->num_pages < 1) return fail(DA_EINVAL, "paged cache needs num_pages >= 1");
    if ((int64_t)p->max_pages_per_seq * p->page_size < p->max_seq_len)
      return fail(DA_EINVAL, "page table row (%d pages of %d) cannot hold max_seq_len %d keys", p->max_pages_per_seq,
                  p->page_size, p->max_seq_len);
  } else {
    if (p->kv_capacity < 1) return fail(DA_EINVAL, "contiguous cache needs kv_capacity >= 1");
  }
  if (p->v_is_k_prefix && p->ov_depth > p->qk_depth)
    return fail(DA_EINVAL, "latent-shared V (ov_depth %d) must fit in the K row (qk_depth %d)", p->ov_depth, p->qk_depth);
  if (p->kernel < DA_KERNEL_AUTO || p->kernel > DA_KERNEL_MFMA) return fail(DA_EINVAL, "unknown kernel hint %d", p->kernel);
  const int g = p->num_q_heads / p->num_kv_heads;
  const int ql = q_len_of(p);
  if (ql < 1 || ql > 16) return fail(DA_EINVAL, "q_len must be in [0, 16] (got %d)", p->q_len);
  if (p->kv_dtype != 0 && p->kv_dtype != DA_FP8_E4M3)
    return fail(DA_EINVAL, "kv_dtype must be 0 or DA_FP8_E4M3 (got %d)", p->kv_dtype);
  if (p->nope_depth < 0 || (p->nope_depth > 0 && p->nope_depth >= p->qk_depth))
    return fail(DA_EINVAL, "nope_depth must be 0 (every K column in k_cache) or in [1, qk_depth) (got %d of %d)",
                p->nope_depth, p->qk_depth);
  // One kv head for many q heads: the shared-kv-head kernel (q.K and P.V as dense
  // contractions over all q heads). MLA-style latent 576/512 with V = the first 512 nope
  // columns, and GLM-style 256/256 (nope 192, V of its own) once q_len x group exceeds the
  // 16 MFMA columns of the GQA kernel; the 64 rotary columns in the K rows or stored apart.
  // Both take an fp8 cache: nope codes (and a V of its own) with per-token scales, the
  // rotary columns apart in bf16 or codes in the K rows (scaled with them).
  const bool latent = p->qk_depth == 576 && p->ov_depth == 512;
  const bool glm_mqa = p->qk_depth == 256 && p->ov_depth == 256 && !p->v_is_k_prefix && p->num_kv_heads == 1 &&
                       ql * g > 16;
  // multi-query attention at depth 128 with more than 16 columns: bf16 caches on the
  // shared-kv-head kernel (K read once per 64 columns); fp8 ones run as virtual kv heads on
  // the GQA kernel
  const bool mqa128 = p->qk_depth == 128 && p->ov_depth == 128 && !p->v_is_k_prefix && p->num_kv_heads == 1 &&
                      ql * g > 16 && p->dtype == DA_BF16 && p->kv_dtype == 0 && p->nope_depth == 0 &&
                      p->kernel != DA_KERNEL_FMA;
  if (mqa128) {
    *var = kVarShared;
    return DA_OK;
  }
  if (latent || glm_mqa) {
    const int nope_apart = latent ? 512 : 192;
    if (p->dtype != DA_BF16 || p->num_kv_heads != 1 || (latent && !p->v_is_k_prefix) || p->kernel == DA_KERNEL_FMA)
      return fail(DA_EUNSUPPORTED,
                  "depth %d/%d with one kv head runs on the shared-kv-head matrix-core kernel: bf16, one kv head%s",
                  p->qk_depth, p->ov_depth, latent ? ", V = the first 512 K columns (v_is_k_prefix)" : "");
    if (p->nope_depth != 0 && p->nope_depth != nope_apart)
      return fail(DA_EUNSUPPORTED, "shared-kv-head kernel at %d/%d: rotary columns apart need nope_depth %d (got %d)",
                  p->qk_depth, p->ov_depth, nope_apart, p->nope_depth);
    if (p->nope_depth > 0 && p->rope_dtype != DA_BF16)
      return fail(DA_EUNSUPPORTED, "rotary columns stored apart must be bf16 (rope_dtype %d)", p->rope_dtype);
    // (pages of 16 keys: the per-token scales are addressed from the start of their tensor)
    if (p->kv_dtype == DA_FP8_E4M3 && p->page_size == kTileKeys / 2 && (int64_t)p->num_pages * 16 * 4 >= INT32_MAX)
      return fail(DA_EUNSUPPORTED, "fp8 on the shared-kv-head kernel with pages of 16 keys: at most %d pages (got %d)",
                  INT32_MAX / 64, p->num_pages);
    *var = kVarShared;
    return DA_OK;
  }
  // Features only the matrix-core kernel has: several queries per sequence, fp8 caches,
  // the wider depth pairs and rotary columns stored apart.
  const bool d128 = p->qk_depth == 128 && p->ov_depth == 128;
  const bool d64 = p->qk_depth == 64 && p->ov_depth == 64;
  const bool wide = (p->qk_depth == 192 && p->ov_depth == 128) || (p->qk_depth == 256 && p->ov_depth == 256);
  if (ql > 1 || p->kv_dtype == DA_FP8_E4M3 || wide || d64 || p->nope_depth > 0) {
    if (!d128 && !d64 && !wide)
      return fail(DA_EUNSUPPORTED,
                  "several queries per sequence, fp8 caches and rotary columns stored apart are supported at "
                  "depths (q.K / V) 64/64, 128/128, 192/128 and 256/256 (got %d/%d)", p->qk_depth, p->ov_depth);
    if (p->nope_depth > 0 && (d128 || d64 || p->qk_depth - p->nope_depth != 64))
      return fail(DA_EUNSUPPORTED, "rotary columns stored apart: 64 of them at depth 192/128 or 256/256 "
                                   "(nope_depth 128 or 192; got %d of %d)", p->nope_depth, p->qk_depth);
    if (p->nope_depth > 0 && p->rope_dtype != DA_BF16)
      return fail(DA_EUNSUPPORTED, "rotary columns stored apart must be bf16 (rope_dtype %d)", p->rope_dtype);
    if (p->dtype != DA_BF16 || p->v_is_k_prefix || p->kernel == DA_KERNEL_FMA)
      return fail(DA_EUNSUPPORTED,
                  "this problem needs the matrix-core kernel: bf16 q and separate K and V caches");
    *var = kVarMfma;
    return DA_OK;
  }

  if (p->qk_depth != 128 || p->ov_depth != 128)
    return fail(DA_EUNSUPPORTED,
                "supported depths (q.K / V): 128/128; 64/64, 192/128 and 256/256 with bf16 q on the matrix-core kernel; "
                "576/512 latent-shared (got %d/%d)", p->qk_depth, p->ov_depth);
  if (p->dtype == DA_F32) {
    if (p->kernel == DA_KERNEL_MFMA) return fail(DA_EUNSUPPORTED, "the matrix-core kernel needs bf16 inputs");
    *var = kVarFma;
  } else if (p->kernel == DA_KERNEL_FMA) {
    // (bf16 with one q head per kv head also runs on the matrix cores by default: 15 of the
    // 16 MFMA columns idle still leave that kernel bound by HBM, at twice the vector-ALU
    // kernel's rate)
    *var = kVarFma;
  } else {
    *var = kVarMfma;
  }
  return DA_OK;
}

int chunk_unit(const da_problem* p) {
  if (p->page_size > 0 && p->page_size % kTileKeys == 0 && p->page_size <= 4096) return p->page_size;
  return kTileKeys;
}

int log2_exact(int v) {
  if (v <= 0 || (v & (v - 1))) return -1;
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

int page_mode(const da_problem* p) {
  if (p->page_size == 0) return da::kContiguous;
  if (p->page_size == kTileKeys / 2) return da::kPagedHalf;
  return (p->page_size >= kTileKeys && log2_exact(p->page_size) >= 0) ? da::kPagedAligned : da::kPagedGeneral;
}


// GQA kernels (matrix-core and vector-ALU): a wave serves at most 16 (query, head) columns.
// A larger group is split into kv_div groups of g / kv_div heads (the largest divisor of g
// with q_len x g / kv_div <= 16), each served as a kv head of its own: a virtual kv head,
// whose waves read the rows of their cached kv head (a second read of the same rows, mostly
// from L2). Shapes, schedules, counters and partial rows count virtual kv heads.
int kv_div_of(const da_problem* p) {
  const int ql = q_len_of(p), g = p->num_q_heads / p->num_kv_heads;
  if (ql * g <= 16) return 1;
  int d = 16 / ql;
  while (d > 1 && g % d) --d;
  return g / d;
}
int virtual_kv_heads(const da_problem* p) { return p->num_kv_heads * kv_div_of(p); }

// Matrix-core kernel shape: HG kv heads per workgroup (their waves read whole token
// rows of the cache together) times KS key splits per kv head, HG * KS = 8 waves.
// HG is as large as possible while the grid still offers a workgroup per CU (one
// 8-wave workgroup per CU fits at three waves per SIMD).
void mfma_shape(const da_problem* p, int32_t max_splits, int cus, int* HG, int* KS) {
  const int hkv = virtual_kv_heads(p);
  int hg = hkv < 8 ? hkv : 8;
  auto wgs = [&](int h) { return (int64_t)max_splits * ((hkv + h - 1) / h) * p->batch; };
  while (hg > 1 && wgs(hg) < (int64_t)cus) hg = (hg + 1) / 2;
  *HG = hg;
  *KS = 8 / hg > 0 ? 8 / hg : 1;
}

// Equal-share schedule shape (automatic splits on the matrix-core kernel): one 8-wave
// workgroup per CU. HG kv heads per workgroup as in mfma_shape, shrunk while even the
// largest possible problem (every sequence at max_seq_len) could not give each CU a share
// of kMinShareTiles tiles; W workers per head group so that W x groups ~ CUs.
void share_shape(const da_problem* p, int cus, int* HG, int* KS, int* W) {
  const int64_t tiles_max = (int64_t)p->batch * ceil_div(p->max_seq_len > 0 ? p->max_seq_len : 1, kTileKeys);
  const int hkv = virtual_kv_heads(p);
  int hg = hkv < 8 ? hkv : 8;
  auto groups = [&](int h) { return (int64_t)((hkv + h - 1) / h); };
  while (hg > 1 && (tiles_max / da::kMinShareTiles) * groups(hg) < (int64_t)cus) hg = (hg + 1) / 2;
  *HG = hg;
  *KS = 8 / hg > 0 ? 8 / hg : 1;
  const int64_t w = ceil_div(cus, groups(hg));
  *W = (int)(w < 1 ? 1 : w);
}

// Workgroups of the partition kernel resident per compute unit (LDS-bound): the vector-ALU
// kernel holds two in bf16, one in fp32; the matrix-core kernels one.
int wgs_per_cu(const da_problem* p, Variant v) { return v == kVarFma && p->dtype == DA_BF16 ? 2 : 1; }

int choose(const da_problem* p, Variant var, int32_t num_splits, int cus, int32_t* chunk_out, int32_t* splits_out) {
  if (num_splits < 0) return fail(DA_EINVAL, "num_splits must be >= 0 (0 = automatic)");
  if (num_splits == 0 && var == kVarMfma) {
    // automatic on the matrix-core kernel: equal shares of all keys over one workgroup
    // per CU (chunk 0 names this schedule; max_splits = workers)
    int HG, KS, W;
    share_shape(p, cus, &HG, &KS, &W);
    *chunk_out = 0;
    *splits_out = W;
    return DA_OK;
  }
  const int unit = chunk_unit(p);
  const int64_t maxlen = p->max_seq_len > 0 ? p->max_seq_len : 1;
  int64_t C;
  if (num_splits > 0) {
    C = ceil_div(maxlen, num_splits);
  } else {
    // Automatic: the host does not see seq_lens (no device sync), so it plans for an
    // average length of max_seq_len / 2 and aims at about four rounds of workgroups
    // over the whole chip; chunks stay within [256, 8192] keys.
    const int slots = cus * wgs_per_cu(p, var);
    // workgroups per (sequence, partition): kv heads, or 64-column blocks on the
    // shared-kv-head kernel
    const int64_t per_part = var == kVarShared ? ceil_div(rows_per_seq(p), 64) : virtual_kv_heads(p);
    const int64_t est_units = (int64_t)p->batch * per_part * ((maxlen + 1) / 2);
    C = ceil_div(est_units, 4LL * slots);
    // (multi-query attention at depth 128 on the shared-kv-head kernel: partitions of 256 keys
    // are dominated by each workgroup's first tiles; measured on the paged MQA workload,
    // 512-key chunks 33.0 us, 256: 40.7, 704: 37.0, 1024: 36.6)
    const int64_t min_chunk = var == kVarShared && p->qk_depth == 128 ? 512 : 256;
    if (C < min_chunk) C = min_chunk;
    if (C > 8192) C = 8192;
  }
  C = ceil_div(C, unit) * unit;
  if (C > ceil_div(maxlen, unit) * unit) C = ceil_div(maxlen, unit) * unit;
  if (var == kVarShared && p->page_size > 0) {
    // the shared-kv-head kernel stages one partition's page indices in LDS (at most 256 pages)
    const int64_t cap = (255LL * p->page_size) / kTileKeys * kTileKeys;
    if (C > cap) C = cap / unit * unit > 0 ? cap / unit * unit : kTileKeys;
  }
  if (C < unit) C = unit;
  const int64_t P = ceil_div(maxlen, C);
  if (C > INT32_MAX || P > INT32_MAX) return fail(DA_EINVAL, "split selection overflow");
  *chunk_out = (int32_t)C;
  *splits_out = (int32_t)P;
  return DA_OK;
}

// Partial rows of a schedule (R = q_len x Hq rows per sequence): fixed chunks
// B * R * max_splits; equal shares (chunk == 0) (max_splits + B) slots of R rows each.
size_t partial_rows(const da_problem* p, int32_t chunk, int32_t max_splits) {
  if (chunk == 0) return ((size_t)max_splits + (size_t)p->batch) * (size_t)rows_per_seq(p);
  return (size_t)p->batch * (size_t)rows_per_seq(p) * (size_t)max_splits;
}

// Workspace: part_ml (fp32 pairs; with equal shares followed by the int32 (first slot,
// count) table of the B sequences), then part_o, then the int32 arrival counters of the
// fused combine ([B][Hkv]), each padded to 256 bytes.
void ws_layout(const da_problem* p, int32_t chunk, int32_t max_splits, size_t* ml_off, size_t* o_off,
               size_t* cnt_off, size_t* total) {
  const size_t rows = partial_rows(p, chunk, max_splits);
  const size_t meta = chunk == 0 ? (size_t)p->batch * 2 * sizeof(int32_t) : 0;
  const size_t ml = (rows * 2 * sizeof(float) + meta + 255) & ~(size_t)255;
  const size_t o = (rows * (size_t)p->ov_depth * sizeof(float) + 255) & ~(size_t)255;
  // arrival counters of the fused combine: one per (sequence, kv head; virtual ones on the
  // matrix-core GQA kernel), or per (sequence, block of 64 columns) on the shared-kv-head kernel
  const size_t per_seq = std::max<size_t>((size_t)virtual_kv_heads(p), (size_t)ceil_div(rows_per_seq(p), 64));
  const size_t cnt = ((size_t)p->batch * per_seq * sizeof(int32_t) + 255) & ~(size_t)255;
  *ml_off = 0;
  *o_off = ml;
  *cnt_off = ml + o;
  *total = ml + o + cnt;
}

// The (first slot, count) table that follows the (m, l) pairs in part_ml (equal shares).
int32_t* meta_of(const da_problem* p, int32_t max_splits, const float* part_ml) {
  return (int32_t*)(part_ml + partial_rows(p, 0, max_splits) * 2);
}

int check_split_args(const da_problem* p, Variant var, int32_t chunk, int32_t max_splits) {
  if (chunk == 0) {
    if (var != kVarMfma)
      return fail(DA_EUNSUPPORTED, "chunk_tokens 0 (equal-share schedule) needs the matrix-core kernel");
    if (max_splits < 1 || max_splits > 65535)
      return fail(DA_EINVAL, "equal-share schedule: max_splits (workers) must be in [1, 65535] (got %d)", max_splits);
    return DA_OK;
  }
  if (chunk < 0 || chunk % kTileKeys) return fail(DA_EINVAL, "chunk_tokens must be 0 or a positive multiple of %d (got %d)", kTileKeys, chunk);
  if (var == kVarShared && p->page_size > 0 && (int64_t)chunk > 255LL * p->page_size)
    return fail(DA_EUNSUPPORTED, "shared-kv-head kernel: chunk_tokens must be <= 255 pages (%d keys)", 255 * p->page_size);
  const int64_t maxlen = p->max_seq_len > 0 ? p->max_seq_len : 1;
  if (max_splits < ceil_div(maxlen, chunk))
    return fail(DA_EINVAL, "max_splits %d < ceil(max_seq_len %d / chunk_tokens %d)", max_splits, p->max_seq_len, chunk);
  return DA_OK;
}

int check_inputs(const da_problem* p, const void* q, const void* k, const void* v, const int32_t* pt,
                 const int32_t* lens) {
  if (!q || !k || !lens) return fail(DA_EINVAL, "q, k_cache and seq_lens must be non-NULL");
  if (!p->v_is_k_prefix && !v) return fail(DA_EINVAL, "v_cache must be non-NULL unless v_is_k_prefix");
  if (p->page_size > 0 && !pt) return fail(DA_EINVAL, "page_table must be non-NULL for a paged cache");
  if (p->page_size == 0 && pt) return fail(DA_EINVAL, "page_table must be NULL for a contiguous cache");
  return DA_OK;
}

int launch_partition(const da_problem* p, Variant var, const da::PartArgs& a, hipStream_t s, int cus) {
  (void)hipGetLastError();
  hipError_t e;
  const int pm = page_mode(p);
  switch (var) {
    case kVarFma:
      e = da::launch_partition_fma(a, p->dtype == DA_F32 ? 0 : 1, pm, s);
      break;
    case kVarMfma: {
      int HG, KS;
      if (a.workers > 0) {
        int W;
        share_shape(p, cus, &HG, &KS, &W);
      } else {
        mfma_shape(p, a.max_splits, cus, &HG, &KS);
      }
      e = da::launch_partition_mfma(a, pm, HG, KS, s);
      break;
    }
    default:
      e = da::launch_partition_shared(a, pm, s);
      break;
  }
  if (e != hipSuccess) return fail(DA_EHIP, "partition kernel launch failed: %s", hipGetErrorString(e));
  return DA_OK;
}

int launch_combine(const da_problem* p, const int32_t* lens, float scale, int32_t chunk, int32_t max_splits,
                   const float* po, const float* pml, void* out, float* lse, float* o32, int skip_single,
                   hipStream_t s) {
  da::CombineArgs c;
  memset(&c, 0, sizeof(c));
  c.part_o = po;
  c.part_ml = pml;
  c.seq_lens = lens;
  c.out = (uint16_t*)out;
  c.lse = lse;
  c.o32 = o32;
  c.B = p->batch;
  c.Hq = (int32_t)rows_per_seq(p);
  c.Dv = p->ov_depth;
  c.chunk = chunk;
  c.max_splits = max_splits;
  c.max_seq_len = p->max_seq_len;
  c.kv_cap_clamp = p->page_size == 0 ? p->kv_capacity : 0;
  c.skip_single = skip_single;
  if (chunk == 0) {
    c.meta = meta_of(p, max_splits, pml);
    c.slots = max_splits + p->batch;
  }
  c.scale = scale;
  c.c = scale * 1.4426950408889634f;
  (void)hipGetLastError();
  const hipError_t e = da::launch_combine(c, s);
  if (e != hipSuccess) return fail(DA_EHIP, "combine kernel launch failed: %s", hipGetErrorString(e));
  return DA_OK;
}

int check_scale(float scale) {
  if (!std::isfinite(scale) || scale <= 0.f) return fail(DA_EINVAL, "scale must be finite and > 0");
  return DA_OK;
}

// The cache tensors must match the problem: fp8 caches come with their K scales (the
// plain entry points, which have no scale arguments, refuse them), and rotary columns
// stored apart come with their tensor.
int check_kv_args(const da_problem* p, const da_kv& kv) {
  if (p->kv_dtype == DA_FP8_E4M3 && !kv.k_scale)
    return fail(DA_EINVAL, "fp8 caches need k_scale (use decode_attn_splitk_fp8 / decode_attn_splitk_kv)");
  if (p->kv_dtype != DA_FP8_E4M3 && (kv.k_scale || kv.v_scale))
    return fail(DA_EINVAL, "k_scale / v_scale are for fp8 caches (kv_dtype = DA_FP8_E4M3)");
  if (p->kv_dtype == DA_FP8_E4M3 && p->v_is_k_prefix && kv.v_scale)
    return fail(DA_EINVAL, "with V the first ov_depth K columns, V is read with the K scales: v_scale must be NULL");
  if (p->nope_depth > 0 && !kv.k_rope)
    return fail(DA_EINVAL, "nope_depth > 0: the rotary columns (k_rope) are needed (use decode_attn_splitk_kv)");
  if (p->nope_depth == 0 && kv.k_rope) return fail(DA_EINVAL, "k_rope is for nope_depth > 0");
  return DA_OK;
}

da_kv make_kv(const void* k, const void* v, const float* k_scale = nullptr, const float* v_scale = nullptr) {
  da_kv kv;
  kv.k_cache = k;
  kv.v_cache = v;
  kv.k_rope = nullptr;
  kv.k_scale = k_scale;
  kv.v_scale = v_scale;
  return kv;
}

// Cache pointers and the fp8 / rotary-column fields of the kernel arguments.
void set_kv_args(const da_problem* p, const da_kv& kv, da::PartArgs* a) {
  a->k_scale = kv.k_scale;
  a->v_scale = kv.v_scale;
  a->kv_fp8 = p->kv_dtype == DA_FP8_E4M3;
  a->k_rope = kv.k_rope;
  a->Dk = p->nope_depth > 0 ? p->nope_depth : p->qk_depth;
}

// Fused combine: the last-arriving workgroup of a (sequence, head group) reads the partials
// of every row of the group alone, at the rate of one CU (about 40 GB/s), while the combine
// launch spreads the same fold over the chip for the cost of a launch (3-4 us). Measured
// (flushed steps): 2 KB and 32 KB of partial O per group, the fold in pass 1 is 1 us faster;
// 256 KB (64 partitions of 8 rows), 5 us slower; 1 MiB (8 partitions of 64 latent rows),
// 19 us slower. The fused entry point therefore folds in pass 1 while a group's partial O
// stays within kFusedFoldBytes, for the largest partition count the schedule allows a row
// (max_splits; under equal shares the workers a sequence of max_seq_len keys can meet);
// forced (mode 2) it always does.
constexpr int64_t kFusedFoldBytes = 64 << 10;

int64_t fused_fold_bytes(const da_problem* p, Variant var, int32_t C, int32_t P, int cus) {
  const int64_t ql = q_len_of(p), g = p->num_q_heads / p->num_kv_heads;
  int64_t rows;
  if (var == kVarFma) {
    rows = ql * (g / kv_div_of(p));   // (sequence, virtual kv head)
  } else if (var == kVarMfma) {
    int HG, KS, W;
    if (C == 0) share_shape(p, cus, &HG, &KS, &W);
    else mfma_shape(p, P, cus, &HG, &KS);
    rows = ql * (g / kv_div_of(p)) * HG;   // (sequence, group of virtual kv heads)
  } else {
    rows = std::min<int64_t>(64, rows_per_seq(p));   // (sequence, block of 64 columns)
  }
  // partials one row can have: max_splits; under equal shares (P = workers) also at most one
  // per share its sequence's tiles meet, and every share holds >= kMinShareTiles tiles
  int64_t parts = P;
  if (C == 0) {
    const int64_t tiles = ceil_div(p->max_seq_len > 0 ? p->max_seq_len : 1, kTileKeys);
    parts = std::min<int64_t>(P, ceil_div(tiles, da::kMinShareTiles) + 1);
  }
  return parts * rows * p->ov_depth * 4;
}

// Fused modes: 0 none (combine launch), 1 where the fold pays, 2 always. Either fused mode
// needs each partial array below 2 GB (the fold addresses them with 32-bit byte offsets).
bool fused_applies(const da_problem* p, Variant var, int32_t C, int32_t P, int cus, int mode) {
  if (mode == 0) return false;
  size_t ml_off, o_off, cnt_off, total;
  ws_layout(p, C, P, &ml_off, &o_off, &cnt_off, &total);
  if (o_off >= (size_t(1) << 31) || cnt_off - o_off >= (size_t(1) << 31)) return false;
  return mode == 2 || fused_fold_bytes(p, var, C, P, cus) <= kFusedFoldBytes;
}

// The whole step. With `fused`, the partition kernel's last-arriving workgroup of each
// (sequence, head group) combines (no second launch). The results are the same either way.
int run_splitk(const da_problem* p, const void* q, const da_kv& kv, const int32_t* page_table, const int32_t* seq_lens,
               float scale, int32_t num_splits, void* out, float* lse_out, float* o_f32_out, void* workspace,
               size_t workspace_bytes, void* stream, int fused) {
  Variant var;
  int r = check_problem(p, &var);
  if (r) return r;
  if ((r = check_kv_args(p, kv))) return r;
  if ((r = check_inputs(p, q, kv.k_cache, kv.v_cache, page_table, seq_lens))) return r;
  if ((r = check_scale(scale))) return r;
  if (!out) return fail(DA_EINVAL, "out must be non-NULL");
  const int cus = device_num_cus();
  int32_t C, P;
  if ((r = choose(p, var, num_splits, cus, &C, &P))) return r;
  size_t ml_off, o_off, cnt_off, need;
  ws_layout(p, C, P, &ml_off, &o_off, &cnt_off, &need);
  if (!workspace || ((uintptr_t)workspace & 255))
    return fail(DA_EWORKSPACE, "workspace must be non-NULL and 256-byte aligned");
  if (workspace_bytes < need)
    return fail(DA_EWORKSPACE, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  float* pml = (float*)((char*)workspace + ml_off);
  float* po = (float*)((char*)workspace + o_off);
  hipStream_t s = (hipStream_t)stream;
  da::PartArgs a = da::build_part_args(p, q, kv.k_cache, kv.v_cache, page_table, seq_lens, scale, C, P,
                                       var == kVarShared ? 1 : kv_div_of(p));
  a.part_o = po;
  a.part_ml = pml;
  if (C == 0) a.meta = meta_of(p, P, pml);
  a.out = (uint16_t*)out;
  a.lse = lse_out;
  a.o32 = o_f32_out;
  a.direct_single = 1;
  set_kv_args(p, kv, &a);
  // (where the fused fold does not apply the step takes the combine launch, with the same
  // results)
  const bool fuse = fused_applies(p, var, C, P, cus, fused);
  if (fuse) a.counters = (int32_t*)((char*)workspace + cnt_off);
  if ((r = launch_partition(p, var, a, s, cus))) return r;
  if (!fuse && (r = launch_combine(p, seq_lens, scale, C, P, po, pml, out, lse_out, o_f32_out, 1, s))) return r;
  return ok();
}

}  // namespace

namespace da {

int page_shift_of(int page_size) { return log2_exact(page_size); }

// Kernel arguments of a partition launch (shared with the tools that time kernels directly).
PartArgs build_part_args(const da_problem* p, const void* q, const void* k, const void* v, const int32_t* pt,
                       const int32_t* lens, float scale, int32_t chunk, int32_t max_splits, int32_t kv_div) {
  PartArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = p->v_is_k_prefix ? k : v;
  a.page_table = pt;
  a.seq_lens = lens;
  a.B = p->batch;
  a.Hq = (int32_t)rows_per_seq(p);
  a.Hq1 = p->num_q_heads;
  a.q_len = q_len_of(p);
  a.kv_div = kv_div < 1 ? 1 : kv_div;
  a.Hkv = p->num_kv_heads * a.kv_div;
  a.g = p->num_q_heads / a.Hkv;
  a.Dqk = p->qk_depth;
  a.Dk = p->nope_depth > 0 ? p->nope_depth : p->qk_depth;
  a.Dv = p->ov_depth;
  a.v_row_len = p->v_is_k_prefix ? p->qk_depth : p->ov_depth;
  a.page_size = p->page_size;
  a.page_shift = page_shift_of(p->page_size);
  a.pt_stride = p->max_pages_per_seq;
  a.num_pages = p->num_pages;
  a.kv_capacity = p->kv_capacity;
  a.max_seq_len = p->max_seq_len;
  a.chunk = chunk;
  a.max_splits = max_splits;
  a.workers = chunk == 0 ? max_splits : 0;
  a.scale = scale;
  a.c = scale * 1.4426950408889634f;
  return a;
}

}  // namespace da

extern "C" {

int da_supported(const da_problem* p) {
  Variant v;
  const int r = check_problem(p, &v);
  return r == DA_OK ? ok() : r;
}

int da_choose_splits(const da_problem* p, int32_t num_splits, int32_t num_cus, int32_t* chunk_tokens,
                     int32_t* max_splits) {
  Variant v;
  int r = check_problem(p, &v);
  if (r) return r;
  if (!chunk_tokens || !max_splits) return fail(DA_EINVAL, "output pointers must be non-NULL");
  r = choose(p, v, num_splits, num_cus > 0 ? num_cus : device_num_cus(), chunk_tokens, max_splits);
  return r ? r : ok();
}

int da_workspace_bytes(const da_problem* p, int32_t num_splits, size_t* bytes) {
  Variant v;
  int r = check_problem(p, &v);
  if (r) return r;
  if (!bytes) return fail(DA_EINVAL, "bytes must be non-NULL");
  int32_t C, P;
  r = choose(p, v, num_splits, device_num_cus(), &C, &P);
  if (r) return r;
  size_t a, b, c;
  ws_layout(p, C, P, &a, &b, &c, bytes);
  return ok();
}

int da_fused_applies(const da_problem* p, int32_t num_splits) {
  Variant v;
  int r = check_problem(p, &v);
  if (r) return r;
  const int cus = device_num_cus();
  int32_t C, P;
  r = choose(p, v, num_splits, cus, &C, &P);
  if (r) return r;
  ok();
  return fused_applies(p, v, C, P, cus, 1) ? 1 : 0;
}

int decode_attn_splitk(const da_problem* p, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* page_table, const int32_t* seq_lens, float scale, int32_t num_splits,
                       void* out, float* lse_out, float* o_f32_out, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return run_splitk(p, q, make_kv(k_cache, v_cache), page_table, seq_lens, scale, num_splits, out, lse_out,
                    o_f32_out, workspace, workspace_bytes, stream, 0);
}

// Scratch memory of decode_attn_splitk_noalloc: the workspace of one step (fp32 partials,
// the equal-share slot table) in a file-scope device array, so that the call allocates
// nothing. Every device the library runs on holds its own copy, at its own address, until
// the process ends. In host code the name `scratch` is a host-side stand-in, never a device
// address: kernels and copies get the address from scratch_ptr().
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

// Device address of the current device's `scratch`, looked up once per device (with that
// device current) and kept.
static int scratch_ptr(void** out) {
  static std::mutex mu;
  static void* ptrs[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fail(DA_EHIP, "no usable current HIP device");
  std::lock_guard<std::mutex> lk(mu);
  if (!ptrs[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(DA_EHIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    ptrs[dev] = ptr;
  }
  *out = ptrs[dev];
  return DA_OK;
}

int decode_attn_splitk_noalloc(const da_problem* p, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* page_table, const int32_t* seq_lens, float scale, int32_t num_splits,
                               void* out, float* lse_out, float* o_f32_out, void* stream) {
  size_t need = 0;
  int r = da_workspace_bytes(p, num_splits, &need);
  if (r) return r;
  if (need > kScratchBytes)
    return fail(DA_EWORKSPACE,
                "decode_attn_splitk_noalloc: this problem needs %zu bytes of workspace, more than the fixed "
                "%zu-byte scratch array (use decode_attn_splitk with a workspace of its size)", need, kScratchBytes);
  void* ws = nullptr;
  if ((r = scratch_ptr(&ws))) return r;
  return run_splitk(p, q, make_kv(k_cache, v_cache), page_table, seq_lens, scale, num_splits, out, lse_out,
                    o_f32_out, ws, kScratchBytes, stream, 0);
}

int decode_attn_splitk_fused(const da_problem* p, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* page_table, const int32_t* seq_lens, float scale, int32_t num_splits,
                             void* out, float* lse_out, float* o_f32_out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return run_splitk(p, q, make_kv(k_cache, v_cache), page_table, seq_lens, scale, num_splits, out, lse_out,
                    o_f32_out, workspace, workspace_bytes, stream, 1);
}

int decode_attn_splitk_fp8(const da_problem* p, const void* q, const void* k_cache, const void* v_cache,
                           const float* k_scale, const float* v_scale, const int32_t* page_table,
                           const int32_t* seq_lens, float scale, int32_t num_splits, void* out, float* lse_out,
                           float* o_f32_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!p) return fail(DA_EINVAL, "problem is NULL");
  if (p->kv_dtype != DA_FP8_E4M3) return fail(DA_EINVAL, "decode_attn_splitk_fp8 needs kv_dtype = DA_FP8_E4M3");
  return run_splitk(p, q, make_kv(k_cache, v_cache, k_scale, v_scale), page_table, seq_lens, scale, num_splits, out,
                    lse_out, o_f32_out, workspace, workspace_bytes, stream, 0);
}

int decode_attn_splitk_kv(const da_problem* p, const void* q, const da_kv* kv, const int32_t* page_table,
                          const int32_t* seq_lens, float scale, int32_t num_splits, int32_t fused, void* out,
                          float* lse_out, float* o_f32_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!kv) return fail(DA_EINVAL, "kv is NULL");
  if (fused < 0 || fused > 2) return fail(DA_EINVAL, "fused must be 0, 1 or 2 (got %d)", fused);
  return run_splitk(p, q, *kv, page_table, seq_lens, scale, num_splits, out, lse_out, o_f32_out, workspace,
                    workspace_bytes, stream, fused);
}

static int partition_impl(const da_problem* p, const void* q, const da_kv& kv, const int32_t* page_table,
                          const int32_t* seq_lens, float scale, int32_t chunk_tokens, int32_t max_splits,
                          float* part_o, float* part_ml, void* stream);

int decode_attn_partition_fp8(const da_problem* p, const void* q, const void* k_cache, const void* v_cache,
                              const float* k_scale, const float* v_scale, const int32_t* page_table,
                              const int32_t* seq_lens, float scale, int32_t chunk_tokens, int32_t max_splits,
                              float* part_o, float* part_ml, void* stream) {
  if (!p) return fail(DA_EINVAL, "problem is NULL");
  if (p->kv_dtype != DA_FP8_E4M3) return fail(DA_EINVAL, "decode_attn_partition_fp8 needs kv_dtype = DA_FP8_E4M3");
  return partition_impl(p, q, make_kv(k_cache, v_cache, k_scale, v_scale), page_table, seq_lens, scale,
                        chunk_tokens, max_splits, part_o, part_ml, stream);
}

int decode_attn_partition(const da_problem* p, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* page_table, const int32_t* seq_lens, float scale, int32_t chunk_tokens,
                          int32_t max_splits, float* part_o, float* part_ml, void* stream) {
  return partition_impl(p, q, make_kv(k_cache, v_cache), page_table, seq_lens, scale, chunk_tokens, max_splits,
                        part_o, part_ml, stream);
}

int decode_attn_partition_kv(const da_problem* p, const void* q, const da_kv* kv, const int32_t* page_table,
                             const int32_t* seq_lens, float scale, int32_t chunk_tokens, int32_t max_splits,
                             float* part_o, float* part_ml, void* stream) {
  if (!kv) return fail(DA_EINVAL, "kv is NULL");
  return partition_impl(p, q, *kv, page_table, seq_lens, scale, chunk_tokens, max_splits, part_o, part_ml, stream);
}

static int partition_impl(const da_problem* p, const void* q, const da_kv& kv, const int32_t* page_table,
                          const int32_t* seq_lens, float scale, int32_t chunk_tokens, int32_t max_splits,
                          float* part_o, float* part_ml, void* stream) {
  Variant var;
  int r = check_problem(p, &var);
  if (r) return r;
  if ((r = check_kv_args(p, kv))) return r;
  if ((r = check_inputs(p, q, kv.k_cache, kv.v_cache, page_table, seq_lens))) return r;
  if ((r = check_scale(scale))) return r;
  if ((r = check_split_args(p, var, chunk_tokens, max_splits))) return r;
  if (!part_o || !part_ml) return fail(DA_EINVAL, "part_o and part_ml must be non-NULL");
  da::PartArgs a = da::build_part_args(p, q, kv.k_cache, kv.v_cache, page_table, seq_lens, scale, chunk_tokens,
                                       max_splits, var == kVarShared ? 1 : kv_div_of(p));
  a.part_o = part_o;
  a.part_ml = part_ml;
  if (chunk_tokens == 0) a.meta = meta_of(p, max_splits, part_ml);
  a.direct_single = 0;
  set_kv_args(p, kv, &a);
  if ((r = launch_partition(p, var, a, (hipStream_t)stream, device_num_cus()))) return r;
  return ok();
}

int decode_attn_combine(const da_problem* p, const int32_t* seq_lens, float scale, int32_t chunk_tokens,
                        int32_t max_splits, const float* part_o, const float* part_ml, void* out, float* lse_out,
                        float* o_f32_out, void* stream) {
  Variant var = kVarFma;
  int r = check_problem(p, &var);
  if (r && r != DA_EUNSUPPORTED) return r;
  if (p->ov_depth != 64 && p->ov_depth != 128 && p->ov_depth != 256 && p->ov_depth != 512)
    return fail(DA_EUNSUPPORTED, "combine supports ov_depth 64, 128, 256 or 512 (got %d)", p->ov_depth);
  if (!seq_lens || !part_o || !part_ml || !out) return fail(DA_EINVAL, "seq_lens, part_o, part_ml and out must be non-NULL");
  if ((r = check_scale(scale))) return r;
  if ((r = check_split_args(p, var, chunk_tokens, max_splits))) return r;
  if ((r = launch_combine(p, seq_lens, scale, chunk_tokens, max_splits, part_o, part_ml, out, lse_out, o_f32_out, 0,
                          (hipStream_t)stream)))
    return r;
  return ok();
}

const char* da_last_error(void) { return g_err; }

const char* da_version(void) { return "decode_attn 0.1 (gfx950)"; }

}  // extern "C"
