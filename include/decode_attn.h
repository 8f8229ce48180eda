/*
 * decode_attn.h -- split-KV decode attention with the log-sum-exp combine,
 * for AMD Instinct MI355X (gfx950). Plain C ABI: no C++ or framework types.
 *
 * What it computes. For every sequence b and query head h (one query per
 * sequence, i.e. decode), with kv head k = h / g and g = Hq / Hkv:
 *     O[b,h,:] = softmax_t(scale * q[b,h,:] . K[b,t,k,:]) @ V[b,t,k,:],  t < L_b
 *     LSE[b,h] = ln sum_t exp(scale * q[b,h,:] . K[b,t,k,:])
 * The keys of each sequence are cut into partitions of `chunk_tokens` keys.
 * Pass 1 (partition kernel) gives every partition its row max m_p (raw q.k
 * units), row sum l_p = sum_t exp(scale*(x_t - m_p)) and NORMALISED partial
 * O_p (fa4_splitk_combine_write, second paragraph). Pass 2 merges them with
 * the combine of fa4_splitk_combine_write (first paragraph):
 *     Gmax = max_p m_p,  e_p = exp2((m_p - Gmax) * c),  c = scale * log2(e)
 *     Gsum = sum_p l_p e_p,  w_p = l_p e_p / Gsum,  O = sum_p w_p O_p
 * and casts O to bf16 (round to nearest even). LSE = scale*Gmax + ln Gsum.
 * GQA heads that share a kv head are processed together so K/V are read once
 * (FA4Config, BM_eff). The cache is contiguous or paged (FA4Config,
 * v_row_major: a block-indirected paged cache). In the latent-shared layout V
 * is the first ov_depth columns of each K row (FA4Config, shared_kv_cols and
 * rope_depth: K = 512 non-rotary columns followed by 64 rotary ones).
 *
 * Conventions for every entry point:
 *  - Pointers named as device pointers must be device (or managed) memory of
 *    the current HIP device; the caller owns all memory. The library never
 *    allocates, frees or retains a pointer after the call returns.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *    No call synchronises with the host.
 *  - Return value: DA_OK (0) or a negative da_status. On error nothing has
 *    been enqueued (except DA_EHIP, where a launch failed), and
 *    da_last_error() returns a message for the calling thread.
 */
#ifndef DECODE_ATTN_H
#define DECODE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DA_OK = 0,
  DA_EINVAL = -1,        /* bad argument: null pointer, bad size, inconsistent shape */
  DA_EUNSUPPORTED = -2,  /* well-formed problem the library has no kernel for */
  DA_EWORKSPACE = -3,    /* workspace pointer null/misaligned or smaller than needed */
  DA_EHIP = -4           /* a HIP runtime call or kernel launch failed */
} da_status;

typedef enum {
  DA_F32 = 0,
  DA_BF16 = 1,
  DA_FP8_E4M3 = 2        /* cache only (kv_dtype): OCP FP8 E4M3 codes with per-token scales */
} da_dtype;

typedef enum {
  DA_KERNEL_AUTO = 0,    /* library's choice */
  DA_KERNEL_FMA = 1,     /* vector-ALU partition kernel (fp32 or bf16, depth 128, one query);
                            the automatic choice for fp32 only */
  DA_KERNEL_MFMA = 2     /* matrix-core partition kernel (bf16 q; bf16 or fp8 caches) */
} da_kernel;

/* Shape and layout of one decode step. All sizes are element counts. */
typedef struct da_problem {
  int32_t batch;             /* B >= 1 */
  int32_t num_q_heads;       /* Hq >= 1 */
  int32_t num_kv_heads;      /* Hkv >= 1, Hq % Hkv == 0; g = Hq / Hkv (FA4Config, group) */
  int32_t qk_depth;          /* Dqk: q/K row length */
  int32_t ov_depth;          /* Dv: V row length and output depth */
  int32_t dtype;             /* da_dtype of q, K and V; the output is always bf16 */
  int32_t page_size;         /* 0 = contiguous cache; > 0 = paged cache, keys per page */
  int32_t max_pages_per_seq; /* paged: row stride of page_table (entries per sequence) */
  int32_t num_pages;         /* paged: pages in the pool (page_table entries must be < this) */
  int32_t kv_capacity;       /* contiguous: key slots per sequence in the cache */
  int32_t max_seq_len;       /* host-side upper bound of seq_lens[]; sizes the grid */
  int32_t v_is_k_prefix;     /* 1 = latent-shared: V[t] = K[t][0:ov_depth], v_cache unused */
  int32_t kernel;            /* da_kernel: AUTO, or force a partition-kernel family */
  int32_t kv_dtype;          /* 0: K and V have `dtype`; DA_FP8_E4M3: fp8 K / V caches (bf16 q),
                                run through the *_fp8 entry points that take the scales */
  int32_t q_len;             /* queries per sequence (0 or 1: one, plain decode; > 1: the
                                sequence's last q_len positions, e.g. speculative tokens) */
  int32_t nope_depth;        /* 0: k_cache rows hold all qk_depth columns. > 0: k_cache holds the
                                first nope_depth ("nope") columns of every K row and a separate
                                tensor (da_kv.k_rope) the last qk_depth - nope_depth rotary ones
                                (FA4Config, rope_depth: the q.K depth minus the nope depth, which
                                need not equal ov_depth) */
  int32_t rope_dtype;        /* da_dtype of the rotary columns stored apart (FA4Config,
                                rope_dtype); DA_BF16 is the one supported. Ignored when
                                nope_depth == 0 */
} da_problem;

/*
 * Layouts (row-major, dense). With q_len > 1 every [B][Hq] below reads [B][q_len][Hq]
 * (q, out, lse_out, o_f32_out) and the partials have q_len * Hq rows per sequence; query i
 * (0-based) stands at position L_b - q_len + i of its sequence and attends the keys up to
 * and including that position (keys t < L_b - q_len + 1 + i: causal among the new tokens).
 *   q          [B][Hq][Dqk]                        dtype
 *   k_cache    contiguous: [B][kv_capacity][Hkv][Dqk]; paged: [num_pages][page_size][Hkv][Dqk]
 *              (with nope_depth > 0: nope_depth columns instead of Dqk)
 *   k_rope     nope_depth > 0 only: same layout with Dqk - nope_depth columns, rope_dtype
 *   v_cache    same as k_cache with Dv (ignored when v_is_k_prefix)
 *   page_table int32 [B][max_pages_per_seq]; key t of sequence b is slot t % page_size of
 *              page page_table[b][t / page_size]. Entries at or beyond ceil(L_b / page_size)
 *              are never read (padding may be any value, e.g. -1).
 *   seq_lens   int32 [B]; L_b keys are attended (no mask). Values < 0 count as 0; values above
 *              max_seq_len (or kv_capacity, contiguous) are clamped to it.
 *   out        bf16 [B][Hq][Dv]
 *   lse_out    fp32 [B][Hq] natural-log LSE (optional); -inf for L_b == 0
 *   o_f32_out  fp32 [B][Hq][Dv] O before the bf16 cast (optional); 0 for L_b == 0
 * Two split schedules name where partitions lie and where their partials go:
 *  - fixed chunks (chunk_tokens > 0): partition p of sequence b covers keys
 *    [p*chunk_tokens, min((p+1)*chunk_tokens, L_b)); sequence b has
 *    P_b = ceil(L_b / chunk_tokens) partitions (at most max_splits);
 *      part_ml  fp32 [B][Hq][max_splits][2] partition (m_p, l_p); m_p in raw q.k units
 *      part_o   fp32 [B][Hq][max_splits][Dv] normalised partition output O_p
 *  - equal shares (chunk_tokens == 0, max_splits = W workers; matrix-core kernel only):
 *    the 32-key tiles of all sequences, laid end to end in batch order and
 *    numbered 0..U-1, are cut into W' = min(W, max(1, floor(U / 8))) shares, share w
 *    holding tiles floor(w U / W') .. floor((w+1) U / W') - 1; every overlap of a share
 *    with a sequence is one partition, and partitions are numbered ("slots") sequence
 *    by sequence, then share by share. With S = W + B slots:
 *      part_ml  fp32 [S][Hq][2] (m, l) followed by int32 [B][2] (first slot, count) per
 *               sequence (written by pass 1, read by pass 2)
 *      part_o   fp32 [S][Hq][Dv]
 * A page_table entry outside [0, num_pages) is clamped into range (no fault; the
 * output of that sequence is then unspecified).
 */

/* DA_OK if a kernel exists for this problem, else DA_EINVAL / DA_EUNSUPPORTED with a
 * message (FA4Config, supported). Supported:
 *  - any group: more than 16 (query, head) columns per kv head run as virtual kv heads of
 *    at most 16 that read the same cache rows (one kv head at depth 128 in bf16 runs on
 *    the shared-kv-head kernel below);
 *  - Dqk == Dv == 128, one query per sequence: f32 (vector-ALU kernel) or bf16
 *    (matrix-core kernel; the vector-ALU one on request with DA_KERNEL_FMA);
 *  - on the matrix-core kernel (bf16 q, separate K and V) the depth pairs Dqk/Dv 64/64,
 *    128/128, 192/128 and 256/256, with the K/V cache in bf16 or fp8 and, at 192/128 and
 *    256/256, optionally the 64 rotary columns stored apart in bf16 (nope_depth 128 or 192);
 *  - with one kv head, on the shared-kv-head kernel (bf16 q, any number of q heads and
 *    q_len): latent 576/512 with V = the first 512 K columns (v_is_k_prefix), and
 *    256/256 with V of its own when q_len x Hq > 16; the 64 rotary columns in the K rows
 *    or stored apart in bf16 (nope_depth 512 or 192). Both also over an fp8 cache with the
 *    rotary columns apart (a V that is the K prefix takes the K scales: v_scale NULL).
 *  - any page_size >= 1 on every form (FA4Config, v_row_major: multi-page tiles of a
 *    block-indirected cache); pages of 16 keys or of a power of two >= 32 load a tile as
 *    runs of consecutive rows, other sizes key by key (with fp8 on the shared-kv-head
 *    kernel and pages of 16 keys, num_pages * 64 bytes of scales must stay below 2 GiB). */
int da_supported(const da_problem* p);

/* Split selection (FA4Config, with_splitk: partitions of the K/V sequence).
 * num_splits > 0: fixed chunks, chunk_tokens = ceil(max_seq_len / num_splits) rounded up
 * to a multiple of the key tile (32) and of page_size when that is a multiple of 32;
 * max_splits = ceil(max_seq_len / chunk_tokens) (>= 1).
 * num_splits == 0: automatic choice for the device's num_cus compute units (num_cus <= 0:
 * query the current device): on the matrix-core kernel (bf16 q with separate K and V, any
 * of its depth pairs and cache dtypes) the equal-share schedule (chunk_tokens = 0,
 * max_splits = workers, about one workgroup per CU), on the other kernels fixed chunks
 * sized for a few waves of workgroups. */
int da_choose_splits(const da_problem* p, int32_t num_splits, int32_t num_cus,
                     int32_t* chunk_tokens, int32_t* max_splits);

/* Bytes of workspace decode_attn_splitk needs for this problem and num_splits
 * (same num_splits / num_cus rule as da_choose_splits with num_cus queried). */
int da_workspace_bytes(const da_problem* p, int32_t num_splits, size_t* bytes);

/* 1 if decode_attn_splitk_fused merges the partials in pass 1 for this problem and
 * num_splits, 0 if it runs the combine launch instead, or an error code as da_supported.
 * The last-arriving workgroup of a group reads the group's partials alone, at the rate of
 * one compute unit, while the combine launch spreads them over the chip; so the merge runs
 * in pass 1 only while those partial outputs stay within 64 KiB: max_splits (under equal
 * shares, the workers a sequence of max_seq_len keys can meet: at most
 * ceil(ceil(max_seq_len / 32) / 8) + 1) times the rows of the head group or 64-column block
 * times Dv x 4 bytes. (On an MI355X that is 1 us faster than the combine launch at 2-32 KiB and
 * 5-19 us slower at 256 KiB-1 MiB.) Each partial array must also stay below 2 GB.
 * (num_splits and the device's compute units as da_workspace_bytes.) */
int da_fused_applies(const da_problem* p, int32_t num_splits);

/* The whole decode step: partition kernel, then LSE combine.
 * q, k_cache, v_cache, page_table (NULL iff page_size == 0), seq_lens: device, read only.
 * scale: finite and > 0 (softmax scale, e.g. 1/sqrt(Dqk)).
 * num_splits: 0 = automatic, else the fixed number of partitions (see da_choose_splits).
 * out: device bf16 [B][Hq][Dv]; lse_out, o_f32_out: optional device outputs (NULL = skip).
 * workspace: device, 256-byte aligned, at least da_workspace_bytes() bytes; its
 * contents on entry do not matter and are clobbered. */
int decode_attn_splitk(const da_problem* p, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* page_table, const int32_t* seq_lens,
                       float scale, int32_t num_splits, void* out, float* lse_out,
                       float* o_f32_out, void* workspace, size_t workspace_bytes, void* stream);

/* The whole decode step of decode_attn_splitk (same arguments and results) without a
 * workspace argument, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation). The partials live in a
 * fixed scratch array of 64 MiB that the library holds on every device it runs on for the
 * life of the process; the call allocates and frees nothing. A problem whose workspace
 * (da_workspace_bytes) exceeds 64 MiB returns DA_EWORKSPACE with nothing enqueued. Every
 * call on one device uses that device's one array: calls that overlap on a device (other
 * streams, other threads) race and must not be issued; calls ordered on one stream are
 * safe (no state carries over from one call to the next). */
int decode_attn_splitk_noalloc(const da_problem* p, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* page_table, const int32_t* seq_lens,
                               float scale, int32_t num_splits, void* out, float* lse_out,
                               float* o_f32_out, void* stream);

/* The whole decode step with the combine fused into pass 1 (fa4_splitk_combine_write,
 * fourth paragraph: the writer that completes the set combines all). Every workgroup of
 * a (sequence, kv-head group) stores its partial, publishes it device-wide and counts
 * itself in on an arrival counter; the last one merges all partials of its heads and
 * writes out / lse_out / o_f32_out, then resets the counter. This saves the second
 * launch. Done by every partition kernel (every depth pair, cache dtype and partition
 * count) where da_fused_applies says so; otherwise the step runs as decode_attn_splitk
 * (decode_attn_splitk_kv with fused = 2 merges in pass 1 wherever the partial arrays stay
 * below 2 GB). The outputs are the same either way. Rows of a sequence without keys are written too
 * (O = 0, LSE = -inf), by one workgroup that holds no keys. Same arguments and workspace
 * size as decode_attn_splitk,
 * with one more rule: the workspace must be zero-filled before its first use with this
 * function (the counters live in it and every call leaves them at zero), and calls that
 * share a workspace must not overlap. */
int decode_attn_splitk_fused(const da_problem* p, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* page_table,
                             const int32_t* seq_lens, float scale, int32_t num_splits, void* out,
                             float* lse_out, float* o_f32_out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* The whole decode step over an fp8 cache (FA4Config: an fp8 qkv_dtype with a per-token
 * scale_dtype for K). kv_dtype must be DA_FP8_E4M3, dtype DA_BF16 (q), a matrix-core depth
 * pair (see da_supported); the cache contiguous or paged (any page_size).
 * k_cache / v_cache hold E4M3 codes (one byte each, same layouts as above); key t of kv
 * head k reads k_scale * code (fp32 scale of that token and kv head) and V likewise with
 * v_scale (NULL = 1). Scale layout, tokens innermost: contiguous [B][Hkv][kv_capacity],
 * paged [num_pages][Hkv][page_size]. Everything else as decode_attn_splitk. */
int decode_attn_splitk_fp8(const da_problem* p, const void* q, const void* k_cache,
                           const void* v_cache, const float* k_scale, const float* v_scale,
                           const int32_t* page_table, const int32_t* seq_lens, float scale,
                           int32_t num_splits, void* out, float* lse_out, float* o_f32_out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Pass 1 only over an fp8 cache (scales as decode_attn_splitk_fp8, partials as
 * decode_attn_partition). */
int decode_attn_partition_fp8(const da_problem* p, const void* q, const void* k_cache,
                              const void* v_cache, const float* k_scale, const float* v_scale,
                              const int32_t* page_table, const int32_t* seq_lens, float scale,
                              int32_t chunk_tokens, int32_t max_splits, float* part_o,
                              float* part_ml, void* stream);

/* The cache tensors of one step, for the entry points that take them together. Host
 * struct, read during the call only; the pointers are device pointers. */
typedef struct da_kv {
  const void* k_cache;   /* K rows: all qk_depth columns, or the first nope_depth of them */
  const void* v_cache;   /* V rows (ignored when v_is_k_prefix) */
  const void* k_rope;    /* nope_depth > 0: the other qk_depth - nope_depth columns of every K
                            row (rope_dtype, k_cache's layout); else NULL */
  const float* k_scale;  /* fp8 caches: per-token scales of k_cache's columns (layout as for
                            decode_attn_splitk_fp8; the rotary columns have none); else NULL */
  const float* v_scale;  /* fp8 caches: per-token V scales, NULL = 1; else NULL */
} da_kv;

/* The whole decode step with the caches described by `kv`: every problem the library
 * supports, including rotary columns stored apart (nope_depth > 0) and fp8 caches.
 * fused = 1 runs it as decode_attn_splitk_fused (same workspace rules); fused = 2 likewise
 * but merges in pass 1 whatever the partials' size (for callers that must avoid the second
 * launch; each partial array below 2 GB); fused = 0 as decode_attn_splitk; other values
 * return DA_EINVAL. Other arguments as decode_attn_splitk. */
int decode_attn_splitk_kv(const da_problem* p, const void* q, const da_kv* kv,
                          const int32_t* page_table, const int32_t* seq_lens, float scale,
                          int32_t num_splits, int32_t fused, void* out, float* lse_out,
                          float* o_f32_out, void* workspace, size_t workspace_bytes, void* stream);

/* Pass 1 only with the caches described by `kv` (partials as decode_attn_partition). */
int decode_attn_partition_kv(const da_problem* p, const void* q, const da_kv* kv,
                             const int32_t* page_table, const int32_t* seq_lens, float scale,
                             int32_t chunk_tokens, int32_t max_splits, float* part_o,
                             float* part_ml, void* stream);

/* Pass 1 only (fa4_splitk_combine_write, second paragraph: each partition stages its
 * normalised O and its (max, sum)). Writes part_ml / part_o (device, layouts above) for
 * p < P_b; entries for p >= P_b are not written. chunk_tokens must be a positive multiple
 * of 32 with max_splits >= ceil(max_seq_len / chunk_tokens), or 0 (equal shares, 1 <=
 * max_splits <= 65535; DA_EUNSUPPORTED unless the matrix-core GQA kernel runs). */
int decode_attn_partition(const da_problem* p, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* page_table,
                          const int32_t* seq_lens, float scale, int32_t chunk_tokens,
                          int32_t max_splits, float* part_o, float* part_ml, void* stream);

/* Pass 2 only: the LSE combine of fa4_splitk_combine_write (first paragraph) over the
 * P_b partials of every row, then the bf16 cast. Reads part_ml / part_o entries p < P_b
 * (device). A partition with l_p == 0 has weight 0. Writes out (required), lse_out and
 * o_f32_out (optional). Same chunk_tokens / max_splits rules as decode_attn_partition. */
int decode_attn_combine(const da_problem* p, const int32_t* seq_lens, float scale,
                        int32_t chunk_tokens, int32_t max_splits, const float* part_o,
                        const float* part_ml, void* out, float* lse_out, float* o_f32_out,
                        void* stream);

/* Message of the last failed call on this thread ("" if none). */
const char* da_last_error(void);

/* Library version string. */
const char* da_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_ATTN_H */
