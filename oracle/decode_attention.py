"""Plain fp64 CPU oracle for split-KV decode attention and its log-sum-exp combine.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module: only the tests, the smoke check and the benchmark's CPU-baseline
leg use it. It shares no code, constant or helper with the HIP library.

What is computed (single query per sequence, i.e. decode):

* ``decode_attention_fp64`` -- the plain definition. For every sequence b and
  query head h, with kv head k = floor(h / g), g = Hq / Hkv:
      x_t  = sum_d q[b,h,d] * K[b,t,k,d]            t < L_b
      m    = max_t x_t
      Z    = sum_t exp(scale * (x_t - m))
      O[d] = sum_t exp(scale * (x_t - m)) * V[b,t,k,d] / Z
      LSE  = scale * m + ln Z
  The split-K method re-associates exactly this sum, so the definition is the
  oracle for the whole path (fa4_splitk_combine_write, first paragraph: the
  per-partition weights sum to one and the partition sums cancel the
  normalisation of each partial O).
* ``partition_partials_fp64`` -- pass 1 of split-K as the pages describe it:
  each key partition yields its row max, row sum and NORMALISED partial O
  (fa4_splitk_combine_write, second paragraph).
* ``equal_share_pieces`` / ``range_partials_fp64`` -- the partition boundaries
  of the equal-share schedule the automatic split uses, and pass 1 over such
  explicit key ranges.
* ``combine_fp64`` -- pass 2, the combine formula of fa4_splitk_combine_write
  (first paragraph) written out in the pages' exp2 form:
      Gmax = max_p max_p,  Gsum = sum_p sum_p * exp2((max_p - Gmax) * c),
      w_p = sum_p * exp2((max_p - Gmax) * c) / Gsum,  O = sum_p w_p * O_p,
  with c = scale * log2(e) (the ``scale_log2e`` argument of that function).
* ``bf16_round_fp64`` -- the final cast to bf16 (same paragraph), read as
  round-to-nearest-even.
* ``fp8_e4m3_to_fp64`` -- the values of an fp8 (E4M3) cache; with per-token scales
  the definition above runs on code value times scale (FA4Config: fp8 qkv_dtype with a
  per-token scale_dtype for K).
* rotary columns stored apart (``k_rope``): the last Dqk - nope columns of every
  K row live in a tensor of their own with their own dtype (FA4Config: rope_depth
  is the padded qk depth minus the padded nope depth, not minus the V depth, and
  rope_dtype may differ from the qkv dtype). The definition runs on the row
  [K nope columns | rotary columns]; per-token scales of an fp8 cache belong to
  the quantised nope columns only (reading: the rotary tensor is not quantised).

Readings where the pages are silent (each is listed in the design notes):
the max is kept in raw q.k units; empty partitions contribute weight 0 and an
empty sequence gives O = 0, LSE = -inf; partitions are contiguous chunks of
``chunk`` keys; q head h reads kv head h // g (FA4Config, BM_eff: a fused
GQA tile covers ``group`` heads); in the latent-shared layout V is the first
``ov_depth`` columns of K (FA4Config, shared_kv_cols / nope_cols_per_cta).

Every function here is pinned by the ``-m "not gpu"`` tests against brute
force, closed forms, library routines and invariants.
"""

from __future__ import annotations

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)


# ---------------------------------------------------------------------------
# fp8 (E4M3, OCP "fn" variant) cache values
# ---------------------------------------------------------------------------
def fp8_e4m3_to_fp64(codes):
    """Decode OCP FP8 E4M3 codes (uint8) to fp64, from the format's definition.

    Bit 7 is the sign, bits 6-3 the exponent e (bias 7), bits 2-0 the mantissa m.
    e = 0 encodes subnormals m/8 * 2^-6; otherwise the value is (1 + m/8) * 2^(e-7).
    The variant has no infinities: e = 15 with m = 7 is NaN, so the largest finite
    magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


def _scale_rows(scales, b, kvh, L, page_table, page_size):
    """Per-token scales of keys 0..L-1 of (sequence b, kv head kvh).

    Layout (tokens innermost so that a tile's scales are contiguous): contiguous
    [B, Hkv, L_cap]; paged [N_pages, Hkv, page_size].
    """
    t = np.arange(L)
    s = np.asarray(scales)
    if page_table is None:
        return s[b, kvh, :L].astype(np.float64)
    pages = np.asarray(page_table)[b, t // page_size]
    return s[pages, kvh, t % page_size].astype(np.float64)


# ---------------------------------------------------------------------------
# gathering one (sequence, kv-head) slice of the cache
# ---------------------------------------------------------------------------
def _key_rows(k_cache, b, kvh, L, page_table, page_size, scales=None):
    """Return the L key vectors of sequence b, kv head kvh, as fp64 [L, D].

    Contiguous layout: k_cache is [B, L_cap, Hkv, D] and key t is k_cache[b, t].
    Paged layout: k_cache is a page pool [N_pages, page_size, Hkv, D] and key t
    lives in page page_table[b, t // page_size] at slot t % page_size
    (FA4Config, v_row_major: a block-indirected paged cache addresses a page's
    rows at block_idx * stride).
    """
    t = np.arange(L)
    if page_table is None:
        rows = k_cache[b, :L, kvh, :]
    else:
        pages = np.asarray(page_table)[b, t // page_size]
        rows = k_cache[pages, t % page_size, kvh, :]
    rows = np.asarray(rows)
    if rows.dtype == np.uint8:
        # fp8 cache: codes times the per-token scale (FA4Config, scale_dtype: per-token
        # scaling of the quantised cache)
        vals = fp8_e4m3_to_fp64(rows)
        s = np.ones(L) if scales is None else _scale_rows(scales, b, kvh, L, page_table, page_size)
        return vals * s[:, None]
    return rows.astype(np.float64)


def _gather(q, k_cache, v_cache, b, kvh, g, L, page_table, page_size, v_is_k_prefix, ov_depth,
            k_scale=None, v_scale=None, k_rope=None):
    qg = np.asarray(q[b, kvh * g:(kvh + 1) * g, :], dtype=np.float64)
    K = _key_rows(k_cache, b, kvh, L, page_table, page_size, k_scale)
    if k_rope is not None:
        # the rotary columns follow the nope columns of the same row (no scale of their own)
        K = np.concatenate([K, _key_rows(k_rope, b, kvh, L, page_table, page_size)], axis=1)
    if v_is_k_prefix:
        V = K[:, :ov_depth]
    else:
        V = _key_rows(v_cache, b, kvh, L, page_table, page_size, v_scale)
    return qg, K, V


def _dims(q, k_cache, v_cache, v_is_k_prefix, ov_depth, k_rope=None):
    B, Hq, Dqk = q.shape
    Hkv = k_cache.shape[2]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    width = k_cache.shape[3] + (0 if k_rope is None else k_rope.shape[3])
    if width != Dqk:
        raise ValueError(f"K row width {width} (nope + rotary columns) must equal the q depth {Dqk}")
    if v_is_k_prefix:
        Dv = Dqk if ov_depth is None else int(ov_depth)
    else:
        Dv = v_cache.shape[3]
    return B, Hq, Hkv, Hq // Hkv, Dqk, Dv


# ---------------------------------------------------------------------------
# the definition
# ---------------------------------------------------------------------------
def decode_attention_fp64(q, k_cache, v_cache, seq_lens, scale, page_table=None, page_size=0,
                          v_is_k_prefix=False, ov_depth=None, k_scale=None, v_scale=None, k_rope=None):
    """Full softmax(scale * q K^T) V per (sequence, head), in fp64.

    q: [B, Hq, Dqk]; caches as described in ``_key_rows``; seq_lens: [B].
    fp8 caches (uint8 E4M3 codes) are read as code value times the per-token scale
    (``k_scale`` / ``v_scale``, layout in ``_scale_rows``; a missing scale is 1).
    ``k_rope``: the rotary columns of every K row, stored apart in the cache's layout
    ([..., Hkv, Dqk - nope]); ``k_cache`` then holds the first nope columns.
    Returns (O [B, Hq, Dv] fp64, LSE [B, Hq] fp64, natural log).
    A sequence of length 0 gives O = 0 and LSE = -inf.

    Several queries per sequence: q [B, q_len, Hq, Dqk] holds the sequence's last q_len
    positions, and query i attends the keys up to its own position, t < L_b - q_len + 1 + i
    (the pages fix no mask for this case; this is the causal reading among the new
    tokens). Returns O [B, q_len, Hq, Dv] and LSE [B, q_len, Hq].
    """
    q_arr = np.asarray(q)
    if q_arr.ndim == 4:
        ql = q_arr.shape[1]
        lens = np.asarray(seq_lens, dtype=np.int64)
        outs = [decode_attention_fp64(q_arr[:, i], k_cache, v_cache, np.clip(lens - ql + 1 + i, 0, lens), scale,
                                      page_table, page_size, v_is_k_prefix, ov_depth, k_scale, v_scale, k_rope)
                for i in range(ql)]
        return np.stack([o for o, _ in outs], 1), np.stack([l for _, l in outs], 1)
    B, Hq, Hkv, g, Dqk, Dv = _dims(q, k_cache, v_cache, v_is_k_prefix, ov_depth, k_rope)
    O = np.zeros((B, Hq, Dv), dtype=np.float64)
    LSE = np.full((B, Hq), -np.inf, dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        for kvh in range(Hkv):
            qg, K, V = _gather(q, k_cache, v_cache, b, kvh, g, L, page_table, page_size,
                               v_is_k_prefix, Dv, k_scale, v_scale, k_rope)
            x = qg @ K.T                                   # [g, L] raw scores
            m = x.max(axis=1, keepdims=True)
            e = np.exp(scale * (x - m))
            Z = e.sum(axis=1, keepdims=True)
            O[b, kvh * g:(kvh + 1) * g] = (e @ V) / Z
            LSE[b, kvh * g:(kvh + 1) * g] = scale * m[:, 0] + np.log(Z[:, 0])
    return O, LSE


# ---------------------------------------------------------------------------
# split-K pass 1: per-partition (max, sum, normalised O)
# ---------------------------------------------------------------------------
def partition_partials_fp64(q, k_cache, v_cache, seq_lens, scale, chunk, num_partitions,
                            page_table=None, page_size=0, v_is_k_prefix=False, ov_depth=None):
    """Per-partition partials of the split-K method.

    Partition p of sequence b covers keys [p*chunk, min((p+1)*chunk, L_b)).
    Returns (m [B,Hq,P], l [B,Hq,P], O [B,Hq,P,Dv]) with m the raw-unit row max,
    l = sum_t exp(scale*(x_t - m)) and O the partition's output already divided
    by l (fa4_splitk_combine_write, second paragraph: the staged O_cta is
    normalised). A partition with no keys holds (m, l, O) = (-inf, 0, 0).
    """
    B, Hq, Hkv, g, Dqk, Dv = _dims(q, k_cache, v_cache, v_is_k_prefix, ov_depth)
    P = int(num_partitions)
    m = np.full((B, Hq, P), -np.inf)
    l = np.zeros((B, Hq, P))
    O = np.zeros((B, Hq, P, Dv))
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        for kvh in range(Hkv):
            qg, K, V = _gather(q, k_cache, v_cache, b, kvh, g, L, page_table, page_size,
                               v_is_k_prefix, Dv)
            x = qg @ K.T
            hs = slice(kvh * g, (kvh + 1) * g)
            for p in range(P):
                lo, hi = p * chunk, min((p + 1) * chunk, L)
                if lo >= hi:
                    continue
                xp = x[:, lo:hi]
                mp = xp.max(axis=1, keepdims=True)
                e = np.exp(scale * (xp - mp))
                lp = e.sum(axis=1, keepdims=True)
                m[b, hs, p] = mp[:, 0]
                l[b, hs, p] = lp[:, 0]
                O[b, hs, p] = (e @ V[lo:hi]) / lp
    return m, l, O


def equal_share_pieces(seq_lens, workers, tile=32, min_tiles=8):
    """Partition boundaries of the equal-share split schedule.

    The pages fix the number of partitions per sequence at compile time and say
    nothing about how a runtime would cut a batch of unequal sequences; this is
    the schedule the automatic split uses instead of fixed-length chunks. The
    ``tile``-key tiles of all sequences are laid end to end in batch order and
    numbered 0 .. U-1 (sequence b has ceil(L_b / tile) of them). With
    W = min(workers, max(1, floor(U / min_tiles))) workers (so a worker owns at
    least min_tiles tiles whenever U >= min_tiles), worker w owns tiles
    floor(w U / W) .. floor((w + 1) U / W) - 1. Every non-empty overlap of a
    worker's tiles with a sequence's tiles is one partition of that sequence;
    partitions are numbered (slots) sequence by sequence, and by worker within a
    sequence.

    Returns (pieces, first, count): pieces is a list of (b, key_start, key_end,
    slot) with key_end clipped to L_b; first[b] / count[b] are the first slot and
    the number of partitions of sequence b (first[b] = the next free slot and
    count[b] = 0 for an empty sequence).
    """
    lens = [max(0, int(x)) for x in seq_lens]
    tiles = [-(-L // tile) for L in lens]
    U = sum(tiles)
    W = min(int(workers), max(1, U // min_tiles))
    bounds = [w * U // W for w in range(W + 1)]
    pieces, first, count = [], [], []
    slot, pre = 0, 0
    for b, (L, n) in enumerate(zip(lens, tiles)):
        first.append(slot)
        c = 0
        for w in range(W):
            lo, hi = max(bounds[w], pre), min(bounds[w + 1], pre + n)
            if lo < hi:
                pieces.append((b, (lo - pre) * tile, min((hi - pre) * tile, L), slot))
                slot += 1
                c += 1
        count.append(c)
        pre += n
    return pieces, first, count


def range_partials_fp64(q, k_cache, v_cache, seq_lens, scale, pieces, page_table=None, page_size=0,
                        v_is_k_prefix=False, ov_depth=None, k_scale=None, v_scale=None, k_rope=None):
    """Pass-1 partials over explicit key ranges.

    pieces: (b, key_start, key_end, slot) tuples as ``equal_share_pieces``
    returns. For each piece and q head: the raw-unit max m, the sum
    l = sum_t exp(scale * (x_t - m)) and the normalised O over keys
    key_start .. key_end - 1 of sequence b (fa4_splitk_combine_write, second
    paragraph). Returns (m [S, Hq], l [S, Hq], O [S, Hq, Dv]) indexed by slot,
    S = 1 + the largest slot; slots no piece names hold (-inf, 0, 0).
    """
    B, Hq, Hkv, g, Dqk, Dv = _dims(q, k_cache, v_cache, v_is_k_prefix, ov_depth, k_rope)
    S = 1 + max((pc[3] for pc in pieces), default=-1)
    m = np.full((S, Hq), -np.inf)
    l = np.zeros((S, Hq))
    O = np.zeros((S, Hq, Dv))
    for b, lo, hi, slot in pieces:
        for kvh in range(Hkv):
            qg, K, V = _gather(q, k_cache, v_cache, b, kvh, g, hi, page_table, page_size,
                               v_is_k_prefix, Dv, k_scale, v_scale, k_rope)
            x = qg @ K[lo:hi].T
            mp = x.max(axis=1, keepdims=True)
            e = np.exp(scale * (x - mp))
            lp = e.sum(axis=1, keepdims=True)
            hs = slice(kvh * g, (kvh + 1) * g)
            m[slot, hs] = mp[:, 0]
            l[slot, hs] = lp[:, 0]
            O[slot, hs] = (e @ V[lo:hi]) / lp
    return m, l, O


# ---------------------------------------------------------------------------
# split-K pass 2: the LSE combine
# ---------------------------------------------------------------------------
def combine_fp64(m, l, O, scale):
    """Merge P partitions per row with the log-sum-exp combine.

    m, l: [..., P]; O: [..., P, Dv]. Follows fa4_splitk_combine_write
    (first paragraph) with c = scale * log2(e). Partitions with l == 0 get
    weight 0; a row whose partitions are all empty gives O = 0, LSE = -inf.
    Returns (O [..., Dv], LSE [...]).
    """
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    O = np.asarray(O, dtype=np.float64)
    c = scale * LOG2E
    lead = m.shape[:-1]
    Dv = O.shape[-1]
    out = np.zeros(lead + (Dv,))
    lse = np.full(lead, -np.inf)
    for idx in np.ndindex(*lead):
        live = l[idx] > 0
        if not live.any():
            continue
        mp, lp, Op = m[idx][live], l[idx][live], O[idx][live]
        gmax = mp.max()
        e = np.exp2((mp - gmax) * c)
        gsum = (lp * e).sum()
        w = lp * e / gsum
        out[idx] = (w[:, None] * Op).sum(axis=0)
        lse[idx] = scale * gmax + math.log(gsum)
    return out, lse


def decode_attention_splitk_fp64(q, k_cache, v_cache, seq_lens, scale, chunk, page_table=None,
                                 page_size=0, v_is_k_prefix=False, ov_depth=None):
    """Split-K pass 1 then the LSE combine, the two steps in the pages' order."""
    max_len = int(np.max(seq_lens)) if len(seq_lens) else 0
    P = max(1, -(-max_len // chunk))
    m, l, O = partition_partials_fp64(q, k_cache, v_cache, seq_lens, scale, chunk, P,
                                      page_table, page_size, v_is_k_prefix, ov_depth)
    return combine_fp64(m, l, O, scale)


# ---------------------------------------------------------------------------
# the bf16 cast
# ---------------------------------------------------------------------------
def bf16_round_fp64(x):
    """Round fp64 values to the nearest bf16 (ties to even), returned as fp64.

    bf16 keeps 8 significant bits and fp32's exponent range: normal values
    have the form k * 2^(e-7) with 128 <= |k| < 256; below 2^-126 the spacing
    is the fixed subnormal step 2^-133; beyond the largest finite bf16 the
    result is +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    mant, expo = np.frexp(xf)                      # xf = mant * 2^expo, 0.5 <= |mant| < 1
    normal = np.abs(xf) >= 2.0 ** -126
    r = np.empty_like(xf)
    r[normal] = np.ldexp(np.rint(np.ldexp(mant[normal], 8)), expo[normal] - 8)
    sub = ~normal
    r[sub] = np.ldexp(np.rint(np.ldexp(xf[sub], 133)), -133)
    max_bf16 = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r[np.abs(r) > max_bf16] = np.copysign(np.inf, r[np.abs(r) > max_bf16])
    out[fin] = r
    return out
