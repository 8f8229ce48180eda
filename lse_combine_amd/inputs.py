"""Seeded synthetic decode-attention inputs (data generation only, no attention math).

Both the HIP path's tests/benchmark and the CPU oracle consume these tensors,
so this module holds nothing but random draws and index bookkeeping. Tensors
are generated on the CPU with ``torch.Generator('cpu')`` so that both sides
see identical bits; callers copy them to the device themselves.

Draw order for every workload: sequence lengths (when variable), page
permutation (when paged), q, K, V (V is not drawn when it aliases K).
Values are ``torch.randn`` in fp32, cast to bf16 (round-to-nearest-even) for
bf16 workloads.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass
class Case:
    """One decode step's inputs plus the metadata the C ABI needs."""

    name: str
    q: torch.Tensor                    # [B, Hq, Dqk]
    k_cache: torch.Tensor              # contiguous [B, Lcap, Hkv, Dqk] or paged [N, ps, Hkv, Dqk]
    v_cache: torch.Tensor | None       # same layout with Dv; None when V is the prefix of K
    seq_lens: torch.Tensor             # int32 [B]
    page_table: torch.Tensor | None    # int32 [B, max_pages] (padding -1) or None
    page_size: int
    scale: float
    num_splits: int                    # 0 = automatic split selection
    v_is_k_prefix: bool = False
    ov_depth: int = 0
    meta: dict = field(default_factory=dict)
    # fp8 caches: the caches hold E4M3 codes (uint8) and these fp32 per-token scales,
    # contiguous [B, Hkv, Lcap] / paged [N, Hkv, ps] (tokens innermost); None otherwise
    k_scale: torch.Tensor | None = None
    v_scale: torch.Tensor | None = None
    # rotary columns stored apart: the last Dqk - nope columns of every K row, bf16, in the
    # cache's layout ([..., Hkv, rope]); k_cache then holds the first nope columns
    k_rope: torch.Tensor | None = None

    @property
    def batch(self):
        return self.q.shape[0]

    @property
    def num_q_heads(self):
        return self.q.shape[-2]

    @property
    def q_len(self):
        return self.q.shape[1] if self.q.dim() == 4 else 1

    @property
    def num_kv_heads(self):
        return self.k_cache.shape[2]

    @property
    def qk_depth(self):
        return self.q.shape[-1]

    @property
    def kv_fp8(self):
        return self.k_cache.dtype == torch.uint8

    @property
    def dtype_name(self):
        q = {torch.float32: "f32", torch.bfloat16: "bf16"}[self.q.dtype]
        return q + "/fp8-kv" if self.kv_fp8 else q

    @property
    def nope_depth(self):
        """K columns held by k_cache (all of them unless the rotary ones are stored apart)."""
        return self.k_cache.shape[-1]

    def kv_bytes(self) -> int:
        """Bytes of K and V that attention must read (attended tokens only)."""
        tokens = int(self.seq_lens.clamp(min=0).sum())
        es = self.k_cache.element_size()
        per_tok = self.num_kv_heads * self.nope_depth * es
        if not self.v_is_k_prefix:
            per_tok += self.num_kv_heads * self.ov_depth * es
        if self.k_rope is not None:
            per_tok += self.num_kv_heads * self.k_rope.shape[-1] * self.k_rope.element_size()
        # the per-token scales of an fp8 cache are read too (4 bytes per token and kv head)
        for sc in (self.k_scale, self.v_scale):
            if sc is not None:
                per_tok += self.num_kv_heads * 4
        return tokens * per_tok

    def flops(self) -> int:
        tokens = int(self.seq_lens.clamp(min=0).sum())
        return 2 * self.q_len * self.num_q_heads * tokens * (self.qk_depth + self.ov_depth)


def _randn(gen, shape, dtype):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


def make_case(name="case", *, batch, num_q_heads, num_kv_heads, qk_depth, ov_depth=None,
              dtype=torch.bfloat16, page_size=0, seq_lens=None, len_range=None, kv_capacity=None,
              num_splits=0, seed=0, v_is_k_prefix=False, scale=None, poison=False,
              spare_pages=0, q_scale=1.0, page_table_width=None, kv_fp8=False, v_scaled=True,
              q_len=1, rope_apart=0) -> Case:
    """Build a seeded case.

    Exactly one of ``seq_lens`` (a list of lengths) or ``len_range``
    ((lo, hi) inclusive, drawn with ``torch.randint``) is given.
    Paged pools hold exactly sum(ceil(L_b / page_size)) pages (+ ``spare_pages``)
    in a seeded random order; page-table padding is -1. ``poison`` fills every
    cache slot that no sequence attends (tail of last pages, spare pages,
    contiguous slots past L_b) with NaN so that a kernel reading them shows up.
    ``q_scale`` multiplies q after the draw (large-logit tests).
    ``q_len`` > 1: q is [B, q_len, Hq, Dqk], the sequences' last q_len positions.
    ``kv_fp8``: K and V are drawn as above (fp32) and stored as E4M3 codes with a
    per-(token, kv head) scale amax / 448 (``v_scaled=False``: V codes of the unscaled
    values, no V scale); q stays in ``dtype``.
    ``rope_apart`` > 0: the last ``rope_apart`` columns of every K row (drawn with the
    rest) are stored apart as bf16 (``k_rope``); k_cache keeps the first
    qk_depth - rope_apart columns (quantised alone when ``kv_fp8``).
    """
    ov_depth = qk_depth if ov_depth is None else ov_depth
    gen = torch.Generator("cpu")
    gen.manual_seed(seed)
    if seq_lens is None:
        lo, hi = len_range
        lens = torch.randint(lo, hi + 1, (batch,), generator=gen, dtype=torch.int64)
    else:
        lens = torch.as_tensor(seq_lens, dtype=torch.int64)
        assert lens.numel() == batch
    lens32 = lens.to(torch.int32)
    pos_lens = lens.clamp(min=0)
    if page_size > 0:
        pages_per_seq = [(-(-int(L) // page_size)) for L in pos_lens]
        n_pages = sum(pages_per_seq) + spare_pages
        n_pages = max(n_pages, 1)
        perm = torch.randperm(n_pages, generator=gen).to(torch.int32)
        width = page_table_width or max(1, max(pages_per_seq) if pages_per_seq else 1)
        pt = torch.full((batch, width), -1, dtype=torch.int32)
        off = 0
        for b, npg in enumerate(pages_per_seq):
            pt[b, :npg] = perm[off:off + npg]
            off += npg
        kv_shape_k = (n_pages, page_size, num_kv_heads, qk_depth)
        kv_shape_v = (n_pages, page_size, num_kv_heads, ov_depth)
    else:
        pt = None
        cap = kv_capacity or max(1, int(pos_lens.max()) if batch else 1)
        kv_shape_k = (batch, cap, num_kv_heads, qk_depth)
        kv_shape_v = (batch, cap, num_kv_heads, ov_depth)
    q_shape = (batch, num_q_heads, qk_depth) if q_len == 1 else (batch, q_len, num_q_heads, qk_depth)
    q = _randn(gen, q_shape, dtype)
    if q_scale != 1.0:
        q = (q.float() * q_scale).to(dtype)
    kv_dtype = torch.float32 if kv_fp8 else dtype
    k = _randn(gen, kv_shape_k, kv_dtype)
    v = None if v_is_k_prefix else _randn(gen, kv_shape_v, kv_dtype)
    k_rope = None
    if rope_apart:
        nope = qk_depth - rope_apart
        k_rope = k[..., nope:].to(torch.bfloat16).contiguous()
        k = k[..., :nope].contiguous()
    k_scale = v_scale = None
    if kv_fp8:
        k, k_scale = _to_fp8(k, True)
        if v is not None:
            v, v_scale = _to_fp8(v, v_scaled)
    if poison:
        _poison(k, v, pos_lens, pt, page_size)
        if k_rope is not None:
            _poison(k_rope, None, pos_lens, pt, page_size)
        for sc in (k_scale, v_scale):
            if sc is not None:   # [rows, Hkv, slots] -> slots second, like the caches
                _poison(sc.transpose(1, 2), None, pos_lens, pt, page_size)
    sc = scale if scale is not None else 1.0 / math.sqrt(qk_depth)
    return Case(name=name, q=q, k_cache=k, v_cache=v, seq_lens=lens32, page_table=pt,
                page_size=page_size, scale=sc, num_splits=num_splits,
                v_is_k_prefix=v_is_k_prefix, ov_depth=ov_depth, meta={"seed": seed},
                k_scale=k_scale, v_scale=v_scale, k_rope=k_rope)


FP8_E4M3_MAX = 448.0   # largest finite E4M3 magnitude


def _to_fp8(x, scaled):
    """fp32 [rows, slots, Hkv, D] -> (E4M3 codes as uint8, fp32 scales [rows, Hkv, slots])."""
    if scaled:
        s = (x.abs().amax(dim=-1) / FP8_E4M3_MAX).clamp(min=2.0 ** -30)
        codes = (x / s[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
        return codes, s.permute(0, 2, 1).contiguous()
    return x.clamp(-FP8_E4M3_MAX, FP8_E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8), None


def _poison(k, v, lens, pt, page_size):
    """Fill the slots no sequence attends with NaN, in place (k and v are [rows, slots, ...],
    views included)."""
    nan = float("nan") if k.dtype != torch.uint8 else 0x7F   # (0x7F: an E4M3 NaN code)
    if pt is None:
        for b, L in enumerate(lens.tolist()):
            k[b, L:] = nan
            if v is not None:
                v[b, L:] = nan
        return
    used = torch.zeros(k.shape[0], k.shape[1], dtype=torch.bool)
    for b, L in enumerate(lens.tolist()):
        for t0 in range(0, L, page_size):
            n = min(page_size, L - t0)
            used[int(pt[b, t0 // page_size]), :n] = True
    k[~used] = nan
    if v is not None:
        v[~used] = nan


# ---------------------------------------------------------------------------
# the five named decode workloads
# ---------------------------------------------------------------------------
WORKLOADS = {
    # batch 1, 1 q head / 1 kv head, D 128, L 1024, fp32, 4 partitions of 256 keys, contiguous
    "tiny": dict(seed=1, batch=1, num_q_heads=1, num_kv_heads=1, qk_depth=128,
                 dtype=torch.float32, page_size=0, seq_lens=[1024], num_splits=4),
    # batch 8, 32/8 heads (group 4), D 128, L 4096, bf16, contiguous, 8 splits
    "gqa": dict(seed=2, batch=8, num_q_heads=32, num_kv_heads=8, qk_depth=128,
                dtype=torch.bfloat16, page_size=0, seq_lens=[4096] * 8, num_splits=8),
    # batch 32, 64/8 heads (group 8), D 128, bf16, page 64, L_b ~ U[512, 32768], automatic splits
    "paged_gqa": dict(seed=3, batch=32, num_q_heads=64, num_kv_heads=8, qk_depth=128,
                      dtype=torch.bfloat16, page_size=64, len_range=(512, 32768),
                      num_splits=0, page_table_width=512),
    # batch 1, 32/4 heads (group 8), D 128, L 131072, bf16, page 64, 64 splits
    "long": dict(seed=4, batch=1, num_q_heads=32, num_kv_heads=4, qk_depth=128,
                 dtype=torch.bfloat16, page_size=64, seq_lens=[131072], num_splits=64),
    # batch 16, 128 q heads / 1 kv head, qk 576 (512 + 64 rotary), ov 512 = K[..., :512],
    # L 8192, bf16, page 64, 8 splits
    "latent": dict(seed=5, batch=16, num_q_heads=128, num_kv_heads=1, qk_depth=576, ov_depth=512,
                   dtype=torch.bfloat16, page_size=64, seq_lens=[8192] * 16, num_splits=8,
                   v_is_k_prefix=True),
    # the paged GQA workload with two queries per sequence (e.g. one speculative token):
    # 2 x 8 (query, head) columns per kv head
    "paged_gqa_q2": dict(seed=3, batch=32, num_q_heads=64, num_kv_heads=8, qk_depth=128,
                         dtype=torch.bfloat16, page_size=64, len_range=(512, 32768),
                         num_splits=0, page_table_width=512, q_len=2),
    # the paged GQA workload with an fp8 (E4M3) K/V cache and per-token K and V scales
    # (same lengths, pages and draws; bf16 q)
    "paged_gqa_fp8": dict(seed=3, batch=32, num_q_heads=64, num_kv_heads=8, qk_depth=128,
                          dtype=torch.bfloat16, page_size=64, len_range=(512, 32768),
                          num_splits=0, page_table_width=512, kv_fp8=True),
    # GLM-style widths, one kv head per q head: qk 256 = 192 nope + 64 rotary columns (the
    # rotary ones stored apart as bf16), V / output 256 (not the nope width); batch 32,
    # 16 heads, bf16, page 64, L_b ~ U[512, 8192], automatic splits
    "paged_glm": dict(seed=6, batch=32, num_q_heads=16, num_kv_heads=16, qk_depth=256, ov_depth=256,
                      dtype=torch.bfloat16, page_size=64, len_range=(512, 8192), num_splits=0,
                      page_table_width=128, rope_apart=64),
    # the latent workload with its 64 rotary columns stored apart (bf16 tensor of their own;
    # the same draws, so the same values as "latent")
    "latent_rope_apart": dict(seed=5, batch=16, num_q_heads=128, num_kv_heads=1, qk_depth=576, ov_depth=512,
                              dtype=torch.bfloat16, page_size=64, seq_lens=[8192] * 16, num_splits=8,
                              v_is_k_prefix=True, rope_apart=64),
    # GLM-style widths with one kv head for all 128 q heads: q.K 256 = 192 nope + 64 rotary
    # (stored apart, bf16), V 256 of its own; batch 16, L 8192, page 64, 8 splits
    "glm_mqa": dict(seed=7, batch=16, num_q_heads=128, num_kv_heads=1, qk_depth=256, ov_depth=256,
                    dtype=torch.bfloat16, page_size=64, seq_lens=[8192] * 16, num_splits=8, rope_apart=64),
    # the latent workload over an fp8 cache: the 512 nope columns as E4M3 codes with a
    # per-token scale (V = their first 512 columns, read with the same scale), the 64 rotary
    # columns stored apart in bf16 (same draws as "latent")
    "latent_fp8": dict(seed=5, batch=16, num_q_heads=128, num_kv_heads=1, qk_depth=576, ov_depth=512,
                       dtype=torch.bfloat16, page_size=64, seq_lens=[8192] * 16, num_splits=8,
                       v_is_k_prefix=True, rope_apart=64, kv_fp8=True),
    # the same over an fp8 cache: nope columns and V as E4M3 codes with per-token scales, the
    # rotary columns bf16 apart (same draws as "glm_mqa")
    "glm_mqa_fp8": dict(seed=7, batch=16, num_q_heads=128, num_kv_heads=1, qk_depth=256, ov_depth=256,
                        dtype=torch.bfloat16, page_size=64, seq_lens=[8192] * 16, num_splits=8, rope_apart=64,
                        kv_fp8=True),
    # the latent workload over an fp8 cache with the 64 rotary columns as codes in the K rows:
    # one per-token scale for all 576 columns, V = the first 512 codes (same draws as "latent")
    "latent_fp8_inline": dict(seed=5, batch=16, num_q_heads=128, num_kv_heads=1, qk_depth=576, ov_depth=512,
                              dtype=torch.bfloat16, page_size=64, seq_lens=[8192] * 16, num_splits=8,
                              v_is_k_prefix=True, kv_fp8=True),
    # one kv head for 48 q heads at head dim 128 (multi-query attention): the group runs as
    # three virtual kv heads of 16 columns on the matrix-core kernel; batch 32, bf16, page 64,
    # L_b ~ U[512, 8192], automatic splits
    "paged_mqa": dict(seed=9, batch=32, num_q_heads=48, num_kv_heads=1, qk_depth=128,
                      dtype=torch.bfloat16, page_size=64, len_range=(512, 8192), num_splits=0,
                      page_table_width=128),
    # heads of 64 dimensions: batch 32, 32 q heads / 8 kv heads (group 4), bf16, page 64,
    # L_b ~ U[512, 8192], automatic splits
    "paged_gqa_d64": dict(seed=10, batch=32, num_q_heads=32, num_kv_heads=8, qk_depth=64,
                          dtype=torch.bfloat16, page_size=64, len_range=(512, 8192), num_splits=0,
                          page_table_width=128),
    # one q head per kv head (multi-head attention, group 1): batch 32, 32 heads, head dim
    # 128, bf16, page 64, L_b ~ U[512, 8192], automatic splits
    "paged_mha": dict(seed=8, batch=32, num_q_heads=32, num_kv_heads=32, qk_depth=128,
                      dtype=torch.bfloat16, page_size=64, len_range=(512, 8192), num_splits=0,
                      page_table_width=128),
    # the same with the nope columns and V as fp8 (E4M3) with per-token scales; the rotary
    # columns stay bf16
    "paged_glm_fp8": dict(seed=6, batch=32, num_q_heads=16, num_kv_heads=16, qk_depth=256, ov_depth=256,
                          dtype=torch.bfloat16, page_size=64, len_range=(512, 8192), num_splits=0,
                          page_table_width=128, rope_apart=64, kv_fp8=True),
}


def workload(name: str, **overrides) -> Case:
    spec = dict(WORKLOADS[name])
    spec.update(overrides)
    return make_case(name, **spec)


def to_device(case: Case, device="cuda") -> Case:
    """Copy of ``case`` with every tensor moved to ``device`` (bit-identical values)."""
    def mv(t):
        return None if t is None else t.to(device).contiguous()
    return Case(name=case.name, q=mv(case.q), k_cache=mv(case.k_cache), v_cache=mv(case.v_cache),
                seq_lens=mv(case.seq_lens), page_table=mv(case.page_table), page_size=case.page_size,
                scale=case.scale, num_splits=case.num_splits, v_is_k_prefix=case.v_is_k_prefix,
                ov_depth=case.ov_depth, meta=dict(case.meta), k_scale=mv(case.k_scale),
                v_scale=mv(case.v_scale), k_rope=mv(case.k_rope))
