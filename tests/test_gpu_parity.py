"""GPU parity: the HIP decode step (through the C ABI) against the fp64 oracle.

Sizes span several key tiles, partitions and ragged tails while the oracle
finishes in seconds. Tolerances are stated in parity_utils.
"""

import dataclasses

import numpy as np
import pytest
import torch

from lse_combine_amd import api
from lse_combine_amd.inputs import make_case, to_device, workload
from oracle import combine_fp64, equal_share_pieces, partition_partials_fp64, range_partials_fp64
from parity_utils import assert_parity, np32, oracle_for

pytestmark = pytest.mark.gpu


def run(case, **kw):
    dc = to_device(case)
    out, lse, o32 = api.case_call(dc, return_lse=True, return_o32=True, **kw)
    torch.cuda.synchronize()
    return out, lse, o32


def check_case(case, what, **kw):
    print(f"[parity] {what}", flush=True)
    out, lse, o32 = run(case, **kw)
    O, LSE = oracle_for(case)
    assert_parity(out, lse, o32, O, LSE, what=what)
    return out, lse, o32


# ---------------------------------------------------------------------------
# kernel families x layouts x group sizes, reduced sizes with ragged tails
# ---------------------------------------------------------------------------
CASES = [
    # name, make_case kwargs, kernel
    ("tiny_fp32_full", dict(batch=1, num_q_heads=1, num_kv_heads=1, qk_depth=128, dtype=torch.float32,
                            seq_lens=[1024], num_splits=4, seed=1), "auto"),
    ("fp32_g4_contig_ragged", dict(batch=3, num_q_heads=8, num_kv_heads=2, qk_depth=128, dtype=torch.float32,
                                   seq_lens=[1000, 77, 300], num_splits=3, seed=21), "auto"),
    ("fp32_g16_paged16", dict(batch=2, num_q_heads=16, num_kv_heads=1, qk_depth=128, dtype=torch.float32,
                              page_size=16, seq_lens=[517, 1201], num_splits=0, seed=22), "auto"),
    ("bf16_g1_fma", dict(batch=3, num_q_heads=4, num_kv_heads=4, qk_depth=128, seq_lens=[2049, 1, 640],
                         num_splits=5, seed=23), "fma"),
    ("bf16_g1_auto", dict(batch=3, num_q_heads=4, num_kv_heads=4, qk_depth=128, page_size=64,
                          seq_lens=[2049, 1, 640], num_splits=0, seed=23), "auto"),
    ("bf16_g1_mfma", dict(batch=3, num_q_heads=4, num_kv_heads=4, qk_depth=128, seq_lens=[2049, 1, 640],
                          num_splits=5, seed=23), "mfma"),
    ("bf16_g4_contig", dict(batch=2, num_q_heads=8, num_kv_heads=2, qk_depth=128, seq_lens=[4096, 1000],
                            num_splits=8, seed=24), "auto"),
    ("bf16_g4_fma", dict(batch=2, num_q_heads=8, num_kv_heads=2, qk_depth=128, seq_lens=[4096, 1000],
                         num_splits=8, seed=24), "fma"),
    ("bf16_g8_paged64_auto", dict(batch=5, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=64,
                                  len_range=(1, 5000), num_splits=0, seed=25), "auto"),
    ("bf16_g8_paged64_splits7", dict(batch=4, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=64,
                                     len_range=(100, 3000), num_splits=7, seed=26), "auto"),
    ("bf16_g6_paged32", dict(batch=3, num_q_heads=12, num_kv_heads=2, qk_depth=128, page_size=32,
                             seq_lens=[33, 1500, 64], num_splits=2, seed=27), "auto"),
    ("bf16_g16_paged32", dict(batch=2, num_q_heads=32, num_kv_heads=2, qk_depth=128, page_size=32,
                              seq_lens=[777, 2048], num_splits=3, seed=28), "auto"),
    ("bf16_g8_paged16", dict(batch=3, num_q_heads=8, num_kv_heads=1, qk_depth=128, page_size=16,
                             seq_lens=[1000, 15, 257], num_splits=4, seed=29), "auto"),
    ("bf16_g2_paged48_general", dict(batch=2, num_q_heads=4, num_kv_heads=2, qk_depth=128, page_size=48,
                                     seq_lens=[1000, 97], num_splits=0, seed=30), "auto"),
    ("bf16_g8_one_split", dict(batch=3, num_q_heads=8, num_kv_heads=1, qk_depth=128, page_size=64,
                               seq_lens=[3000, 64, 1], num_splits=1, seed=31), "auto"),
    ("bf16_g8_v_is_k", dict(batch=2, num_q_heads=8, num_kv_heads=1, qk_depth=128, page_size=64,
                            seq_lens=[700, 1300], num_splits=3, seed=32, v_is_k_prefix=True), "auto"),
    # latent-shared: one kv head, K rows of 576 (512 + 64 rotary), V = K[..., :512]
    ("latent_g64_paged64", dict(batch=2, num_q_heads=64, num_kv_heads=1, qk_depth=576, ov_depth=512,
                                page_size=64, seq_lens=[700, 1313], num_splits=3, seed=33,
                                v_is_k_prefix=True), "auto"),
    ("latent_g128_paged64_one_split", dict(batch=2, num_q_heads=128, num_kv_heads=1, qk_depth=576,
                                           ov_depth=512, page_size=64, seq_lens=[90, 31], num_splits=1,
                                           seed=34, v_is_k_prefix=True), "auto"),
    ("latent_g16_contig", dict(batch=3, num_q_heads=16, num_kv_heads=1, qk_depth=576, ov_depth=512,
                               seq_lens=[100, 33, 1], num_splits=2, seed=35, v_is_k_prefix=True), "auto"),
    ("latent_g48_paged16", dict(batch=2, num_q_heads=48, num_kv_heads=1, qk_depth=576, ov_depth=512,
                                        page_size=16, seq_lens=[517, 64], num_splits=0, seed=36,
                                        v_is_k_prefix=True), "auto"),
    # 80 heads: one full block of 64 and a second block with one of its four head blocks
    ("latent_g80_paged32", dict(batch=3, num_q_heads=80, num_kv_heads=1, qk_depth=576, ov_depth=512,
                                page_size=32, seq_lens=[1025, 32, 2], num_splits=4, seed=37,
                                v_is_k_prefix=True), "auto"),
]


@pytest.mark.parametrize("name,kw,kernel", CASES, ids=[c[0] for c in CASES])
def test_parity(name, kw, kernel):
    case = make_case(name, **kw)
    check_case(case, name, kernel=kernel)


def test_empty_and_tiny_sequences():
    # L = 0 rows give O = 0 and LSE = -inf; L = 1 gives V_0
    case = make_case("edge", batch=4, num_q_heads=8, num_kv_heads=1, qk_depth=128, page_size=64,
                     seq_lens=[0, 1, 2, 65], num_splits=0, seed=40)
    out, lse, o32 = check_case(case, "empty/tiny")
    assert torch.all(out[0].float() == 0) and torch.all(torch.isneginf(lse[0]))


def test_poisoned_unattended_slots_are_never_read():
    for pg, kern, n in [(64, "auto", 3), (16, "auto", 3), (0, "auto", 3), (64, "fma", 3), (64, "auto", 0),
                        (0, "auto", 0)]:
        case = make_case("poison", batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=pg,
                         seq_lens=[100, 1, 1025], num_splits=n, seed=41, poison=True, spare_pages=3)
        out, lse, o32 = check_case(case, f"poison ps={pg} {kern} splits={n}", kernel=kern)
        assert torch.isfinite(o32).all()


@pytest.mark.parametrize("lens", [[0, 0, 0], [0] * 70 + [5], [3000] + [0] * 100 + [1, 2]],
                         ids=["all_empty", "70_empty_then_one", "long_then_100_empty"])
def test_automatic_split_edge_batches(lens):
    case = make_case("auto_edge", batch=len(lens), num_q_heads=8, num_kv_heads=1, qk_depth=128, page_size=64,
                     seq_lens=lens, num_splits=0, seed=46)
    out, lse, o32 = check_case(case, f"auto edge B={len(lens)}")
    for b, L in enumerate(lens):
        if L == 0:
            assert torch.all(out[b].float() == 0) and torch.all(torch.isneginf(lse[b]))


def test_automatic_split_many_sequences():
    # more than 64 sequences: the schedule scans seq_lens in several chunks
    case = make_case("auto_many", batch=150, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=32,
                     len_range=(0, 700), num_splits=0, seed=47)
    check_case(case, "auto B=150")


def test_large_logits_overflow_safety():
    # q scaled by 64: raw scores reach several hundred; the fp32 score's own rounding
    # (~1e-4 absolute) then bounds the O agreement, so o32 is checked at 1e-4
    case = make_case("big", batch=2, num_q_heads=8, num_kv_heads=1, qk_depth=128, page_size=64,
                     seq_lens=[3000, 500], num_splits=4, seed=42, q_scale=64.0)
    out, lse, o32 = run(case)
    O, LSE = oracle_for(case)
    assert torch.isfinite(o32).all()
    assert_parity(out, lse, o32, O, LSE, o32_row_rtol=1e-4, what="large logits")


def test_latent_fused_entry_point_writes_every_row():
    # the fold in pass 1 forced on a latent-shared problem: the last workgroup of each column
    # block combines; outputs (rows of an empty sequence included) match the oracle
    print("[parity] latent through the fused entry point", flush=True)
    case = make_case("latent_fused", batch=3, num_q_heads=64, num_kv_heads=1, qk_depth=576, ov_depth=512,
                     page_size=64, seq_lens=[900, 0, 65], num_splits=2, seed=38, v_is_k_prefix=True)
    dc = to_device(case)
    prob = api.make_problem(dc.q, dc.k_cache, dc.v_cache, dc.page_table, page_size=case.page_size,
                            v_is_k_prefix=True, ov_depth=case.ov_depth)
    ws = torch.zeros(api.workspace_bytes(prob, case.num_splits), dtype=torch.uint8, device="cuda")
    rows = api.row_shape(prob)
    out = torch.full(rows + (prob.ov_depth,), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full(rows, float("nan"), dtype=torch.float32, device="cuda")
    o32 = torch.full(rows + (prob.ov_depth,), float("nan"), dtype=torch.float32, device="cuda")
    api.case_call(dc, out=out, lse=lse, o32=o32, fused="force", workspace=ws)
    torch.cuda.synchronize()
    O, LSE = oracle_for(case)
    assert_parity(out, lse, o32, O, LSE, what="latent fused entry point")


def test_latent_large_logits_take_the_second_pass():
    # raw scores of several thousand: later tiles exceed the first tile's max by more than
    # the kernel's fixed-reference headroom, so the partition is run again with its exact max
    case = make_case("big_latent", batch=2, num_q_heads=64, num_kv_heads=1, qk_depth=576, ov_depth=512,
                     page_size=64, seq_lens=[1300, 700], num_splits=2, seed=48, q_scale=64.0,
                     v_is_k_prefix=True)
    out, lse, o32 = run(case)
    O, LSE = oracle_for(case)
    assert torch.isfinite(o32).all()
    assert_parity(out, lse, o32, O, LSE, o32_row_rtol=1e-4, what="latent large logits")


# ---------------------------------------------------------------------------
# the shared-kv-head kernel: one kv head for every q head. Latent rows (q.K 576 = 512 nope
# + 64 rotary, V = the first 512 nope columns) and GLM-style widths with a V of its own
# (q.K 256 = 192 nope + 64 rotary, V 256); rotary columns in the K rows or stored apart,
# one or several queries, column counts that are not multiples of 16 or 64
# ---------------------------------------------------------------------------
LATENT = dict(num_kv_heads=1, qk_depth=576, ov_depth=512, v_is_k_prefix=True)
GLM_MQA = dict(num_kv_heads=1, qk_depth=256, ov_depth=256)
SHARED = [
    ("latent_apart_g64_paged64", dict(batch=2, num_q_heads=64, page_size=64, seq_lens=[700, 1313], num_splits=3,
                                      seed=160, rope_apart=64, **LATENT)),
    ("latent_apart_g128_contig", dict(batch=3, num_q_heads=128, seq_lens=[100, 33, 1], num_splits=2, seed=161,
                                      rope_apart=64, **LATENT)),
    ("latent_apart_g40_paged16", dict(batch=2, num_q_heads=40, page_size=16, seq_lens=[517, 64],
                                      num_splits=0, seed=162, rope_apart=64, **LATENT)),
    ("latent_q2_g64_paged64", dict(batch=3, num_q_heads=64, page_size=64, seq_lens=[1, 900, 2100], num_splits=3,
                                   seed=163, q_len=2, **LATENT)),
    ("latent_q3_g20_apart_paged32", dict(batch=2, num_q_heads=20, page_size=32, seq_lens=[2, 1500], num_splits=2,
                                         seed=164, q_len=3, rope_apart=64, **LATENT)),
    ("latent_g24_paged64", dict(batch=3, num_q_heads=24, page_size=64, seq_lens=[1025, 32, 2], num_splits=4,
                                seed=165, **LATENT)),
    ("latent_apart_poisoned", dict(batch=3, num_q_heads=64, page_size=64, seq_lens=[100, 1, 1025], num_splits=2,
                                   seed=166, rope_apart=64, poison=True, spare_pages=3, **LATENT)),
    ("glm_mqa_g64_apart_paged64", dict(batch=2, num_q_heads=64, page_size=64, seq_lens=[1500, 333], num_splits=3,
                                       seed=170, rope_apart=64, **GLM_MQA)),
    ("glm_mqa_g128_inline_contig", dict(batch=2, num_q_heads=128, seq_lens=[2000, 77], num_splits=2, seed=171,
                                        **GLM_MQA)),
    ("glm_mqa_g17_apart_paged64", dict(batch=3, num_q_heads=17, page_size=64, seq_lens=[1, 640, 3000],
                                       num_splits=4, seed=172, rope_apart=64, **GLM_MQA)),
    ("glm_mqa_q2_g32_apart_paged32", dict(batch=3, num_q_heads=32, page_size=32, seq_lens=[1, 700, 1700],
                                          num_splits=2, seed=173, q_len=2, rope_apart=64, **GLM_MQA)),
    ("glm_mqa_g64_apart_paged48_general", dict(batch=2, num_q_heads=64, page_size=48, seq_lens=[1000, 97],
                                               num_splits=0, seed=174, rope_apart=64, **GLM_MQA)),
    ("glm_mqa_apart_poisoned", dict(batch=3, num_q_heads=64, page_size=64, seq_lens=[100, 1, 1025], num_splits=2,
                                    seed=175, rope_apart=64, poison=True, spare_pages=3, **GLM_MQA)),
    # latent over an fp8 cache (nope codes + per-token K scales, rotary bf16 apart)
    ("latent_fp8_g64_paged64", dict(batch=2, num_q_heads=64, page_size=64, seq_lens=[700, 1313], num_splits=3,
                                    seed=180, rope_apart=64, kv_fp8=True, **LATENT)),
    ("latent_fp8_g128_contig_ragged", dict(batch=3, num_q_heads=128, seq_lens=[100, 33, 1], num_splits=2,
                                           seed=181, rope_apart=64, kv_fp8=True, **LATENT)),
    ("latent_fp8_g40_paged32_auto", dict(batch=3, num_q_heads=40, page_size=32, seq_lens=[517, 64, 2000],
                                         num_splits=0, seed=182, rope_apart=64, kv_fp8=True, **LATENT)),
    ("latent_fp8_q2_g64_paged64", dict(batch=3, num_q_heads=64, page_size=64, seq_lens=[1, 900, 2100],
                                       num_splits=3, seed=183, q_len=2, rope_apart=64, kv_fp8=True, **LATENT)),
    ("latent_fp8_one_split", dict(batch=2, num_q_heads=128, page_size=64, seq_lens=[90, 31], num_splits=1,
                                  seed=184, rope_apart=64, kv_fp8=True, **LATENT)),
    ("latent_fp8_poisoned", dict(batch=3, num_q_heads=64, page_size=64, seq_lens=[100, 1, 1025], num_splits=2,
                                 seed=185, rope_apart=64, kv_fp8=True, poison=True, spare_pages=3, **LATENT)),
    # GLM widths on one kv head over an fp8 cache (nope 192 and V 256 as codes, V scales or none)
    ("glm_mqa_fp8_g64_paged64", dict(batch=2, num_q_heads=64, page_size=64, seq_lens=[1500, 333], num_splits=3,
                                     seed=186, rope_apart=64, kv_fp8=True, **GLM_MQA)),
    ("glm_mqa_fp8_g128_contig_no_v_scale", dict(batch=2, num_q_heads=128, seq_lens=[2000, 77], num_splits=2,
                                                seed=187, rope_apart=64, kv_fp8=True, v_scaled=False, **GLM_MQA)),
    ("glm_mqa_fp8_q2_g32_paged32", dict(batch=3, num_q_heads=32, page_size=32, seq_lens=[1, 700, 1700],
                                        num_splits=2, seed=188, q_len=2, rope_apart=64, kv_fp8=True, **GLM_MQA)),
    ("glm_mqa_fp8_poisoned", dict(batch=3, num_q_heads=64, page_size=64, seq_lens=[100, 1, 1025], num_splits=2,
                                  seed=189, rope_apart=64, kv_fp8=True, poison=True, spare_pages=3, **GLM_MQA)),
    # fp8 caches with the rotary columns as codes in the K rows (scaled with the nope columns)
    ("latent_fp8_inline_g64_paged64", dict(batch=2, num_q_heads=64, page_size=64, seq_lens=[700, 1313],
                                           num_splits=3, seed=190, kv_fp8=True, **LATENT)),
    ("latent_fp8_inline_g128_contig_ragged", dict(batch=3, num_q_heads=128, seq_lens=[100, 33, 1], num_splits=2,
                                                  seed=191, kv_fp8=True, **LATENT)),
    ("latent_fp8_inline_q2_g40_paged16_poisoned", dict(batch=3, num_q_heads=40, page_size=16,
                                                       seq_lens=[100, 1, 1025], num_splits=2, seed=192, q_len=2,
                                                       kv_fp8=True, poison=True, spare_pages=3, **LATENT)),
    ("glm_mqa_fp8_inline_g64_paged32", dict(batch=2, num_q_heads=64, page_size=32, seq_lens=[1500, 333],
                                            num_splits=3, seed=193, kv_fp8=True, **GLM_MQA)),
    ("glm_mqa_fp8_inline_no_v_scale_paged16", dict(batch=3, num_q_heads=32, page_size=16, seq_lens=[1, 700, 1700],
                                                   num_splits=0, seed=194, kv_fp8=True, v_scaled=False,
                                                   **GLM_MQA)),
]


@pytest.mark.parametrize("name,kw", SHARED, ids=[c[0] for c in SHARED])
def test_shared_kv_head_parity(name, kw):
    case = make_case(name, **kw)
    out, lse, o32 = check_case(case, f"shared kv head {name}")
    assert torch.isfinite(o32).all()
    if case.q_len > 1:
        for b, L in enumerate(case.seq_lens.tolist()):
            for i in range(case.q_len):
                if L - case.q_len + 1 + i <= 0:
                    assert torch.all(out[b, i].float() == 0) and torch.all(torch.isneginf(lse[b, i]))


@pytest.mark.parametrize("kw", [dict(rope_apart=64, **GLM_MQA), dict(rope_apart=64, **LATENT),
                                dict(rope_apart=64, kv_fp8=True, **LATENT), dict(rope_apart=64, kv_fp8=True, **GLM_MQA),
                                dict(kv_fp8=True, **LATENT)],
                         ids=["glm_mqa_apart", "latent_apart", "latent_fp8", "glm_mqa_fp8", "latent_fp8_inline"])
def test_shared_kv_head_large_logits_take_the_second_pass(kw):
    case = make_case("big_shared", batch=2, num_q_heads=64, page_size=64, seq_lens=[1300, 700], num_splits=2,
                     seed=176, q_scale=64.0, **kw)
    out, lse, o32 = run(case)
    O, LSE = oracle_for(case)
    assert torch.isfinite(o32).all()
    assert_parity(out, lse, o32, O, LSE, o32_row_rtol=1e-4, what="shared kv head large logits")


@pytest.mark.parametrize("kw", [dict(rope_apart=64, **GLM_MQA), dict(q_len=2, **LATENT)],
                         ids=["glm_mqa_apart", "latent_q2"])
def test_shared_kv_head_partials_match_oracle(kw):
    # pass 1 alone: every partition's (m, l) and normalised O against the oracle's partials
    case = make_case("shared_parts", batch=2, num_q_heads=64, page_size=64, seq_lens=[1500, 333], seed=177, **kw)
    dc = to_device(case)
    chunk, P = 512, 3
    po_t, pml_t = api.partition(dc.q, dc.k_cache, dc.v_cache, dc.page_table, dc.seq_lens, case.scale, chunk, P,
                                page_size=64, v_is_k_prefix=case.v_is_k_prefix, ov_depth=case.ov_depth,
                                k_rope=dc.k_rope)
    torch.cuda.synchronize()
    q = np32(case.q)
    k = np32(case.k_cache)
    if case.k_rope is not None:
        k = np.concatenate([k, np32(case.k_rope)], axis=-1)
    v = k[..., :case.ov_depth] if case.v_is_k_prefix else np32(case.v_cache)
    lens = case.seq_lens.numpy().astype(np.int64)
    ql = case.q_len
    for i in range(ql):
        qi = q[:, i] if ql > 1 else q
        li = np.clip(lens - ql + 1 + i, 0, lens)
        m, l, O = partition_partials_fp64(qi, k, v, li, case.scale, chunk, P, page_table=case.page_table.numpy(),
                                          page_size=64)
        rows = slice(i * case.q.shape[-2], (i + 1) * case.q.shape[-2])
        ml = np32(pml_t)[:, rows]
        po = np32(po_t)[:, rows]
        for b in range(case.batch):
            for pp in range(-(-int(lens[b]) // chunk)):
                live = l[b, :, pp] > 0
                np.testing.assert_allclose(ml[b, live, pp, 0], m[b, live, pp], rtol=1e-5, atol=1e-4)
                np.testing.assert_allclose(ml[b, live, pp, 1], l[b, live, pp], rtol=1e-5)
                err = np.abs(po[b, live, pp] - O[b, live, pp]).max(-1)
                assert (err / np.abs(O[b, live, pp]).max(-1)).max() <= 1e-5


DETERMINISM = [
    ("gqa_paged_auto", dict(batch=4, num_q_heads=32, num_kv_heads=4, qk_depth=128, page_size=64,
                            len_range=(500, 6000), num_splits=0, seed=43), {}),
    ("gqa_paged_auto_fused", dict(batch=4, num_q_heads=32, num_kv_heads=4, qk_depth=128, page_size=64,
                                  len_range=(500, 6000), num_splits=0, seed=44), {"fused": "force"}),
    ("latent_splits4", dict(batch=3, num_q_heads=128, num_kv_heads=1, qk_depth=576, ov_depth=512,
                            v_is_k_prefix=True, page_size=64, seq_lens=[3000, 700, 64], num_splits=4,
                            seed=45), {}),
    ("fp8_paged_auto", dict(batch=4, num_q_heads=32, num_kv_heads=4, qk_depth=128, page_size=64,
                            len_range=(500, 6000), num_splits=0, seed=46, kv_fp8=True), {}),
    ("d256_rotary_apart", dict(batch=3, num_q_heads=16, num_kv_heads=16, qk_depth=256, ov_depth=256,
                               page_size=64, len_range=(1, 3000), num_splits=0, seed=47, rope_apart=64), {}),
    # the fold in pass 1 with the folding workgroup's own partial kept in registers
    ("fused_own_partial", dict(batch=2, num_q_heads=8, num_kv_heads=2, qk_depth=128, seq_lens=[4096, 1000],
                               num_splits=8, seed=48), {"fused": True}),
]


@pytest.mark.parametrize("name,kw,call", DETERMINISM, ids=[c[0] for c in DETERMINISM])
def test_determinism_bitwise(name, kw, call):
    # two calls on the same inputs give bit-identical outputs (no atomics in any sum; the
    # fused combine folds the partials in partition order, whichever workgroup arrives last)
    case = make_case(name, **kw)
    dc = to_device(case)
    print(f"[parity] determinism {name}", flush=True)
    a = api.case_call(dc, return_lse=True, return_o32=True, **call)
    b = api.case_call(dc, return_lse=True, return_o32=True, **call)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


FOLD_EQUALS_COMBINE = [
    # one thread per unit and at most 8 partitions on both sides: the fold in pass 1 (own
    # partial from registers: matrix-core kernel with key splits, vector-ALU kernel) and the
    # combine launch take the same partials in the same order
    ("mfma_key_splits", dict(batch=2, num_q_heads=8, num_kv_heads=2, qk_depth=128, seq_lens=[4096, 1000],
                             num_splits=8, seed=49)),
    ("vector_alu_fp32", dict(batch=2, num_q_heads=4, num_kv_heads=2, qk_depth=128, dtype=torch.float32,
                             seq_lens=[2000, 700], num_splits=5, seed=50)),
]


@pytest.mark.parametrize("name,kw", FOLD_EQUALS_COMBINE, ids=[c[0] for c in FOLD_EQUALS_COMBINE])
def test_fused_fold_equals_combine_launch_bitwise(name, kw):
    case = make_case(name, **kw)
    dc = to_device(case)
    print(f"[parity] fused fold == combine launch {name}", flush=True)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")
    a = api.case_call(dc, return_lse=True, return_o32=True, fused=True, workspace=ws)
    b = api.case_call(dc, return_lse=True, return_o32=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_fused_fold_repeated_calls_equal_combine_launch_bitwise():
    # publication under load: 256 workgroups in 32 groups of 8 per call, the fold in pass 1
    # (forced) on one workspace for 30 calls in a row, every call bit-identical to the
    # combine launch (one thread per unit and 8 partitions on both sides: the same fold)
    case = make_case("fold_repeated", batch=8, num_q_heads=32, num_kv_heads=8, qk_depth=128,
                     seq_lens=[4096] * 8, num_splits=8, seed=51)
    dc = to_device(case)
    print("[parity] fused fold, 30 calls against the combine launch", flush=True)
    ref = api.case_call(dc, return_lse=True, return_o32=True)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")
    outs = [api.case_call(dc, return_lse=True, return_o32=True, fused="force", workspace=ws) for _ in range(30)]
    torch.cuda.synchronize()
    for i, got in enumerate(outs):
        for x, y in zip(got, ref):
            assert torch.equal(x, y), f"call {i}"


def test_seq_len_above_max_is_clamped():
    # seq_lens may not exceed max_seq_len; larger values are clamped to it
    case = make_case("clamp", batch=2, num_q_heads=8, num_kv_heads=1, qk_depth=128, page_size=64,
                     seq_lens=[1000, 800], num_splits=0, seed=44)
    dc = to_device(case)
    out, lse, o32 = api.case_call(dc, return_lse=True, return_o32=True, max_seq_len=640)
    torch.cuda.synchronize()
    case.seq_lens = torch.tensor([640, 640], dtype=torch.int32)
    O, LSE = oracle_for(case)
    assert_parity(out, lse, o32, O, LSE, what="clamped")


# ---------------------------------------------------------------------------
# pass 1 and pass 2 separately
# ---------------------------------------------------------------------------
def test_partition_partials_match_oracle():
    case = make_case("parts", batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=64,
                     seq_lens=[1000, 64, 2500], seed=45)
    dc = to_device(case)
    chunk, P = 512, 5
    po, pml = api.partition(dc.q, dc.k_cache, dc.v_cache, dc.page_table, dc.seq_lens, case.scale, chunk, P,
                            page_size=64)
    torch.cuda.synchronize()
    m, l, O = partition_partials_fp64(np32(case.q), np32(case.k_cache), np32(case.v_cache),
                                      case.seq_lens.numpy(), case.scale, chunk, P,
                                      page_table=case.page_table.numpy(), page_size=64)
    po, pml = np32(po), np32(pml)
    live = l > 0
    np.testing.assert_allclose(pml[..., 0][live], m[live], rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(pml[..., 1][live], l[live], rtol=1e-5)
    err = np.abs(po - O).max(-1)[live]
    ref = np.abs(O).max(-1)[live]
    assert (err / ref).max() <= 1e-5


FUSED = [
    # (equal shares: one kv head of 8 q heads keeps the bound on the last workgroup's fold,
    # 256 workers x 8 rows x 512 B, within 1 MiB)
    ("paged64_auto", dict(batch=5, num_q_heads=8, num_kv_heads=1, qk_depth=128, page_size=64,
                          len_range=(1, 5000), num_splits=0, seed=60)),
    ("contig_splits8", dict(batch=2, num_q_heads=8, num_kv_heads=2, qk_depth=128, seq_lens=[4096, 1000],
                            num_splits=8, seed=61)),
    ("one_kv_head_key_splits", dict(batch=3, num_q_heads=8, num_kv_heads=1, qk_depth=128, page_size=64,
                                    seq_lens=[3000, 64, 1], num_splits=3, seed=62)),
    ("g16_two_mfma", dict(batch=2, num_q_heads=32, num_kv_heads=2, qk_depth=128, page_size=32,
                          seq_lens=[777, 2048], num_splits=3, seed=63)),
    ("empty_and_single", dict(batch=4, num_q_heads=8, num_kv_heads=1, qk_depth=128, page_size=64,
                              seq_lens=[0, 1, 2, 6500], num_splits=0, seed=64)),
    # 64 partitions of one long sequence: the last workgroup folds 64 partials per row with
    # 4 threads per unit (and 17..64 for the 20 splits of the second case)
    ("long_64_splits", dict(batch=1, num_q_heads=32, num_kv_heads=4, qk_depth=128, page_size=64,
                            seq_lens=[20000], num_splits=64, seed=70)),
    ("splits20_two_seqs", dict(batch=2, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=32,
                               seq_lens=[6000, 333], num_splits=20, seed=71)),
    # 100 partitions: 16 threads per unit
    ("splits100", dict(batch=1, num_q_heads=8, num_kv_heads=1, qk_depth=128, page_size=32,
                       seq_lens=[6400], num_splits=100, seed=72)),
    # one long sequence in a batch of short ones under equal shares: most workers meet it
    ("auto_one_long_many_short", dict(batch=40, num_q_heads=8, num_kv_heads=1, qk_depth=128, page_size=64,
                                      seq_lens=[30000] + [64] * 39, num_splits=0, seed=74)),
    # one kv head for all q heads (the shared-kv-head kernel): latent, latent over fp8 with
    # an empty sequence, several queries, GLM widths with the rotary columns apart, and 20
    # partitions (4 threads per unit in the fold)
    ("latent_g64_paged64", dict(batch=2, num_q_heads=64, page_size=64, seq_lens=[700, 1313], num_splits=3,
                                seed=90, **LATENT)),
    ("latent_fp8_empty_seq", dict(batch=3, num_q_heads=128, page_size=64, seq_lens=[900, 0, 65], num_splits=2,
                                  seed=91, rope_apart=64, kv_fp8=True, **LATENT)),
    ("latent_q2_contig", dict(batch=2, num_q_heads=40, seq_lens=[1000, 3], num_splits=4, seed=92, q_len=2,
                              **LATENT)),
    ("glm_mqa_apart_paged32", dict(batch=2, num_q_heads=128, page_size=32, seq_lens=[1500, 333], num_splits=3,
                                   seed=93, rope_apart=64, **GLM_MQA)),
    ("glm_mqa_20_splits", dict(batch=1, num_q_heads=32, page_size=64, seq_lens=[5000], num_splits=20, seed=94,
                               rope_apart=64, **GLM_MQA)),
    # the vector-ALU kernel: fp32 (its automatic choice) and bf16 on request
    ("fp32_tiny", dict(batch=1, num_q_heads=1, num_kv_heads=1, qk_depth=128, dtype=torch.float32,
                       seq_lens=[1024], num_splits=4, seed=75)),
    ("fp32_g4_ragged_empty", dict(batch=4, num_q_heads=8, num_kv_heads=2, qk_depth=128, dtype=torch.float32,
                                  seq_lens=[1000, 0, 77, 300], num_splits=3, seed=76)),
    ("fp32_g16_paged16_auto", dict(batch=2, num_q_heads=16, num_kv_heads=1, qk_depth=128, dtype=torch.float32,
                                   page_size=16, seq_lens=[517, 1201], num_splits=0, seed=77)),
    ("fp32_g2_40_splits", dict(batch=2, num_q_heads=4, num_kv_heads=2, qk_depth=128, dtype=torch.float32,
                               page_size=64, seq_lens=[5000, 130], num_splits=40, seed=78)),
    ("bf16_fma_g8_paged64", dict(batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=64,
                                 seq_lens=[3000, 0, 65], num_splits=6, seed=79, kernel="fma")),
]


@pytest.mark.parametrize("name,kw", FUSED, ids=[c[0] for c in FUSED])
def test_fused_combine_matches_oracle_on_repeated_calls(name, kw):
    # the last-arriving workgroup combines; its counters must return to zero, so three
    # calls on one workspace all give the oracle's result
    print(f"[parity] fused {name}", flush=True)
    kw = dict(kw)
    kernel = kw.pop("kernel", "auto")
    case = make_case(name, **kw)
    dc = to_device(case)
    prob = api.make_problem(dc.q, dc.k_cache, dc.v_cache, dc.page_table, page_size=case.page_size, kernel=kernel,
                            v_is_k_prefix=case.v_is_k_prefix, ov_depth=case.ov_depth, k_rope=dc.k_rope)
    # (forced: the fold runs in pass 1 whatever the size of the partials)
    ws = torch.zeros(api.workspace_bytes(prob, case.num_splits), dtype=torch.uint8, device="cuda")
    O, LSE = oracle_for(case)
    for rep in range(3):
        out, lse, o32 = api.case_call(dc, return_lse=True, return_o32=True, fused="force", workspace=ws,
                                      kernel=kernel)
        torch.cuda.synchronize()
        assert_parity(out, lse, o32, O, LSE, what=f"fused {name} call {rep}")


def test_fused_entry_takes_the_combine_launch_for_a_fold_beyond_64_kib():
    # equal shares over 256 workers: any one sequence may meet every share, so the last
    # workgroup of a kv head could have to fold 256 partials of its 16 rows (2 MiB); the fused
    # entry point runs the combine launch instead (same results), here on a workspace that
    # was never zero-filled
    print("[parity] fused entry point, fold beyond 64 KiB", flush=True)
    case = make_case("fold_beyond_64kib", batch=2, num_q_heads=16, num_kv_heads=1, qk_depth=128, page_size=64,
                     seq_lens=[9000, 100], num_splits=0, seed=73)
    dc = to_device(case)
    prob = api.make_problem(dc.q, dc.k_cache, dc.v_cache, dc.page_table, page_size=case.page_size)
    assert not api.fused_applies(prob, 0)
    ws = torch.full((api.workspace_bytes(prob, 0),), 255, dtype=torch.uint8, device="cuda")
    O, LSE = oracle_for(case)
    out, lse, o32 = api.case_call(dc, return_lse=True, return_o32=True, fused=True, workspace=ws)
    torch.cuda.synchronize()
    assert_parity(out, lse, o32, O, LSE, what="fused entry point, fold beyond 64 KiB")


FUSED_WHERE_IT_PAYS = [
    # 8 partitions x 4 rows (one kv head of 4 q heads per workgroup) x 512 B = 16 KiB
    ("contig_splits8", dict(batch=2, num_q_heads=8, num_kv_heads=2, qk_depth=128, seq_lens=[4096, 1000],
                            num_splits=8, seed=61)),
    # the vector-ALU kernel: 4 partitions of one row
    ("fp32_tiny", dict(batch=1, num_q_heads=1, num_kv_heads=1, qk_depth=128, dtype=torch.float32,
                       seq_lens=[1024], num_splits=4, seed=75)),
    # equal shares over short sequences: at most ceil(16 tiles / 8) + 1 = 3 pieces of 8 rows
    ("auto_short_seqs", dict(batch=8, num_q_heads=8, num_kv_heads=1, qk_depth=128, page_size=64,
                             len_range=(1, 512), num_splits=0, seed=98)),
    # one kv head for all q heads: 2 partitions x 24 rows x 1 KiB (GLM widths) = 48 KiB
    ("glm_mqa_24_heads", dict(batch=2, num_q_heads=24, page_size=64, seq_lens=[1500, 0], num_splits=2, seed=97,
                              rope_apart=64, **GLM_MQA)),
]


@pytest.mark.parametrize("name,kw", FUSED_WHERE_IT_PAYS, ids=[c[0] for c in FUSED_WHERE_IT_PAYS])
def test_fused_entry_point_folds_in_pass_1_where_it_pays(name, kw):
    print(f"[parity] fused entry point folds in pass 1: {name}", flush=True)
    case = make_case(name, **kw)
    dc = to_device(case)
    prob = api.make_problem(dc.q, dc.k_cache, dc.v_cache, dc.page_table, page_size=case.page_size,
                            v_is_k_prefix=case.v_is_k_prefix, ov_depth=case.ov_depth, k_rope=dc.k_rope)
    assert api.fused_applies(prob, case.num_splits)
    ws = torch.zeros(api.workspace_bytes(prob, case.num_splits), dtype=torch.uint8, device="cuda")
    O, LSE = oracle_for(case)
    for rep in range(2):
        out, lse, o32 = api.case_call(dc, return_lse=True, return_o32=True, fused=True, workspace=ws)
        torch.cuda.synchronize()
        assert_parity(out, lse, o32, O, LSE, what=f"fused where it pays {name} call {rep}")


FUSED_EMPTY = [
    ("fixed8_bf16", dict(batch=5, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=64,
                         seq_lens=[0, 1, 33, 0, 2442], num_splits=8, seed=65)),
    ("fixed3_fp8_d192", dict(batch=4, num_q_heads=8, num_kv_heads=2, qk_depth=192, ov_depth=128, page_size=32,
                             seq_lens=[31, 0, 32, 0], num_splits=3, kv_fp8=True, seed=66)),
    ("fixed1_contig", dict(batch=3, num_q_heads=8, num_kv_heads=1, qk_depth=128, seq_lens=[0, 2, 700],
                           num_splits=1, seed=67)),
    ("auto_bf16", dict(batch=6, num_q_heads=8, num_kv_heads=1, qk_depth=128, page_size=64,
                       seq_lens=[0, 3000, 0, 5, 0, 0], num_splits=0, seed=68)),
    ("auto_all_empty", dict(batch=3, num_q_heads=8, num_kv_heads=1, qk_depth=128, page_size=64,
                            seq_lens=[0, 0, 0], num_splits=0, seed=69)),
    ("latent_fixed2", dict(batch=4, num_q_heads=80, page_size=64, seq_lens=[0, 1, 700, 0], num_splits=2,
                           seed=95, **LATENT)),
    ("fp32_vector_alu", dict(batch=3, num_q_heads=4, num_kv_heads=2, qk_depth=128, dtype=torch.float32,
                             seq_lens=[0, 300, 0], num_splits=2, seed=96)),
]


@pytest.mark.parametrize("name,kw", FUSED_EMPTY, ids=[c[0] for c in FUSED_EMPTY])
def test_fused_combine_writes_rows_of_empty_sequences(name, kw):
    # with the fused combine there is no combine launch: the rows of a sequence without
    # keys (O = 0, LSE = -inf) must still be written; outputs start as NaN to show it
    print(f"[parity] fused empty rows {name}", flush=True)
    case = make_case(name, **kw)
    dc = to_device(case)
    prob = api.make_problem(dc.q, dc.k_cache, dc.v_cache, dc.page_table, page_size=case.page_size,
                            v_is_k_prefix=case.v_is_k_prefix, ov_depth=case.ov_depth, k_rope=dc.k_rope)
    ws = torch.zeros(api.workspace_bytes(prob, case.num_splits), dtype=torch.uint8, device="cuda")
    rows = api.row_shape(prob)
    out = torch.empty(rows + (prob.ov_depth,), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    o32 = torch.empty(rows + (prob.ov_depth,), dtype=torch.float32, device="cuda")
    O, LSE = oracle_for(case)
    for rep in range(2):
        for t in (out, lse, o32):
            t.fill_(float("nan"))
        api.case_call(dc, out=out, lse=lse, o32=o32, fused="force", workspace=ws)
        torch.cuda.synchronize()
        assert_parity(out, lse, o32, O, LSE, what=f"fused empty rows {name} call {rep}")


EQUAL_SHARE = [
    # name, make_case kwargs, workers
    ("ragged_paged64", dict(batch=5, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=64,
                            seq_lens=[1000, 0, 2500, 64, 1], seed=50), 7),
    ("many_short_contig", dict(batch=53, num_q_heads=8, num_kv_heads=1, qk_depth=128,
                               seq_lens=[40] * 50 + [0] * 3, seed=51), 5),
    ("two_scan_chunks", dict(batch=150, num_q_heads=8, num_kv_heads=2, qk_depth=128, page_size=32,
                             len_range=(0, 300), seed=52), 9),
    ("fewer_active_workers", dict(batch=2, num_q_heads=32, num_kv_heads=4, qk_depth=128, page_size=16,
                                  seq_lens=[100, 50], seed=53), 64),
    ("g16_two_mfma", dict(batch=3, num_q_heads=32, num_kv_heads=2, qk_depth=128, page_size=64,
                          seq_lens=[3000, 5, 700], seed=54), 11),
]


@pytest.mark.parametrize("name,kw,workers", EQUAL_SHARE, ids=[c[0] for c in EQUAL_SHARE])
def test_equal_share_partials_match_oracle(name, kw, workers):
    print(f"[parity] equal shares {name} workers={workers}", flush=True)
    case = make_case(name, num_splits=0, **kw)
    dc = to_device(case)
    prob = api.make_problem(dc.q, dc.k_cache, dc.v_cache, dc.page_table, page_size=case.page_size)
    po_t, pml_t = api.partition(dc.q, dc.k_cache, dc.v_cache, dc.page_table, dc.seq_lens, case.scale, 0,
                                workers, page_size=case.page_size)
    torch.cuda.synchronize()
    lens = case.seq_lens.numpy().astype(np.int64)
    pieces, first, count = equal_share_pieces(lens, workers)
    ml_t, table = api.slot_table(prob, workers, pml_t)
    # the (first slot, count) table is integer work: exact
    np.testing.assert_array_equal(table.cpu().numpy(), np.stack([first, count], -1))
    pt = None if case.page_table is None else case.page_table.numpy()
    m, l, O = range_partials_fp64(np32(case.q), np32(case.k_cache), np32(case.v_cache), lens, case.scale, pieces,
                                  page_table=pt, page_size=case.page_size)
    S = len(pieces)
    ml, po = np32(ml_t)[:S], np32(po_t)[:S]
    np.testing.assert_allclose(ml[..., 0], m, rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(ml[..., 1], l, rtol=1e-5)
    err = np.abs(po - O).max(-1)
    ref = np.abs(O).max(-1)
    assert (err / ref).max() <= 1e-5
    # pass 2 on these partials gives the definition
    out, lse, o32 = api.combine(prob, dc.seq_lens, case.scale, 0, workers, po_t, pml_t)
    torch.cuda.synchronize()
    Oref, Lref = oracle_for(case)
    assert_parity(out, lse, o32, Oref, Lref, what=f"equal shares {name} combine")


@pytest.mark.parametrize("Dv,P", [(64, 4), (64, 40), (64, 300), (128, 4), (128, 16), (128, 24), (128, 64),
                                  (256, 8), (256, 40), (512, 8), (512, 20)])
def test_combine_only_on_oracle_partials(Dv, P):
    # oracle partials (with empty partitions) fed to the HIP combine
    r = np.random.default_rng(Dv + P)
    B, Hq, chunk = 3, 8, 64
    lens = np.array([P * chunk, chunk // 2, (P // 2) * chunk + 3])
    m = r.standard_normal((B, Hq, P)) * 4
    l = r.uniform(0.5, 30.0, (B, Hq, P))
    O = r.standard_normal((B, Hq, P, Dv)) * 0.1
    for b in range(B):
        pb = -(-lens[b] // chunk)
        m[b, :, pb:] = -np.inf
        l[b, :, pb:] = 0
        O[b, :, pb:] = 0
    m32, l32, O32 = m.astype(np.float32), l.astype(np.float32), O.astype(np.float32)
    Oref, Lref = combine_fp64(m32, l32, O32, 0.125)
    prob = api._lib.DaProblem()
    prob.batch, prob.num_q_heads, prob.num_kv_heads = B, Hq, 1
    prob.qk_depth = {64: 64, 128: 128, 256: 256, 512: 576}[Dv]
    prob.ov_depth, prob.dtype, prob.page_size, prob.kv_capacity = Dv, 1, 0, P * chunk
    prob.max_seq_len = P * chunk
    prob.v_is_k_prefix = 1 if Dv == 512 else 0
    ml = torch.from_numpy(np.stack([m32, l32], -1)).cuda().contiguous()
    po = torch.from_numpy(O32).cuda().contiguous()
    lens_t = torch.from_numpy(lens.astype(np.int32)).cuda()
    out, lse, o32 = api.combine(prob, lens_t, 0.125, chunk, P, po, ml)
    torch.cuda.synchronize()
    assert_parity(out, lse, o32, Oref, Lref, what=f"combine Dv={Dv} P={P}")


# ---------------------------------------------------------------------------
# the named workloads at full size
# ---------------------------------------------------------------------------
# Every (sequence, query, head) row of every named workload is compared element by element
# with the oracle: the method is an exact re-association of the definition, so no row may
# differ beyond the stated tolerances (the oracle runs the largest of these in seconds).
FULL_WORKLOADS = ["tiny", "gqa", "paged_gqa", "long", "latent", "paged_gqa_q2", "paged_gqa_fp8", "paged_glm",
                  "paged_glm_fp8", "latent_rope_apart", "glm_mqa", "paged_mha", "latent_fp8", "glm_mqa_fp8",
                  "latent_fp8_inline", "paged_mqa", "paged_gqa_d64"]


@pytest.mark.parametrize("name", FULL_WORKLOADS)
def test_workload_full(name):
    out, lse, o32 = check_case(workload(name), f"workload {name} (all rows)")
    assert torch.isfinite(o32).all()
    del out, lse, o32
    torch.cuda.empty_cache()


FP8 = [
    ("paged64_auto_g8", dict(batch=5, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=64,
                             len_range=(1, 5000), num_splits=0, seed=80)),
    ("contig_splits8_g4", dict(batch=2, num_q_heads=8, num_kv_heads=2, qk_depth=128, seq_lens=[4096, 1000],
                               num_splits=8, seed=81)),
    ("paged32_g16_two_mfma", dict(batch=2, num_q_heads=32, num_kv_heads=2, qk_depth=128, page_size=32,
                                  seq_lens=[777, 2048], num_splits=3, seed=82)),
    ("no_v_scale", dict(batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=64,
                        seq_lens=[1000, 64, 2500], num_splits=0, seed=83, v_scaled=False)),
    ("one_kv_head_key_splits", dict(batch=4, num_q_heads=8, num_kv_heads=1, qk_depth=128, page_size=64,
                                    seq_lens=[0, 1, 3000, 65], num_splits=3, seed=84)),
    ("poisoned_tails", dict(batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=64,
                            seq_lens=[100, 1, 1025], num_splits=0, seed=85, poison=True, spare_pages=3)),
]


@pytest.mark.parametrize("name,kw", FP8, ids=[c[0] for c in FP8])
def test_fp8_cache_parity(name, kw):
    # E4M3 caches with per-token scales against the oracle on the same codes and scales
    case = make_case(name, kv_fp8=True, **kw)
    out, lse, o32 = check_case(case, f"fp8 {name}")
    assert torch.isfinite(o32).all()


def test_fp8_partition_partials_match_oracle():
    case = make_case("f8parts", batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=64,
                     seq_lens=[1000, 64, 2500], seed=86, kv_fp8=True)
    dc = to_device(case)
    chunk, P = 512, 5
    po, pml = api.partition(dc.q, dc.k_cache, dc.v_cache, dc.page_table, dc.seq_lens, case.scale, chunk, P,
                            page_size=64, k_scale=dc.k_scale, v_scale=dc.v_scale)
    torch.cuda.synchronize()
    pieces = [(b, p * chunk, min((p + 1) * chunk, int(L)), b * P + p)
              for b, L in enumerate(case.seq_lens.tolist()) for p in range(P) if p * chunk < L]
    m, l, O = range_partials_fp64(np32(case.q), np32(case.k_cache), np32(case.v_cache), case.seq_lens.numpy(),
                                  case.scale, pieces, page_table=case.page_table.numpy(), page_size=64,
                                  k_scale=case.k_scale.numpy(), v_scale=case.v_scale.numpy())
    po, pml = np32(po), np32(pml)   # [B, Hq, P, ...]
    for b, lo, hi, sl in pieces:
        p = sl % P
        np.testing.assert_allclose(pml[b, :, p, 0], m[sl], rtol=1e-5, atol=1e-4)
        np.testing.assert_allclose(pml[b, :, p, 1], l[sl], rtol=1e-5)
        err = np.abs(po[b, :, p] - O[sl]).max(-1)
        assert (err / np.abs(O[sl]).max(-1)).max() <= 1e-5


MULTIQ = [
    ("q2_g8_paged64_auto", dict(batch=5, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=64,
                                len_range=(1, 5000), num_splits=0, seed=100, q_len=2)),
    ("q2_g4_contig_splits8", dict(batch=2, num_q_heads=8, num_kv_heads=2, qk_depth=128, seq_lens=[4096, 1000],
                                  num_splits=8, seed=101, q_len=2)),
    ("q4_g4_short_sequences", dict(batch=4, num_q_heads=8, num_kv_heads=2, qk_depth=128, page_size=32,
                                   seq_lens=[1, 3, 100, 2000], num_splits=0, seed=102, q_len=4)),
    ("q3_g2_one_kv_head_key_splits", dict(batch=3, num_q_heads=2, num_kv_heads=1, qk_depth=128, page_size=64,
                                          seq_lens=[2, 700, 3000], num_splits=3, seed=103, q_len=3)),
    ("q2_g8_fp8_cache", dict(batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=64,
                             seq_lens=[33, 1000, 2500], num_splits=0, seed=104, q_len=2, kv_fp8=True)),
]


@pytest.mark.parametrize("name,kw", MULTIQ, ids=[c[0] for c in MULTIQ])
def test_multiquery_parity(name, kw):
    # q_len queries per sequence, each attending the keys up to its own position
    case = make_case(name, **kw)
    out, lse, o32 = check_case(case, f"multi-query {name}")
    for b, L in enumerate(case.seq_lens.tolist()):
        for i in range(case.q_len):
            if L - case.q_len + 1 + i <= 0:   # a query with no key before it
                assert torch.all(out[b, i].float() == 0) and torch.all(torch.isneginf(lse[b, i]))


def test_multiquery_fused_combine():
    case = make_case("mq_fused", batch=4, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=64,
                     len_range=(1, 4000), num_splits=0, seed=105, q_len=2)
    dc = to_device(case)
    O, LSE = oracle_for(case)
    prob = api.make_problem(dc.q, dc.k_cache, dc.v_cache, dc.page_table, page_size=case.page_size)
    ws = torch.zeros(api.workspace_bytes(prob, 0), dtype=torch.uint8, device="cuda")
    for rep in range(2):
        out, lse, o32 = api.case_call(dc, return_lse=True, return_o32=True, fused="force", workspace=ws)
        torch.cuda.synchronize()
        assert_parity(out, lse, o32, O, LSE, what=f"multi-query fused call {rep}")


# ---------------------------------------------------------------------------
# page sizes: pages of 16 keys (each half of a 32-key tile is a page) and the per-key page
# lookup (any other page size, down to one key per page) on every form; ragged last tiles
# end in either half, poisoned cases fill every slot no sequence attends (codes, rotary
# columns and fp8 scales) with NaN
# ---------------------------------------------------------------------------
PAGE_FORMS = [
    ("fp8_g8_paged16_auto", dict(batch=4, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=16,
                                 seq_lens=[1201, 17, 0, 2500], num_splits=0, seed=130, kv_fp8=True)),
    ("fp8_g4_paged16_splits3_poisoned", dict(batch=3, num_q_heads=8, num_kv_heads=2, qk_depth=128, page_size=16,
                                             seq_lens=[100, 1, 1025], num_splits=3, seed=131, kv_fp8=True,
                                             poison=True, spare_pages=3)),
    ("fp8_g16_paged16_two_mfma", dict(batch=2, num_q_heads=32, num_kv_heads=2, qk_depth=128, page_size=16,
                                      seq_lens=[777, 2048], num_splits=3, seed=132, kv_fp8=True)),
    ("fp8_g8_paged16_no_v_scale", dict(batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=16,
                                       seq_lens=[1000, 64, 2500], num_splits=0, seed=133, kv_fp8=True,
                                       v_scaled=False)),
    ("q2_g8_paged16_auto", dict(batch=4, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=16,
                                seq_lens=[1, 517, 1201, 3000], num_splits=0, seed=134, q_len=2)),
    ("q2_fp8_g8_paged16", dict(batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=16,
                               seq_lens=[33, 1000, 2500], num_splits=0, seed=135, q_len=2, kv_fp8=True)),
    ("d192_apart_g8_paged16", dict(batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=192, ov_depth=128,
                                   page_size=16, seq_lens=[1000, 33, 2100], num_splits=0, seed=136,
                                   rope_apart=64)),
    ("d256_apart_fp8_g4_paged16_poisoned", dict(batch=3, num_q_heads=8, num_kv_heads=2, qk_depth=256,
                                                ov_depth=256, page_size=16, seq_lens=[100, 1, 1025],
                                                num_splits=0, seed=137, rope_apart=64, kv_fp8=True, poison=True,
                                                spare_pages=3)),
    ("d256_inline_fp8_g8_paged16", dict(batch=2, num_q_heads=16, num_kv_heads=2, qk_depth=256, ov_depth=256,
                                        page_size=16, seq_lens=[1200, 45], num_splits=2, seed=138, kv_fp8=True)),
    ("d192_apart_fp8_q2_g1_paged16", dict(batch=3, num_q_heads=2, num_kv_heads=2, qk_depth=192, ov_depth=128,
                                          page_size=16, seq_lens=[2, 900, 2048], num_splits=0, seed=139,
                                          rope_apart=64, kv_fp8=True, q_len=2)),
    # one kv head for all q heads, pages of 16 keys
    ("latent_g64_inline_paged16", dict(batch=2, num_q_heads=64, page_size=16, seq_lens=[700, 1313], num_splits=3,
                                       seed=140, **LATENT)),
    ("latent_fp8_g64_paged16", dict(batch=3, num_q_heads=64, page_size=16, seq_lens=[700, 1313, 17],
                                    num_splits=3, seed=141, rope_apart=64, kv_fp8=True, **LATENT)),
    ("latent_fp8_g128_paged16_poisoned", dict(batch=3, num_q_heads=128, page_size=16, seq_lens=[100, 1, 1025],
                                              num_splits=2, seed=142, rope_apart=64, kv_fp8=True, poison=True,
                                              spare_pages=3, **LATENT)),
    ("glm_mqa_fp8_q2_g32_paged16", dict(batch=3, num_q_heads=32, page_size=16, seq_lens=[1, 700, 1700],
                                        num_splits=2, seed=143, q_len=2, rope_apart=64, kv_fp8=True, **GLM_MQA)),
    ("glm_mqa_fp8_no_v_scale_paged16_poisoned", dict(batch=3, num_q_heads=64, page_size=16,
                                                     seq_lens=[100, 1, 1025], num_splits=2, seed=144,
                                                     rope_apart=64, kv_fp8=True, v_scaled=False, poison=True,
                                                     spare_pages=3, **GLM_MQA)),
    ("glm_mqa_apart_g64_paged16", dict(batch=2, num_q_heads=64, page_size=16, seq_lens=[1500, 333], num_splits=3,
                                       seed=145, rope_apart=64, **GLM_MQA)),
    # per-key page lookup
    ("q2_g8_paged48_general", dict(batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=48,
                                   seq_lens=[1, 1000, 2100], num_splits=0, seed=146, q_len=2)),
    ("q3_g4_paged8_general_splits3", dict(batch=3, num_q_heads=8, num_kv_heads=2, qk_depth=128, page_size=8,
                                          seq_lens=[2, 700, 1500], num_splits=3, seed=147, q_len=3)),
    ("d192_inline_g8_paged48_general", dict(batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=192, ov_depth=128,
                                            page_size=48, seq_lens=[1000, 33, 2100], num_splits=0, seed=148)),
    ("d256_inline_g4_paged24_general_poisoned", dict(batch=3, num_q_heads=8, num_kv_heads=2, qk_depth=256,
                                                     ov_depth=256, page_size=24, seq_lens=[100, 1, 1025],
                                                     num_splits=0, seed=149, poison=True, spare_pages=3)),
    ("d256_inline_q2_g8_paged8_general", dict(batch=2, num_q_heads=16, num_kv_heads=2, qk_depth=256,
                                              ov_depth=256, page_size=8, seq_lens=[900, 2], num_splits=2,
                                              seed=150, q_len=2)),
    ("latent_apart_g40_paged48_general", dict(batch=2, num_q_heads=40, page_size=48, seq_lens=[517, 64],
                                              num_splits=0, seed=151, rope_apart=64, **LATENT)),
    ("latent_g24_paged8_general", dict(batch=2, num_q_heads=24, page_size=8, seq_lens=[300, 45], num_splits=2,
                                       seed=152, **LATENT)),
    # per-key page lookup with fp8 caches (scales key by key) and rotary columns stored apart
    ("fp8_g8_paged48_general_auto", dict(batch=4, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=48,
                                         seq_lens=[1201, 17, 0, 2500], num_splits=0, seed=153, kv_fp8=True)),
    ("fp8_g4_paged8_general_splits3_poisoned", dict(batch=3, num_q_heads=8, num_kv_heads=2, qk_depth=128,
                                                    page_size=8, seq_lens=[100, 1, 1025], num_splits=3,
                                                    seed=154, kv_fp8=True, poison=True, spare_pages=3)),
    ("fp8_q2_g8_paged24_general_no_v_scale", dict(batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=128,
                                                  page_size=24, seq_lens=[2, 700, 1500], num_splits=0, seed=155,
                                                  q_len=2, kv_fp8=True, v_scaled=False)),
    ("d192_apart_fp8_g4_paged8_general", dict(batch=3, num_q_heads=8, num_kv_heads=2, qk_depth=192, ov_depth=128,
                                              page_size=8, seq_lens=[1000, 33, 2100], num_splits=0, seed=156,
                                              rope_apart=64, kv_fp8=True)),
    ("d256_apart_g8_paged40_general_poisoned", dict(batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=256,
                                                    ov_depth=256, page_size=40, seq_lens=[100, 1, 1025],
                                                    num_splits=0, seed=157, rope_apart=64, poison=True,
                                                    spare_pages=3)),
    ("d256_inline_fp8_g4_paged1_general", dict(batch=3, num_q_heads=8, num_kv_heads=2, qk_depth=256, ov_depth=256,
                                               page_size=1, seq_lens=[300, 45, 2], num_splits=0, seed=158,
                                               kv_fp8=True)),
    ("latent_fp8_g64_paged48_general", dict(batch=2, num_q_heads=64, page_size=48, seq_lens=[700, 1313],
                                            num_splits=3, seed=159, rope_apart=64, kv_fp8=True, **LATENT)),
    ("latent_fp8_inline_q2_g40_paged8_general_poisoned", dict(batch=3, num_q_heads=40, page_size=8,
                                                              seq_lens=[100, 1, 1025], num_splits=2, seed=195,
                                                              q_len=2, kv_fp8=True, poison=True, spare_pages=3,
                                                              **LATENT)),
    ("glm_mqa_fp8_g64_paged24_general", dict(batch=2, num_q_heads=64, page_size=24, seq_lens=[1500, 333],
                                             num_splits=3, seed=196, rope_apart=64, kv_fp8=True, **GLM_MQA)),
    ("glm_mqa_fp8_inline_no_v_scale_paged1_general", dict(batch=3, num_q_heads=32, page_size=1,
                                                          seq_lens=[300, 45, 2], num_splits=2, seed=197,
                                                          kv_fp8=True, v_scaled=False, **GLM_MQA)),
]


@pytest.mark.parametrize("name,kw", PAGE_FORMS, ids=[c[0] for c in PAGE_FORMS])
def test_page_size_forms(name, kw):
    # the combine launch, then the fold in pass 1 on the same inputs
    case = make_case(name, **kw)
    print(f"[parity] page sizes {name}", flush=True)
    dc = to_device(case)
    O, LSE = oracle_for(case)
    for fused in (False, "force"):
        out, lse, o32 = api.case_call(dc, return_lse=True, return_o32=True, fused=fused)
        torch.cuda.synchronize()
        assert torch.isfinite(o32).all()
        assert_parity(out, lse, o32, O, LSE, what=f"page sizes {name} fused={fused}")


# ---------------------------------------------------------------------------
# more than 16 (query, head) columns per kv head on the GQA kernels: the group is split into
# virtual kv heads of at most 16 columns that read the same cached kv head (multi-query bf16
# at depth 128 runs on the shared-kv-head kernel instead: the first case)
# ---------------------------------------------------------------------------
LARGE_GROUPS = [
    ("mqa_g32_paged64_auto", dict(batch=3, num_q_heads=32, num_kv_heads=1, qk_depth=128, page_size=64,
                                  seq_lens=[1500, 33, 2600], num_splits=0, seed=200)),
    ("g24_hkv2_contig_splits5", dict(batch=2, num_q_heads=48, num_kv_heads=2, qk_depth=128, seq_lens=[2000, 77],
                                     num_splits=5, seed=201)),
    ("g17_prime_paged16", dict(batch=2, num_q_heads=34, num_kv_heads=2, qk_depth=128, page_size=16,
                               seq_lens=[700, 1313], num_splits=0, seed=202)),
    ("q3_g8_paged32", dict(batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=32,
                           seq_lens=[2, 700, 1500], num_splits=0, seed=203, q_len=3)),
    ("q2_g16_fp8_paged64", dict(batch=3, num_q_heads=32, num_kv_heads=2, qk_depth=128, page_size=64,
                                seq_lens=[33, 1000, 2500], num_splits=0, seed=204, q_len=2, kv_fp8=True)),
    ("d256_apart_g32_hkv2_paged48_general", dict(batch=2, num_q_heads=64, num_kv_heads=2, qk_depth=256,
                                                 ov_depth=256, page_size=48, seq_lens=[1000, 97], num_splits=0,
                                                 seed=205, rope_apart=64)),
    ("d192_fp8_q4_g8_contig_splits3", dict(batch=2, num_q_heads=16, num_kv_heads=2, qk_depth=192, ov_depth=128,
                                           seq_lens=[900, 3], num_splits=3, seed=206, q_len=4, kv_fp8=True)),
    ("mqa_g48_fp8_paged16_poisoned", dict(batch=3, num_q_heads=48, num_kv_heads=1, qk_depth=128, page_size=16,
                                          seq_lens=[100, 1, 1025], num_splits=0, seed=207, kv_fp8=True, poison=True,
                                          spare_pages=3)),
    # fp32 on the vector-ALU kernel, same split into virtual kv heads
    ("fp32_mqa_g32_paged64", dict(batch=2, num_q_heads=32, num_kv_heads=1, qk_depth=128, dtype=torch.float32,
                                  page_size=64, seq_lens=[1000, 77], num_splits=0, seed=208)),
    ("fp32_g24_hkv2_contig_splits3", dict(batch=2, num_q_heads=48, num_kv_heads=2, qk_depth=128,
                                          dtype=torch.float32, seq_lens=[600, 1300], num_splits=3, seed=209)),
]


@pytest.mark.parametrize("name,kw", LARGE_GROUPS, ids=[c[0] for c in LARGE_GROUPS])
def test_large_group_parity(name, kw):
    # the combine launch, then the fold in pass 1 on the same inputs
    case = make_case(name, **kw)
    print(f"[parity] large group {name}", flush=True)
    dc = to_device(case)
    O, LSE = oracle_for(case)
    for fused in (False, "force"):
        out, lse, o32 = api.case_call(dc, return_lse=True, return_o32=True, fused=fused)
        torch.cuda.synchronize()
        assert torch.isfinite(o32).all()
        assert_parity(out, lse, o32, O, LSE, what=f"large group {name} fused={fused}")


# ---------------------------------------------------------------------------
# heads of 64 dimensions (q.K 64 / V 64) on the matrix-core kernel
# ---------------------------------------------------------------------------
D64 = [
    ("d64_g4_contig_splits3", dict(batch=2, num_q_heads=16, num_kv_heads=4, qk_depth=64, seq_lens=[1000, 77],
                                   num_splits=3, seed=210)),
    ("d64_g8_paged64_auto", dict(batch=4, num_q_heads=16, num_kv_heads=2, qk_depth=64, page_size=64,
                                 len_range=(1, 4000), num_splits=0, seed=211)),
    ("d64_fp8_g8_paged16_poisoned", dict(batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=64, page_size=16,
                                         seq_lens=[100, 1, 1025], num_splits=0, seed=212, kv_fp8=True, poison=True,
                                         spare_pages=3)),
    ("d64_q2_g16_paged48_general", dict(batch=3, num_q_heads=32, num_kv_heads=2, qk_depth=64, page_size=48,
                                        seq_lens=[2, 700, 1500], num_splits=0, seed=213, q_len=2)),
    ("d64_fp8_g1_contig_key_splits", dict(batch=2, num_q_heads=4, num_kv_heads=4, qk_depth=64,
                                          seq_lens=[3000, 1], num_splits=2, seed=214, kv_fp8=True)),
    ("d64_mqa_g32_paged32", dict(batch=2, num_q_heads=32, num_kv_heads=1, qk_depth=64, page_size=32,
                                 seq_lens=[1500, 333], num_splits=0, seed=215)),
]


@pytest.mark.parametrize("name,kw", D64, ids=[c[0] for c in D64])
def test_depth64_parity(name, kw):
    # the combine launch, then the fold in pass 1 on the same inputs
    case = make_case(name, **kw)
    print(f"[parity] depth 64 {name}", flush=True)
    dc = to_device(case)
    O, LSE = oracle_for(case)
    for fused in (False, "force"):
        out, lse, o32 = api.case_call(dc, return_lse=True, return_o32=True, fused=fused)
        torch.cuda.synchronize()
        assert torch.isfinite(o32).all()
        assert_parity(out, lse, o32, O, LSE, what=f"depth 64 {name} fused={fused}")


# ---------------------------------------------------------------------------
# wider depth pairs: q.K 192 / V 128 and q.K 256 / V 256 (nope 192 != V 256), with the
# 64 rotary columns in the K rows or stored apart in bf16, bf16 or fp8 caches
# ---------------------------------------------------------------------------
WIDE = [
    ("d256_apart_g1_paged64_auto", dict(batch=4, num_q_heads=4, num_kv_heads=4, qk_depth=256, ov_depth=256,
                                        page_size=64, len_range=(1, 3000), num_splits=0, seed=110,
                                        rope_apart=64)),
    ("d256_apart_g4_contig_splits3", dict(batch=2, num_q_heads=8, num_kv_heads=2, qk_depth=256, ov_depth=256,
                                          seq_lens=[2000, 77], num_splits=3, seed=111, rope_apart=64)),
    ("d256_inline_g8_paged32", dict(batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=256, ov_depth=256,
                                    page_size=32, seq_lens=[1500, 1, 640], num_splits=0, seed=112)),
    ("d256_apart_g16_key_splits", dict(batch=2, num_q_heads=16, num_kv_heads=1, qk_depth=256, ov_depth=256,
                                       page_size=64, seq_lens=[3000, 100], num_splits=2, seed=113,
                                       rope_apart=64)),
    ("d192_apart_g8_paged64", dict(batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=192, ov_depth=128,
                                   page_size=64, seq_lens=[1000, 33, 2100], num_splits=0, seed=114,
                                   rope_apart=64)),
    ("d192_inline_g4_contig", dict(batch=2, num_q_heads=8, num_kv_heads=2, qk_depth=192, ov_depth=128,
                                   seq_lens=[700, 1300], num_splits=0, seed=115)),
    ("d256_apart_fp8_g1_paged64", dict(batch=4, num_q_heads=4, num_kv_heads=4, qk_depth=256, ov_depth=256,
                                       page_size=64, len_range=(1, 3000), num_splits=0, seed=116,
                                       rope_apart=64, kv_fp8=True)),
    ("d256_inline_fp8_g8_contig", dict(batch=2, num_q_heads=16, num_kv_heads=2, qk_depth=256, ov_depth=256,
                                       seq_lens=[1200, 45], num_splits=2, seed=117, kv_fp8=True)),
    ("d192_apart_fp8_g8_noscale_v", dict(batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=192, ov_depth=128,
                                         page_size=64, seq_lens=[900, 1, 2048], num_splits=0, seed=118,
                                         rope_apart=64, kv_fp8=True, v_scaled=False)),
    ("d256_apart_q2_g4", dict(batch=3, num_q_heads=8, num_kv_heads=2, qk_depth=256, ov_depth=256, page_size=64,
                              seq_lens=[1, 600, 2500], num_splits=0, seed=119, rope_apart=64, q_len=2)),
    ("d256_apart_poisoned", dict(batch=3, num_q_heads=4, num_kv_heads=2, qk_depth=256, ov_depth=256,
                                 page_size=64, seq_lens=[100, 1, 1025], num_splits=0, seed=120, rope_apart=64,
                                 poison=True, spare_pages=3)),
]


@pytest.mark.parametrize("name,kw", WIDE, ids=[c[0] for c in WIDE])
def test_wide_depth_parity(name, kw):
    case = make_case(name, **kw)
    out, lse, o32 = check_case(case, f"wide depth {name}")
    assert torch.isfinite(o32).all()


def test_wide_depth_fused_combine():
    case = make_case("wide_fused", batch=4, num_q_heads=8, num_kv_heads=2, qk_depth=256, ov_depth=256,
                     page_size=64, len_range=(1, 4000), num_splits=0, seed=121, rope_apart=64, kv_fp8=True)
    dc = to_device(case)
    O, LSE = oracle_for(case)
    prob = api.make_problem(dc.q, dc.k_cache, dc.v_cache, dc.page_table, page_size=case.page_size,
                            k_rope=dc.k_rope)
    ws = torch.zeros(api.workspace_bytes(prob, 0), dtype=torch.uint8, device="cuda")
    for rep in range(2):
        out, lse, o32 = api.case_call(dc, return_lse=True, return_o32=True, fused="force", workspace=ws)
        torch.cuda.synchronize()
        assert_parity(out, lse, o32, O, LSE, what=f"wide depth fused call {rep}")


@pytest.mark.parametrize("fp8", [False, True])
def test_wide_depth_equal_share_partials(fp8):
    print(f"[parity] wide depth equal-share partials fp8={fp8}", flush=True)
    case = make_case("wide_parts", batch=3, num_q_heads=4, num_kv_heads=4, qk_depth=256, ov_depth=256,
                     page_size=64, seq_lens=[1000, 64, 2500], seed=122, rope_apart=64, kv_fp8=fp8)
    dc = to_device(case)
    workers = 6
    prob = api.make_problem(dc.q, dc.k_cache, dc.v_cache, dc.page_table, page_size=64, k_rope=dc.k_rope)
    po_t, pml_t = api.partition(dc.q, dc.k_cache, dc.v_cache, dc.page_table, dc.seq_lens, case.scale, 0, workers,
                                page_size=64, k_scale=dc.k_scale, v_scale=dc.v_scale, k_rope=dc.k_rope)
    torch.cuda.synchronize()
    lens = case.seq_lens.numpy().astype(np.int64)
    pieces, first, count = equal_share_pieces(lens, workers)
    ml_t, table = api.slot_table(prob, workers, pml_t)
    np.testing.assert_array_equal(table.cpu().numpy(), np.stack([first, count], -1))
    ks = None if case.k_scale is None else case.k_scale.numpy()
    vs = None if case.v_scale is None else case.v_scale.numpy()
    m, l, O = range_partials_fp64(np32(case.q), np32(case.k_cache), np32(case.v_cache), lens, case.scale, pieces,
                                  page_table=case.page_table.numpy(), page_size=64, k_scale=ks, v_scale=vs,
                                  k_rope=np32(case.k_rope))
    S = len(pieces)
    ml, po = np32(ml_t)[:S], np32(po_t)[:S]
    np.testing.assert_allclose(ml[..., 0], m, rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(ml[..., 1], l, rtol=1e-5)
    err = np.abs(po - O).max(-1)
    assert (err / np.abs(O).max(-1)).max() <= 1e-5
    out, lse, o32 = api.combine(prob, dc.seq_lens, case.scale, 0, workers, po_t, pml_t)
    torch.cuda.synchronize()
    Oref, Lref = oracle_for(case)
    assert_parity(out, lse, o32, Oref, Lref, what="wide depth equal shares combine")


@pytest.mark.parametrize("fp8", [False, True])
def test_pieces_longer_than_one_page_segment(fp8):
    # Two workers for one long sequence: each piece spans more than the 511 page indices
    # staged in LDS at a time, so the kernel runs it as several segments (the fp8 loop keeps
    # two tiles in flight and must not prefetch across a segment boundary).
    print(f"[parity] multi-segment pieces fp8={fp8}", flush=True)
    case = make_case("segments", batch=2, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=32,
                     seq_lens=[40000, 333], seed=123, kv_fp8=fp8)
    dc = to_device(case)
    workers = 2
    prob = api.make_problem(dc.q, dc.k_cache, dc.v_cache, dc.page_table, page_size=32)
    po_t, pml_t = api.partition(dc.q, dc.k_cache, dc.v_cache, dc.page_table, dc.seq_lens, case.scale, 0, workers,
                                page_size=32, k_scale=dc.k_scale, v_scale=dc.v_scale)
    torch.cuda.synchronize()
    lens = case.seq_lens.numpy().astype(np.int64)
    pieces, first, count = equal_share_pieces(lens, workers)
    assert max(hi - lo for _, lo, hi, _ in pieces) > 511 * 32
    ks = None if case.k_scale is None else case.k_scale.numpy()
    vs = None if case.v_scale is None else case.v_scale.numpy()
    m, l, O = range_partials_fp64(np32(case.q), np32(case.k_cache), np32(case.v_cache), lens, case.scale, pieces,
                                  page_table=case.page_table.numpy(), page_size=32, k_scale=ks, v_scale=vs)
    ml_t, table = api.slot_table(prob, workers, pml_t)
    S = len(pieces)
    ml, po = np32(ml_t)[:S], np32(po_t)[:S]
    np.testing.assert_allclose(ml[..., 0], m, rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(ml[..., 1], l, rtol=1e-5)
    err = np.abs(po - O).max(-1)
    assert (err / np.abs(O).max(-1)).max() <= 1e-5


# ---------------------------------------------------------------------------
# size limits
# ---------------------------------------------------------------------------
def test_half_million_key_sequence():
    # 2^19 keys in one sequence (8192 pages of 64): key, page and tile counts far beyond the
    # workloads', through the automatic (equal-share) schedule
    L = 1 << 19
    case = make_case("512K", batch=1, num_q_heads=8, num_kv_heads=1, qk_depth=128, page_size=64, seq_lens=[L],
                     num_splits=0, seed=124)
    print("[parity] one sequence of 2^19 keys", flush=True)
    out, lse, o32 = run(case)
    O, LSE = oracle_for(case)
    assert_parity(out, lse, o32, O, LSE, what="2^19 keys")


def test_many_sequences_and_sixteen_queries():
    # 4096 sequences of 1-40 keys (the schedule scans lengths 64 at a time) and, separately,
    # 16 queries per sequence with one q head per kv head (all 16 MFMA columns in use)
    case = make_case("many", batch=4096, num_q_heads=2, num_kv_heads=1, qk_depth=128, page_size=32,
                     len_range=(0, 40), num_splits=0, seed=125)
    print("[parity] 4096 short sequences", flush=True)
    out, lse, o32 = run(case)
    O, LSE = oracle_for(case)
    assert_parity(out, lse, o32, O, LSE, what="4096 sequences")
    case = make_case("q16", batch=3, num_q_heads=2, num_kv_heads=2, qk_depth=128, page_size=64,
                     seq_lens=[15, 700, 2049], num_splits=0, seed=126, q_len=16)
    print("[parity] q_len 16, one q head per kv head", flush=True)
    out, lse, o32 = run(case)
    O, LSE = oracle_for(case)
    assert_parity(out, lse, o32, O, LSE, what="q_len 16")


def pages_past(dc, min_offset_bytes):
    """The device case ``dc`` with its pages moved past ``min_offset_bytes`` of larger pools.

    Every pool-shaped tensor (first dimension = pages: K, V, their fp8 scales, the rotary
    columns) gets ``shift`` zero pages in front, and the page table points past them. The
    attended values do not change, so the oracle of the original case still applies."""
    page_bytes = dc.k_cache[0].numel() * dc.k_cache.element_size()
    shift = -(-min_offset_bytes // page_bytes)

    def grow(t):
        if t is None:
            return None
        big = torch.zeros((t.shape[0] + shift,) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
        big[shift:] = t
        return big

    pt = dc.page_table.clone()
    pt[pt >= 0] += shift
    return dataclasses.replace(dc, k_cache=grow(dc.k_cache), v_cache=grow(dc.v_cache), k_scale=grow(dc.k_scale),
                               v_scale=grow(dc.v_scale), k_rope=grow(dc.k_rope), page_table=pt)


BEYOND_4G = [
    ("gqa_bf16_auto", dict(batch=3, num_q_heads=32, num_kv_heads=8, qk_depth=128, page_size=64,
                           seq_lens=[700, 3000, 64], num_splits=0, seed=130)),
    ("gqa_fp8_splits3", dict(batch=2, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=64,
                             seq_lens=[2500, 333], num_splits=3, seed=131, kv_fp8=True)),
    ("latent_splits4", dict(batch=2, num_q_heads=64, num_kv_heads=1, qk_depth=576, ov_depth=512,
                            v_is_k_prefix=True, page_size=64, seq_lens=[1500, 300], num_splits=4, seed=132)),
    ("d256_rotary_apart", dict(batch=2, num_q_heads=8, num_kv_heads=8, qk_depth=256, ov_depth=256,
                               page_size=64, seq_lens=[1200, 65], num_splits=0, seed=133, rope_apart=64)),
    ("fp32_g1_vector_alu", dict(batch=2, num_q_heads=2, num_kv_heads=2, qk_depth=128, dtype=torch.float32,
                                page_size=64, seq_lens=[900, 130], num_splits=2, seed=134)),
]


@pytest.mark.parametrize("name,kw", BEYOND_4G, ids=[c[0] for c in BEYOND_4G])
def test_pages_beyond_4gib(name, kw):
    # caches of serving size: the attended pages sit past 4.5 GiB of each pool, so every
    # byte offset into the cache needs more than 32 bits (and row indices times row bytes
    # overflow 32-bit arithmetic)
    case = make_case(name, **kw)
    dc = pages_past(to_device(case), 9 << 29)
    print(f"[parity] {name}: pages past 4.5 GiB ({dc.k_cache.shape[0]} pages)", flush=True)
    out, lse, o32 = api.case_call(dc, return_lse=True, return_o32=True)
    torch.cuda.synchronize()
    O, LSE = oracle_for(case)
    assert_parity(out, lse, o32, O, LSE, what=f"{name} beyond 4 GiB")
    del dc, out, lse, o32
    torch.cuda.empty_cache()


def capacity_past(dc, min_offset_bytes):
    """The contiguous device case ``dc`` with each sequence's capacity grown (zero rows after
    the original ones) so that sequence 1 starts past ``min_offset_bytes`` of the cache."""
    row_bytes = dc.k_cache[0, 0].numel() * dc.k_cache.element_size()
    cap = max(dc.k_cache.shape[1], -(-min_offset_bytes // row_bytes))

    def grow(t):
        if t is None:
            return None
        if t.dim() == 3:   # fp8 scales, tokens innermost: [B][Hkv][L_cap]
            big = torch.zeros(t.shape[:2] + (cap,), dtype=t.dtype, device=t.device)
            big[:, :, :t.shape[2]] = t
            return big
        big = torch.zeros((t.shape[0], cap) + tuple(t.shape[2:]), dtype=t.dtype, device=t.device)
        big[:, :t.shape[1]] = t
        return big

    return dataclasses.replace(dc, k_cache=grow(dc.k_cache), v_cache=grow(dc.v_cache), k_scale=grow(dc.k_scale),
                               v_scale=grow(dc.v_scale), k_rope=grow(dc.k_rope))


CONTIG_BEYOND_4G = [
    ("gqa_bf16_splits8", dict(batch=3, num_q_heads=32, num_kv_heads=8, qk_depth=128, seq_lens=[4096, 1000, 33],
                              num_splits=8, seed=140)),
    ("gqa_fp8_auto", dict(batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=128, seq_lens=[2000, 700, 64],
                          num_splits=0, seed=141, kv_fp8=True)),
    ("latent_splits2", dict(batch=3, num_q_heads=16, num_kv_heads=1, qk_depth=576, ov_depth=512,
                            v_is_k_prefix=True, seq_lens=[900, 64, 300], num_splits=2, seed=142)),
    ("d256_rotary_apart", dict(batch=3, num_q_heads=8, num_kv_heads=2, qk_depth=256, ov_depth=256,
                               seq_lens=[1500, 77, 200], num_splits=3, seed=143, rope_apart=64)),
    ("fp32_g4_vector_alu", dict(batch=3, num_q_heads=8, num_kv_heads=2, qk_depth=128, dtype=torch.float32,
                                seq_lens=[800, 50, 129], num_splits=2, seed=144)),
]


@pytest.mark.parametrize("name,kw", CONTIG_BEYOND_4G, ids=[c[0] for c in CONTIG_BEYOND_4G])
def test_contiguous_rows_beyond_4gib(name, kw):
    # contiguous caches whose sequences 1 and 2 start past 2.25 and 4.5 GiB of the cache
    case = make_case(name, **kw)
    dc = capacity_past(to_device(case), 9 << 28)
    print(f"[parity] {name}: capacity {dc.k_cache.shape[1]} rows per sequence", flush=True)
    out, lse, o32 = api.case_call(dc, return_lse=True, return_o32=True)
    torch.cuda.synchronize()
    O, LSE = oracle_for(case)
    assert_parity(out, lse, o32, O, LSE, what=f"{name} beyond 4 GiB")
    del dc, out, lse, o32
    torch.cuda.empty_cache()
