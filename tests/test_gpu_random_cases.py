"""Seeded random problems across every kernel family, each checked against the oracle.

Each case draws a family (GQA matrix-core depths 64/64, 128/128, 192/128, 256/256 with rotary
columns inline or apart; fp32 and bf16 on the vector-ALU kernel; one kv head for all q
heads in the latent and GLM widths), a cache dtype (bf16, or fp8 where the family has it),
a page size (contiguous, powers of two from 1 to 128 keys, 24 or 48), 1-5 sequences with random lengths
(empty ones included), one to three queries per sequence, a split count (automatic or
fixed) and a combine (separate launch, fused where it pays, fold forced in pass 1). Draws
the library does not support (da_supported) are drawn again. Every case prints its draw
before it runs.
"""

import ctypes
import random

import pytest
import torch

from lse_combine_amd import _lib, api
from lse_combine_amd.inputs import make_case, to_device
from parity_utils import assert_parity, oracle_for

pytestmark = pytest.mark.gpu

N_CASES = 120


def _draw(rng):
    fam = rng.choice(["gqa128", "gqa128", "wide", "fp32", "fma_bf16", "latent", "glm_mqa", "d64"])
    kw = dict(batch=rng.randint(1, 5), seed=rng.randint(0, 1 << 30))
    kernel = "auto"
    page = rng.choice([0, 16, 32, 64, 128, 48, 8, 24, 1])
    q_len = rng.choice([1, 1, 1, 2, 3])
    kv_fp8 = False
    if fam == "gqa128":
        hkv = rng.choice([1, 2, 4, 8])
        kw.update(num_kv_heads=hkv, num_q_heads=hkv * rng.choice([1, 2, 4, 8, 16, 24, 32]), qk_depth=128)
        kv_fp8 = rng.random() < 0.3
    elif fam == "d64":
        hkv = rng.choice([1, 2, 4])
        kw.update(num_kv_heads=hkv, num_q_heads=hkv * rng.choice([1, 4, 8, 16, 24]), qk_depth=64)
        kv_fp8 = rng.random() < 0.3
    elif fam == "wide":
        hkv = rng.choice([1, 2, 4])
        kw.update(num_kv_heads=hkv, num_q_heads=hkv * rng.choice([1, 4, 8]))
        if rng.random() < 0.5:
            kw.update(qk_depth=192, ov_depth=128)
        else:
            kw.update(qk_depth=256, ov_depth=256)
        if rng.random() < 0.5:
            kw.update(rope_apart=64)
        kv_fp8 = rng.random() < 0.3
    elif fam == "fp32":
        hkv = rng.choice([1, 2])
        kw.update(num_kv_heads=hkv, num_q_heads=hkv * rng.choice([1, 2, 4, 8, 20]), qk_depth=128, dtype=torch.float32)
    elif fam == "fma_bf16":
        hkv = rng.choice([1, 2])
        kw.update(num_kv_heads=hkv, num_q_heads=hkv * rng.choice([1, 4, 8, 16]), qk_depth=128)
        kernel = "fma"
        q_len = 1
    elif fam == "latent":
        kw.update(num_kv_heads=1, num_q_heads=rng.choice([17, 32, 64, 100, 128]), qk_depth=576, ov_depth=512,
                  v_is_k_prefix=True)
        if rng.random() < 0.5:
            kw.update(rope_apart=64)
        kv_fp8 = rng.random() < 0.4
    else:
        kw.update(num_kv_heads=1, num_q_heads=rng.choice([24, 64, 128]), qk_depth=256, ov_depth=256)
        if rng.random() < 0.6:
            kw.update(rope_apart=64)
        kv_fp8 = rng.random() < 0.4
    lens = [rng.choice([0, rng.randint(1, 64), rng.randint(1, 2500)]) for _ in range(kw["batch"])]
    kw.update(page_size=page, seq_lens=lens, q_len=q_len, kv_fp8=kv_fp8,
              num_splits=rng.choice([0, 0, 1, 2, 3, 5, 8, 13]))
    fused = rng.choice([False, True, "force"])
    return fam, kw, kernel, fused


def _supported(case, kernel):
    prob = api.make_problem(case.q, case.k_cache, case.v_cache, case.page_table, page_size=case.page_size,
                            v_is_k_prefix=case.v_is_k_prefix, ov_depth=case.ov_depth, kernel=kernel,
                            k_rope=case.k_rope)
    return _lib.load().da_supported(ctypes.byref(prob)) == _lib.DA_OK


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case_matches_oracle(i):
    rng = random.Random(9000 + i)
    for _ in range(50):
        fam, kw, kernel, fused = _draw(rng)
        case = make_case(f"random{i}", **kw)
        if _supported(case, kernel):
            break
    else:
        pytest.skip("no supported draw")
    print(f"[parity] random {i}: {fam} kernel={kernel} fused={fused} "
          + " ".join(f"{k}={v}" for k, v in kw.items() if k != "seed") + f" seed={kw['seed']}", flush=True)
    dc = to_device(case)
    O, LSE = oracle_for(case)
    out, lse, o32 = api.case_call(dc, return_lse=True, return_o32=True, fused=fused, kernel=kernel)
    torch.cuda.synchronize()
    assert_parity(out, lse, o32, O, LSE, what=f"random {i} ({fam})")
