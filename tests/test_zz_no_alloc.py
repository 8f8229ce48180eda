"""The allocation-free entry point decode_attn_splitk_noalloc, through the C ABI.

Its results must equal those of decode_attn_splitk (same kernels, same schedule) bit for
bit, and match the oracle to the stated tolerances; two calls in a row, the second on a
smaller problem, check that nothing of the first call's scratch contents leaks into the
second.
"""

import ctypes

import numpy as np
import pytest
import torch

from lse_combine_amd import _lib, api
from lse_combine_amd.inputs import make_case, to_device
from parity_utils import assert_parity, oracle_for

pytestmark = pytest.mark.gpu

P = ctypes.c_void_p


def _ptr(t):
    return None if t is None else P(t.data_ptr())


def _outputs(prob, dev):
    rows = api.row_shape(prob)
    Dv = prob.ov_depth
    return (torch.full(rows + (Dv,), float("nan"), dtype=torch.bfloat16, device=dev),
            torch.full(rows, float("nan"), dtype=torch.float32, device=dev),
            torch.full(rows + (Dv,), float("nan"), dtype=torch.float32, device=dev))


def _same(a, b):
    a, b = a.cpu(), b.cpu()
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def run_pair(case):
    """(noalloc outputs, splitk outputs) of one case, both through the C ABI on one stream."""
    lib = _lib.load()
    dc = to_device(case)
    prob = api.make_problem(dc.q, dc.k_cache, dc.v_cache, dc.page_table, page_size=case.page_size,
                            v_is_k_prefix=case.v_is_k_prefix, ov_depth=case.ov_depth)
    stream = P(torch.cuda.current_stream().cuda_stream)
    free = _outputs(prob, "cuda")
    _lib.check(lib.decode_attn_splitk_noalloc(ctypes.byref(prob), _ptr(dc.q), _ptr(dc.k_cache), _ptr(dc.v_cache),
                                              _ptr(dc.page_table), _ptr(dc.seq_lens), float(case.scale),
                                              int(case.num_splits), *[_ptr(t) for t in free], stream))
    ref = _outputs(prob, "cuda")
    need = api.workspace_bytes(prob, case.num_splits)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    _lib.check(lib.decode_attn_splitk(ctypes.byref(prob), _ptr(dc.q), _ptr(dc.k_cache), _ptr(dc.v_cache),
                                      _ptr(dc.page_table), _ptr(dc.seq_lens), float(case.scale),
                                      int(case.num_splits), *[_ptr(t) for t in ref], _ptr(ws), ws.numel(), stream))
    torch.cuda.synchronize()
    return free, ref


def test_noalloc_matches_splitk_on_two_calls_in_a_row():
    big = make_case("noalloc_big", batch=6, num_q_heads=32, num_kv_heads=4, qk_depth=128, page_size=64,
                    len_range=(1, 6000), num_splits=0, seed=150)
    small = make_case("noalloc_small", batch=2, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=32,
                      seq_lens=[700, 33], num_splits=3, seed=151)
    for case in (big, small):
        print(f"[noalloc] {case.name}", flush=True)
        free, ref = run_pair(case)
        for name, a, b in zip(("out", "lse", "o32"), free, ref):
            assert _same(a, b), f"{case.name}: {name} differs from decode_attn_splitk"
        O, LSE = oracle_for(case)
        assert_parity(*free, O, LSE, what=f"noalloc {case.name}")


def test_noalloc_latent_and_empty_rows():
    # the latent-shared kernel's workspace (64 heads x 2 splits) and a sequence without keys
    case = make_case("noalloc_latent", batch=3, num_q_heads=64, num_kv_heads=1, qk_depth=576, ov_depth=512,
                     page_size=64, seq_lens=[900, 0, 65], num_splits=2, seed=152, v_is_k_prefix=True)
    print("[noalloc] latent", flush=True)
    free, ref = run_pair(case)
    for name, a, b in zip(("out", "lse", "o32"), free, ref):
        assert _same(a, b), f"latent: {name} differs from decode_attn_splitk"
    O, LSE = oracle_for(case)
    assert_parity(*free, O, LSE, what="noalloc latent")
    assert torch.all(free[0][1].float() == 0) and torch.all(torch.isneginf(free[1][1]))


def test_noalloc_refuses_problems_beyond_its_scratch():
    lib = _lib.load()
    p = _lib.DaProblem()
    for k, v in dict(batch=64, num_q_heads=128, num_kv_heads=1, qk_depth=576, ov_depth=512, dtype=_lib.DA_BF16,
                     page_size=64, max_pages_per_seq=128, num_pages=8192, max_seq_len=8192, v_is_k_prefix=1).items():
        setattr(p, k, v)
    fake = P(0x1000)   # never dereferenced: the size check comes first
    code = lib.decode_attn_splitk_noalloc(ctypes.byref(p), fake, fake, None, fake, fake, 0.05, 8, fake, None, None,
                                          None)
    assert code == _lib.DA_EWORKSPACE
    assert b"scratch" in lib.da_last_error()
