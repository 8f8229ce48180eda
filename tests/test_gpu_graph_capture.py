"""The decode step captured in a HIP graph and replayed.

The entry points allocate nothing, synchronise nothing and enqueue only kernel launches on
the caller's stream, so a step can be captured once and replayed on new inputs written
into the same buffers. Each replay is checked bit for bit against the same call made
eagerly on the same inputs (the path is run-to-run deterministic), with eager work and
synchronisations between the replays, and the first one against the oracle.
"""

import ctypes

import pytest
import torch

from lse_combine_amd import _lib, api
from lse_combine_amd.inputs import make_case, to_device
from parity_utils import assert_parity, oracle_for

pytestmark = pytest.mark.gpu

P = ctypes.c_void_p

# (name, case, fused): fixed splits with a fold that pays (8 partitions x 8 rows x 512 B),
# the same through the combine launch, and automatic splits (equal shares)
CASES = [
    ("fixed8_fused", dict(batch=4, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=64,
                          len_range=(100, 2000), num_splits=8, seed=120), True),
    ("fixed8_combine_launch", dict(batch=4, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=64,
                                   len_range=(100, 2000), num_splits=8, seed=121), False),
    ("auto_equal_shares", dict(batch=6, num_q_heads=32, num_kv_heads=4, qk_depth=128, page_size=64,
                               len_range=(1, 3000), num_splits=0, seed=122), False),
]


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("name,kw,fused", CASES, ids=[c[0] for c in CASES])
def test_plan_replays_in_a_graph(name, kw, fused):
    print(f"[graph] plan {name}", flush=True)
    case = make_case(name, **kw)
    dc = to_device(case)
    prob = api.make_problem(dc.q, dc.k_cache, dc.v_cache, dc.page_table, page_size=case.page_size)
    rows = api.row_shape(prob)
    lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    o32 = torch.empty(rows + (prob.ov_depth,), dtype=torch.float32, device="cuda")
    plan = api.DecodePlan(dc.q, dc.k_cache, dc.v_cache, dc.page_table, dc.seq_lens, case.scale, case.num_splits,
                          page_size=case.page_size, lse=lse, o32=o32, fused=fused)
    if fused:
        assert api.fused_applies(prob, case.num_splits), "the case must fold in pass 1"
    plan.run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.run()
    torch.cuda.synchronize()
    gen = torch.Generator("cpu").manual_seed(1000 + kw["seed"])
    for rep in range(3):
        q_new = torch.randn(dc.q.shape, generator=gen).to(dc.q.dtype)
        dc.q.copy_(q_new.to("cuda"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (plan.out, lse, o32)]
        for t in (plan.out, lse, o32):
            t.fill_(float("nan"))
        plan.run()
        torch.cuda.synchronize()
        for g, e in zip(got, (plan.out, lse, o32)):
            assert _same(g, e), f"{name}: replay {rep} differs from the eager call"
        if rep == 0:
            case.q = q_new
            O, LSE = oracle_for(case)
            assert_parity(got[0], got[1], got[2], O, LSE, what=f"graph replay {name}")


def test_noalloc_replays_in_a_graph():
    print("[graph] allocation-free entry point", flush=True)
    lib = _lib.load()
    case = make_case("noalloc_graph", batch=3, num_q_heads=16, num_kv_heads=2, qk_depth=128, page_size=64,
                     len_range=(1, 2500), num_splits=0, seed=123)
    dc = to_device(case)
    prob = api.make_problem(dc.q, dc.k_cache, dc.v_cache, dc.page_table, page_size=case.page_size)
    rows = api.row_shape(prob)
    out = torch.empty(rows + (prob.ov_depth,), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(rows, dtype=torch.float32, device="cuda")

    def call():
        stream = P(torch.cuda.current_stream().cuda_stream)
        _lib.check(lib.decode_attn_splitk_noalloc(ctypes.byref(prob), P(dc.q.data_ptr()), P(dc.k_cache.data_ptr()),
                                                  P(dc.v_cache.data_ptr()), P(dc.page_table.data_ptr()),
                                                  P(dc.seq_lens.data_ptr()), float(case.scale), 0,
                                                  P(out.data_ptr()), P(lse.data_ptr()), None, stream))

    call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    gen = torch.Generator("cpu").manual_seed(2000)
    for rep in range(3):
        dc.q.copy_(torch.randn(dc.q.shape, generator=gen).to(dc.q.dtype).to("cuda"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (out.clone(), lse.clone())
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        call()
        torch.cuda.synchronize()
        assert _same(got[0], out) and _same(got[1], lse), f"replay {rep} differs from the eager call"
