"""Pins for the fp64 oracle: each check ties it to something other than itself.

The pages print no worked numeric example, so the oracle is pinned by
brute force, closed forms, library routines (scipy, torch) and the
invariants of softmax attention and of the split-K combine
(fa4_splitk_combine_write, first and second paragraphs).
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import (
    bf16_round_fp64,
    combine_fp64,
    decode_attention_fp64,
    decode_attention_splitk_fp64,
    equal_share_pieces,
    fp8_e4m3_to_fp64,
    partition_partials_fp64,
    range_partials_fp64,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng_case(seed, B=2, Hq=4, Hkv=2, D=8, Dv=None, L=(5, 9), paged=0, dtype=np.float64):
    r = np.random.default_rng(seed)
    Dv = D if Dv is None else Dv
    lens = np.array([L[b % len(L)] for b in range(B)])
    q = r.standard_normal((B, Hq, D))
    if paged:
        npg = [-(-int(x) // paged) for x in lens]
        n = sum(npg) + 2
        perm = r.permutation(n)
        pt = -np.ones((B, max(npg)), dtype=np.int64)
        off = 0
        for b in range(B):
            pt[b, :npg[b]] = perm[off:off + npg[b]]
            off += npg[b]
        k = r.standard_normal((n, paged, Hkv, D))
        v = r.standard_normal((n, paged, Hkv, Dv))
        return q, k, v, lens, pt
    cap = int(lens.max())
    k = r.standard_normal((B, cap, Hkv, D))
    v = r.standard_normal((B, cap, Hkv, Dv))
    return q, k, v, lens, None


# ---------------------------------------------------------------------------
# brute force: pure-Python loops with math.exp and math.fsum
# ---------------------------------------------------------------------------
def brute(q, k, v, lens, scale, pt=None, ps=0):
    B, Hq, D = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    Dv = v.shape[3]
    O = [[[0.0] * Dv for _ in range(Hq)] for _ in range(B)]
    LSE = [[-math.inf] * Hq for _ in range(B)]
    for b in range(B):
        L = int(lens[b])
        for h in range(Hq):
            kv = h // g
            keys, vals = [], []
            for t in range(L):
                if pt is None:
                    keys.append(k[b][t][kv]); vals.append(v[b][t][kv])
                else:
                    page = int(pt[b][t // ps]); slot = t % ps
                    keys.append(k[page][slot][kv]); vals.append(v[page][slot][kv])
            if not keys:
                continue
            xs = [math.fsum(float(q[b][h][d]) * float(kk[d]) for d in range(D)) for kk in keys]
            # exact log-sum-exp of scale*x without a max shift would overflow for big x;
            # shift by the first score instead of the max to stay independent of the oracle
            s0 = xs[0]
            ws = [math.exp(scale * (x - s0)) for x in xs]
            Z = math.fsum(ws)
            for d in range(Dv):
                O[b][h][d] = math.fsum(w * float(vv[d]) for w, vv in zip(ws, vals)) / Z
            LSE[b][h] = scale * s0 + math.log(Z)
    return np.array(O), np.array(LSE)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("paged", [0, 4])
def test_brute_force_tiny(seed, paged):
    q, k, v, lens, pt = rng_case(seed, B=2, Hq=4, Hkv=2, D=6, Dv=5, L=(7, 13), paged=paged)
    scale = 0.37
    O, LSE = decode_attention_fp64(q, k, v, lens, scale, page_table=pt, page_size=paged)
    Ob, Lb = brute(q, k, v, lens, scale, pt, paged)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(LSE, Lb, rtol=1e-14, atol=1e-13)


def test_brute_force_group1_and_group4():
    for Hq, Hkv in [(3, 3), (8, 2), (4, 1)]:
        q, k, v, lens, pt = rng_case(10 + Hq, B=2, Hq=Hq, Hkv=Hkv, D=4, L=(3, 11))
        O, LSE = decode_attention_fp64(q, k, v, lens, 0.9)
        Ob, Lb = brute(q, k, v, lens, 0.9)
        np.testing.assert_allclose(O, Ob, atol=1e-13)
        np.testing.assert_allclose(LSE, Lb, atol=1e-13)


# ---------------------------------------------------------------------------
# library routines: scipy's logsumexp / softmax
# ---------------------------------------------------------------------------
def test_matches_scipy_softmax_and_logsumexp():
    q, k, v, lens, _ = rng_case(5, B=1, Hq=2, Hkv=1, D=16, L=(40,))
    scale = 0.25
    O, LSE = decode_attention_fp64(q, k, v, lens, scale)
    for h in range(2):
        x = scale * (k[0, :40, 0, :] @ q[0, h])
        np.testing.assert_allclose(LSE[0, h], scipy.special.logsumexp(x), rtol=1e-14)
        np.testing.assert_allclose(O[0, h], scipy.special.softmax(x) @ v[0, :40, 0, :], atol=1e-14)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
def test_constant_v_gives_v():
    q, k, v, lens, _ = rng_case(7, B=2, Hq=4, Hkv=2, D=8, L=(33, 17))
    u = np.linspace(-2, 3, 8)
    v[:] = u
    O, _ = decode_attention_fp64(q, k, v, lens, 0.5)
    np.testing.assert_allclose(O, np.broadcast_to(u, O.shape), rtol=0, atol=4e-16 * 3)


def test_zero_k_gives_mean_v_and_log_len():
    q, k, v, lens, _ = rng_case(8, B=2, Hq=2, Hkv=1, D=8, L=(21, 9))
    k[:] = 0
    O, LSE = decode_attention_fp64(q, k, v, lens, 0.3)
    for b in range(2):
        L = lens[b]
        np.testing.assert_allclose(O[b], np.broadcast_to(v[b, :L, 0].mean(0), O[b].shape), atol=1e-15)
        np.testing.assert_allclose(LSE[b], math.log(L), rtol=1e-15)


def test_single_key_and_two_keys():
    q, k, v, lens, _ = rng_case(9, B=1, Hq=1, Hkv=1, D=8, L=(1,))
    s = 0.7
    O, LSE = decode_attention_fp64(q, k, v, lens, s)
    np.testing.assert_allclose(O[0, 0], v[0, 0, 0], atol=0)
    np.testing.assert_allclose(LSE[0, 0], s * float(q[0, 0] @ k[0, 0, 0]), rtol=1e-15)
    q, k, v, lens, _ = rng_case(11, B=1, Hq=1, Hkv=1, D=8, L=(2,))
    O, LSE = decode_attention_fp64(q, k, v, lens, s)
    x0, x1 = float(q[0, 0] @ k[0, 0, 0]), float(q[0, 0] @ k[0, 1, 0])
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))  # noqa: E731
    ref = sig(s * (x0 - x1)) * v[0, 0, 0] + sig(s * (x1 - x0)) * v[0, 1, 0]
    np.testing.assert_allclose(O[0, 0], ref, atol=1e-15)
    np.testing.assert_allclose(LSE[0, 0], math.log(math.exp(s * x0) + math.exp(s * x1)), rtol=1e-14)


def test_empty_sequence():
    q, k, v, lens, _ = rng_case(12, B=2, Hq=2, Hkv=1, D=4, L=(0, 5))
    O, LSE = decode_attention_fp64(q, k, v, lens, 1.0)
    assert np.all(O[0] == 0) and np.all(np.isneginf(LSE[0]))
    assert np.all(np.isfinite(LSE[1]))


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
def test_shift_invariance_and_overflow_safety():
    q, k, v, lens, _ = rng_case(13, B=1, Hq=2, Hkv=1, D=8, L=(50,))
    s = 0.5
    O, LSE = decode_attention_fp64(q, k, v, lens, s)
    a = np.full(8, 400.0)  # scale*q.a is far beyond exp's range: needs the max shift
    k2 = k + a
    O2, LSE2 = decode_attention_fp64(q, k2, v, lens, s)
    np.testing.assert_allclose(O2, O, atol=1e-11)
    np.testing.assert_allclose(LSE2, LSE + s * (q[0] @ a), rtol=1e-12)
    assert np.all(np.isfinite(O2))


def test_key_permutation_invariance():
    q, k, v, lens, _ = rng_case(14, B=1, Hq=2, Hkv=1, D=8, L=(30,))
    perm = np.random.default_rng(0).permutation(30)
    O, LSE = decode_attention_fp64(q, k, v, lens, 0.4)
    O2, LSE2 = decode_attention_fp64(q, k[:, perm], v[:, perm], lens, 0.4)
    np.testing.assert_allclose(O2, O, atol=1e-14)
    np.testing.assert_allclose(LSE2, LSE, rtol=1e-14)


def test_paged_equals_contiguous_gather():
    q, k, v, lens, pt = rng_case(15, B=3, Hq=4, Hkv=2, D=8, L=(13, 4, 9), paged=4)
    ps = 4
    cap = int(lens.max())
    kc = np.zeros((3, cap, 2, 8)); vc = np.zeros((3, cap, 2, 8))
    for b in range(3):
        for t in range(lens[b]):
            kc[b, t] = k[pt[b, t // ps], t % ps]
            vc[b, t] = v[pt[b, t // ps], t % ps]
    O, LSE = decode_attention_fp64(q, k, v, lens, 0.6, page_table=pt, page_size=ps)
    O2, LSE2 = decode_attention_fp64(q, kc, vc, lens, 0.6)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(LSE, LSE2)


def test_gqa_equals_mha_with_repeated_heads():
    q, k, v, lens, _ = rng_case(16, B=2, Hq=8, Hkv=2, D=8, L=(12, 7))
    O, LSE = decode_attention_fp64(q, k, v, lens, 0.8)
    k_rep = np.repeat(k, 4, axis=2)
    v_rep = np.repeat(v, 4, axis=2)
    O2, LSE2 = decode_attention_fp64(q, k_rep, v_rep, lens, 0.8)
    # same sums, different BLAS blocking: equal up to fp64 rounding
    np.testing.assert_allclose(O, O2, atol=1e-14)
    np.testing.assert_allclose(LSE, LSE2, rtol=1e-14)


def test_latent_shared_equals_materialised_v():
    q, k, _, lens, pt = rng_case(17, B=2, Hq=4, Hkv=1, D=12, L=(9, 20), paged=4)
    O, LSE = decode_attention_fp64(q, k, None, lens, 0.3, page_table=pt, page_size=4,
                                   v_is_k_prefix=True, ov_depth=10)
    v = np.ascontiguousarray(k[..., :10])
    O2, LSE2 = decode_attention_fp64(q, k, v, lens, 0.3, page_table=pt, page_size=4)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(LSE, LSE2)
    assert O.shape[-1] == 10


# ---------------------------------------------------------------------------
# split-K: P-way combine equals the P = 1 result
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("chunk", [1, 3, 8, 16, 64])
def test_splitk_combine_equals_definition(chunk):
    q, k, v, lens, pt = rng_case(18, B=3, Hq=4, Hkv=2, D=8, L=(37, 16, 1), paged=8)
    O, LSE = decode_attention_fp64(q, k, v, lens, 0.45, page_table=pt, page_size=8)
    O2, LSE2 = decode_attention_splitk_fp64(q, k, v, lens, 0.45, chunk, page_table=pt, page_size=8)
    np.testing.assert_allclose(O2, O, atol=1e-14)
    np.testing.assert_allclose(LSE2, LSE, rtol=1e-14)


def test_partitions_are_normalised_and_empty_ones_are_neutral():
    q, k, v, lens, _ = rng_case(19, B=2, Hq=2, Hkv=1, D=8, L=(10, 3))
    m, l, O = partition_partials_fp64(q, k, v, lens, 1.0, chunk=4, num_partitions=5)
    # sequence 1 has one partition; partitions 1..4 are empty
    assert np.all(np.isneginf(m[1, :, 1:])) and np.all(l[1, :, 1:] == 0) and np.all(O[1, :, 1:] == 0)
    # a normalised partial of constant V is V itself
    v2 = np.ones_like(v)
    _, _, O1 = partition_partials_fp64(q, k, v2, lens, 1.0, chunk=4, num_partitions=3)
    np.testing.assert_allclose(O1[0], 1.0, atol=1e-15)
    # the combine of a single partition returns it unchanged
    Oc, Lc = combine_fp64(m[1, :, :1], l[1, :, :1], O[1, :, :1], 1.0)
    np.testing.assert_array_equal(Oc, O[1, :, 0])
    np.testing.assert_allclose(Lc, m[1, :, 0] + np.log(l[1, :, 0]), rtol=1e-15)


def test_combine_is_order_independent_and_all_empty_row():
    r = np.random.default_rng(3)
    m = r.standard_normal((5, 6)) * 3
    l = r.uniform(0.5, 4, (5, 6))
    O = r.standard_normal((5, 6, 7))
    perm = r.permutation(6)
    a, la = combine_fp64(m, l, O, 0.7)
    b, lb = combine_fp64(m[:, perm], l[:, perm], O[:, perm], 0.7)
    np.testing.assert_allclose(a, b, atol=1e-14)
    np.testing.assert_allclose(la, lb, rtol=1e-14)
    z, lz = combine_fp64(np.full((1, 3), -np.inf), np.zeros((1, 3)), np.zeros((1, 3, 2)), 1.0)
    assert np.all(z == 0) and np.isneginf(lz[0])


# ---------------------------------------------------------------------------
# bf16 cast: torch's fp32 -> bf16 cast (round-to-nearest-even) as the library pin
# ---------------------------------------------------------------------------
def test_bf16_round_matches_torch_on_fp32_values():
    r = np.random.default_rng(4)
    x = np.concatenate([
        r.standard_normal(20000) * 10.0 ** r.integers(-30, 30, 20000),
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2.0 ** -130, 3 * 2.0 ** -134,
                  3.3895313892515355e38, 3.39e38, -3.4e38, 0.0, 65504.0]),
    ]).astype(np.float32)
    ours = bf16_round_fp64(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_bf16_ties_to_even():
    assert bf16_round_fp64(np.array([1 + 2 ** -8]))[0] == 1.0
    assert bf16_round_fp64(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6
    assert bf16_round_fp64(np.array([1 + 2 ** -8 + 2 ** -40]))[0] == 1 + 2 ** -7


# ---------------------------------------------------------------------------
# hand-derived golden fixtures (the pages print no worked example)
# ---------------------------------------------------------------------------
def _load_golden():
    out = []
    for fn in sorted(os.listdir(GOLDEN)):
        if fn.endswith(".json"):
            with open(os.path.join(GOLDEN, fn)) as f:
                out.append((fn, json.load(f)))
    return out


@pytest.mark.parametrize("fn,case", _load_golden(), ids=[f for f, _ in _load_golden()])
def test_golden_fixture(fn, case):
    kind = case["kind"]
    if kind == "attention":
        q = np.array(case["q"], dtype=np.float64)
        k = np.array(case["k_cache"], dtype=np.float64)
        v = np.array(case["v_cache"], dtype=np.float64)
        pt = np.array(case["page_table"]) if case.get("page_table") is not None else None
        O, LSE = decode_attention_fp64(q, k, v, np.array(case["seq_lens"]), case["scale"],
                                       page_table=pt, page_size=case.get("page_size", 0))
        np.testing.assert_allclose(O, np.array(case["expected_o"]), atol=1e-14)
        np.testing.assert_allclose(LSE, np.array(case["expected_lse"]), rtol=1e-14)
        if "chunk" in case:
            O2, L2 = decode_attention_splitk_fp64(q, k, v, np.array(case["seq_lens"]), case["scale"],
                                                  case["chunk"], page_table=pt,
                                                  page_size=case.get("page_size", 0))
            np.testing.assert_allclose(O2, np.array(case["expected_o"]), atol=1e-14)
            np.testing.assert_allclose(L2, np.array(case["expected_lse"]), rtol=1e-14)
    elif kind == "combine":
        O, LSE = combine_fp64(np.array(case["m"]), np.array(case["l"]), np.array(case["o"]),
                              case["scale"])
        np.testing.assert_allclose(O, np.array(case["expected_o"]), atol=1e-14)
        np.testing.assert_allclose(LSE, np.array(case["expected_lse"]), rtol=1e-14)
    else:
        raise AssertionError(kind)


# ---------------------------------------------------------------------------
# the equal-share schedule of the automatic split and pass 1 over its ranges
# ---------------------------------------------------------------------------
def test_equal_share_pieces_worked_example():
    # worked by hand: tiles of 32 keys per sequence [4, 0, 2, 2], U = 8; 3 workers with
    # at least 2 tiles each -> W = min(3, 8 // 2) = 3, shares [0, 2), [2, 5), [5, 8)
    pieces, first, count = equal_share_pieces([100, 0, 33, 64], workers=3, tile=32, min_tiles=2)
    assert pieces == [(0, 0, 64, 0), (0, 64, 100, 1), (2, 0, 32, 2), (2, 32, 33, 3), (3, 0, 64, 4)]
    assert first == [0, 2, 2, 4] and count == [2, 0, 2, 1]


@pytest.mark.parametrize("seed", range(6))
def test_equal_share_pieces_cover_and_balance(seed):
    r = np.random.default_rng(seed)
    B = int(r.integers(1, 40))
    lens = r.integers(0, 3000, B)
    lens[r.random(B) < 0.2] = 0
    workers = int(r.integers(1, 300))
    pieces, first, count = equal_share_pieces(lens, workers)
    tiles = [-(-int(L) // 32) for L in lens]
    U = sum(tiles)
    W = min(workers, max(1, U // 8))
    # every key of every sequence exactly once, in order, cut only at tile boundaries
    for b in range(B):
        mine = [pc for pc in pieces if pc[0] == b]
        assert len(mine) == count[b]
        assert [pc[3] for pc in mine] == list(range(first[b], first[b] + count[b]))
        pos = 0
        for _, lo, hi, _ in mine:
            assert lo == pos and hi > lo and lo % 32 == 0
            pos = hi
        assert pos == lens[b]
    # slots are 0 .. S-1 in order; at most one extra slot per sequence boundary
    assert [pc[3] for pc in pieces] == list(range(len(pieces)))
    assert len(pieces) <= (W + B - 1 if U else 0)
    # brute force over the tiles in batch order: the tiles of one piece belong to one
    # worker, different pieces of one worker lie in different sequences, and the shares
    # differ by at most one tile and (with enough tiles) hold at least the minimum
    tile_owner = []
    for w in range(W):
        tile_owner += [w] * ((w + 1) * U // W - w * U // W)
    assert len(tile_owner) == U
    seq_of_tile = [b for b in range(B) for _ in range(tiles[b])]
    piece_worker = {}
    pos = 0
    for b, lo, hi, slot in pieces:
        n = -(-(hi - lo) // 32)
        ws = set(tile_owner[pos:pos + n])
        assert len(ws) == 1 and set(seq_of_tile[pos:pos + n]) == {b}
        piece_worker[slot] = ws.pop()
        pos += n
    assert pos == U
    per_worker = {}
    for b, lo, hi, slot in pieces:
        per_worker.setdefault(piece_worker[slot], []).append(b)
    assert all(len(set(bs)) == len(bs) for bs in per_worker.values())
    if U:
        shares = [tile_owner.count(w) for w in range(W)]
        assert max(shares) - min(shares) <= 1
        if U >= 8:
            assert min(shares) >= 8


def test_range_partials_combine_to_the_definition():
    q, k, v, lens, pt = rng_case(31, B=4, Hq=6, Hkv=2, D=8, L=(100, 0, 33, 64), paged=16)
    O, LSE = decode_attention_fp64(q, k, v, lens, 0.3, page_table=pt, page_size=16)
    pieces, first, count = equal_share_pieces(lens, workers=3, tile=32, min_tiles=2)
    m, l, Op = range_partials_fp64(q, k, v, lens, 0.3, pieces, page_table=pt, page_size=16)
    for b in range(4):
        sl = slice(first[b], first[b] + count[b])
        Oc, Lc = combine_fp64(m[sl].T, l[sl].T, Op[sl].transpose(1, 0, 2), 0.3)
        np.testing.assert_allclose(Oc, O[b], atol=1e-14)
        np.testing.assert_allclose(Lc, LSE[b], rtol=1e-14)
    # a piece that is a fixed chunk equals pass 1 with that chunk
    mf, lf, Of = partition_partials_fp64(q, k, v, lens, 0.3, chunk=64, num_partitions=2,
                                         page_table=pt, page_size=16)
    np.testing.assert_allclose(m[0], mf[0, :, 0], rtol=1e-15)
    np.testing.assert_allclose(l[0], lf[0, :, 0], rtol=1e-14)
    np.testing.assert_allclose(Op[0], Of[0, :, 0], atol=1e-15)


# ---------------------------------------------------------------------------
# fp8 (E4M3) caches with per-token scales
# ---------------------------------------------------------------------------
def test_fp8_decode_matches_torch_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8_e4m3_to_fp64(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    assert np.array_equal(ours[~np.isnan(ours)], lib[~np.isnan(lib)])


def test_fp8_decode_special_codes():
    # worked from the format: sign | exponent (bias 7) | 3-bit mantissa
    got = fp8_e4m3_to_fp64(np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x7E, 0xFE, 0x7F, 0xFF],
                                    dtype=np.uint8))
    want = [0.0, -0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.5, 448.0, -448.0]
    np.testing.assert_array_equal(got[:9], want)
    assert np.signbit(got[1]) and np.isnan(got[9]) and np.isnan(got[10])


def _fp8_case(seed, paged):
    from lse_combine_amd.inputs import make_case
    return make_case("f8", batch=3, num_q_heads=4, num_kv_heads=2, qk_depth=8, page_size=4 if paged else 0,
                     seq_lens=[9, 1, 6], seed=seed, kv_fp8=True, dtype=torch.float32)


@pytest.mark.parametrize("paged", [0, 1])
def test_fp8_cache_brute_force_with_torch_decode(paged):
    c = _fp8_case(70 + paged, paged)
    pt = None if c.page_table is None else c.page_table.numpy()
    O, LSE = decode_attention_fp64(c.q.numpy(), c.k_cache.numpy(), c.v_cache.numpy(), c.seq_lens.numpy(),
                                   c.scale, page_table=pt, page_size=c.page_size,
                                   k_scale=c.k_scale.numpy(), v_scale=c.v_scale.numpy())
    # the cache values as torch decodes them, times the scale of their (token, kv head);
    # scales are stored tokens-innermost, the cache rows token-major
    kd = c.k_cache.view(torch.float8_e4m3fn).double() * c.k_scale.double().permute(0, 2, 1)[..., None]
    vd = c.v_cache.view(torch.float8_e4m3fn).double() * c.v_scale.double().permute(0, 2, 1)[..., None]
    Ob, Lb = brute(c.q.double().numpy(), kd.numpy(), vd.numpy(), c.seq_lens.numpy(), c.scale, pt,
                   c.page_size)
    np.testing.assert_allclose(O, Ob, atol=1e-13)
    np.testing.assert_allclose(LSE, Lb, rtol=1e-13)


def test_fp8_scales_act_as_closed_forms():
    c = _fp8_case(72, 1)
    pt = c.page_table.numpy()
    base = dict(page_table=pt, page_size=c.page_size)
    args = (c.q.numpy(), c.k_cache.numpy(), c.v_cache.numpy(), c.seq_lens.numpy())
    ks, vs = c.k_scale.numpy(), c.v_scale.numpy()
    O, LSE = decode_attention_fp64(*args, c.scale, k_scale=ks, v_scale=vs, **base)
    # all K scales times 4 = the softmax scale times 4
    O4, L4 = decode_attention_fp64(*args, 4 * c.scale, k_scale=ks, v_scale=vs, **base)
    O4b, L4b = decode_attention_fp64(*args, c.scale, k_scale=4 * ks, v_scale=vs, **base)
    np.testing.assert_allclose(O4b, O4, atol=1e-14)
    np.testing.assert_allclose(L4b, L4, rtol=1e-14)
    # all V scales times 3 = O times 3, LSE unchanged
    O3, L3 = decode_attention_fp64(*args, c.scale, k_scale=ks, v_scale=3 * vs.astype(np.float64), **base)
    np.testing.assert_allclose(O3, 3 * O, atol=1e-14)
    np.testing.assert_allclose(L3, LSE, rtol=1e-15)


# ---------------------------------------------------------------------------
# several queries per sequence (causal among the last q_len positions)
# ---------------------------------------------------------------------------
def brute_multiquery(q4, k, v, lens, scale, pt=None, ps=0):
    # each query i of q_len, at position L - q_len + i, over the keys up to that position
    B, ql = q4.shape[:2]
    Os, Ls = [], []
    for i in range(ql):
        li = [max(0, min(int(L), int(L) - ql + 1 + i)) for L in lens]
        o, l = brute(q4[:, i], k, v, li, scale, pt, ps)
        Os.append(o)
        Ls.append(l)
    return np.stack(Os, 1), np.stack(Ls, 1)


@pytest.mark.parametrize("paged", [0, 4])
def test_multiquery_brute_force(paged):
    q, k, v, lens, pt = rng_case(90 + paged, B=3, Hq=4, Hkv=2, D=8, L=(7, 2, 5), paged=paged)
    r = np.random.default_rng(91)
    q4 = r.standard_normal((3, 3, 4, 8))          # q_len 3 (one sequence shorter than q_len)
    O, LSE = decode_attention_fp64(q4, k, v, lens, 0.6, page_table=pt, page_size=paged)
    Ob, Lb = brute_multiquery(q4, k, v, lens, 0.6, pt, paged)
    np.testing.assert_allclose(O, Ob, atol=1e-13)
    np.testing.assert_allclose(LSE, Lb, rtol=1e-13)
    # the last query sees the whole sequence: it is the single-query result
    O1, L1 = decode_attention_fp64(q4[:, -1], k, v, lens, 0.6, page_table=pt, page_size=paged)
    np.testing.assert_allclose(O[:, -1], O1, atol=0)
    # a sequence of 2 keys with q_len 3: query 0 sees nothing (O = 0, LSE = -inf)
    assert np.all(O[1, 0] == 0) and np.all(np.isneginf(LSE[1, 0]))


# ---------------------------------------------------------------------------
# rotary columns stored apart (own tensor, own dtype), V depth != nope depth
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("paged", [0, 4])
def test_rope_apart_is_the_row_nope_then_rotary(paged):
    # splitting a K row into [nope | rotary] storage changes nothing; the other order would
    q, k, v, lens, pt = rng_case(95 + paged, B=3, Hq=4, Hkv=2, D=10, Dv=7, L=(9, 1, 6), paged=paged)
    O, LSE = decode_attention_fp64(q, k, v, lens, 0.4, page_table=pt, page_size=paged)
    Oa, La = decode_attention_fp64(q, k[..., :6], v, lens, 0.4, page_table=pt, page_size=paged, k_rope=k[..., 6:])
    np.testing.assert_array_equal(Oa, O)
    np.testing.assert_array_equal(La, LSE)
    Ob, Lb = brute(q, k, v, lens, 0.4, pt, paged)
    np.testing.assert_allclose(Oa, Ob, atol=1e-13)
    Ow, _ = decode_attention_fp64(q, k[..., 4:], v, lens, 0.4, page_table=pt, page_size=paged, k_rope=k[..., :4])
    assert np.abs(Ow - O).max() > 1e-3
    with pytest.raises(ValueError):
        decode_attention_fp64(q, k[..., :6], v, lens, 0.4, page_table=pt, page_size=paged, k_rope=k[..., 7:])


@pytest.mark.parametrize("paged", [0, 1])
def test_fp8_nope_with_bf16_rotary_brute_force_with_torch_decode(paged):
    # GLM-style shape in miniature: nope 8 (fp8, per-token scales) + 4 rotary (bf16) and
    # V depth 10 != nope; the scales apply to the nope columns only
    from lse_combine_amd.inputs import make_case
    c = make_case("glm", batch=3, num_q_heads=4, num_kv_heads=2, qk_depth=12, ov_depth=10,
                  page_size=4 if paged else 0, seq_lens=[9, 1, 6], seed=96 + paged, kv_fp8=True,
                  dtype=torch.float32, rope_apart=4)
    assert c.k_cache.shape[-1] == 8 and c.k_rope.shape[-1] == 4 and c.k_rope.dtype == torch.bfloat16
    pt = None if c.page_table is None else c.page_table.numpy()
    O, LSE = decode_attention_fp64(c.q.numpy(), c.k_cache.numpy(), c.v_cache.numpy(), c.seq_lens.numpy(),
                                   c.scale, page_table=pt, page_size=c.page_size, k_scale=c.k_scale.numpy(),
                                   v_scale=c.v_scale.numpy(), k_rope=c.k_rope.float().numpy())
    kn = c.k_cache.view(torch.float8_e4m3fn).double() * c.k_scale.double().permute(0, 2, 1)[..., None]
    kd = torch.cat([kn, c.k_rope.double()], dim=-1)
    vd = c.v_cache.view(torch.float8_e4m3fn).double() * c.v_scale.double().permute(0, 2, 1)[..., None]
    Ob, Lb = brute(c.q.double().numpy(), kd.numpy(), vd.numpy(), c.seq_lens.numpy(), c.scale, pt, c.page_size)
    np.testing.assert_allclose(O, Ob, atol=1e-13)
    np.testing.assert_allclose(LSE, Lb, rtol=1e-13)
    assert O.shape[-1] == 10


# ---------------------------------------------------------------------------
# one kv head for every q head: latent rows with the rotary columns stored apart, and a V
# of its own whose depth differs from the nope depth; one and several queries
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("paged", [0, 4])
@pytest.mark.parametrize("q_len", [1, 2])
def test_latent_rows_with_rotary_apart_brute_force(paged, q_len):
    # K row = [nope 8 | rotary 4], V = the first 6 nope columns (a prefix of the stored K
    # columns, scale-free); brute force on the materialised full row and V
    q, k, _, lens, pt = rng_case(200 + paged + q_len, B=3, Hq=6, Hkv=1, D=12, L=(9, 1, 14), paged=paged)
    if q_len > 1:
        q = np.random.default_rng(201).standard_normal((3, q_len, 6, 12))
    O, LSE = decode_attention_fp64(q, k[..., :8], None, lens, 0.45, page_table=pt, page_size=paged,
                                   v_is_k_prefix=True, ov_depth=6, k_rope=k[..., 8:])
    v = np.ascontiguousarray(k[..., :6])
    if q_len > 1:
        Ob, Lb = brute_multiquery(q, k, v, lens, 0.45, pt, paged)
    else:
        Ob, Lb = brute(q, k, v, lens, 0.45, pt, paged)
    np.testing.assert_allclose(O, Ob, atol=1e-13)
    np.testing.assert_allclose(LSE, Lb, rtol=1e-13)
    assert O.shape[-1] == 6
    # a V taken from other columns of the row (here the last 6) gives another result
    O_wrong, _ = decode_attention_fp64(q, k, np.ascontiguousarray(k[..., 6:]), lens, 0.45, page_table=pt,
                                       page_size=paged)
    assert np.abs(O_wrong - O).max() > 1e-3


@pytest.mark.parametrize("paged", [0, 4])
@pytest.mark.parametrize("q_len", [1, 3])
def test_one_kv_head_own_v_depth_brute_force(paged, q_len):
    # GLM-style widths in miniature with one kv head for all 8 q heads: K = [nope 6 | rotary
    # 2] stored apart, V of depth 9 (!= nope 6) in a cache of its own
    q, k, v, lens, pt = rng_case(210 + paged + q_len, B=2, Hq=8, Hkv=1, D=8, Dv=9, L=(11, 5), paged=paged)
    if q_len > 1:
        q = np.random.default_rng(211).standard_normal((2, q_len, 8, 8))
    O, LSE = decode_attention_fp64(q, k[..., :6], v, lens, 0.5, page_table=pt, page_size=paged, k_rope=k[..., 6:])
    if q_len > 1:
        Ob, Lb = brute_multiquery(q, k, v, lens, 0.5, pt, paged)
    else:
        Ob, Lb = brute(q, k, v, lens, 0.5, pt, paged)
    np.testing.assert_allclose(O, Ob, atol=1e-13)
    np.testing.assert_allclose(LSE, Lb, rtol=1e-13)
    assert O.shape[-1] == 9


@pytest.mark.parametrize("paged", [0, 1])
def test_fp8_latent_v_is_scaled_k_prefix_brute_force_with_torch_decode(paged):
    # MLA-style latent in miniature over an fp8 cache: K row = [nope 8 as E4M3 codes with a
    # per-token scale | rotary 4 in bf16, stored apart], V = the first 6 nope columns, so V
    # is read as code x the token's K scale (no V scale of its own)
    from lse_combine_amd.inputs import make_case
    c = make_case("lat8", batch=3, num_q_heads=6, num_kv_heads=1, qk_depth=12, ov_depth=6,
                  page_size=4 if paged else 0, seq_lens=[9, 1, 14], seed=230 + paged, kv_fp8=True,
                  dtype=torch.float32, rope_apart=4, v_is_k_prefix=True)
    assert c.v_cache is None and c.v_scale is None and c.k_cache.dtype == torch.uint8
    pt = None if c.page_table is None else c.page_table.numpy()
    O, LSE = decode_attention_fp64(c.q.numpy(), c.k_cache.numpy(), None, c.seq_lens.numpy(), c.scale,
                                   page_table=pt, page_size=c.page_size, v_is_k_prefix=True, ov_depth=6,
                                   k_scale=c.k_scale.numpy(), k_rope=c.k_rope.float().numpy())
    kn = c.k_cache.view(torch.float8_e4m3fn).double() * c.k_scale.double().permute(0, 2, 1)[..., None]
    kd = torch.cat([kn, c.k_rope.double()], dim=-1)
    vd = kn[..., :6].contiguous()
    Ob, Lb = brute(c.q.double().numpy(), kd.numpy(), vd.numpy(), c.seq_lens.numpy(), c.scale, pt, c.page_size)
    np.testing.assert_allclose(O, Ob, atol=1e-13)
    np.testing.assert_allclose(LSE, Lb, rtol=1e-13)
    # V from the unscaled codes (the scale dropped on the V side) gives another result
    Ow, _ = brute(c.q.double().numpy(), kd.numpy(),
                  c.k_cache.view(torch.float8_e4m3fn).double()[..., :6].contiguous().numpy(),
                  c.seq_lens.numpy(), c.scale, pt, c.page_size)
    assert np.abs(Ow - O).max() > 1e-3
