"""Host-side checks of the C ABI (no GPU needed): symbols, validation, split
selection, workspace sizing and error paths. Nothing here launches a kernel."""

import ctypes
import math

import pytest

from lse_combine_amd import _lib
from lse_combine_amd._lib import (DA_EINVAL, DA_EUNSUPPORTED, DA_EWORKSPACE, DA_OK, DaProblem)

FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def prob(**kw):
    p = DaProblem()
    base = dict(batch=2, num_q_heads=16, num_kv_heads=2, qk_depth=128, ov_depth=128, dtype=1, page_size=64,
                max_pages_per_seq=64, num_pages=128, kv_capacity=0, max_seq_len=4096, v_is_k_prefix=0, kernel=0)
    base.update(kw)
    for k, v in base.items():
        setattr(p, k, v)
    return p


def test_exports_every_declared_function(lib):
    names = _lib.header_functions()
    assert {"decode_attn_splitk", "decode_attn_splitk_fused", "decode_attn_partition", "decode_attn_combine",
            "da_supported",
            "da_choose_splits", "da_workspace_bytes", "da_last_error", "da_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert b"gfx950" in lib.da_version()


def test_probe_library_is_apart_from_the_product():
    # the measurement probes live in their own library and header; the attention library
    # neither declares nor exports them
    probe = _lib.load_probe()
    names = _lib.header_functions(_lib.PROBE_HEADER)
    assert set(names) == {"da_read_probe", "da_copy_probe"}
    for n in names:
        assert hasattr(probe, n), n
        assert n not in _lib.header_functions()
    prod = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert not hasattr(prod, n), n


@pytest.mark.parametrize("kw,code", [
    (dict(), DA_OK),
    (dict(dtype=0), DA_OK),
    (dict(num_q_heads=2, num_kv_heads=2), DA_OK),
    (dict(num_q_heads=32, num_kv_heads=2), DA_OK),             # group 16
    (dict(num_q_heads=34, num_kv_heads=2), DA_OK),             # group 17: 17 virtual kv heads of one
    (dict(num_q_heads=34, num_kv_heads=2, dtype=0), DA_OK),          # ... also on the vector ALU
    (dict(num_q_heads=15, num_kv_heads=2), DA_EINVAL),         # not a multiple
    (dict(qk_depth=96, ov_depth=96), DA_EUNSUPPORTED),
    (dict(dtype=7), DA_EINVAL),
    (dict(batch=0), DA_EINVAL),
    (dict(page_size=-1), DA_EINVAL),
    (dict(max_pages_per_seq=10), DA_EINVAL),                   # 10 * 64 < 4096
    (dict(page_size=0, kv_capacity=0), DA_EINVAL),
    (dict(page_size=0, kv_capacity=4096), DA_OK),
    (dict(dtype=0, kernel=2), DA_EUNSUPPORTED),                # matrix cores need bf16
    (dict(kernel=5), DA_EINVAL),
    (dict(v_is_k_prefix=1, ov_depth=600, qk_depth=576), DA_EINVAL),
    (dict(num_q_heads=128, num_kv_heads=2, qk_depth=576, ov_depth=512, v_is_k_prefix=1), DA_EUNSUPPORTED),
    (dict(num_q_heads=128, num_kv_heads=1, qk_depth=576, ov_depth=512, v_is_k_prefix=1), DA_OK),
    (dict(num_q_heads=24, num_kv_heads=1, qk_depth=576, ov_depth=512, v_is_k_prefix=1), DA_OK),   # any head count
    (dict(num_q_heads=128, num_kv_heads=1, qk_depth=576, ov_depth=512, v_is_k_prefix=1, nope_depth=512,
          rope_dtype=1), DA_OK),                                                                    # rotary apart
    (dict(num_q_heads=128, num_kv_heads=1, qk_depth=576, ov_depth=512, v_is_k_prefix=1, nope_depth=448,
          rope_dtype=1), DA_EUNSUPPORTED),
    (dict(num_q_heads=128, num_kv_heads=1, qk_depth=256, ov_depth=256), DA_OK),       # one kv head, own V
    (dict(num_q_heads=128, num_kv_heads=1, qk_depth=256, ov_depth=256, nope_depth=192, rope_dtype=1), DA_OK),
    (dict(num_q_heads=128, num_kv_heads=1, qk_depth=256, ov_depth=256, nope_depth=192, rope_dtype=0),
     DA_EUNSUPPORTED),
    (dict(num_q_heads=128, num_kv_heads=2, qk_depth=256, ov_depth=256), DA_OK),   # group 64: 4 virtual x 16
    (dict(num_q_heads=128, num_kv_heads=1, qk_depth=576, ov_depth=512, v_is_k_prefix=0), DA_EUNSUPPORTED),
    (dict(num_q_heads=128, num_kv_heads=1, qk_depth=576, ov_depth=512, v_is_k_prefix=1, dtype=0), DA_EUNSUPPORTED),
])
def test_supported(lib, kw, code):
    p = prob(**kw)
    assert lib.da_supported(ctypes.byref(p)) == code
    if code != DA_OK:
        assert lib.da_last_error()


def test_supported_null(lib):
    assert lib.da_supported(None) == DA_EINVAL
    assert b"NULL" in lib.da_last_error()


def splits(lib, p, n, cus=256):
    C, P = ctypes.c_int32(), ctypes.c_int32()
    assert lib.da_choose_splits(ctypes.byref(p), n, cus, ctypes.byref(C), ctypes.byref(P)) == DA_OK
    return C.value, P.value


def test_fixed_splits_match_the_named_workloads(lib):
    # tiny: L 1024, 4 partitions of 256 keys, contiguous
    assert splits(lib, prob(batch=1, num_q_heads=1, num_kv_heads=1, dtype=0, page_size=0, kv_capacity=1024,
                            max_seq_len=1024), 4) == (256, 4)
    # GQA: L 4096, 8 splits
    assert splits(lib, prob(batch=8, num_q_heads=32, num_kv_heads=8, page_size=0, kv_capacity=4096,
                            max_seq_len=4096), 8) == (512, 8)
    # long: L 131072, page 64, 64 splits
    assert splits(lib, prob(batch=1, num_q_heads=32, num_kv_heads=4, max_pages_per_seq=2048,
                            max_seq_len=131072), 64) == (2048, 64)
    # latent-shared: L 8192, page 64, 8 splits
    assert splits(lib, prob(batch=16, num_q_heads=128, num_kv_heads=1, qk_depth=576, ov_depth=512,
                            v_is_k_prefix=1, max_pages_per_seq=128, max_seq_len=8192), 8) == (1024, 8)


def test_fused_fold_applies_where_one_workgroup_reads_at_most_64_kib(lib):
    # (compute units: the device's, 256 on this host without one, as on an MI355X)
    applies = lambda p, n: lib.da_fused_applies(ctypes.byref(p), n)
    tiny = prob(batch=1, num_q_heads=1, num_kv_heads=1, dtype=0, page_size=0, kv_capacity=1024, max_seq_len=1024)
    gqa = prob(batch=8, num_q_heads=32, num_kv_heads=8, page_size=0, kv_capacity=4096, max_seq_len=4096)
    long_ = prob(batch=1, num_q_heads=32, num_kv_heads=4, max_pages_per_seq=2048, max_seq_len=131072)
    latent = prob(batch=16, num_q_heads=128, num_kv_heads=1, qk_depth=576, ov_depth=512, v_is_k_prefix=1,
                  max_pages_per_seq=128, max_seq_len=8192)
    paged = prob(batch=32, num_q_heads=64, num_kv_heads=8, max_pages_per_seq=512, max_seq_len=32768)
    assert applies(tiny, 4) == 1      # 4 partials x 1 row x 512 B
    assert applies(gqa, 8) == 1       # 8 x 8 rows (2 kv heads per workgroup) x 512 B = 32 KiB
    assert applies(gqa, 16) == 0      # 4 kv heads per workgroup: 16 x 16 rows x 512 B = 128 KiB
    assert applies(long_, 64) == 0    # 64 x 8 rows x 512 B = 256 KiB
    assert applies(latent, 8) == 0    # 8 x 64 rows x 2 KiB = 1 MiB
    # equal shares: a sequence of max_seq_len keys meets at most ceil(tiles / 8) + 1 of the
    # 256 workers' shares
    assert applies(long_, 0) == 0     # min(256, 513) x 32 rows x 512 B
    assert applies(paged, 0) == 0     # 129 x 64 rows x 512 B
    short = prob(batch=8, num_q_heads=8, num_kv_heads=1, max_pages_per_seq=8, max_seq_len=512)
    assert applies(short, 0) == 1     # 3 x 8 rows x 512 B = 12 KiB
    assert applies(prob(batch=8, num_q_heads=8, num_kv_heads=1, max_pages_per_seq=64, max_seq_len=4096), 0) == 0
    assert applies(prob(batch=0), 8) == DA_EINVAL


def test_fused_mode_argument(lib):
    p = prob()
    kv = _lib.DaKv(FAKE.value, FAKE.value, None, None, None)
    for bad in (-1, 3):
        r = lib.decode_attn_splitk_kv(ctypes.byref(p), FAKE, ctypes.byref(kv), FAKE, FAKE, 0.1, 0, bad, FAKE,
                                      None, None, FAKE, 1 << 20, None)
        assert r == DA_EINVAL and b"fused" in lib.da_last_error()


@pytest.mark.parametrize("L,n,ps,dtype", [(1000, 3, 0, 1), (1000, 3, 64, 1), (77, 5, 0, 1), (5000, 7, 16, 1),
                                          (1, 1, 0, 1), (4096, 4096, 0, 1), (32768, 0, 64, 0), (131072, 0, 64, 0),
                                          (100, 0, 48, 0)])
def test_split_invariants(lib, L, n, ps, dtype):
    # fixed chunks: explicit splits, and the automatic choice of the vector-ALU kernel (fp32)
    kw = dict(max_seq_len=L, dtype=dtype)
    if ps:
        kw.update(page_size=ps, max_pages_per_seq=-(-L // ps))
    else:
        kw.update(page_size=0, kv_capacity=L)
    C, P = splits(lib, prob(**kw), n)
    assert C % 32 == 0 and C >= 32
    if ps and ps % 32 == 0:
        assert C % ps == 0
    assert P == math.ceil(L / C) and (P - 1) * C < L <= P * C   # no empty trailing partition
    if n:
        assert P <= n


@pytest.mark.parametrize("B,Hkv,L,cus,hg", [(32, 8, 32768, 256, 8), (8, 8, 4096, 256, 4), (1, 4, 131072, 256, 4),
                                             (1, 1, 100, 256, 1), (2, 2, 300, 80, 1), (64, 8, 512, 304, 2)])
def test_automatic_split_is_equal_shares_on_matrix_cores(lib, B, Hkv, L, cus, hg):
    # bf16 GQA, automatic: chunk 0 names the equal-share schedule, max_splits the workers per
    # kv-head group; one 8-wave workgroup per CU in total
    p = prob(batch=B, num_q_heads=8 * Hkv, num_kv_heads=Hkv, max_seq_len=L, max_pages_per_seq=-(-L // 64))
    C, W = splits(lib, p, 0, cus)
    groups = -(-Hkv // hg)
    assert C == 0 and W == -(-cus // groups)


def test_equal_share_workspace_and_checks(lib):
    p = prob(batch=3, num_q_heads=8, num_kv_heads=1, max_seq_len=1000, max_pages_per_seq=16)
    n = ctypes.c_size_t()
    assert lib.da_workspace_bytes(ctypes.byref(p), 0, ctypes.byref(n)) == DA_OK
    C, W = splits(lib, p, 0)
    assert C == 0
    align = lambda x: (x + 255) // 256 * 256  # noqa: E731
    rows = (W + 3) * 8
    assert n.value == align(rows * 2 * 4 + 3 * 2 * 4) + align(rows * 128 * 4) + align(3 * 1 * 4)
    f = lib.decode_attn_partition
    # chunk 0 needs the matrix-core kernel and 1 <= workers <= 65535
    fp32 = prob(dtype=0)
    assert f(ctypes.byref(fp32), FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, 0, 8, FAKE, FAKE, None) == DA_EUNSUPPORTED
    assert f(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, 0, 0, FAKE, FAKE, None) == DA_EINVAL
    assert f(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, -32, 8, FAKE, FAKE, None) == DA_EINVAL


def test_workspace_bytes(lib):
    p = prob(batch=3, num_q_heads=8, num_kv_heads=1, max_seq_len=1000, max_pages_per_seq=16)
    n = ctypes.c_size_t()
    assert lib.da_workspace_bytes(ctypes.byref(p), 4, ctypes.byref(n)) == DA_OK
    C, P = splits(lib, p, 4)
    rows = 3 * 8 * P
    align = lambda x: (x + 255) // 256 * 256  # noqa: E731
    # (m, l) pairs, partial outputs, and the [B][Hkv] arrival counters of the fused combine
    assert n.value == align(rows * 2 * 4) + align(rows * 128 * 4) + align(3 * 1 * 4)


def call_splitk(lib, p, scale=0.1, ws=FAKE, ws_bytes=1 << 30, q=FAKE, k=FAKE, v=FAKE, pt=FAKE, lens=FAKE, out=FAKE):
    return lib.decode_attn_splitk(ctypes.byref(p), q, k, v, pt, lens, scale, 0, out, None, None, ws, ws_bytes, None)


def test_error_paths_return_codes_without_launching(lib):
    p = prob()
    assert call_splitk(lib, p, q=None) == DA_EINVAL
    assert call_splitk(lib, p, pt=None) == DA_EINVAL                     # paged needs a table
    assert call_splitk(lib, prob(page_size=0, kv_capacity=4096)) == DA_EINVAL  # contiguous must not get one
    assert call_splitk(lib, p, out=None) == DA_EINVAL
    assert call_splitk(lib, p, scale=0.0) == DA_EINVAL
    assert call_splitk(lib, p, scale=float("nan")) == DA_EINVAL
    assert call_splitk(lib, p, scale=-1.0) == DA_EINVAL
    assert call_splitk(lib, p, ws=None) == DA_EWORKSPACE
    assert call_splitk(lib, p, ws=ctypes.c_void_p(0x1008)) == DA_EWORKSPACE   # misaligned
    assert call_splitk(lib, p, ws_bytes=16) == DA_EWORKSPACE
    assert b"workspace too small" in lib.da_last_error()
    assert call_splitk(lib, prob(num_q_heads=15)) == DA_EINVAL


def test_partition_and_combine_argument_checks(lib):
    p = prob()
    f = lib.decode_attn_partition
    assert f(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, 100, 64, FAKE, FAKE, None) == DA_EINVAL  # chunk % 32
    assert f(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, 256, 8, FAKE, FAKE, None) == DA_EINVAL   # splits
    assert f(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, 256, 16, None, FAKE, None) == DA_EINVAL
    c = lib.decode_attn_combine
    assert c(ctypes.byref(p), FAKE, 0.1, 256, 16, FAKE, FAKE, None, None, None, None) == DA_EINVAL
    assert c(ctypes.byref(p), FAKE, 0.1, 33, 16, FAKE, FAKE, FAKE, None, None, None) == DA_EINVAL
    assert c(ctypes.byref(prob(ov_depth=96, qk_depth=96)), FAKE, 0.1, 256, 16, FAKE, FAKE, FAKE, None, None,
             None) == DA_EUNSUPPORTED


def test_probe_argument_checks():
    probe = _lib.load_probe()
    assert probe.da_read_probe(FAKE, 15, FAKE, None) == DA_EINVAL
    assert probe.da_copy_probe(FAKE, None, 16, None) == DA_EINVAL


@pytest.mark.parametrize("kw,code", [
    (dict(kv_dtype=2), DA_OK),                                   # paged 64, bf16 q
    (dict(kv_dtype=2, page_size=0, kv_capacity=4096), DA_OK),    # contiguous
    (dict(kv_dtype=2, page_size=16, max_pages_per_seq=256), DA_OK),             # a page per half tile
    (dict(kv_dtype=2, page_size=8, max_pages_per_seq=512), DA_OK),              # per-key page lookup
    (dict(kv_dtype=2, page_size=48, max_pages_per_seq=100), DA_OK),             # not a power of two
    (dict(kv_dtype=2, dtype=0), DA_EUNSUPPORTED),                # fp32 q
    (dict(kv_dtype=2, kernel=1), DA_EUNSUPPORTED),               # vector-ALU kernel
    # latent over fp8: the rotary columns apart in bf16 or as codes in the K rows, any page size
    (dict(kv_dtype=2, num_q_heads=128, num_kv_heads=1, qk_depth=576, ov_depth=512, v_is_k_prefix=1),
     DA_OK),                                                                 # rotary codes in the K rows
    (dict(kv_dtype=2, num_q_heads=128, num_kv_heads=1, qk_depth=576, ov_depth=512, v_is_k_prefix=1,
          nope_depth=512, rope_dtype=1), DA_OK),
    (dict(kv_dtype=2, num_q_heads=16, num_kv_heads=1, qk_depth=576, ov_depth=512, v_is_k_prefix=1,
          nope_depth=512, rope_dtype=1, q_len=3, page_size=0, kv_capacity=4096), DA_OK),
    (dict(kv_dtype=2, num_q_heads=128, num_kv_heads=1, qk_depth=576, ov_depth=512, v_is_k_prefix=1,
          nope_depth=512, rope_dtype=1, page_size=48, max_pages_per_seq=100), DA_OK),
    (dict(kv_dtype=2, num_q_heads=128, num_kv_heads=1, qk_depth=576, ov_depth=512, v_is_k_prefix=1,
          nope_depth=512, rope_dtype=1, page_size=16, max_pages_per_seq=256), DA_OK),
    (dict(kv_dtype=2, num_q_heads=128, num_kv_heads=1, qk_depth=576, ov_depth=512, v_is_k_prefix=1,
          nope_depth=512, rope_dtype=1, page_size=16, max_pages_per_seq=256, num_pages=1 << 25),
     DA_EUNSUPPORTED),                                                       # scales past 2 GiB
    (dict(kv_dtype=2, num_q_heads=128, num_kv_heads=1, qk_depth=256, ov_depth=256, nope_depth=192,
          rope_dtype=1), DA_OK),                                             # one-kv-head GLM widths
    (dict(kv_dtype=2, num_q_heads=128, num_kv_heads=1, qk_depth=256, ov_depth=256), DA_OK),   # rotary inline
    (dict(kv_dtype=2, num_q_heads=128, num_kv_heads=1, qk_depth=256, ov_depth=256, page_size=48,
          max_pages_per_seq=100), DA_OK),
    (dict(kv_dtype=2, num_q_heads=128, num_kv_heads=1, qk_depth=256, ov_depth=256, nope_depth=192,
          rope_dtype=1, page_size=48, max_pages_per_seq=100), DA_OK),
    (dict(kv_dtype=7), DA_EINVAL),
])
def test_fp8_cache_support(lib, kw, code):
    assert lib.da_supported(ctypes.byref(prob(**kw))) == code


def test_fp8_entry_points_need_their_scales(lib):
    p8 = prob(kv_dtype=2)
    # the plain entry point has no scale argument: an fp8 problem is refused
    assert call_splitk(lib, p8) == DA_EINVAL
    assert b"k_scale" in lib.da_last_error()
    f = lib.decode_attn_splitk_fp8
    args = (FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 0.1, 0, FAKE, None, None, FAKE, 1 << 30, None)
    assert f(ctypes.byref(p8), *args) == DA_EINVAL                 # k_scale NULL
    assert f(ctypes.byref(prob()), *args) == DA_EINVAL             # not an fp8 problem
    g = lib.decode_attn_partition_fp8
    assert g(ctypes.byref(prob()), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 0.1, 256, 16, FAKE, FAKE,
             None) == DA_EINVAL


@pytest.mark.parametrize("kw,code", [
    (dict(q_len=2), DA_OK),                                        # 2 x 8 columns
    (dict(q_len=2, page_size=0, kv_capacity=4096), DA_OK),
    (dict(q_len=3, num_q_heads=16, num_kv_heads=2), DA_OK),        # 24 columns: 2 virtual kv heads of 4
    (dict(q_len=2, dtype=0), DA_EUNSUPPORTED),                     # vector-ALU kernel
    (dict(q_len=2, page_size=16, max_pages_per_seq=256), DA_OK),
    (dict(q_len=2, page_size=48, max_pages_per_seq=100), DA_OK),   # per-key page lookup
    (dict(q_len=2, page_size=48, max_pages_per_seq=100, kv_dtype=2), DA_OK),
    (dict(q_len=2, kv_dtype=2), DA_OK),
    (dict(q_len=17), DA_EINVAL),
    (dict(q_len=2, num_q_heads=128, num_kv_heads=1, qk_depth=576, ov_depth=512, v_is_k_prefix=1), DA_OK),
    (dict(q_len=3, num_q_heads=32, num_kv_heads=1, qk_depth=256, ov_depth=256, nope_depth=192, rope_dtype=1),
     DA_OK),                                                       # 96 columns on the shared-kv-head kernel
])
def test_multiquery_support(lib, kw, code):
    assert lib.da_supported(ctypes.byref(prob(**kw))) == code


def test_multiquery_workspace_rows(lib):
    p1, p2 = prob(batch=3, num_q_heads=8, num_kv_heads=1, max_seq_len=1000, max_pages_per_seq=16), \
        prob(batch=3, num_q_heads=8, num_kv_heads=1, max_seq_len=1000, max_pages_per_seq=16, q_len=2)
    n1, n2 = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.da_workspace_bytes(ctypes.byref(p1), 4, ctypes.byref(n1)) == DA_OK
    assert lib.da_workspace_bytes(ctypes.byref(p2), 4, ctypes.byref(n2)) == DA_OK
    C, P = splits(lib, p1, 4)
    align = lambda x: (x + 255) // 256 * 256  # noqa: E731
    rows = 3 * 8 * 2 * P   # (query, head) rows
    assert n2.value == align(rows * 2 * 4) + align(rows * 128 * 4) + align(3 * 1 * 4)


def test_binding_refuses_output_buffers_without_every_row():
    """The library writes B * q_len * Hq rows through raw pointers; the binding checks
    the caller's buffers hold them all before anything is launched."""
    import torch
    from lse_combine_amd import api
    p1 = prob(batch=3, num_q_heads=8, num_kv_heads=1, max_seq_len=1000, max_pages_per_seq=16)
    p2 = prob(batch=3, num_q_heads=8, num_kv_heads=1, max_seq_len=1000, max_pages_per_seq=16, q_len=2)
    assert api.row_shape(p1) == (3, 8) and api.row_shape(p2) == (3, 2, 8)
    too_small = torch.empty((3, 8, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="shape"):
        api.check_outputs(p2, out=too_small)
    with pytest.raises(ValueError, match="shape"):
        api.check_outputs(p2, lse=torch.empty((3, 8), dtype=torch.float32))
    with pytest.raises(ValueError, match="shape"):
        api.check_outputs(p1, o32=torch.empty((3, 8, 128), dtype=torch.bfloat16))
    # right size and type: only the device is left to object on a CPU-only host
    with pytest.raises(ValueError, match="GPU"):
        api.check_outputs(p2, out=torch.empty((3, 2, 8, 128), dtype=torch.bfloat16))
    api.check_outputs(p1)   # nothing given, nothing to check


@pytest.mark.parametrize("kw,code", [
    (dict(qk_depth=256, ov_depth=256), DA_OK),
    (dict(qk_depth=256, ov_depth=256, nope_depth=192, rope_dtype=1), DA_OK),
    (dict(qk_depth=256, ov_depth=256, nope_depth=192, rope_dtype=1, kv_dtype=2), DA_OK),
    (dict(qk_depth=192, ov_depth=128, nope_depth=128, rope_dtype=1), DA_OK),
    (dict(qk_depth=192, ov_depth=128, kv_dtype=2, q_len=2), DA_OK),
    (dict(qk_depth=256, ov_depth=256, num_q_heads=2, num_kv_heads=2), DA_OK),    # one q head per kv head
    (dict(qk_depth=256, ov_depth=256, nope_depth=192, rope_dtype=0), DA_EUNSUPPORTED),   # fp32 rotary
    (dict(qk_depth=256, ov_depth=256, nope_depth=128, rope_dtype=1), DA_EUNSUPPORTED),   # 128 rotary
    (dict(qk_depth=128, ov_depth=128, nope_depth=64, rope_dtype=1), DA_EUNSUPPORTED),
    (dict(qk_depth=256, ov_depth=256, nope_depth=256, rope_dtype=1), DA_EINVAL),
    (dict(qk_depth=256, ov_depth=256, nope_depth=-1), DA_EINVAL),
    (dict(qk_depth=256, ov_depth=128), DA_EUNSUPPORTED),
    (dict(qk_depth=256, ov_depth=256, dtype=0), DA_EUNSUPPORTED),
    (dict(qk_depth=64, ov_depth=64), DA_OK),                        # heads of 64
    (dict(qk_depth=64, ov_depth=64, kv_dtype=2, q_len=2, page_size=24, max_pages_per_seq=200), DA_OK),
    (dict(qk_depth=64, ov_depth=64, dtype=0), DA_EUNSUPPORTED),     # fp32: the vector-ALU kernel is depth 128
    (dict(qk_depth=64, ov_depth=64, nope_depth=32, rope_dtype=1), DA_EUNSUPPORTED),
    (dict(qk_depth=64, ov_depth=128), DA_EUNSUPPORTED),
    (dict(qk_depth=256, ov_depth=256, page_size=16, max_pages_per_seq=256), DA_OK),
    (dict(qk_depth=256, ov_depth=256, page_size=24, max_pages_per_seq=200), DA_OK),   # per-key page lookup
    (dict(qk_depth=256, ov_depth=256, nope_depth=192, rope_dtype=1, page_size=24, max_pages_per_seq=200),
     DA_OK),
    (dict(qk_depth=192, ov_depth=128, kv_dtype=2, page_size=16, max_pages_per_seq=256), DA_OK),
    (dict(qk_depth=256, ov_depth=256, kernel=1), DA_EUNSUPPORTED),
    (dict(qk_depth=256, ov_depth=256, num_q_heads=34, num_kv_heads=2), DA_OK),   # group 17
])
def test_wide_depth_support(lib, kw, code):
    assert lib.da_supported(ctypes.byref(prob(**kw))) == code, lib.da_last_error()


def test_wide_depth_workspace_and_splits(lib):
    p = prob(batch=3, num_q_heads=8, num_kv_heads=8, qk_depth=256, ov_depth=256, nope_depth=192, rope_dtype=1,
             max_seq_len=1000, max_pages_per_seq=16)
    C, P = ctypes.c_int32(), ctypes.c_int32()
    assert lib.da_choose_splits(ctypes.byref(p), 0, 256, ctypes.byref(C), ctypes.byref(P)) == DA_OK
    assert C.value == 0 and P.value >= 1   # equal shares on the matrix-core kernel
    n = ctypes.c_size_t()
    assert lib.da_workspace_bytes(ctypes.byref(p), 4, ctypes.byref(n)) == DA_OK
    # fixed chunks: B * Hq * P (m, l) pairs and B * Hq * P * 256 fp32 partial outputs (+ counters)
    need = lambda x: -(-x // 256) * 256
    assert n.value == need(3 * 8 * 4 * 8) + need(3 * 8 * 4 * 256 * 4) + need(3 * 8 * 4)


def test_rotary_columns_apart_need_their_tensor(lib):
    from lse_combine_amd._lib import DaKv
    p = prob(qk_depth=256, ov_depth=256, nope_depth=192, rope_dtype=1)
    # the plain entry point has no place for them
    assert call_splitk(lib, p) == DA_EINVAL
    assert b"k_rope" in lib.da_last_error()
    kv = DaKv(0x1000, 0x1000, None, None, None)
    r = lib.decode_attn_splitk_kv(ctypes.byref(p), FAKE, ctypes.byref(kv), FAKE, FAKE, 0.1, 0, 0, FAKE, None, None,
                                  FAKE, 1 << 30, None)
    assert r == DA_EINVAL and b"k_rope" in lib.da_last_error()
    p0 = prob(qk_depth=256, ov_depth=256)
    kv = DaKv(0x1000, 0x1000, 0x1000, None, None)
    r = lib.decode_attn_splitk_kv(ctypes.byref(p0), FAKE, ctypes.byref(kv), FAKE, FAKE, 0.1, 0, 0, FAKE, None, None,
                                  FAKE, 1 << 30, None)
    assert r == DA_EINVAL
    assert lib.decode_attn_splitk_kv(ctypes.byref(p0), FAKE, None, FAKE, FAKE, 0.1, 0, 0, FAKE, None, None, FAKE,
                                     1 << 30, None) == DA_EINVAL
    # a V read as the first K columns takes the K scales: a V scale of its own is refused
    pl = prob(kv_dtype=2, num_q_heads=128, num_kv_heads=1, qk_depth=576, ov_depth=512, v_is_k_prefix=1,
              nope_depth=512, rope_dtype=1)
    kv = DaKv(0x1000, None, 0x1000, 0x1000, 0x1000)
    r = lib.decode_attn_partition_kv(ctypes.byref(pl), FAKE, ctypes.byref(kv), FAKE, FAKE, 0.1, 256, 16, FAKE, FAKE,
                                     None)
    assert r == DA_EINVAL and b"v_scale" in lib.da_last_error()
    # fp8 caches need their K scales here too
    p8 = prob(qk_depth=256, ov_depth=256, nope_depth=192, rope_dtype=1, kv_dtype=2)
    kv = DaKv(0x1000, 0x1000, 0x1000, None, None)
    r = lib.decode_attn_partition_kv(ctypes.byref(p8), FAKE, ctypes.byref(kv), FAKE, FAKE, 0.1, 256, 16, FAKE, FAKE,
                                     None)
    assert r == DA_EINVAL and b"k_scale" in lib.da_last_error()


def test_binding_fused_modes():
    from lse_combine_amd import api
    assert api._fused_mode(False) == 0 and api._fused_mode(True) == 1 and api._fused_mode("force") == 2
    with pytest.raises(ValueError):
        api._fused_mode("always")
