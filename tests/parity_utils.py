"""Helpers for parity tests: run the oracle on a Case and compare with the GPU outputs.

Tolerances (derived from the arithmetic; the fp32 partials and the bf16 cast):
  out (bf16)   |gpu - O| <= 1e-2 + 1e-2 |O| elementwise
  o32 (fp32)   max_d |gpu - O| <= 1e-5 max_d |O| per row
  lse (fp32)   |gpu - LSE| <= 1e-5 max(|LSE|, 1): relative, read as relative to the softmax
               normaliser Z = exp(LSE) where |LSE| < 1 (1e-5 on Z is 1e-5 on LSE; a relative
               bound on a log that cancels to near 0 would ask more than fp32 can hold)
"""

import numpy as np
import torch

from oracle import decode_attention_fp64

OUT_ATOL, OUT_RTOL = 1e-2, 1e-2
O32_ROW_RTOL = 1e-5
LSE_RTOL = 1e-5


def np32(t):
    """fp32 numpy copy of a tensor; fp8 caches (uint8 codes) stay raw codes."""
    if t is None:
        return None
    t = t.detach().cpu()
    return t.numpy() if t.dtype == torch.uint8 else t.float().numpy()


def oracle_for(case, batch_rows=None):
    """fp64 oracle (O, LSE) for all sequences or the listed batch rows."""
    q = np32(case.q)
    k = np32(case.k_cache)
    v = None if case.v_cache is None else np32(case.v_cache)
    lens = case.seq_lens.cpu().numpy().astype(np.int64)
    pt = None if case.page_table is None else case.page_table.cpu().numpy()
    ks = None if case.k_scale is None else case.k_scale.cpu().numpy()
    vs = None if case.v_scale is None else case.v_scale.cpu().numpy()
    kr = np32(case.k_rope)
    if batch_rows is not None:
        q = q[batch_rows]
        lens = lens[batch_rows]
        if pt is not None:
            pt = pt[batch_rows]
        else:
            k = k[batch_rows]
            v = None if v is None else v[batch_rows]
            ks = None if ks is None else ks[batch_rows]
            vs = None if vs is None else vs[batch_rows]
            kr = None if kr is None else kr[batch_rows]
    lens = np.maximum(lens, 0)
    return decode_attention_fp64(q, k, v, lens, case.scale, page_table=pt, page_size=case.page_size,
                                 v_is_k_prefix=case.v_is_k_prefix, ov_depth=case.ov_depth, k_scale=ks,
                                 v_scale=vs, k_rope=kr)


def assert_parity(out, lse, o32, O, LSE, o32_row_rtol=O32_ROW_RTOL, lse_rtol=LSE_RTOL, what=""):
    out = np32(out).astype(np.float64)
    err = np.abs(out - O)
    bound = OUT_ATOL + OUT_RTOL * np.abs(O)
    assert np.all(err <= bound), f"{what} bf16 out: max excess {(err - bound).max():.3e}"
    if o32 is not None:
        o = np32(o32).astype(np.float64)
        row_err = np.abs(o - O).max(axis=-1)
        row_ref = np.abs(O).max(axis=-1)
        live = row_ref > 0
        rel = row_err[live] / row_ref[live]
        assert np.all(row_err[~live] == 0), f"{what} o32: nonzero output for an empty row"
        assert rel.size == 0 or rel.max() <= o32_row_rtol, f"{what} o32 row-relative error {rel.max():.3e}"
    if lse is not None:
        l = np32(lse).astype(np.float64)
        fin = np.isfinite(LSE)
        assert np.array_equal(np.isneginf(l), np.isneginf(LSE)), f"{what} lse: -inf rows differ"
        rel = np.abs(l[fin] - LSE[fin]) / np.maximum(np.abs(LSE[fin]), 1.0)
        assert rel.size == 0 or rel.max() <= lse_rtol, f"{what} lse relative error {rel.max():.3e}"
