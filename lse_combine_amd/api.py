"""Thin PyTorch binding of the C ABI: argument marshalling only.

Every step of the decode step runs in the HIP library; this module checks
tensor shapes/devices, passes ``data_ptr()`` values and the current HIP
stream, and allocates outputs and the workspace with PyTorch.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import DaProblem, check

_DTYPES = {torch.float32: _lib.DA_F32, torch.bfloat16: _lib.DA_BF16}
_KERNELS = {"auto": _lib.DA_KERNEL_AUTO, "fma": _lib.DA_KERNEL_FMA, "mfma": _lib.DA_KERNEL_MFMA}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _kv(k_cache, v_cache, k_rope=None, k_scale=None, v_scale=None):
    """da_kv of the cache tensors (the tensors must outlive its use)."""
    def addr(t):
        return None if t is None else t.data_ptr()
    return _lib.DaKv(addr(k_cache), addr(v_cache), addr(k_rope), addr(k_scale), addr(v_scale))


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_problem(q, k_cache, v_cache=None, page_table=None, *, page_size=0, max_seq_len=None,
                 v_is_k_prefix=False, ov_depth=None, kernel="auto", num_pages=None, k_rope=None) -> DaProblem:
    """Describe one decode step from its tensors (shapes as in include/decode_attn.h).

    q is [B, Hq, Dqk], or [B, q_len, Hq, Dqk] for several queries per sequence.
    k_rope (bf16, k_cache's layout) holds the last Dqk - nope rotary columns of every K row
    when they are stored apart; k_cache then holds the first nope columns.
    """
    if q.dim() not in (3, 4) or k_cache.dim() != 4:
        raise ValueError("q must be [B, Hq, Dqk] or [B, q_len, Hq, Dqk] and k_cache 4-D")
    q_len = q.shape[1] if q.dim() == 4 else 1
    if q.dim() == 4:
        q = q[:, 0]
    fp8 = k_cache.dtype == torch.uint8   # E4M3 codes
    if q.dtype not in _DTYPES:
        raise ValueError("q must be float32 or bfloat16")
    if not fp8 and (k_cache.dtype != q.dtype or (v_cache is not None and v_cache.dtype != q.dtype)):
        raise ValueError("q, k_cache and v_cache must share dtype float32 or bfloat16 (or uint8 fp8 caches)")
    if fp8 and v_cache is not None and v_cache.dtype != torch.uint8:
        raise ValueError("an fp8 k_cache needs an fp8 (uint8) v_cache")
    B, Hq, Dqk = q.shape
    Hkv = k_cache.shape[2]
    nope = 0
    if k_rope is not None:
        if k_rope.dtype != torch.bfloat16 or tuple(k_rope.shape[:3]) != tuple(k_cache.shape[:3]):
            raise ValueError("k_rope must be bfloat16 and match k_cache in its first three dimensions")
        nope = k_cache.shape[3]
        if nope + k_rope.shape[3] != Dqk:
            raise ValueError("k_cache depth + k_rope depth must equal q depth")
    elif k_cache.shape[3] != Dqk:
        raise ValueError("k_cache depth must equal q depth")
    if v_is_k_prefix:
        Dv = int(ov_depth if ov_depth is not None else Dqk)
    else:
        if v_cache is None:
            raise ValueError("v_cache is required unless v_is_k_prefix")
        Dv = v_cache.shape[3]
        if tuple(v_cache.shape[:3]) != tuple(k_cache.shape[:3]):
            raise ValueError("v_cache must match k_cache in its first three dimensions")
    p = DaProblem()
    p.batch, p.num_q_heads, p.num_kv_heads, p.qk_depth, p.ov_depth = B, Hq, Hkv, Dqk, Dv
    p.dtype = _DTYPES[q.dtype]
    p.kv_dtype = _lib.DA_FP8_E4M3 if fp8 else 0
    p.q_len = q_len
    p.nope_depth = nope
    p.rope_dtype = _lib.DA_BF16 if nope else 0
    p.kernel = _KERNELS[kernel]
    p.v_is_k_prefix = 1 if v_is_k_prefix else 0
    if page_table is not None:
        if page_size <= 0 or k_cache.shape[1] != page_size:
            raise ValueError("paged cache: page_size must be > 0 and equal k_cache.shape[1]")
        p.page_size = page_size
        p.max_pages_per_seq = page_table.shape[1]
        p.num_pages = k_cache.shape[0] if num_pages is None else num_pages
        cap = page_table.shape[1] * page_size
    else:
        p.page_size = 0
        if k_cache.shape[0] != B:
            raise ValueError("contiguous cache must be [B, L_cap, Hkv, Dqk]")
        p.kv_capacity = k_cache.shape[1]
        cap = k_cache.shape[1]
    p.max_seq_len = cap if max_seq_len is None else int(max_seq_len)
    return p


def row_shape(problem: DaProblem):
    """Leading shape of out / lse: (B, Hq), or (B, q_len, Hq) with several queries."""
    if problem.q_len > 1:
        return (problem.batch, problem.q_len, problem.num_q_heads)
    return (problem.batch, problem.num_q_heads)


def check_outputs(problem: DaProblem, out=None, lse=None, o32=None):
    """Refuse output buffers that do not hold every (query, head) row: the library writes
    through raw pointers and cannot see their sizes."""
    rows = row_shape(problem)
    n = 1
    for d in rows:
        n *= d
    for t, per_row, dtype, name in ((out, problem.ov_depth, torch.bfloat16, "out"), (lse, 1, torch.float32, "lse"),
                                    (o32, problem.ov_depth, torch.float32, "o32")):
        if t is None:
            continue
        if t.dtype != dtype or t.numel() != n * per_row or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape "
                             f"{rows + ((per_row,) if per_row > 1 else ())}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")


def _check_tensors(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


def choose_splits(problem: DaProblem, num_splits=0, num_cus=0):
    lib = _lib.load()
    C, P = ctypes.c_int32(), ctypes.c_int32()
    check(lib.da_choose_splits(ctypes.byref(problem), num_splits, num_cus, ctypes.byref(C), ctypes.byref(P)))
    return C.value, P.value


def workspace_bytes(problem: DaProblem, num_splits=0):
    lib = _lib.load()
    n = ctypes.c_size_t()
    check(lib.da_workspace_bytes(ctypes.byref(problem), num_splits, ctypes.byref(n)))
    return n.value


def _fused_mode(fused):
    """fused=False: combine launch; True: fold in pass 1 where it pays; "force": always."""
    if fused == "force":
        return 2
    if fused in (False, True, 0, 1):
        return int(bool(fused))
    raise ValueError(f"fused must be False, True or 'force' (got {fused!r})")


def fused_applies(problem: DaProblem, num_splits=0):
    """True if the fused entry point merges the partials in pass 1 for this problem (else it
    runs the combine launch, with the same results)."""
    lib = _lib.load()
    r = lib.da_fused_applies(ctypes.byref(problem), num_splits)
    if r < 0:
        check(r)
    return r == 1


def decode_attn(q, k_cache, v_cache, page_table, seq_lens, scale, num_splits=0, *, page_size=0,
                max_seq_len=None, v_is_k_prefix=False, ov_depth=None, out=None, lse=None, o32=None,
                return_lse=False, return_o32=False, workspace=None, kernel="auto", fused=False,
                k_scale=None, v_scale=None, k_rope=None):
    """The whole split-K decode step. Returns out (bf16 [B, Hq, Dv]) or (out, lse, o32).

    fused=True runs decode_attn_splitk_fused (the combine done by each group's last
    workgroup where that pays, see ``fused_applies``), fused="force" always does it in pass 1;
    a workspace passed in must then have been zero-filled before its first use.
    fp8 caches take k_scale / v_scale; rotary columns stored apart take k_rope (both run
    through the entry points that accept those tensors).
    """
    lib = _lib.load()
    mode = _fused_mode(fused)
    prob = make_problem(q, k_cache, v_cache, page_table, page_size=page_size, max_seq_len=max_seq_len,
                        v_is_k_prefix=v_is_k_prefix, ov_depth=ov_depth, kernel=kernel, k_rope=k_rope)
    _check_tensors(q, k_cache, v_cache, page_table, seq_lens)
    rows = row_shape(prob)
    Dv = prob.ov_depth
    if out is None:
        out = torch.empty(rows + (Dv,), dtype=torch.bfloat16, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty(rows, dtype=torch.float32, device=q.device)
    if return_o32 and o32 is None:
        o32 = torch.empty(rows + (Dv,), dtype=torch.float32, device=q.device)
    check_outputs(prob, out, lse, o32)
    need = workspace_bytes(prob, num_splits)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=q.device)
    ws = (_ptr(workspace), workspace.numel() * workspace.element_size(), _stream())
    if k_rope is not None or (prob.kv_dtype and mode) or mode == 2:
        _check_tensors(k_rope, k_scale, v_scale)
        kv = _kv(k_cache, v_cache, k_rope, k_scale, v_scale)
        check(lib.decode_attn_splitk_kv(ctypes.byref(prob), _ptr(q), ctypes.byref(kv), _ptr(page_table),
                                        _ptr(seq_lens), float(scale), int(num_splits), mode, _ptr(out),
                                        _ptr(lse), _ptr(o32), *ws))
    elif prob.kv_dtype:
        _check_tensors(k_scale, v_scale)
        check(lib.decode_attn_splitk_fp8(ctypes.byref(prob), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                         _ptr(v_scale), _ptr(page_table), _ptr(seq_lens), float(scale),
                                         int(num_splits), _ptr(out), _ptr(lse), _ptr(o32), *ws))
    else:
        fn = lib.decode_attn_splitk_fused if mode else lib.decode_attn_splitk
        check(fn(ctypes.byref(prob), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), _ptr(seq_lens),
                 float(scale), int(num_splits), _ptr(out), _ptr(lse), _ptr(o32), *ws))
    if return_lse or return_o32:
        return out, lse, o32
    return out


def alloc_partials(problem: DaProblem, chunk_tokens, max_splits, device):
    """Buffers for pass 1 / pass 2 of the split API.

    Fixed chunks (chunk_tokens > 0): part_o [B, Hq, max_splits, Dv] and part_ml
    [B, Hq, max_splits, 2]. Equal-share schedule (chunk_tokens == 0, max_splits =
    workers): part_o [slots, Hq, Dv] with slots = max_splits + B, and part_ml a flat
    fp32 buffer of slots * Hq (m, l) pairs followed by the int32 (first slot, count)
    pair of each sequence (see ``slot_table``).
    """
    B, Dv = problem.batch, problem.ov_depth
    Hq = problem.num_q_heads * max(1, problem.q_len)   # rows per sequence
    f32 = dict(dtype=torch.float32, device=device)
    if chunk_tokens == 0:
        slots = max_splits + B
        return torch.zeros((slots, Hq, Dv), **f32), torch.zeros(slots * Hq * 2 + 2 * B, **f32)
    return torch.zeros((B, Hq, max_splits, Dv), **f32), torch.zeros((B, Hq, max_splits, 2), **f32)


def slot_table(problem: DaProblem, max_splits, part_ml):
    """Equal-share schedule: split part_ml into (ml [slots, Hq, 2] fp32, table [B, 2] int32)."""
    B, Hq = problem.batch, problem.num_q_heads * max(1, problem.q_len)
    slots = max_splits + B
    ml = part_ml[:slots * Hq * 2].view(slots, Hq, 2)
    table = part_ml[slots * Hq * 2:slots * Hq * 2 + 2 * B].view(torch.int32).view(B, 2)
    return ml, table


def partition(q, k_cache, v_cache, page_table, seq_lens, scale, chunk_tokens, max_splits, *, page_size=0,
              max_seq_len=None, v_is_k_prefix=False, ov_depth=None, part_o=None, part_ml=None, kernel="auto",
              k_scale=None, v_scale=None, k_rope=None):
    """Pass 1 only. Returns (part_o, part_ml) fp32 in the layout ``alloc_partials`` describes."""
    lib = _lib.load()
    prob = make_problem(q, k_cache, v_cache, page_table, page_size=page_size, max_seq_len=max_seq_len,
                        v_is_k_prefix=v_is_k_prefix, ov_depth=ov_depth, kernel=kernel, k_rope=k_rope)
    _check_tensors(q, k_cache, v_cache, page_table, seq_lens)
    if part_o is None or part_ml is None:
        po, pml = alloc_partials(prob, chunk_tokens, max_splits, q.device)
        part_o = po if part_o is None else part_o
        part_ml = pml if part_ml is None else part_ml
    if k_rope is not None:
        _check_tensors(k_rope, k_scale, v_scale)
        kv = _kv(k_cache, v_cache, k_rope, k_scale, v_scale)
        check(lib.decode_attn_partition_kv(ctypes.byref(prob), _ptr(q), ctypes.byref(kv), _ptr(page_table),
                                           _ptr(seq_lens), float(scale), int(chunk_tokens), int(max_splits),
                                           _ptr(part_o), _ptr(part_ml), _stream()))
    elif prob.kv_dtype:
        check(lib.decode_attn_partition_fp8(ctypes.byref(prob), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                            _ptr(k_scale), _ptr(v_scale), _ptr(page_table), _ptr(seq_lens),
                                            float(scale), int(chunk_tokens), int(max_splits), _ptr(part_o),
                                            _ptr(part_ml), _stream()))
    else:
        check(lib.decode_attn_partition(ctypes.byref(prob), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(page_table), _ptr(seq_lens), float(scale), int(chunk_tokens),
                                        int(max_splits), _ptr(part_o), _ptr(part_ml), _stream()))
    return part_o, part_ml


def combine(problem: DaProblem, seq_lens, scale, chunk_tokens, max_splits, part_o, part_ml, *, out=None,
            lse=None, o32=None):
    """Pass 2 only (the LSE combine). Returns (out bf16, lse fp32, o32 fp32)."""
    lib = _lib.load()
    _check_tensors(seq_lens, part_o, part_ml)
    rows, Dv = row_shape(problem), problem.ov_depth
    dev = part_o.device
    out = torch.empty(rows + (Dv,), dtype=torch.bfloat16, device=dev) if out is None else out
    lse = torch.empty(rows, dtype=torch.float32, device=dev) if lse is None else lse
    o32 = torch.empty(rows + (Dv,), dtype=torch.float32, device=dev) if o32 is None else o32
    check_outputs(problem, out, lse, o32)
    check(lib.decode_attn_combine(ctypes.byref(problem), _ptr(seq_lens), float(scale), int(chunk_tokens),
                                  int(max_splits), _ptr(part_o), _ptr(part_ml), _ptr(out), _ptr(lse), _ptr(o32),
                                  _stream()))
    return out, lse, o32


def case_call(case, device="cuda", **kw):
    """Run a lse_combine_amd.inputs.Case already moved to ``device`` (see ``to_device``)."""
    return decode_attn(case.q, case.k_cache, case.v_cache, case.page_table, case.seq_lens, case.scale,
                       case.num_splits, page_size=case.page_size, v_is_k_prefix=case.v_is_k_prefix,
                       ov_depth=case.ov_depth, k_scale=case.k_scale, v_scale=case.v_scale, k_rope=case.k_rope,
                       **kw)


class DecodePlan:
    """Pre-marshalled arguments for repeated decode steps on fixed buffers.

    Holds the problem description, the device pointers and a workspace so that
    ``run()`` is a single C call (useful when the host must keep up with short
    steps, and under graph capture: the call allocates nothing).
    """

    def __init__(self, q, k_cache, v_cache, page_table, seq_lens, scale, num_splits=0, *, page_size=0,
                 max_seq_len=None, v_is_k_prefix=False, ov_depth=None, kernel="auto", out=None, lse=None,
                 o32=None, fused=False, k_scale=None, v_scale=None, k_rope=None):
        self.lib = _lib.load()
        self.prob = make_problem(q, k_cache, v_cache, page_table, page_size=page_size, max_seq_len=max_seq_len,
                                 v_is_k_prefix=v_is_k_prefix, ov_depth=ov_depth, kernel=kernel, k_rope=k_rope)
        _check_tensors(q, k_cache, v_cache, page_table, seq_lens)
        self.out = (torch.empty(row_shape(self.prob) + (self.prob.ov_depth,), dtype=torch.bfloat16, device=q.device)
                    if out is None else out)
        check_outputs(self.prob, self.out, lse, o32)
        self.lse, self.o32 = lse, o32
        need = workspace_bytes(self.prob, num_splits)
        # zero-filled once: the fused step keeps its arrival counters here
        self.workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=q.device)
        mode = _fused_mode(fused)
        self.fn = self.lib.decode_attn_splitk_fused if mode else self.lib.decode_attn_splitk
        self.chunk, self.max_splits = choose_splits(self.prob, num_splits)
        self._keep = (q, k_cache, v_cache, page_table, seq_lens, k_scale, v_scale, k_rope)
        if k_rope is not None or (self.prob.kv_dtype and mode) or mode == 2:
            self.fn = self.lib.decode_attn_splitk_kv
            self.kv = _kv(k_cache, v_cache, k_rope, k_scale, v_scale)
            self._args = (ctypes.byref(self.prob), _ptr(q), ctypes.byref(self.kv), _ptr(page_table), _ptr(seq_lens),
                          float(scale), int(num_splits), mode, _ptr(self.out), _ptr(lse), _ptr(o32),
                          _ptr(self.workspace), self.workspace.numel())
        elif self.prob.kv_dtype:
            self.fn = self.lib.decode_attn_splitk_fp8
            self._args = (ctypes.byref(self.prob), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                          _ptr(v_scale), _ptr(page_table), _ptr(seq_lens), float(scale), int(num_splits),
                          _ptr(self.out), _ptr(lse), _ptr(o32), _ptr(self.workspace), self.workspace.numel())
        else:
            self._args = (ctypes.byref(self.prob), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
                          _ptr(seq_lens), float(scale), int(num_splits), _ptr(self.out), _ptr(lse), _ptr(o32),
                          _ptr(self.workspace), self.workspace.numel())

    def run(self, stream=None):
        s = _stream() if stream is None else ctypes.c_void_p(stream)
        check(self.fn(*self._args, s))
        return self.out
