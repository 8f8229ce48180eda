"""ctypes loaders for libdecode_attn.so (the C ABI declared in include/decode_attn.h) and
for the benchmark's probe library libda_probe.so (include/da_probe.h)."""

from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "lib", "libdecode_attn.so")
HEADER = os.path.join(ROOT, "include", "decode_attn.h")
PROBE_LIB_PATH = os.path.join(PKG, "lib", "libda_probe.so")
PROBE_HEADER = os.path.join(ROOT, "include", "da_probe.h")

DA_OK, DA_EINVAL, DA_EUNSUPPORTED, DA_EWORKSPACE, DA_EHIP = 0, -1, -2, -3, -4
DA_F32, DA_BF16, DA_FP8_E4M3 = 0, 1, 2
DA_KERNEL_AUTO, DA_KERNEL_FMA, DA_KERNEL_MFMA = 0, 1, 2


class DaProblem(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "batch", "num_q_heads", "num_kv_heads", "qk_depth", "ov_depth", "dtype", "page_size",
        "max_pages_per_seq", "num_pages", "kv_capacity", "max_seq_len", "v_is_k_prefix", "kernel", "kv_dtype", "q_len",
        "nope_depth", "rope_dtype")]


class DaKv(ctypes.Structure):
    """The cache tensors of one step (da_kv): device pointers, NULL where unused."""
    _fields_ = [(name, ctypes.c_void_p) for name in ("k_cache", "v_cache", "k_rope", "k_scale", "v_scale")]


class DaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"decode_attn error {code}: {msg}")
        self.code = code


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SIGS = {
    "da_supported": (ctypes.c_int, [ctypes.POINTER(DaProblem)]),
    "da_choose_splits": (ctypes.c_int, [ctypes.POINTER(DaProblem), _I32, _I32,
                                        ctypes.POINTER(_I32), ctypes.POINTER(_I32)]),
    "da_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(DaProblem), _I32, ctypes.POINTER(ctypes.c_size_t)]),
    "da_fused_applies": (ctypes.c_int, [ctypes.POINTER(DaProblem), _I32]),
    "decode_attn_splitk": (ctypes.c_int, [ctypes.POINTER(DaProblem), _P, _P, _P, _P, _P, ctypes.c_float, _I32,
                                          _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "decode_attn_splitk_noalloc": (ctypes.c_int, [ctypes.POINTER(DaProblem), _P, _P, _P, _P, _P, ctypes.c_float,
                                                  _I32, _P, _P, _P, _P]),
    "decode_attn_splitk_fused": (ctypes.c_int, [ctypes.POINTER(DaProblem), _P, _P, _P, _P, _P, ctypes.c_float,
                                                _I32, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "decode_attn_splitk_fp8": (ctypes.c_int, [ctypes.POINTER(DaProblem), _P, _P, _P, _P, _P, _P, _P,
                                              ctypes.c_float, _I32, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "decode_attn_partition_fp8": (ctypes.c_int, [ctypes.POINTER(DaProblem), _P, _P, _P, _P, _P, _P, _P,
                                                 ctypes.c_float, _I32, _I32, _P, _P, _P]),
    "decode_attn_splitk_kv": (ctypes.c_int, [ctypes.POINTER(DaProblem), _P, ctypes.POINTER(DaKv), _P, _P,
                                             ctypes.c_float, _I32, _I32, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "decode_attn_partition_kv": (ctypes.c_int, [ctypes.POINTER(DaProblem), _P, ctypes.POINTER(DaKv), _P, _P,
                                                ctypes.c_float, _I32, _I32, _P, _P, _P]),
    "decode_attn_partition": (ctypes.c_int, [ctypes.POINTER(DaProblem), _P, _P, _P, _P, _P, ctypes.c_float,
                                             _I32, _I32, _P, _P, _P]),
    "decode_attn_combine": (ctypes.c_int, [ctypes.POINTER(DaProblem), _P, ctypes.c_float, _I32, _I32, _P, _P,
                                           _P, _P, _P, _P]),
    "da_last_error": (ctypes.c_char_p, []),
    "da_version": (ctypes.c_char_p, []),
}

_PROBE_SIGS = {
    "da_read_probe": (ctypes.c_int, [_P, ctypes.c_size_t, _P, _P]),
    "da_copy_probe": (ctypes.c_int, [_P, _P, ctypes.c_size_t, _P]),
}

_lib = None
_probe = None


def load():
    """Load the built library; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def load_probe():
    """Load the measurement-probe library (benchmark only)."""
    global _probe
    if _probe is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError(f"{PROBE_LIB_PATH} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(PROBE_LIB_PATH)
        for name, (res, args) in _PROBE_SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _probe = lib
    return _probe


def check(code):
    if code != DA_OK:
        raise DaError(code, load().da_last_error().decode())
    return code


def header_functions(header=HEADER):
    """Names of the functions a header (default include/decode_attn.h) declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(da_\w+|decode_attn_\w+)\s*\(", text, flags=re.M)))
