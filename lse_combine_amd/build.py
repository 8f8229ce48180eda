"""Build the HIP libraries (gfx950) in-tree: lse_combine_amd/lib/libdecode_attn.so (the
decode-attention library) and lse_combine_amd/lib/libda_probe.so (the benchmark's
measurement probes, a library of its own)."""

from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libdecode_attn.so")
PROBE_LIB = os.path.join(LIBDIR, "libda_probe.so")
PROBE_SRC = os.path.join(CSRC, "probe", "probe.hip")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU ops are disabled on purpose: the compiler may otherwise form
# v_pk_{add,mul,fma}_f32 from plain float code. -fno-honor-nans lets fmaxf lower to a
# single v_max (the kernels never produce NaN from finite inputs; -inf is used and kept).
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no NaN inputs are assumed (max/min need no canonicalisation); infinities stay honoured
    "-fno-honor-nans",
    "-Wall", "-Wno-unused-function", "-Wno-unused-result",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every HIP source for gfx950 and link both shared libraries. Always rebuilds."""
    os.makedirs(LIBDIR, exist_ok=True)
    objdir = os.path.join(ROOT, "_build", "obj")
    os.makedirs(objdir, exist_ok=True)
    srcs = sources() + [PROBE_SRC]
    procs = []
    objs = []
    for src in srcs:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _drain(procs)
    _drain(procs)
    _link(objs[:-1], LIB, verbose)
    _link(objs[-1:], PROBE_LIB, verbose)
    return LIB


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if out.returncode != 0:
        raise RuntimeError("link failed:\n" + out.stdout)
    os.replace(tmp, lib)


def _drain(procs):
    while procs:
        src, p = procs.pop(0)
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{text}")
        errs = [ln for ln in text.splitlines() if "error" in ln.lower()]
        if errs:
            print(text, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
