"""Build libpkv.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpkv.so")
SOURCES = [os.path.join(CSRC, "pkv_api.hip"), os.path.join(CSRC, "pkv_alloc.cpp")]
DEPS = SOURCES + [os.path.join(CSRC, "pkv_kernels.hpp"), os.path.join(CSRC, "pkv_prefill.hpp"),
                  os.path.join(CSRC, "pkv_q8.hpp"),
                  os.path.join(INCLUDE, "pkv.h")]
# Measurement aid used by bench.py only (streaming-read bandwidth probe).
PROBE_LIB = os.path.join(PKG, "libpkv_probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "probe_read.hip")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpkv.so)")


def command(out: str = LIB, extra=(), sources=None) -> list:
    return [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA accumulators in VGPRs: the softmax rescale touches them
            # with VALU ops, which AGPRs would need copies for.
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            # A fused-step ticket is one lane's atomic whose result is needed
            # only at the end; the wave-combining rewrite would wait for it
            # (and every load before it) right where it is issued.
            "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
            "-Wall", "-Wno-unused-function",
            "-I", INCLUDE, "-I", CSRC, *extra, *(sources or SOURCES), "-o", out]


def _compile(out: str, sources, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = command(tmp, sources=sources)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stderr or "").splitlines()
            if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every HIP source (libpkv.so and the bench probe library) next
    to this file, always."""
    _compile(PROBE_LIB, PROBE_SOURCES, verbose)
    return _compile(LIB, SOURCES, verbose)


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(d) > t for d in DEPS)


if __name__ == "__main__":
    print(build(verbose=True))
