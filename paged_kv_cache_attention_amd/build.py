"""Compile libpkv.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m paged_kv_cache_attention_amd.build

hipcc cross-compiles without a GPU.  Packed-FP32 VALU instructions are
disabled for the device code (``-packed-fp32-ops``); hipcc's host pass warns
that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import pathlib
import shutil
import subprocess
import sys

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB = PKG / "libpkv.so"
PROBE_LIB = PKG / "libpkv_probe.so"      # diagnostic read-bandwidth probe, not part of the pkv ABI
SOURCES = ["pkv_api.hip", "pkv_decode.hip", "pkv_stream.hip", "pkv_verify.hip", "pkv_prefill.hip", "pkv_prefix.hip", "pkv_reduce.hip", "pkv_copy.hip", "pkv_rope.hip", "pkv_engine.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; ROCm is required to build libpkv")


def command(out: pathlib.Path = LIB, extra=()) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            f"-I{INCLUDE}", f"-I{CSRC}", *extra, "-o", str(out), *[str(CSRC / s) for s in SOURCES]]


def _compile(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> pathlib.Path:
    """Always recompiles; writes libpkv.so (and the probe library) next to this file atomically."""
    ptmp = PROBE_LIB.with_suffix(".so.tmp")
    _compile([hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
              "-o", str(ptmp), str(CSRC / "probe_read.hip")], verbose)
    os.replace(ptmp, PROBE_LIB)
    tmp = LIB.with_suffix(".so.tmp")
    cmd = command(tmp)
    _compile(cmd, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
