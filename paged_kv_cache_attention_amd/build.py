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
SOURCES = ["pkv_api.hip", "pkv_decode.hip", "pkv_stream.hip", "pkv_verify.hip", "pkv_prefill.hip", "pkv_devattr.hip", "pkv_reduce.hip", "pkv_copy.hip", "pkv_rope.hip", "pkv_engine.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; ROCm is required to build libpkv")


OBJ_DIR = ROOT / "_build"
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def command(out: pathlib.Path = LIB, extra=()) -> list:
    """One hipcc line that compiles and links every source (what build() runs, file by file)."""
    return [hipcc(), *FLAGS, "-shared", f"-I{INCLUDE}", f"-I{CSRC}", *extra, "-o", str(out),
            *[str(CSRC / s) for s in SOURCES]]


def object_command(src: str, extra=()) -> list:
    return [hipcc(), *FLAGS, "-c", f"-I{INCLUDE}", f"-I{CSRC}", *extra, "-o", str(OBJ_DIR / (src + ".o")),
            str(CSRC / src)]


BUILD_INFO = PKG / "build_info.json"   # commit and source hash of the last build (not tracked)


def sources_sha256() -> str:
    """Hash of every kernel/host source and the public headers."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(CSRC.iterdir()):
        if f.is_file():
            h.update(f.read_bytes())
    for f in ("pkv.h", "pkv_engine.h"):
        h.update((INCLUDE / f).read_bytes())
    return h.hexdigest()


def _write_build_info():
    import json
    commit = None
    try:
        head = subprocess.run(["git", "-C", str(ROOT), "rev-parse", "HEAD"], capture_output=True, text=True)
        if head.returncode == 0:
            dirty = subprocess.run(["git", "-C", str(ROOT), "status", "--porcelain", "--", "paged_kv_cache_attention_amd",
                                    "include"], capture_output=True, text=True).stdout.strip()
            commit = head.stdout.strip() + ("-dirty" if dirty else "")
    except OSError:
        pass
    version = None
    try:
        out = subprocess.run([hipcc(), "--version"], capture_output=True, text=True, timeout=60).stdout
        version = next((l.strip() for l in out.splitlines() if "version" in l.lower()), None)
    except (OSError, subprocess.SubprocessError):
        pass
    BUILD_INFO.write_text(json.dumps({"commit": commit, "sources_sha256": sources_sha256(), "hipcc": version}) + "\n")


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
    # each source compiles to its own object (its kernels and their host
    # launchers live in one file), in parallel; then one link
    OBJ_DIR.mkdir(exist_ok=True)
    from concurrent.futures import ThreadPoolExecutor
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda src: _compile(object_command(src), verbose), SOURCES))
    tmp = LIB.with_suffix(".so.tmp")
    _compile([hipcc(), *FLAGS, "-shared", "-o", str(tmp), *[str(OBJ_DIR / (src + ".o")) for src in SOURCES]], verbose)
    os.replace(tmp, LIB)
    _write_build_info()
    return LIB


SANITIZED_LIB = OBJ_DIR / "libpkv_host_sanitized.so"
# Host code only: device code is built as usual; each -fsanitize= applies to
# the host pass through -Xarch_host.
SANITIZE_FLAGS = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def sanitizer_runtime() -> pathlib.Path:
    """The ASan runtime of ROCm's clang (it carries the UBSan handlers too);
    a process loading the sanitized library preloads it."""
    rts = sorted(pathlib.Path("/opt/rocm/llvm/lib/clang").glob("*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rts:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/llvm/lib/clang")
    return rts[-1]


def build_sanitized(verbose: bool = False) -> pathlib.Path:
    """libpkv with the host code (engine, argument checks, launchers) built
    with AddressSanitizer and UndefinedBehaviorSanitizer, for the CPU tests."""
    OBJ_DIR.mkdir(exist_ok=True)
    from concurrent.futures import ThreadPoolExecutor

    def obj(src):
        return OBJ_DIR / (src + ".san.o")
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda src: _compile([hipcc(), *FLAGS, *SANITIZE_FLAGS, "-c", f"-I{INCLUDE}", f"-I{CSRC}", "-o",
                                          str(obj(src)), str(CSRC / src)], verbose), SOURCES))
    tmp = SANITIZED_LIB.with_suffix(".so.tmp")
    _compile([hipcc(), *FLAGS, *SANITIZE_FLAGS, "-shared", "-o", str(tmp), *[str(obj(src)) for src in SOURCES]],
             verbose)
    os.replace(tmp, SANITIZED_LIB)
    return SANITIZED_LIB


if __name__ == "__main__":
    print(build(verbose=True))
