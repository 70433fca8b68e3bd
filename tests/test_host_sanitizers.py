"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the engine tests (block manager, prefix cache, copy-on-write,
continuous batching, randomised workloads) and the C-ABI argument tests run in
a subprocess against libpkv built with those sanitizers on its host pass, the
sanitizer runtime preloaded.  Any report fails the test."""
import os
import pathlib
import subprocess
import sys

from paged_kv_cache_attention_amd import build

ROOT = pathlib.Path(__file__).resolve().parent.parent

DRIVER = """
import pathlib, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import paged_kv_cache_attention_amd as pkv
pkv.load_library(pathlib.Path({lib!r}))
import pytest
# -s: a sanitizer report goes straight to the process's stderr, not to a
# captured buffer that an aborting process never prints
sys.exit(pytest.main(["-q", "-s", "-x", "-p", "no:cacheprovider", "-m", "not gpu", {tests!r} + "/test_engine_cpu.py",
                      {tests!r} + "/test_abi_cpu.py", "-k", "not binding_checks_attention_arguments"]))
"""


def test_engine_and_abi_checks_under_asan_and_ubsan():
    lib = build.build_sanitized()
    env = dict(os.environ,
               LD_PRELOAD=str(build.sanitizer_runtime()),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = DRIVER.format(root=str(ROOT), tests=str(ROOT / "tests"), lib=str(lib))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=900)
    report = r.stdout[-3000:] + r.stderr[-6000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
    assert r.returncode == 0, report
    assert " passed" in r.stdout, report
