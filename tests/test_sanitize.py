"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code and of the oracle (CPU only).

Two programs are built with the host compilers (g++, gcc) and -fsanitize=address,undefined, and run:

* tests/sanitize/host_driver.cpp with the library's host sources (api.cpp: every C-ABI entry point's
  argument checks, split choice and workspace layout; codebook.cpp: Lloyd-Max, k-means, the encode's cell
  grid).  The kernel launchers and the handful of HIP runtime calls are stand-ins, so nothing reaches a
  GPU; the stand-ins also check each recorded launch against the read kernels' launch invariants.
* tests/sanitize/oracle_driver.c with oracle/kvq_oracle.c: every oracle function on small inputs.

A sanitizer report aborts the program, and any failed expectation makes it exit nonzero.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")


def _run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)


def _build_and_run(tmp_path, compiler, sources, flags, name):
    if shutil.which(compiler) is None:
        pytest.skip("%s not installed" % compiler)
    exe = str(tmp_path / name)
    b = _run([compiler] + flags + SAN + sources + ["-o", exe] + (["-lm"] if compiler == "gcc" else []))
    assert b.returncode == 0, b.stderr[-4000:]
    # verify_asan_link_order=0: the environment may preload a library ahead of the sanitizer runtime
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([exe], env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert out.strip().splitlines()[-1].startswith("OK"), out[-2000:]


def test_host_code_under_sanitizers(tmp_path):
    if not os.path.isfile(os.path.join(ROCM_INCLUDE, "hip", "hip_runtime_api.h")):
        pytest.skip("HIP headers not found")
    csrc = os.path.join(ROOT, "quantized_kv_cache_encode_amd", "csrc")
    flags = ["-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I" + ROCM_INCLUDE, "-I" + os.path.join(ROOT, "include"),
             "-I" + csrc]
    sources = [os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"), os.path.join(csrc, "api.cpp"),
               os.path.join(csrc, "codebook.cpp")]
    _build_and_run(tmp_path, "g++", sources, flags, "host_driver")


def test_oracle_under_sanitizers(tmp_path):
    sources = [os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), os.path.join(ROOT, "oracle", "kvq_oracle.c")]
    _build_and_run(tmp_path, "gcc", sources, ["-std=c11"], "oracle_driver")
