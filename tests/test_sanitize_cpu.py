"""Host-side AddressSanitizer / UndefinedBehaviorSanitizer runs (CPU only).

* The oracle's C code, built with both sanitizers (``oracle.build(sanitize=
  True)``), driven through every entry point by tests/native/oracle_check.c.
* The host code of the library (contract checks, split plan, options,
  workspace bookkeeping, thread-local error strings), built with both
  sanitizers on the host pass (``build.build(sanitize=True)``), driven by
  tests/native/abi_host_check.hip with the kernel launches stubbed out.

Either process exits non-zero on a sanitizer report or a failed
expectation.
"""
import os
import shutil
import subprocess

import pytest

import oracle
from sparse_index_paged_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ENV = dict(os.environ, UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
           ASAN_OPTIONS="abort_on_error=0:halt_on_error=1")


def _run(cmd, env=ENV, timeout=300):
    res = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


def test_oracle_under_asan_ubsan():
    obj = oracle.build(sanitize=True)
    exe = os.path.join(os.path.dirname(obj), "oracle_check")
    _run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-fopenmp", "-std=c11",
          os.path.join(NATIVE, "oracle_check.c"), obj, "-lm", "-o", exe])
    res = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1"))
    assert "oracle_check: ok" in res.stdout


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc missing")
def test_host_api_under_asan_ubsan():
    obj = hip_build.build(sanitize=True)
    out_dir = os.path.dirname(obj)
    drv = os.path.join(out_dir, "abi_host_check.o")
    exe = os.path.join(out_dir, "abi_host_check")
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++20", "-I", os.path.join(ROOT, "include"),
              *hip_build.SANITIZE_FLAGS]
    _run([HIPCC, *common, "-c", os.path.join(NATIVE, "abi_host_check.hip"), "-o", drv])
    _run([HIPCC, "--offload-arch=gfx950", *hip_build.SANITIZE_FLAGS, drv, obj, "-o", exe])
    # the HIP runtime's own allocations outlive main: leak checking is off
    res = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1"))
    assert "abi_host_check: ok" in res.stdout
