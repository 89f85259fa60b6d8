"""Build libqsa.so (HIP, gfx950 only) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("qsa_decode.hip", "qsa_store.hip", "qsa_index.hip", "qsa_api.hip")]
LIB = os.path.join(PKG, "libqsa.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-shared",
    "-Wall",
    # no packed-fp32 VALU forms anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # leading scalar kernel arguments (up to 10 dwords) preloaded into scalar
    # registers at wave launch; the code object keeps a prologue that loads
    # them itself where the dispatcher does not
    "-mllvm", "-amdgpu-kernarg-preload-count=10",
    "-I", os.path.join(ROOT, "include"),
]


# Host-side sanitizer build of the library's host code (contract checks,
# plan, workspace bookkeeping): AddressSanitizer and UndefinedBehavior-
# Sanitizer on the host compilation only; the device pass is unchanged.
SANITIZE_DIR = os.path.join(ROOT, "_build", "sanitize")
SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
]


def build_sanitize(verbose: bool = False) -> str:
    """Compile the host API (qsa_api.hip) with the host sanitizers into an
    object file that a driver links against; returns its path."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(SANITIZE_DIR, exist_ok=True)
    obj = os.path.join(SANITIZE_DIR, "qsa_api_host.o")
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++20", "-fPIC", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), *SANITIZE_FLAGS, "-c",
           os.path.join(CSRC, "qsa_api.hip"), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building the sanitizer object of qsa_api.hip")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Build libqsa.so; with sanitize=True build the host-sanitizer object
    of the host API instead (see build_sanitize)."""
    if sanitize:
        return build_sanitize(verbose)
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libqsa.so")
    # hipcc's host pass does not know the packed-fp32 feature; that warning
    # is expected, anything else is shown
    noise = [ln for ln in res.stderr.splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln and "warning generated" not in ln]
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, LIB)
    build_probe(verbose)
    build_stamps(verbose)
    return LIB


PROBE_LIB = os.path.join(PKG, "libqsa_probe.so")
STAMPS_LIB = os.path.join(PKG, "libqsa_stamps.so")


def build_stamps(verbose: bool = False) -> str:
    """Build the measurement build libqsa_stamps.so: the same sources with the
    decode kernel's per-workgroup phase stamps (include/qsa_stamps.h)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = STAMPS_LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-DQSA_PHASE_STAMPS", "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libqsa_stamps.so")
    os.replace(tmp, STAMPS_LIB)
    return STAMPS_LIB


def build_probe(verbose: bool = False) -> str:
    """Build the measurement helper libqsa_probe.so (the bare gather and the
    random line reads)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-o", tmp, os.path.join(CSRC, "qsa_probe.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libqsa_probe.so")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose=True))
