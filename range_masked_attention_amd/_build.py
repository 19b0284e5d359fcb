"""Build the HIP library in-tree with hipcc for gfx950.

``python -m range_masked_attention_amd._build`` compiles every source under
``csrc/`` and links ``_lib/libffa.so``.  Objects go to ``_build/`` at the repo
root.  ``build_planner_sanitized`` builds the host planner into a standalone
sanitizer-instrumented test driver (CPU only, plain g++).
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libffa.so")
PROBE_SRC = os.path.join(ROOT, "tests", "native", "mfma_rate.hip")
PROBE_LIB = os.path.join(LIBDIR, "libffa_probe.so")
BUILD = os.path.join(ROOT, "_build")
ARCH = "gfx950"


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


# packed fp32 VALU forms are kept out of the generated code on purpose
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-command-line-argument"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def source_hash() -> str:
    """First 16 hex digits of a SHA-256 over the library's sources (csrc/
    and include/ffa.h, names and contents); ffa_build_info reports the value
    the library was built with, so a stale build can be told apart."""
    files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp", ".hpp")))
    h = hashlib.sha256()
    for rel in [os.path.join("csrc", f) for f in files] + [os.path.join("..", "include", "ffa.h")]:
        h.update(rel.encode())
        with open(os.path.join(PKG, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _compile(src: str, hipcc: str, src_hash: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc, *HIP_FLAGS, f'-DFFA_SOURCE_HASH="{src_hash}"', "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-c", src, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = sources()
    src_hash = source_hash()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc, src_hash), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_probe(hipcc)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_probe(hipcc: str) -> str:
    """The matrix-core rate probe bench.py --mfma-ceiling loads: a library of
    its own, so nothing of it sits in libffa.so."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc, "-x", "hip", *HIP_FLAGS, "-shared", PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build_planner_sanitized(out: str) -> str:
    """Host-only planner test driver (tests/native/planner_driver.cpp) with
    AddressSanitizer and UndefinedBehaviorSanitizer: plain g++, no GPU code."""
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-I", CSRC, os.path.join(CSRC, "planner.cpp"),
           os.path.join(ROOT, "tests", "native", "planner_driver.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitizer build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
