"""Builds the sanitizer harnesses of tests/sanitize/ (host code only).

* oracle_harness: the C oracle and its harness, gcc with AddressSanitizer and
  UndefinedBehaviorSanitizer;
* lru_harness: the expert cache's residency bookkeeping (csrc/lru.h), g++
  with both sanitizers;
* abi_harness: the library's host files (k3moe.cpp, cache.cpp) with both
  sanitizers on their host side, linked with the regular build's kernel
  objects, driven through the C ABI.

Every build goes to _build/sanitize/. Returns the paths of the executables.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(ROOT, "_build", "sanitize")
CSRC = os.path.join(ROOT, "mxfp4_expert_matmul_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
# env for running a harness: stop at the first report; leak checks are off
# because the HIP runtime keeps its allocations until exit
RUN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")


def build_oracle() -> str:
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_harness")
    _run(["gcc", "-std=c99", "-O1", "-g", "-ffp-contract=off", *SAN,
          os.path.join(HERE, "oracle_harness.c"), os.path.join(ROOT, "oracle", "k3oracle.c"),
          "-lm", "-o", exe])
    return exe


def build_lru() -> str:
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "lru_harness")
    _run(["g++", "-std=c++17", "-O1", "-g", *SAN, "-I", CSRC,
          os.path.join(HERE, "lru_harness.cpp"), "-o", exe])
    return exe


def build_abi() -> str:
    """Needs the regular build's kernel objects (_build/k3moe/*.o)."""
    from mxfp4_expert_matmul_amd import build as kbuild
    os.makedirs(OUT, exist_ok=True)
    kobj = [os.path.join(kbuild.BUILD, os.path.splitext(s)[0] + ".o")
            for s in kbuild.SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in kobj):
        kbuild.build()
    host = []
    for src in ("k3moe.cpp", "cache.cpp"):
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".asan.o")
        # sanitizers on the host side only: each flag behind -Xarch_host
        flags = [f for s in SAN for f in ("-Xarch_host", s)]
        _run([os.path.join(ROCM, "bin", "hipcc"), "-x", "hip", "--offload-arch=gfx950", "-O1", "-g",
              "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              *flags, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj])
        host.append(obj)
    cc = os.path.join(ROCM, "llvm", "bin", "clang")
    hobj = os.path.join(OUT, "abi_harness.o")
    _run([cc, "-O1", "-g", *SAN, "-I", INCLUDE, "-c", os.path.join(HERE, "abi_harness.c"), "-o", hobj])
    exe = os.path.join(OUT, "abi_harness")
    _run([cc + "++", "--hip-link", "--offload-arch=gfx950", *SAN, hobj, *host, *kobj, "-o", exe,
          "-L", os.path.join(ROCM, "lib"), "-lamdhip64"])
    return exe


if __name__ == "__main__":
    for fn in (build_oracle, build_lru, build_abi):
        print("built", fn())
