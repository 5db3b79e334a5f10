"""Builds oracle/libk3oracle.so from k3oracle.c with gcc (plain C99,
single-threaded, no fast-math). Test infrastructure only."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "k3oracle.c")
LIB = os.path.join(HERE, "libk3oracle.so")
CC = os.environ.get("CC", "gcc")
FLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
         "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    res = subprocess.run([CC, *FLAGS, SRC, "-o", tmp, "-lm"], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"{CC} failed on oracle/k3oracle.c:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def is_stale() -> bool:
    return (not os.path.exists(LIB)) or os.path.getmtime(LIB) < os.path.getmtime(SRC)


if __name__ == "__main__":
    build(verbose=True)
