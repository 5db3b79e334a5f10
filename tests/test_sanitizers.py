"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer: the C
oracle, the expert cache's residency bookkeeping and the C ABI's host-side
checks, each driven by a harness in tests/sanitize/. A harness passes when
it exits 0 and neither sanitizer reported anything."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "sanitize"))
import build as sbuild  # noqa: E402


def _run(exe):
    env = dict(os.environ, **sbuild.RUN_ENV)
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    return out


def test_oracle_under_sanitizers():
    assert "all checks passed" in _run(sbuild.build_oracle())


def test_lru_bookkeeping_under_sanitizers():
    assert "all checks passed" in _run(sbuild.build_lru())


def test_abi_host_code_under_sanitizers():
    if not os.path.exists(os.path.join(sbuild.ROCM, "bin", "hipcc")):
        pytest.skip("hipcc not installed")
    assert "all checks passed" in _run(sbuild.build_abi())
