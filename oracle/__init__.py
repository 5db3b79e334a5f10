"""CPU oracle for the sparse MoE layer with MXFP4 expert weights.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call, link or
run anything under this directory: only the tests, the package smoke check and
the benchmark's CPU-baseline leg use it. It shares no code with the HIP path.
"""
from .k3oracle import *  # noqa: F401,F403
