"""Host-side checks of the ctypes binding's argument marshalling (no GPU):
device-pointer arguments must be contiguous GPU tensors of the documented
element type, since the library itself can check only their alignment."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mxfp4_expert_matmul_amd as k3  # noqa: E402
from mxfp4_expert_matmul_amd import _binding as b  # noqa: E402


class _FakeGpu:
    """Stands in for a GPU tensor (no GPU here): only what _dev reads."""

    def __init__(self, dtype, contiguous=True):
        self.is_cuda = True
        self.dtype = dtype
        self._c = contiguous

    def is_contiguous(self):
        return self._c

    def data_ptr(self):
        return 4096


def test_dev_accepts_the_documented_layouts():
    assert b._dev(None, "y", b._F32) is None
    assert b._dev(_FakeGpu(torch.float32), "y", b._F32).value == 4096
    assert b._dev(_FakeGpu(torch.bfloat16), "x", b._BF16).value == 4096
    assert b._dev(_FakeGpu(torch.int16), "x", b._BF16).value == 4096


@pytest.mark.parametrize("t, dtypes, what", [
    (torch.zeros(4, dtype=torch.float32), b._F32, "GPU tensor"),
    (_FakeGpu(torch.float32, contiguous=False), b._F32, "contiguous"),
    (_FakeGpu(torch.int64), b._I32, "dtype"),
    (_FakeGpu(torch.float16), b._BF16, "dtype"),
])
def test_dev_refuses_host_strided_and_mistyped_tensors(t, dtypes, what):
    with pytest.raises(ValueError, match=what):
        b._dev(t, "arg", dtypes)


def test_forward_refuses_a_host_tensor_before_calling_the_library():
    try:
        k3.load_library()
    except Exception:
        pytest.skip("library not built")
    x = torch.zeros((1, 128), dtype=torch.bfloat16)
    y = torch.zeros((1, 128), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        k3.k3moe_layer_forward(None, x, y)


def test_cache_weights_take_host_experts_and_a_device_router():
    names = [n for n, _ in b._Weights._fields_]
    host = {n: np.zeros(64, dtype=np.uint8) for n in names if n not in ("router_w", "router_b")}
    host["router_w"] = torch.zeros(4, dtype=torch.float32)  # on the host: refused
    with pytest.raises(ValueError, match="router_w: expected a GPU tensor"):
        b._weights(host, host_experts=True)
    host["router_w"] = _FakeGpu(torch.float32)
    w = b._weights(host, host_experts=True)
    assert w.router_w == 4096 and w.router_b is None
    assert w.gate_q == host["gate_q"].ctypes.data
