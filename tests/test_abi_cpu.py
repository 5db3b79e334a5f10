"""The C-ABI library loads on a host without a GPU, exports every symbol
include/k3moe.h declares, and rejects invalid configurations before any
device call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "k3moe.h")).read()
    return sorted(set(re.findall(r"\b(k3moe_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    import mxfp4_expert_matmul_amd as k3m
    if not os.path.exists(k3m.library_path()):
        pytest.skip("libk3moe.so not built")
    return k3m


def test_exports_every_declared_symbol(lib):
    dll = ctypes.CDLL(lib.library_path())
    names = _declared()
    assert {"k3moe_create", "k3moe_destroy", "k3moe_layer_forward", "k3moe_status_str"} <= set(names)
    for n in names:
        assert hasattr(dll, n), n


def test_status_strings(lib):
    for code in (lib.K3MOE_OK, lib.K3MOE_EINVAL, lib.K3MOE_ENOMEM, lib.K3MOE_EHIP,
                 lib.K3MOE_EUNSUPPORTED, 12345):
        assert isinstance(lib.k3moe_status_str(code), str) and lib.k3moe_status_str(code)


@pytest.mark.parametrize("cfg,want", [
    ((128, 8, 2, 256, 1), "ok"),
    ((7168, 896, 16, 2048, 4096), "ok"),
    ((100, 8, 2, 256, 1), -1),       # d not whole MX blocks
    ((160, 8, 2, 256, 1), -4),       # d % 128 != 0
    ((128, 8, 9, 256, 1), -1),       # k > E
    ((128, 8, 2, 256, 0), -1),       # no tokens
    ((128, 8, 2, 8192, 1), -4),      # f beyond the supported range
    ((128, 8000, 2, 256, 1), -4),    # E beyond the supported range
    ((128, 8, 64, 256, 1), -1),      # k > E
    ((128, 64, 64, 256, 2 ** 26), -4),  # T*k overflows int32
    ((8192, 8, 2, 256, 2 ** 17 + 1), -4),  # T*d plane beyond 2^30 bytes
    ((128, 896, 16, 4096, 2 ** 14 + 1), -4),  # T*k*f plane beyond 2^30 bytes
    ((7168, 896, 16, 2048, 32768), "ok"),  # largest K3 token count within both limits
    ((7168, 896, 16, 2048, 32769), -4),
])
def test_workspace_bytes_validation(lib, cfg, want):
    n = lib.k3moe_workspace_bytes(lib.Config(*cfg))
    if want == "ok":
        assert n > 0
    else:
        assert n == want


def test_workspace_scales_with_tokens(lib):
    a = lib.k3moe_workspace_bytes(lib.Config(7168, 896, 16, 2048, 1))
    b = lib.k3moe_workspace_bytes(lib.Config(7168, 896, 16, 2048, 4096))
    assert 0 < a < b < 2_500_000_000


def test_create_without_gpu_returns_status(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("host has a GPU")
    with pytest.raises(lib.K3MoEError) as ei:
        lib.Layer(lib.Config(128, 8, 2, 256, 1), {}, 0)
    assert ei.value.status in (lib.K3MOE_EINVAL, lib.K3MOE_EHIP)


def test_cache_create_validates_before_any_device_call(lib):
    """k3moe_cache_create checks its arguments on the host first: these
    calls return their status without touching a GPU."""
    import ctypes as C
    from mxfp4_expert_matmul_amd._binding import _Weights
    dll = lib.load_library()
    out = C.c_void_p()
    good = lib.Config(2048, 64, 8, 1024, 4)._c()
    buf = (C.c_uint8 * 64)()
    p = C.cast(C.addressof(buf) + (-C.addressof(buf)) % 16, C.c_void_p).value  # 16-byte aligned
    w = _Weights(p, None, p, p, p, p, p, p)
    assert dll.k3moe_cache_create(C.byref(good), None, 16, 0, C.byref(out)) == lib.K3MOE_EINVAL
    for n_slots in (7, 65):  # fewer than top-k, more than the experts
        assert dll.k3moe_cache_create(C.byref(good), C.byref(w), n_slots, 0, C.byref(out)) == lib.K3MOE_EINVAL
    bad = lib.Config(160, 64, 8, 1024, 4)._c()  # d % 128 != 0
    assert dll.k3moe_cache_create(C.byref(bad), C.byref(w), 16, 0, C.byref(out)) == lib.K3MOE_EUNSUPPORTED
    nodown = _Weights(p, None, p, p, p, p, p, None)
    assert dll.k3moe_cache_create(C.byref(good), C.byref(nodown), 16, 0, C.byref(out)) == lib.K3MOE_EINVAL
    assert out.value is None
    assert dll.k3moe_cache_stats(None, None, None, None, None) == lib.K3MOE_EINVAL
    dll.k3moe_cache_destroy(None)  # NULL-safe
    # the device-planned variant: unknown flags, and its two entry points on NULL
    for flags in (2, 3, 0x80000000):
        assert dll.k3moe_cache_create_ex(C.byref(good), C.byref(w), 16, 0, flags,
                                         C.byref(out)) == lib.K3MOE_EINVAL
    assert dll.k3moe_cache_create_ex(C.byref(good), None, 16, 0, lib.K3MOE_CACHE_DEVICE_PLAN,
                                     C.byref(out)) == lib.K3MOE_EINVAL
    assert out.value is None
    assert dll.k3moe_cache_prefetch_device(None, p, 2, None) == lib.K3MOE_EINVAL
    assert dll.k3moe_cache_device_counters(None, None, None) == lib.K3MOE_EINVAL


def test_noalloc_validates_before_any_device_call(lib):
    """k3moe_layer_forward_noalloc checks its arguments on the host first:
    malformed calls return EINVAL and calls beyond its scratch array or the
    decode path return EUNSUPPORTED, without touching a GPU."""
    import ctypes as C
    from mxfp4_expert_matmul_amd._binding import _Weights
    dll = lib.load_library()
    buf = (C.c_uint8 * 64)()
    p = C.cast(C.addressof(buf) + (-C.addressof(buf)) % 16, C.c_void_p).value  # 16-byte aligned
    w = _Weights(p, None, p, p, p, p, p, p)
    good = lib.Config(2048, 64, 8, 1024, 8)._c()
    f = dll.k3moe_layer_forward_noalloc
    assert f(None, C.byref(w), p, 1, p, None, None, None) == lib.K3MOE_EINVAL
    assert f(C.byref(good), None, p, 1, p, None, None, None) == lib.K3MOE_EINVAL
    assert f(C.byref(good), C.byref(w), p, 9, p, None, None, None) == lib.K3MOE_EINVAL   # T > max_tokens
    assert f(C.byref(good), C.byref(w), None, 1, p, None, None, None) == lib.K3MOE_EINVAL
    assert f(C.byref(good), C.byref(w), p, 1, p, p, None, None) == lib.K3MOE_EINVAL      # idx without gate
    assert f(C.byref(good), C.byref(w), p, 5, p, None, None, None) == lib.K3MOE_EUNSUPPORTED  # T > 4
    big = lib.Config(4096, 4096, 64, 4096, 4)._c()  # 4 MiB of h at T = 4
    assert f(C.byref(big), C.byref(w), p, 4, p, None, None, None) == lib.K3MOE_EUNSUPPORTED
    nodown = _Weights(p, None, p, p, p, p, p, None)
    assert f(C.byref(good), C.byref(nodown), p, 1, p, None, None, None) == lib.K3MOE_EINVAL
    assert f(C.byref(good), C.byref(w), p, 0, p, None, None, None) == lib.K3MOE_OK       # T = 0


def test_flags_validation(lib):
    """flags: 0 and the selection-only bias bit are valid, any other bit is
    refused."""
    assert lib.k3moe_workspace_bytes(lib.Config(128, 8, 2, 256, 1, 0)) > 0
    assert lib.k3moe_workspace_bytes(lib.Config(128, 8, 2, 256, 1, lib.K3MOE_FLAG_BIAS_SELECT_ONLY)) > 0
    for bad in (2, 4, 3, 1 << 31):
        assert lib.k3moe_workspace_bytes(lib.Config(128, 8, 2, 256, 1, bad)) == lib.K3MOE_EINVAL
