"""ctypes binding of libk3moe.so with the C entry points' names.

Tensors are torch tensors on the handle's GPU; only their data pointers and
the current HIP stream handle cross the boundary.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libk3moe.so")

K3MOE_OK = 0
K3MOE_EINVAL = -1
K3MOE_ENOMEM = -2
K3MOE_EHIP = -3
K3MOE_EUNSUPPORTED = -4
K3MOE_FLAG_BIAS_SELECT_ONLY = 1  # k3moe_config.flags: the router bias only ranks the experts
K3MOE_CACHE_DEVICE_PLAN = 1  # k3moe_cache_create_ex flags: residency tables and planning on the device


class K3MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {k3moe_status_str(status)} (status {status})")


class _Config(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class _Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("router_w", "router_b", "gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")]


@dataclasses.dataclass(frozen=True)
class Config:
    d_model: int
    n_experts: int
    top_k: int
    d_ff: int
    max_tokens: int
    flags: int = 0

    def _c(self) -> _Config:
        return _Config(self.d_model, self.n_experts, self.top_k, self.d_ff, self.max_tokens,
                       self.flags)


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libk3moe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with mxfp4_expert_matmul_amd/build.py "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.k3moe_status_str.argtypes = [ctypes.c_int]
    lib.k3moe_status_str.restype = ctypes.c_char_p
    lib.k3moe_workspace_bytes.argtypes = [ctypes.POINTER(_Config)]
    lib.k3moe_workspace_bytes.restype = i64
    lib.k3moe_create.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Weights), ctypes.c_int,
                                 ctypes.POINTER(vp)]
    lib.k3moe_create.restype = ctypes.c_int
    lib.k3moe_destroy.argtypes = [vp]
    lib.k3moe_destroy.restype = None
    lib.k3moe_layer_forward.argtypes = [vp, vp, i32, vp, vp, vp, vp]
    lib.k3moe_layer_forward.restype = ctypes.c_int
    lib.k3moe_route.argtypes = [vp, vp, i32, vp, vp, vp, vp]
    lib.k3moe_route.restype = ctypes.c_int
    lib.k3moe_group.argtypes = [vp, vp, i32, vp, vp, vp, vp]
    lib.k3moe_group.restype = ctypes.c_int
    lib.k3moe_experts_forward.argtypes = [vp, vp, i32, vp, vp, vp, vp]
    lib.k3moe_experts_forward.restype = ctypes.c_int
    lib.k3moe_pack_mxfp4.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
    lib.k3moe_pack_mxfp4.restype = ctypes.c_int
    lib.k3moe_pack_mxfp4_from_host.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
    lib.k3moe_pack_mxfp4_from_host.restype = ctypes.c_int
    lib.k3moe_tiled_scale_bytes.argtypes = [i32, i32, i32]
    lib.k3moe_tiled_scale_bytes.restype = i64
    lib.k3moe_profile_begin.argtypes = [vp, i32]
    lib.k3moe_profile_begin.restype = ctypes.c_int
    lib.k3moe_profile_end.argtypes = [vp, vp, vp]
    lib.k3moe_profile_end.restype = ctypes.c_int
    lib.k3moe_profile_begin_stages.argtypes = [vp, i32, ctypes.c_uint32]
    lib.k3moe_profile_begin_stages.restype = ctypes.c_int
    lib.k3moe_cache_create.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Weights), i32,
                                       ctypes.c_int, ctypes.POINTER(vp)]
    lib.k3moe_cache_create.restype = ctypes.c_int
    lib.k3moe_cache_forward.argtypes = [vp, vp, i32, vp, vp, vp, vp]
    lib.k3moe_cache_forward.restype = ctypes.c_int
    lib.k3moe_cache_stats.argtypes = [vp, vp, vp, vp, vp]
    lib.k3moe_cache_stats.restype = ctypes.c_int
    lib.k3moe_cache_destroy.argtypes = [vp]
    lib.k3moe_cache_destroy.restype = None
    lib.k3moe_cache_prefetch.argtypes = [vp, vp, i32, vp]
    lib.k3moe_cache_prefetch.restype = ctypes.c_int
    lib.k3moe_layer_forward_noalloc.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Weights),
                                                vp, i32, vp, vp, vp, vp]
    lib.k3moe_layer_forward_noalloc.restype = ctypes.c_int
    lib.k3moe_cache_prefetch_stats.argtypes = [vp, vp, vp]
    lib.k3moe_cache_prefetch_stats.restype = ctypes.c_int
    lib.k3moe_cache_create_ex.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(_Weights), i32,
                                          ctypes.c_int, ctypes.c_uint32, ctypes.POINTER(vp)]
    lib.k3moe_cache_create_ex.restype = ctypes.c_int
    lib.k3moe_cache_prefetch_device.argtypes = [vp, vp, i32, vp]
    lib.k3moe_cache_prefetch_device.restype = ctypes.c_int
    lib.k3moe_cache_device_counters.argtypes = [vp, vp, vp]
    lib.k3moe_cache_device_counters.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# dtypes the C ABI reads (by name, so torch is imported only when used)
_BF16 = ("bfloat16", "int16")  # x: bf16 values or their bit patterns
_F32, _I32, _U8 = ("float32",), ("int32",), ("uint8",)


def _dev(t, name, dtypes):
    """Device pointer of a contiguous GPU tensor of one of `dtypes` (None
    stays NULL). The library can check alignment only: a host pointer, a
    strided view or another element type would be read as if it were the
    documented layout, so they are refused here."""
    if t is None:
        return None
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name}: expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if str(t.dtype).replace("torch.", "") not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {' or '.join(dtypes)}")
    return ctypes.c_void_p(t.data_ptr())


_WEIGHT_DTYPES = {"router_w": _F32, "router_b": _F32}


def _weights(weights: dict, host_experts: bool = False) -> "_Weights":
    """The weight pointers: device tensors, except the six expert tensors of
    a cache (host_experts), which are host tensors."""
    ptrs = []
    for n, _ in _Weights._fields_:
        t = weights.get(n)
        if t is None:
            ptrs.append(None)
        elif host_experts and n not in _WEIGHT_DTYPES:
            ptrs.append(_host_ptr(t).value)
        else:
            ptrs.append(_dev(t, n, _WEIGHT_DTYPES.get(n, _U8)).value)
    return _Weights(*ptrs)


def _stream(stream, device):
    if stream is not None:
        return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(rc: int, where: str):
    if rc != K3MOE_OK:
        raise K3MoEError(rc, where)


def k3moe_status_str(status: int) -> str:
    return load_library().k3moe_status_str(int(status)).decode()


def k3moe_workspace_bytes(cfg: Config) -> int:
    c = cfg._c()
    return int(load_library().k3moe_workspace_bytes(ctypes.byref(c)))


def k3moe_create(cfg: Config, weights: dict, device: int = 0) -> ctypes.c_void_p:
    """weights: dict of device tensors router_w, router_b (or None), gate_q,
    gate_s, up_q, up_s, down_q, down_s in the layout of include/k3moe.h."""
    lib = load_library()
    c = cfg._c()
    w = _weights(weights)
    out = ctypes.c_void_p()
    rc = lib.k3moe_create(ctypes.byref(c), ctypes.byref(w), int(device), ctypes.byref(out))
    _check(rc, "k3moe_create")
    return out


def k3moe_destroy(handle) -> None:
    if handle:
        load_library().k3moe_destroy(handle)


def k3moe_layer_forward(handle, x, y, topk_idx=None, topk_gate=None, stream=None, device=None):
    T = x.shape[0]
    rc = load_library().k3moe_layer_forward(handle, _dev(x, "x", _BF16), T, _dev(y, "y", _F32),
                                            _dev(topk_idx, "topk_idx", _I32),
                                            _dev(topk_gate, "topk_gate", _F32),
                                            _stream(stream, device or x.device))
    _check(rc, "k3moe_layer_forward")


def k3moe_layer_forward_noalloc(cfg: Config, weights: dict, x, y, topk_idx=None, topk_gate=None,
                                stream=None):
    """Decode-sized forward (T <= 4) without a handle or any allocation, on
    the current device; weights as for k3moe_create."""
    c = cfg._c()
    w = _weights(weights)
    rc = load_library().k3moe_layer_forward_noalloc(ctypes.byref(c), ctypes.byref(w),
                                                    _dev(x, "x", _BF16), x.shape[0],
                                                    _dev(y, "y", _F32),
                                                    _dev(topk_idx, "topk_idx", _I32),
                                                    _dev(topk_gate, "topk_gate", _F32),
                                                    _stream(stream, x.device))
    _check(rc, "k3moe_layer_forward_noalloc")


def k3moe_route(handle, x, idx, gate, logits=None, stream=None):
    rc = load_library().k3moe_route(handle, _dev(x, "x", _BF16), x.shape[0],
                                    _dev(logits, "logits", _F32), _dev(idx, "idx", _I32),
                                    _dev(gate, "gate", _F32), _stream(stream, x.device))
    _check(rc, "k3moe_route")


def k3moe_group(handle, idx, counts, offsets, perm, stream=None):
    rc = load_library().k3moe_group(handle, _dev(idx, "idx", _I32), idx.shape[0],
                                    _dev(counts, "counts", _I32), _dev(offsets, "offsets", _I32),
                                    _dev(perm, "perm", _I32), _stream(stream, idx.device))
    _check(rc, "k3moe_group")


def k3moe_experts_forward(handle, x, idx, gate, y, stream=None):
    rc = load_library().k3moe_experts_forward(handle, _dev(x, "x", _BF16), x.shape[0],
                                              _dev(idx, "idx", _I32), _dev(gate, "gate", _F32),
                                              _dev(y, "y", _F32), _stream(stream, x.device))
    _check(rc, "k3moe_experts_forward")


def k3moe_tiled_scale_bytes(n: int, R: int, K: int) -> int:
    return int(load_library().k3moe_tiled_scale_bytes(n, R, K))


def k3moe_pack_mxfp4(codes, scales, n, R, K, tiled_codes, tiled_scales, stream=None):
    rc = load_library().k3moe_pack_mxfp4(_dev(codes, "codes", _U8), _dev(scales, "scales", _U8),
                                         n, R, K, _dev(tiled_codes, "tiled_codes", _U8),
                                         _dev(tiled_scales, "tiled_scales", _U8),
                                         _stream(stream, codes.device))
    _check(rc, "k3moe_pack_mxfp4")


def _host_ptr(a):
    """Data pointer of a host numpy array or CPU torch tensor (C-contiguous)."""
    if hasattr(a, "data_ptr"):
        if a.is_cuda or not a.is_contiguous():
            raise ValueError("expected a contiguous host tensor")
        return ctypes.c_void_p(a.data_ptr())
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("expected a C-contiguous host array")
    return ctypes.c_void_p(a.ctypes.data)


def k3moe_pack_mxfp4_from_host(codes, scales, n, R, K, tiled_codes, tiled_scales, stream=None):
    """Row-major host codes/scales (numpy or CPU tensors) -> tiled device tensors."""
    rc = load_library().k3moe_pack_mxfp4_from_host(_host_ptr(codes), _host_ptr(scales), n, R, K,
                                                   _dev(tiled_codes, "tiled_codes", _U8),
                                                   _dev(tiled_scales, "tiled_scales", _U8),
                                                   _stream(stream, tiled_codes.device))
    _check(rc, "k3moe_pack_mxfp4_from_host")


def pack_mxfp4_from_host(codes, scales, n, R, K, device="cuda"):
    """Row-major host matrices -> new tiled device tensors (flat uint8)."""
    import torch
    tc = torch.empty(n * R * K // 2, dtype=torch.uint8, device=device)
    ts = torch.empty(k3moe_tiled_scale_bytes(n, R, K), dtype=torch.uint8, device=device)
    k3moe_pack_mxfp4_from_host(codes, scales, n, R, K, tc, ts)
    return tc, ts


def pack_layer_weights_from_host(w: dict, E: int, d: int, f: int, device="cuda") -> dict:
    """Row-major layer weights in host memory (the six MXFP4 tensors; router_w
    and router_b as host arrays or None) -> device weights for k3moe_create."""
    import numpy as np
    import torch
    out = {}
    for name, (R, K) in (("gate", (f, d)), ("up", (f, d)), ("down", (d, f))):
        out[name + "_q"], out[name + "_s"] = pack_mxfp4_from_host(w[name + "_q"], w[name + "_s"],
                                                                  E, R, K, device)
    for name in ("router_w", "router_b"):
        v = w.get(name)
        out[name] = None if v is None else torch.as_tensor(np.asarray(v, dtype=np.float32)).to(device)
    return out


def pack_mxfp4(codes, scales, n, R, K):
    """Row-major device tensors -> new tiled device tensors (flat uint8)."""
    import torch
    tc = torch.empty(n * R * K // 2, dtype=torch.uint8, device=codes.device)
    ts = torch.empty(k3moe_tiled_scale_bytes(n, R, K), dtype=torch.uint8, device=codes.device)
    k3moe_pack_mxfp4(codes, scales, n, R, K, tc, ts)
    return tc, ts


def pack_layer_weights(w: dict, E: int, d: int, f: int) -> dict:
    """Row-major layer weights on the device -> tiled copies (other entries kept)."""
    out = dict(w)
    for name, (R, K) in (("gate", (f, d)), ("up", (f, d)), ("down", (d, f))):
        out[name + "_q"], out[name + "_s"] = pack_mxfp4(w[name + "_q"], w[name + "_s"], E, R, K)
    return out


class Layer:
    """Owns one k3moe handle. Weights are borrowed: keep the tensors alive."""

    def __init__(self, cfg: Config, weights: dict, device: int = 0):
        self.cfg = cfg
        self.device = device
        self._weights = weights  # keep borrowed tensors alive
        self.handle = k3moe_create(cfg, weights, device)

    def forward(self, x, stream=None):
        """x: [T][d] bf16 (torch.bfloat16 or int16 bit patterns) on the GPU.
        Returns (y fp32 [T][d], idx int32 [T][k], gate fp32 [T][k])."""
        import torch
        T = x.shape[0]
        dev = x.device
        y = torch.empty((T, self.cfg.d_model), dtype=torch.float32, device=dev)
        idx = torch.empty((T, self.cfg.top_k), dtype=torch.int32, device=dev)
        gate = torch.empty((T, self.cfg.top_k), dtype=torch.float32, device=dev)
        k3moe_layer_forward(self.handle, x, y, idx, gate, stream=stream)
        return y, idx, gate

    def close(self):
        if self.handle:
            k3moe_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class CachedLayer:
    """A layer whose expert weights stay in host memory behind an HBM cache
    of n_slots experts (k3moe_cache_*). host_weights: router_w / router_b as
    device tensors, the six expert tensors as host (CPU, ideally pinned)
    tensors in the tiled layout. All are borrowed: keep them alive."""

    def __init__(self, cfg: Config, host_weights: dict, n_slots: int, device: int = 0,
                 device_plan: bool = False):
        lib = load_library()
        self.cfg = cfg
        self._weights = host_weights
        self.device_plan = bool(device_plan)
        c = cfg._c()
        w = _weights(host_weights, host_experts=True)
        out = ctypes.c_void_p()
        flags = K3MOE_CACHE_DEVICE_PLAN if device_plan else 0
        _check(lib.k3moe_cache_create_ex(ctypes.byref(c), ctypes.byref(w), int(n_slots),
                                         int(device), flags, ctypes.byref(out)),
               "k3moe_cache_create_ex")
        self.handle = out

    def forward(self, x, stream=None):
        """Like Layer.forward: returns (y, idx, gate) for x [T][d] bf16 on the GPU."""
        import torch
        T = x.shape[0]
        dev = x.device
        y = torch.empty((T, self.cfg.d_model), dtype=torch.float32, device=dev)
        idx = torch.empty((T, self.cfg.top_k), dtype=torch.int32, device=dev)
        gate = torch.empty((T, self.cfg.top_k), dtype=torch.float32, device=dev)
        _check(load_library().k3moe_cache_forward(self.handle, _dev(x, "x", _BF16), T, _ptr(y),
                                                  _ptr(idx), _ptr(gate), _stream(stream, dev)),
               "k3moe_cache_forward")
        return y, idx, gate

    def prefetch(self, experts, stream=None, device: int = 0):
        """Copy the listed experts (host ints) into the arena on `stream`
        (torch stream or None for the current one); the next forward waits
        for the copies."""
        import torch
        ids = (ctypes.c_int32 * len(experts))(*[int(e) for e in experts])
        _check(load_library().k3moe_cache_prefetch(self.handle, ids, len(experts),
                                                   _stream(stream, torch.device("cuda", device))),
               "k3moe_cache_prefetch")

    def prefetch_device(self, experts, stream=None):
        """Device-planned caches: prefetch the experts listed in `experts`, a
        contiguous int32 tensor on the GPU (read when the plan runs), on
        `stream` (torch stream or None for the current one)."""
        n = experts.numel()
        ptr = _dev(experts, "experts", _I32)
        _check(load_library().k3moe_cache_prefetch_device(
            self.handle, ptr if n else None, n, _stream(stream, experts.device)),
            "k3moe_cache_prefetch_device")

    def device_counters(self) -> dict:
        """Device-planned caches: refused prefetches and skipped prefetch ids."""
        v = [ctypes.c_int64() for _ in range(2)]
        _check(load_library().k3moe_cache_device_counters(self.handle, *[ctypes.byref(a) for a in v]),
               "k3moe_cache_device_counters")
        return {"refused_prefetches": v[0].value, "ignored_ids": v[1].value}

    def stats(self) -> dict:
        """calls, hits (raw: including experts a prefetch brought in), misses,
        bytes_in (forwards and prefetches), prefetched and prefetch_hits; true
        resident hits are hits - prefetch_hits."""
        lib = load_library()
        v = [ctypes.c_int64() for _ in range(6)]
        _check(lib.k3moe_cache_stats(self.handle, *[ctypes.byref(a) for a in v[:4]]),
               "k3moe_cache_stats")
        _check(lib.k3moe_cache_prefetch_stats(self.handle, *[ctypes.byref(a) for a in v[4:]]),
               "k3moe_cache_prefetch_stats")
        return dict(zip(("calls", "hits", "misses", "bytes_in", "prefetched", "prefetch_hits"),
                        (a.value for a in v)))

    def close(self):
        if self.handle:
            load_library().k3moe_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
