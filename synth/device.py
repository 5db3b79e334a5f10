"""Device-resident synthetic workloads (torch tensors on a GPU).

Integer streams (codes, scales) are generated on the device by
libk3synth.so, bit-identical to the host generator; floating-point streams
(activations, router weights, bias) are generated on the host and copied.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import (LayerConfig, WEIGHT_STREAMS, gen_bias, gen_router_w, gen_x, stream_key)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_HERE, "libk3synth.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError(f"{_LIB} is missing: build it with synth/build.py")
        lib = ctypes.CDLL(_LIB)
        for fn in (lib.k3synth_fill_codes, lib.k3synth_fill_scales):
            fn.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p]
            fn.restype = ctypes.c_int
        for fn in (lib.k3synth_fill_codes_tiled, lib.k3synth_fill_scales_tiled):
            fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                           ctypes.c_uint64, ctypes.c_void_p]
            fn.restype = ctypes.c_int
        _lib = lib
    return _lib


def tiled_scale_bytes(n: int, R: int, K: int) -> int:
    """Bytes of scales for n stacked R x K matrices in the tiled layout."""
    return n * (R // 16) * ((K // 128 + 3) // 4) * 256


def device_tensor(cfg: LayerConfig, name: str, device="cuda:0", tiled: bool = True):
    """One MXFP4 weight tensor of the layer (gate_q, gate_s, up_q, up_s,
    down_q or down_s) on the device, uint8, generated in place: in the tiled
    layout the layer library reads (flat; the same draws placed by their
    row-major index) or row-major ([E][R][K/2] codes, [E][R][K/32] scales)."""
    import torch
    lib = _load()
    dev = torch.device(device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    dims = {"gate": (cfg.f, cfg.d), "up": (cfg.f, cfg.d), "down": (cfg.d, cfg.f)}
    shape = cfg.tensor_shapes()[name]
    key = stream_key(cfg.seed, WEIGHT_STREAMS[name])
    R, K = dims[name[:-2]]
    if tiled:
        nbytes = int(np.prod(shape)) if name.endswith("_q") else tiled_scale_bytes(cfg.E, R, K)
        t = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        fn = lib.k3synth_fill_codes_tiled if name.endswith("_q") else lib.k3synth_fill_scales_tiled
        rc = fn(ctypes.c_void_p(t.data_ptr()), cfg.E, R, K, key, stream)
    else:
        t = torch.empty(shape, dtype=torch.uint8, device=dev)
        fn = lib.k3synth_fill_codes if name.endswith("_q") else lib.k3synth_fill_scales
        rc = fn(ctypes.c_void_p(t.data_ptr()), t.numel(), key, stream)
    if rc != 0:
        raise RuntimeError(f"synth fill of {name} failed ({rc})")
    return t


def device_weights(cfg: LayerConfig, device="cuda:0", tiled: bool = True) -> dict:
    """All layer weights on the device: router_w, router_b (or None) and the
    six MXFP4 tensors (uint8), generated in place, tiled or row-major as in
    device_tensor."""
    import torch
    dev = torch.device(device)
    out = {}
    for name in cfg.tensor_shapes():
        out[name] = device_tensor(cfg, name, dev, tiled)
    out["router_w"] = torch.from_numpy(gen_router_w(cfg)).to(dev)
    b = gen_bias(cfg)
    out["router_b"] = None if b is None else torch.from_numpy(b).to(dev)
    return out


def device_x(cfg: LayerConfig, T: int | None = None, start_token: int = 0, stream: int = 1,
             device="cuda:0"):
    """Activations [T][d] as torch.bfloat16 on the device (same bits as gen_x)."""
    import torch
    x = gen_x(cfg, T=T, start_token=start_token, stream=stream)
    return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)


def host_weights_to_device(w: dict, router_w: np.ndarray, bias, device="cuda:0") -> dict:
    """Row-major host weights copied to the device as they are."""
    import torch
    out = {k: torch.from_numpy(np.ascontiguousarray(v)).to(device) for k, v in w.items()}
    out["router_w"] = torch.from_numpy(np.ascontiguousarray(router_w)).to(device)
    out["router_b"] = None if bias is None else torch.from_numpy(np.asarray(bias)).to(device)
    return out
