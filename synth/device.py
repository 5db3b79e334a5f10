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
        _lib = lib
    return _lib


def device_weights(cfg: LayerConfig, device="cuda:0") -> dict:
    """All layer weights on the device: router_w, router_b (or None) and the
    six MXFP4 tensors (uint8), generated in place."""
    import torch
    lib = _load()
    dev = torch.device(device)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    out = {}
    for name, shape in cfg.tensor_shapes().items():
        t = torch.empty(shape, dtype=torch.uint8, device=dev)
        key = stream_key(cfg.seed, WEIGHT_STREAMS[name])
        fn = lib.k3synth_fill_codes if name.endswith("_q") else lib.k3synth_fill_scales
        rc = fn(ctypes.c_void_p(t.data_ptr()), t.numel(), key, stream)
        if rc != 0:
            raise RuntimeError(f"synth fill of {name} failed ({rc})")
        out[name] = t
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
    import torch
    out = {k: torch.from_numpy(np.ascontiguousarray(v)).to(device) for k, v in w.items()}
    out["router_w"] = torch.from_numpy(np.ascontiguousarray(router_w)).to(device)
    out["router_b"] = None if bias is None else torch.from_numpy(np.asarray(bias)).to(device)
    return out
