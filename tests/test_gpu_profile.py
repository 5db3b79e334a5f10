"""GPU tests of the stage-timing entry points (k3moe_profile_begin /
k3moe_profile_end): which stages a call times, the cap on timed launches per
stage, that the events are released at the end, and the refusals."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# stage order of the K3MOE_STAGE_* constants
STAGES = ("router_logits", "topk", "group", "quant_x", "gateup", "combine", "down")
N_STAGES = len(STAGES)


@pytest.fixture(scope="module")
def k3():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp4_expert_matmul_amd as k3m
    k3m.load_library()
    return k3m


def _layer(k3, cfg, max_tokens):
    from synth.device import host_weights_to_device
    W = synth.gen_weights(cfg)
    wr = synth.gen_router_w(cfg)
    dw = k3.pack_layer_weights(host_weights_to_device(W, wr, None), cfg.E, cfg.d, cfg.f)
    return k3.Layer(k3.Config(cfg.d, cfg.E, cfg.k, cfg.f, max_tokens), dw, 0)


def _x(cfg, T, stream):
    bits = synth.gen_x(cfg, T=T, stream=stream)
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _end(lib, handle):
    total = (ctypes.c_float * N_STAGES)()
    launches = (ctypes.c_int32 * N_STAGES)()
    rc = lib.k3moe_profile_end(handle, total, launches)
    return rc, list(total), list(launches)


def test_stage_profile(k3):
    lib = k3.load_library()
    cfg = synth.CONFIGS[1]  # d 2048, 64 experts, top-8
    layer = _layer(k3, cfg, 64)
    h = layer.handle

    # refusals: end before begin, and a non-positive cap
    assert _end(lib, h)[0] == k3.K3MOE_EINVAL
    assert lib.k3moe_profile_begin(h, 0) == k3.K3MOE_EINVAL

    # decode (T <= 4): router, gate/up (the top-k inside it) and down, at most
    # max_calls timed launches per stage
    assert lib.k3moe_profile_begin(h, 2) == k3.K3MOE_OK
    for i in range(3):
        layer.forward(_x(cfg, 1, 30 + i))
    rc, total, launches = _end(lib, h)
    assert rc == k3.K3MOE_OK
    want = {"router_logits": 2, "gateup": 2, "down": 2}
    assert launches == [want.get(s, 0) for s in STAGES]
    for s, ms, n in zip(STAGES, total, launches):
        assert (ms > 0.0) == (n > 0), (s, ms, n)

    # the events were released: a second end is refused
    assert _end(lib, h)[0] == k3.K3MOE_EINVAL

    # grouped path (T > 4): every stage once, the x split timed on the side
    # stream of the handle; untimed calls after the cap still run
    assert lib.k3moe_profile_begin(h, 1) == k3.K3MOE_OK
    y0, _, _ = layer.forward(_x(cfg, 40, 40))
    y1, _, _ = layer.forward(_x(cfg, 40, 40))
    torch.cuda.synchronize()
    rc, total, launches = _end(lib, h)
    assert rc == k3.K3MOE_OK
    assert launches == [1] * N_STAGES
    assert all(ms > 0.0 for ms in total), dict(zip(STAGES, total))
    assert torch.equal(y0, y1)

    # timing changes nothing: the same call without it gives the same output
    y2, _, _ = layer.forward(_x(cfg, 40, 40))
    torch.cuda.synchronize()
    assert torch.equal(y0, y2)
    layer.close()


def test_stage_profile_mask(k3):
    """k3moe_profile_begin_stages times only the masked stages; a zero mask
    or one with bits past the last stage is refused."""
    lib = k3.load_library()
    cfg = synth.CONFIGS[1]
    layer = _layer(k3, cfg, 64)
    h = layer.handle
    gateup = STAGES.index("gateup")
    assert lib.k3moe_profile_begin_stages(h, 4, 0) == k3.K3MOE_EINVAL
    assert lib.k3moe_profile_begin_stages(h, 4, 1 << N_STAGES) == k3.K3MOE_EINVAL
    assert lib.k3moe_profile_begin_stages(h, 0, 1 << gateup) == k3.K3MOE_EINVAL
    for T, mask in ((40, 1 << gateup), (1, 1 << gateup), (40, (1 << gateup) | 1)):
        assert lib.k3moe_profile_begin_stages(h, 2, mask) == k3.K3MOE_OK
        for i in range(3):
            layer.forward(_x(cfg, T, 50 + i))
        rc, total, launches = _end(lib, h)
        assert rc == k3.K3MOE_OK
        want = [2 if (mask >> i) & 1 else 0 for i in range(N_STAGES)]
        assert launches == want, (T, mask, launches)
        for s, ms, n in zip(STAGES, total, launches):
            assert (ms > 0.0) == (n > 0), (T, s, ms, n)
    layer.close()
