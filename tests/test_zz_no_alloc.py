"""k3moe_layer_forward_noalloc: the decode-sized layer forward that keeps its
scratch in a fixed device array and allocates nothing. Its outputs must equal
k3moe_layer_forward's (the same kernels on the same data) on consecutive calls
that reuse the array, the second with fewer tokens; calls beyond the array's
size are refused before anything runs."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests._parity import check_output

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def k3():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp4_expert_matmul_amd as k3m
    k3m.load_library()
    return k3m


def _xd(x_bits):
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda().view(torch.bfloat16)


def _outs(cfg, T):
    return (torch.full((T, cfg.d), float("nan"), dtype=torch.float32, device="cuda"),
            torch.full((T, cfg.k), -7, dtype=torch.int32, device="cuda"),
            torch.full((T, cfg.k), float("nan"), dtype=torch.float32, device="cuda"))


def _check_pair(k3, cfg, dw, x_big, x_small, label):
    """noalloc(T=len(x_big)) then noalloc(T=len(x_small)) against the handle's
    forward on the same inputs: bit-equal routing, gates and outputs."""
    c = k3.Config(cfg.d, cfg.E, cfg.k, cfg.f, 4)
    layer = k3.Layer(c, dw, 0)
    ref = [layer.forward(x) for x in (x_big, x_small)]
    torch.cuda.synchronize()
    # first call with caller routing outputs, second with the routing kept in
    # the scratch array (only y is returned)
    y1, i1, g1 = _outs(cfg, x_big.shape[0])
    k3.k3moe_layer_forward_noalloc(c, dw, x_big, y1, i1, g1)
    y2, _, _ = _outs(cfg, x_small.shape[0])
    k3.k3moe_layer_forward_noalloc(c, dw, x_small, y2)
    torch.cuda.synchronize()
    assert torch.equal(i1, ref[0][1]) and torch.equal(g1, ref[0][2]), f"{label}: routing differs"
    assert torch.equal(y1, ref[0][0]), f"{label}: first call output differs"
    assert torch.equal(y2, ref[1][0]), f"{label}: second (smaller) call output differs"
    layer.close()
    return y1, y2, ref


def test_noalloc_equals_layer_forward_small(k3):
    """Small layer (d=2048, 64 experts, top-8): T=4 then T=1, and the second
    output against the oracle too."""
    from synth.device import host_weights_to_device
    cfg = synth.CONFIGS[1]
    W = synth.gen_weights(cfg)
    wr = synth.gen_router_w(cfg)
    dw = k3.pack_layer_weights(host_weights_to_device(W, wr, None), cfg.E, cfg.d, cfg.f)
    x = synth.gen_x(cfg, T=5, stream=19)
    _, y2, _ = _check_pair(k3, cfg, dw, _xd(x[:4]), _xd(x[4:5]), "small")
    r = oracle.layer_forward(x[4:5], wr, None, synth.ExpertSource(cfg, W), cfg.k)
    check_output(y2.cpu().numpy(), r["y64"], "noalloc small T=1")


@pytest.mark.timeout(600)
def test_noalloc_equals_layer_forward_k3(k3):
    """K3 decode shape (d=7168, 896 experts, top-16, f=2048): T=3 then T=1."""
    from synth.device import device_weights, device_x
    cfg = synth.CONFIGS[2]
    dw = device_weights(cfg, torch.device("cuda:0"))
    xp = device_x(cfg, T=4, stream=10, device=torch.device("cuda:0"))
    _check_pair(k3, cfg, dw, xp[:3], xp[3:4], "k3")
    del dw
    torch.cuda.empty_cache()


def test_noalloc_graph_replay(k3):
    """Captured in a HIP graph (what callers that cannot allocate do), two
    calls of 4 and 1 tokens replay to the eager outputs, with eager calls that
    overwrite the scratch array in between."""
    from synth.device import host_weights_to_device
    cfg = synth.CONFIGS[1]
    W = synth.gen_weights(cfg)
    wr = synth.gen_router_w(cfg)
    dw = k3.pack_layer_weights(host_weights_to_device(W, wr, None), cfg.E, cfg.d, cfg.f)
    c = k3.Config(cfg.d, cfg.E, cfg.k, cfg.f, 4)
    x = synth.gen_x(cfg, T=9, stream=20)
    xa, xb, xo = _xd(x[:4]), _xd(x[4:5]), _xd(x[5:9])
    oa, ob = _outs(cfg, 4), _outs(cfg, 1)
    k3.k3moe_layer_forward_noalloc(c, dw, xa, *oa)
    k3.k3moe_layer_forward_noalloc(c, dw, xb, *ob)
    torch.cuda.synchronize()
    ref = [tuple(t.clone() for t in o) for o in (oa, ob)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        k3.k3moe_layer_forward_noalloc(c, dw, xa, *oa)
        k3.k3moe_layer_forward_noalloc(c, dw, xb, *ob)
    other = _outs(cfg, 4)
    for rep in range(3):
        for o in (oa, ob):
            o[0].fill_(float("nan"))
            o[1].fill_(-7)
            o[2].fill_(float("nan"))
        k3.k3moe_layer_forward_noalloc(c, dw, xo, *other)  # eager use of the same scratch
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, r in zip((oa, ob), ref):
            assert all(torch.equal(a, b) for a, b in zip(o, r)), f"replay {rep} differs"
    del graph


def test_noalloc_refusals(k3):
    """Refused before anything runs: more than 4 tokens, a shape whose scratch
    exceeds the 2 MiB array, T above max_tokens, only one of idx/gate."""
    dummy = {n: torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
             for n in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")}
    dummy["router_w"] = torch.zeros(1 << 14, dtype=torch.float32, device="cuda")
    dummy["router_b"] = None
    x = torch.zeros((5, 4096), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((5, 4096), dtype=torch.float32, device="cuda")
    cases = [
        (k3.Config(2048, 64, 8, 1024, 8), 5, k3.K3MOE_EUNSUPPORTED),     # T > 4
        (k3.Config(4096, 4096, 64, 4096, 4), 4, k3.K3MOE_EUNSUPPORTED),  # 4.06 MiB of scratch
        (k3.Config(2048, 64, 8, 1024, 2), 3, k3.K3MOE_EINVAL),           # T > max_tokens
    ]
    for cfg, T, want in cases:
        with pytest.raises(k3.K3MoEError) as ei:
            k3.k3moe_layer_forward_noalloc(cfg, dummy, x[:T, :cfg.d_model].contiguous(),
                                           y[:T, :cfg.d_model].contiguous())
        assert ei.value.status == want, (cfg, T)
    idx = torch.zeros((1, 8), dtype=torch.int32, device="cuda")
    with pytest.raises(k3.K3MoEError) as ei:
        k3.k3moe_layer_forward_noalloc(k3.Config(2048, 64, 8, 1024, 4), dummy,
                                       x[:1, :2048].contiguous(), y[:1, :2048].contiguous(),
                                       topk_idx=idx)
    assert ei.value.status == k3.K3MOE_EINVAL
