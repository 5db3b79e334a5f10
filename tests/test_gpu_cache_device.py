"""GPU tests of the device-planned expert cache (k3moe_cache_create_ex with
K3MOE_CACHE_DEVICE_PLAN): the residency tables live in device memory, a
one-workgroup kernel plans each call and a fill kernel copies the missing
experts from pinned host memory, so a forward is only enqueued.

Its outputs must equal the all-resident layer's bit for bit, and its counts
(hits, misses, prefetches and prefetch hits) must equal the host-planned
cache's on the same calls: both follow one replacement rule, and the
host-planned cache is itself checked against a Python model of the rule
(test_gpu_cache.py). Calls captured into a HIP graph are replayed several
times, with eager work in between, and every replay is checked."""
from __future__ import annotations

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

EXPERT_TENSORS = ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")


@pytest.fixture(scope="module")
def k3():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp4_expert_matmul_amd as k3m
    k3m.load_library()
    return k3m


def _host_weights(dw):
    host = {n: dw[n].cpu().pin_memory() for n in EXPERT_TENSORS}
    host["router_w"] = dw["router_w"]
    host["router_b"] = dw.get("router_b")
    return host


def _setup(k3, cfg, max_tokens, n_slots):
    """The resident layer, a device-planned cache and a host-planned one
    (the model of the counts) over the same host tensors."""
    from synth.device import host_weights_to_device
    W = synth.gen_weights(cfg)
    wr = synth.gen_router_w(cfg)
    dw = k3.pack_layer_weights(host_weights_to_device(W, wr, None), cfg.E, cfg.d, cfg.f)
    host = _host_weights(dw)
    c = k3.Config(cfg.d, cfg.E, cfg.k, cfg.f, max_tokens)
    full = k3.Layer(c, dw, 0)
    dev = k3.CachedLayer(c, host, n_slots, 0, device_plan=True)
    model = k3.CachedLayer(c, host, n_slots, 0)
    return full, dev, model, host


def _xd(x_bits):
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda().view(torch.bfloat16)


def _close(*objs):
    for o in objs:
        o.close()


def _same(y_ref, y):
    return torch.equal(y_ref[0], y[0]) and torch.equal(y_ref[1], y[1]) and torch.equal(y_ref[2], y[2])


@pytest.mark.parametrize("T", [1, 3, 6])
def test_device_planned_equals_resident_and_host_counts(k3, T):
    """Calls that hit, miss and evict (GEMV path for T <= 4, grouped GEMM
    above), enqueued back to back with no synchronisation: every output
    equals the resident layer's, and the counts equal the host-planned
    cache's."""
    cfg = synth.CONFIGS[1]  # 64 experts, top-8
    n_slots = max(24, T * cfg.k)
    full, dev, model, _ = _setup(k3, cfg, 8, n_slots)
    pool = synth.gen_x(cfg, T=T * 12, stream=10)
    xs = [_xd(pool[i * T:(i + 1) * T]) for i in range(12)]
    refs = [full.forward(x) for x in xs]
    outs = [dev.forward(x) for x in xs]
    for x in xs:
        model.forward(x)
    torch.cuda.synchronize()
    for i, (r, o) in enumerate(zip(refs, outs)):
        assert _same(r, o), f"call {i} differs"
    st, ref = dev.stats(), model.stats()
    assert st == ref, (st, ref)
    assert st["calls"] == 12 and st["misses"] > 0 and st["hits"] > 0
    assert dev.device_counters() == {"refused_prefetches": 0, "ignored_ids": 0}
    _close(dev, model, full)


@pytest.mark.parametrize("flags", [0, 1], ids=["bias_added", "bias_select_only"])
def test_device_planned_skewed_bias(k3, flags):
    """The device-planned forward selects each token's experts inside its plan
    kernel: with the skewed router bias, added to the logits or used for the
    selection only (K3MOE_FLAG_BIAS_SELECT_ONLY), its idx, gates and outputs
    equal the resident layer's bit for bit, and its counts the host-planned
    cache's (GEMV and grouped paths)."""
    from synth.device import host_weights_to_device
    cfg = synth.LayerConfig("small_skew", 2048, 64, 8, 1024, 96, 5, skew_bias=True)
    assert flags in (0, k3.K3MOE_FLAG_BIAS_SELECT_ONLY)
    W = synth.gen_weights(cfg)
    dw = k3.pack_layer_weights(host_weights_to_device(W, synth.gen_router_w(cfg), synth.gen_bias(cfg)),
                               cfg.E, cfg.d, cfg.f)
    host = _host_weights(dw)
    c = k3.Config(cfg.d, cfg.E, cfg.k, cfg.f, 6, flags)
    full = k3.Layer(c, dw, 0)
    dev = k3.CachedLayer(c, host, 48, 0, device_plan=True)
    model = k3.CachedLayer(c, host, 48, 0)
    pool = synth.gen_x(cfg, T=40, stream=17)
    calls = [pool[0:1], pool[1:4], pool[4:10], pool[10:11], pool[11:17], pool[17:20]]
    for i, xb in enumerate(calls):
        x = _xd(xb)
        r = full.forward(x)
        o = dev.forward(x)
        model.forward(x)
        torch.cuda.synchronize()
        assert _same(r, o), f"call {i} (T={xb.shape[0]}) differs"
    st, ref = dev.stats(), model.stats()
    assert st == ref, (st, ref)
    _close(dev, model, full)


def test_device_planned_prefetch_overlapped(k3):
    """Call n + 1's experts, a device array, are prefetched on a copy stream
    right after call n is enqueued (call n's kernels may still run); no
    synchronisation until the end. Outputs equal the resident layer's; the
    counts equal the host-planned cache given the same lists; nothing is
    missed after the first call."""
    cfg = synth.CONFIGS[1]
    T, n_calls = 2, 12
    full, dev, model, _ = _setup(k3, cfg, 8, 40)
    pool = synth.gen_x(cfg, T=T * n_calls, stream=14)
    xs = [_xd(pool[i * T:(i + 1) * T]) for i in range(n_calls)]
    refs = [full.forward(x) for x in xs]
    lists_dev = [r[1].reshape(-1).contiguous() for r in refs]
    torch.cuda.synchronize()
    lists = [li.cpu().numpy().tolist() for li in lists_dev]
    copy = torch.cuda.Stream()
    outs = [dev.forward(xs[0])]
    for n in range(1, n_calls):
        dev.prefetch_device(lists_dev[n], stream=copy)
        outs.append(dev.forward(xs[n]))
    model.forward(xs[0])
    for n in range(1, n_calls):
        model.prefetch(lists[n])
        model.forward(xs[n])
    torch.cuda.synchronize()
    for n, (r, o) in enumerate(zip(refs, outs)):
        assert _same(r, o), f"call {n} differs"
    st, ref = dev.stats(), model.stats()
    assert st == ref, (st, ref)
    first_misses = len(set(lists[0]))
    assert st["misses"] == first_misses, "a prefetched expert was missed"
    assert st["prefetched"] > 0 and st["prefetch_hits"] == st["prefetched"]
    _close(dev, model, full)


def test_device_planned_graph_replay(k3):
    """Eight forwards (and a device prefetch between them) captured into one
    graph, replayed three times with eager calls and synchronisations in
    between: every replay's outputs equal the resident layer's, and after
    all of it the counts equal the host-planned cache's over the same
    sequence of calls."""
    cfg = synth.CONFIGS[1]
    T, K = 2, 8
    full, dev, model, _ = _setup(k3, cfg, 8, 40)  # a prefetch always finds 24 eligible slots
    pool = synth.gen_x(cfg, T=T * (K + 2), stream=16)
    xs = [_xd(pool[i * T:(i + 1) * T]) for i in range(K + 2)]
    refs = [full.forward(x) for x in xs]
    torch.cuda.synchronize()
    pf_list = refs[5][1].reshape(-1).contiguous()
    pf_host = pf_list.cpu().numpy().tolist()

    def model_sequence():
        for i in range(K):
            if i == 5:
                model.prefetch(pf_host)
            model.forward(xs[i])

    # eager warm-up on the capture stream, then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dev.forward(xs[K])
        model.forward(xs[K])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    outs = []
    with torch.cuda.graph(g, stream=s):
        for i in range(K):
            if i == 5:
                dev.prefetch_device(pf_list)
            outs.append(dev.forward(xs[i]))
    torch.cuda.synchronize()
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for i in range(K):
            assert _same(refs[i], outs[i]), f"replay {rep}, call {i} differs"
        model_sequence()
        # eager calls between the replays
        y = dev.forward(xs[K + 1])
        model.forward(xs[K + 1])
        torch.cuda.synchronize()
        assert _same(refs[K + 1], y), f"eager call after replay {rep} differs"
    st, ref = dev.stats(), model.stats()
    assert st == ref, (st, ref)
    assert st["calls"] == 1 + 3 * (K + 1)
    _close(dev, model, full)


def test_device_planned_refusals(k3):
    """Pageable host tensors and unknown flags are refused at create; a call
    with T * top_k above the slots is refused before anything runs; the
    host-list prefetch and the device-list prefetch each refuse the other
    kind of cache; a device prefetch that needs more slots than are eligible
    is refused on the device with nothing changed, and ids outside [0, E)
    are skipped and counted. The cache keeps working throughout."""
    cfg = synth.CONFIGS[1]
    n_slots = 20
    full, dev, model, host = _setup(k3, cfg, 8, n_slots)
    c = k3.Config(cfg.d, cfg.E, cfg.k, cfg.f, 8)
    pageable = dict(host)
    pageable["down_s"] = host["down_s"].clone()  # not pinned
    assert not pageable["down_s"].is_pinned()
    with pytest.raises(k3.K3MoEError) as ei:
        k3.CachedLayer(c, pageable, n_slots, 0, device_plan=True)
    assert ei.value.status == k3.K3MOE_EINVAL
    lib = k3.load_library()
    import ctypes
    out = ctypes.c_void_p()
    w = k3._binding._Weights(*[host.get(n).data_ptr() if host.get(n) is not None else None
                               for n, _ in k3._binding._Weights._fields_])
    assert lib.k3moe_cache_create_ex(ctypes.byref(c._c()), ctypes.byref(w), n_slots, 0, 6,
                                      ctypes.byref(out)) == k3.K3MOE_EINVAL
    x3 = _xd(synth.gen_x(cfg, T=3, stream=15))  # 24 pairs > 20 slots
    with pytest.raises(k3.K3MoEError) as ei:
        dev.forward(x3)
    assert ei.value.status == k3.K3MOE_EUNSUPPORTED
    with pytest.raises(k3.K3MoEError) as ei:
        dev.prefetch([1, 2])
    assert ei.value.status == k3.K3MOE_EINVAL
    with pytest.raises(k3.K3MoEError) as ei:
        model.prefetch_device(torch.tensor([1, 2], dtype=torch.int32, device="cuda"))
    assert ei.value.status == k3.K3MOE_EINVAL
    assert dev.stats()["calls"] == 0
    x = x3[:2]
    r0 = full.forward(x)
    o0 = dev.forward(x)
    model.forward(x)
    torch.cuda.synchronize()
    assert _same(r0, o0)
    used = set(r0[1].cpu().numpy().reshape(-1).tolist())
    others = [e for e in range(cfg.E) if e not in used]
    free = n_slots - len(used)
    before = dev.stats()
    too_many = torch.tensor(others[:free + 1], dtype=torch.int32, device="cuda")
    dev.prefetch_device(too_many)
    assert dev.stats() == before
    assert dev.device_counters() == {"refused_prefetches": 1, "ignored_ids": 0}
    with pytest.raises(k3.K3MoEError):
        model.prefetch(others[:free + 1])
    # exactly the free slots, with two ids outside [0, E) skipped
    fits = torch.tensor([-1] + others[:free] + [cfg.E], dtype=torch.int32, device="cuda")
    dev.prefetch_device(fits)
    model.prefetch(others[:free])
    o1 = dev.forward(x)  # its experts are still resident
    model.forward(x)
    torch.cuda.synchronize()
    assert _same(r0, o1)
    assert dev.device_counters() == {"refused_prefetches": 1, "ignored_ids": 2}
    st, ref = dev.stats(), model.stats()
    assert st == ref, (st, ref)
    assert st["prefetched"] == free and st["misses"] == before["misses"]
    dev.prefetch_device(torch.empty(0, dtype=torch.int32, device="cuda"))  # does nothing
    _close(dev, model, full)


@pytest.mark.timeout(600)
def test_device_planned_k3_decode(k3):
    """K3 shape (896 experts, 21 GB of MXFP4 experts in pinned host memory)
    behind a 64-slot arena: eight device-planned decode steps equal the
    resident layer's, then eight more captured into a graph with a
    route-ahead device prefetch of each next step, replayed twice; the counts
    equal the host-planned cache's over the same calls."""
    from synth.device import device_weights, device_x
    cfg = synth.CONFIGS[2]
    dw = device_weights(cfg, torch.device("cuda:0"))
    host = {}
    for n in EXPERT_TENSORS:
        h = torch.empty(dw[n].numel(), dtype=torch.uint8, pin_memory=True)
        h.copy_(dw[n].view(-1))
        host[n] = h
    host["router_w"] = dw["router_w"]
    host["router_b"] = dw.get("router_b")
    c = k3.Config(cfg.d, cfg.E, cfg.k, cfg.f, 1)
    full = k3.Layer(c, dw, 0)
    dev = k3.CachedLayer(c, host, 64, 0, device_plan=True)
    model = k3.CachedLayer(c, host, 64, 0)
    xp = device_x(cfg, T=17, stream=10, device=torch.device("cuda:0"))
    xs = [xp[i:i + 1] for i in range(17)]
    refs = [full.forward(x) for x in xs]
    torch.cuda.synchronize()
    outs = [dev.forward(xs[i]) for i in range(8)]
    for i in range(8):
        model.forward(xs[i])
    torch.cuda.synchronize()
    for i in range(8):
        assert _same(refs[i], outs[i]), f"token {i}"
    lists = [r[1].reshape(-1).contiguous() for r in refs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    gouts = []
    with torch.cuda.graph(g, stream=s):
        for i in range(8, 16):
            gouts.append(dev.forward(xs[i]))
            dev.prefetch_device(lists[i + 1])
    torch.cuda.synchronize()
    for rep in range(2):
        g.replay()
        torch.cuda.synchronize()
        for j, i in enumerate(range(8, 16)):
            assert _same(refs[i], gouts[j]), f"replay {rep}, token {i}"
        for i in range(8, 16):
            model.forward(xs[i])
            model.prefetch(lists[i + 1].cpu().numpy().tolist())
        torch.cuda.synchronize()
    st, ref = dev.stats(), model.stats()
    assert st == ref, (st, ref)
    assert st["calls"] == 24 and st["misses"] >= 64 and st["prefetched"] > 0
    _close(dev, model, full)
    del dw, host
    torch.cuda.empty_cache()
