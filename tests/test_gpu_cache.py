"""GPU tests of the HBM expert cache (k3moe_cache_*): expert weights in host
memory, n_slots of them resident in HBM, replaced least-recently-used.

The cached layer runs the same kernels on the same data as the all-resident
layer, so its outputs must equal k3moe_layer_forward bit for bit; the hit and
miss counts must follow the LRU rule exactly; and one output is checked
against the C oracle as well."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests._parity import check_output

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


def _layers(k3, cfg, max_tokens, n_slots, bias=None):
    from synth.device import host_weights_to_device
    W = synth.gen_weights(cfg)
    wr = synth.gen_router_w(cfg)
    dw = k3.pack_layer_weights(host_weights_to_device(W, wr, bias), cfg.E, cfg.d, cfg.f)
    host = {n: dw[n].cpu().pin_memory() for n in EXPERT_TENSORS}
    host["router_w"] = dw["router_w"]
    host["router_b"] = dw["router_b"]
    c = k3.Config(cfg.d, cfg.E, cfg.k, cfg.f, max_tokens)
    full = k3.Layer(c, dw, 0)
    cached = k3.CachedLayer(c, host, n_slots, 0)
    return W, wr, full, cached


def _xd(x_bits):
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda().view(torch.bfloat16)


@pytest.mark.parametrize("T", [1, 3, 12])
def test_cached_equals_resident_layer(k3, T):
    """Calls that hit, miss and evict give exactly the all-resident outputs
    (GEMV path for T <= 4, grouped GEMM above)."""
    cfg = synth.CONFIGS[1]  # 64 experts, top-8
    n_slots = min(cfg.E, max(24, T * cfg.k))
    _, _, full, cached = _layers(k3, cfg, 16, n_slots)
    pool = synth.gen_x(cfg, T=T * 10, stream=10)
    for i in range(10):
        x = _xd(pool[i * T:(i + 1) * T])
        y0, i0, g0 = full.forward(x)
        y1, i1, g1 = cached.forward(x)
        torch.cuda.synchronize()
        assert torch.equal(i0, i1) and torch.equal(g0, g1), f"call {i}: routing differs"
        assert torch.equal(y0, y1), f"call {i}: output differs"
    st = cached.stats()
    assert st["calls"] == 10
    assert st["misses"] > 0 and st["hits"] > 0
    cached.close()
    full.close()


def test_lru_accounting(k3):
    """Hit/miss counts against a host model of the LRU rule, with a cache
    smaller than the experts the calls touch."""
    cfg = synth.CONFIGS[1]
    n_slots = 20
    _, _, full, cached = _layers(k3, cfg, 4, n_slots)
    pool = synth.gen_x(cfg, T=40, stream=11)
    resident, last, hits, misses = {}, {}, 0, 0  # expert -> slot, slot -> last call
    for call in range(1, 21):
        x = _xd(pool[2 * (call - 1):2 * call])
        _, idx, _ = cached.forward(x)
        torch.cuda.synchronize()
        uniq = list(dict.fromkeys(int(e) for e in idx.cpu().numpy().reshape(-1)))
        for e in uniq:
            if e in resident:
                hits += 1
                last[resident[e]] = call
        for e in uniq:
            if e in resident:
                continue
            free = [s for s in range(n_slots) if last.get(s, 0) < call]
            v = min(free, key=lambda s: (last.get(s, 0), s))
            for old, s in list(resident.items()):
                if s == v:
                    del resident[old]
            resident[e] = v
            last[v] = call
            misses += 1
    st = cached.stats()
    assert (st["hits"], st["misses"]) == (hits, misses)
    assert st["bytes_in"] == misses * cfg.expert_bytes()
    cached.close()
    full.close()


def test_cached_layer_against_oracle(k3):
    cfg = synth.CONFIGS[1]
    W, wr, full, cached = _layers(k3, cfg, 8, 16)
    x = synth.gen_x(cfg, T=2, stream=12)
    for _ in range(2):  # the second call hits
        y, idx, gate = cached.forward(_xd(x))
    torch.cuda.synchronize()
    ref = oracle.layer_forward(x, wr, None, synth.ExpertSource(cfg, W), cfg.k)
    assert np.array_equal(idx.cpu().numpy(), ref["idx"])
    check_output(y.cpu().numpy(), ref["y64"], "cached layer")
    cached.close()
    full.close()


def test_too_many_distinct_experts_is_refused(k3):
    """A call that routes to more distinct experts than there are slots is
    refused after routing, before any expert is copied or computed; the
    cache keeps working afterwards."""
    cfg = synth.CONFIGS[1]
    _, _, full, cached = _layers(k3, cfg, 16, 8)  # 8 slots, top-8
    x = synth.gen_x(cfg, T=16, stream=13)
    with pytest.raises(k3.K3MoEError) as ei:
        cached.forward(_xd(x))
    assert ei.value.status == k3.K3MOE_EUNSUPPORTED
    assert cached.stats() == {"calls": 0, "hits": 0, "misses": 0, "bytes_in": 0,
                              "prefetched": 0, "prefetch_hits": 0}
    y0, _, _ = full.forward(_xd(x[:1]))
    y1, _, _ = cached.forward(_xd(x[:1]))
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    cached.close()
    full.close()


def test_cache_create_rejects_bad_arguments(k3):
    cfg = synth.CONFIGS[1]
    c = k3.Config(cfg.d, cfg.E, cfg.k, cfg.f, 4)
    host = {n: torch.zeros(16, dtype=torch.uint8) for n in EXPERT_TENSORS}
    host["router_w"] = torch.zeros((cfg.E, cfg.d), dtype=torch.float32, device="cuda")
    for n_slots in (cfg.k - 1, cfg.E + 1):  # fewer slots than top-k, more than experts
        with pytest.raises(k3.K3MoEError) as ei:
            k3.CachedLayer(c, host, n_slots, 0)
        assert ei.value.status == k3.K3MOE_EINVAL
    bad = dict(host)
    bad["down_s"] = None
    with pytest.raises(k3.K3MoEError) as ei:
        k3.CachedLayer(c, bad, 16, 0)
    assert ei.value.status == k3.K3MOE_EINVAL


@pytest.mark.timeout(600)
def test_cached_k3_decode_equals_resident(k3):
    """K3 shape (896 experts, 21 GB of MXFP4 experts in pinned host memory)
    behind a 64-slot arena: decode steps that miss and evict give exactly the
    resident layer's outputs, with and without a prefetch of the next step
    overlapping the current one."""
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
    cached = k3.CachedLayer(c, host, 64, 0)
    xp = device_x(cfg, T=16, stream=10, device=torch.device("cuda:0"))
    for i in range(8):
        y0, i0, _ = full.forward(xp[i:i + 1])
        y1, i1, _ = cached.forward(xp[i:i + 1])
        torch.cuda.synchronize()
        assert torch.equal(i0, i1) and torch.equal(y0, y1), f"token {i}"
    st = cached.stats()
    assert st["calls"] == 8 and st["misses"] >= 64  # the arena was refilled
    # then 8 more decode steps, each prefetched on a copy stream while the
    # previous step's expert kernels run
    xs = [xp[i:i + 1] for i in range(8, 16)]
    refs = [full.forward(x) for x in xs]
    torch.cuda.synchronize()
    st, new = _prefetch_overlapped(cached, xs, refs, cfg)
    assert new > 0
    cached.close()
    full.close()
    del dw, host
    torch.cuda.empty_cache()


def _prefetch_overlapped(cached, xs, refs, cfg):
    """Call n + 1's experts are prefetched on a copy stream right after call n
    is enqueued, while call n's expert kernels may still run (its kernels read
    the slots the prefetch must not overwrite); no synchronisation until the
    last call. Every output must equal the resident layer's bit for bit.
    After the first call nothing is missed, every prefetched expert is a
    prefetch hit, and raw hits (all) exceed true resident hits (hits minus
    prefetch hits) by exactly those."""
    lists = [r[1].cpu().numpy().reshape(-1).tolist() for r in refs]  # host, before the calls
    copy = torch.cuda.Stream()
    torch.cuda.synchronize()
    start = cached.stats()
    outs = [cached.forward(xs[0])]
    after_first = cached.stats()
    for n in range(1, len(xs)):
        cached.prefetch(lists[n], stream=copy)
        outs.append(cached.forward(xs[n]))
    torch.cuda.synchronize()
    for n, ((y, idx, gate), (ry, ri, rg)) in enumerate(zip(outs, refs)):
        assert torch.equal(idx, ri) and torch.equal(gate, rg), f"call {n}: routing differs"
        assert torch.equal(y, ry), f"call {n}: output differs"
    st = cached.stats()
    assert st["misses"] == after_first["misses"], "a prefetched expert was missed"
    assert st["hits"] - after_first["hits"] == sum(len(set(li)) for li in lists[1:])
    new = st["prefetched"] - start["prefetched"]
    assert st["prefetch_hits"] - start["prefetch_hits"] == new
    assert st["bytes_in"] - after_first["bytes_in"] == new * cfg.expert_bytes()
    return st, new


def test_prefetch_ahead_on_a_copy_stream(k3):
    """Small shape (64 experts, top-8, 40 slots), 12 calls of 2 tokens."""
    cfg = synth.CONFIGS[1]
    T, n_calls = 2, 12
    _, _, full, cached = _layers(k3, cfg, 8, 40)
    pool = synth.gen_x(cfg, T=T * n_calls, stream=14)
    xs = [_xd(pool[i * T:(i + 1) * T]) for i in range(n_calls)]
    refs = [full.forward(x) for x in xs]
    torch.cuda.synchronize()
    st, new = _prefetch_overlapped(cached, xs, refs, cfg)
    assert new > 0 and st["hits"] - st["prefetch_hits"] > 0
    cached.close()
    full.close()


def test_prefetch_refusals(k3):
    """Invalid ids are refused; an empty list does nothing; a prefetch that
    needs more slots than those the last call leaves free is refused with
    nothing changed, and the cache keeps working."""
    cfg = synth.CONFIGS[1]
    n_slots = 20  # a call of 2 tokens uses at most 16: at least 4 stay free
    _, _, full, cached = _layers(k3, cfg, 8, n_slots)
    for bad in ([cfg.E], [-1], [0, cfg.E + 5]):
        with pytest.raises(k3.K3MoEError) as ei:
            cached.prefetch(bad)
        assert ei.value.status == k3.K3MOE_EINVAL
    cached.prefetch([])
    x = _xd(synth.gen_x(cfg, T=2, stream=15))
    _, idx, _ = cached.forward(x)
    torch.cuda.synchronize()
    used = set(idx.cpu().numpy().reshape(-1).tolist())
    others = [e for e in range(cfg.E) if e not in used]
    before = cached.stats()
    with pytest.raises(k3.K3MoEError) as ei:
        cached.prefetch(others[:n_slots - len(used) + 1])
    assert ei.value.status == k3.K3MOE_EUNSUPPORTED
    assert cached.stats() == before
    free = n_slots - len(used)
    cached.prefetch(others[:free])  # exactly the free slots
    # listed resident experts are refreshed, which takes their slots: the
    # free ones refreshed leave no slot for one more expert
    filled = cached.stats()
    with pytest.raises(k3.K3MoEError) as ei:
        cached.prefetch(others[:free] + [others[free]])
    assert ei.value.status == k3.K3MOE_EUNSUPPORTED
    assert cached.stats() == filled
    cached.prefetch(others[1:free] + [others[free]])  # one slot left by the refresh
    y0, _, _ = full.forward(x)
    y1, _, _ = cached.forward(x)  # its experts are still resident
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    st = cached.stats()
    assert st["misses"] == before["misses"] and st["prefetch_hits"] == 0
    assert st["prefetched"] == free + 1
    cached.close()
    full.close()


def test_layer_stack_route_ahead_prefetch(k3):
    """Four layers (each its own seeded weights, 64 experts, top-8) with their
    experts in host memory behind 24-slot arenas, joined by a residual update
    (x + 0.25 y at x's RMS, in bf16). While layer l runs, layer l+1's experts
    are predicted by routing layer l's input through layer l+1's router on a
    side stream and prefetched on a copy stream (the last layer predicts the
    next step's layer 0). Every layer's output of every step equals the
    all-resident stack's bit for bit; prefetched experts are hit, and the true
    resident hits (hits minus prefetch hits) stay below the raw ones."""
    import dataclasses
    from synth.device import host_weights_to_device
    base = synth.CONFIGS[1]
    L, T, steps, alpha = 4, 2, 8, 0.25
    c = k3.Config(base.d, base.E, base.k, base.f, T)
    full, cached, routers = [], [], []
    stub = torch.zeros(256, dtype=torch.uint8, device="cuda")
    for l in range(L):
        cfg = dataclasses.replace(base, seed=base.seed + 100 * (l + 1))
        _, _, f_l, c_l = _layers(k3, cfg, T, 40)
        full.append(f_l)
        cached.append(c_l)
        wr = synth.gen_router_w(cfg)
        routers.append(k3.Layer(c, dict({n: stub for n in EXPERT_TENSORS},
                                        router_w=torch.from_numpy(wr).cuda(), router_b=None), 0))

    def update(x, y):
        xf = x.float()
        rx = xf.pow(2).mean(dim=-1, keepdim=True).sqrt()
        ry = y.pow(2).mean(dim=-1, keepdim=True).sqrt().clamp_min(1e-30)
        return (xf + y * (alpha * rx / ry)).to(torch.bfloat16)

    pool = [_xd(x) for x in np.split(synth.gen_x(base, T=T * (steps + 1), stream=22), steps + 1)]
    ref = []
    for i in range(steps):
        x, ys = pool[i], []
        for l in range(L):
            y, _, _ = full[l].forward(x)
            ys.append(y)
            x = update(x, y)
        ref.append(ys)
    torch.cuda.synchronize()
    route_st, copy_st = torch.cuda.Stream(), torch.cuda.Stream()
    ridx = torch.empty((T, base.k), dtype=torch.int32, device="cuda")
    rgate = torch.empty((T, base.k), dtype=torch.float32, device="cuda")
    out = []
    for i in range(steps):
        x, ys = pool[i], []
        for l in range(L):
            y, _, _ = cached[l].forward(x)
            ys.append(y)
            nl, nx = (l + 1, x) if l + 1 < L else (0, pool[i + 1])
            with torch.cuda.stream(route_st):
                route_st.wait_stream(torch.cuda.current_stream())
                k3.k3moe_route(routers[nl].handle, nx, ridx, rgate, stream=route_st)
                guess = ridx.cpu().reshape(-1).tolist()
            cached[nl].prefetch(guess, stream=copy_st)
            x = update(x, y)
        out.append(ys)
    torch.cuda.synchronize()
    for i in range(steps):
        for l in range(L):
            assert torch.equal(out[i][l], ref[i][l]), f"step {i} layer {l}: output differs"
    for l in range(L):
        st = cached[l].stats()
        assert st["prefetched"] > 0 and st["prefetch_hits"] > 0, (l, st)
        assert st["hits"] - st["prefetch_hits"] < st["hits"], (l, st)
    for obj in full + cached + routers:
        obj.close()
