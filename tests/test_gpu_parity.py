"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle on
seeded synthetic workloads: the five layer shapes (tiny, small, K3-scale
decode, prefill chunk, long skewed prefill) plus ragged and edge cases."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests._parity import check_output, compare_routing

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def k3():
    _require_gpu()
    import mxfp4_expert_matmul_amd as k3m
    k3m.load_library()  # raises if the HIP library was not built
    return k3m


GATE_TOL = 4e-5
TILE_M = 96  # tokens per tile of the grouped expert GEMM (kTileM in the kernels)


def _say(msg):
    print(msg, flush=True)


class Small:
    """A small layer fully resident on host (oracle) and device."""

    def __init__(self, cfg, max_tokens):
        import mxfp4_expert_matmul_amd as k3m
        from synth.device import host_weights_to_device
        self.cfg = cfg
        self.W = synth.gen_weights(cfg)
        self.wr = synth.gen_router_w(cfg)
        self.bias = synth.gen_bias(cfg)
        self.src = synth.ExpertSource(cfg, self.W)
        rowmajor = host_weights_to_device(self.W, self.wr, self.bias)
        self.dw = k3m.pack_layer_weights(rowmajor, cfg.E, cfg.d, cfg.f)


def _layer(k3, cfg, dw, max_tokens, flags=0):
    c = k3.Config(cfg.d, cfg.E, cfg.k, cfg.f, max_tokens, flags)
    return k3.Layer(c, dw, 0)


def _x_dev(x_bits):
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda().view(torch.bfloat16)


def _run_and_check(k3, layer, cfg, x_bits, src, wr, bias, tokens=None, label="",
                   select_only=False):
    """Full forward on the GPU; routing check on every token, output check on
    `tokens` (all if None). select_only: the layer uses the selection-only
    bias (the bias ranks the experts, the gates come from unbiased logits)."""
    T = x_bits.shape[0]
    y, idx, gate = layer.forward(_x_dev(x_bits))
    torch.cuda.synchronize()
    y, idx, gate = y.cpu().numpy(), idx.cpu().numpy(), gate.cpu().numpy()
    logits = oracle.router_logits(x_bits, wr, bias)
    if select_only:
        ridx, rgate = oracle.topk_gates(logits, cfg.k,
                                        gate_logits=oracle.router_logits(x_bits, wr, None))
    else:
        ridx, rgate = oracle.topk_gates(logits, cfg.k)
    excused, log = compare_routing(idx, logits, ridx, cfg.k)
    for line in log:
        _say(f"[{label}] {line}")
    ok = np.setdiff1d(np.arange(T), excused)
    gerr = float(np.max(np.abs(gate[ok] - rgate[ok]))) if len(ok) else 0.0
    _say(f"[{label}] max |gate - ref| = {gerr:.3e}")
    # gates: |dg_j| <= 2 max|dl| for softmax; fp32 router sums over d terms
    # are within GATE_TOL / 2 of the exact logits at these sizes
    assert gerr <= GATE_TOL, f"{label}: gate error {gerr}"
    assert np.all(np.abs(gate.astype(np.float64).sum(axis=1) - 1.0) <= 1e-5)
    check = np.arange(T) if tokens is None else np.asarray(tokens)
    use_idx = np.where(np.isin(np.arange(T), excused)[:, None], idx, ridx)[check]
    use_gate = np.where(np.isin(np.arange(T), excused)[:, None], gate.astype(np.float64), rgate)[check]
    yref = oracle.experts_forward(x_bits[check], use_idx, use_gate, src)
    ratio = check_output(y[check], yref, label)
    _say(f"[{label}] T={T} checked {len(check)} tokens, max|err|/rms = {ratio:.3e}, excused {len(excused)}")
    if len(check) > 1:
        rms = float(np.sqrt(np.mean(yref ** 2)))
        per = np.max(np.abs(y[check].astype(np.float64) - yref), axis=1) / rms
        worst = np.argsort(-per)[:8]
        _say(f"[{label}] worst tokens (token: max|err|/rms): "
             + ", ".join(f"{int(check[i])}: {per[i]:.2e}" for i in worst))
    return y, idx, gate


# ----------------------------------------------------------------- generator

def _tiled_reference(codes, scales, R, K):
    """The tiled layout written out from its definition in k3moe.h (numpy)."""
    n = codes.shape[0]
    RT, KT = R // 16, K // 128
    KG = (KT + 3) // 4
    tc = np.zeros((n, RT, KT, 64, 16), dtype=np.uint8)
    ts = np.full((n, RT, KG, 64, 4), 127, dtype=np.uint8)
    for lane in range(64):
        r, g = lane % 16, lane // 16
        for rt in range(RT):
            row = 16 * rt + r
            for kt in range(KT):
                tc[:, rt, kt, lane, :] = codes[:, row, 64 * kt + 16 * g: 64 * kt + 16 * g + 16]
                ts[:, rt, kt // 4, lane, kt % 4] = scales[:, row, 4 * kt + g]
    return tc.reshape(-1), ts.reshape(-1)


def test_pack_matches_layout_definition(k3):
    rng = np.random.default_rng(5)
    for n, R, K in [(2, 32, 128), (1, 48, 640), (3, 16, 512)]:
        codes = rng.integers(0, 256, (n, R, K // 2), dtype=np.uint8)
        scales = rng.integers(0, 256, (n, R, K // 32), dtype=np.uint8)
        tc, ts = k3.pack_mxfp4(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), n, R, K)
        torch.cuda.synchronize()
        wc, ws = _tiled_reference(codes, scales, R, K)
        assert np.array_equal(tc.cpu().numpy(), wc), (n, R, K)
        assert np.array_equal(ts.cpu().numpy(), ws), (n, R, K)


def test_pack_from_host_matches_layout_definition(k3):
    """Row-major matrices in host memory (numpy, and pinned CPU tensors) ->
    the tiled device layout, against the layout written out from its
    definition; a shape big enough to take several staging chunks against
    the device-side pack of the same bytes."""
    rng = np.random.default_rng(6)
    for n, R, K in [(2, 32, 128), (1, 48, 640), (3, 16, 512)]:
        codes = rng.integers(0, 256, (n, R, K // 2), dtype=np.uint8)
        scales = rng.integers(0, 256, (n, R, K // 32), dtype=np.uint8)
        wc, ws = _tiled_reference(codes, scales, R, K)
        for src in ("numpy", "pinned"):
            c_h, s_h = codes, scales
            if src == "pinned":
                c_h = torch.from_numpy(codes).pin_memory()
                s_h = torch.from_numpy(scales).pin_memory()
            tc, ts = k3.pack_mxfp4_from_host(c_h, s_h, n, R, K)
            assert np.array_equal(tc.cpu().numpy(), wc), (n, R, K, src)
            assert np.array_equal(ts.cpu().numpy(), ws), (n, R, K, src)
    n, R, K = 40, 1024, 4096  # 2 MB per matrix: three chunks of the 32 MiB staging buffer
    codes = rng.integers(0, 256, (n, R, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (n, R, K // 32), dtype=np.uint8)
    tc, ts = k3.pack_mxfp4_from_host(codes, scales, n, R, K)
    dc, ds = k3.pack_mxfp4(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), n, R, K)
    torch.cuda.synchronize()
    assert torch.equal(tc, dc) and torch.equal(ts, ds)
    bad = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(k3.K3MoEError) as ei:  # misaligned destination
        k3.k3moe_pack_mxfp4_from_host(codes, scales, 1, R, K, bad[1:], bad)
    assert ei.value.status == k3.K3MOE_EINVAL
    with pytest.raises(k3.K3MoEError) as ei:  # R not a multiple of 16
        k3.k3moe_pack_mxfp4_from_host(codes, scales, 1, 15, K, bad, bad)
    assert ei.value.status == k3.K3MOE_EINVAL


def test_device_generator_matches_host(k3):
    from synth.device import device_weights, host_weights_to_device
    cfg = synth.CONFIGS[1]
    W = synth.gen_weights(cfg)
    rowmajor = device_weights(cfg, tiled=False)
    for name, arr in W.items():
        assert np.array_equal(rowmajor[name].cpu().numpy(), arr), name
    assert np.array_equal(rowmajor["router_w"].cpu().numpy(), synth.gen_router_w(cfg))
    tiled = device_weights(cfg)
    packed = k3.pack_layer_weights(host_weights_to_device(W, synth.gen_router_w(cfg), None),
                                   cfg.E, cfg.d, cfg.f)
    for name in W:
        assert np.array_equal(tiled[name].cpu().numpy(), packed[name].cpu().numpy()), name


# ----------------------------------------------------------------- small layers

CUSTOM = synth.LayerConfig("ragged_d640_e16_k4_f384", 640, 16, 4, 384, 1, 11)
# k = 40: a decode wave walks five slots (h re-staged every second slot);
# f = 640 leaves a partial 4-tile chunk
WIDE_K = synth.LayerConfig("wide_k_d256_e64_k40_f640", 256, 64, 40, 640, 1, 12)
# f = 2304: the largest decode h staging (8 KB per slot) and a partial chunk
WIDE_F = synth.LayerConfig("wide_f_d256_e16_k4_f2304", 256, 16, 4, 2304, 1, 13)


@pytest.mark.parametrize("cfg,T", [
    (synth.CONFIGS[0], 1), (synth.CONFIGS[0], 3), (synth.CONFIGS[0], 5), (synth.CONFIGS[0], 130),
    (synth.CONFIGS[1], 1), (synth.CONFIGS[1], 4), (synth.CONFIGS[1], 9), (synth.CONFIGS[1], 256),
    (CUSTOM, 2), (CUSTOM, 77),
    (WIDE_K, 1), (WIDE_K, 3), (WIDE_K, 40), (WIDE_F, 1), (WIDE_F, 2), (WIDE_F, 33),
])
def test_layer_forward_small(k3, cfg, T):
    _say(f"case {cfg.name} T={T}")
    s = Small(cfg, T)
    layer = _layer(k3, cfg, s.dw, max(T, 8))
    x = synth.gen_x(cfg, T=T)
    _run_and_check(k3, layer, cfg, x, s.src, s.wr, s.bias, label=f"{cfg.name} T={T}")
    layer.close()


TOP1 = synth.LayerConfig("top1_d256_e16_k1_f256", 256, 16, 1, 256, 1, 14)
ALLK = synth.LayerConfig("allk_d256_e8_k8_f256", 256, 8, 8, 256, 1, 15)


@pytest.mark.parametrize("cfg", [TOP1, ALLK], ids=["k=1", "k=E"])
def test_routing_extremes(k3, cfg):
    """top-1: every gate is exactly 1.0; top-k = E: every expert is selected,
    in (logit desc, index asc) order, and the gates are a full softmax (sum 1).
    Outputs against the oracle on both paths."""
    s = Small(cfg, 24)
    layer = _layer(k3, cfg, s.dw, 24)
    for T in (1, 3, 24):
        x = synth.gen_x(cfg, T=T)
        _, idx, gate = _run_and_check(k3, layer, cfg, x, s.src, s.wr, s.bias,
                                      label=f"{cfg.name} T={T}")
        if cfg.k == 1:
            assert np.all(gate == 1.0), f"T={T}: top-1 gate is not exactly 1"
        else:
            assert np.all(np.sort(idx, axis=1) == np.arange(cfg.E)), f"T={T}: not every expert"
            assert np.all(np.abs(gate.astype(np.float64).sum(axis=1) - 1.0) < 1e-6)
    layer.close()


def test_skewed_bias_small(k3):
    cfg = synth.LayerConfig("small_skew", 2048, 64, 8, 1024, 96, 5, skew_bias=True)
    s = Small(cfg, 96)
    layer = _layer(k3, cfg, s.dw, 96)
    _run_and_check(k3, layer, cfg, synth.gen_x(cfg), s.src, s.wr, s.bias, label="small skew")
    layer.close()


class Custom(Small):
    """A small layer with caller-chosen weights (host and device)."""

    def __init__(self, cfg, W):
        import mxfp4_expert_matmul_amd as k3m
        from synth.device import host_weights_to_device
        self.cfg = cfg
        self.W = W
        self.wr = synth.gen_router_w(cfg)
        self.bias = None
        self.src = synth.ExpertSource(cfg, W)
        self.dw = k3m.pack_layer_weights(host_weights_to_device(W, self.wr, None), cfg.E, cfg.d, cfg.f)


EDGE = synth.LayerConfig("edge_d256_e8_k2_f256", 256, 8, 2, 256, 1, 21)


@pytest.mark.parametrize("T", [1, 3, 40])
def test_wide_scale_exponents(k3, T):
    """E8M0 scale bytes spread over 100..150 (2^-27 .. 2^23), far outside the
    workload's 123..127: the kernels' scale decoding and the MFMA scale
    operands must apply each block's own power of two (GEMV path for T <= 4,
    grouped GEMM above)."""
    cfg = EDGE
    W = synth.gen_weights(cfg)
    rng = np.random.default_rng(31)
    for name in ("gate_s", "up_s", "down_s"):
        W[name] = rng.integers(100, 151, W[name].shape).astype(np.uint8)
    s = Custom(cfg, W)
    layer = _layer(k3, cfg, s.dw, 64)
    x = synth.gen_x(cfg, T=T)
    y, _, _ = _run_and_check(k3, layer, cfg, x, s.src, s.wr, None, label=f"wide scales T={T}")
    assert np.all(np.isfinite(y))
    layer.close()


@pytest.mark.parametrize("cfg", [EDGE, synth.CONFIGS[1]], ids=lambda c: c.name)
@pytest.mark.parametrize("spread", [4, 16, 32, 51])
def test_scale_spread_sweep(k3, cfg, spread):
    """Grouped path (T = 40) with the weights' E8M0 scale bytes uniform over
    `spread` binades about 2^-2 (4: the generator's own spread; 51: the wide
    case above). The two-term activation split is exact to about 2^-8 of a
    block's largest value, so the output error grows as fewer blocks dominate
    each sum: the wider the spread and the fewer blocks per row (8 at d = 256,
    64 at d = 2048), the larger. Logged per case; each within the bar."""
    W = synth.gen_weights(cfg)
    rng = np.random.default_rng(37)
    lo = 125 - spread // 2
    for name in ("gate_s", "up_s", "down_s"):
        W[name] = rng.integers(lo, lo + spread, W[name].shape).astype(np.uint8)
    s = Custom(cfg, W)
    T = 40
    layer = _layer(k3, cfg, s.dw, T)
    x = synth.gen_x(cfg, T=T)
    y, _, _ = _run_and_check(k3, layer, cfg, x, s.src, s.wr, None,
                             label=f"scale spread {spread} {cfg.name}")
    assert np.all(np.isfinite(y))
    layer.close()


@pytest.mark.parametrize("T", [3, 64])
def test_activation_outlier_channels(k3, T):
    """Four hidden channels 32x larger than the rest (as real activations
    have): the two-term split keeps each element's own exponent, so the
    other values of an outlier's block keep their precision (GEMV path for
    T <= 4, grouped GEMM above)."""
    cfg = synth.CONFIGS[1]
    s = Small(cfg, T)
    layer = _layer(k3, cfg, s.dw, max(T, 8))
    xf = synth.bf16_bits_to_f32(synth.gen_x(cfg, T=T))
    ch = np.random.default_rng(41).choice(cfg.d, 4, replace=False)
    xf[:, ch] *= 32.0  # exact in bf16
    x = synth.f32_to_bf16_bits(xf)
    _run_and_check(k3, layer, cfg, x, s.src, s.wr, s.bias, label=f"outlier channels T={T}")
    layer.close()


class Biased(Small):
    """A small layer with the seeded weights and a caller-chosen router bias."""

    def __init__(self, cfg, bias):
        import mxfp4_expert_matmul_amd as k3m
        from synth.device import host_weights_to_device
        self.cfg = cfg
        self.W = synth.gen_weights(cfg)
        self.wr = synth.gen_router_w(cfg)
        self.bias = np.asarray(bias, dtype=np.float32)
        self.src = synth.ExpertSource(cfg, self.W)
        self.dw = k3m.pack_layer_weights(host_weights_to_device(self.W, self.wr, self.bias),
                                         cfg.E, cfg.d, cfg.f)


@pytest.mark.parametrize("T", [1, 3, 40])
def test_nan_router_bias_never_selected(k3, T):
    """NaN bias entries make those experts' logits NaN for every token; a NaN
    logit ranks as -inf, so with enough finite logits it is never selected,
    and routing, gates and outputs match the oracle (the top-k fused into the
    decode GEMV for T <= 4, the top-k kernel above). The NaN experts are the
    ones the bias would otherwise rank first."""
    cfg = synth.CONFIGS[1]
    bias = 0.5 * np.random.default_rng(61).standard_normal(cfg.E).astype(np.float32)
    nan_experts = np.concatenate([np.argsort(-bias)[:3], [0, 17, cfg.E - 1]])
    bias[nan_experts] = np.nan
    s = Biased(cfg, bias)
    layer = _layer(k3, cfg, s.dw, max(T, 8))
    x = synth.gen_x(cfg, T=T, stream=16)
    _, idx, _ = _run_and_check(k3, layer, cfg, x, s.src, s.wr, s.bias, label=f"NaN bias T={T}")
    assert not np.any(np.isin(idx, nan_experts)), "a NaN-logit expert was selected"
    layer.close()


@pytest.mark.parametrize("T", [1, 5])
def test_nan_router_bias_fewer_than_k_finite(k3, T):
    """Only one finite logit per token with k = 2: the second selection is the
    lowest-index NaN expert (NaN ties with -inf, lower index first) with gate
    exactly 0, and the output is the finite expert's alone."""
    cfg = EDGE
    bias = np.full(cfg.E, np.nan, dtype=np.float32)
    bias[5] = 0.25
    s = Biased(cfg, bias)
    layer = _layer(k3, cfg, s.dw, 8)
    x = synth.gen_x(cfg, T=T, stream=17)
    _, idx, gate = _run_and_check(k3, layer, cfg, x, s.src, s.wr, s.bias,
                                  label=f"one finite logit T={T}")
    assert np.all(idx == np.array([5, 0], dtype=np.int32))
    assert np.all(gate[:, 0] == 1.0) and np.all(gate[:, 1] == 0.0)
    layer.close()


def _check_with_nans(y_gpu, y_ref, label):
    """NaN positions must match exactly; finite outputs meet the parity bar
    against the RMS of the finite reference outputs."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    nan_g, nan_r = np.isnan(y_gpu), np.isnan(y_ref)
    assert np.array_equal(nan_g, nan_r), (f"{label}: NaN at {int(nan_g.sum())} outputs, "
                                          f"expected {int(nan_r.sum())}")
    fin = ~nan_r
    assert np.any(fin), f"{label}: no finite output to compare"
    assert np.all(np.isfinite(y_gpu[fin])), f"{label}: Inf where the reference is finite"
    rms = float(np.sqrt(np.mean(y_ref[fin] ** 2)))
    err = float(np.max(np.abs(y_gpu[fin] - y_ref[fin])))
    assert err <= 2e-2 * rms, f"{label}: max abs err {err:.4g} > 2e-2 * rms {rms:.4g}"
    return int(nan_r.sum()), err / rms


@pytest.mark.parametrize("T", [1, 3, 40])
def test_nan_scale_block_propagates(k3, T):
    """An E8M0 scale byte 0xFF (NaN) in one block: in row m of an expert's
    down projection it makes output m of the tokens routed there NaN and
    nothing else; in a row of another expert's gate projection, and of a
    third expert's up projection, it makes every output of their tokens NaN
    (through h). The NaN pattern equals the oracle's exactly, on the decode
    GEMV (T <= 4) and the grouped MFMA GEMM (T > 4)."""
    cfg = EDGE
    x = synth.gen_x(cfg, T=T, stream=18)
    wr = synth.gen_router_w(cfg)
    ridx, _ = oracle.topk_gates(oracle.router_logits(x, wr, None), cfg.k)
    used = list(dict.fromkeys(int(e) for e in ridx.reshape(-1)))
    W = synth.gen_weights(cfg)
    m0 = 37
    W["down_s"][used[0], m0, 3] = 0xFF  # token 0's first expert: its output m0 only
    # gate and up blocks on experts token 0 does not use, so its other
    # outputs stay finite
    others = [e for e in used if e not in ridx[0]]
    if len(others) > 0:
        W["gate_s"][others[0], 7, 2] = 0xFF
    if len(others) > 1:
        W["up_s"][others[1], 100, 5] = 0xFF
    s = Custom(cfg, W)
    layer = _layer(k3, cfg, s.dw, 64)
    y, idx, _ = layer.forward(_x_dev(x))
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ridx)
    yref = oracle.experts_forward(x, ridx, oracle.topk_gates(oracle.router_logits(x, wr, None), cfg.k)[1],
                                  s.src)
    n_nan, ratio = _check_with_nans(y.cpu().numpy(), yref, f"NaN scale T={T}")
    assert n_nan > 0
    _say(f"[NaN scale T={T}] {n_nan} NaN outputs as expected; finite max|err|/rms = {ratio:.3e}")
    layer.close()


@pytest.mark.parametrize("T", [1, 3, 40, 96])
def test_selection_only_bias(k3, T):
    """K3MOE_FLAG_BIAS_SELECT_ONLY with the skewed bias 2(rank+1)^-1.2 at the
    small shape: the bias ranks the experts, the gates are the softmax of the
    unbiased logits of the chosen ones. Routing, gates and outputs against the
    oracle's selection-only mode, on the fused decode top-k (T <= 4) and the
    top-k kernel with the grouped GEMM; the default mode on the same layer
    chooses the same experts with other gates."""
    cfg = synth.LayerConfig("small_skew_select_only", 2048, 64, 8, 1024, 96, 5, skew_bias=True)
    s = Small(cfg, 96)
    sel = _layer(k3, cfg, s.dw, 96, flags=k3.K3MOE_FLAG_BIAS_SELECT_ONLY)
    x = synth.gen_x(cfg, T=T, stream=21)
    _, idx, gate = _run_and_check(k3, sel, cfg, x, s.src, s.wr, s.bias, select_only=True,
                                  label=f"select-only bias T={T}")
    both = _layer(k3, cfg, s.dw, 96)
    _, idx2, gate2 = both.forward(_x_dev(x))
    torch.cuda.synchronize()
    assert np.array_equal(idx, idx2.cpu().numpy())
    assert np.max(np.abs(gate - gate2.cpu().numpy())) > 1e-3  # the bias no longer reaches the gates
    logits = torch.empty((T, cfg.E), dtype=torch.float32, device="cuda")
    i3 = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    g3 = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
    k3.k3moe_route(sel.handle, _x_dev(x), i3, g3, logits)
    torch.cuda.synchronize()
    raw = oracle.router_logits(x, s.wr, None)  # the route step reports unbiased logits
    assert np.max(np.abs(logits.cpu().numpy() - raw)) < 1e-4
    sel.close()
    both.close()


@pytest.mark.parametrize("code_byte", [0x00, 0x88])
def test_zero_codes_give_zero(k3, code_byte):
    """All codes +0 (0x00) or -0 (0x88): every output is exactly zero on both
    paths, whatever the scales."""
    cfg = EDGE
    W = synth.gen_weights(cfg)
    for name in ("gate_q", "up_q", "down_q"):
        W[name] = np.full_like(W[name], code_byte)
    s = Custom(cfg, W)
    layer = _layer(k3, cfg, s.dw, 64)
    for T in (1, 3, 40):
        y, idx, _ = layer.forward(_x_dev(synth.gen_x(cfg, T=T)))
        torch.cuda.synchronize()
        assert np.all(y.cpu().numpy() == 0.0), f"T={T}: non-zero output from zero weights"
    layer.close()


DEQ = synth.LayerConfig("dequant_d256_e2_k1_f256", 256, 2, 1, 256, 8, 5)


def _one_weight_matrices(test, i0):
    """Expert 0's weights for a one-hot x at column i0 (expert 1 all zero),
    testing one matrix's MXFP4 decode. Row n of the tested matrix holds code
    n % 16 (all 16 E2M1 codes, twice per 32 rows) at its one non-zero
    element, with scale byte base + n // 32 for that element's block.
      gate: g[n] = dq(n), u[n] = 1, down = identity -> y[n] = SiLU(dq(n));
      up:   g[n] = 96 (SiLU(96) = 96 in fp32), u[n] = dq(n), down = identity
            -> y[n] = 96 dq(n), exact in fp32;
      down: h[n] = 96, down row m holds dq(m) at column m -> y[m] = 96 dq(m).
    Returns the weights and the reference y (float64)."""
    cfg = DEQ
    d, f = cfg.d, cfg.f
    W = {"gate_q": np.zeros((2, f, d // 2), np.uint8), "up_q": np.zeros((2, f, d // 2), np.uint8),
         "down_q": np.zeros((2, d, f // 2), np.uint8),
         "gate_s": np.full((2, f, d // 32), 127, np.uint8), "up_s": np.full((2, f, d // 32), 127, np.uint8),
         "down_s": np.full((2, d, f // 32), 127, np.uint8)}
    base = {"gate": 128, "up": 120, "down": 112}[test]
    n = np.arange(f)
    codes, sbytes = n % 16, base + n // 32
    dq = np.array([oracle.e2m1_value(int(c)) * oracle.e8m0_value(int(b)) for c, b in zip(codes, sbytes)])

    def put(name, rows, col, code, sbyte):  # element (row, col) of matrix `name` of expert 0
        q, sc = W[name + "_q"], W[name + "_s"]
        rows, col = np.broadcast_arrays(rows, col)
        code = np.broadcast_to(np.asarray(code, np.uint8), rows.shape)
        byte = q[0, rows, col // 2]
        # low nibble = even element, high nibble = odd element
        q[0, rows, col // 2] = np.where(col % 2 == 0, (byte & 0xF0) | code, (byte & 0x0F) | (code << 4))
        sc[0, rows, col // 32] = sbyte

    if test == "gate":
        put("gate", n, i0, codes, sbytes)
        put("up", n, i0, 2, 127)          # 1.0
        put("down", n, n, 2, 127)         # identity
        with np.errstate(over="ignore"):  # exp(-dq) = inf for large negative dq: SiLU -> -0
            ref = dq / (1.0 + np.exp(-dq))
    elif test == "up":
        put("gate", n, i0, 7, 131)        # 6 * 16 = 96
        put("up", n, i0, codes, sbytes)
        put("down", n, n, 2, 127)
        ref = 96.0 * dq
    else:
        put("gate", n, i0, 7, 131)
        put("up", n, i0, 2, 127)
        put("down", n, n, codes, sbytes)  # row m: dq(m) at column m
        ref = 96.0 * dq
    return W, ref


@pytest.mark.parametrize("test", ["gate", "up", "down"])
def test_mxfp4_decode_every_code_on_gpu(k3, test):
    """The kernels' MXFP4 decode, matrix by matrix, for all 16 E2M1 codes
    (both signed zeros included) under 8 scale bytes each, through the GEMV
    (T = 1) and the grouped MFMA GEMM (T = 8): with a one-hot x every gate or
    up output is one dequantised weight, and the down projection reads one
    weight per output. Up and down outputs are exact products in fp32 (the
    two-term split represents them exactly), so both paths must match bit for
    bit; gate outputs pass through SiLU, checked to fp32 rounding on the GEMV
    and to the split's bound (relative to each 32-row block) on the GEMM."""
    cfg = DEQ
    i0 = 37
    W, ref = _one_weight_matrices(test, i0)
    s = Custom(cfg, W)
    layer = _layer(k3, cfg, s.dw, 8)
    for T in (1, 8):
        xb = np.zeros((T, cfg.d), np.uint16)
        xb[:, i0] = 0x3F80  # bf16 1.0
        idx = torch.zeros((T, 1), dtype=torch.int32, device="cuda")
        gate = torch.ones((T, 1), dtype=torch.float32, device="cuda")
        y = torch.empty((T, cfg.d), dtype=torch.float32, device="cuda")
        k3.k3moe_experts_forward(layer.handle, _x_dev(xb), idx, gate, y)
        torch.cuda.synchronize()
        yv = y.cpu().numpy().astype(np.float64)
        for t in range(T):
            if test != "gate":
                bad = np.flatnonzero(yv[t] != ref)
                assert bad.size == 0, f"T={T} {test}: rows {bad[:8]} give {yv[t][bad[:8]]}, want {ref[bad[:8]]}"
            else:
                blockmax = np.repeat(np.abs(ref).reshape(-1, 32).max(axis=1), 32)
                tol = (4e-7 * np.abs(ref) + 1e-7 * blockmax) if T == 1 else (2.0 ** -7 * np.abs(ref) + 2.0 ** -14 * blockmax)
                err = np.abs(yv[t] - ref)
                assert np.all(err <= tol), f"T={T} gate: worst row {int(np.argmax(err / tol))}"
    layer.close()


def test_batch_invariance(k3):
    """A token's output does not depend on the batch it is in (chunk-union
    prefill equals the per-token path). Within the grouped-GEMM path only the
    order of the fp32 scatter-adds differs between batches; across the GEMV
    (T <= 4) and GEMM paths the activation/h representations differ, so the
    bar there is the parity bar."""
    cfg = synth.CONFIGS[1]
    s = Small(cfg, 64)
    layer = _layer(k3, cfg, s.dw, 64)
    x = synth.gen_x(cfg, T=64)
    yb, ib, _ = layer.forward(_x_dev(x))
    yb, ib = yb.cpu().numpy(), ib.cpu().numpy()
    rms = np.sqrt(np.mean(yb.astype(np.float64) ** 2))
    perm = np.random.default_rng(2).permutation(64)[:37]
    yp, ip, _ = layer.forward(_x_dev(x[perm]))
    assert np.array_equal(ip.cpu().numpy(), ib[perm])
    same = np.max(np.abs(yp.cpu().numpy() - yb[perm]))
    _say(f"grouped path, other batch: max diff / rms = {same / rms:.3e}")
    assert same <= 1e-5 * rms
    for t in range(0, 64, 7):
        y1, i1, _ = layer.forward(_x_dev(x[t:t + 1]))
        assert np.array_equal(i1.cpu().numpy()[0], ib[t])
        assert np.max(np.abs(y1.cpu().numpy()[0] - yb[t])) <= 2e-2 * rms
    layer.close()


def _check_graph_replay(k3, layer, cfg, T):
    """Three forwards captured in one HIP graph (each with its own input and
    output buffers) and replayed three times, with eager forwards of the same
    layer in between, give exactly the eager outputs on every replay."""
    xs = [_x_dev(synth.gen_x(cfg, T=T, stream=10 + i)) for i in range(3)]
    outs = [(torch.empty((T, cfg.d), dtype=torch.float32, device="cuda"),
             torch.empty((T, cfg.k), dtype=torch.int32, device="cuda"),
             torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")) for _ in xs]
    ref = []
    for x, (y, i, g) in zip(xs, outs):
        k3.k3moe_layer_forward(layer.handle, x, y, i, g)
        torch.cuda.synchronize()
        ref.append((y.clone(), i.clone(), g.clone()))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for x, (y, i, g) in zip(xs, outs):
            k3.k3moe_layer_forward(layer.handle, x, y, i, g)
    other = _x_dev(synth.gen_x(cfg, T=5, stream=20))
    for rep in range(3):
        for y, i, g in outs:  # stale values must be overwritten by the replay
            y.fill_(float("nan"))
            i.fill_(-7)
            g.fill_(float("nan"))
        layer.forward(other)  # eager work on the same handle between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (y, i, g), (ry, ri, rg) in zip(outs, ref):
            assert torch.equal(i, ri) and torch.equal(g, rg), f"replay {rep}: routing differs"
            assert torch.equal(y, ry), f"replay {rep}: output differs"
    del graph


@pytest.mark.parametrize("T", [1, 3, 40])
def test_graph_replay_matches_eager(k3, T):
    """Graph replay equals eager (decode GEMV path for T <= 4, grouped path
    above: both deterministic)."""
    cfg = synth.CONFIGS[1]
    s = Small(cfg, 64)
    layer = _layer(k3, cfg, s.dw, 64)
    _check_graph_replay(k3, layer, cfg, T)
    layer.close()


@pytest.mark.parametrize("pattern", ["lanes_first", "all_tied", "random"])
def test_topk_selection_patterns(k3, pattern):
    """Top-k with E = 896 under logit patterns that take each branch of the
    selection: ranks concentrated in a few lanes of the 64-lane selection
    (more than 64 keys above the lower bound: the round-by-round branch), all
    logits tied (ties resolve to the lowest indices), and random. x = 0, so
    the logits are exactly the router bias."""
    from synth.device import host_weights_to_device
    cfg = synth.LayerConfig("topk_patterns", 128, 896, 16, 128, 4, 11)
    W = synth.gen_weights(cfg)
    wr = synth.gen_router_w(cfg)
    e = np.arange(cfg.E)
    if pattern == "lanes_first":
        # experts e = lane + 64 j rank by (lane, j): lanes 0, 1, ... hold the largest
        bias = (-0.01 * ((e % 64) * 14 + e // 64)).astype(np.float32)
    elif pattern == "all_tied":
        bias = np.full(cfg.E, 0.5, dtype=np.float32)
    else:
        bias = np.random.default_rng(5).standard_normal(cfg.E).astype(np.float32)
    dw = k3.pack_layer_weights(host_weights_to_device(W, wr, bias), cfg.E, cfg.d, cfg.f)
    layer = _layer(k3, cfg, dw, 8)
    x = np.zeros((cfg.T, cfg.d), dtype=np.uint16)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    gate = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    k3.k3moe_route(layer.handle, _x_dev(x), idx, gate)
    torch.cuda.synchronize()
    ridx, rgate = oracle.topk_gates(oracle.router_logits(x, wr, bias), cfg.k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.max(np.abs(gate.cpu().numpy() - rgate)) <= 1e-6
    layer.close()


def test_route_and_group_entry_points(k3):
    cfg = synth.CONFIGS[1]
    s = Small(cfg, 300)
    layer = _layer(k3, cfg, s.dw, 300)
    x = synth.gen_x(cfg, T=300)
    idx = torch.empty((300, cfg.k), dtype=torch.int32, device="cuda")
    gate = torch.empty((300, cfg.k), dtype=torch.float32, device="cuda")
    logits = torch.empty((300, cfg.E), dtype=torch.float32, device="cuda")
    k3.k3moe_route(layer.handle, _x_dev(x), idx, gate, logits)
    torch.cuda.synchronize()
    ref_logits = oracle.router_logits(x, s.wr, None)
    assert np.max(np.abs(logits.cpu().numpy() - ref_logits)) < 1e-4
    ridx, _ = oracle.topk_gates(ref_logits, cfg.k)
    compare_routing(idx.cpu().numpy(), ref_logits, ridx, cfg.k)
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(cfg.E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(300 * cfg.k, dtype=torch.int32, device="cuda")
    k3.k3moe_group(layer.handle, idx, counts, offsets, perm)
    torch.cuda.synchronize()
    rc, ro, rp = oracle.group_pairs(idx.cpu().numpy(), cfg.E)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(perm.cpu().numpy(), rp)
    layer.close()


@pytest.mark.parametrize("pattern", ["one_expert", "random", "empty", "invalid"])
def test_group_patterns(k3, pattern):
    cfg = synth.CONFIGS[1]
    s = Small(cfg, 1000)
    layer = _layer(k3, cfg, s.dw, 1000)
    rng = np.random.default_rng(3)
    T = 0 if pattern == "empty" else 1000
    if pattern == "one_expert":  # every token picks experts 0..k-1 (maximum skew)
        idx = np.tile(np.arange(cfg.k, dtype=np.int32), (T, 1))
    else:
        idx = np.array([rng.permutation(cfg.E)[:cfg.k] for _ in range(T)], dtype=np.int32).reshape(T, cfg.k)
    if pattern == "invalid":
        idx[5, 2] = -1
        idx[17, 0] = cfg.E
    counts = torch.full((cfg.E,), -7, dtype=torch.int32, device="cuda")
    offsets = torch.full((cfg.E + 1,), -7, dtype=torch.int32, device="cuda")
    perm = torch.full((max(T * cfg.k, 1),), -7, dtype=torch.int32, device="cuda")
    k3.k3moe_group(layer.handle, torch.from_numpy(idx).cuda(), counts, offsets, perm)
    torch.cuda.synchronize()
    valid = (idx >= 0) & (idx < cfg.E)
    flat = idx.reshape(-1)
    keep = valid.reshape(-1)
    rc = np.bincount(flat[keep], minlength=cfg.E)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(offsets.cpu().numpy(), np.concatenate([[0], np.cumsum(rc)]))
    n = int(rc.sum())
    want = np.nonzero(keep)[0][np.argsort(flat[keep], kind="stable")]
    assert np.array_equal(perm.cpu().numpy()[:n], want)
    layer.close()


def test_experts_forward_injected_routing(k3):
    """Caller routing, including one expert taking every token (max skew),
    and a dropped pair (expert index out of range contributes zero)."""
    cfg = synth.CONFIGS[1]
    s = Small(cfg, 200)
    layer = _layer(k3, cfg, s.dw, 200)
    T = 200
    x = synth.gen_x(cfg, T=T)
    rng = np.random.default_rng(9)
    idx = np.stack([np.concatenate([[3], rng.permutation(np.delete(np.arange(cfg.E), 3))[:cfg.k - 1]])
                    for _ in range(T)]).astype(np.int32)
    gate = rng.random((T, cfg.k)).astype(np.float32)
    idx[7, 4] = cfg.E + 5  # dropped pair
    y = torch.empty((T, cfg.d), dtype=torch.float32, device="cuda")
    k3.k3moe_experts_forward(layer.handle, _x_dev(x), torch.from_numpy(idx).cuda(),
                             torch.from_numpy(gate).cuda(), y)
    torch.cuda.synchronize()
    yref = oracle.experts_forward(x, idx, gate.astype(np.float64), s.src, n_experts=cfg.E)
    check_output(y.cpu().numpy(), yref, "injected routing")
    for T2 in (1, 3):  # decode path with the same routing
        y2 = torch.empty((T2, cfg.d), dtype=torch.float32, device="cuda")
        k3.k3moe_experts_forward(layer.handle, _x_dev(x[5:5 + T2]), torch.from_numpy(idx[5:5 + T2].copy()).cuda(),
                                 torch.from_numpy(gate[5:5 + T2].copy()).cuda(), y2)
        torch.cuda.synchronize()
        check_output(y2.cpu().numpy(), yref[5:5 + T2], f"injected routing decode T={T2}")
    layer.close()


def _routing_with_counts(counts, T, k, E, seed):
    """idx [T][k] in which expert e is chosen by exactly counts[e] distinct
    tokens; every other slot holds the dropped index E + 1."""
    rng = np.random.default_rng(seed)
    idx = np.full((T, k), E + 1, dtype=np.int32)
    used = np.zeros(T, dtype=np.int64)
    for e in rng.permutation(len(counts)):
        c = int(counts[e])
        if c == 0:
            continue
        # the tokens with the most free slots (random among equals) keep it feasible
        order = np.lexsort((rng.random(T), used))
        toks = order[:c]
        assert used[toks].max() < k, "counts exceed the slots"
        idx[toks, used[toks]] = e
        used[toks] += 1
    for t in range(T):  # the pairs' slot order within a token, shuffled
        idx[t] = idx[t][rng.permutation(k)]
    return idx


def test_tile_sizes_across_column_tile_counts(k3):
    """The grouped GEMMs at every tile size class: experts with exactly 1,
    15-17, 31-33, ..., 95-97 and 191-193 tokens give tiles of 1 to 6 16-token
    column tiles, ragged and full (tiles of 96), and a third ragged tile.
    Tiles of 4 or more column tiles and smaller ones run different K loop
    schedules; every token is compared with the oracle."""
    cfg = synth.CONFIGS[1]
    T = 300
    counts = np.zeros(cfg.E, dtype=np.int64)
    sizes = [1, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64, 65, 79, 80, 81, 95, 96, 97,
             143, 144, 145, 191, 192, 193]
    counts[:len(sizes)] = sizes
    idx = _routing_with_counts(counts, T, cfg.k, cfg.E, seed=31)
    got = np.bincount(idx[idx < cfg.E], minlength=cfg.E)
    assert np.array_equal(got, counts)
    s = Small(cfg, T)
    layer = _layer(k3, cfg, s.dw, T)
    x = synth.gen_x(cfg, T=T)
    gate = np.random.default_rng(32).random((T, cfg.k)).astype(np.float32)
    y = torch.empty((T, cfg.d), dtype=torch.float32, device="cuda")
    k3.k3moe_experts_forward(layer.handle, _x_dev(x), torch.from_numpy(idx).cuda(),
                             torch.from_numpy(gate).cuda(), y)
    torch.cuda.synchronize()
    yref = oracle.experts_forward(x, idx, gate.astype(np.float64), s.src, n_experts=cfg.E)
    ratio = check_output(y.cpu().numpy(), yref, "tile sizes")
    _say(f"[tile sizes] {len(sizes)} experts, {int(counts.sum())} pairs, "
         f"max|err|/rms = {ratio:.3e}")
    layer.close()


def test_abi_rejects_bad_calls(k3):
    cfg = synth.CONFIGS[0]
    s = Small(cfg, 4)
    layer = _layer(k3, cfg, s.dw, 4)
    x = _x_dev(synth.gen_x(cfg, T=5))
    y = torch.empty((5, cfg.d), dtype=torch.float32, device="cuda")
    with pytest.raises(k3.K3MoEError) as ei:
        k3.k3moe_layer_forward(layer.handle, x, y)  # T = 5 > max_tokens = 4
    assert ei.value.status == k3.K3MOE_EINVAL
    yz = torch.empty((0, cfg.d), dtype=torch.float32, device="cuda")
    k3.k3moe_layer_forward(layer.handle, x[:0], yz)  # T = 0 is a no-op
    bad = dict(s.dw)
    bad["gate_q"] = s.dw["gate_q"].view(-1)[1:]  # misaligned
    with pytest.raises(k3.K3MoEError):
        k3.Layer(k3.Config(cfg.d, cfg.E, cfg.k, cfg.f, 4), bad, 0)
    with pytest.raises(k3.K3MoEError) as ei:
        k3.Layer(k3.Config(cfg.d, cfg.E, cfg.k, cfg.f, 4), s.dw, 99)
    assert ei.value.status == k3.K3MOE_EINVAL
    layer.close()


def _sample_tokens(ridx, E, n, seed, label):
    """Seeded sample of n tokens whose outputs are checked, chosen so the
    grouped GEMM's hard places are in it. Pairs are grouped by (expert, token)
    and cut into tiles of TILE_M consecutive tokens of one expert, so an
    expert's i-th token (in token order) sits in row i % TILE_M of tile
    i // TILE_M. The sample always holds: the first and last token; the
    hottest expert's first tile (rows 0, 1, 17, 40, the last) and last tile
    (its first row, a row past 16 when the tile has one, its last row); the
    first and last rows of the last partial tile of the next hottest experts
    with more than TILE_M tokens; a row past 16 of an expert with 17..TILE_M
    tokens. The rest are seeded random tokens."""
    T = ridx.shape[0]
    counts = np.bincount(ridx.reshape(-1), minlength=E)
    order = np.argsort(-counts, kind="stable")
    per = lambda e: np.nonzero(np.any(ridx == e, axis=1))[0]  # noqa: E731
    want = [0, T - 1]
    hot = int(order[0])
    ht = per(hot)
    c = len(ht)
    last0 = TILE_M * ((c - 1) // TILE_M)
    for i in (0, 1, 17, 40, min(TILE_M, c) - 1, last0, last0 + 20, c - 1):
        if 0 <= i < c and (i < TILE_M or i >= last0):
            want.append(int(ht[i]))
    multi = [int(e) for e in order[1:] if counts[e] > TILE_M][:3]
    for e in multi:
        et = per(e)
        l0 = TILE_M * ((len(et) - 1) // TILE_M)
        want += [int(et[l0]), int(et[-1])]
    mid = [int(e) for e in order if 16 < counts[e] <= TILE_M]
    if mid:
        et = per(mid[0])
        want += [int(et[16]), int(et[-1])]
    want = list(dict.fromkeys(want))[:n]
    rng = np.random.default_rng(seed)
    rest = rng.permutation(np.setdiff1d(np.arange(T), want))[:max(0, n - len(want))]
    tokens = np.sort(np.concatenate([np.asarray(want, dtype=np.int64), rest]))
    _say(f"[{label}] hottest expert {hot}: {c} tokens ({(c + TILE_M - 1) // TILE_M} tiles); "
         f"experts touched {int((counts > 0).sum())}; experts over one tile {int((counts > TILE_M).sum())}; "
         f"checking {len(tokens)} tokens, {len(want)} chosen for their tile rows")
    return tokens


# ----------------------------------------------------------------- K3 scale

@pytest.fixture(scope="module")
def big_layers(k3):
    """One device-resident K3-scale layer at a time (about 21 GB each)."""
    from synth.device import device_weights
    state = {}

    def get(ci, max_tokens):
        if ci is None:  # release
            state.clear()
            torch.cuda.empty_cache()
            return None
        if state.get("ci") != ci:
            state.clear()
            torch.cuda.empty_cache()
            cfg = synth.CONFIGS[ci]
            dw = device_weights(cfg)
            state.update(ci=ci, cfg=cfg, dw=dw,
                         layer=_layer(k3, cfg, dw, max_tokens),
                         src=synth.ExpertSource(cfg), wr=synth.gen_router_w(cfg),
                         bias=synth.gen_bias(cfg))
        return state
    yield get
    state.clear()
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_k3_decode(k3, big_layers):
    _say("case k3 decode T=1")
    st = big_layers(2, 4096)
    cfg = st["cfg"]
    x = synth.gen_x(cfg)
    _run_and_check(k3, st["layer"], cfg, x, st["src"], st["wr"], st["bias"], label="k3 decode")


@pytest.mark.timeout(600)
def test_k3_layer_from_row_major_host_weights(k3, big_layers):
    """A K3-shape layer loaded the way a checkpoint would be: all six MXFP4
    tensors (21 GB) row-major in pinned host memory, packed into the tiled
    device layout through k3moe_pack_mxfp4_from_host (the device then holds
    the tiled tensors and a staging buffer of at most 32 MiB, never a second
    full copy). The tiled tensors equal the generator's tiled ones bit for
    bit, and the layer created from them matches the oracle at decode."""
    from synth.device import device_tensor
    big_layers(None, 0)  # release the resident K3 layer first
    cfg = synth.CONFIGS[2]
    host = {}
    for name in cfg.tensor_shapes():
        t = device_tensor(cfg, name, tiled=False)
        h = torch.empty(t.shape, dtype=torch.uint8, pin_memory=True)
        h.copy_(t)
        host[name] = h
        del t
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    tiled_bytes = sum(int(np.prod(s)) for n, s in cfg.tensor_shapes().items() if n.endswith("_q"))
    tiled_bytes += sum(k3.k3moe_tiled_scale_bytes(cfg.E, *rk) for rk in
                       ((cfg.f, cfg.d), (cfg.f, cfg.d), (cfg.d, cfg.f)))
    free0 = torch.cuda.mem_get_info()[0]
    host["router_w"] = synth.gen_router_w(cfg)
    host["router_b"] = None
    dw = k3.pack_layer_weights_from_host(host, cfg.E, cfg.d, cfg.f)
    torch.cuda.synchronize()
    used = free0 - torch.cuda.mem_get_info()[0]
    _say(f"[k3 host load] tiled tensors {tiled_bytes / 1e9:.3f} GB; device memory taken {used / 1e9:.3f} GB")
    assert used < tiled_bytes + (256 << 20)  # the tensors (+ the router), the staging freed again
    for name in cfg.tensor_shapes():
        ref = device_tensor(cfg, name, tiled=True)
        assert torch.equal(dw[name], ref), name
        del ref
    del host
    layer = _layer(k3, cfg, dw, 8)
    x = synth.gen_x(cfg, T=2)
    try:
        _run_and_check(k3, layer, cfg, x, synth.ExpertSource(cfg), synth.gen_router_w(cfg), None,
                       label="k3 from host row-major")
    finally:
        layer.close()
        del dw
        torch.cuda.empty_cache()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("T", [4, 16])
def test_k3_small_batches(k3, big_layers, T):
    """A few tokens at the K3 shape (speculative-verify and multi-sequence
    decode batches): T = 4 runs the GEMV path with several tokens, T = 16 the
    grouped GEMM with one or two tokens per expert tile. Every token is
    checked; the tokens follow the decode token in the seeded stream."""
    _say(f"case k3 small batch T={T}")
    st = big_layers(2, 4096)
    cfg = st["cfg"]
    x = synth.gen_x(cfg, T=T, start_token=1)
    _run_and_check(k3, st["layer"], cfg, x, st["src"], st["wr"], st["bias"],
                   label=f"k3 small batch T={T}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("T", [1, 16])
def test_k3_graph_replay(k3, big_layers, T):
    """At the K3 shape, graph replay (how decode steps are timed) equals eager
    on every replay."""
    _say(f"case k3 graph replay T={T}")
    st = big_layers(2, 4096)
    _check_graph_replay(k3, st["layer"], st["cfg"], T)


@pytest.mark.timeout(600)
def test_k3_prefill_256(k3, big_layers):
    _say("case k3 prefill T=256")
    st = big_layers(3, 4096)
    cfg = st["cfg"]
    x = synth.gen_x(cfg)
    logits = oracle.router_logits(x, st["wr"], st["bias"])
    ridx, _ = oracle.topk_gates(logits, cfg.k)
    tokens = _sample_tokens(ridx, cfg.E, 64, cfg.seed, "k3 prefill 256")
    _run_and_check(k3, st["layer"], cfg, x, st["src"], st["wr"], st["bias"], tokens=tokens,
                   label="k3 prefill 256")


@pytest.mark.timeout(600)
def test_k3_prefill_4096_skewed(k3, big_layers):
    _say("case k3 prefill T=4096 skewed")
    st = big_layers(4, 4096)
    cfg = st["cfg"]
    x = synth.gen_x(cfg)
    logits = oracle.router_logits(x, st["wr"], st["bias"])
    ridx, _ = oracle.topk_gates(logits, cfg.k)
    tokens = _sample_tokens(ridx, cfg.E, 64, cfg.seed, "k3 prefill 4096 skew")
    _run_and_check(k3, st["layer"], cfg, x, st["src"], st["wr"], st["bias"], tokens=tokens,
                   label="k3 prefill 4096 skew")


@pytest.mark.timeout(600)
def test_k3_prefill_4096_select_only_bias(k3, big_layers):
    """The long skewed prefill with the bias read as selection-only: routing
    on every token, outputs on 16 sampled tokens."""
    _say("case k3 prefill T=4096 skewed, selection-only bias")
    st = big_layers(4, 4096)
    cfg = st["cfg"]
    layer = _layer(k3, cfg, st["dw"], cfg.T, flags=k3.K3MOE_FLAG_BIAS_SELECT_ONLY)
    x = synth.gen_x(cfg)
    ridx, _ = oracle.topk_gates(oracle.router_logits(x, st["wr"], st["bias"]), cfg.k)
    tokens = _sample_tokens(ridx, cfg.E, 16, cfg.seed + 100, "k3 prefill 4096 select-only")
    try:
        _run_and_check(k3, layer, cfg, x, st["src"], st["wr"], st["bias"], tokens=tokens,
                       select_only=True, label="k3 prefill 4096 select-only")
    finally:
        layer.close()


@pytest.mark.timeout(900)
def test_k3_prefill_max_tokens(k3, big_layers):
    """The largest T the K3 shape accepts (T*k*f = 2^30: 32768 tokens, 524288
    pairs): every offset of the grouped path at its widest. Routing is checked
    for every token, outputs for 16 sampled tokens that include the hottest
    expert's first and last tiles, rows past 16 inside a tile and another
    expert's last partial tile."""
    st = big_layers(4, 4096)
    cfg = st["cfg"]
    T = (1 << 30) // (cfg.k * cfg.f)
    _say(f"case k3 prefill max tokens T={T}")
    layer = _layer(k3, cfg, st["dw"], T)
    x = synth.gen_x(cfg, T=T)
    logits = oracle.router_logits(x, st["wr"], st["bias"])
    ridx, _ = oracle.topk_gates(logits, cfg.k)
    del logits
    tokens = _sample_tokens(ridx, cfg.E, 16, cfg.seed, f"k3 prefill T={T}")
    try:
        _run_and_check(k3, layer, cfg, x, st["src"], st["wr"], st["bias"], tokens=tokens,
                       label=f"k3 prefill T={T}")
    finally:
        layer.close()
        torch.cuda.empty_cache()
