"""Pins of the fp64 oracle against facts outside itself: the OCP MX format
tables, closed forms, brute force on tiny inputs and invariants the pages
state (chunk-union prefill equals the per-token path; a layer's result does
not depend on how tokens are batched or ordered)."""
import itertools
import math
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
import synth
from _dense_check import dense_masked_forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- formats

def test_e2m1_matches_ocp_table():
    rows = _read_table("ocp_mx_e2m1.txt")
    assert len(rows) == 16
    for bits, val in rows:
        code = int(bits, 2)
        got = oracle.e2m1_value(code)
        assert got == float(val)
        assert math.copysign(1.0, got) == math.copysign(1.0, float(val))  # -0 for code 8
    assert np.array_equal(oracle.E2M1_VALUES, [float(v) for _, v in rows])


def test_e8m0_matches_ocp_table():
    for hx, val in _read_table("ocp_mx_e8m0.txt"):
        got = oracle.e8m0_value(int(hx, 16))
        if val == "NaN":
            assert math.isnan(got)
        else:
            assert got == 2.0 ** int(val[2:])
    for b in range(254):
        assert oracle.e8m0_value(b + 1) == 2.0 * oracle.e8m0_value(b)


def test_dequant_exhaustive_exact_in_fp32():
    # every (code, scale byte) pair once: row b uses scale byte b, codes 0..15
    q = np.zeros((256, 16), dtype=np.uint8)           # K = 32 per row
    q[:, :8] = np.array([c | ((c + 8) << 4) for c in range(8)], dtype=np.uint8)
    s = np.arange(256, dtype=np.uint8).reshape(256, 1)
    w = oracle.dequant(q, s)
    table = {int(b, 2): float(v) for b, v in _read_table("ocp_mx_e2m1.txt")}
    for b in range(256):
        for c in range(16):
            pos = 2 * c if c < 8 else 2 * (c - 8) + 1
            got = w[b, pos]
            if b == 255:
                assert math.isnan(got)
                continue
            want = table[c] * 2.0 ** (b - 127)
            assert got == want
            # exactly representable in fp32 wherever fp32 has the range
            # (|value| < 2^128; 6 * 2^127 overflows)
            if abs(got) < 2.0 ** 128:
                assert float(np.float32(got)) == got


def test_dequant_layout_by_hand():
    # one row, K = 64 (two blocks). Byte 0 = 0x21: element 0 is code 1 (0.5),
    # element 1 is code 2 (1.0). Byte 1 = 0xF7: element 2 = code 7 (6.0),
    # element 3 = code 15 (-6.0). Byte 16 = 0x5B: element 32 = code 11 (-1.5),
    # element 33 = code 5 (3.0). Scales: block 0 = 0x80 (x2), block 1 = 0x7E (x0.5).
    q = np.zeros((1, 32), dtype=np.uint8)
    q[0, 0], q[0, 1], q[0, 16] = 0x21, 0xF7, 0x5B
    s = np.array([[0x80, 0x7E]], dtype=np.uint8)
    w = oracle.dequant(q, s)
    want = np.zeros(64)
    want[0], want[1], want[2], want[3] = 1.0, 2.0, 12.0, -12.0
    want[32], want[33] = -0.75, 1.5
    assert np.array_equal(w[0], want)


# ---------------------------------------------------------------- router

def test_router_logits_match_exact_sums():
    rng = np.random.default_rng(0)
    T, E, d = 3, 5, 96
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    wr = (0.02 * rng.standard_normal((E, d))).astype(np.float32)
    bias = rng.standard_normal(E).astype(np.float32)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    got = oracle.router_logits(x, wr)
    gotb = oracle.router_logits(x, wr, bias)
    for t in range(T):
        for e in range(E):
            exact = math.fsum(float(xf[t, i]) * float(wr[e, i]) for i in range(d))
            assert got[t, e] == np.float32(exact)
            assert gotb[t, e] == np.float32(np.float32(exact) + bias[e])


def _brute_topk(row, k):
    E = len(row)
    best, best_key = None, None
    for sub in itertools.combinations(range(E), k):
        key = (math.fsum(float(row[e]) for e in sub), tuple(-e for e in sub))
        if best_key is None or key > best_key:
            best, best_key = sub, key
    return sorted(best, key=lambda e: (-float(row[e]), e))


@pytest.mark.parametrize("E,k", [(8, 2), (8, 3), (6, 1), (7, 7)])
def test_topk_brute_force_subsets(E, k):
    rng = np.random.default_rng(E * 10 + k)
    for trial in range(60):
        if trial % 3 == 0:  # many exact ties
            row = rng.integers(-2, 3, E).astype(np.float32)
        else:
            row = rng.standard_normal(E).astype(np.float32)
        idx, gate = oracle.topk_gates(row[None, :], k)
        assert list(idx[0]) == _brute_topk(row, k)


def test_topk_special_cases():
    E, k = 8, 3
    idx, gate = oracle.topk_gates(np.zeros((1, E), np.float32), k)
    assert list(idx[0]) == [0, 1, 2]
    assert np.allclose(gate[0], 1.0 / k, rtol=0, atol=1e-15)
    # k = 1: gate exactly one
    row = np.random.default_rng(1).standard_normal((4, E)).astype(np.float32)
    _, g1 = oracle.topk_gates(row, 1)
    assert np.all(g1 == 1.0)
    # k = E: full softmax in logit order
    idx, g = oracle.topk_gates(row, E)
    for t in range(4):
        sm = softmax(row[t].astype(np.float64))
        assert np.allclose(g[t], sm[idx[t]], rtol=1e-14, atol=0)
        assert list(idx[t]) == list(np.lexsort((np.arange(E), -row[t])))


def test_topk_nan_logits_count_as_minus_inf():
    """A NaN logit counts as -inf, in the ranking and in the gates. Pinned by
    a chain of reductions to the brute force above: NaN -> -inf leaves
    selection and gates unchanged; -inf -> one common finite value below
    every other logit leaves the selection unchanged (equal values rank by
    index), so the brute force over subsets decides it; the gates of the
    selected -inf logits are exactly 0 and the others are the softmax of the
    selected finite logits."""
    # worked example: three finite logits, then the -inf/NaN ties by index
    row = np.array([np.nan, 0.5, np.nan, -np.inf, 0.1, np.nan, -np.inf, 0.3], np.float32)
    idx, gate = oracle.topk_gates(row[None, :], 5)
    assert list(idx[0]) == [1, 7, 4, 0, 2]
    assert np.allclose(gate[0, :3], softmax(np.array([0.5, 0.3, 0.1], np.float32).astype(np.float64)),
                       rtol=1e-14, atol=0)
    assert np.all(gate[0, 3:] == 0.0)
    rng = np.random.default_rng(17)
    E = 8
    for trial in range(200):
        k = int(rng.integers(1, E + 1))
        row = (rng.integers(-2, 3, E) if trial % 2 else rng.standard_normal(E)).astype(np.float32)
        kind = rng.integers(0, 3, E)  # 0 finite, 1 NaN, 2 -inf
        kind[rng.integers(0, E)] = 0  # at least one finite logit
        row[kind == 1] = np.nan
        row[kind == 2] = -np.inf
        idx, gate = oracle.topk_gates(row[None, :], k)
        inf_row = np.where(np.isnan(row), np.float32(-np.inf), row)
        idx2, gate2 = oracle.topk_gates(inf_row[None, :], k)
        assert np.array_equal(idx, idx2) and np.array_equal(gate, gate2), (row, k)
        fin = np.isfinite(inf_row)
        low = np.float32(np.min(inf_row[fin]) - 64.0)
        fin_row = np.where(fin, inf_row, low)
        idx3, _ = oracle.topk_gates(fin_row[None, :], k)
        assert np.array_equal(idx, idx3), (row, k)
        assert list(idx3[0]) == _brute_topk(fin_row, k), (row, k)
        sel = idx[0]
        on = fin[sel]
        assert np.all(gate[0][~on] == 0.0)
        want = softmax(inf_row[sel[on]].astype(np.float64))
        assert np.allclose(gate[0][on], want, rtol=1e-14, atol=0), (row, k)
    # nothing finite: every gate is NaN (l_j - l_first is -inf - -inf)
    idx, gate = oracle.topk_gates(np.array([[np.nan, -np.inf, np.nan]], np.float32), 2)
    assert list(idx[0]) == [0, 1] and np.all(np.isnan(gate))


def test_selection_only_bias():
    """The selection-only reading of a router bias: the bias ranks the
    experts, the gates are a softmax of the unbiased logits of the chosen
    ones. Pinned by: zero bias gives the default mode exactly; the selection
    is the brute-force top-k of the biased logits; the gates do not change
    under any bias that keeps the selection, nor under a shift of all
    logits; x = 0 gives gates 1/k; and the default mode's gates follow from
    these by g_default_j = g_j e^(b_j) / sum_i g_i e^(b_i)."""
    rng = np.random.default_rng(23)
    for trial in range(120):
        E = int(rng.integers(2, 9))
        k = int(rng.integers(1, E + 1))
        raw = (rng.integers(-2, 3, E) if trial % 3 == 0 else rng.standard_normal(E)).astype(np.float32)
        bias = (0.7 * rng.standard_normal(E)).astype(np.float32)
        sel = raw + bias  # fp32, as the router adds it
        idx, g = oracle.topk_gates(sel[None, :], k, gate_logits=raw[None, :])
        assert list(idx[0]) == _brute_topk(sel, k)
        i0, g0 = oracle.topk_gates(raw[None, :], k, gate_logits=raw[None, :])
        d0, dg = oracle.topk_gates(raw[None, :], k)
        assert np.array_equal(i0, d0) and np.array_equal(g0, dg)
        # another bias with the same selection: the gates stay
        shift = np.zeros(E, np.float32)
        shift[idx[0]] = 0.25  # raising the chosen ones keeps them chosen
        _, g2 = oracle.topk_gates((sel + shift)[None, :], k, gate_logits=raw[None, :])
        assert np.allclose(g2, g, rtol=1e-14, atol=0)
        # (the shifted fp32 logits are rounded again: differences move by ~2^-24)
        _, g3 = oracle.topk_gates(sel[None, :], k, gate_logits=(raw + np.float32(0.5))[None, :])
        assert np.allclose(g3, g, rtol=1e-6, atol=1e-12)
        # the default mode on the biased logits, from these gates
        di, dgb = oracle.topk_gates(sel[None, :], k)
        assert np.array_equal(di, idx)
        w = g[0] * np.exp(sel[idx[0]].astype(np.float64) - raw[idx[0]].astype(np.float64))
        assert np.allclose(dgb[0], w / w.sum(), rtol=1e-12, atol=1e-15)
    # a bias far larger than the logits (selection by bias alone) leaves the
    # gates the softmax of the raw logits: no term may under- or overflow
    raw = np.array([0.3, -1.2, 2.0, 0.1, -0.4, 1.1], np.float32)
    big = np.array([900.0, 0.0, 850.0, -900.0, 880.0, 0.0], np.float32)
    idx, g = oracle.topk_gates((raw + big)[None, :], 3, gate_logits=raw[None, :])
    assert list(idx[0]) == [0, 4, 2]
    assert np.allclose(g[0], softmax(raw[[0, 4, 2]].astype(np.float64)), rtol=1e-14, atol=0)
    cfg = synth.CONFIGS[1]
    bias = synth.skew_bias(4, cfg.E)
    x0 = np.zeros((1, cfg.d), dtype=np.uint16)
    wr = synth.gen_router_w(cfg)
    r = oracle.layer_forward(x0, wr, bias, synth.ExpertSource(cfg, synth.gen_weights(cfg)), cfg.k,
                             bias_select_only=True)
    assert list(r["idx"][0]) == list(np.argsort(-bias.astype(np.float64), kind="stable")[:cfg.k])
    assert np.all(r["gate"] == 1.0 / cfg.k)
    # zero bias: the whole layer equals the default mode bit for bit
    x = synth.gen_x(cfg, T=3)
    src = synth.ExpertSource(cfg, synth.gen_weights(cfg))
    zero = np.zeros(cfg.E, np.float32)
    a = oracle.layer_forward(x, wr, zero, src, cfg.k, bias_select_only=True)
    b = oracle.layer_forward(x, wr, zero, src, cfg.k)
    assert np.array_equal(a["idx"], b["idx"]) and np.array_equal(a["y64"], b["y64"])


def test_gates_sum_to_one_and_bias_selects():
    cfg = synth.CONFIGS[1]
    E, k = cfg.E, cfg.k
    bias = synth.skew_bias(4, E)
    x0 = np.zeros((1, cfg.d), dtype=np.uint16)
    logits = oracle.router_logits(x0, synth.gen_router_w(cfg), bias)
    assert np.array_equal(logits[0], bias)  # x = 0: logits are the bias
    idx, gate = oracle.topk_gates(logits, k)
    assert list(idx[0]) == list(np.argsort(-bias.astype(np.float64), kind="stable")[:k])
    assert np.allclose(gate[0], softmax(bias[idx[0]].astype(np.float64)), rtol=1e-14)
    x = synth.gen_x(cfg, T=64)
    _, g = oracle.topk_gates(oracle.router_logits(x, synth.gen_router_w(cfg)), k)
    assert np.all(np.abs(g.sum(axis=1) - 1.0) < 1e-12)
    assert np.all(np.abs(g.astype(np.float32).sum(axis=1, dtype=np.float32) - 1.0) < 1e-6)


# ---------------------------------------------------------------- expert FFN

def test_silu_closed_form():
    z = np.concatenate([np.linspace(-40, 40, 2001), [0.0, 1e-300, -1e-300]])
    assert np.allclose(oracle.silu(z), z * expit(z), rtol=1e-14, atol=1e-300)
    big = oracle.silu(np.array([-1000.0, 1000.0, -750.0]))
    assert not np.any(np.isnan(big))
    assert big[0] == 0.0 and big[1] == 1000.0 and big[2] == 0.0


def _selection_matrix(rows, cols, pick, code, scale_bytes):
    """MXFP4 matrix with one non-zero per row: W[r, pick[r]] = E2M1[code] *
    2^(scale_bytes[r] - 127); every other element is code 0."""
    q = np.zeros((rows, cols // 2), dtype=np.uint8)
    s = np.full((rows, cols // 32), 127, dtype=np.uint8)
    for r in range(rows):
        c = pick[r]
        q[r, c // 2] |= (code << 4) if c % 2 else code
        s[r, c // 32] = scale_bytes[r]
    return q, s


def test_expert_ffn_selection_closed_form():
    rng = np.random.default_rng(7)
    d, f = 64, 96
    pg = rng.integers(0, d, f)
    pu = rng.integers(0, d, f)
    pd = rng.integers(0, f, d)
    sg = rng.integers(124, 131, f)
    su = rng.integers(124, 131, f)
    sd = rng.integers(124, 131, d)
    w = {}
    w["gate_q"], w["gate_s"] = _selection_matrix(f, d, pg, 5, sg)    # code 5 = 3.0
    w["up_q"], w["up_s"] = _selection_matrix(f, d, pu, 10, su)       # code 10 = -1.0
    w["down_q"], w["down_s"] = _selection_matrix(d, f, pd, 4, sd)    # code 4 = 2.0
    x = rng.standard_normal((3, d))
    o, h = oracle.expert_ffn(x, w, return_h=True)
    g = 3.0 * x[:, pg] * 2.0 ** (sg - 127)
    u = -1.0 * x[:, pu] * 2.0 ** (su - 127)
    want_h = g * expit(g) * u
    want_o = 2.0 * want_h[:, pd] * 2.0 ** (sd - 127)
    assert np.allclose(h, want_h, rtol=1e-14, atol=0)
    assert np.allclose(o, want_o, rtol=1e-14, atol=0)


def test_zero_weights_give_zero():
    cfg = synth.CONFIGS[0]
    W = synth.gen_weights(cfg)
    for code_byte in (0x00, 0x88):  # +0 and -0 codes
        Z = dict(W)
        for name in ("gate_q", "up_q", "down_q"):
            Z[name] = np.full_like(W[name], code_byte)
        x = synth.gen_x(cfg, T=2)
        r = oracle.layer_forward(x, synth.gen_router_w(cfg), None, synth.ExpertSource(cfg, Z), cfg.k)
        assert np.all(r["y64"] == 0.0)


def test_nan_scale_byte_propagates():
    """E8M0 byte 0xFF is NaN (OCP MX v1.0): a NaN block in row m of an
    expert's down projection makes exactly output m of the tokens routed to
    that expert NaN; a NaN block in its gate projection makes every output of
    those tokens NaN (through h). Tokens routed elsewhere stay finite and
    equal to the unmodified layer."""
    cfg = synth.CONFIGS[0]
    W = synth.gen_weights(cfg)
    wr = synth.gen_router_w(cfg)
    x = synth.gen_x(cfg, T=12, stream=3)
    base = oracle.layer_forward(x, wr, None, synth.ExpertSource(cfg, W), cfg.k)
    used = np.unique(base["idx"])
    e_down, e_gate = int(used[0]), int(used[1])
    m0 = 5
    W2 = {n: a.copy() for n, a in W.items()}
    W2["down_s"][e_down, m0, 3] = 0xFF
    W2["gate_s"][e_gate, 7, 2] = 0xFF
    r = oracle.layer_forward(x, wr, None, synth.ExpertSource(cfg, W2), cfg.k)
    assert np.array_equal(r["idx"], base["idx"])
    for t in range(x.shape[0]):
        sel = set(r["idx"][t].tolist())
        want = np.zeros(cfg.d, dtype=bool)
        if e_down in sel:
            want[m0] = True
        if e_gate in sel:
            want[:] = True
        assert np.array_equal(np.isnan(r["y64"][t]), want), t
        assert np.array_equal(r["y64"][t][~want], base["y64"][t][~want]), t


def test_scale_homogeneity():
    cfg = synth.CONFIGS[0]
    W = synth.gen_weights(cfg)
    x = synth.gen_x(cfg, T=2)
    wr = synth.gen_router_w(cfg)
    base = oracle.layer_forward(x, wr, None, synth.ExpertSource(cfg, W), cfg.k)["y64"]
    for name in ("down_s", "up_s"):
        W2 = dict(W)
        W2[name] = (W[name] + 1).astype(np.uint8)
        y2 = oracle.layer_forward(x, wr, None, synth.ExpertSource(cfg, W2), cfg.k)["y64"]
        assert np.array_equal(y2, 2.0 * base)


# ---------------------------------------------------------------- whole layer

@pytest.mark.parametrize("ci,T", [(0, 1), (0, 5), (1, 3)])
def test_dense_masked_equals_sparse(ci, T):
    cfg = synth.CONFIGS[ci]
    W = synth.gen_weights(cfg)
    src = synth.ExpertSource(cfg, W)
    x = synth.gen_x(cfg, T=T)
    wr = synth.gen_router_w(cfg)
    r = oracle.layer_forward(x, wr, None, src, cfg.k)
    sparse = r["y64"]
    dense, mask = dense_masked_forward(x, wr, None, src, cfg.k, cfg.E)
    for t in range(T):  # the same experts are selected
        assert set(np.nonzero(mask[t])[0]) == set(r["idx"][t].tolist())
    rms = np.sqrt(np.mean(sparse ** 2))
    # fp64 with different summation orders (BLAS products vs the oracle's
    # index-order sums): agreement to a few ulps of the accumulated terms
    assert np.max(np.abs(dense - sparse)) <= 1e-12 * rms


def test_batch_and_permutation_invariance():
    cfg = synth.CONFIGS[1]
    W = synth.gen_weights(cfg)
    src = synth.ExpertSource(cfg, W)
    x = synth.gen_x(cfg, T=6)
    wr = synth.gen_router_w(cfg)
    full = oracle.layer_forward(x, wr, None, src, cfg.k)
    for t in range(6):
        one = oracle.layer_forward(x[t:t + 1], wr, None, src, cfg.k)
        assert np.array_equal(one["idx"][0], full["idx"][t])
        assert np.array_equal(one["y64"][0], full["y64"][t])
    p = np.array([3, 0, 5, 1, 4, 2])
    perm = oracle.layer_forward(x[p], wr, None, src, cfg.k)
    assert np.array_equal(perm["y64"], full["y64"][p])
    assert np.array_equal(perm["idx"], full["idx"][p])


# ---------------------------------------------------------------- grouping

@pytest.mark.parametrize("T,k,E", [(1, 2, 8), (37, 4, 16), (300, 16, 896), (5, 8, 8)])
def test_group_pairs_matches_stable_sort(T, k, E):
    rng = np.random.default_rng(T + k + E)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, perm = oracle.group_pairs(idx, E)
    flat = idx.reshape(-1)
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))


def test_failed_expert_contributes_zero():
    # a slot whose expert index is outside [0, E) adds nothing (the pages'
    # batched-prefill fix: a failed expert contributes zero, never garbage)
    cfg = synth.CONFIGS[0]
    W = synth.gen_weights(cfg)
    src = synth.ExpertSource(cfg, W)
    x = synth.gen_x(cfg, T=3)
    idx = np.array([[1, 4], [2, 7], [0, 5]], dtype=np.int32)
    gate = np.array([[0.75, 0.25], [0.5, 0.5], [0.9, 0.1]])
    bad = idx.copy()
    bad[0, 1], bad[2, 0] = cfg.E, -1
    y_bad = oracle.experts_forward(x, bad, gate, src, n_experts=cfg.E)
    g0 = gate.copy()
    g0[0, 1] = g0[2, 0] = 0.0
    y_ref = oracle.experts_forward(x, idx, g0, src, n_experts=cfg.E)
    assert np.array_equal(y_bad, y_ref)
    single = oracle.expert_ffn(oracle.bf16_to_f64(x[2:3]), src(5))[0]
    assert np.array_equal(y_bad[2], 0.0 + 0.1 * single)


def test_group_pairs_leaves_out_invalid():
    idx = np.array([[2, 0], [9, 2], [-1, 1]], dtype=np.int32)
    counts, offsets, perm = oracle.group_pairs(idx, 3)
    assert counts.tolist() == [1, 1, 2]
    assert offsets.tolist() == [0, 1, 2, 4]
    assert perm.tolist() == [1, 5, 0, 3]


def test_thread_count_does_not_change_results():
    cfg = synth.CONFIGS[1]
    src = synth.ExpertSource(cfg, synth.gen_weights(cfg))
    x = synth.gen_x(cfg, T=5)
    wr = synth.gen_router_w(cfg)
    before = oracle.get_threads()
    try:
        oracle.set_threads(1)
        a = oracle.layer_forward(x, wr, None, src, cfg.k)
        oracle.set_threads(4)
        b = oracle.layer_forward(x, wr, None, src, cfg.k)
    finally:
        oracle.set_threads(before)
    assert np.array_equal(a["logits"], b["logits"])
    assert np.array_equal(a["y64"], b["y64"])
