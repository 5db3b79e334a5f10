"""The shared input generator: its counter-based PRNG against the published
SplitMix64 outputs, and the distributions the workloads call for."""
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_mix64_matches_splitmix64_reference():
    want = [int(l) for l in open(os.path.join(GOLDEN, "splitmix64.txt"))
            if l.strip() and not l.startswith("#")]
    state = 1234567
    got = []
    for _ in range(5):
        state = (state + 0x9E3779B97F4A7C15) & synth.M64
        got.append(int(synth.mix64(np.uint64(state))))
    assert got == want


def test_random_access_slices_agree():
    a = synth.code_bytes(3, 4, 0, 1000)
    for start, n in [(0, 7), (5, 11), (13, 100), (999, 1)]:
        assert np.array_equal(synth.code_bytes(3, 4, start, n), a[start:start + n])
    s = synth.scale_bytes(3, 7, 0, 500)
    assert np.array_equal(synth.scale_bytes(3, 7, 123, 77), s[123:200])
    cfg = synth.CONFIGS[0]
    W = synth.gen_weights(cfg)
    e5 = synth.gen_expert(cfg, 5)
    for name in W:
        assert np.array_equal(W[name][5], e5[name])


def test_distributions():
    z = synth.normals(9, 1, 0, 400000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1.0) < 0.01
    assert abs(np.mean(z ** 4) - 3.0) < 0.05  # normal kurtosis
    b = synth.code_bytes(9, 3, 0, 200000)
    nib = np.concatenate([b & 15, b >> 4])
    cnt = np.bincount(nib, minlength=16)
    assert cnt.min() > 0.9 * len(nib) / 16 and cnt.max() < 1.1 * len(nib) / 16
    s = synth.scale_bytes(9, 6, 0, 100000)
    assert set(np.unique(s)) == {123, 124, 125, 126, 127}
    cfg = synth.CONFIGS[1]
    wr = synth.gen_router_w(cfg)
    assert wr.dtype == np.float32 and abs(wr.std() - 0.02) < 0.001
    x = synth.gen_x(cfg, T=2)
    xf = synth.bf16_bits_to_f32(x)
    assert np.array_equal(synth.f32_to_bf16_bits(xf), x)


def test_bf16_rounding_ties_to_even():
    f = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 1.0 + 2 ** -8 + 2 ** -20],
                 dtype=np.float32)
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(f))
    assert list(got) == [1.0, 1.0 + 2 ** -6, -1.0, 1.0 + 2 ** -7]


def test_skew_bias():
    b = synth.skew_bias(4, 896)
    want = np.sort(2.0 * (np.arange(896) + 1.0) ** -1.2)[::-1]
    assert np.allclose(np.sort(b.astype(np.float64))[::-1], want, rtol=1e-7)
    assert b.dtype == np.float32
