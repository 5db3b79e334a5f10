"""Seeded, counter-based synthetic inputs for one sparse MoE layer with MXFP4
expert weights.

This module is shared by the oracle side (tests, CPU baseline) and the HIP side
(tests, benchmark). It holds none of the layer's arithmetic: it only draws
random bytes and numbers and lays them out in the layer's input formats.

Generator
---------
Every draw is a pure function of (seed, stream, index), so any slice of any
tensor can be regenerated on its own, on the host (numpy, here) or on the
device (``synth/fill.hip``, bit-identical for the integer streams):

    mix64(z)            SplitMix64 output finaliser (Steele, Lea & Flood,
                        "Fast splittable pseudorandom number generators",
                        OOPSLA 2014): z ^= z>>30; z *= 0xbf58476d1ce4e5b9;
                        z ^= z>>27; z *= 0x94d049bb133111eb; z ^= z>>31
    key(seed, s)        mix64(seed ^ (s << 56))
    draw(seed, s, i)    mix64(key(seed, s) + i)          (all mod 2^64)

Workloads (the Kimi K3 MoE layer shapes that the pages describe: 896 routed
experts with top-16 routing per token, MXFP4 expert weights, SwiGLU experts):

* activations x: bf16 from N(0,1); router weights: fp32 from N(0, 0.02^2)
  (0.02 is the standard deviation); normals by the Box-Muller cosine branch
  in double from two 53-bit uniforms (draws 2i and 2i+1), rounded double ->
  fp32 (RNE) -> bf16 (RNE) for x and double -> fp32 for the router weights;
* expert weight codes: packed E2M1 nibbles, uniform over all 16 codes; byte b
  of a tensor is byte (b % 8) of draw(b // 8);
* expert scale bytes (E8M0): 127 + (-4 + draw % 5), i.e. exponents uniform on
  the integers -4..0;
* skewed router bias (long-prefill workload): a Fisher-Yates permutation
  rank of 0..E-1 (j = draw(i) % (i+1) for i = E-1 .. 1) and
  bias[e] = fp32(2 * (rank[e] + 1) ** -1.2).
"""
from __future__ import annotations

import dataclasses
import numpy as np

M64 = 0xFFFFFFFFFFFFFFFF

STREAM_X = 1
STREAM_ROUTER_W = 2
STREAM_GATE_Q, STREAM_UP_Q, STREAM_DOWN_Q = 3, 4, 5
STREAM_GATE_S, STREAM_UP_S, STREAM_DOWN_S = 6, 7, 8
STREAM_BIAS = 9
STREAM_POOL = 10  # decode benchmark token pool

WEIGHT_STREAMS = {
    "gate_q": STREAM_GATE_Q, "up_q": STREAM_UP_Q, "down_q": STREAM_DOWN_Q,
    "gate_s": STREAM_GATE_S, "up_s": STREAM_UP_S, "down_s": STREAM_DOWN_S,
}


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """Shape of one MoE layer workload."""
    name: str
    d: int          # hidden size (reduction dim of gate/up, output dim of down)
    E: int          # routed experts
    k: int          # experts per token
    f: int          # expert FFN width
    T: int          # tokens
    seed: int
    skew_bias: bool = False  # per-expert router bias 2*(rank+1)^-1.2

    def tensor_shapes(self):
        d, E, f = self.d, self.E, self.f
        return {
            "gate_q": (E, f, d // 2), "gate_s": (E, f, d // 32),
            "up_q": (E, f, d // 2), "up_s": (E, f, d // 32),
            "down_q": (E, d, f // 2), "down_s": (E, d, f // 32),
        }

    def expert_bytes(self) -> int:
        return sum(int(np.prod(s[1:])) for s in self.tensor_shapes().values())


# The five workloads: tiny, small, K3-scale decode, prefill chunk, long
# prefill with skewed routing.
CONFIGS = [
    LayerConfig("tiny_d128_e8_k2_f256_t1", 128, 8, 2, 256, 1, 0),
    LayerConfig("small_d2048_e64_k8_f1024_t1", 2048, 64, 8, 1024, 1, 1),
    LayerConfig("k3_decode_d7168_e896_k16_f2048_t1", 7168, 896, 16, 2048, 1, 2),
    LayerConfig("k3_prefill_d7168_e896_k16_f2048_t256", 7168, 896, 16, 2048, 256, 3),
    LayerConfig("k3_prefill_skew_d7168_e896_k16_f2048_t4096", 7168, 896, 16, 2048, 4096, 4,
                skew_bias=True),
]


def mix64(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = z ^ (z >> np.uint64(30))
        z = z * np.uint64(0xBF58476D1CE4E5B9)
        z = z ^ (z >> np.uint64(27))
        z = z * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
    return z


def stream_key(seed: int, stream: int) -> int:
    return int(mix64(np.uint64((seed ^ (stream << 56)) & M64)))


def draws(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """draw(seed, stream, i) for i in [start, start+count), as uint64."""
    key = np.uint64(stream_key(seed, stream))
    idx = np.arange(start, start + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(idx + key)


def uniforms53(r: np.ndarray) -> np.ndarray:
    """53-bit uniform in (0, 1): ((r >> 11) + 0.5) * 2^-53."""
    return ((r >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def normals(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Standard normals n_i, i in [start, start+count), float64 (Box-Muller)."""
    r = draws(seed, stream, 2 * start, 2 * count)
    u1 = uniforms53(r[0::2])
    u2 = uniforms53(r[1::2])
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def gen_x(cfg: LayerConfig, T: int | None = None, start_token: int = 0,
          stream: int = STREAM_X) -> np.ndarray:
    """Activations [T][d] as bf16 bit patterns (uint16)."""
    T = cfg.T if T is None else T
    z = normals(cfg.seed, stream, start_token * cfg.d, T * cfg.d)
    return f32_to_bf16_bits(z.astype(np.float32)).reshape(T, cfg.d)


def gen_router_w(cfg: LayerConfig) -> np.ndarray:
    """Router weights [E][d] fp32 from N(0, 0.02^2)."""
    z = normals(cfg.seed, STREAM_ROUTER_W, 0, cfg.E * cfg.d)
    return (0.02 * z).astype(np.float32).reshape(cfg.E, cfg.d)


def gen_bias(cfg: LayerConfig) -> np.ndarray | None:
    """Skewed per-expert router bias [E] fp32, or None for unbiased workloads."""
    if not cfg.skew_bias:
        return None
    return skew_bias(cfg.seed, cfg.E)


def skew_bias(seed: int, E: int) -> np.ndarray:
    perm = np.arange(E, dtype=np.int64)
    r = draws(seed, STREAM_BIAS, 0, E)
    for i in range(E - 1, 0, -1):
        j = int(r[i] % np.uint64(i + 1))
        perm[i], perm[j] = perm[j], perm[i]
    rank = perm
    return (2.0 * (rank.astype(np.float64) + 1.0) ** -1.2).astype(np.float32)


def code_bytes(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Packed E2M1 code bytes [start, start+count) of one tensor (uint8)."""
    w0 = start // 8
    w1 = (start + count + 7) // 8
    words = draws(seed, stream, w0, w1 - w0)
    b = words.view(np.uint8)  # little-endian: byte (i % 8) of word i // 8
    off = start - 8 * w0
    return b[off:off + count].copy()


def scale_bytes(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """E8M0 scale bytes [start, start+count): 123 + draw % 5."""
    r = draws(seed, stream, start, count)
    return (np.uint64(123) + r % np.uint64(5)).astype(np.uint8)


def gen_expert(cfg: LayerConfig, e: int) -> dict:
    """All six weight tensors of expert e (host, uint8)."""
    out = {}
    for name, shape in cfg.tensor_shapes().items():
        n = int(np.prod(shape[1:]))
        gen = code_bytes if name.endswith("_q") else scale_bytes
        out[name] = gen(cfg.seed, WEIGHT_STREAMS[name], e * n, n).reshape(shape[1:])
    return out


def gen_weights(cfg: LayerConfig) -> dict:
    """All experts' weights on the host (only for small layers)."""
    out = {}
    for name, shape in cfg.tensor_shapes().items():
        n = int(np.prod(shape))
        gen = code_bytes if name.endswith("_q") else scale_bytes
        out[name] = gen(cfg.seed, WEIGHT_STREAMS[name], 0, n).reshape(shape)
    return out


class ExpertSource:
    """Lazy per-expert weight source with a small cache (host)."""

    def __init__(self, cfg: LayerConfig, full: dict | None = None):
        self.cfg = cfg
        self.full = full
        self._cache = {}

    def __call__(self, e: int) -> dict:
        if self.full is not None:
            return {k: v[e] for k, v in self.full.items()}
        if e not in self._cache:
            if len(self._cache) > 64:
                self._cache.clear()
            self._cache[e] = gen_expert(self.cfg, e)
        return self._cache[e]
