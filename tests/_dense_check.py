"""An independent dense computation of the MoE layer, used only to pin the C
oracle: every expert runs on every token and y = sum_e m[t,e] * p[t,e] *
o_e(x_t), where p is the full softmax over all E logits and m masks the k
selected experts (p renormalised over the mask). Written with numpy's own
dequantisation (a lookup table of the OCP MX E2M1 values and 2^(b-127)
scales) and fp64 matrix products, so it shares no arithmetic with the C
oracle beyond the definition itself."""
from __future__ import annotations

import numpy as np

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                 -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def dequant_np(q, s):
    q = np.asarray(q, dtype=np.uint8)
    codes = np.stack([q & 15, q >> 4], axis=-1).reshape(q.shape[0], -1)
    scale = np.exp2(np.asarray(s, dtype=np.float64) - 127.0)
    return E2M1[codes] * np.repeat(scale, 32, axis=1)


def bf16_np(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dense_masked_forward(x_bits, router_w, bias, experts, k, E):
    x = bf16_np(x_bits)
    logits = (x @ np.asarray(router_w, np.float32).astype(np.float64).T).astype(np.float32)
    if bias is not None:
        logits = (logits + np.asarray(bias, np.float32)[None, :]).astype(np.float32)
    lg = logits.astype(np.float64)
    T = x.shape[0]
    mask = np.zeros((T, E), dtype=bool)
    for t in range(T):
        order = np.lexsort((np.arange(E), -lg[t]))
        mask[t, order[:k]] = True
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    pm = np.where(mask, p, 0.0)
    pm = pm / pm.sum(axis=1, keepdims=True)
    y = np.zeros_like(x)
    for e in range(E):
        w = experts(e)
        g = x @ dequant_np(w["gate_q"], w["gate_s"]).T
        u = x @ dequant_np(w["up_q"], w["up_s"]).T
        h = g / (1.0 + np.exp(-g)) * u
        y += pm[:, e:e + 1] * (h @ dequant_np(w["down_q"], w["down_s"]).T)
    return y, mask
