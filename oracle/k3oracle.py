"""Plain, slow fp64 reference of one sparse Mixture-of-Experts layer whose
expert weights are stored in MXFP4 (the Kimi K3 layer of the pages: 896 routed
experts, 16 selected per token, expert weights kept as 4-bit codes with a
per-block scale and consumed without materialising a dequantised copy).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg may use this module; the product path never does.
It shares no code, table or helper with the HIP path.

What is computed, and where it comes from
-----------------------------------------
* kimi-k3-in-c pages ("four reductions" overview; decision guide): experts
  are "already nibbles" in MXFP4, about half a byte per parameter; each layer
  has 896 experts and wakes 16 per token.
* CHANGELOG walk-through page, 0.1.0 section: the MoE router picks top-16 of
  896 routed experts; the expert FFN is a gated linear unit (printed as
  "SiTU-GLU"; read here as SwiGLU); the MXFP4 matmul consumes packed nibbles
  directly; chunk-union prefill gives results identical to the per-token path
  (so the per-token definition below is the whole definition).
* The pages leave the router function, tie rule, gate normalisation, block
  layout and formats open. The readings taken (see the design notes) are:
  - router logits l[t,e] = sum_i x[t,i] * Wr[e,i] accumulated exactly (fp64)
    and rounded to fp32, plus an optional fp32 bias per expert added to the
    fp32 logit (before both selection and softmax);
  - top-k by (logit descending, expert index ascending);
  - gates: softmax over the k selected logits (equal to a full softmax
    renormalised over the selection), evaluated in fp64;
  - expert: g = Wg x, u = Wu x, h = SiLU(g) * u with SiLU(z) = z / (1 + e^-z),
    o = Wd h; y[t] = sum_j gate[t,j] * o_j, j in selection order;
  - MXFP4 = OCP Microscaling v1.0: E2M1 element codes (sign, 2-bit exponent
    with bias 1, 1-bit mantissa) and one E8M0 scale (2^(b-127), 0xFF = NaN)
    per 32 consecutive elements along the reduction dimension; the even
    element of a pair sits in the low nibble; matrices are [out][in] with the
    reduction dimension contiguous.
* All floating point is fp64 except where the definition fixes fp32 (the
  router logits and the bias add). Matrix products use numpy's fp64 matmul
  as a library step.

Parity pins: every function here is pinned by the "not gpu" tests against
values of the OCP MX specification, closed forms and brute force (see
tests/test_oracle_pins.py). Fidelity to the real Kimi K3 checkpoint is
parity unpinned (no checkpoint exists here).
"""
from __future__ import annotations

import math
import numpy as np

__all__ = [
    "e2m1_value", "E2M1_VALUES", "e8m0_value", "dequant", "bf16_to_f64",
    "router_logits", "topk_gates", "silu", "expert_ffn", "experts_forward",
    "layer_forward", "dense_masked_forward", "group_pairs",
]


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code (OCP MX v1.0, FP4 element format):
    sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; exponent 0 is
    subnormal (0.5 * mantissa)."""
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp = (code >> 1) & 3
    man = code & 1
    if exp == 0:
        mag = 0.5 * man
    else:
        mag = 2.0 ** (exp - 1) * (1.0 + 0.5 * man)
    return sign * mag


# The 16 code values, evaluated from the closed form above (code 8 is -0).
E2M1_VALUES = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e8m0_value(b: int) -> float:
    """Value of an E8M0 scale byte (OCP MX v1.0): 2^(b-127); 0xFF is NaN."""
    if b == 255:
        return math.nan
    return math.ldexp(1.0, int(b) - 127)


_E8M0_VALUES = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64)


def dequant(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Dequantise an MXFP4 matrix.

    q: [rows][K/2] uint8, element 2i in the low nibble, 2i+1 in the high one.
    s: [rows][K/32] uint8 E8M0 scales, one per 32 consecutive K elements.
    Returns W [rows][K] float64 with W[r, i] = E2M1(code[r, i]) * 2^(s[r, i//32]-127).
    """
    q = np.asarray(q, dtype=np.uint8)
    rows, half = q.shape
    codes = np.empty((rows, 2 * half), dtype=np.uint8)
    codes[:, 0::2] = q & 0x0F
    codes[:, 1::2] = q >> 4
    vals = E2M1_VALUES[codes]
    scale = _E8M0_VALUES[np.asarray(s, dtype=np.uint8)]
    return vals * np.repeat(scale, 32, axis=1)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def router_logits(x_bits: np.ndarray, router_w: np.ndarray,
                  bias: np.ndarray | None = None) -> np.ndarray:
    """fp32 logits [T][E]: exact sum of x*Wr (fp64 accumulation) rounded to
    fp32, then + bias[e] in fp32."""
    x = bf16_to_f64(x_bits)
    w = np.asarray(router_w, dtype=np.float32).astype(np.float64)
    logits = (x @ w.T).astype(np.float32)
    if bias is not None:
        logits = (logits + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    return logits


def topk_gates(logits: np.ndarray, k: int):
    """Per token: the k experts with the largest fp32 logits, ordered by
    (logit descending, index ascending); gates = softmax over those k logits
    in fp64. Returns idx [T][k] int32 and gate [T][k] float64."""
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), dtype=np.int32)
    gate = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        row = logits[t]
        order = sorted(range(E), key=lambda e: (-float(row[e]), e))[:k]
        idx[t] = order
        sel = np.array([float(row[e]) for e in order], dtype=np.float64)
        w = np.exp(sel - sel[0])
        gate[t] = w / w.sum()
    return idx, gate


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + exp(-z)) in fp64 (exp overflow gives -0, not NaN)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(x: np.ndarray, w: dict, return_h: bool = False):
    """One SwiGLU expert on fp64 activations x [n][d]:
    g = x Wg^T, u = x Wu^T, h = SiLU(g) * u, o = h Wd^T. Returns o [n][d]
    (and h [n][f] if asked)."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    wg = dequant(w["gate_q"], w["gate_s"])
    wu = dequant(w["up_q"], w["up_s"])
    wd = dequant(w["down_q"], w["down_s"])
    g = x @ wg.T
    u = x @ wu.T
    h = silu(g) * u
    o = h @ wd.T
    return (o, h) if return_h else o


def experts_forward(x_bits: np.ndarray, idx: np.ndarray, gate: np.ndarray,
                    experts) -> np.ndarray:
    """y[t] = sum_j gate[t,j] * expert_{idx[t,j]}(x[t]), j in order, fp64.

    experts: callable e -> dict of the expert's six uint8 tensors.
    Each (token, slot) pair is evaluated on its own token row; experts are
    visited once each (the pairs that route to an expert are evaluated with
    that expert's dequantised matrices)."""
    x = bf16_to_f64(x_bits)
    idx = np.asarray(idx)
    T, k = idx.shape
    d = x.shape[1]
    outs = np.zeros((T, k, d), dtype=np.float64)
    for e in np.unique(idx):
        ts, js = np.nonzero(idx == e)
        w = experts(int(e))
        for t, j in zip(ts, js):
            outs[t, j] = expert_ffn(x[t:t + 1], w)[0]
    y = np.zeros((T, d), dtype=np.float64)
    for j in range(k):
        y += np.asarray(gate, dtype=np.float64)[:, j:j + 1] * outs[:, j, :]
    return y


def layer_forward(x_bits, router_w, bias, experts, k: int):
    """Whole layer. Returns dict(y64, y32, idx, gate, logits)."""
    logits = router_logits(x_bits, router_w, bias)
    idx, gate = topk_gates(logits, k)
    y = experts_forward(x_bits, idx, gate, experts)
    return {"y64": y, "y32": y.astype(np.float32), "idx": idx, "gate": gate,
            "logits": logits}


def dense_masked_forward(x_bits, router_w, bias, experts, k: int, E: int):
    """Dense check of the sparse layer: every expert runs on every token and
    y = sum_e m[t,e] * p[t,e] * o_e(x_t), where m masks the k selected experts
    and p is the full softmax over all E logits renormalised over the mask."""
    x = bf16_to_f64(x_bits)
    logits = router_logits(x_bits, router_w, bias).astype(np.float64)
    T = x.shape[0]
    # mask: ranks by (logit desc, index asc) computed by a full sort
    mask = np.zeros((T, E), dtype=bool)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t]))
        mask[t, order[:k]] = True
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    pm = np.where(mask, p, 0.0)
    pm = pm / pm.sum(axis=1, keepdims=True)
    y = np.zeros_like(x)
    for e in range(E):
        o = expert_ffn(x, experts(e))
        y += pm[:, e:e + 1] * o
    return y


def group_pairs(idx: np.ndarray, E: int):
    """Token-to-expert grouping (the chunk-union step): the (token, slot)
    pairs p = t*k + j are bucketed by expert with a stable counting sort.
    Returns counts [E], offsets [E+1] (exclusive prefix sum) and perm [T*k]:
    pair ids ordered by (expert, t, j)."""
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    counts = [0] * E
    for e in flat:
        counts[int(e)] += 1
    offsets = [0] * (E + 1)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:E]
    cursor = list(cursor)
    perm = [0] * len(flat)
    for p, e in enumerate(flat):
        perm[cursor[int(e)]] = p
        cursor[int(e)] += 1
    return (np.array(counts, dtype=np.int32), np.array(offsets, dtype=np.int32),
            np.array(perm, dtype=np.int32))
