"""Python face of the C oracle (oracle/k3oracle.c): argument marshalling only.

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg may use this module; the product path never does.
It shares no code, table or helper with the HIP path.

Every number is computed by the plain single-threaded C99 oracle in
k3oracle.c, whose header states the definition and the readings of the pages
it follows (the kimi-k3-in-c pages: a routed MoE layer, 896 experts with 16
woken per token, MXFP4 expert nibbles, a SwiGLU expert, chunk-union prefill
equal to the per-token path). This module converts numpy arrays to pointers,
walks the experts one at a time (so a K3-size layer never has to sit in host
memory whole) and scatters each expert's rows back to their (token, slot)
places.

Independent tokens can be spread over host threads (`set_threads`); each
thread runs the single-threaded C code on its own rows, so the results do not
depend on the thread count. The default is one thread.

Parity pins: tests/test_oracle_pins.py checks every function here against the
OCP MX value tables, closed forms, exact sums, brute force and an independent
dense all-experts computation. Fidelity to the real Kimi K3 checkpoint is
parity unpinned (no checkpoint exists here).
"""
from __future__ import annotations

import concurrent.futures
import ctypes
import os

import numpy as np

from . import build as _build

__all__ = [
    "e2m1_value", "E2M1_VALUES", "e8m0_value", "dequant", "bf16_to_f64",
    "router_logits", "topk_gates", "silu", "expert_ffn", "experts_forward",
    "layer_forward", "group_pairs", "set_threads", "get_threads",
]

_I64 = ctypes.c_int64
_P = ctypes.c_void_p
_lib = None
_threads = 1


def _load():
    global _lib
    if _lib is None:
        if _build.is_stale():
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.k3o_e2m1.restype = ctypes.c_double
        lib.k3o_e2m1.argtypes = [ctypes.c_int]
        lib.k3o_e8m0.restype = ctypes.c_double
        lib.k3o_e8m0.argtypes = [ctypes.c_int]
        lib.k3o_dequant.restype = ctypes.c_int
        lib.k3o_dequant.argtypes = [_P, _P, _I64, _I64, _P]
        lib.k3o_bf16_to_f64.restype = None
        lib.k3o_bf16_to_f64.argtypes = [_P, _I64, _P]
        lib.k3o_router_logits.restype = ctypes.c_int
        lib.k3o_router_logits.argtypes = [_P, _P, _P, _I64, _I64, _I64, _P]
        lib.k3o_topk_gates.restype = ctypes.c_int
        lib.k3o_topk_gates.argtypes = [_P, _I64, _I64, _I64, _P, _P]
        lib.k3o_topk_gates_split.restype = ctypes.c_int
        lib.k3o_topk_gates_split.argtypes = [_P, _P, _I64, _I64, _I64, _P, _P]
        lib.k3o_silu_array.restype = None
        lib.k3o_silu_array.argtypes = [_P, _I64, _P]
        lib.k3o_expert_ffn.restype = ctypes.c_int
        lib.k3o_expert_ffn.argtypes = [_P, _I64, _I64, _I64] + [_P] * 6 + [_P, _P, _P]
        lib.k3o_combine.restype = ctypes.c_int
        lib.k3o_combine.argtypes = [_P, _P, _P, _I64, _I64, _I64, _I64, _P]
        lib.k3o_group_pairs.restype = ctypes.c_int64
        lib.k3o_group_pairs.argtypes = [_P, _I64, _I64, _P, _P, _P]
        _lib = lib
    return _lib


def set_threads(n: int) -> None:
    """Host threads over which independent tokens are spread (>= 1)."""
    global _threads
    _threads = max(1, int(n))


def get_threads() -> int:
    return _threads


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_P) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc < 0:
        raise ValueError(f"oracle {what}: invalid arguments (status {rc})")


def _shards(n: int):
    """Contiguous row ranges, one per thread."""
    parts = min(_threads, max(n, 1))
    edges = np.linspace(0, n, parts + 1).astype(np.int64)
    return [(int(a), int(b)) for a, b in zip(edges[:-1], edges[1:]) if b > a]


def _run_sharded(n: int, fn):
    shards = _shards(n)
    if len(shards) <= 1:
        for a, b in shards:
            fn(a, b)
        return
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(shards)) as ex:
        for fut in [ex.submit(fn, a, b) for a, b in shards]:
            fut.result()


# ------------------------------------------------------------------ formats

def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code (OCP MX v1.0 FP4 element)."""
    return float(_load().k3o_e2m1(int(code)))


def e8m0_value(b: int) -> float:
    """Value of an E8M0 scale byte (OCP MX v1.0): 2^(b-127); 0xFF is NaN."""
    return float(_load().k3o_e8m0(int(b)))


E2M1_VALUES = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def dequant(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """W [rows][K] float64 from codes q [rows][K/2] and scales s [rows][K/32]."""
    q = _c(q, np.uint8)
    s = _c(s, np.uint8)
    rows, half = q.shape
    W = np.empty((rows, 2 * half), dtype=np.float64)
    _check(_load().k3o_dequant(_ptr(q), _ptr(s), rows, 2 * half, _ptr(W)), "dequant")
    return W


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    _load().k3o_bf16_to_f64(_ptr(b), b.size, _ptr(out))
    return out


# ------------------------------------------------------------------ router

def router_logits(x_bits: np.ndarray, router_w: np.ndarray,
                  bias: np.ndarray | None = None) -> np.ndarray:
    """fp32 logits [T][E]: fp64 sum of x*Wr rounded to fp32, + bias in fp32."""
    x = _c(np.atleast_2d(x_bits), np.uint16)
    w = _c(router_w, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    T, d = x.shape
    E = w.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    lib = _load()

    def run(a, b_):
        _check(lib.k3o_router_logits(_ptr(x[a:b_]), _ptr(w), _ptr(b), b_ - a, d, E,
                                     _ptr(out[a:b_])), "router_logits")
    _run_sharded(T, run)
    return out


def topk_gates(logits: np.ndarray, k: int, gate_logits: np.ndarray | None = None):
    """idx [T][k] int32 (logit descending, index ascending) and fp64 gates.
    With gate_logits, `logits` only choose the experts and the gates are the
    softmax of the chosen experts' gate_logits (the selection-only bias)."""
    lg = _c(np.atleast_2d(logits), np.float32)
    T, E = lg.shape
    idx = np.empty((T, k), dtype=np.int32)
    gate = np.empty((T, k), dtype=np.float64)
    if gate_logits is None:
        _check(_load().k3o_topk_gates(_ptr(lg), T, E, int(k), _ptr(idx), _ptr(gate)), "topk_gates")
    else:
        gl = _c(np.atleast_2d(gate_logits), np.float32)
        if gl.shape != lg.shape:
            raise ValueError("gate_logits must have the shape of logits")
        _check(_load().k3o_topk_gates_split(_ptr(lg), _ptr(gl), T, E, int(k), _ptr(idx),
                                            _ptr(gate)), "topk_gates_split")
    return idx, gate


# ------------------------------------------------------------------ expert

def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + exp(-z)) in fp64."""
    z = _c(z, np.float64)
    out = np.empty_like(z)
    _load().k3o_silu_array(_ptr(z), z.size, _ptr(out))
    return out


def _expert_rows(x64: np.ndarray, w: dict, want_h: bool, shard: bool = True):
    n, d = x64.shape
    f = w["gate_q"].shape[0]
    mats = [_c(w[name], np.uint8) for name in
            ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")]
    o = np.empty((n, d), dtype=np.float64)
    h = np.empty((n, f), dtype=np.float64) if want_h else None
    lib = _load()

    def run(a, b):
        hbuf = np.empty(f, dtype=np.float64)
        _check(lib.k3o_expert_ffn(_ptr(x64[a:b]), b - a, d, f, *[_ptr(m) for m in mats],
                                  _ptr(hbuf), _ptr(o[a:b]),
                                  _ptr(h[a:b]) if want_h else None), "expert_ffn")
    if shard:
        _run_sharded(n, run)
    else:
        run(0, n)
    return o, h


def expert_ffn(x: np.ndarray, w: dict, return_h: bool = False):
    """One SwiGLU expert on fp64 rows x [n][d]: o [n][d] (and h [n][f])."""
    x64 = _c(np.atleast_2d(x), np.float64)
    o, h = _expert_rows(x64, w, return_h)
    return (o, h) if return_h else o


def experts_forward(x_bits: np.ndarray, idx: np.ndarray, gate: np.ndarray,
                    experts, n_experts: int | None = None) -> np.ndarray:
    """y[t] = sum_j gate[t,j] * expert_{idx[t,j]}(x[t]), j in order, fp64.

    experts: callable e -> dict of the expert's six uint8 arrays; experts are
    fetched one at a time. A slot whose expert index lies outside
    [0, n_experts) is a failed expert and contributes zero (without
    n_experts, only negative indices are out of range)."""
    x64 = bf16_to_f64(np.atleast_2d(x_bits))
    idx = _c(np.atleast_2d(idx), np.int32)
    gate = _c(np.atleast_2d(gate), np.float64)
    T, k = idx.shape
    d = x64.shape[1]
    E = int(n_experts) if n_experts is not None else (int(idx.max()) + 1 if idx.size else 1)
    E = max(E, 1)
    outs = np.zeros((T, k, d), dtype=np.float64)
    work = [int(e) for e in np.unique(idx) if 0 <= e < E]

    def one(e):  # every pair routed to expert e; each row computed on its own
        ts, js = np.nonzero(idx == e)
        o, _ = _expert_rows(np.ascontiguousarray(x64[ts]), experts(e), False, shard=False)
        outs[ts, js] = o
    if _threads > 1 and len(work) > 1:
        with concurrent.futures.ThreadPoolExecutor(max_workers=_threads) as ex:
            for fut in [ex.submit(one, e) for e in work]:
                fut.result()
    else:
        for e in work:
            one(e)
    y = np.empty((T, d), dtype=np.float64)
    _check(_load().k3o_combine(_ptr(outs), _ptr(gate), _ptr(idx), T, k, d, E, _ptr(y)),
           "combine")
    return y


def layer_forward(x_bits, router_w, bias, experts, k: int, bias_select_only: bool = False):
    """Whole layer. Returns dict(y64, y32, idx, gate, logits). With
    bias_select_only the bias ranks the experts but the gates come from the
    unbiased logits (and `logits` are the unbiased ones)."""
    if bias_select_only and bias is not None:
        logits = router_logits(x_bits, router_w, None)
        idx, gate = topk_gates(router_logits(x_bits, router_w, bias), k, gate_logits=logits)
        y = experts_forward(x_bits, idx, gate, experts, n_experts=np.shape(router_w)[0])
        return {"y64": y, "y32": y.astype(np.float32), "idx": idx, "gate": gate,
                "logits": logits}
    logits = router_logits(x_bits, router_w, bias)
    idx, gate = topk_gates(logits, k)
    y = experts_forward(x_bits, idx, gate, experts, n_experts=np.shape(router_w)[0])
    return {"y64": y, "y32": y.astype(np.float32), "idx": idx, "gate": gate,
            "logits": logits}


# ------------------------------------------------------------------ grouping

def group_pairs(idx: np.ndarray, E: int):
    """counts [E], offsets [E+1], perm: pair ids t*k+j ordered by
    (expert, t, j); pairs with an expert outside [0, E) are left out."""
    flat = _c(np.asarray(idx).reshape(-1), np.int32)
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(flat.size, dtype=np.int32)
    n = _load().k3o_group_pairs(_ptr(flat), flat.size, int(E), _ptr(counts), _ptr(offsets),
                                _ptr(perm))
    _check(n, "group_pairs")
    return counts, offsets, perm[:n].copy()


if os.environ.get("K3ORACLE_THREADS"):
    set_threads(int(os.environ["K3ORACLE_THREADS"]))
