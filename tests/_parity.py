"""Comparison rules shared by the GPU parity tests.

* Routing: indices must match the oracle exactly, except where the oracle's
  k-th and (k+1)-th fp32 logits differ by less than 1e-5 (the selected set
  may differ) or where adjacent selected logits differ by less than 1e-5
  (their order may differ). Such tokens are logged and their outputs are
  checked against the oracle run with the GPU's routing.
* Outputs: max |y_gpu - y_ref| <= 2e-2 * RMS(y_ref) over the checked tokens.
"""
from __future__ import annotations

import numpy as np

TIE_EPS = 1e-5
OUT_TOL = 2e-2


def compare_routing(gpu_idx, ref_logits, ref_idx, k):
    """Returns (excused_token_list, log_lines). Raises AssertionError on a
    mismatch that no near tie explains."""
    gpu_idx = np.asarray(gpu_idx)
    ref_idx = np.asarray(ref_idx)
    excused, log = [], []
    bad = np.nonzero(np.any(gpu_idx != ref_idx, axis=1))[0]
    for t in bad:
        lg = ref_logits[t].astype(np.float64)
        order = np.lexsort((np.arange(len(lg)), -lg))
        vals = lg[order]
        g, r = gpu_idx[t], ref_idx[t]
        ok = True
        if set(g.tolist()) != set(r.tolist()):
            ok = len(vals) > k and abs(vals[k - 1] - vals[k]) < TIE_EPS
            # every expert the GPU picked must be within the tie band or selected
            band = vals[k - 1] - TIE_EPS
            ok = ok and all(lg[e] >= band for e in g)
        else:
            # same set, different order: each swapped position must be a near tie
            for j in range(k):
                if g[j] != r[j] and abs(lg[g[j]] - lg[r[j]]) >= TIE_EPS:
                    ok = False
        assert ok, (f"token {t}: routing mismatch not explained by a near tie: gpu {g.tolist()} "
                    f"ref {r.tolist()} logits {[float(lg[e]) for e in r]}")
        excused.append(int(t))
        log.append(f"near tie excused: token {t} gpu {g.tolist()} ref {r.tolist()}")
    return excused, log


def check_output(y_gpu, y_ref, what=""):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite GPU output"
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    err = float(np.max(np.abs(y_gpu - y_ref))) if y_ref.size else 0.0
    assert err <= OUT_TOL * rms, f"{what}: max abs err {err:.4g} > {OUT_TOL} * rms {rms:.4g} (ratio {err / rms:.4g})"
    return err / rms if rms > 0 else 0.0
