"""Shared helpers of the GPU parity tests: compare one GPU layer pass with the
oracle on the same inputs (teacher forcing: the oracle takes the GPU's own
bf16 layer input).

Selection rule at near-ties: for identical fp32 logits the indices must match
exactly.  End to end, a token's selection may differ from the oracle's only if
the oracle's float64 gap between the last selected and the first unselected
logit is at most 2 * max_e |L32_gpu - L| for that token; such tokens are counted
and their outputs are checked with the GPU's selection.
"""

import numpy as np
import torch

from oracle import formats as F
from oracle import moe as M


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def to_np(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def check_selection(L64, L32_gpu, idx_gpu, k):
    """Returns the number of tokens whose selection legitimately differs (near
    ties); raises AssertionError for any other difference."""
    L32_gpu = np.asarray(L32_gpu, dtype=np.float32)
    # identical fp32 logits -> identical indices
    assert np.array_equal(M.topk(L32_gpu, k), idx_gpu), "top-k differs on identical logits"
    idx_o = M.topk(L64.astype(np.float32), k)
    flips = 0
    for t in range(L64.shape[0]):
        if np.array_equal(idx_o[t], idx_gpu[t]):
            continue
        order = np.lexsort((np.arange(L64.shape[1]), -L64[t]))
        gap = L64[t, order[k - 1]] - L64[t, order[k]]
        err = np.max(np.abs(L32_gpu[t].astype(np.float64) - L64[t]))
        assert gap <= 2 * err, f"token {t}: selection differs with gap {gap} > 2*{err}"
        flips += 1
    return flips


def check_layer(layer_np, x_np, gpu, out_dtype, tol, token_ids=None):
    """Compare one layer.  layer_np: oracle layer (host copy); x_np: float64
    view of the GPU's layer input for the checked tokens; gpu: dict with logits
    (fp32 [T,E] or None), idx, w and y for the checked tokens.  Returns stats."""
    k = layer_np["k"]
    L64 = M.router_logits(layer_np["router_w"], layer_np["router_b"], x_np)
    stats = {"flips": 0}
    if gpu.get("logits") is not None:
        L32 = gpu["logits"]
        stats["logit_err"] = float(np.max(np.abs(L32.astype(np.float64) - L64)))
        stats["flips"] = check_selection(L64, L32, gpu["idx"], k)
    idx = gpu["idx"]
    w = M.gate_weights(L64, idx)
    assert np.allclose(gpu["w"], w, rtol=2e-5, atol=1e-6), "gate weights differ"
    y_ref = M.layer_from_selection(layer_np, x_np, idx, w, out_dtype="f64", cache=False)
    err = rel_l2(gpu["y"], y_ref)
    stats["rel_l2"] = err
    assert err <= tol, f"rel-L2 {err:.3e} > {tol:.1e}"
    return stats
