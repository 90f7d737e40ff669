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


def bf16_ulp(v):
    """Spacing of bfloat16 values at |v| (2^(e - 7) in the binade [2^e, 2^(e+1)),
    2^-133 below 2^-126)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a >= 2.0 ** -126, np.exp2(e - 7), 2.0 ** -133)


def check_bf16_glue(xg, x_ref, what, max_frac=1e-3):
    """A bf16 layer input formed in fp32 on the GPU against the oracle's
    (rounded once from float64): every element equal, or one bf16 step away
    (the fp32 normalisation landed on the other side of a rounding midpoint),
    and such elements rare.  Returns the number of one-step differences."""
    xg = np.asarray(xg, dtype=np.float64)
    x_ref = np.asarray(x_ref, dtype=np.float64)
    diff = xg != x_ref
    n = int(diff.sum())
    if n:
        step = np.maximum(bf16_ulp(xg[diff]), bf16_ulp(x_ref[diff]))
        far = np.abs(xg[diff] - x_ref[diff]) > step
        assert not far.any(), f"{what}: {int(far.sum())} elements differ by more than one bf16 step"
    assert n <= max_frac * xg.size, f"{what}: {n} of {xg.size} elements differ by one bf16 step"
    return n


def to_np(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def check_selection(L64, L32_gpu, idx_gpu, k):
    """Returns the number of tokens whose selection or slot order legitimately
    differs (near ties); raises AssertionError for any other difference.

    The slots are ordered by logit, so the same near-tie rule covers two
    selected experts whose order differs: each pair the GPU orders against the
    oracle's float64 logits must be within twice the token's logit error."""
    L32_gpu = np.asarray(L32_gpu, dtype=np.float32)
    # identical fp32 logits -> identical indices
    assert np.array_equal(M.topk(L32_gpu, k), idx_gpu), "top-k differs on identical logits"
    idx_o = M.topk(L64.astype(np.float32), k)
    flips = 0
    for t in range(L64.shape[0]):
        if np.array_equal(idx_o[t], idx_gpu[t]):
            continue
        err = np.max(np.abs(L32_gpu[t].astype(np.float64) - L64[t]))
        if set(idx_o[t].tolist()) != set(idx_gpu[t].tolist()):
            order = np.lexsort((np.arange(L64.shape[1]), -L64[t]))
            gap = L64[t, order[k - 1]] - L64[t, order[k]]
            assert gap <= 2 * err, f"token {t}: selection differs with gap {gap} > 2*{err}"
        g = idx_gpu[t]
        for a in range(k):
            for b in range(a + 1, k):
                ea, eb = int(g[a]), int(g[b])
                # the GPU puts ea first: against float64 that needs L[ea] >= L[eb]
                # (lower id first on ties), or a gap within the logit error
                if L64[t, ea] < L64[t, eb] or (L64[t, ea] == L64[t, eb] and ea > eb):
                    gap = L64[t, eb] - L64[t, ea]
                    assert gap <= 2 * err, f"token {t}: slot order of {ea}, {eb} differs with gap {gap} > 2*{err}"
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
    # and token by token
    yg = np.asarray(gpu["y"], dtype=np.float64)
    per_tok = np.linalg.norm(yg - y_ref, axis=1) / np.maximum(np.linalg.norm(y_ref, axis=1), 1e-300)
    stats["rel_l2_token_max"] = float(per_tok.max())
    assert per_tok.max() <= tol, f"token {int(per_tok.argmax())}: rel-L2 {per_tok.max():.3e} > {tol:.1e}"
    return stats
