"""Oracle: the routed-expert MoE feed-forward layer, written out in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The method reaches, up to rounding order, a result with a plain definition: a
top-k routed mixture of SwiGLU experts plus an always-on shared expert, with the
expert weights dequantised exactly.  This module is that definition, step by
step, with no blocking, fusion or reordering:

1. router logits  L = W_r x + b                 (float64; products are exact)
2. top-k          the k largest float32(L), descending, lower index first on ties
3. gate weights   softmax over the k selected logits (renormalised; sums to 1)
4. expert plan    per-expert counts, exclusive offsets, a stable scatter of the
                  (token, slot) pairs by expert, the inverse map and the active
                  list (the "device-planned MoE tail" of "What was changed",
                  UD-IQ2_XS (L4 fix) page)
5. experts        h = silu(W_g x) * (W_u x),  o = W_d h   (per routed pair)
6. shared expert  s = the same FFN with the shared weights, weight 1
7. combine        y_t = s_t + sum_j w[t, j] * o[(t, j)]
8. stack glue     x_l = bf16(rmsnorm(h_l)), h_{l+1} = h_l + y_l: the helpers
                  that join stacked layers (rmsnorm_to_bf16, residual_add)

Routing picks only selected experts per token ("RAM and VRAM Hold Different
Parts of the Expert Weights", setup-guide page).  The rest of the layer (router,
softmax/top-k, SwiGLU, shared expert, combine) follows the workload definition
of the routed-expert layer; where that definition leaves a point open the
reading taken is the plainest one and is listed with the design notes.
"""

import numpy as np

from . import formats


# ----------------------------------------------------------------------------
# Step 1-3: routing
# ----------------------------------------------------------------------------

def router_logits(router_w, router_b, x):
    """L[t, e] = sum_i W_r[e, i] * x[t, i] + b[e] in float64.

    router_w: [E, d] float32; router_b: [E] float32 or None; x: [T, d] (bf16
    values or float32).  Each product of two values with <= 24 significant bits
    is exact in float64; only the summation rounds.
    """
    W = np.asarray(router_w, dtype=np.float64)
    X = np.asarray(x, dtype=np.float64)
    L = X @ W.T
    if router_b is not None:
        L = L + np.asarray(router_b, dtype=np.float64)[None, :]
    return L


def topk(logits32, k):
    """Indices of the k largest float32 logits per token, in slot order:
    descending logit, lower expert index first when logits tie.

    logits32: [T, E] float32.  Returns int32 [T, k].
    """
    L = np.asarray(logits32, dtype=np.float32)
    T, E = L.shape
    out = np.empty((T, k), dtype=np.int32)
    ids = np.arange(E)
    for t in range(T):
        # np.lexsort sorts by the last key first: primary key -L, then index.
        order = np.lexsort((ids, -L[t].astype(np.float64)))
        out[t] = order[:k]
    return out


def gate_weights(logits, idx):
    """w[t, j] = exp(L[t, idx[t, j]] - m) / sum_j' exp(L[t, idx[t, j']] - m),
    float64, m = the largest selected logit.  This equals a softmax over all
    experts followed by top-k and renormalisation (the full denominator cancels).
    """
    L = np.asarray(logits, dtype=np.float64)
    T, k = idx.shape
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        sel = L[t, idx[t]]
        m = sel.max()
        e = np.exp(sel - m)
        w[t] = e / e.sum()
    return w


def route(router_w, router_b, x, k):
    """Steps 1-3.  Returns (L float64 [T,E], L32 float32 [T,E], idx int32 [T,k], w float64 [T,k])."""
    L = router_logits(router_w, router_b, x)
    L32 = L.astype(np.float32)
    idx = topk(L32, k)
    w = gate_weights(L, idx)
    return L, L32, idx, w


# ----------------------------------------------------------------------------
# Step 4: the expert plan
# ----------------------------------------------------------------------------

def plan(idx, E):
    """Build the expert plan from the top-k indices idx [T, k].

    counts[e]      number of (t, j) pairs routed to expert e
    offsets[e]     exclusive prefix sum of counts; offsets[E] = T*k
    row_token[r]   token of plan row r; rows of expert e are
                   [offsets[e], offsets[e+1]) in ascending token order
    row_slot[r]    slot j of plan row r
    slot_row[t*k + j]  the plan row of pair (t, j)
    active         expert ids with counts > 0 ascending, padded with -1 to E
    n_active       number of active experts

    Pairs whose expert id is outside [0, E) are dropped (they get no row; their
    slot_row entry is -1) and reported through bit 1 of ``error``.  A top-k
    selection never names an expert twice for one token, so a plan built from
    one has distinct ids per token; for an index array that repeats an id
    within a token, the pair with the lowest slot j is kept and every later
    repeat is dropped the same way and reported through bit 4.
    """
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    in_range = (idx >= 0) & (idx < E)
    valid = in_range.copy()
    for t in range(T):
        for j in range(k):
            if in_range[t, j] and idx[t, j] in idx[t, :j][in_range[t, :j]]:
                valid[t, j] = False
    error = (0 if in_range.all() else 1) | (0 if (valid == in_range).all() else 4)
    counts = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            if valid[t, j]:
                counts[idx[t, j]] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    n_rows = int(offsets[E])
    row_token = np.full(T * k, -1, dtype=np.int64)
    row_slot = np.full(T * k, -1, dtype=np.int64)
    slot_row = np.full(T * k, -1, dtype=np.int64)
    fill = offsets[:E].copy()
    for t in range(T):              # ascending t gives the stable order
        for j in range(k):
            if not valid[t, j]:
                continue
            e = idx[t, j]
            r = fill[e]
            fill[e] += 1
            row_token[r] = t
            row_slot[r] = j
            slot_row[t * k + j] = r
    active = np.full(E, -1, dtype=np.int64)
    act = [e for e in range(E) if counts[e] > 0]
    active[:len(act)] = act
    return {
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "row_token": row_token.astype(np.int32),
        "row_slot": row_slot.astype(np.int32),
        "slot_row": slot_row.astype(np.int32),
        "active": active.astype(np.int32),
        "n_active": np.int32(len(act)),
        "n_rows": n_rows,
        "error": np.int32(error),
    }


# ----------------------------------------------------------------------------
# Steps 5-7: experts, shared expert, combine
# ----------------------------------------------------------------------------

def silu(z):
    """silu(z) = z / (1 + exp(-z)), evaluated without overflow for either sign."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = z[~pos] * ez / (1.0 + ez)
    return out


def expert_ffn(Wg, Wu, Wd, x):
    """SwiGLU expert on one or more tokens: o = W_d (silu(W_g x) * (W_u x)).

    Wg, Wu: [f, d]; Wd: [d, f] float64; x: [n, d].  Returns (h [n, f], o [n, d]).
    """
    X = np.asarray(x, dtype=np.float64)
    g = X @ Wg.T
    u = X @ Wu.T
    h = silu(g) * u
    o = h @ Wd.T
    return h, o


class DenseExperts:
    """Exactly dequantised expert weights of one layer, decoded on demand.

    ``mats`` maps 'gate' / 'up' / 'down' to a dict with keys type, codes, scales
    and (NVFP4) tensor_scale, each indexed by expert on the first axis.
    """

    def __init__(self, mats, cache=True):
        self.mats = mats
        self.cache = cache
        self._cache = {}

    def weight(self, name, e):
        key = (name, int(e))
        if key in self._cache:
            return self._cache[key]
        m = self.mats[name]
        ts = None if m.get("tensor_scale") is None else m["tensor_scale"][e]
        w = formats.dequant(m["type"], m["codes"][e], m["scales"][e], ts)
        if self.cache:
            self._cache[key] = w
        return w

    def ffn(self, e, x):
        return expert_ffn(self.weight("gate", e), self.weight("up", e), self.weight("down", e), x)


def moe_layer(layer, x, out_dtype="f32", return_parts=False):
    """One routed-expert layer on tokens x [T, d] (float64 view of the inputs).

    layer: dict with d, f, E, k, router_w, router_b, routed (mats dict as in
    DenseExperts) and shared (mats dict with one expert, or None).
    Returns y rounded once at the end to float32 ('f32') or bfloat16 ('bf16'),
    as float64; with return_parts also the intermediates.
    """
    k = layer["k"]
    E = layer["E"]
    L, L32, idx, w = route(layer["router_w"], layer.get("router_b"), x, k)
    p = plan(idx, E)
    return layer_from_selection(layer, x, idx, w, p, out_dtype, return_parts, extra={"L": L, "L32": L32})


def layer_from_selection(layer, x, idx, w, p=None, out_dtype="f32", return_parts=False, extra=None,
                         cache=True):
    """Steps 5-7 for a given selection idx [T,k] and weights w [T,k].  With
    cache=False each expert's weights are decoded, used and dropped (large
    layers)."""
    X = np.asarray(x, dtype=np.float64)
    T, d = X.shape
    k = idx.shape[1]
    if p is None:
        p = plan(idx, layer["E"])
    routed = DenseExperts(layer["routed"], cache=cache)
    o_rows = np.zeros((T * k, d))
    h_rows = np.zeros((T * k, layer["f"]))
    for e in range(layer["E"]):
        lo, hi = p["offsets"][e], p["offsets"][e + 1]
        if hi == lo:
            continue
        toks = p["row_token"][lo:hi]
        h, o = routed.ffn(e, X[toks])
        o_rows[lo:hi] = o
        h_rows[lo:hi] = h
    if layer.get("shared") is not None:
        shared = DenseExperts(layer["shared"], cache=cache)
        h_s, s = shared.ffn(0, X)
    else:
        h_s, s = None, np.zeros((T, d))
    y = s.copy()
    for t in range(T):
        for j in range(k):
            r = p["slot_row"][t * k + j]
            if r >= 0:
                y[t] += w[t, j] * o_rows[r]
    y_out = round_output(y, out_dtype)
    if not return_parts:
        return y_out
    parts = {"idx": idx, "w": w, "plan": p, "h_rows": h_rows, "o_rows": o_rows,
             "h_shared": h_s, "shared": s, "y64": y}
    if extra:
        parts.update(extra)
    return y_out, parts


def round_output(y, out_dtype):
    """Round the float64 combine once: to float32 or to bfloat16 (RNE)."""
    if out_dtype == "f32":
        return np.asarray(y, dtype=np.float64).astype(np.float32).astype(np.float64)
    if out_dtype == "bf16":
        return formats.round_to_bf16(y)
    if out_dtype == "f64":
        return np.asarray(y, dtype=np.float64)
    raise ValueError(out_dtype)


def dense_mixture(layer, x):
    """(1/E) * sum_e FFN_e(x) + shared(x): the value a uniform router with k = E
    must reproduce (every expert selected with weight 1/E)."""
    X = np.asarray(x, dtype=np.float64)
    routed = DenseExperts(layer["routed"])
    acc = np.zeros_like(X)
    for e in range(layer["E"]):
        acc += routed.ffn(e, X)[1]
    acc /= layer["E"]
    if layer.get("shared") is not None:
        acc += DenseExperts(layer["shared"]).ffn(0, X)[1]
    return acc


# ----------------------------------------------------------------------------
# Step 8: layer chaining for the multi-layer stack
# ----------------------------------------------------------------------------

RMS_EPS = 1e-6


def rmsnorm_to_bf16(h):
    """x = bf16(h / sqrt(mean(h^2) + 1e-6)) per token (unit weight).

    The pages do not say what joins the MoE layers of the stack; the reading is
    a pre-norm residual chain so that every layer sees unit-RMS inputs."""
    H = np.asarray(h, dtype=np.float64)
    r = np.sqrt(np.mean(H * H, axis=-1, keepdims=True) + RMS_EPS)
    return formats.round_to_bf16(H / r)


def residual_add(h, y):
    """h_{l+1} = h_l + y_l, carried in float32 like the residual stream."""
    return (np.asarray(h, dtype=np.float32) + np.asarray(y, dtype=np.float32)).astype(np.float64)
