"""Pins for the oracle's layer arithmetic (CPU only).

Each step is checked against brute force on tiny inputs, exact rational
arithmetic, independent library routines or closed-form special cases, chosen
so that a plausible mistake (a dropped term, a wrong sign or index, a transposed
operand) fails at least one of them; the mutation tests at the end plant such
mistakes into the oracle and check that a pin catches each one."""

import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import moe as M

import exact_round as ER
from test_oracle_formats import test_bf16_round_once_against_exact_rationals as _pin_bf16
from test_oracle_formats import test_fp16_exhaustive_against_numpy as _pin_fp16
from test_oracle_formats import test_iq4_nl_nibble_order_and_exact_values as _pin_iq4_order


# ---------------------------------------------------------------- tiny layers

def _rand_matrix(rng, qtype, n, rows, cols, scale_lo=0.002, scale_hi=0.02):
    if qtype == "q8_0":
        codes = rng.integers(-127, 128, size=(n, rows, cols)).astype(np.int8)
        sc = np.float16(rng.uniform(scale_lo, scale_hi, size=(n, rows, cols // 32)) / 127 * 8)
        return {"type": qtype, "codes": codes, "scales": sc.view(np.uint16), "tensor_scale": None}
    if qtype == "iq4_nl":
        codes = rng.integers(0, 256, size=(n, rows, cols // 2)).astype(np.uint8)
        sc = np.float16(rng.uniform(scale_lo, scale_hi, size=(n, rows, cols // 32)) / 127 * 8)
        sc = np.where(rng.random(sc.shape) < 0.5, sc, -sc).astype(np.float16)
        return {"type": qtype, "codes": codes, "scales": sc.view(np.uint16), "tensor_scale": None}
    if qtype == "nvfp4":
        codes = rng.integers(0, 256, size=(n, rows, cols // 2)).astype(np.uint8)
        sc = rng.integers(0x20, 0x50, size=(n, rows, cols // 16)).astype(np.uint8)
        ts = rng.uniform(1e-3, 1e-2, size=n).astype(np.float32)
        return {"type": qtype, "codes": codes, "scales": sc, "tensor_scale": ts}
    if qtype == "q5_1":
        codes = rng.integers(0, 256, size=(n, rows, cols // 2)).astype(np.uint8)
        nb = cols // 32
        d = np.float16(rng.uniform(scale_lo, scale_hi, size=(n, rows, nb)) / 31 * 4).view(np.uint16)
        m = np.float16(-rng.uniform(scale_lo, scale_hi, size=(n, rows, nb)) * 2).view(np.uint16)
        word = rng.integers(0, 2 ** 32, size=(n, rows, nb), dtype=np.uint64).astype(np.uint32)
        rec = np.stack([d & 0xFF, d >> 8, m & 0xFF, m >> 8, word & 0xFF, (word >> 8) & 0xFF,
                        (word >> 16) & 0xFF, word >> 24], axis=-1).astype(np.uint8)
        return {"type": qtype, "codes": codes, "scales": rec.reshape(n, rows, nb * 8), "tensor_scale": None}
    raise ValueError(qtype)


def tiny_layer(seed=0, d=32, f=32, E=6, k=2, qtypes=("q8_0", "iq4_nl", "nvfp4"), shared=True, bias=True):
    rng = np.random.default_rng(seed)
    qg, qu, qd = qtypes
    layer = {
        "d": d, "f": f, "E": E, "k": k,
        "router_w": rng.normal(0, 0.3, size=(E, d)).astype(np.float32),
        "router_b": rng.normal(0, 0.5, size=E).astype(np.float32) if bias else None,
        "routed": {"gate": _rand_matrix(rng, qg, E, f, d), "up": _rand_matrix(rng, qu, E, f, d),
                   "down": _rand_matrix(rng, qd, E, d, f)},
        "shared": None,
    }
    if shared:
        layer["shared"] = {"gate": _rand_matrix(rng, qg, 1, f, d), "up": _rand_matrix(rng, qu, 1, f, d),
                           "down": _rand_matrix(rng, qd, 1, d, f)}
    return layer


def tiny_tokens(seed, T, d):
    rng = np.random.default_rng(100 + seed)
    return F.round_to_bf16(rng.normal(0, 1, size=(T, d)))


def _dense(layer, name, e, shared=False):
    m = (layer["shared"] if shared else layer["routed"])[name]
    ts = None if m["tensor_scale"] is None else m["tensor_scale"][e]
    return F.dequant(m["type"], m["codes"][e], m["scales"][e], ts)


# ---------------------------------------------------------------- router

def test_router_logits_match_exact_rational_sum():
    layer = tiny_layer(1, d=32, E=5)
    x = tiny_tokens(1, 3, 32)
    L = M.router_logits(layer["router_w"], layer["router_b"], x)
    for t in range(3):
        for e in range(5):
            exact = sum(Fraction(float(layer["router_w"][e, i])) * Fraction(float(x[t, i])) for i in range(32))
            exact += Fraction(float(layer["router_b"][e]))
            bound = 1e-15 * sum(abs(float(layer["router_w"][e, i]) * float(x[t, i])) for i in range(32))
            assert abs(L[t, e] - float(exact)) <= bound + 1e-300


def _topk_bruteforce(v, k):
    E = len(v)
    beats = lambda i, j: (v[i] > v[j]) or (v[i] == v[j] and i < j)  # noqa: E731
    valid = []
    for S in itertools.combinations(range(E), k):
        rest = [j for j in range(E) if j not in S]
        if all(beats(i, j) for i in S for j in rest):
            valid.append(S)
    assert len(valid) == 1
    S = list(valid[0])
    # slot order: selection sort under the same relation
    out = []
    while S:
        best = S[0]
        for i in S[1:]:
            if beats(i, best):
                best = i
        out.append(best)
        S.remove(best)
    return out


@pytest.mark.parametrize("seed", range(20))
def test_topk_matches_bruteforce_with_ties(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(2, 9))
    k = int(rng.integers(1, E + 1))
    # few distinct values -> many ties
    v = rng.integers(-3, 4, size=(4, E)).astype(np.float32) * np.float32(0.25)
    got = M.topk(v, k)
    for t in range(4):
        assert list(got[t]) == _topk_bruteforce(list(v[t]), k)


def test_topk_all_equal_gives_lowest_indices():
    v = np.zeros((3, 16), dtype=np.float32)
    assert np.array_equal(M.topk(v, 5), np.tile(np.arange(5), (3, 1)))


def test_topk_matches_stable_argsort():
    rng = np.random.default_rng(9)
    v = rng.normal(size=(50, 64)).astype(np.float32)
    v[:, 10] = v[:, 20]  # exact ties
    got = M.topk(v, 8)
    ref = np.argsort(-v.astype(np.float64), axis=1, kind="stable")[:, :8]
    assert np.array_equal(got, ref)


def test_gate_weights_sum_to_one_and_equal_renormalised_softmax():
    rng = np.random.default_rng(3)
    L = rng.normal(0, 3, size=(10, 32))
    idx = M.topk(L.astype(np.float32), 6)
    w = M.gate_weights(L, idx)
    assert np.allclose(w.sum(1), 1.0, atol=1e-15, rtol=0)
    full = np.exp(L - L.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    sel = np.take_along_axis(full, idx.astype(np.int64), 1)
    assert np.allclose(w, sel / sel.sum(1, keepdims=True), atol=1e-15, rtol=0)
    # descending by slot
    assert np.all(np.diff(w, axis=1) <= 1e-15)


def test_gate_weight_k1_is_one():
    L = np.random.default_rng(4).normal(size=(5, 7))
    idx = M.topk(L.astype(np.float32), 1)
    assert np.all(M.gate_weights(L, idx) == 1.0)


# ---------------------------------------------------------------- plan

def _check_plan_invariants(idx, E, p):
    T, k = idx.shape
    assert p["counts"].sum() == T * k
    assert np.all(np.diff(p["offsets"]) >= 0) and p["offsets"][0] == 0 and p["offsets"][E] == T * k
    pairs = set(zip(p["row_token"].tolist(), p["row_slot"].tolist()))
    assert pairs == {(t, j) for t in range(T) for j in range(k)}
    for r in range(T * k):
        assert p["slot_row"][p["row_token"][r] * k + p["row_slot"][r]] == r
        e = idx[p["row_token"][r], p["row_slot"][r]]
        assert p["offsets"][e] <= r < p["offsets"][e + 1]
    for e in range(E):
        toks = p["row_token"][p["offsets"][e]:p["offsets"][e + 1]]
        assert np.all(np.diff(toks) > 0)  # ascending tokens, each token once


@pytest.mark.parametrize("seed", range(8))
def test_plan_matches_library_routines(seed):
    rng = np.random.default_rng(seed)
    T, E, k = int(rng.integers(1, 40)), int(rng.integers(2, 40)), 0
    k = int(rng.integers(1, min(E, 8) + 1))
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    p = M.plan(idx, E)
    _check_plan_invariants(idx, E, p)
    assert np.array_equal(p["counts"], np.bincount(idx.ravel(), minlength=E))
    assert np.array_equal(p["offsets"][1:], np.cumsum(np.bincount(idx.ravel(), minlength=E)))
    order = np.argsort(idx.ravel(), kind="stable")
    assert np.array_equal(p["row_token"], order // k)
    assert np.array_equal(p["row_slot"], order % k)
    act = np.flatnonzero(np.bincount(idx.ravel(), minlength=E))
    assert p["n_active"] == len(act)
    assert np.array_equal(p["active"][:len(act)], act) and np.all(p["active"][len(act):] == -1)
    assert p["error"] == 0


def test_plan_drops_out_of_range_ids_and_flags_error():
    idx = np.array([[0, 5], [1, -1], [2, 1]], dtype=np.int32)
    p = M.plan(idx, 3)
    assert p["error"] == 1
    assert p["counts"].tolist() == [1, 2, 1]
    assert p["slot_row"][1] == -1 and p["slot_row"][3] == -1
    assert p["offsets"][3] == 4


def test_plan_keeps_first_of_repeated_ids():
    """A repeated id within a token: the lowest slot keeps its row, later
    repeats are dropped exactly as an out-of-range id is, with bit 4 set."""
    rng = np.random.default_rng(21)
    T, k, E = 9, 4, 6
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[2, 3] = idx[2, 0]
    idx[5, 1] = idx[5, 2] = idx[5, 3] = idx[5, 0]
    idx[7, 2] = idx[7, 1]
    idx[8, 0] = -3       # out of range first ...
    idx[8, 3] = -3       # ... a repeated out-of-range id is only out of range
    p = M.plan(idx, E)
    assert p["error"] == 1 | 4
    ref = idx.copy()
    ref[2, 3] = ref[5, 1] = ref[5, 2] = ref[5, 3] = ref[7, 2] = -1
    q = M.plan(ref, E)
    assert q["error"] == 1
    for n in ("counts", "offsets", "row_token", "row_slot", "slot_row", "active"):
        assert np.array_equal(p[n], q[n]), n
    assert p["slot_row"][2 * k + 0] >= 0 and p["slot_row"][2 * k + 3] == -1
    assert p["n_rows"] == T * k - 5 - 2


# ---------------------------------------------------------------- experts / layer

def _silu_exact_ref(z):
    return z / (1.0 + np.exp(-z))


def test_silu_against_plain_formula_and_extremes():
    z = np.linspace(-30, 30, 1001)
    assert np.allclose(M.silu(z), _silu_exact_ref(z), rtol=1e-14, atol=1e-300)
    big = np.array([-1000.0, 1000.0])
    assert np.array_equal(M.silu(big), np.array([-0.0, 1000.0]))
    assert M.silu(np.array([0.0]))[0] == 0.0


@pytest.mark.parametrize("qtypes", [("q8_0", "q8_0", "q8_0"), ("iq4_nl", "iq4_nl", "iq4_nl"),
                                    ("nvfp4", "nvfp4", "nvfp4"), ("iq4_nl", "iq4_nl", "q8_0"),
                                    ("iq4_nl", "iq4_nl", "q5_1")])
def test_layer_matches_bruteforce_loops(qtypes):
    d, f, E, k, T = 32, 32, 5, 2, 3
    layer = tiny_layer(11, d=d, f=f, E=E, k=k, qtypes=qtypes)
    x = tiny_tokens(11, T, d)
    y = M.moe_layer(layer, x, out_dtype="f64")
    # brute force: per token, per selected expert, per element
    W = {(n, e): _dense(layer, n, e) for n in ("gate", "up", "down") for e in range(E)}
    S = {n: _dense(layer, n, 0, shared=True) for n in ("gate", "up", "down")}
    for t in range(T):
        logits = [sum(float(layer["router_w"][e, i]) * x[t, i] for i in range(d)) + float(layer["router_b"][e])
                  for e in range(E)]
        sel = _topk_bruteforce([np.float32(v) for v in logits], k)
        m = max(logits[e] for e in sel)
        ex = [np.exp(logits[e] - m) for e in sel]
        wts = [v / sum(ex) for v in ex]

        def ffn(Wg, Wu, Wd):
            h = []
            for r in range(f):
                g = sum(Wg[r, i] * x[t, i] for i in range(d))
                u = sum(Wu[r, i] * x[t, i] for i in range(d))
                h.append(g / (1 + np.exp(-g)) * u)
            return [sum(Wd[o, r] * h[r] for r in range(f)) for o in range(d)]

        want = np.array(ffn(S["gate"], S["up"], S["down"]))
        for wj, e in zip(wts, sel):
            want += wj * np.array(ffn(W[("gate", e)], W[("up", e)], W[("down", e)]))
        assert np.allclose(y[t], want, rtol=1e-12, atol=1e-12)


def test_k_equals_E_with_uniform_router_is_dense_mixture():
    layer = tiny_layer(12, E=6, k=6)
    layer["router_w"] = np.zeros_like(layer["router_w"])
    layer["router_b"] = None
    x = tiny_tokens(12, 4, 32)
    y = M.moe_layer(layer, x, out_dtype="f64")
    assert np.allclose(y, M.dense_mixture(layer, x), rtol=1e-13, atol=1e-14)
    _, parts = M.moe_layer(layer, x, out_dtype="f64", return_parts=True)
    assert np.allclose(parts["w"], 1.0 / 6, atol=1e-16)


def test_zero_scale_block_contributes_nothing():
    layer = tiny_layer(13, qtypes=("iq4_nl", "q8_0", "nvfp4"))
    x = tiny_tokens(13, 3, 32)
    for name, blk_elems in (("gate", 32), ("up", 32), ("down", 16)):
        a = tiny_layer(13, qtypes=("iq4_nl", "q8_0", "nvfp4"))
        b = tiny_layer(13, qtypes=("iq4_nl", "q8_0", "nvfp4"))
        for L in (a, b):
            for e in range(L["E"]):
                L["routed"][name]["scales"][e][:, 0] = 0
        # change the codes under the zeroed scale in b only
        codes = b["routed"][name]["codes"]
        if codes.dtype == np.int8:
            codes[:, :, :blk_elems] = -codes[:, :, :blk_elems] // 2
        else:
            codes[:, :, :blk_elems // 2] ^= 0x5A
        assert np.array_equal(M.moe_layer(a, x, "f64"), M.moe_layer(b, x, "f64"))
    del layer


def test_zero_gate_gives_shared_only():
    layer = tiny_layer(14, qtypes=("q8_0", "iq4_nl", "iq4_nl"))
    for e in range(layer["E"]):
        layer["routed"]["gate"]["scales"][e][:] = 0
    x = tiny_tokens(14, 3, 32)
    S = {n: _dense(layer, n, 0, shared=True) for n in ("gate", "up", "down")}
    _, s = M.expert_ffn(S["gate"], S["up"], S["down"], x)
    assert np.allclose(M.moe_layer(layer, x, "f64"), s, rtol=1e-14, atol=1e-15)


def test_one_hot_expert_closed_form():
    d = f = 32
    p, i_out, r_mid = 7, 19, 3
    a, b, c = np.float16(0.75), np.float16(-1.5), np.float16(0.125)
    def q8(rows, cols, rr, cc, val):
        codes = np.zeros((1, rows, cols), np.int8)
        codes[0, rr, cc] = 1
        sc = np.zeros((1, rows, cols // 32), np.float16)
        sc[0, rr, cc // 32] = val
        return {"type": "q8_0", "codes": codes, "scales": sc.view(np.uint16), "tensor_scale": None}
    layer = {"d": d, "f": f, "E": 1, "k": 1, "router_w": np.zeros((1, d), np.float32), "router_b": None,
             "routed": {"gate": q8(f, d, r_mid, p, a), "up": q8(f, d, r_mid, p, b), "down": q8(d, f, i_out, r_mid, c)},
             "shared": None}
    x = tiny_tokens(15, 2, d)
    y = M.moe_layer(layer, x, "f64")
    for t in range(2):
        g = float(a) * x[t, p]
        want = float(c) * (g / (1 + np.exp(-g))) * (float(b) * x[t, p])
        assert np.isclose(y[t, i_out], want, rtol=1e-15, atol=0)
        assert np.count_nonzero(y[t]) <= 1


def test_swapping_experts_with_router_rows_is_invariant():
    layer = tiny_layer(16, E=6, k=2)
    x = tiny_tokens(16, 5, 32)
    y = M.moe_layer(layer, x, "f64")
    perm = np.array([3, 1, 0, 5, 4, 2])
    sw = tiny_layer(16, E=6, k=2)
    sw["router_w"] = layer["router_w"][perm]
    sw["router_b"] = layer["router_b"][perm]
    for n in ("gate", "up", "down"):
        for key in ("codes", "scales"):
            sw["routed"][n][key] = layer["routed"][n][key][perm]
        if layer["routed"][n]["tensor_scale"] is not None:
            sw["routed"][n]["tensor_scale"] = layer["routed"][n]["tensor_scale"][perm]
    assert np.allclose(M.moe_layer(sw, x, "f64"), y, rtol=1e-13, atol=1e-15)


def test_token_output_independent_of_batch():
    layer = tiny_layer(17)
    x = tiny_tokens(17, 6, 32)
    y = M.moe_layer(layer, x, "f64")
    for t in range(6):
        # BLAS may sum in a different order for a different batch size
        assert np.allclose(M.moe_layer(layer, x[t:t + 1], "f64")[0], y[t], rtol=1e-13, atol=1e-16)


def test_output_rounding_once():
    layer = tiny_layer(18)
    x = tiny_tokens(18, 2, 32)
    y64 = M.moe_layer(layer, x, "f64")
    assert np.array_equal(M.moe_layer(layer, x, "f32"), y64.astype(np.float32).astype(np.float64))
    assert np.array_equal(M.moe_layer(layer, x, "bf16"), F.round_to_bf16(y64))


# ---------------------------------------------------------------- stack glue

def _glue_rows(seed=19, d=16):
    """Residual rows in float32: unit scale (eps negligible), 1e-3 scale (mean
    square about eps, so eps matters), a zero row, a row with one nonzero entry
    and a row of a constant value."""
    rng = np.random.default_rng(seed)
    rows = [rng.normal(0, 1, size=d), rng.normal(0, 5, size=d), rng.normal(0, 1e-3, size=d),
            rng.normal(0, 7e-4, size=d), np.zeros(d), np.eye(1, d, 3)[0] * 2.5e-3, np.full(d, -0.75)]
    return np.stack(rows).astype(np.float32)


def test_rmsnorm_matches_exact_rational_rounding():
    """x_i = RNE_bf16(h_i / sqrt(sum_j h_j^2 / d + 1e-6)), decided exactly with
    rationals (no square root is taken: v >= c <=> h^2 >= c^2 S)."""
    h = _glue_rows()
    d = h.shape[1]
    x = M.rmsnorm_to_bf16(h.astype(np.float64))
    eps = Fraction(1e-6)  # the float64 value of 1e-6, as the oracle uses it
    n_checked = 0
    for t in range(h.shape[0]):
        S = sum(Fraction(float(v)) ** 2 for v in h[t]) / d + eps
        for i in range(d):
            want, dist = ER.rne_sqrt_ratio(Fraction(float(h[t, i])), S, ER.BF16)
            if dist < 1e-9:
                continue  # within float64 rounding of a midpoint: either neighbour is correct
            assert Fraction(float(x[t, i])) == want, (t, i, x[t, i], float(want))
            n_checked += 1
    assert n_checked >= h.size - 2
    assert np.all(x[4] == 0)


def test_residual_add_is_float32_rounded_sum():
    """h + y rounded once to float32, against exact rationals and torch."""
    import torch
    rng = np.random.default_rng(20)
    h = rng.normal(0, 3, size=(3, 64)).astype(np.float32)
    y = (rng.normal(0, 1, size=(3, 64)) * np.exp(rng.uniform(-20, 5, size=(3, 64)))).astype(np.float32)
    got = M.residual_add(h, y)
    for a, b, g in zip(h.ravel(), y.ravel(), got.ravel()):
        assert Fraction(float(g)) == ER.rne(Fraction(float(a)) + Fraction(float(b)), ER.F32)
    assert np.array_equal(got, (torch.from_numpy(h) + torch.from_numpy(y)).numpy().astype(np.float64))


# ---------------------------------------------------------------- planted mistakes

def _expect_pin_failure(monkeypatch, target, attr, bad, pin, *args):
    monkeypatch.setattr(target, attr, bad)
    with pytest.raises(AssertionError):
        pin(*args)
    monkeypatch.undo()


def test_planted_mistakes_are_caught(monkeypatch):
    # (1) IQ4_NL nibble order swapped
    def bad_unpack(codes):
        b = np.asarray(codes).astype(np.uint8)
        rs = b.shape[:-1]
        nb = b.shape[-1] // 16
        b = b.reshape(rs + (nb, 16))
        return np.concatenate([b >> 4, b & 15], axis=-1).reshape(rs + (nb * 32,))
    _expect_pin_failure(monkeypatch, F, "iq4_nl_unpack", bad_unpack, _pin_iq4_order)

    # (2) router bias dropped
    orig_logits = M.router_logits
    _expect_pin_failure(monkeypatch, M, "router_logits",
                        lambda w, b, x: orig_logits(w, None, x), test_router_logits_match_exact_rational_sum)

    # (3) top-k tie broken toward the higher index
    def bad_topk(L32, k):
        L = np.asarray(L32, np.float32)
        return np.stack([np.lexsort((-np.arange(L.shape[1]), -L[t].astype(np.float64)))[:k]
                         for t in range(L.shape[0])]).astype(np.int32)
    _expect_pin_failure(monkeypatch, M, "topk", bad_topk, test_topk_all_equal_gives_lowest_indices)

    # (4) down projection applied transposed
    def bad_ffn(Wg, Wu, Wd, x):
        X = np.asarray(x, np.float64)
        h = M.silu(X @ Wg.T) * (X @ Wu.T)
        return h, h @ Wd
    _expect_pin_failure(monkeypatch, M, "expert_ffn", bad_ffn, test_layer_matches_bruteforce_loops,
                        ("q8_0", "q8_0", "q8_0"))

    # (5) SwiGLU with silu on the wrong operand
    def bad_ffn2(Wg, Wu, Wd, x):
        X = np.asarray(x, np.float64)
        h = (X @ Wg.T) * M.silu(X @ Wu.T)
        return h, h @ Wd.T
    _expect_pin_failure(monkeypatch, M, "expert_ffn", bad_ffn2, test_one_hot_expert_closed_form)

    # (6) softmax over all experts without renormalising over the selection
    def bad_weights(L, idx):
        L = np.asarray(L, np.float64)
        full = np.exp(L - L.max(1, keepdims=True))
        full /= full.sum(1, keepdims=True)
        return np.take_along_axis(full, idx.astype(np.int64), 1)
    _expect_pin_failure(monkeypatch, M, "gate_weights", bad_weights,
                        test_gate_weights_sum_to_one_and_equal_renormalised_softmax)

    # (7) fp16 exponent bias off by one
    orig_fp16 = F.fp16_bits_to_float
    _expect_pin_failure(monkeypatch, F, "fp16_bits_to_float", lambda b: orig_fp16(b) * 2.0,
                        _pin_fp16)

    # (8) plan not stable (descending tokens inside a bucket)
    orig_plan = M.plan
    def bad_plan(idx, E):
        p = orig_plan(idx, E)
        for e in range(E):
            lo, hi = p["offsets"][e], p["offsets"][e + 1]
            p["row_token"][lo:hi] = p["row_token"][lo:hi][::-1].copy()
            p["row_slot"][lo:hi] = p["row_slot"][lo:hi][::-1].copy()
        return p
    _expect_pin_failure(monkeypatch, M, "plan", bad_plan, test_plan_matches_library_routines, 3)

    # (9) plan keeps the last of repeated ids instead of the first
    def bad_plan_dup(idx, E):
        return _plan_keep_last(orig_plan, idx, E)
    _expect_pin_failure(monkeypatch, M, "plan", bad_plan_dup, test_plan_keeps_first_of_repeated_ids)

    # (10) RMSNorm with the wrong eps, the wrong denominator, eps outside the root
    orig_round = F.round_to_bf16
    for bad in (lambda H: orig_round(H / np.sqrt(np.mean(H * H, -1, keepdims=True) + 1e-5)),
                lambda H: orig_round(H / np.sqrt(np.mean(H * H, -1, keepdims=True))),
                lambda H: orig_round(H / np.sqrt(np.sum(H * H, -1, keepdims=True) / (H.shape[-1] - 1) + 1e-6)),
                lambda H: orig_round(H / (np.sqrt(np.mean(H * H, -1, keepdims=True)) + 1e-6))):
        _expect_pin_failure(monkeypatch, M, "rmsnorm_to_bf16", lambda h, bad=bad: bad(np.asarray(h, np.float64)),
                            test_rmsnorm_matches_exact_rational_rounding)

    # (11) bf16 rounding through a float32 intermediate (two roundings)
    def bad_round(x):
        f = np.asarray(x, np.float64).astype(np.float32)
        return F.bf16_bits_to_float(F.f32_to_bf16_bits(f))
    _expect_pin_failure(monkeypatch, F, "round_to_bf16", bad_round, _pin_bf16)

    # (12) residual sum left in float64
    _expect_pin_failure(monkeypatch, M, "residual_add",
                        lambda h, y: np.asarray(h, np.float32).astype(np.float64) + np.asarray(y, np.float32),
                        test_residual_add_is_float32_rounded_sum)


def _plan_keep_last(orig_plan, idx, E):
    """The plan with, among repeated ids of a token, the LAST slot kept."""
    idx = np.asarray(idx, dtype=np.int32).copy()
    T, k = idx.shape
    for t in range(T):
        for j in range(k):
            if 0 <= idx[t, j] < E and idx[t, j] in idx[t, j + 1:]:
                idx[t, j] = -1
    p = orig_plan(idx, E)
    return p
