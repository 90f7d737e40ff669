"""GPU parity tests: the HIP library, called through the C ABI, against the
CPU oracle on the same seeded inputs.

Bars: bit-exact dequantised weights, top-k indices (near-tie rule in
parity_common) and expert plan; rel-L2 <= 1e-4 for the fp32-accumulated decode
path and <= 1e-2 for the fp16-MFMA prefill path (weights and SwiGLU
activations rounded to fp16)."""

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import moe as M
from quantized_routed_expert_amd import lib, synth
from quantized_routed_expert_amd.stack import Stack

from parity_common import check_layer, check_selection, rel_l2, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL_DECODE = 1e-4
TOL_PREFILL = 1e-2


def _say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------- dequantisation

def _edge_matrix(qtype, n=2, rows=32, cols=256, seed=0):
    g = np.random.default_rng(seed)
    if qtype == "q8_0":
        codes = g.integers(-128, 128, size=(n, rows, cols)).astype(np.int8)
        codes.reshape(-1)[:256] = np.arange(-128, 128)
        sc = g.integers(0, 0x7C00, size=(n, rows, cols // 32)).astype(np.uint16)
        sc |= (g.integers(0, 2, size=sc.shape) << 15).astype(np.uint16)
        sc.reshape(-1)[:6] = [0x0000, 0x8000, 0x0001, 0x03FF, 0x7BFF, 0xFBFF]
        return {"type": qtype, "n": n, "rows": rows, "cols": cols, "codes": torch.from_numpy(codes),
                "scales": torch.from_numpy(sc.view(np.int16)).view(torch.float16), "tensor_scale": None}
    if qtype == "iq4_nl":
        codes = g.integers(0, 256, size=(n, rows, cols // 2)).astype(np.uint8)
        codes.reshape(-1)[:256] = np.arange(256)
        sc = g.integers(0, 0x7C00, size=(n, rows, cols // 32)).astype(np.uint16)
        sc |= (g.integers(0, 2, size=sc.shape) << 15).astype(np.uint16)
        sc.reshape(-1)[:6] = [0x0000, 0x8000, 0x0001, 0x03FF, 0x7BFF, 0xFBFF]
        return {"type": qtype, "n": n, "rows": rows, "cols": cols, "codes": torch.from_numpy(codes),
                "scales": torch.from_numpy(sc.view(np.int16)).view(torch.float16), "tensor_scale": None}
    codes = g.integers(0, 256, size=(n, rows, cols // 2)).astype(np.uint8)
    codes.reshape(-1)[:256] = np.arange(256)
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    sc = g.choice(finite, size=(n, rows, cols // 16)).astype(np.uint8)
    sc.reshape(-1)[:len(finite)] = finite
    ts = g.uniform(1e-4, 3.0, size=n).astype(np.float32)
    return {"type": qtype, "n": n, "rows": rows, "cols": cols, "codes": torch.from_numpy(codes),
            "scales": torch.from_numpy(sc), "tensor_scale": torch.from_numpy(ts)}


@pytest.mark.parametrize("qtype", ["q8_0", "iq4_nl", "nvfp4"])
def test_dequantize_bit_exact(qtype):
    _say(f"[dequant] {qtype}")
    m = _edge_matrix(qtype)
    host = synth.matrix_to_numpy(m)
    dm = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in m.items()}
    q = lib.qmatrix(dm)
    for e in range(m["n"]):
        ts = None if host["tensor_scale"] is None else host["tensor_scale"][e]
        want = F.dequant(qtype, host["codes"][e], host["scales"][e], ts)
        out = torch.empty((m["rows"], m["cols"]), dtype=torch.float32, device=DEV)
        lib.moe_dequantize(q, e, lib.MOE_F32, out)
        got = out.cpu().numpy().astype(np.float64)
        assert np.array_equal(got, want), f"{qtype} expert {e}: {np.sum(got != want)} mismatches"
        outb = torch.empty((m["rows"], m["cols"]), dtype=torch.bfloat16, device=DEV)
        lib.moe_dequantize(q, e, lib.MOE_BF16, outb)
        gotb = outb.float().cpu().numpy().astype(np.float64)
        assert np.array_equal(gotb, F.round_to_bf16(want)), f"{qtype} bf16 expert {e}"


# ---------------------------------------------------------------- routing

def _small_layer(seed, d=256, f=128, E=16, k=4, types=("iq4_nl", "iq4_nl", "iq4_nl"), shared=True, zipf=1.1):
    wl = synth.Workload("t", d=d, f=f, E=E, k=k, T=1, n_layers=1, gate_type=types[0], up_type=types[1],
                        down_type=types[2], shared=shared, x_dtype="bf16", y_dtype="f32", zipf_s=zipf,
                        tokens="iid", seed=seed, stack=False)
    return wl, synth.make_layer(wl, 0, DEV)


@pytest.mark.parametrize("T,d", [(1, 256), (7, 256), (64, 256), (200, 256), (37, 1024), (64, 3072)])
def test_router_topk_exact(T, d):
    _say(f"[route] T={T} d={d}")
    wl, layer = _small_layer(10 + T, d=d, E=64, k=6)
    # duplicate router rows -> exact ties, lower id must win
    layer["router_w"][9] = layer["router_w"][3]
    layer["router_b"][9] = layer["router_b"][3]
    x = torch.randn((T, wl.d), generator=torch.Generator(device=DEV).manual_seed(T), device=DEV).to(torch.bfloat16)
    L = lib.layer_struct(layer)
    idx = torch.empty((T, wl.k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, wl.k), dtype=torch.float32, device=DEV)
    logits = torch.empty((T, wl.E), dtype=torch.float32, device=DEV)
    wsb = lib.moe_workspace_size(L, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    lib.moe_route(L, x, lib.MOE_BF16, T, idx, w, logits, ws, wsb)
    torch.cuda.synchronize()
    L64 = M.router_logits(layer["router_w"].cpu().numpy(), layer["router_b"].cpu().numpy(), to_np(x))
    L32 = logits.cpu().numpy()
    err = np.abs(L32.astype(np.float64) - L64)
    # fp64 sums (T <= 8, or rows that the small-batch MFMA router does not
    # take): the rounded result equals the oracle's rounding
    if T <= 8 or (T <= 64 and d % 512 != 0):
        assert np.mean(L32 == L64.astype(np.float32)) > 0.999
    assert np.all(err <= 1e-5 * (1 + np.abs(L64)))
    gi = idx.cpu().numpy()
    check_selection(L64, L32, gi, wl.k)
    assert not np.any((gi == 9).any(1) & ~(gi == 3).any(1)), "tie broken toward the higher id"
    wg = w.cpu().numpy()
    assert np.allclose(wg.sum(1), 1.0, atol=1e-6)
    assert np.allclose(wg, M.gate_weights(L32.astype(np.float64), gi), rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("E,k", [(16, 2), (64, 8), (512, 8), (1000, 32)])
@pytest.mark.parametrize("T,d", [(3, 256), (40, 512)])
def test_topk_heavy_ties(E, k, T, d):
    """All-equal logits (a zero router) and a few equal maxima: lower ids first
    (T = 40, d = 512: the K-split router and its slice-summing top-k)."""
    _say(f"[ties] E={E} k={k} T={T} d={d}")
    wl, layer = _small_layer(40 + E, d=d, E=E, k=k)
    layer["router_w"].zero_()
    layer["router_b"].zero_()
    layer["router_b"][E // 2] = 1.0   # token-independent: one clear winner ...
    layer["router_b"][E - 1] = 0.5    # ... then two equal runners-up
    layer["router_b"][1] = 0.5
    x = torch.randn((T, wl.d), device=DEV).to(torch.bfloat16)
    L = lib.layer_struct(layer)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    wsb = lib.moe_workspace_size(L, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    lib.moe_route(L, x, lib.MOE_BF16, T, idx, w, logits, ws, wsb)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    want = M.topk(logits.cpu().numpy(), k)
    assert np.array_equal(gi, want)
    assert list(gi[0, :min(3, k)]) == [E // 2, 1, E - 1][:k]
    assert np.allclose(w.cpu().numpy(), M.gate_weights(logits.cpu().numpy().astype(np.float64), gi), rtol=1e-5)


# ---------------------------------------------------------------- plan

@pytest.mark.parametrize("T,k,E,bad", [(1, 8, 512, False), (8, 8, 512, False), (64, 8, 512, False),
                                       (65, 4, 16, False), (300, 8, 512, False), (4096, 8, 512, False),
                                       (5000, 6, 300, False), (33, 3, 7, True)])
def test_plan_bit_exact(T, k, E, bad):
    _say(f"[plan] T={T} k={k} E={E} bad={bad}")
    g = np.random.default_rng(T * 31 + k)
    # Zipf-like skew so buckets are uneven
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    idx = np.stack([g.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    if bad:
        idx[3, 1] = -1
        idx[10, 0] = E
        idx[T - 1, k - 1] = E + 100
    plan = lib.Plan(T, k, E, DEV)
    wsb = 1 << 24
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    lib.moe_plan(torch.from_numpy(idx).to(DEV), T, k, E, plan, ws, wsb)
    torch.cuda.synchronize()
    got = plan.host()
    want = M.plan(idx, E)
    for name in ("counts", "offsets", "row_token", "row_slot", "slot_row", "active"):
        assert np.array_equal(got[name], want[name]), name
    assert got["n_active"][0] == want["n_active"]
    assert got["error"][0] == want["error"]


# ---------------------------------------------------------------- one layer

def _run_single(layer, x, x_dtype, y_dtype):
    st = Stack([layer], x.shape[0], y_dtype=y_dtype, x_dtype=x_dtype, chain=False)
    st.set_tokens(x)
    y = st.step()
    torch.cuda.synchronize()
    b = st.bufs[0]
    return st, {"logits": b.logits.cpu().numpy(), "idx": b.topk_idx.cpu().numpy(), "w": b.topk_w.cpu().numpy(),
                "y": to_np(y)}


def test_tiny_workload_full():
    """The tiny single-layer workload end to end (Q8_0, fp32 tokens, no shared)."""
    wl = synth.WORKLOADS["tiny"]
    _say("[tiny] generating")
    layer_cpu = synth.make_layer(wl, 0, "cpu")
    x = synth.make_tokens(wl, "cpu")
    layer = {k: v for k, v in layer_cpu.items()}
    layer["router_w"] = layer_cpu["router_w"].to(DEV)
    layer["routed"] = {n: {kk: (vv.to(DEV) if isinstance(vv, torch.Tensor) else vv) for kk, vv in m.items()}
                       for n, m in layer_cpu["routed"].items()}
    st, gpu = _run_single(layer, x, "f32", "f32")
    lnp = synth.layer_to_numpy(layer_cpu)
    stats = check_layer(lnp, x.numpy().astype(np.float64), gpu, "f32", TOL_DECODE)
    _say(f"[tiny] {stats}")
    # the full oracle pass agrees too (no selection flips at this size)
    y_ref = M.moe_layer(lnp, x.numpy().astype(np.float64), out_dtype="f32")
    assert rel_l2(gpu["y"], y_ref) <= TOL_DECODE


FORMATS = [("iq4_nl", "iq4_nl", "iq4_nl"), ("iq4_nl", "iq4_nl", "q8_0"), ("nvfp4", "nvfp4", "nvfp4"),
           ("q8_0", "q8_0", "q8_0")]


@pytest.mark.parametrize("types", FORMATS, ids=lambda t: "-".join(t))
@pytest.mark.parametrize("T,x_dtype", [(1, "bf16"), (3, "f32"), (8, "bf16"), (37, "bf16"), (64, "f32")])
def test_decode_path_small(types, T, x_dtype):
    _say(f"[decode] {types} T={T} x={x_dtype}")
    wl, layer = _small_layer(100 + T, d=512, f=256, E=16, k=4, types=types)
    x = torch.randn((T, wl.d), generator=torch.Generator().manual_seed(T))
    if x_dtype == "bf16":
        x = x.to(torch.bfloat16)
    st, gpu = _run_single(layer, x, x_dtype, "f32")
    lnp = synth.layer_to_numpy(layer)
    xn = x.float().numpy().astype(np.float64)
    stats = check_layer(lnp, xn, gpu, "f32", TOL_DECODE)
    err = int(st.bufs[0].plan.error.item())
    assert err == 0
    _say(f"[decode] {stats}")


def test_decode_path_many_experts():
    """The largest per-layer decode batch over the widest router: T = 64,
    k = 32, E = 1000 (up to 1000 active experts in the slot table, counts
    from 1 to 64 in the counting sort)."""
    T = 64
    _say(f"[decode many] T={T} k=32 E=1000")
    wl, layer = _small_layer(77, d=512, f=128, E=1000, k=32, types=("iq4_nl", "iq4_nl", "q8_0"))
    x = torch.randn((T, wl.d), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    st, gpu = _run_single(layer, x, "bf16", "f32")
    lnp = synth.layer_to_numpy(layer)
    stats = check_layer(lnp, x.float().numpy().astype(np.float64), gpu, "f32", TOL_DECODE)
    assert int(st.bufs[0].plan.error.item()) == 0
    _say(f"[decode many] {stats}")


@pytest.mark.parametrize("T,x_dtype", [(40, "bf16"), (23, "f32")])
def test_decode_path_long_rows(T, x_dtype):
    """Rows longer than the codes kept in registers (Q8_0, d = 4096: 16 steps
    per wave, rolled forward) with several column passes per item, and a
    router row length the small-batch MFMA router takes (bf16 tokens)."""
    _say(f"[decode long] T={T} x={x_dtype}")
    wl, layer = _small_layer(300 + T, d=4096, f=256, E=32, k=6, types=("q8_0", "q8_0", "q8_0"))
    x = torch.randn((T, wl.d), generator=torch.Generator().manual_seed(T))
    if x_dtype == "bf16":
        x = x.to(torch.bfloat16)
    st, gpu = _run_single(layer, x, x_dtype, "f32")
    lnp = synth.layer_to_numpy(layer)
    xn = x.float().numpy().astype(np.float64)
    stats = check_layer(lnp, xn, gpu, "f32", TOL_DECODE)
    assert int(st.bufs[0].plan.error.item()) == 0
    _say(f"[decode long] {stats}")


@pytest.mark.parametrize("types", FORMATS, ids=lambda t: "-".join(t))
@pytest.mark.parametrize("T,y_dtype", [(65, "bf16"), (300, "f32")])
def test_prefill_path_small(types, T, y_dtype):
    _say(f"[prefill] {types} T={T} y={y_dtype}")
    wl, layer = _small_layer(200 + T, d=512, f=256, E=16, k=4, types=types)
    x = torch.randn((T, wl.d), generator=torch.Generator().manual_seed(T)).to(torch.bfloat16)
    st, gpu = _run_single(layer, x, "bf16", y_dtype)
    lnp = synth.layer_to_numpy(layer)
    stats = check_layer(lnp, x.float().numpy().astype(np.float64), gpu, "f64", TOL_PREFILL)
    _say(f"[prefill] {stats}")


@pytest.mark.parametrize("types", [("q8_0", "q8_0", "iq4_nl"), ("iq4_nl", "iq4_nl", "nvfp4")], ids=lambda t: "-".join(t))
def test_prefill_narrow_shapes_fp32_tokens(types):
    """d not a multiple of 256 (half-width down tiles), f = 128 (one gate/up
    tile), fp32 tokens rounded to fp16 when staged, many ragged M-tiles."""
    T = 200
    _say(f"[prefill narrow] {types} T={T}")
    wl, layer = _small_layer(500, d=384, f=128, E=24, k=3, types=types)
    x = torch.randn((T, wl.d), generator=torch.Generator().manual_seed(7))
    st, gpu = _run_single(layer, x, "f32", "f32")
    lnp = synth.layer_to_numpy(layer)
    # the router sees the fp32 tokens; the fp16 expert products see them rounded to
    # fp16, an error of the same order as the fp16 weights', inside the prefill bar
    stats = check_layer(lnp, x.numpy().astype(np.float64), gpu, "f64", TOL_PREFILL)
    _say(f"[prefill narrow] {stats}")


def test_swiglu_overflow_is_flagged():
    _say("[overflow]")
    wl, layer = _small_layer(7, d=256, f=128, E=8, k=2, types=("q8_0", "q8_0", "q8_0"))
    for n in ("gate", "up"):
        layer["routed"][n]["scales"].fill_(30000.0)
        layer["shared"][n]["scales"].fill_(30000.0)
    x = torch.randn((2, wl.d)).to(torch.bfloat16)
    st, _ = _run_single(layer, x, "bf16", "f32")
    assert int(st.bufs[0].plan.error.item()) & 2


# ---------------------------------------------------------------- full-size shapes

def _full_stack(name, n_layers, T=None):
    wl = synth.WORKLOADS[name]
    wl = synth.scaled(wl, n_layers=n_layers, T=T or wl.T)
    _say(f"[{name}] generating {n_layers} layers at d={wl.d} f={wl.f} E={wl.E}")
    layers = [synth.make_layer(wl, l, DEV) for l in range(n_layers)]
    h0 = synth.make_tokens(wl, DEV)
    st = Stack(layers, wl.T, y_dtype=wl.y_dtype, x_dtype="bf16", chain=True)
    st.set_tokens(h0)
    st.step()
    torch.cuda.synchronize()
    return wl, layers, st


def _check_stack_layer(wl, layers, st, l, tol, tokens=None):
    b = st.bufs[l]
    idx = b.topk_idx.cpu().numpy()
    sel = np.arange(wl.T) if tokens is None else np.asarray(tokens)
    experts = set(idx[sel].ravel().tolist())
    lnp = synth.layer_to_numpy(layers[l], experts)
    x_np = to_np(st.xs[l])[sel]
    gpu = {"logits": b.logits.cpu().numpy()[sel], "idx": idx[sel], "w": b.topk_w.cpu().numpy()[sel],
           "y": to_np(b.y)[sel]}
    stats = check_layer(lnp, x_np, gpu, "f64", tol)
    stats["U"] = int(b.plan.n_active.item())
    return stats


@pytest.mark.parametrize("name", ["decode", "verify", "slots"])
def test_full_size_decode_workloads(name):
    wl, layers, st = _full_stack(name, 2)
    for l in range(2):
        stats = _check_stack_layer(wl, layers, st, l, TOL_DECODE)
        _say(f"[{name}] layer {l}: {stats}")
        assert int(st.bufs[l].plan.error.item()) == 0
    # glue: x_1 = bf16(rmsnorm(h_0 + y_0)) on the GPU's own h_0 (layer-0 residual)
    h0 = st.h0.cpu().numpy().astype(np.float64)
    y0 = to_np(st.bufs[0].y)
    x1 = M.rmsnorm_to_bf16(M.residual_add(h0, y0))
    x1g = to_np(st.xs[1])
    assert np.mean(x1g == x1) > 0.999 and rel_l2(x1g, x1) < 4e-3


def test_full_size_prefill_sampled_tokens():
    wl, layers, st = _full_stack("prefill", 1)
    g = np.random.default_rng(5)
    tokens = np.sort(g.choice(wl.T, size=12, replace=False))
    tokens[0] = 0
    tokens[-1] = wl.T - 1
    stats = _check_stack_layer(wl, layers, st, 0, TOL_PREFILL, tokens)
    _say(f"[prefill] layer 0 sampled: {stats}")
    # plan of the full batch, bit exact against the oracle from the GPU's indices
    want = M.plan(st.bufs[0].topk_idx.cpu().numpy(), wl.E)
    got = st.bufs[0].plan.host()
    for n in ("counts", "offsets", "row_token", "row_slot", "slot_row", "active"):
        assert np.array_equal(got[n], want[n]), n


# ---------------------------------------------------------------- determinism / graphs

def test_bitwise_repeatable_and_graph_replay():
    _say("[graph]")
    wl = synth.scaled(synth.WORKLOADS["verify"], d=512, f=256, E=32, n_layers=3)
    layers = [synth.make_layer(wl, l, DEV) for l in range(3)]
    st = Stack(layers, wl.T, y_dtype="f32", chain=True)
    st.set_tokens(synth.make_tokens(wl, DEV))
    st.step()
    torch.cuda.synchronize()
    ref = st.h.clone()
    st.step()
    torch.cuda.synchronize()
    assert torch.equal(st.h, ref)
    st.capture()
    for _ in range(3):
        st.h.zero_()
        st.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.h, ref)
        # eager work between replays
        _ = (torch.randn(1000, device=DEV) * 2).sum().item()
    st.step()
    torch.cuda.synchronize()
    assert torch.equal(st.h, ref)
