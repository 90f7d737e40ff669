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

from parity_common import check_bf16_glue, check_layer, check_selection, rel_l2, to_np

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
    if qtype == "q5_1":
        # every code byte; d and m of either sign over the finite binary16 range
        # (subnormals, zeros, the maximum: 31 d + m then overflows fp16); random
        # high-bit words with the all-zero and all-one words among them
        codes = g.integers(0, 256, size=(n, rows, cols // 2)).astype(np.uint8)
        codes.reshape(-1)[:256] = np.arange(256)
        nb = cols // 32
        d = g.integers(0, 0x7C00, size=(n, rows, nb)).astype(np.uint16)
        d |= (g.integers(0, 2, size=d.shape) << 15).astype(np.uint16)
        m = g.integers(0, 0x7C00, size=(n, rows, nb)).astype(np.uint16)
        m |= (g.integers(0, 2, size=m.shape) << 15).astype(np.uint16)
        d.reshape(-1)[:6] = [0x0000, 0x8000, 0x0001, 0x03FF, 0x7BFF, 0xFBFF]
        m.reshape(-1)[:6] = [0x8000, 0x0000, 0x8001, 0x0400, 0x7BFF, 0x7BFF]
        # ordinary blocks: m about -16 d, as an encoder produces
        d.reshape(-1)[6:40] = 0x1C00
        m.reshape(-1)[6:40] = 0xA800
        qh = g.integers(0, 1 << 32, size=(n, rows, nb), dtype=np.uint64).astype(np.uint32)
        qh.reshape(-1)[:2] = [0, 0xFFFFFFFF]
        rec = np.zeros((n, rows, nb, 8), dtype=np.uint8)
        rec[..., 0:2] = d.view(np.uint8).reshape(n, rows, nb, 2)
        rec[..., 2:4] = m.view(np.uint8).reshape(n, rows, nb, 2)
        rec[..., 4:8] = qh.astype("<u4").view(np.uint8).reshape(n, rows, nb, 4)
        return {"type": qtype, "n": n, "rows": rows, "cols": cols, "codes": torch.from_numpy(codes),
                "scales": torch.from_numpy(rec.reshape(n, rows, nb * 8).copy()), "tensor_scale": None}
    codes = g.integers(0, 256, size=(n, rows, cols // 2)).astype(np.uint8)
    codes.reshape(-1)[:256] = np.arange(256)
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    sc = g.choice(finite, size=(n, rows, cols // 16)).astype(np.uint8)
    sc.reshape(-1)[:len(finite)] = finite
    ts = g.uniform(1e-4, 3.0, size=n).astype(np.float32)
    return {"type": qtype, "n": n, "rows": rows, "cols": cols, "codes": torch.from_numpy(codes),
            "scales": torch.from_numpy(sc), "tensor_scale": torch.from_numpy(ts)}


@pytest.mark.parametrize("qtype", ["q8_0", "iq4_nl", "nvfp4", "q5_1"])
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
        # Q5_1: d q + m need not be an fp32 value; the fp32 output is its
        # round-to-nearest-even (numpy's float64 -> float32 conversion rounds once)
        want32 = want.astype(np.float32).astype(np.float64) if qtype == "q5_1" else want
        assert np.array_equal(got, want32), f"{qtype} expert {e}: {np.sum(got != want32)} mismatches"
        outb = torch.empty((m["rows"], m["cols"]), dtype=torch.bfloat16, device=DEV)
        lib.moe_dequantize(q, e, lib.MOE_BF16, outb)
        gotb = outb.float().cpu().numpy().astype(np.float64)
        assert np.array_equal(gotb, F.round_to_bf16(want32)), f"{qtype} bf16 expert {e}"
        # the prefill GEMM's fp16 weight tile, through its own decode routine:
        # fp16 round-to-nearest-even of the exact value (NVFP4-style: without
        # the tensor scale; Q5_1: of d q + m), infinities included
        want16 = want if ts is None else F.dequant(qtype, host["codes"][e], host["scales"][e], 1.0)
        outh = torch.empty((m["rows"], m["cols"]), dtype=torch.float16, device=DEV)
        lib.moe_dequantize(q, e, lib.MOE_F16, outh)
        goth = outh.cpu().numpy()
        assert np.array_equal(goth, want16.astype(np.float16)), \
            f"{qtype} fp16 tile expert {e}: {np.sum(goth != want16.astype(np.float16))} mismatches"
        if qtype != "nvfp4":
            assert np.isinf(goth).any() and (goth[np.isfinite(goth)] != 0).any()


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
                                       (5000, 6, 300, False), (33, 3, 7, True), (40, 6, 50, "dup"),
                                       (200, 8, 64, "dup")])
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
    if bad == "dup":
        # repeated ids within a token: the lowest slot keeps its row (bit 4)
        idx[5, k - 1] = idx[5, 0]
        idx[7, 1:] = idx[7, 0]
        idx[T - 2, 2] = idx[T - 2, 1]
        idx[T - 1, 0] = idx[T - 1, k - 1]  # (slot k-1 is out of range here: no repeat)
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
           ("q8_0", "q8_0", "q8_0"), ("iq4_nl", "iq4_nl", "q5_1"), ("nvfp4", "nvfp4", "q5_1")]


@pytest.mark.parametrize("types", FORMATS, ids=lambda t: "-".join(t))
@pytest.mark.parametrize("T,x_dtype", [(1, "bf16"), (3, "f32"), (8, "bf16"), (37, "bf16"), (64, "f32"),
                                       (48, "bf16"), (64, "bf16")])
def test_decode_path_small(types, T, x_dtype):
    """Every batch of at most 64 tokens meets the 1e-4 bar, on the decode
    kernels or (NVFP4-style weights, bf16 tokens, more than 40 tokens) on the
    prefill GEMMs' exact mode."""
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


@pytest.mark.parametrize("T,fmt", [(2, "q8_0"), (80, "q8_0"), (64, "nvfp4")])
def test_swiglu_overflow_is_flagged(T, fmt):
    """Error bit 2: the decode path (T <= 64, also the prefill GEMMs' exact
    mode there) keeps h in fp32 and scales each row into fp16 parts, so it
    flags only an h that is not finite (here: tokens of 1e25 against gate /
    up scales of 30000); the prefill path flags an h beyond the fp16 range
    (scales of 30000 suffice)."""
    _say(f"[overflow] T={T} {fmt}")
    wl, layer = _small_layer(7, d=256, f=128, E=8, k=2, types=(fmt, fmt, fmt))
    for n in ("gate", "up"):
        for grp in ("routed", "shared"):
            m = layer[grp][n]
            if fmt == "nvfp4":
                m["tensor_scale"].fill_(30000.0)
            else:
                m["scales"].fill_(30000.0)
    x = torch.randn((T, wl.d)) * (1e25 if T <= 64 else 1.0)
    st, _ = _run_single(layer, x.to(torch.bfloat16), "bf16", "f32")
    assert int(st.bufs[0].plan.error.item()) & 2
    if T <= 64:
        # the same weights on ordinary tokens: h up to about 1e13, finite, no flag
        st, _ = _run_single(layer, torch.randn((T, wl.d)).to(torch.bfloat16), "bf16", "f32")
        assert int(st.bufs[0].plan.error.item()) == 0


def _shrink_gate_up(layer, factor):
    for grp in ("routed", "shared"):
        if layer.get(grp) is None:
            continue
        for n in ("gate", "up"):
            m = layer[grp][n]
            if m["type"] == "nvfp4":
                m["tensor_scale"].mul_(factor)
            else:
                m["scales"].mul_(factor)


@pytest.mark.parametrize("types", [("iq4_nl", "iq4_nl", "iq4_nl"), ("q8_0", "q8_0", "q5_1"),
                                   ("nvfp4", "nvfp4", "nvfp4")], ids=lambda t: "-".join(t))
@pytest.mark.parametrize("T", [1, 8, 37, 64])
def test_decode_path_small_activations(types, T):
    """SwiGLU outputs about 1e-5 (gate and up scales divided by 2^7): each h
    row is scaled by a power of two before it is split into fp16 parts, so
    the decode path keeps its 1e-4 bar."""
    _say(f"[decode small h] {types} T={T}")
    wl, layer = _small_layer(900 + T, d=512, f=256, E=16, k=4, types=types)
    _shrink_gate_up(layer, 2.0 ** -7)
    x = torch.randn((T, wl.d), generator=torch.Generator().manual_seed(T)).to(torch.bfloat16)
    st, gpu = _run_single(layer, x, "bf16", "f32")
    assert int(st.bufs[0].plan.error.item()) == 0
    lnp = synth.layer_to_numpy(layer)
    xn = x.float().numpy().astype(np.float64)
    stats = check_layer(lnp, xn, gpu, "f32", TOL_DECODE)
    _, parts = M.moe_layer(lnp, xn[:1], "f64", return_parts=True)
    hmax = max(np.abs(parts["h_rows"]).max(), np.abs(parts["h_shared"]).max())
    _say(f"[decode small h] max |h| (token 0) {hmax:.2e}; {stats}")
    assert hmax < 1e-4


@pytest.mark.parametrize("T,types", [(5, ("iq4_nl", "iq4_nl", "q8_0")), (40, ("iq4_nl", "iq4_nl", "q8_0")),
                                     (100, ("iq4_nl", "iq4_nl", "q8_0")), (64, ("nvfp4", "nvfp4", "nvfp4"))],
                         ids=lambda v: "-".join(v) if isinstance(v, tuple) else str(v))
def test_ffn_forward_with_dropped_pairs(T, types):
    """A plan that dropped pairs (ids out of range, ids repeated within a
    token) through moe_ffn_forward: the dropped pairs contribute nothing, the
    others match the oracle, and nothing is written outside the buffers (the
    workspace is bracketed by guard regions that must stay untouched).  The
    NVFP4-style case at 64 tokens runs the prefill GEMMs' exact mode, whose
    h rows of dropped pairs are never written."""
    _say(f"[dropped pairs] T={T} {types}")
    wl, layer = _small_layer(600 + T, d=256, f=128, E=16, k=4, types=types)
    g = np.random.default_rng(T)
    idx = np.stack([g.permutation(16)[:4] for _ in range(T)]).astype(np.int32)
    idx[0, 1] = -1
    idx[1, 3] = 16
    idx[2, 2] = idx[2, 0]
    idx[T - 1, 1:] = idx[T - 1, 0]
    w = g.uniform(0.1, 1.0, size=(T, 4))
    w /= w.sum(1, keepdims=True)
    x = torch.randn((T, wl.d), generator=torch.Generator().manual_seed(T)).to(torch.bfloat16)
    L = lib.layer_struct(layer)
    plan = lib.Plan(T, 4, 16, DEV)
    wsb = lib.moe_workspace_size(L, T)
    guard = 1 << 16
    buf = torch.full((wsb + 2 * guard,), 0x5A, dtype=torch.uint8, device=DEV)
    ws = buf[guard:guard + wsb]
    xd = x.to(DEV)
    idx_d = torch.from_numpy(idx).to(DEV)
    w_d = torch.from_numpy(w.astype(np.float32)).to(DEV)
    y = torch.empty((T, wl.d), dtype=torch.float32, device=DEV)
    lib.moe_plan(idx_d, T, 4, 16, plan, ws, wsb)
    lib.moe_ffn_forward(L, xd, lib.MOE_BF16, T, w_d, plan, y, lib.MOE_F32, ws, wsb)
    torch.cuda.synchronize()
    assert int(plan.error.item()) == 1 | 4
    assert torch.all(buf[:guard] == 0x5A) and torch.all(buf[guard + wsb:] == 0x5A), "write outside the workspace"
    lnp = synth.layer_to_numpy(layer)
    xn = x.float().numpy().astype(np.float64)
    p_ref = M.plan(idx, 16)
    assert p_ref["error"] == 1 | 4
    got = plan.host()
    for n in ("counts", "offsets", "row_token", "row_slot", "slot_row", "active"):
        assert np.array_equal(got[n], p_ref[n]), n
    y_ref = M.layer_from_selection(lnp, xn, idx, w.astype(np.float32).astype(np.float64), p_ref, out_dtype="f64")
    err = rel_l2(y.cpu().numpy(), y_ref)
    assert err <= (TOL_DECODE if T <= 64 else TOL_PREFILL), err


@pytest.mark.parametrize("types", [("q8_0", "q8_0", "q8_0"), ("iq4_nl", "iq4_nl", "iq4_nl")],
                         ids=lambda t: "-".join(t))
def test_prefill_extreme_scales(types):
    """Prefill at the edges of the fp16 weight range.  Subnormal block scales
    (0x0001 .. 0x03FF) give exact or 2^-11-accurate fp16 weights: parity
    holds.  A block scale of 0x7BFF (65504) can overflow fp16: error bit 8."""
    T = 100
    _say(f"[prefill extreme] {types}")
    wl, layer = _small_layer(700, d=256, f=128, E=8, k=2, types=types, shared=False)
    g = torch.Generator(device=DEV).manual_seed(3)
    sc = layer["routed"]["down"]["scales"]
    bits = torch.randint(1, 0x400, sc.shape, generator=g, device=DEV, dtype=torch.int32)
    sc.copy_(bits.to(torch.int16).view(torch.float16))
    x = torch.randn((T, wl.d), generator=torch.Generator().manual_seed(9)).to(torch.bfloat16)
    st, gpu = _run_single(layer, x, "bf16", "f32")
    assert int(st.bufs[0].plan.error.item()) == 0
    lnp = synth.layer_to_numpy(layer)
    stats = check_layer(lnp, x.float().numpy().astype(np.float64), gpu, "f64", TOL_PREFILL)
    _say(f"[prefill extreme] subnormal down scales: {stats}")
    # one block scale of every routed gate matrix at the fp16 maximum
    layer["routed"]["gate"]["scales"][:, 5, 2] = 65504.0
    st, gpu = _run_single(layer, x, "bf16", "f32")
    assert int(st.bufs[0].plan.error.item()) & 8


def _set_q5_1_records(mat, d_bits, m_bits):
    """Overwrite d and m of every block record of a Q5_1 matrix (device tensors
    of int32 binary16 bit patterns, one per block)."""
    rec = mat["scales"].view(*mat["scales"].shape[:-1], -1, 8)
    rec[..., 0] = (d_bits & 0xFF).to(torch.uint8)
    rec[..., 1] = ((d_bits >> 8) & 0xFF).to(torch.uint8)
    rec[..., 2] = (m_bits & 0xFF).to(torch.uint8)
    rec[..., 3] = ((m_bits >> 8) & 0xFF).to(torch.uint8)


def test_prefill_q5_1_extreme_records():
    """Prefill with Q5_1 down projections at the edges of the fp16 weight
    range: subnormal d and m (weights exact or 2^-11-accurate in fp16) keep
    parity; a block whose 31 d + m reaches 65520 sets error bit 8, and so does
    one whose m alone does."""
    T = 100
    _say("[prefill q5_1 extreme]")
    wl, layer = _small_layer(710, d=256, f=128, E=8, k=2, types=("iq4_nl", "iq4_nl", "q5_1"), shared=False)
    dn = layer["routed"]["down"]
    nb = dn["scales"].shape[-1] // 8
    g = torch.Generator(device=DEV).manual_seed(4)
    shp = dn["scales"].shape[:-1] + (nb,)
    d_bits = torch.randint(1, 0x400, shp, generator=g, device=DEV, dtype=torch.int32)
    m_bits = torch.randint(1, 0x400, shp, generator=g, device=DEV, dtype=torch.int32) | 0x8000
    _set_q5_1_records(dn, d_bits, m_bits)
    x = torch.randn((T, wl.d), generator=torch.Generator().manual_seed(9)).to(torch.bfloat16)
    st, gpu = _run_single(layer, x, "bf16", "f32")
    assert int(st.bufs[0].plan.error.item()) == 0
    lnp = synth.layer_to_numpy(layer)
    stats = check_layer(lnp, x.float().numpy().astype(np.float64), gpu, "f64", TOL_PREFILL)
    _say(f"[prefill q5_1 extreme] subnormal records: {stats}")
    # d = 2114, m = -14: 31 d + m = 65520 exactly, the first value that rounds to infinity
    rec = dn["scales"].view(*shp, 8)
    for e in range(wl.E):
        rec[e, 7, 1, 0:4] = torch.tensor([0x21, 0x68, 0x00, 0xCB], dtype=torch.uint8)
    st, _ = _run_single(layer, x, "bf16", "f32")
    assert int(st.bufs[0].plan.error.item()) & 8
    # one below (m = -14 - 2^-7: 65519.99): in range
    _set_q5_1_records(dn, d_bits, m_bits)
    for e in range(wl.E):
        rec[e, 7, 1, 0:4] = torch.tensor([0x21, 0x68, 0x01, 0xCB], dtype=torch.uint8)
    st, _ = _run_single(layer, x, "bf16", "f32")
    assert int(st.bufs[0].plan.error.item()) == 0
    # m alone at the binary16 maximum's neighbourhood, d = 0: in range (65504)
    # then an infinite m: out of range
    for e in range(wl.E):
        rec[e, 3, 2, 0:4] = torch.tensor([0x00, 0x00, 0xFF, 0x7B], dtype=torch.uint8)
    st, _ = _run_single(layer, x, "bf16", "f32")
    assert int(st.bufs[0].plan.error.item()) == 0
    for e in range(wl.E):
        rec[e, 3, 2, 0:4] = torch.tensor([0x00, 0x00, 0x00, 0x7C], dtype=torch.uint8)
    st, _ = _run_single(layer, x, "bf16", "f32")
    assert int(st.bufs[0].plan.error.item()) & 8


def test_q5_1_gate_up_rejected():
    """Q5_1 is a down format: a layer with Q5_1 gate / up projections is
    rejected before any launch."""
    _say("[q5_1 gate rejected]")
    wl, layer = _small_layer(720, d=256, f=128, E=8, k=2, types=("q5_1", "q5_1", "q8_0"), shared=False)
    L = lib.layer_struct(layer)
    T = 4
    plan = lib.Plan(T, 2, 8, DEV)
    wsb = lib.moe_workspace_size(L, T)
    ws = torch.empty((wsb,), dtype=torch.uint8, device=DEV)
    x = torch.zeros((T, wl.d), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((T, 2), dtype=torch.int32, device=DEV)
    idx[:, 1] = 1
    w = torch.full((T, 2), 0.5, dtype=torch.float32, device=DEV)
    y = torch.empty((T, wl.d), dtype=torch.float32, device=DEV)
    lib.moe_plan(idx, T, 2, 8, plan, ws, wsb)
    with pytest.raises(lib.MoeError) as ei:
        lib.moe_ffn_forward(L, x, lib.MOE_BF16, T, w, plan, y, lib.MOE_F32, ws, wsb)
    assert ei.value.status == lib.MOE_ERR_UNSUPPORTED


# ---------------------------------------------------------------- full-size shapes

# (full-size stacks: tests/test_gpu_full.py)


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
