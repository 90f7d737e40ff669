"""GPU parity tests of the fused decode step (moe_decode_stack) against the CPU
oracle, layer by layer with teacher forcing: each layer's recorded bf16 input
is fed to the oracle, which must reproduce the recorded logits, selection,
gate weights and layer output; the recorded inputs must follow from the
residual stream by the RMSNorm glue; and the final residual must equal the
fp32 sum of the recorded layer outputs exactly."""

import numpy as np
import pytest
import torch

from oracle import moe as M
from quantized_routed_expert_amd import synth
from quantized_routed_expert_amd.stack import FusedStack

from parity_common import check_bf16_glue, check_layer, rel_l2, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL_DECODE = 1e-4


def _say(*a):
    print(*a, flush=True)


def _make(wl, n_layers):
    layers = [synth.make_layer(wl, l, DEV) for l in range(n_layers)]
    st = FusedStack(layers, wl.T, record=True, device=DEV)
    st.set_tokens(synth.make_tokens(wl, DEV))
    st.step()
    torch.cuda.synchronize()
    return layers, st


def _check_fused(wl, layers, st, tol):
    errs = st.rec_error.cpu().numpy()
    assert np.all(errs == 0), f"plan / overflow flags {errs}"
    h = st.h0.cpu().numpy().astype(np.float32)
    out = []
    for l in range(len(layers)):
        # glue: x_l = bf16(rmsnorm(h_l)), h_l the fp32 residual before layer l
        x_ref = M.rmsnorm_to_bf16(h.astype(np.float64))
        xg = to_np(st.xs[l])
        check_bf16_glue(xg, x_ref, f"layer {l} input")
        b = st.bufs[l]
        idx = b.topk_idx.cpu().numpy()
        lnp = synth.layer_to_numpy(layers[l], set(idx.ravel().tolist()))
        gpu = {"logits": b.logits.cpu().numpy(), "idx": idx, "w": b.topk_w.cpu().numpy(), "y": to_np(b.y)}
        stats = check_layer(lnp, xg, gpu, "f64", tol)
        out.append(stats)
        h = (h + b.y.cpu().numpy()).astype(np.float32)
    # the final residual is the fp32 sum of the recorded outputs, bit for bit
    assert np.array_equal(st.h.cpu().numpy(), h)
    return out


CASES = [
    # (types, T, d, f, E, k, shared)
    (("iq4_nl", "iq4_nl", "iq4_nl"), 1, 1024, 256, 64, 4, True),
    (("iq4_nl", "iq4_nl", "q8_0"), 8, 2048, 256, 64, 8, True),
    (("nvfp4", "nvfp4", "nvfp4"), 3, 1024, 384, 64, 4, True),
    (("q8_0", "q8_0", "q8_0"), 5, 4096, 256, 600, 6, False),
    (("nvfp4", "nvfp4", "nvfp4"), 1, 3072, 256, 1024, 8, False),
    (("q8_0", "q8_0", "iq4_nl"), 2, 1024, 128, 16, 3, True),
    # T * E not a multiple of 4: per-layer logit records are not 16-byte aligned
    (("q8_0", "q8_0", "q8_0"), 3, 1024, 128, 21, 3, True),
    # one token, other format pairs of the single-launch gate/up + down path
    (("q8_0", "q8_0", "q8_0"), 1, 2048, 256, 128, 6, True),
    (("iq4_nl", "iq4_nl", "q8_0"), 1, 3072, 768, 256, 8, True),
    (("nvfp4", "nvfp4", "iq4_nl"), 1, 1024, 512, 64, 2, True),
    # one token whose gate/up pass has more steps than are issued up front
    # (the separate gate/up and down launches)
    (("q8_0", "q8_0", "q8_0"), 1, 4096, 256, 600, 6, False),
    # Q5_1 down projections: several tokens, and one token (the persistent step)
    (("iq4_nl", "iq4_nl", "q5_1"), 4, 2048, 512, 128, 8, True),
    (("q8_0", "q8_0", "q5_1"), 8, 1024, 256, 64, 4, False),
    (("iq4_nl", "iq4_nl", "q5_1"), 1, 3072, 768, 512, 8, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{'-'.join(c[0])}-T{c[1]}-d{c[2]}-E{c[4]}")
def test_fused_stack_small(case):
    types, T, d, f, E, k, shared = case
    _say(f"[fused] {case}")
    wl = synth.Workload("t", d=d, f=f, E=E, k=k, T=T, n_layers=3, gate_type=types[0], up_type=types[1],
                        down_type=types[2], shared=shared, x_dtype="bf16", y_dtype="f32", zipf_s=1.1,
                        tokens="walk", seed=300 + T + E, stack=True)
    layers, st = _make(wl, 3)
    stats = _check_fused(wl, layers, st, TOL_DECODE)
    _say(f"[fused] {stats}")


@pytest.mark.parametrize("T", [1, 3])
def test_fused_heavy_ties(T):
    """A zero router: every logit equal, so each token takes experts 0..k-1."""
    wl = synth.scaled(synth.WORKLOADS["verify"], d=1024, f=256, E=512, n_layers=2, T=T)
    layers = [synth.make_layer(wl, l, DEV) for l in range(2)]
    for L in layers:
        L["router_w"].zero_()
        L["router_b"].zero_()
    st = FusedStack(layers, wl.T, record=True, device=DEV)
    st.set_tokens(synth.make_tokens(wl, DEV))
    st.step()
    torch.cuda.synchronize()
    idx = st.rec_idx.cpu().numpy()
    assert np.array_equal(idx, np.broadcast_to(np.arange(wl.k), idx.shape))
    assert np.allclose(st.rec_w.cpu().numpy(), 1.0 / wl.k, rtol=1e-6)
    _check_fused(wl, layers, st, TOL_DECODE)


@pytest.mark.parametrize("T", [1, 4])
def test_fused_repeatable_and_graph_replay(T):
    _say(f"[fused graph] T={T}")
    wl = synth.scaled(synth.WORKLOADS["verify"], d=1024, f=256, E=64, n_layers=4, T=T)
    layers, st = _make(wl, 4)
    ref = st.h.clone()
    ref_idx = st.rec_idx.clone()
    st.step()
    torch.cuda.synchronize()
    assert torch.equal(st.h, ref) and torch.equal(st.rec_idx, ref_idx)
    st.capture()
    for _ in range(3):
        st.h.zero_()
        st.rec_idx.fill_(-7)
        st.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.h, ref) and torch.equal(st.rec_idx, ref_idx)
        _ = (torch.randn(1000, device=DEV) * 2).sum().item()
    st.step()
    torch.cuda.synchronize()
    assert torch.equal(st.h, ref)


@pytest.mark.parametrize("T", [2, 8])
def test_fused_small_activations(T):
    """SwiGLU outputs about 1e-5 (gate and up scales divided by 2^7) through
    the per-layer launches of the fused step: h rows are scaled by a power of
    two before the fp16 split, so the 1e-4 bar holds."""
    wl = synth.Workload("t", d=1024, f=256, E=64, k=4, T=T, n_layers=2, gate_type="iq4_nl", up_type="iq4_nl",
                        down_type="q8_0", shared=True, x_dtype="bf16", y_dtype="f32", zipf_s=1.1,
                        tokens="walk", seed=950 + T, stack=True)
    layers = [synth.make_layer(wl, l, DEV) for l in range(2)]
    for L in layers:
        for grp in ("routed", "shared"):
            for n in ("gate", "up"):
                L[grp][n]["scales"].mul_(2.0 ** -7)
    st = FusedStack(layers, T, record=True, device=DEV)
    st.set_tokens(synth.make_tokens(wl, DEV))
    st.step()
    torch.cuda.synchronize()
    stats = _check_fused(wl, layers, st, TOL_DECODE)
    lnp = synth.layer_to_numpy(layers[0])
    _, parts = M.moe_layer(lnp, to_np(st.xs[0])[:1], "f64", return_parts=True)
    hmax = max(np.abs(parts["h_rows"]).max(), np.abs(parts["h_shared"]).max())
    _say(f"[fused small h] T={T} max |h| {hmax:.2e}; {stats}")
    assert hmax < 1e-4
