"""GPU parity tests of the persistent single-token decode step (moe_decode_stack
at T = 1 where moe_decode_stack_persistent says so): layer by layer with
teacher forcing against the oracle, against the per-layer launches on the
same inputs, with small SwiGLU activations, and under graph replay."""

import os

import numpy as np
import pytest
import torch

from oracle import moe as M
from quantized_routed_expert_amd import lib, synth
from quantized_routed_expert_amd.stack import FusedStack

from parity_common import check_layer, rel_l2, to_np
from test_gpu_fused import _check_fused

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL_DECODE = 1e-4


def _say(*a):
    print(*a, flush=True)


def _wl(types, d, f, E, k, shared, n_layers, seed):
    return synth.Workload("t", d=d, f=f, E=E, k=k, T=1, n_layers=n_layers, gate_type=types[0], up_type=types[1],
                          down_type=types[2], shared=shared, x_dtype="bf16", y_dtype="f32", zipf_s=1.1,
                          tokens="iid", seed=seed, stack=True)


def _step(layers, h0, launches=False):
    """One decode step of the stack from residual h0; launches=True forces the
    per-layer launches (the environment switch is read at every call)."""
    if launches:
        os.environ["QRE_DECODE_LAUNCHES"] = "1"
    try:
        st = FusedStack(layers, 1, record=True, device=DEV)
        st.set_tokens(h0)
        st.step()
        torch.cuda.synchronize()
    finally:
        os.environ.pop("QRE_DECODE_LAUNCHES", None)
    return st


CASES = [
    # (types, d, f, E, k, shared)
    (("iq4_nl", "iq4_nl", "iq4_nl"), 1024, 256, 64, 4, True),
    (("iq4_nl", "iq4_nl", "q8_0"), 3072, 768, 256, 8, True),
    (("nvfp4", "nvfp4", "nvfp4"), 2048, 512, 512, 6, True),
    (("q8_0", "q8_0", "nvfp4"), 1024, 384, 128, 3, False),
    (("nvfp4", "nvfp4", "iq4_nl"), 3072, 256, 1024, 8, False),
    (("q8_0", "q8_0", "q8_0"), 1024, 128, 16, 16, True),
    # Q5_1 down projections (8-byte block records, several scale chunks a thread)
    (("iq4_nl", "iq4_nl", "q5_1"), 3072, 768, 512, 8, True),
    (("nvfp4", "nvfp4", "q5_1"), 1024, 256, 64, 4, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{'-'.join(c[0])}-d{c[1]}-f{c[2]}-E{c[3]}-k{c[4]}")
def test_persistent_step_against_oracle_and_launches(case):
    types, d, f, E, k, shared = case
    _say(f"[persist] {case}")
    wl = _wl(types, d, f, E, k, shared, 4, 400 + E + k)
    layers = [synth.make_layer(wl, l, DEV) for l in range(4)]
    structs = [lib.layer_struct(L) for L in layers]
    assert lib.moe_decode_stack_persistent(lib.layer_array(structs), 4, 1)
    h0 = synth.make_tokens(wl, DEV)
    st = _step(layers, h0)
    stats = _check_fused(wl, layers, st, TOL_DECODE)
    _say(f"[persist] {stats}")
    # the per-layer launches on the same inputs: the same first-layer input and
    # selection, outputs equal to within the two paths' rounding
    st2 = _step(layers, h0, launches=True)
    assert torch.equal(st.rec_x[0], st2.rec_x[0])
    assert torch.equal(st.rec_idx[0], st2.rec_idx[0])
    assert torch.equal(st.rec_logits[0], st2.rec_logits[0])
    assert rel_l2(st.rec_y[0].cpu().numpy(), st2.rec_y[0].cpu().numpy()) < 2e-6


def test_persistent_small_activations():
    """SwiGLU outputs about 1e-5 in magnitude (gate and up block scales divided
    by 2^7): the persistent step scales each h row by a power of two before
    splitting it into fp16 parts, so it keeps the 1e-4 bar."""
    wl = _wl(("iq4_nl", "iq4_nl", "iq4_nl"), 1024, 256, 64, 4, True, 2, 77)
    layers = [synth.make_layer(wl, l, DEV) for l in range(2)]
    for L in layers:
        for grp in ("routed", "shared"):
            for n in ("gate", "up"):
                L[grp][n]["scales"].mul_(2.0 ** -7)
    h0 = synth.make_tokens(wl, DEV)
    st = _step(layers, h0)
    stats = _check_fused(wl, layers, st, TOL_DECODE)
    lnp = synth.layer_to_numpy(layers[0])
    x0 = to_np(st.xs[0])
    _, parts = M.moe_layer(lnp, x0, "f64", return_parts=True)
    hmax = max(np.abs(parts["h_rows"]).max(), np.abs(parts["h_shared"]).max())
    _say(f"[persist small h] max |h| {hmax:.2e}; {stats}")
    assert hmax < 1e-4


def test_persistent_repeatable_and_graph_replay():
    wl = _wl(("iq4_nl", "iq4_nl", "q8_0"), 1024, 256, 128, 6, True, 5, 91)
    layers = [synth.make_layer(wl, l, DEV) for l in range(5)]
    st = FusedStack(layers, 1, record=True, device=DEV)
    st.set_tokens(synth.make_tokens(wl, DEV))
    st.step()
    torch.cuda.synchronize()
    ref, ref_idx = st.h.clone(), st.rec_idx.clone()
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
        assert int(st.rec_error.abs().sum().item()) == 0
        _ = (torch.randn(1000, device=DEV) * 2).sum().item()


def test_persistent_poll_bound_ends_the_step():
    """Failure handling, forced from the host: with every wait's poll bound
    lowered to one round (QRE_PERSIST_SPIN_MAX=1) the waits between
    workgroups give up.  The launch still ends (every wait is bounded and the
    abort word ends the others), error bit 16 is reported in a layer's record,
    and the next step with the normal bound is exact again (the set-up launch
    clears the counters, the abort word and the records)."""
    wl = _wl(("iq4_nl", "iq4_nl", "iq4_nl"), 1024, 256, 64, 4, True, 4, 4242)
    layers = [synth.make_layer(wl, l, DEV) for l in range(4)]
    structs = [lib.layer_struct(L) for L in layers]
    assert lib.moe_decode_stack_persistent(lib.layer_array(structs), 4, 1)
    h0 = synth.make_tokens(wl, DEV)
    os.environ["QRE_PERSIST_SPIN_MAX"] = "1"
    try:
        st = _step(layers, h0)
    finally:
        os.environ.pop("QRE_PERSIST_SPIN_MAX", None)
    errs = st.rec_error.cpu().numpy()
    _say(f"[persist poll bound 1] error words {errs.tolist()}")
    assert (errs & 16).any(), "no wait reported giving up"
    st2 = _step(layers, h0)
    assert not (st2.rec_error.cpu().numpy() != 0).any()
    stats = _check_fused(wl, layers, st2, TOL_DECODE)
    _say(f"[persist after the forced give-up] {stats}")
