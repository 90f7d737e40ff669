"""GPU test of moe_decode_stack_noalloc, the allocation-free decode step: two
calls in a row through the C ABI (the second with fewer tokens), each checked
bit for bit against moe_decode_stack with a caller workspace on the same
inputs (the same kernels run on both)."""

import numpy as np
import pytest
import torch

from quantized_routed_expert_amd import lib, synth
from quantized_routed_expert_amd.stack import FusedStack

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _run(st, T, h0, noalloc):
    """One decode step from residual h0 through moe_decode_stack or its
    allocation-free variant; returns the final residual and the records."""
    h = h0.clone()
    n, k, d, E = st.n, st.k, st.d, st.E
    rec_idx = torch.full((n, T, k), -1, dtype=torch.int32, device=DEV)
    rec_w = torch.zeros((n, T, k), dtype=torch.float32, device=DEV)
    rec_y = torch.zeros((n, T, d), dtype=torch.float32, device=DEV)
    rec_err = torch.full((n,), -1, dtype=torch.int32, device=DEV)
    rec = lib.stack_record(None, rec_idx, rec_w, None, rec_y, rec_err)
    if noalloc:
        lib.moe_decode_stack_noalloc(st.arr, n, h, T, 1e-6, rec)
    else:
        wsb = lib.moe_decode_stack_workspace_size(st.structs[0], T)
        ws = torch.empty(wsb + 256, dtype=torch.uint8, device=DEV)
        ptr = (ws.data_ptr() + 255) // 256 * 256
        lib.moe_decode_stack(st.arr, n, h, T, 1e-6, rec, ptr, wsb)
    torch.cuda.synchronize()
    return h, rec_idx, rec_w, rec_y, rec_err


@pytest.mark.parametrize("T0,T1", [(4, 1), (8, 3)])
def test_noalloc_matches_workspace_entry_point(T0, T1):
    print(f"[noalloc] T {T0} then {T1}", flush=True)
    wl = synth.Workload("t", d=2048, f=256, E=128, k=6, T=T0, n_layers=3, gate_type="iq4_nl",
                        up_type="iq4_nl", down_type="q8_0", shared=True, x_dtype="bf16", y_dtype="f32",
                        zipf_s=1.1, tokens="walk", seed=900 + T0, stack=True)
    layers = [synth.make_layer(wl, l, DEV) for l in range(3)]
    st = FusedStack(layers, T0, record=False, device=DEV)
    h_all = synth.make_tokens(wl, DEV)
    assert lib.moe_decode_stack_workspace_size(st.structs[0], T0) <= lib.moe_decode_stack_scratch_bytes()
    for T in (T0, T1):  # the second call has fewer tokens and follows the first on the same scratch
        h0 = h_all[:T].contiguous()
        got = _run(st, T, h0, noalloc=True)
        want = _run(st, T, h0, noalloc=False)
        assert int((got[4] != 0).sum()) == 0, f"error flags {got[4].tolist()}"
        for g, w, name in zip(got, want, ("h", "topk_idx", "topk_w", "y", "error")):
            assert torch.equal(g, w), f"T={T}: {name} differs"
        assert not torch.equal(got[0], h0)
