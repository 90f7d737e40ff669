"""Sanity checks of the seeded input generator's encoders (not parity: any
deterministic encoder is valid, since both sides read the same bytes)."""

import numpy as np
import torch

from oracle import formats as F
from quantized_routed_expert_amd import synth


def test_q8_0_round_trip_within_half_step():
    w = torch.randn(3, 8, 128, generator=torch.Generator().manual_seed(0)) * 0.02
    codes, d16 = synth.encode_q8_0(w)
    back = F.dequant_q8_0(codes.numpy(), d16.view(torch.int16).numpy().view(np.uint16))
    d = np.repeat(d16.float().numpy().astype(np.float64), 32, axis=-1)
    amax = np.repeat(w.abs().reshape(3, 8, 4, 32).amax(-1).numpy().astype(np.float64), 32, axis=-1)
    bound = d / 2 + np.maximum(0, amax - 127 * d) + 1e-12
    assert np.all(np.abs(back - w.numpy().astype(np.float64)) <= bound)


def test_iq4_nl_picks_nearest_codebook_entry():
    w = torch.randn(2, 4, 64, generator=torch.Generator().manual_seed(1)) * 0.02
    codes, d16 = synth.encode_iq4_nl(w)
    idx = F.iq4_nl_unpack(codes.numpy())
    d = np.repeat(d16.float().numpy().astype(np.float64), 32, axis=-1)
    r = w.numpy().astype(np.float64) / d
    dist = np.abs(r[..., None] - F.IQ4_NL_CODEBOOK)
    best = dist.min(-1)
    chosen = np.take_along_axis(dist, idx[..., None].astype(np.int64), -1)[..., 0]
    assert np.allclose(chosen, best, rtol=1e-6, atol=1e-9)
    # the largest-magnitude element maps to codebook[0]
    blocks = w.reshape(2, 4, 2, 32).abs().argmax(-1).numpy()
    for a in range(2):
        for b in range(4):
            for c in range(2):
                assert idx[a, b, 32 * c + blocks[a, b, c]] == 0


def test_q5_1_round_trip_within_half_step():
    """The Q5_1 encoder's codes decode (through the oracle) to within half a
    step d of the drawn weights, plus the rounding of the block minimum to m;
    every code 0..31 is used and each block reaches both ends."""
    w = torch.randn(2, 8, 128, generator=torch.Generator().manual_seed(2)) * 0.02
    codes, rec = synth.encode_q5_1(w)
    assert codes.shape == (2, 8, 64) and rec.shape == (2, 8, 32)
    q, d, m = F.q5_1_unpack(codes.numpy(), rec.numpy())
    wn = w.numpy().astype(np.float64).reshape(2, 8, 4, 32)
    dq = F.dequant_q5_1(codes.numpy(), rec.numpy()).reshape(2, 8, 4, 32)
    # slack: half a step, the rounding of the minimum to m, and at the top of
    # the block the rounding of the step to binary16 (31 steps of it)
    mn, mx = wn.min(-1), wn.max(-1)
    slack = 0.5 * d + np.abs(m - mn) + 31.0 * np.abs(d - (mx - mn) / 31.0) + 1e-12
    assert np.all(np.abs(dq - wn).max(-1) <= slack)
    qb = q.reshape(2, 8, 4, 32)
    assert set(np.unique(q)) == set(range(32))
    assert np.all(qb.min(-1) == 0) and np.all(qb.max(-1) == 31)


def test_nvfp4_codes_nearest_and_saturating():
    w = torch.randn(2, 4, 64, generator=torch.Generator().manual_seed(2)) * 0.02
    codes, sc, ts = synth.encode_nvfp4(w)
    assert sc.dtype == torch.uint8 and ts.shape == (2,)
    for e in range(2):
        back = F.dequant_nvfp4(codes[e].numpy(), sc[e].numpy(), ts[e].item())
        blk_scale = np.repeat(F.e4m3_bits_to_float(sc[e].numpy()), 16, axis=-1) * ts[e].item()
        err = np.abs(back - w[e].numpy())
        # grid spacing is at most 2 * blk_scale (between 4 and 6); saturation at 6
        assert np.all(err <= blk_scale * 1.0 + 1e-9)


def test_zipf_bias_and_token_recipes():
    wl = synth.scaled(synth.WORKLOADS["decode"], d=128, f=128, E=32, n_layers=1)
    layer = synth.make_layer(wl, 0)
    b = layer["router_b"].numpy()
    ranks = np.round(np.exp(-b / 1.1)).astype(int)
    assert sorted(ranks.tolist()) == list(range(1, 33))
    walk = synth.make_tokens(synth.scaled(synth.WORKLOADS["verify"], d=64))
    steps = (walk[1:] - walk[:-1]).numpy()
    assert abs(steps.std() - 0.1) < 0.03
    slots = synth.make_tokens(synth.scaled(synth.WORKLOADS["slots"], d=64))
    assert slots.shape == (64, 64)
    # 8 independent sequences: a jump between sequences is O(1), inside them O(0.1)
    jumps = np.abs(slots[8::8].numpy() - slots[7:-1:8].numpy()).mean()
    assert jumps > 0.5
