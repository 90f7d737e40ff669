"""Seeded synthetic workloads for the routed-expert layer (input preparation only).

This module draws the random inputs and packs them into the block formats; it
holds none of the layer's arithmetic (no decoding, routing or matrix products).
Both the GPU library and the CPU oracle consume the packed bytes it produces.

Recipe (all seeded):

* Every expert / shared-expert weight is drawn fp32 N(0, 0.02^2) and encoded
  into its block format; router weights are fp32 N(0, 0.02^2).
* The router bias is log-Zipf: b_e = -s * ln(rank_e) with s = 1.1 and rank a
  seeded permutation of 1..E per layer, so that hot experts recur.
* Token activations are N(0, 1): i.i.d. (decode, prefill), or random walks
  x_i = x_{i-1} + N(0, 0.1^2) for speculative-verify drafts (one walk of 8, or 8
  independent walks of 8 for parallel slots).

Encoders (any deterministic choice is valid; both sides read the same bytes):

* Q8_0: d = fp16(absmax / 127); q = clamp(round_half_away(x / d), -127, 127).
* IQ4_NL: x* = the block's largest-magnitude element (first on ties),
  d = fp16(-x* / 127), code = nearest codebook entry to x / d (lower index on
  ties); d == 0 gives code 8.
* NVFP4-style: ts = amax_matrix / (6 * 448); s_b = e4m3_rne(amax_block / (6 ts));
  code = e2m1_rne(x / (s_b ts)), saturating at 6.

On the GPU the draws use torch's device generator, on the CPU torch's CPU
generator: the same seed gives different (equally valid) numbers per device.
"""

from dataclasses import dataclass, field
import math

import numpy as np
import torch

# Encoder tables (the encode direction only).
_IQ4_NL_VALUES = [-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113]

QTYPE_ID = {"q8_0": 1, "iq4_nl": 2, "nvfp4": 3, "q5_1": 4}


@dataclass(frozen=True)
class Workload:
    name: str
    d: int
    f: int
    E: int
    k: int
    T: int
    n_layers: int
    gate_type: str
    up_type: str
    down_type: str
    shared: bool
    x_dtype: str          # 'f32' or 'bf16' layer input
    y_dtype: str          # 'f32' or 'bf16' layer output
    zipf_s: float         # 0 = no router bias
    tokens: str           # 'iid', 'walk', 'slots'
    seed: int
    stack: bool = True    # chained layers with the residual / RMSNorm glue
    note: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload("tiny", d=256, f=128, E=16, k=2, T=4, n_layers=1,
                     gate_type="q8_0", up_type="q8_0", down_type="q8_0", shared=False,
                     x_dtype="f32", y_dtype="f32", zipf_s=0.0, tokens="iid", seed=0,
                     stack=False, note="single layer, fp32 tokens"),
    "decode": Workload("decode", d=3072, f=768, E=512, k=8, T=1, n_layers=48,
                       gate_type="iq4_nl", up_type="iq4_nl", down_type="iq4_nl", shared=True,
                       x_dtype="bf16", y_dtype="f32", zipf_s=1.1, tokens="iid", seed=1,
                       note="batch-1 decode"),
    "verify": Workload("verify", d=3072, f=768, E=512, k=8, T=8, n_layers=48,
                       gate_type="iq4_nl", up_type="iq4_nl", down_type="q8_0", shared=True,
                       x_dtype="bf16", y_dtype="f32", zipf_s=1.1, tokens="walk", seed=2,
                       note="speculative verify: 7 drafts + 1"),
    "slots": Workload("slots", d=3072, f=768, E=512, k=8, T=64, n_layers=48,
                      gate_type="nvfp4", up_type="nvfp4", down_type="nvfp4", shared=True,
                      x_dtype="bf16", y_dtype="f32", zipf_s=1.1, tokens="slots", seed=3,
                      note="8 sequences x 8 verify tokens"),
    "prefill": Workload("prefill", d=3072, f=768, E=512, k=8, T=4096, n_layers=48,
                        gate_type="iq4_nl", up_type="iq4_nl", down_type="iq4_nl", shared=True,
                        x_dtype="bf16", y_dtype="bf16", zipf_s=1.1, tokens="iid", seed=4,
                        note="4096-token prefill chunk"),
    # the prefill chunk with NVIDIA's NVFP4 routed-expert format (the pages'
    # seven-engine benchmark runs NVFP4 routed experts bit-exact)
    "prefill_nvfp4": Workload("prefill_nvfp4", d=3072, f=768, E=512, k=8, T=4096, n_layers=48,
                              gate_type="nvfp4", up_type="nvfp4", down_type="nvfp4", shared=True,
                              x_dtype="bf16", y_dtype="bf16", zipf_s=1.1, tokens="iid", seed=5,
                              note="4096-token prefill chunk, NVFP4-style experts"),
}


def scaled(wl, **kw):
    """A copy of workload ``wl`` with some fields replaced (smaller test shapes)."""
    d = dict(wl.__dict__)
    d.update(kw)
    return Workload(**d)


# ----------------------------------------------------------------------------
# seeding
# ----------------------------------------------------------------------------

TENSOR_IDS = {"router_w": 1, "router_perm": 2, "gate": 3, "up": 4, "down": 5,
              "shared_gate": 6, "shared_up": 7, "shared_down": 8, "tokens": 9}


def _seed(cfg_seed, layer, tensor):
    ss = np.random.SeedSequence([int(cfg_seed), int(layer), int(TENSOR_IDS[tensor])])
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64((1 << 63) - 1))


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


# ----------------------------------------------------------------------------
# encoders (torch; run on the device the draws are on)
# ----------------------------------------------------------------------------

def encode_q8_0(w):
    """fp32 [..., rows, cols] -> (int8 codes [..., rows, cols], fp16 scales [..., rows, cols/32])."""
    shp = w.shape
    b = w.reshape(*shp[:-1], shp[-1] // 32, 32)
    amax = b.abs().amax(dim=-1)
    d16 = (amax / 127.0).to(torch.float16)
    dq = d16.float().unsqueeze(-1)
    r = torch.where(dq > 0, b / torch.where(dq > 0, dq, torch.ones_like(dq)), torch.zeros_like(b))
    q = torch.sign(r) * torch.floor(r.abs() + 0.5)
    q = q.clamp(-127, 127).to(torch.int8)
    return q.reshape(shp), d16


def encode_iq4_nl(w):
    """fp32 [..., rows, cols] -> (uint8 codes [..., rows, cols/2], fp16 scales [..., rows, cols/32])."""
    shp = w.shape
    b = w.reshape(*shp[:-1], shp[-1] // 32, 32)
    am = b.abs().argmax(dim=-1, keepdim=True)  # first maximal element
    xstar = torch.gather(b, -1, am)
    d16 = (xstar / -127.0).to(torch.float16)
    dq = d16.float()
    nz = dq != 0
    r = b / torch.where(nz, dq, torch.ones_like(dq))
    vals = torch.tensor(_IQ4_NL_VALUES, dtype=torch.float32, device=w.device)
    mids = (vals[1:] + vals[:-1]) * 0.5
    idx = torch.bucketize(r, mids, right=False)  # ties go to the lower entry
    idx = torch.where(nz.expand_as(idx), idx, torch.full_like(idx, 8)).to(torch.uint8)
    lo = idx[..., :16]
    hi = idx[..., 16:]
    codes = (lo | (hi << 4)).reshape(*shp[:-1], shp[-1] // 2)
    return codes, d16.squeeze(-1)


def encode_q5_1(w):
    """fp32 [..., rows, cols] -> (uint8 codes [..., rows, cols/2], uint8 block records
    [..., rows, cols/32 * 8]).

    Per 32-element block: d = fp16((max - min) / 31), m = fp16(min), q = the
    nearest of 0..31 to (x - m) / d (halves up).  Codes hold the low four bits
    in the IQ4_NL byte order (element j low nibble, j + 16 high nibble of byte
    j); a record is d, m (binary16, little-endian) and a little-endian uint32
    whose bit e is the fifth bit of element e."""
    shp = w.shape
    b = w.reshape(*shp[:-1], shp[-1] // 32, 32)
    mn = b.amin(dim=-1)
    mx = b.amax(dim=-1)
    d16 = ((mx - mn) / 31.0).to(torch.float16)
    m16 = mn.to(torch.float16)
    dq = d16.float().unsqueeze(-1)
    nz = dq > 0
    r = (b - m16.float().unsqueeze(-1)) / torch.where(nz, dq, torch.ones_like(dq))
    q = torch.where(nz, torch.floor(r + 0.5), torch.zeros_like(r)).clamp(0, 31).to(torch.int64)
    low = q & 15
    codes = (low[..., :16] | (low[..., 16:] << 4)).to(torch.uint8).reshape(*shp[:-1], shp[-1] // 2)
    bit = torch.arange(32, device=w.device, dtype=torch.int64)
    word = ((q >> 4) << bit).sum(dim=-1)
    dbits = d16.view(torch.int16).to(torch.int64) & 0xFFFF
    mbits = m16.view(torch.int16).to(torch.int64) & 0xFFFF
    rec = torch.stack([dbits & 0xFF, dbits >> 8, mbits & 0xFF, mbits >> 8,
                       word & 0xFF, (word >> 8) & 0xFF, (word >> 16) & 0xFF, (word >> 24) & 0xFF], dim=-1)
    records = rec.to(torch.uint8).reshape(*shp[:-1], (shp[-1] // 32) * 8)
    return codes.contiguous(), records.contiguous()


def _e2m1_rne(r):
    """float -> E2M1 nibble, round to nearest, ties to even mantissa, saturating at 6."""
    a = r.abs()
    mag = ((a > 0.25).to(torch.uint8) + (a >= 0.75).to(torch.uint8) + (a > 1.25).to(torch.uint8)
           + (a >= 1.75).to(torch.uint8) + (a > 2.5).to(torch.uint8) + (a >= 3.5).to(torch.uint8)
           + (a > 5.0).to(torch.uint8))
    sign = ((r < 0) & (mag > 0)).to(torch.uint8) << 3
    return mag | sign


def encode_nvfp4(w):
    """fp32 [n, rows, cols] -> (uint8 codes [n, rows, cols/2], uint8 E4M3 scales [n, rows, cols/16],
    fp32 tensor scale [n])."""
    n, rows, cols = w.shape
    amax_t = w.abs().reshape(n, -1).amax(dim=-1)
    ts = amax_t / (6.0 * 448.0)
    ts = torch.where(ts > 0, ts, torch.ones_like(ts))
    b = w.reshape(n, rows, cols // 16, 16)
    amax_b = b.abs().amax(dim=-1)
    sb = (amax_b / (6.0 * ts[:, None, None])).clamp(max=448.0)
    sb8 = sb.to(torch.float8_e4m3fn)
    sbq = sb8.float()
    denom = (sbq * ts[:, None, None]).unsqueeze(-1)
    r = torch.where(denom > 0, b / torch.where(denom > 0, denom, torch.ones_like(denom)), torch.zeros_like(b))
    nib = _e2m1_rne(r).reshape(n, rows, cols)
    codes = nib[..., 0::2] | (nib[..., 1::2] << 4)
    return codes.contiguous(), sb8.view(torch.uint8).contiguous(), ts.float().contiguous()


# ----------------------------------------------------------------------------
# weights and tokens
# ----------------------------------------------------------------------------

def make_matrix(qtype, n, rows, cols, seed, device="cpu", chunk_elems=1 << 27):
    """Draw n expert matrices [rows, cols] ~ N(0, 0.02^2) and encode them.

    Returns a dict: type, codes, scales, tensor_scale (NVFP4) and n/rows/cols.
    Draws proceed in chunks of whole experts from one seeded generator."""
    g = _gen(device, seed)
    per = max(1, chunk_elems // (rows * cols))
    codes_l, scales_l, ts_l = [], [], []
    for e0 in range(0, n, per):
        m = min(per, n - e0)
        w = torch.randn((m, rows, cols), generator=g, device=device, dtype=torch.float32) * 0.02
        if qtype == "q8_0":
            c, s = encode_q8_0(w)
        elif qtype == "iq4_nl":
            c, s = encode_iq4_nl(w)
        elif qtype == "nvfp4":
            c, s, t = encode_nvfp4(w)
            ts_l.append(t)
        elif qtype == "q5_1":
            c, s = encode_q5_1(w)
        else:
            raise ValueError(qtype)
        codes_l.append(c)
        scales_l.append(s)
        del w
    out = {"type": qtype, "n": n, "rows": rows, "cols": cols,
           "codes": torch.cat(codes_l).contiguous() if len(codes_l) > 1 else codes_l[0].contiguous(),
           "scales": torch.cat(scales_l).contiguous() if len(scales_l) > 1 else scales_l[0].contiguous(),
           "tensor_scale": (torch.cat(ts_l) if ts_l else None)}
    return out


def make_layer(wl, layer, device="cpu"):
    """All tensors of layer ``layer`` of workload ``wl`` (torch, on ``device``)."""
    s = wl.seed
    g = _gen(device, _seed(s, layer, "router_w"))
    router_w = torch.randn((wl.E, wl.d), generator=g, device=device, dtype=torch.float32) * 0.02
    if wl.zipf_s > 0:
        gp = torch.Generator(device="cpu")
        gp.manual_seed(_seed(s, layer, "router_perm"))
        rank = torch.randperm(wl.E, generator=gp).to(torch.float64) + 1.0
        router_b = (-wl.zipf_s * torch.log(rank)).to(torch.float32).to(device)
    else:
        router_b = None
    routed = {
        "gate": make_matrix(wl.gate_type, wl.E, wl.f, wl.d, _seed(s, layer, "gate"), device),
        "up": make_matrix(wl.up_type, wl.E, wl.f, wl.d, _seed(s, layer, "up"), device),
        "down": make_matrix(wl.down_type, wl.E, wl.d, wl.f, _seed(s, layer, "down"), device),
    }
    shared = None
    if wl.shared:
        shared = {
            "gate": make_matrix(wl.gate_type, 1, wl.f, wl.d, _seed(s, layer, "shared_gate"), device),
            "up": make_matrix(wl.up_type, 1, wl.f, wl.d, _seed(s, layer, "shared_up"), device),
            "down": make_matrix(wl.down_type, 1, wl.d, wl.f, _seed(s, layer, "shared_down"), device),
        }
    return {"d": wl.d, "f": wl.f, "E": wl.E, "k": wl.k, "router_w": router_w,
            "router_b": router_b, "routed": routed, "shared": shared}


def make_tokens(wl, device="cpu"):
    """Token activations [T, d] fp32 for layer 0 (the residual stream for stacked
    workloads, the layer input itself for the single-layer workload)."""
    g = _gen(device, _seed(wl.seed, 0, "tokens"))
    T, d = wl.T, wl.d
    if wl.tokens == "iid":
        return torch.randn((T, d), generator=g, device=device, dtype=torch.float32)
    if wl.tokens in ("walk", "slots"):
        n_seq = 1 if wl.tokens == "walk" else max(1, T // 8)
        per = T // n_seq
        x0 = torch.randn((n_seq, 1, d), generator=g, device=device, dtype=torch.float32)
        eps = torch.randn((n_seq, per - 1, d), generator=g, device=device, dtype=torch.float32) * 0.1
        walk = torch.cat([x0, x0 + torch.cumsum(eps, dim=1)], dim=1)
        return walk.reshape(n_seq * per, d).contiguous()
    raise ValueError(wl.tokens)


# ----------------------------------------------------------------------------
# host views for the oracle
# ----------------------------------------------------------------------------

def matrix_to_numpy(m, experts=None):
    """Copy (a subset of) an encoded matrix to host numpy arrays in the oracle's
    raw-bit conventions (fp16 scales as uint16 bits, E4M3 scales as uint8 bits)."""
    sel = slice(None) if experts is None else torch.as_tensor(list(experts), dtype=torch.long,
                                                                device=m["codes"].device)
    codes = m["codes"][sel].cpu()
    scales = m["scales"][sel].cpu()
    if m["type"] in ("q8_0", "iq4_nl"):
        scales_np = scales.view(torch.int16).numpy().view(np.uint16)
    else:
        scales_np = scales.numpy().astype(np.uint8)
    if m["type"] == "q8_0":
        codes_np = codes.numpy().astype(np.int8)
    else:
        codes_np = codes.numpy().astype(np.uint8)
    ts = None
    if m.get("tensor_scale") is not None:
        ts = m["tensor_scale"][sel].cpu().numpy().astype(np.float32)
    return {"type": m["type"], "codes": codes_np, "scales": scales_np, "tensor_scale": ts}


class _ExpertSubset(dict):
    """Dict-like view mapping global expert ids onto a copied subset."""


def layer_to_numpy(layer, experts=None):
    """Host copy of a layer for the oracle.  With ``experts`` given, only those
    routed experts are copied, and the returned mats are indexed by a remap so
    that mats['codes'][e] works for every e in ``experts``."""
    out = {"d": layer["d"], "f": layer["f"], "E": layer["E"], "k": layer["k"],
           "router_w": layer["router_w"].cpu().numpy().astype(np.float32),
           "router_b": None if layer["router_b"] is None else layer["router_b"].cpu().numpy().astype(np.float32)}
    routed = {}
    for name in ("gate", "up", "down"):
        m = layer["routed"][name]
        if experts is None:
            routed[name] = matrix_to_numpy(m)
        else:
            ex = sorted(set(int(e) for e in experts))
            sub = matrix_to_numpy(m, ex)
            routed[name] = _remap(sub, ex, m["n"])
    out["routed"] = routed
    if layer["shared"] is not None:
        out["shared"] = {name: matrix_to_numpy(layer["shared"][name]) for name in ("gate", "up", "down")}
    else:
        out["shared"] = None
    return out


class _Remapped:
    def __init__(self, arr, ex, n):
        self.arr = arr
        self.pos = {e: i for i, e in enumerate(ex)}
        self.n = n

    def __getitem__(self, e):
        return self.arr[self.pos[int(e)]]


def _remap(sub, ex, n):
    out = {"type": sub["type"]}
    out["codes"] = _Remapped(sub["codes"], ex, n)
    out["scales"] = _Remapped(sub["scales"], ex, n)
    out["tensor_scale"] = None if sub["tensor_scale"] is None else _Remapped(sub["tensor_scale"], ex, n)
    return out
