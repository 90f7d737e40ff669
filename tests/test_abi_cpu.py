"""CPU tests of the C-ABI library: it loads, exports every symbol declared in
include/moe.h, and rejects bad arguments on the host before any GPU work
(no compute call is made here)."""

import ctypes
import os
import re

import pytest

from quantized_routed_expert_amd import lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    txt = open(os.path.join(ROOT, "include", "moe.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    names = _declared_symbols()
    assert set(names) == set(lib.EXPORTED), names
    so = lib.library()
    for n in names:
        assert hasattr(so, n), n


def test_status_strings_and_version():
    assert lib.status_string(0) == "ok"
    for s in (-1, -2, -3, -4, -5):
        assert lib.status_string(s) not in ("", "unknown status")
    assert "gfx950" in lib.version()


def _fake_layer(d=256, f=128, E=16, k=2, qtype=lib.MOE_Q8_0, down=lib.MOE_Q8_0, shared=False, base=1 << 20):
    L = lib.Layer()
    L.d, L.f, L.E, L.k = d, f, E, k
    L.router_w = base
    L.router_bias = 0
    def q(t, rows, cols, n, off):
        m = lib.QMatrix()
        m.type, m.n_expert, m.rows, m.cols = t, n, rows, cols
        m.codes = base + off
        m.scales = base + off + (1 << 16)
        m.tensor_scale = base + off + (1 << 17) if t == lib.MOE_NVFP4 else 0
        return m
    L.gate, L.up, L.down = q(qtype, f, d, E, 1 << 18), q(qtype, f, d, E, 2 << 18), q(down, d, f, E, 3 << 18)
    L.has_shared = 1 if shared else 0
    if shared:
        L.shared_gate, L.shared_up, L.shared_down = (q(qtype, f, d, 1, 4 << 18), q(qtype, f, d, 1, 5 << 18),
                                                     q(down, d, f, 1, 6 << 18))
    return L


def _route(L, T=4, x=1 << 30, ws=1 << 31, ws_bytes=1 << 30):
    so = lib.library()
    return so.moe_route(ctypes.byref(L), x, lib.MOE_BF16, T, 1 << 32, 1 << 33, None, ws, ws_bytes, None)


def _ffn(L, T=4, ws=1 << 31, ws_bytes=1 << 30, x=1 << 30, y=1 << 34, plan=None, xd=lib.MOE_BF16, yd=lib.MOE_F32):
    so = lib.library()
    if plan is None:
        plan = lib.PlanBuf(*[(1 << 35) + 4096 * i for i in range(8)])
    return so.moe_ffn_forward(ctypes.byref(L), x, xd, T, 1 << 33, ctypes.byref(plan), y, yd, ws, ws_bytes, None)


def test_route_validation():
    L = _fake_layer()
    so = lib.library()
    assert so.moe_route(None, 1, 1, 1, 1, 1, None, 1, 1, None) == lib.MOE_ERR_INVALID_ARG
    bad = _fake_layer(k=17)  # k > E
    assert _route(bad) == lib.MOE_ERR_INVALID_ARG
    assert _route(_fake_layer(d=200)) == lib.MOE_ERR_UNSUPPORTED
    assert _route(_fake_layer(E=2048)) == lib.MOE_ERR_UNSUPPORTED
    assert _route(_fake_layer(k=33, E=64)) == lib.MOE_ERR_UNSUPPORTED
    assert _route(L, T=0) == lib.MOE_ERR_INVALID_ARG
    assert _route(L, x=0) == lib.MOE_ERR_INVALID_ARG
    assert _route(L, ws=0) == lib.MOE_ERR_WORKSPACE
    assert _route(L, ws_bytes=10) == lib.MOE_ERR_WORKSPACE
    assert _route(L, ws=(1 << 31) + 8) == lib.MOE_ERR_ALIGNMENT
    L2 = _fake_layer()
    L2.router_w = (1 << 20) + 4
    assert _route(L2) == lib.MOE_ERR_ALIGNMENT


def test_plan_validation():
    so = lib.library()
    pb = lib.PlanBuf(*[(1 << 35) + 4096 * i for i in range(8)])
    ok = dict(idx=1 << 30, T=4, k=2, E=16, ws=1 << 31, wsb=1 << 20)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return so.moe_plan(a["idx"], a["T"], a["k"], a["E"], ctypes.byref(a.get("pb", pb)), a["ws"], a["wsb"], None)

    assert call(idx=0) == lib.MOE_ERR_INVALID_ARG
    assert call(T=0) == lib.MOE_ERR_INVALID_ARG
    assert call(k=17) == lib.MOE_ERR_INVALID_ARG
    assert call(E=5000, k=2) == lib.MOE_ERR_UNSUPPORTED
    assert call(wsb=4) == lib.MOE_ERR_WORKSPACE
    assert call(ws=(1 << 31) + 4) == lib.MOE_ERR_ALIGNMENT
    bad = lib.PlanBuf(*[(1 << 35) + 4096 * i for i in range(8)])
    bad.error = None
    assert call(pb=bad) == lib.MOE_ERR_INVALID_ARG


def test_ffn_validation():
    L = _fake_layer()
    assert _ffn(L, ws=0) == lib.MOE_ERR_WORKSPACE
    assert _ffn(L, ws_bytes=1000) == lib.MOE_ERR_WORKSPACE
    assert _ffn(L, T=0) == lib.MOE_ERR_INVALID_ARG
    assert _ffn(L, y=0) == lib.MOE_ERR_INVALID_ARG
    assert _ffn(L, xd=7) == lib.MOE_ERR_INVALID_ARG
    assert _ffn(L, x=(1 << 30) + 2) == lib.MOE_ERR_ALIGNMENT
    # gate and up in different formats are not covered
    L2 = _fake_layer()
    L2.up.type = lib.MOE_IQ4_NL
    assert _ffn(L2) == lib.MOE_ERR_UNSUPPORTED
    # an unknown format is not covered (the fast path needs every format covered)
    L3 = _fake_layer()
    L3.down.type = 9
    assert _ffn(L3) == lib.MOE_ERR_UNSUPPORTED
    # wrong matrix shape
    L4 = _fake_layer()
    L4.down.rows = 128
    assert _ffn(L4) == lib.MOE_ERR_INVALID_ARG
    # misaligned codes
    L5 = _fake_layer()
    L5.gate.codes += 8
    assert _ffn(L5) == lib.MOE_ERR_ALIGNMENT
    # NVFP4 without a tensor scale
    L6 = _fake_layer(qtype=lib.MOE_NVFP4, down=lib.MOE_NVFP4)
    L6.up.tensor_scale = 0
    assert _ffn(L6) == lib.MOE_ERR_INVALID_ARG
    # shared expert must use the routed formats
    L7 = _fake_layer(shared=True)
    L7.shared_down.type = lib.MOE_IQ4_NL
    assert _ffn(L7) == lib.MOE_ERR_UNSUPPORTED
    L8 = _fake_layer(shared=True)
    L8.shared_up.n_expert = 2
    assert _ffn(L8) == lib.MOE_ERR_INVALID_ARG


def test_dequant_and_glue_validation():
    so = lib.library()
    q = lib.QMatrix(lib.MOE_IQ4_NL, 4, 16, 64, 1 << 20, 1 << 21, 0)
    assert so.moe_dequantize(ctypes.byref(q), 4, lib.MOE_F32, 1 << 22, None) == lib.MOE_ERR_INVALID_ARG
    assert so.moe_dequantize(ctypes.byref(q), -1, lib.MOE_F32, 1 << 22, None) == lib.MOE_ERR_INVALID_ARG
    assert so.moe_dequantize(ctypes.byref(q), 0, lib.MOE_F32, None, None) == lib.MOE_ERR_INVALID_ARG
    q2 = lib.QMatrix(lib.MOE_IQ4_NL, 4, 16, 48, 1 << 20, 1 << 21, 0)
    assert so.moe_dequantize(ctypes.byref(q2), 0, lib.MOE_F32, 1 << 22, None) == lib.MOE_ERR_UNSUPPORTED
    q3 = lib.QMatrix(lib.MOE_NVFP4, 4, 16, 64, 1 << 20, 1 << 21, 0)
    assert so.moe_dequantize(ctypes.byref(q3), 0, lib.MOE_F32, 1 << 22, None) == lib.MOE_ERR_INVALID_ARG
    q4 = lib.QMatrix(lib.MOE_Q8_0, 4, 16, 64, (1 << 20) + 4, 1 << 21, 0)
    assert so.moe_dequantize(ctypes.byref(q4), 0, lib.MOE_F32, 1 << 22, None) == lib.MOE_ERR_ALIGNMENT
    assert so.moe_residual_rmsnorm(None, None, 0, 1, 8, ctypes.c_float(1e-6), 1 << 20, None) == \
        lib.MOE_ERR_INVALID_ARG
    assert so.moe_residual_rmsnorm(1 << 20, None, 0, 0, 8, ctypes.c_float(1e-6), 1 << 21, None) == \
        lib.MOE_ERR_INVALID_ARG
    assert so.moe_residual_rmsnorm(1 << 20, None, 0, 1, 6, ctypes.c_float(1e-6), 1 << 21, None) == \
        lib.MOE_ERR_UNSUPPORTED
    assert so.moe_residual_rmsnorm((1 << 20) + 8, None, 0, 1, 8, ctypes.c_float(1e-6), 1 << 21, None) == \
        lib.MOE_ERR_ALIGNMENT


def test_workspace_size_monotone_and_covers_paths():
    L = _fake_layer(d=3072, f=768, E=512, k=8)
    assert lib.moe_workspace_size(_fake_layer(d=100), 4) == 0
    assert lib.moe_workspace_size(L, 0) == 0
    sizes = [lib.moe_workspace_size(L, t) for t in (1, 8, 64, 65, 4096)]
    assert all(s > 0 for s in sizes)
    assert sizes == sorted(sizes)
    # the prefill path needs at least the bf16 H and O rows
    R = 4096 * 8 + 4096
    assert sizes[-1] >= R * (768 + 3072) * 2


def test_decode_stack_validation():
    so = lib.library()
    L = _fake_layer(d=1024, f=256, E=64, k=4, qtype=lib.MOE_IQ4_NL, down=lib.MOE_Q8_0, shared=True)
    arr = lib.layer_array([L, L])
    wsb = lib.moe_decode_stack_workspace_size(L, 8)
    assert wsb > 0
    assert lib.moe_decode_stack_workspace_size(L, 9) == 0  # more tokens than the fused step covers
    assert lib.moe_decode_stack_workspace_size(_fake_layer(d=512), 1) == 0  # d not a multiple of 1024
    assert lib.moe_decode_stack_workspace_size(_fake_layer(d=5120), 1) == 0  # d above 4096
    sizes = [lib.moe_decode_stack_workspace_size(L, t) for t in range(1, 9)]
    assert sizes == sorted(sizes)
    wsb = sizes[3]  # T = 4

    def call(arr=arr, n=2, h=1 << 30, T=4, eps=1e-6, ws=1 << 31, wsb=wsb):
        return so.moe_decode_stack(arr, n, h, T, ctypes.c_float(eps), None, ws, wsb, None)

    assert call(arr=None) == lib.MOE_ERR_INVALID_ARG
    assert call(n=0) == lib.MOE_ERR_INVALID_ARG
    assert call(h=0) == lib.MOE_ERR_INVALID_ARG
    assert call(T=0) == lib.MOE_ERR_INVALID_ARG
    assert call(T=9) == lib.MOE_ERR_UNSUPPORTED
    assert call(eps=-1.0) == lib.MOE_ERR_INVALID_ARG
    assert call(h=(1 << 30) + 4) == lib.MOE_ERR_ALIGNMENT
    assert call(ws=0) == lib.MOE_ERR_WORKSPACE
    assert call(wsb=wsb - 1) == lib.MOE_ERR_WORKSPACE
    assert call(ws=(1 << 31) + 64) == lib.MOE_ERR_ALIGNMENT
    # layers of different shapes or formats are not covered
    L2 = _fake_layer(d=1024, f=256, E=64, k=4, qtype=lib.MOE_IQ4_NL, down=lib.MOE_IQ4_NL, shared=True)
    assert call(arr=lib.layer_array([L, L2])) == lib.MOE_ERR_UNSUPPORTED
    L3 = _fake_layer(d=1024, f=256, E=64, k=4, qtype=lib.MOE_IQ4_NL, down=lib.MOE_Q8_0, shared=False)
    assert call(arr=lib.layer_array([L, L3])) == lib.MOE_ERR_UNSUPPORTED
    # d outside the fused step's coverage
    L4 = _fake_layer(d=512, f=256, E=64, k=4)
    assert call(arr=lib.layer_array([L4]), n=1) == lib.MOE_ERR_UNSUPPORTED
    # a bad layer anywhere in the stack is caught
    L5 = _fake_layer(d=1024, f=256, E=64, k=4, qtype=lib.MOE_IQ4_NL, down=lib.MOE_Q8_0, shared=True)
    L5.router_w = 0
    assert call(arr=lib.layer_array([L, L5])) == lib.MOE_ERR_INVALID_ARG
    # misaligned record pointers
    rec = lib.StackRecord(None, None, None, (1 << 32) + 2, None, None, None)
    assert so.moe_decode_stack(arr, 2, 1 << 30, 4, ctypes.c_float(1e-6), ctypes.byref(rec), 1 << 31, wsb,
                               None) == lib.MOE_ERR_ALIGNMENT


def test_decode_stack_noalloc_validates_on_the_host():
    """The allocation-free decode step rejects bad arguments, unsupported
    shapes and shapes beyond its scratch array before touching any GPU."""
    so = lib.library()
    assert so.moe_decode_stack_scratch_bytes() == 8 << 20
    arr = lib.layer_array([_fake_layer(d=1024, f=256, E=64, k=4, qtype=lib.MOE_IQ4_NL, down=lib.MOE_IQ4_NL)])
    h = 1 << 30
    assert so.moe_decode_stack_noalloc(arr, 0, h, 1, ctypes.c_float(1e-6), None, None) == lib.MOE_ERR_INVALID_ARG
    assert so.moe_decode_stack_noalloc(arr, 1, h, 9, ctypes.c_float(1e-6), None, None) == lib.MOE_ERR_UNSUPPORTED
    big = lib.layer_array([_fake_layer(d=4096, f=16384, E=1024, k=32, qtype=lib.MOE_IQ4_NL,
                                       down=lib.MOE_IQ4_NL)])
    assert so.moe_decode_stack_workspace_size(ctypes.byref(big[0]), 8) > 8 << 20
    assert so.moe_decode_stack_noalloc(big, 1, h, 8, ctypes.c_float(1e-6), None, None) == lib.MOE_ERR_WORKSPACE


def test_q5_1_gate_up_rejected():
    """Q5_1 is covered as the down projection's format only."""
    assert _ffn(_fake_layer(qtype=lib.MOE_Q5_1, down=lib.MOE_Q8_0)) == lib.MOE_ERR_UNSUPPORTED
    L = _fake_layer(qtype=lib.MOE_Q8_0, down=lib.MOE_Q5_1)
    L.router_w = 0  # any later check still fires: the format itself passed validation
    assert _ffn(L) != lib.MOE_ERR_UNSUPPORTED


def test_persistent_coverage_query(monkeypatch):
    """moe_decode_stack_persistent answers 1 exactly for the stacks the
    persistent launch covers, and 0 for any stack moe_decode_stack rejects."""
    monkeypatch.delenv("QRE_DECODE_LAUNCHES", raising=False)

    def covered(n=2, T=1, **kw):
        args = dict(d=3072, f=768, E=512, k=8, qtype=lib.MOE_IQ4_NL, down=lib.MOE_IQ4_NL, shared=True)
        args.update(kw)
        L = _fake_layer(**args)
        return lib.moe_decode_stack_persistent(lib.layer_array([L] * n), n, T)

    assert covered()
    assert not covered(T=2)
    assert not covered(f=1024)  # down rows too long to issue up front
    assert not covered(d=4096)  # gate/up rows too long for IQ4_NL
    assert covered(d=1024, qtype=lib.MOE_Q8_0, down=lib.MOE_Q8_0)
    assert not covered(d=2048, qtype=lib.MOE_Q8_0, down=lib.MOE_Q8_0)
    assert covered(n=128)
    assert not covered(n=129)
    assert covered(down=lib.MOE_Q5_1)
    assert not covered(d=512)  # outside the fused step altogether
    # a stack moe_decode_stack would reject is never reported as persistent
    L = _fake_layer(d=3072, f=768, E=512, k=8, qtype=lib.MOE_IQ4_NL, down=lib.MOE_IQ4_NL, shared=True)
    bad = _fake_layer(d=3072, f=768, E=512, k=8, qtype=lib.MOE_IQ4_NL, down=lib.MOE_IQ4_NL, shared=True)
    bad.router_w = 0
    assert not lib.moe_decode_stack_persistent(lib.layer_array([L, bad]), 2, 1)
    mixed = _fake_layer(d=3072, f=768, E=512, k=8, qtype=lib.MOE_IQ4_NL, down=lib.MOE_Q8_0, shared=True)
    assert not lib.moe_decode_stack_persistent(lib.layer_array([L, mixed]), 2, 1)
    assert not covered(qtype=lib.MOE_Q5_1, down=lib.MOE_Q5_1)
