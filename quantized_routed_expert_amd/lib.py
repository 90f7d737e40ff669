"""Thin Python binding of the C ABI in include/moe.h (ctypes).

Argument marshalling only: every step of the layer runs in the HIP library
``libqre_moe.so`` built next to this file.  Importing this module loads the
library and raises if it is missing -- there is no fallback path.  Device
buffers are torch tensors (PyTorch provides device memory and streams only);
the stream passed to every call is torch's current HIP stream.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqre_moe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_ALIGNMENT = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_HIP = -5

MOE_F32 = 0
MOE_BF16 = 1
MOE_F16 = 2

MOE_Q8_0 = 1
MOE_IQ4_NL = 2
MOE_NVFP4 = 3
MOE_Q5_1 = 4

QTYPE = {"q8_0": MOE_Q8_0, "iq4_nl": MOE_IQ4_NL, "nvfp4": MOE_NVFP4, "q5_1": MOE_Q5_1}
DTYPE = {"f32": MOE_F32, "bf16": MOE_BF16}

EXPORTED = ["moe_route", "moe_plan", "moe_ffn_forward", "moe_ffn_prepare", "moe_ffn_gateup", "moe_ffn_down",
            "moe_ffn_combine", "moe_dequantize", "moe_residual_rmsnorm", "moe_decode_stack",
            "moe_decode_stack_workspace_size", "moe_decode_stack_noalloc", "moe_decode_stack_scratch_bytes",
            "moe_decode_stack_persistent",
            "moe_workspace_size", "moe_status_string", "moe_version"]


class MoeError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class QMatrix(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int32), ("n_expert", ctypes.c_int32), ("rows", ctypes.c_int32),
                ("cols", ctypes.c_int32), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p)]


class Layer(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("f", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("gate", QMatrix), ("up", QMatrix), ("down", QMatrix),
                ("has_shared", ctypes.c_int32),
                ("shared_gate", QMatrix), ("shared_up", QMatrix), ("shared_down", QMatrix)]


class PlanBuf(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("counts", "offsets", "row_token", "row_slot", "slot_row", "active", "n_active", "error")]


class StackRecord(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("logits", "topk_idx", "topk_w", "x", "y", "error", "events")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          f"`python -m quantized_routed_expert_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    LP, PP, QP = ctypes.POINTER(Layer), ctypes.POINTER(PlanBuf), ctypes.POINTER(QMatrix)
    sig = {
        "moe_route": (i32, [LP, vp, i32, i32, vp, vp, vp, vp, sz, vp]),
        "moe_plan": (i32, [vp, i32, i32, i32, PP, vp, sz, vp]),
        "moe_ffn_forward": (i32, [LP, vp, i32, i32, vp, PP, vp, i32, vp, sz, vp]),
        "moe_ffn_prepare": (i32, [LP, vp, i32, i32, PP, vp, sz, vp]),
        "moe_ffn_gateup": (i32, [LP, vp, i32, i32, PP, vp, sz, vp]),
        "moe_ffn_down": (i32, [LP, i32, i32, PP, vp, sz, vp]),
        "moe_ffn_combine": (i32, [LP, i32, i32, vp, PP, vp, i32, vp, sz, vp]),
        "moe_dequantize": (i32, [QP, i32, i32, vp, vp]),
        "moe_residual_rmsnorm": (i32, [vp, vp, i32, i32, i32, ctypes.c_float, vp, vp]),
        "moe_decode_stack": (i32, [LP, i32, vp, i32, ctypes.c_float, ctypes.POINTER(StackRecord), vp, sz, vp]),
        "moe_decode_stack_workspace_size": (sz, [LP, i32]),
        "moe_decode_stack_noalloc": (i32, [LP, i32, vp, i32, ctypes.c_float, ctypes.POINTER(StackRecord), vp]),
        "moe_decode_stack_scratch_bytes": (sz, []),
        "moe_decode_stack_persistent": (i32, [LP, i32, i32]),
        "moe_workspace_size": (sz, [LP, i32]),
        "moe_status_string": (ctypes.c_char_p, [i32]),
        "moe_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def library():
    return _lib


def status_string(s):
    return _lib.moe_status_string(int(s)).decode()


def version():
    return _lib.moe_version().decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(st, what):
    if st != MOE_OK:
        raise MoeError(st, what)


# ---------------------------------------------------------------- structs

def qmatrix(m):
    """QMatrix struct for an encoded matrix dict (synth.make_matrix layout)."""
    q = QMatrix()
    q.type = QTYPE[m["type"]]
    q.n_expert = m["n"]
    q.rows = m["rows"]
    q.cols = m["cols"]
    q.codes = _ptr(m["codes"])
    q.scales = _ptr(m["scales"])
    q.tensor_scale = _ptr(m.get("tensor_scale"))
    return q


def layer_struct(layer):
    """Layer struct for a device layer dict (synth.make_layer layout).  The
    caller keeps the dict (and so the tensors) alive while the struct is used."""
    L = Layer()
    L.d, L.f, L.E, L.k = layer["d"], layer["f"], layer["E"], layer["k"]
    L.router_w = _ptr(layer["router_w"])
    L.router_bias = _ptr(layer.get("router_b"))
    L.gate = qmatrix(layer["routed"]["gate"])
    L.up = qmatrix(layer["routed"]["up"])
    L.down = qmatrix(layer["routed"]["down"])
    sh = layer.get("shared")
    L.has_shared = 1 if sh is not None else 0
    if sh is not None:
        L.shared_gate = qmatrix(sh["gate"])
        L.shared_up = qmatrix(sh["up"])
        L.shared_down = qmatrix(sh["down"])
    return L


class Plan:
    """Device buffers of one expert plan for up to T tokens x k slots."""

    def __init__(self, T, k, E, device="cuda"):
        i32 = dict(dtype=torch.int32, device=device)
        self.T, self.k, self.E = T, k, E
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.row_token = torch.empty(T * k, **i32)
        self.row_slot = torch.empty(T * k, **i32)
        self.slot_row = torch.empty(T * k, **i32)
        self.active = torch.empty(E, **i32)
        self.n_active = torch.empty(1, **i32)
        self.error = torch.empty(1, **i32)
        self.struct = PlanBuf()
        for n in ("counts", "offsets", "row_token", "row_slot", "slot_row", "active", "n_active", "error"):
            setattr(self.struct, n, getattr(self, n).data_ptr())

    def host(self):
        return {n: getattr(self, n).cpu().numpy() for n in
                ("counts", "offsets", "row_token", "row_slot", "slot_row", "active", "n_active", "error")}


# ---------------------------------------------------------------- entry points

def moe_workspace_size(L, T_max):
    return int(_lib.moe_workspace_size(ctypes.byref(L), int(T_max)))


def moe_route(L, x, x_dtype, T, topk_idx, topk_w, logits, ws, ws_bytes, stream=None):
    st = _lib.moe_route(ctypes.byref(L), _ptr(x), int(x_dtype), int(T), _ptr(topk_idx), _ptr(topk_w),
                        _ptr(logits), _ptr(ws), int(ws_bytes), _stream(stream))
    _check(st, "moe_route")


def moe_plan(topk_idx, T, k, E, plan, ws, ws_bytes, stream=None):
    st = _lib.moe_plan(_ptr(topk_idx), int(T), int(k), int(E), ctypes.byref(plan.struct), _ptr(ws),
                       int(ws_bytes), _stream(stream))
    _check(st, "moe_plan")


def moe_ffn_forward(L, x, x_dtype, T, topk_w, plan, y, y_dtype, ws, ws_bytes, stream=None):
    st = _lib.moe_ffn_forward(ctypes.byref(L), _ptr(x), int(x_dtype), int(T), _ptr(topk_w),
                              ctypes.byref(plan.struct), _ptr(y), int(y_dtype), _ptr(ws), int(ws_bytes),
                              _stream(stream))
    _check(st, "moe_ffn_forward")


def moe_ffn_prepare(L, x, x_dtype, T, plan, ws, ws_bytes, stream=None):
    st = _lib.moe_ffn_prepare(ctypes.byref(L), _ptr(x), int(x_dtype), int(T), ctypes.byref(plan.struct), _ptr(ws),
                              int(ws_bytes), _stream(stream))
    _check(st, "moe_ffn_prepare")


def moe_ffn_gateup(L, x, x_dtype, T, plan, ws, ws_bytes, stream=None):
    st = _lib.moe_ffn_gateup(ctypes.byref(L), _ptr(x), int(x_dtype), int(T), ctypes.byref(plan.struct), _ptr(ws),
                             int(ws_bytes), _stream(stream))
    _check(st, "moe_ffn_gateup")


def moe_ffn_down(L, x_dtype, T, plan, ws, ws_bytes, stream=None):
    st = _lib.moe_ffn_down(ctypes.byref(L), int(x_dtype), int(T), ctypes.byref(plan.struct), _ptr(ws),
                           int(ws_bytes), _stream(stream))
    _check(st, "moe_ffn_down")


def moe_ffn_combine(L, x_dtype, T, topk_w, plan, y, y_dtype, ws, ws_bytes, stream=None):
    st = _lib.moe_ffn_combine(ctypes.byref(L), int(x_dtype), int(T), _ptr(topk_w), ctypes.byref(plan.struct),
                              _ptr(y), int(y_dtype), _ptr(ws), int(ws_bytes), _stream(stream))
    _check(st, "moe_ffn_combine")


def moe_dequantize(q, expert, out_dtype, dst, stream=None):
    st = _lib.moe_dequantize(ctypes.byref(q), int(expert), int(out_dtype), _ptr(dst), _stream(stream))
    _check(st, "moe_dequantize")


def moe_residual_rmsnorm(h, y, y_dtype, T, d, eps, x_out, stream=None):
    st = _lib.moe_residual_rmsnorm(_ptr(h), _ptr(y), int(y_dtype), int(T), int(d), float(eps), _ptr(x_out),
                                   _stream(stream))
    _check(st, "moe_residual_rmsnorm")


def moe_decode_stack_workspace_size(L, T_max):
    return int(_lib.moe_decode_stack_workspace_size(ctypes.byref(L), int(T_max)))


def layer_array(structs):
    """Contiguous host array of Layer structs (moe_decode_stack's `layers`)."""
    arr = (Layer * len(structs))()
    for i, L in enumerate(structs):
        arr[i] = L
    return arr


def stack_record(logits=None, topk_idx=None, topk_w=None, x=None, y=None, error=None, events=None):
    """events: None, or a list of 2*n_layers torch.cuda.Event (created with
    enable_timing=True and already initialised by a first record)."""
    ev = None
    if events is not None:
        ev = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    r = StackRecord(_ptr(logits), _ptr(topk_idx), _ptr(topk_w), _ptr(x), _ptr(y), _ptr(error),
                    ctypes.cast(ev, ctypes.c_void_p) if ev is not None else None)
    r._keep = ev  # the handle array must outlive the struct
    return r


def moe_decode_stack_noalloc(layers, n_layers, h, T, eps, rec, stream=None):
    """moe_decode_stack with the library's own per-GPU scratch array as workspace."""
    st = _lib.moe_decode_stack_noalloc(layers, int(n_layers), _ptr(h), int(T), float(eps),
                                       ctypes.byref(rec) if rec is not None else None, _stream(stream))
    _check(st, "moe_decode_stack_noalloc")


def moe_decode_stack_persistent(layers, n_layers, T):
    """True if moe_decode_stack runs this stack as one persistent launch."""
    return bool(_lib.moe_decode_stack_persistent(layers, int(n_layers), int(T)))


def moe_decode_stack_scratch_bytes():
    return int(_lib.moe_decode_stack_scratch_bytes())


def moe_decode_stack(layers, n_layers, h, T, eps, rec, ws, ws_bytes, stream=None):
    """layers: a ctypes array from layer_array(); rec: a StackRecord or None."""
    st = _lib.moe_decode_stack(layers, int(n_layers), _ptr(h), int(T), float(eps),
                               ctypes.byref(rec) if rec is not None else None, _ptr(ws), int(ws_bytes),
                               _stream(stream))
    _check(st, "moe_decode_stack")
