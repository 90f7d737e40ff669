"""Harness around the C ABI: one layer (route -> plan -> experts + combine) and a
stack of layers joined by the residual / RMSNorm glue, eagerly or replayed
from a HIP graph captured on torch's current stream.

FusedStack runs the same stack for up to 8 tokens through the single fused
entry point moe_decode_stack (three or four launches per layer).

Every compute step is a call into libqre_moe.so; this module only allocates
torch device buffers and sequences the calls.
"""

import torch

from . import lib

RMS_EPS = 1e-6


class LayerBuffers:
    """Per-layer device outputs kept for inspection (routing, plan, output)."""

    def __init__(self, T, d, E, k, y_dtype, device, keep_logits=True):
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=device)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.logits = torch.empty((T, E), dtype=torch.float32, device=device) if keep_logits else None
        self.plan = lib.Plan(T, k, E, device)
        self.y = torch.empty((T, d), dtype=torch.bfloat16 if y_dtype == "bf16" else torch.float32, device=device)


class Stack:
    """A stack of routed-expert layers on one GPU.

    layers: device layer dicts (synth.make_layer layout).  T: tokens per step.
    y_dtype: 'f32' or 'bf16' layer output.  For a single unchained layer pass
    chain=False: the step then runs the layer directly on the given tokens.
    """

    def __init__(self, layers, T, y_dtype="f32", x_dtype="bf16", chain=True, keep_logits=True,
                 device="cuda"):
        self.layers = layers
        self.structs = [lib.layer_struct(L) for L in layers]
        L0 = layers[0]
        self.T, self.d, self.E, self.k = T, L0["d"], L0["E"], L0["k"]
        self.y_dtype, self.x_dtype, self.chain = y_dtype, x_dtype, chain
        self.device = device
        self.ws_bytes = max(lib.moe_workspace_size(s, T) for s in self.structs)
        self.ws = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=device)
        self.ws_ptr = (self.ws.data_ptr() + 255) // 256 * 256
        self.bufs = [LayerBuffers(T, self.d, self.E, self.k, y_dtype, device, keep_logits) for _ in layers]
        self.h = torch.empty((T, self.d), dtype=torch.float32, device=device)
        xdt = torch.bfloat16 if x_dtype == "bf16" else torch.float32
        self.xs = [torch.empty((T, self.d), dtype=xdt, device=device) for _ in layers]
        self.x_final = torch.empty((T, self.d), dtype=torch.bfloat16, device=device)
        self.h0 = None
        self.graph = None

    # -- single layer ------------------------------------------------------
    def run_layer(self, i, x, x_dtype=None):
        """route -> plan -> experts + combine for layer i on tokens x."""
        L, b = self.structs[i], self.bufs[i]
        xd = lib.DTYPE[x_dtype or self.x_dtype]
        lg = b.logits
        lib.moe_route(L, x, xd, self.T, b.topk_idx, b.topk_w, lg, self.ws_ptr, self.ws_bytes)
        lib.moe_plan(b.topk_idx, self.T, self.k, self.E, b.plan, self.ws_ptr, self.ws_bytes)
        lib.moe_ffn_forward(L, x, xd, self.T, b.topk_w, b.plan, b.y, lib.DTYPE[self.y_dtype], self.ws_ptr,
                            self.ws_bytes)
        return b.y

    # -- the whole step ----------------------------------------------------
    def set_tokens(self, h0):
        """Tokens of layer 0: the fp32 residual stream (chained) or the layer
        input itself (unchained)."""
        self.h0 = h0.to(self.device).contiguous()

    def step(self):
        """One pass of the hot path over the whole stack."""
        if not self.chain:
            x = self.xs[0]
            x.copy_(self.h0.to(x.dtype))
            return self.run_layer(0, x)
        self.h.copy_(self.h0)
        ydt = lib.DTYPE[self.y_dtype]
        for i in range(len(self.layers)):
            prev = None if i == 0 else self.bufs[i - 1].y
            lib.moe_residual_rmsnorm(self.h, prev, ydt, self.T, self.d, RMS_EPS, self.xs[i])
            self.run_layer(i, self.xs[i], "bf16")
        # fold the last layer's output into the residual stream
        lib.moe_residual_rmsnorm(self.h, self.bufs[-1].y, ydt, self.T, self.d, RMS_EPS, self.x_final)
        return self.h

    def capture(self, warmup=1):
        """Capture one step into a HIP graph on a side stream (torch's graph API)."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(warmup):
                self.step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step()
        torch.cuda.synchronize()
        self.graph = g
        return g

    def replay(self):
        self.graph.replay()


class _LayerView:
    """Per-layer views into FusedStack's records (same names as LayerBuffers)."""

    def __init__(self, st, l):
        self.logits = st.rec_logits[l] if st.rec_logits is not None else None
        self.topk_idx = st.rec_idx[l]
        self.topk_w = st.rec_w[l]
        self.y = st.rec_y[l]
        self.error = st.rec_error[l:l + 1]


class FusedStack:
    """The stack of layers through moe_decode_stack (T <= 8, bf16 layer inputs,
    fp32 layer outputs).  With record=True every layer's logits, selection,
    input and output are kept (views in .bufs[l] and .xs[l])."""

    def __init__(self, layers, T, record=True, device="cuda"):
        self.layers = layers
        self.structs = [lib.layer_struct(L) for L in layers]
        self.arr = lib.layer_array(self.structs)
        L0 = layers[0]
        self.n, self.T, self.d, self.E, self.k = len(layers), T, L0["d"], L0["E"], L0["k"]
        self.device = device
        self.ws_bytes = lib.moe_decode_stack_workspace_size(self.structs[0], T)
        if self.ws_bytes == 0:
            raise ValueError("layer shape or T not covered by moe_decode_stack")
        self.ws = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=device)
        self.ws_ptr = (self.ws.data_ptr() + 255) // 256 * 256
        self.h = torch.empty((T, self.d), dtype=torch.float32, device=device)
        n, k, d, E = self.n, self.k, self.d, self.E
        self.rec_error = torch.zeros(n, dtype=torch.int32, device=device)
        self.rec_idx = torch.empty((n, T, k), dtype=torch.int32, device=device)
        self.rec_w = torch.empty((n, T, k), dtype=torch.float32, device=device)
        if record:
            self.rec_logits = torch.empty((n, T, E), dtype=torch.float32, device=device)
            self.rec_x = torch.empty((n, T, d), dtype=torch.bfloat16, device=device)
            self.rec_y = torch.empty((n, T, d), dtype=torch.float32, device=device)
        else:
            self.rec_logits = self.rec_x = self.rec_y = None
        self.record = lib.stack_record(self.rec_logits, self.rec_idx, self.rec_w, self.rec_x, self.rec_y,
                                       self.rec_error)
        self.bufs = [_LayerView(self, l) for l in range(n)] if record else None
        self.xs = [self.rec_x[l] for l in range(n)] if record else None
        self.h0 = None
        self.graph = None

    def set_tokens(self, h0):
        self.h0 = h0.to(self.device).contiguous()

    def step(self, record=None):
        """One pass over the whole stack: h = h0, then every layer in order.
        record: a StackRecord to use instead of the stack's own (lib.stack_record()
        for none at all)."""
        self.h.copy_(self.h0)
        lib.moe_decode_stack(self.arr, self.n, self.h, self.T, RMS_EPS, self.record if record is None else record,
                             self.ws_ptr, self.ws_bytes)
        return self.h

    def timed_record(self, events):
        """A record that also times each layer's gate/up launch (eager calls only)."""
        r = self.record
        return lib.stack_record(r.logits, r.topk_idx, r.topk_w, r.x, r.y, r.error, events)

    def capture(self, warmup=1, record=None):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(warmup):
                self.step(record)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step(record)
        torch.cuda.synchronize()
        self.graph = g
        return g

    def replay(self):
        self.graph.replay()
