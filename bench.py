"""Benchmark: tokens/s through a stack of routed-expert MoE layers on one MI355X.

One step = one pass of the whole hot path over the stack for one batch of
synthetic tokens: per layer the residual/RMSNorm glue, router + top-k, the
expert plan and the grouped experts with combine, replayed from a HIP graph.
Up to 8 tokens the step is the fused entry point moe_decode_stack (one
persistent launch for a single token); above that it is the per-layer entry
points.  Inputs are resident in HBM before the timed region starts.

Prints one JSON line with the metric of the headline workload (batch-1
decode by default), the roofline of its dominant kernel (timed live with HIP
events on the stream it runs on) and the CPU oracle's rate on a bounded
sample as a reported baseline; under "workloads" the same figures for the
speculative-verify batch, the parallel slots, the 4096-token prefill chunk and
the same chunk with NVFP4-style experts (each stack generated, measured and
freed in turn), and a streaming-read reference measured in the same run.

    python bench.py [--steps K] [--warmup W] [--workload decode|verify|slots|prefill|prefill_nvfp4]
                    [--only]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at batch 1/8/64/4096; % of HBM BW (decode), % MFMA peak"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 / fp16 MFMA, TFLOP/s
ALL_WORKLOADS = ["decode", "verify", "slots", "prefill", "prefill_nvfp4"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=ALL_WORKLOADS,
                    help="the headline workload of the JSON line")
    ap.add_argument("--only", action="store_true", help="measure the headline workload only")
    ap.add_argument("--layers", type=int, default=None, help="override the layer count (default: the workload's)")
    ap.add_argument("--kernel-passes", type=int, default=3, help="instrumented passes for the kernel timing")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of each oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB, 5 times (HBM counter calibration)")
    return ap.parse_args()


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


_CS = "quantized_routed_expert_amd/csrc/"
DOMINANT = {
    # dominant kernel -> (name, pattern of its symbol in rocprofv3 output, sources it is built from)
    "decode_persistent": ("k_ps_decode (the whole 48-layer single-token step, one launch)", r"qre::k_ps_decode<",
                          [_CS + "moe_persist.hip", _CS + "moe_dq.h", _CS + "moe_device.h"]),
    "fused_gateup": ("k_fz_gateup (top-k + plan + gate/up + SwiGLU)", r"qre::k_fz_gateup<",
                     [_CS + "moe_fused.hip", _CS + "moe_dq.h", _CS + "moe_device.h"]),
    "slots": ("k_pf_gemm gate/up (NVFP4, exact mode)", r"qre::k_pf_gemm<3, true, \d, true>",
              [_CS + "moe_prefill.hip", _CS + "moe_device.h"]),
    "prefill": ("k_pf_gemm gate/up (IQ4_NL)", r"qre::k_pf_gemm<2, true, 4, false>",
                [_CS + "moe_prefill.hip", _CS + "moe_device.h"]),
    "prefill_nvfp4": ("k_pf_gemm gate/up (NVFP4)", r"qre::k_pf_gemm<3, true, 4, false>",
                      [_CS + "moe_prefill.hip", _CS + "moe_device.h"]),
}


def matrix_bytes(qtype, rows, cols):
    """Algorithmic bytes of one expert matrix: codes + block scales (+ the fp32
    tensor scale of the NVFP4-style format).  IQ4_NL: 18 B per 32 weights; Q5_1:
    24 B per 32 (16 of codes, an 8-byte record)."""
    n = rows * cols
    return {"q8_0": n // 32 * 34, "iq4_nl": n // 32 * 18, "nvfp4": n // 16 * 9 + 4, "q5_1": n // 32 * 24}[qtype]


def traffic_from_profile(key, digest):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{key}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_digest") != digest:
        return None
    return t.get("bytes_per_launch")


def stream_read_gbs(torch, gib=4):
    """Same-run reference: GB/s of a plain device reduction over `gib` GiB
    (torch's sum over int64 words, a read-bound kernel)."""
    n = (gib << 30) // 8
    buf = torch.ones(n, dtype=torch.int64, device="cuda")
    for _ in range(2):
        buf.sum()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        buf.sum()
    e1.record()
    torch.cuda.synchronize()
    gbs = reps * n * 8 / (e0.elapsed_time(e1) / 1e3) / 1e9
    del buf
    torch.cuda.empty_cache()
    return round(gbs, 1)


def measure(name, args, with_cpu):
    """Generate the stack of workload `name`, time the step, the dominant kernel
    and (optionally) the CPU oracle; returns the figures as a dict."""
    import numpy as np
    import torch

    from quantized_routed_expert_amd import lib, synth
    from quantized_routed_expert_amd.stack import FusedStack, Stack

    wl = synth.WORKLOADS[name]
    if args.layers:
        wl = synth.scaled(wl, n_layers=args.layers)
    dev = "cuda"

    # ---------------------------------------------------------------- inputs
    t0 = time.time()
    layers = []
    for l in range(wl.n_layers):
        layers.append(synth.make_layer(wl, l, dev))
        if l % 16 == 15 or l == wl.n_layers - 1:
            torch.cuda.synchronize()
            log(f"[bench {name}] generated {l + 1}/{wl.n_layers} layers ({time.time() - t0:.1f}s)")
    h0 = synth.make_tokens(wl, dev)
    # T <= 8 with fp32 layer outputs: the fused decode step (moe_decode_stack);
    # otherwise the per-layer entry points (route -> plan -> ffn_forward + glue).
    fused = wl.T <= 8 and wl.y_dtype == "f32"
    if fused:
        st = FusedStack(layers, wl.T, record=True, device=dev)
    else:
        st = Stack(layers, wl.T, y_dtype=wl.y_dtype, x_dtype="bf16", chain=True, keep_logits=False)
    st.set_tokens(h0)
    st.step()
    torch.cuda.synchronize()
    if fused:
        errs = st.rec_error.cpu().tolist()
        idx_all = st.rec_idx.cpu().numpy()
        U = [len(np.unique(idx_all[l])) for l in range(wl.n_layers)]
    else:
        errs = [int(b.plan.error.item()) for b in st.bufs]
        U = [int(b.plan.n_active.item()) for b in st.bufs]
    assert not any(errs), f"plan/experts error flags {errs}"
    persistent = fused and lib.moe_decode_stack_persistent(st.arr, wl.n_layers, wl.T)
    path = "moe_decode_stack, one persistent launch" if persistent else (
        "moe_decode_stack, per-layer launches" if fused else "per-layer entry points")
    log(f"[bench {name}] eager step ok ({path}); U per layer mean {np.mean(U):.1f} (min {min(U)}, max {max(U)})")

    # ---------------------------------------------------------------- timed region
    # The timed graph writes no records (the fused step's only outputs are h).
    if fused:
        st.capture(record=lib.stack_record())
    else:
        st.capture()
    for _ in range(args.warmup):
        st.replay()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(args.steps):
        st.replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    total_ms = evs[0].elapsed_time(evs[-1])
    ms_per_step = total_ms / args.steps
    value = wl.T / (ms_per_step / 1e3)
    log(f"[bench {name}] {args.steps} steps: {ms_per_step:.4f} ms/step (median {np.median(per):.4f}, "
        f"min {per.min():.4f}, p90 {np.percentile(per, 90):.4f}) -> {value:.1f} tokens/s")

    # ---------------------------------------------------------------- per-layer work
    d, f, E, k, T = wl.d, wl.f, wl.E, wl.k, wl.T
    gate_b = matrix_bytes(wl.gate_type, f, d)
    up_b = matrix_bytes(wl.up_type, f, d)
    down_b = matrix_bytes(wl.down_type, d, f)
    router_b = E * d * 4 + E * 4
    act_b = T * d * 2 + T * d * (2 if wl.y_dtype == "bf16" else 4)
    stack_bytes = sum(router_b + (u + 1) * (gate_b + up_b + down_b) + act_b for u in U)
    stack_flops = wl.n_layers * 2 * T * (k + 1) * 3 * d * f
    stack_hbm_frac = stack_bytes / (ms_per_step / 1e3) / (HBM_PEAK_GBS * 1e9)
    stack_mfma_frac = stack_flops / (ms_per_step / 1e3) / (MFMA_BF16_PEAK_TFS * 1e12)

    # ---------------------------------------------------------------- dominant kernel, live
    # Instrumented eager passes: HIP events attached to the dominant launch on
    # the stream it runs on (the persistent step's single launch, or every
    # layer's grouped gate/up launch).
    stream = torch.cuda.current_stream()
    durations, launch_bytes, launch_flops = [], [], []
    xd = lib.MOE_BF16
    for _ in range(args.kernel_passes if fused else 0):
        evs_k = [torch.cuda.Event(enable_timing=True) for _ in range(2 * wl.n_layers)]
        for e in evs_k:
            e.record(stream)  # creates the underlying HIP events
        st.step(st.timed_record(evs_k))
        if persistent:
            # one launch runs the whole step: its events bracket it, and its
            # algorithmic bytes are the step's
            durations.append((evs_k[0], evs_k[1]))
            launch_bytes.append(stack_bytes)
            launch_flops.append(stack_flops)
            continue
        for i in range(wl.n_layers):
            durations.append((evs_k[2 * i], evs_k[2 * i + 1]))
            u = U[i]
            launch_bytes.append((u + 1) * (gate_b + up_b) + T * E * 4 + T * d * 2 + T * (k + 1) * f * 4)
            launch_flops.append(2 * T * (k + 1) * 2 * d * f)
    for _ in range(0 if fused else args.kernel_passes):
        st.h.copy_(st.h0)
        for i in range(wl.n_layers):
            prev = None if i == 0 else st.bufs[i - 1].y
            lib.moe_residual_rmsnorm(st.h, prev, lib.DTYPE[wl.y_dtype], T, d, 1e-6, st.xs[i])
            L, b = st.structs[i], st.bufs[i]
            lib.moe_route(L, st.xs[i], xd, T, b.topk_idx, b.topk_w, b.logits, st.ws_ptr, st.ws_bytes)
            lib.moe_plan(b.topk_idx, T, k, E, b.plan, st.ws_ptr, st.ws_bytes)
            lib.moe_ffn_prepare(L, st.xs[i], xd, T, b.plan, st.ws_ptr, st.ws_bytes)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            lib.moe_ffn_gateup(L, st.xs[i], xd, T, b.plan, st.ws_ptr, st.ws_bytes)
            e1.record(stream)
            lib.moe_ffn_down(L, xd, T, b.plan, st.ws_ptr, st.ws_bytes)
            lib.moe_ffn_combine(L, xd, T, b.topk_w, b.plan, b.y, lib.DTYPE[wl.y_dtype], st.ws_ptr, st.ws_bytes)
            durations.append((e0, e1))
            u = U[i]
            launch_bytes.append((u + 1) * (gate_b + up_b) + T * d * 2 + T * (k + 1) * f * 4)
            launch_flops.append(2 * T * (k + 1) * 2 * d * f)
    torch.cuda.synchronize()
    dur_ms = np.array([a.elapsed_time(b) for a, b in durations])
    avg_ms = float(dur_ms.mean())
    key = "decode_persistent" if persistent else ("fused_gateup" if fused else name)
    kname, _, ksrc = DOMINANT[key]
    digest = source_digest(ksrc)
    mfma_bound = name.startswith("prefill")
    if mfma_bound:
        achieved = float(np.mean(launch_flops)) / (avg_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFS, 4)}
    else:
        achieved = float(np.mean(launch_bytes)) / (avg_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["traffic"] = traffic_from_profile(name, digest)
    roof["kernel"] = kname
    roof["avg_launch_us"] = round(avg_ms * 1e3, 2)
    roof["alg_bytes_per_launch"] = int(np.mean(launch_bytes))
    roof["alg_flops_per_launch"] = int(np.mean(launch_flops))
    roof["source_digest"] = digest
    log(f"[bench {name}] dominant kernel {kname}: {avg_ms * 1e3:.2f} us/launch -> {roof['achieved']} "
        f"{roof['unit']} ({100 * roof['frac']:.1f}% of peak)")

    cpu = cpu_baseline(wl, st, args.cpu_seconds) if with_cpu else None
    out = {
        "value": round(value, 2), "unit": "tokens/s", "ms_per_step": round(ms_per_step, 5),
        "dtype": "f16",
        "config": {
            "workload": f"{wl.name}: {wl.n_layers}-layer routed-expert stack, T={T} tokens/step",
            "T": T, "layers": wl.n_layers, "d": d, "f": f, "E": E, "k": k, "shared_expert": wl.shared,
            "formats": f"{wl.gate_type}/{wl.up_type}/{wl.down_type}", "path": path,
            "U_mean": round(float(np.mean(U)), 2),
            "step_ms_median": round(float(np.median(per)), 5), "step_ms_min": round(float(per.min()), 5),
            "step_ms_p90": round(float(np.percentile(per, 90)), 5),
            "stack_alg_bytes": int(stack_bytes), "stack_hbm_frac": round(stack_hbm_frac, 4),
            "stack_alg_flops": int(stack_flops), "stack_mfma_frac": round(stack_mfma_frac, 4),
        },
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    # free the stack before the next workload is generated
    del st, layers, h0
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              f"this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.copy_calibration} MiB x 5")
        return

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    with_cpu = not args.no_cpu_baseline
    head = measure(args.workload, args, with_cpu)
    others = {}
    if not args.only:
        for name in ALL_WORKLOADS:
            if name != args.workload:
                others[name] = measure(name, args, with_cpu)
    ref = stream_read_gbs(torch)
    log(f"[bench] streaming-read reference: {ref} GB/s")
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
        "roofline": dict(head["roofline"], stream_read_ref_gbs=ref),
        "cpu_baseline": head["cpu_baseline"],
        "workloads": others,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(wl, st, target_s):
    """The oracle, as it stands, on a bounded sample of the same workload: whole
    layers (every token) for T <= 64, a token sample of one layer for prefill,
    fed with the GPU run's own layer inputs.  Scaled to tokens/s of the stack.
    BLAS runs with as many threads as this process may use cores."""
    import numpy as np

    from oracle import moe as M
    from quantized_routed_expert_amd import synth

    cores = len(os.sched_getaffinity(0))
    blas = "unknown"
    limiter = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')} ({os.path.basename(info[0].get('filepath', ''))})"
        limiter = threadpool_limits(limits=cores, user_api="blas")
    except Exception:
        pass
    T = wl.T
    tokens = np.arange(T) if T <= 64 else np.arange(0, T, T // 8)[:8]
    t_layers, n_done = 0.0, 0
    try:
        for l in range(wl.n_layers):
            b = st.bufs[l]
            x = st.xs[l].float().cpu().numpy().astype(np.float64)[tokens]
            idx = b.topk_idx.cpu().numpy()[tokens]
            lnp = synth.layer_to_numpy(st.layers[l], set(idx.ravel().tolist()))
            t0 = time.perf_counter()
            L64, L32, oidx, w = M.route(lnp["router_w"], lnp["router_b"], x, wl.k)
            M.layer_from_selection(lnp, x, oidx, w, out_dtype=wl.y_dtype, cache=False)
            t_layers += time.perf_counter() - t0
            n_done += 1
            if t_layers >= target_s:
                break
    finally:
        if limiter is not None:
            limiter.restore_original_limits()
    per_layer = t_layers / n_done
    tok_s = len(tokens) / (per_layer * wl.n_layers)
    sample = (f"{n_done} of {wl.n_layers} layers, {len(tokens)} of {T} tokens per layer, oracle float64 "
              f"(route + experts + combine), {t_layers:.1f} s; rate scaled to the full stack")
    log(f"[bench {wl.name}] cpu oracle: {tok_s:.4f} tokens/s ({sample}, {cores} cores, BLAS {blas})")
    return {"value": round(tok_s, 5), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": sample, "blas": blas}


if __name__ == "__main__":
    main()
