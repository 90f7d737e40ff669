/*
 * moe.h -- C ABI of the MI355X (gfx950) routed-expert MoE feed-forward library.
 *
 * The library computes one routed-expert layer of a mixture-of-experts model:
 *   router GEMV -> softmax over the top-k (renormalised, lower index first on
 *   ties) -> device-side expert plan (per-expert counts, prefix scan, stable
 *   token scatter) -> grouped dequantising gate/up projections with fused
 *   SwiGLU -> down projection -> shared expert -> deterministic weighted combine.
 *
 * Sources.  "Qwen3.8-Flash-Next UD-IQ2_XS (L4 fix) for Basalt", section "What
 * was changed": the routed experts run through a device-planned MoE tail plus
 * grouped kernels, which only run when every layer's expert format is covered
 * (covered down formats include IQ4_NL, NVFP4 and Q8_0; IQ4_NL is 4.5 bits per
 * weight).  "Basalt at 665 tok/s? ...", section "RAM and VRAM Hold Different
 * Parts of the Expert Weights": each token uses only its selected experts.
 * The model card ("The fastest inference engine for Qwen3.8-Flash-Next on
 * Blackwell", section "Sources"): tensors are GGUF tensors copied unchanged, so
 * quant blocks run along each matrix row's reduction (input) dimension.  The
 * router, top-k rule, SwiGLU, shared expert, combine and block layouts follow
 * the workload definition of the routed-expert layer.
 *
 * Conventions (all entry points):
 *  - Every pointer named "device" is GPU memory owned by the caller; the
 *    library never allocates or frees device memory and keeps no per-call
 *    state.  Host structs (moe_layer, moe_qmatrix, moe_plan_buf) are read
 *    during the call only.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *    work and return without synchronising, so they may be captured into a
 *    HIP graph.
 *  - Arguments are validated on the host before anything is enqueued; on an
 *    error nothing is launched and the status says why.  A failed launch
 *    returns MOE_ERR_HIP.
 *  - Calls that share a workspace must not overlap in time (same stream, or
 *    ordered by events).
 *  - Thread-safe: no mutable global state.
 */
#ifndef QRE_MOE_H
#define QRE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, bad size, k > E, T < 1, ... */
  MOE_ERR_UNSUPPORTED = -2, /* a (format, role, shape) the kernels do not cover */
  MOE_ERR_ALIGNMENT = -3,   /* a device pointer is not suitably aligned */
  MOE_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required */
  MOE_ERR_HIP = -5          /* a HIP launch or runtime call failed */
} moe_status;

/* Activation / output element types.  MOE_F16 is accepted by moe_dequantize
 * only (the prefill path's fp16 weight tile). */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_F16 = 2 } moe_dtype;

/* Block formats; all blocks run along a row's reduction dimension (cols).
 *  MOE_Q8_0   32-element blocks; codes int8 [n][rows][cols]; scales IEEE
 *             binary16 [n][rows][cols/32]; w = code * scale.
 *  MOE_IQ4_NL 32-element blocks; codes uint8 [n][rows][cols/2], a block's 16
 *             bytes hold element j in the low nibble of byte j and element
 *             j+16 in the high nibble; scales binary16 [n][rows][cols/32];
 *             w = codebook[nibble] * scale with the IQ4_NL codebook
 *             {-127,-104,-83,-65,-49,-35,-22,-10,1,13,25,38,53,69,89,113}.
 *  MOE_NVFP4  16-element blocks; codes uint8 [n][rows][cols/2] of FP4 E2M1,
 *             element 2i in the low nibble of byte i; scales FP8 E4M3 (OCP)
 *             [n][rows][cols/16]; tensor_scale fp32 [n];
 *             w = fp32(e2m1 * e4m3 * tensor_scale).
 *  MOE_Q5_1   32-element blocks of 5-bit codes q (ggml's Q5_1, a covered down
 *             format); codes uint8 [n][rows][cols/2] hold the low 4 bits in
 *             the IQ4_NL byte order; scales [n][rows][cols/32] 8-byte records:
 *             binary16 d, binary16 m, then a little-endian uint32 whose bit e
 *             is the fifth bit of block element e; w = d * q + m.  Down
 *             projections only (MOE_ERR_UNSUPPORTED for gate / up).
 */
typedef enum { MOE_Q8_0 = 1, MOE_IQ4_NL = 2, MOE_NVFP4 = 3, MOE_Q5_1 = 4 } moe_qtype;

/* One projection for n_expert experts, structure of arrays (codes and scales
 * in separate device arrays).  rows = outputs, cols = reduction dimension.
 * codes and scales must be 16-byte aligned, tensor_scale 4-byte. */
typedef struct {
  int32_t type;              /* moe_qtype */
  int32_t n_expert;
  int32_t rows;
  int32_t cols;
  const void* codes;         /* device */
  const void* scales;        /* device */
  const float* tensor_scale; /* device, MOE_NVFP4 only, else NULL */
} moe_qmatrix;

/* One MoE layer.  gate/up: rows = f, cols = d; down: rows = d, cols = f.
 * gate and up share one format (Q8_0, IQ4_NL or NVFP4-style); down takes any
 * of the four; the shared expert (if any) uses the routed experts' format for
 * each role and has n_expert = 1.  Kernel coverage: d and f multiples of 128,
 * 1 <= k <= E <= 1024, k <= 32. */
typedef struct {
  int32_t d, f, E, k;
  const float* router_w;     /* device fp32 [E][d] */
  const float* router_bias;  /* device fp32 [E], or NULL for no bias */
  moe_qmatrix gate, up, down;
  int32_t has_shared;        /* 0 or 1 */
  moe_qmatrix shared_gate, shared_up, shared_down;
} moe_layer;

/* The expert plan for T tokens with k slots each (all device int32):
 *  counts[E]        pairs routed to each expert (pairs kept, see error)
 *  offsets[E+1]     exclusive prefix sum of counts; offsets[E] = valid pairs
 *  row_token[T*k]   token of plan row r; rows of expert e are
 *                   [offsets[e], offsets[e+1]) in ascending token order
 *  row_slot[T*k]    slot j of plan row r
 *  slot_row[T*k]    plan row of pair (t, j) at index t*k + j (-1 if dropped)
 *  active[E]        ids with counts > 0, ascending, padded with -1
 *  n_active[1]      number of active experts
 *  error[1]         0, or bits set:
 *                     1 = an expert id outside [0, E) was dropped;
 *                     2 = an SwiGLU activation was not finite (T <= 64,
 *                         where h is kept in fp32) or exceeded the fp16
 *                         range (the prefill path, T > 64)
 *                         (moe_ffn_forward, moe_decode_stack);
 *                     4 = an id repeated within a token was dropped (a top-k
 *                         selection names each expert once; of repeats the
 *                         lowest slot j keeps its row);
 *                     8 = the prefill path (T > 64) met a Q8_0 / IQ4_NL block
 *                         scale whose product with the format's largest code
 *                         magnitude (128 / 127) is not finite in fp16, i.e.
 *                         |scale| >= 512 (Q8_0) or >= 516 (IQ4_NL), or a
 *                         non-finite scale, or a Q5_1 block whose
 *                         max(|m|, |31 d + m|) reaches 65520: such weights
 *                         may be infinite.
 *                   A dropped pair gets slot_row -1 and no plan row.
 * Rows past offsets[E] in row_token / row_slot are set to -1. */
typedef struct {
  int32_t* counts;
  int32_t* offsets;
  int32_t* row_token;
  int32_t* row_slot;
  int32_t* slot_row;
  int32_t* active;
  int32_t* n_active;
  int32_t* error;
} moe_plan_buf;

/* Router, top-k and gate weights for T tokens ("RAM and VRAM Hold Different
 * Parts of the Expert Weights": each token runs only its selected experts).
 *   logits[t][e] = fp32( sum_i router_w[e][i] * x[t][i] + bias[e] )
 *   topk_idx[t][j]  the k largest logits, descending, lower id first on ties
 *   topk_w[t][j]    softmax over the k selected logits (sums to 1)
 * x: device [T][d] of x_dtype (MOE_F32 or MOE_BF16).  logits: device fp32
 * [T][E] output, or NULL (then the workspace holds them).  The sum is
 * accumulated in fp64 for T <= 8 and for fp32 tokens up to T = 64; otherwise
 * in fp32 (bf16 tokens: exact products with three bf16 parts of each weight,
 * on MFMA; for 8 < T <= 64 over slices of d added in a fixed order).  ws:
 * device workspace of at least moe_workspace_size(layer, T) bytes, 256-byte
 * aligned; it may be NULL only where logits is given and no slices are used
 * (MOE_ERR_WORKSPACE otherwise). */
moe_status moe_route(const moe_layer* layer, const void* x, int32_t x_dtype, int32_t T,
                     int32_t* topk_idx, float* topk_w, float* logits,
                     void* ws, size_t ws_bytes, void* stream);

/* Expert plan ("device-planned MoE tail", "What was changed") from topk_idx
 * device [T][k]: fills every array of *plan (see moe_plan_buf), in a fixed,
 * deterministic order.  Out-of-range ids are dropped and flagged in error. */
moe_status moe_plan(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                    const moe_plan_buf* plan, void* ws, size_t ws_bytes, void* stream);

/* Routed experts + shared expert + combine ("grouped kernels", "What was
 * changed"):
 *   for every plan row r = (t, e):  h_r = silu(W_g[e] x_t) * (W_u[e] x_t),
 *                                   o_r = W_d[e] h_r
 *   s_t = the same with the shared expert (weight 1), if present
 *   y_t = s_t + sum_j topk_w[t][j] * o_{slot_row[t*k+j]}   (slots in order j)
 * x: device [T][d] of x_dtype; y: device [T][d] of y_dtype.  For T <= 64 the
 * decode path runs: exact dequantisation, fp32 accumulation; tokens enter the
 * products as fp16 with a power-of-two scale per token (fp32 tokens as hi/lo
 * pairs), and each SwiGLU row h, formed in fp32, as fp16 hi/lo parts scaled by
 * a power of two per row (error bit 2 if an h is not finite).  Batches of 29
 * to 64 bf16 tokens with NVFP4-style gate, up and down weights take the
 * prefill GEMMs instead, in a mode with these same numerics (the weights are
 * exact in fp16, h is kept in fp32 and split per row as above, the expert
 * outputs are fp32), which is faster at those sizes.  For T > 64 the prefill
 * path runs: weights are rounded to fp16 (code times block scale, rounded
 * once: relative error at most 2^-11, never a lossy subnormal, since a
 * product below 2^-14 has a subnormal scale and is then an exact multiple of
 * 2^-24; error bit 8 flags scales at which a weight can overflow;
 * NVFP4-style weights are exact and their tensor scale is applied in fp32),
 * tokens are scaled by a power of two per token into fp16 (exact for bf16
 * tokens), SwiGLU activations are rounded to fp16 (error bit 2 if one
 * exceeds 65504 in magnitude; values below 2^-14 keep an absolute precision
 * of 2^-25), fp16 MFMA with fp32 accumulation.
 * The combine never uses atomics: results are bitwise reproducible. */
moe_status moe_ffn_forward(const moe_layer* layer, const void* x, int32_t x_dtype, int32_t T,
                           const float* topk_w, const moe_plan_buf* plan,
                           void* y, int32_t y_dtype, void* ws, size_t ws_bytes, void* stream);

/* The four stages of moe_ffn_forward, callable one by one (same arguments and
 * order, one stream, one workspace; the stages pass their intermediates
 * through the workspace, whose contents are only valid between the stages of
 * one call sequence with the same layer, T and x_dtype):
 *  moe_ffn_prepare  activation layout for the expert products: fp16 tokens
 *                   with per-token power-of-two scales, and the order in
 *                   which the expert passes take the active experts (T <= 64:
 *                   by descending token count; prefill: the device tile list
 *                   over the plan)
 *  moe_ffn_gateup   grouped gate/up projections + SwiGLU -> h rows
 *  moe_ffn_down     grouped down projections -> o rows
 *  moe_ffn_combine  y_t = s_t + sum_j topk_w[t][j] * o_{slot_row[t*k+j]}
 * Each stage is one kernel launch. */
moe_status moe_ffn_prepare(const moe_layer* layer, const void* x, int32_t x_dtype, int32_t T,
                           const moe_plan_buf* plan, void* ws, size_t ws_bytes, void* stream);
moe_status moe_ffn_gateup(const moe_layer* layer, const void* x, int32_t x_dtype, int32_t T,
                          const moe_plan_buf* plan, void* ws, size_t ws_bytes, void* stream);
moe_status moe_ffn_down(const moe_layer* layer, int32_t x_dtype, int32_t T, const moe_plan_buf* plan,
                        void* ws, size_t ws_bytes, void* stream);
moe_status moe_ffn_combine(const moe_layer* layer, int32_t x_dtype, int32_t T, const float* topk_w,
                           const moe_plan_buf* plan, void* y, int32_t y_dtype, void* ws, size_t ws_bytes,
                           void* stream);

/* Test hook: dequantise expert `expert` of `m` into dst device [rows][cols]:
 *  MOE_F32   exact values (NVFP4-style: fp32(e2m1 * e4m3 * tensor_scale);
 *            Q5_1: fp32(d * q + m), one rounding of the exact value);
 *  MOE_BF16  round-to-nearest-even of those values;
 *  MOE_F16   the fp16 weight tile the prefill GEMM multiplies, produced by the
 *            GEMM's own decode routine: Q8_0 / IQ4_NL the code times the
 *            block scale in fp16 arithmetic (one rounding to nearest even of
 *            the exact product; subnormal below 2^-14, infinite when the
 *            product reaches 65520 -- see error bit 8); Q5_1 d * q + m in fp16
 *            arithmetic (one fused rounding); NVFP4-style
 *            e2m1 * e4m3 (exact), without the tensor scale, which the GEMM
 *            applies to its fp32 result.
 * dst must be 4-byte aligned. */
moe_status moe_dequantize(const moe_qmatrix* m, int32_t expert, int32_t out_dtype, void* dst,
                          void* stream);

/* Pre-norm residual glue between stacked layers (the pages do not say what
 * joins the MoE layers; this is the plain pre-norm residual chain):
 *   if y != NULL:  h[t][i] += y[t][i]            (fp32 residual, y of y_dtype)
 *   x[t][i] = bf16( h[t][i] / sqrt(mean_i h[t][i]^2 + eps) )
 * h: device fp32 [T][d] (updated in place, 16-byte aligned); x_out: device
 * bf16 [T][d] (8-byte aligned); y: 8-byte (bf16) or 16-byte (fp32) aligned.
 * d must be a multiple of 4 (MOE_ERR_UNSUPPORTED otherwise). */
moe_status moe_residual_rmsnorm(float* h, const void* y, int32_t y_dtype, int32_t T, int32_t d,
                                float eps, void* x_out, void* stream);

/* Optional per-layer records of moe_decode_stack (device pointers, each NULL
 * to skip; layer l's entries start at l * (per-layer size)). */
typedef struct moe_stack_record {
  float* logits;      /* [n_layers][T][E] fp32 router logits */
  int32_t* topk_idx;  /* [n_layers][T][k] selected experts (descending logit) */
  float* topk_w;      /* [n_layers][T][k] renormalised gate weights */
  void* x;            /* [n_layers][T][d] bf16 layer inputs */
  float* y;           /* [n_layers][T][d] fp32 layer outputs */
  int32_t* error;     /* [n_layers] plan / overflow flags of each layer (bits as moe_plan_buf.error) */
  void** events;      /* [n_layers][2] hipEvent_t handles (created by the caller), attached to each
                         layer's gate/up launch so that they carry that kernel's start and end; for
                         timing the kernel in eager (not graph-captured) calls.  When the step is the
                         persistent launch (moe_decode_stack_persistent), entries 0 and 1 carry that
                         launch's start and end and the others are unused. */
} moe_stack_record;

/* Fused decode step through a stack of routed-expert layers for T <= 8
 * tokens: for each layer l in order
 *   x_l = bf16(rmsnorm(h)),  y_l = the routed-expert layer l on x_l,  h += y_l
 * (the same computation as moe_residual_rmsnorm -> moe_route -> moe_plan ->
 * moe_ffn_forward(y fp32) per layer, with the glue described at
 * moe_residual_rmsnorm; the layer itself follows the routing and expert
 * passages cited at moe_route, moe_plan and moe_ffn_forward).  Each layer is
 * three kernel launches for T = 1 (glue + router; top-k + plan + gate/up +
 * SwiGLU; down, whose last workgroup per 64-column tile forms the combine and
 * the new residual) and four for T > 1 (the glue gets its own launch).
 * Routing and the plan
 * are recomputed in every workgroup of the gate/up launch from the logits,
 * so no launch waits on a separate plan kernel.
 *   layers:  HOST array of n_layers descriptors of one shape (d, f, E, k,
 *            formats and has_shared equal); all weights device-resident.
 *   h:       device fp32 [T][d], the residual stream; updated in place.
 *   rec:     optional records (host struct of device pointers, or NULL).
 *   ws:      device workspace of moe_decode_stack_workspace_size bytes,
 *            256-byte aligned; contents are scratch between calls.
 * Coverage: 1 <= T <= 8, d a multiple of 1024 and at most 4096, activation
 * layout and numerics as the decode path of moe_ffn_forward (bf16 inputs).
 * Errors: validation codes as the per-layer entry points; plan or overflow
 * flags are reported only through rec->error.  Asynchronous on `stream`. */
moe_status moe_decode_stack(const moe_layer* layers, int32_t n_layers, float* h, int32_t T, float eps,
                            const moe_stack_record* rec, void* ws, size_t ws_bytes, void* stream);

/* 1 if moe_decode_stack runs this stack (layers[0]'s shape, n_layers, T) as
 * one persistent launch, 0 if as per-layer launches (always 0 for a stack
 * moe_decode_stack rejects).  The persistent step takes T = 1, at most 128
 * layers, E up to 1024, k up to 32, and rows short enough that every step's
 * weight codes are issued up front: f a multiple of 128 up to 768, d a
 * multiple of 1024 up to 3072 (IQ4_NL / NVFP4-style gate/up) or 1024 (Q8_0
 * gate/up); unless the environment sets QRE_DECODE_LAUNCHES=1.
 * It computes the same layer with the same numerics.  A wait between its
 * workgroups that does not end within its poll bound (2^20 polls; the
 * environment can lower it with QRE_PERSIST_SPIN_MAX=n, read at every call,
 * to exercise this path) sets error bit 16 in the record of the layer it
 * belongs to and an abort word that ends every other wait, so the step ends
 * early: h and the records of that layer and later ones are then incomplete
 * and must not be used. */
int32_t moe_decode_stack_persistent(const moe_layer* layers, int32_t n_layers, int32_t T);

/* Workspace bytes for moe_decode_stack on this layer shape with up to T_max
 * tokens (0 on invalid or unsupported arguments). */
size_t moe_decode_stack_workspace_size(const moe_layer* layer, int32_t T_max);

/* moe_decode_stack for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation, kernels and records, with the workspace taken from a
 * library-owned device array of moe_decode_stack_scratch_bytes() bytes
 * (8 MiB; one per GPU, held until the process ends) instead of a caller
 * workspace.  The caller still passes h and the records.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); its first
 * call on a device looks up that device's array address once.
 *   Errors: as moe_decode_stack; MOE_ERR_WORKSPACE when the shape needs more
 *   than the array holds (moe_decode_stack_workspace_size > 8 MiB), before
 *   any launch; MOE_ERR_HIP if the array's address cannot be obtained.
 *   Every call on one GPU shares that GPU's array and leaves its contents
 *   behind: calls that overlap in time on one GPU (different streams, or
 *   host threads) race and must be serialised by the caller. */
moe_status moe_decode_stack_noalloc(const moe_layer* layers, int32_t n_layers, float* h, int32_t T, float eps,
                                    const moe_stack_record* rec, void* stream);

/* Size in bytes of the array moe_decode_stack_noalloc uses on each GPU. */
size_t moe_decode_stack_scratch_bytes(void);

/* Workspace bytes needed by moe_route / moe_plan / moe_ffn_forward for up to
 * T_max tokens on this layer shape (0 on invalid arguments). */
size_t moe_workspace_size(const moe_layer* layer, int32_t T_max);

/* Static description of a status code. */
const char* moe_status_string(moe_status s);

/* Library version string. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* QRE_MOE_H */
