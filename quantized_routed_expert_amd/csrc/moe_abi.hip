// C ABI entry points (include/moe.h): host-side validation, workspace
// accounting and dispatch to the kernel launchers.  Nothing here allocates
// device memory or synchronises.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <mutex>

#include "moe.h"
#include "moe_launch.h"

using namespace qre;

namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

bool valid_qtype(int t) { return t == MOE_Q8_0 || t == MOE_IQ4_NL || t == MOE_NVFP4 || t == MOE_Q5_1; }
bool valid_dtype(int t) { return t == MOE_F32 || t == MOE_BF16; }

moe_status check_qmatrix(const moe_qmatrix& m, int n_expert, int rows, int cols) {
  if (!valid_qtype(m.type)) return MOE_ERR_UNSUPPORTED;
  if (m.n_expert != n_expert || m.rows != rows || m.cols != cols) return MOE_ERR_INVALID_ARG;
  if (!m.codes || !m.scales) return MOE_ERR_INVALID_ARG;
  if (m.type == MOE_NVFP4 && !m.tensor_scale) return MOE_ERR_INVALID_ARG;
  if (!aligned(m.codes, 16) || !aligned(m.scales, 16)) return MOE_ERR_ALIGNMENT;
  if (m.tensor_scale && !aligned(m.tensor_scale, 4)) return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

moe_status check_dims(const moe_layer* L) {
  if (!L) return MOE_ERR_INVALID_ARG;
  if (L->d <= 0 || L->f <= 0 || L->E <= 0 || L->k <= 0 || L->k > L->E) return MOE_ERR_INVALID_ARG;
  if (L->E > kMaxE || L->k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (L->d % 128 != 0 || L->f % 128 != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_router(const moe_layer* L) {
  moe_status st = check_dims(L);
  if (st != MOE_OK) return st;
  if (!L->router_w) return MOE_ERR_INVALID_ARG;
  if (!aligned(L->router_w, 16) || (L->router_bias && !aligned(L->router_bias, 4))) return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

moe_status check_layer(const moe_layer* L) {
  moe_status st = check_dims(L);
  if (st != MOE_OK) return st;
  if ((st = check_qmatrix(L->gate, L->E, L->f, L->d)) != MOE_OK) return st;
  if ((st = check_qmatrix(L->up, L->E, L->f, L->d)) != MOE_OK) return st;
  if ((st = check_qmatrix(L->down, L->E, L->d, L->f)) != MOE_OK) return st;
  if (L->gate.type != L->up.type) return MOE_ERR_UNSUPPORTED;
  if (L->gate.type == MOE_Q5_1) return MOE_ERR_UNSUPPORTED;  // a down format only
  if (L->has_shared != 0 && L->has_shared != 1) return MOE_ERR_INVALID_ARG;
  if (L->has_shared) {
    if ((st = check_qmatrix(L->shared_gate, 1, L->f, L->d)) != MOE_OK) return st;
    if ((st = check_qmatrix(L->shared_up, 1, L->f, L->d)) != MOE_OK) return st;
    if ((st = check_qmatrix(L->shared_down, 1, L->d, L->f)) != MOE_OK) return st;
    if (L->shared_gate.type != L->gate.type || L->shared_up.type != L->up.type ||
        L->shared_down.type != L->down.type)
      return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

// moe_route's workspace: the logits when the caller passes none, then the
// K-split router's slices (bf16 tokens, 8 < T <= 64).
size_t route_ws(const moe_layer* L, int T, int x_dtype) {
  return align_up((size_t)T * L->E * 4, 256) + align_up(router_partials_bytes(T, L->E, L->d, x_dtype), 256);
}

size_t ffn_ws(const moe_layer* L, int T, int x_dtype) {
  if (T <= kDecodeMaxT && !prefill_exact(*L, T, x_dtype)) return decode_ws_bytes(T, L->d, L->f, L->k, x_dtype);
  if (T <= kDecodeMaxT) return prefill_exact_ws_bytes(T, L->d, L->f, L->k);
  return prefill_ws_bytes(T, L->d, L->f, L->k);
}

moe_status check_plan_buf(const moe_plan_buf* p) {
  if (!p || !p->counts || !p->offsets || !p->row_token || !p->row_slot || !p->slot_row || !p->active ||
      !p->n_active || !p->error)
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_version(void) { return "quantized_routed_expert_amd 0.1 (gfx950)"; }

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported format or shape";
    case MOE_ERR_ALIGNMENT: return "misaligned device pointer";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch or runtime error";
  }
  return "unknown status";
}

size_t moe_workspace_size(const moe_layer* layer, int32_t T_max) {
  if (check_dims(layer) != MOE_OK || T_max < 1) return 0;
  const int Td = T_max < kDecodeMaxT ? T_max : kDecodeMaxT;
  // the router's slices grow with T up to 64 tokens
  size_t need = align_up((size_t)T_max * layer->E * 4, 256) +
                align_up(router_partials_bytes(T_max < 64 ? T_max : 64, layer->E, layer->d, MOE_BF16), 256);
  const size_t pl = plan_ws_bytes(T_max, layer->E);
  if (pl > need) need = pl;
  const size_t dec = decode_ws_bytes(Td, layer->d, layer->f, layer->k, MOE_F32);
  if (dec > need) need = dec;
  if (prefill_exact(*layer, Td, MOE_BF16)) {  // (grows with T: the largest batch that takes it)
    const size_t ex = prefill_exact_ws_bytes(Td, layer->d, layer->f, layer->k);
    if (ex > need) need = ex;
  }
  if (T_max > kDecodeMaxT) {
    const size_t pf = prefill_ws_bytes(T_max, layer->d, layer->f, layer->k);
    if (pf > need) need = pf;
  }
  return need;
}

moe_status moe_route(const moe_layer* layer, const void* x, int32_t x_dtype, int32_t T, int32_t* topk_idx,
                     float* topk_w, float* logits, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_router(layer);
  if (st != MOE_OK) return st;
  if (!x || !topk_idx || !topk_w || T < 1 || !valid_dtype(x_dtype)) return MOE_ERR_INVALID_ARG;
  float* lg = logits;
  float* partials = nullptr;
  const bool slices = router_partials_bytes(T, layer->E, layer->d, x_dtype) > 0;
  if (!lg || slices) {
    if (!ws || ws_bytes < route_ws(layer, T, x_dtype)) return MOE_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return MOE_ERR_ALIGNMENT;
    if (!lg) lg = (float*)ws;
    partials = (float*)((char*)ws + align_up((size_t)T * layer->E * 4, 256));
  }
  hipStream_t s = (hipStream_t)stream;
  return hip_status(launch_route(layer->router_w, layer->router_bias, x, x_dtype, T, layer->E, layer->d, layer->k, lg,
                                 partials, topk_idx, topk_w, s));
}

moe_status moe_plan(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E, const moe_plan_buf* plan, void* ws,
                    size_t ws_bytes, void* stream) {
  if (!topk_idx || T < 1 || k < 1 || E < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (E > kMaxE || k > kMaxK) return MOE_ERR_UNSUPPORTED;
  moe_status st = check_plan_buf(plan);
  if (st != MOE_OK) return st;
  if (!ws || ws_bytes < plan_ws_bytes(T, E)) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return MOE_ERR_ALIGNMENT;
  return hip_status(launch_plan(topk_idx, T, k, E, plan_dev(*plan), ws, (hipStream_t)stream));
}

static moe_status ffn_checked(int stage_lo, int stage_hi, const moe_layer* layer, const void* x, int32_t x_dtype,
                              int32_t T, const float* topk_w, const moe_plan_buf* plan, void* y, int32_t y_dtype,
                              void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_layer(layer);
  if (st != MOE_OK) return st;
  if (T < 1 || !valid_dtype(x_dtype)) return MOE_ERR_INVALID_ARG;
  const bool need_x = stage_lo <= kStageGateUp;
  const bool need_y = stage_hi >= kStageCombine;
  if (need_x && !x) return MOE_ERR_INVALID_ARG;
  if (need_y && (!topk_w || !y || !valid_dtype(y_dtype))) return MOE_ERR_INVALID_ARG;
  if ((st = check_plan_buf(plan)) != MOE_OK) return st;
  if ((need_x && !aligned(x, 16)) || (need_y && !aligned(y, 16))) return MOE_ERR_ALIGNMENT;
  if (!ws || ws_bytes < ffn_ws(layer, T, x_dtype)) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return MOE_ERR_ALIGNMENT;
  FfnCall c{layer, x, x_dtype, T, topk_w, plan_dev(*plan), y, y_dtype, ws};
  hipStream_t s = (hipStream_t)stream;
  for (int stage = stage_lo; stage <= stage_hi; ++stage) {
    const hipError_t e = (T <= kDecodeMaxT && !prefill_exact(*layer, T, x_dtype)) ? launch_decode_stage(stage, c, s)
                                                                                  : launch_prefill_stage(stage, c, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

moe_status moe_ffn_forward(const moe_layer* layer, const void* x, int32_t x_dtype, int32_t T, const float* topk_w,
                           const moe_plan_buf* plan, void* y, int32_t y_dtype, void* ws, size_t ws_bytes,
                           void* stream) {
  return ffn_checked(kStagePrepare, kStageCombine, layer, x, x_dtype, T, topk_w, plan, y, y_dtype, ws, ws_bytes,
                     stream);
}

moe_status moe_ffn_prepare(const moe_layer* layer, const void* x, int32_t x_dtype, int32_t T,
                           const moe_plan_buf* plan, void* ws, size_t ws_bytes, void* stream) {
  return ffn_checked(kStagePrepare, kStagePrepare, layer, x, x_dtype, T, nullptr, plan, nullptr, MOE_F32, ws,
                     ws_bytes, stream);
}

moe_status moe_ffn_gateup(const moe_layer* layer, const void* x, int32_t x_dtype, int32_t T,
                          const moe_plan_buf* plan, void* ws, size_t ws_bytes, void* stream) {
  return ffn_checked(kStageGateUp, kStageGateUp, layer, x, x_dtype, T, nullptr, plan, nullptr, MOE_F32, ws, ws_bytes,
                     stream);
}

moe_status moe_ffn_down(const moe_layer* layer, int32_t x_dtype, int32_t T, const moe_plan_buf* plan, void* ws,
                        size_t ws_bytes, void* stream) {
  return ffn_checked(kStageDown, kStageDown, layer, nullptr, x_dtype, T, nullptr, plan, nullptr, MOE_F32, ws,
                     ws_bytes, stream);
}

moe_status moe_ffn_combine(const moe_layer* layer, int32_t x_dtype, int32_t T, const float* topk_w,
                           const moe_plan_buf* plan, void* y, int32_t y_dtype, void* ws, size_t ws_bytes,
                           void* stream) {
  return ffn_checked(kStageCombine, kStageCombine, layer, nullptr, x_dtype, T, topk_w, plan, y, y_dtype, ws,
                     ws_bytes, stream);
}

moe_status moe_dequantize(const moe_qmatrix* m, int32_t expert, int32_t out_dtype, void* dst, void* stream) {
  if (!m || !dst || !(valid_dtype(out_dtype) || out_dtype == MOE_F16)) return MOE_ERR_INVALID_ARG;
  if (!valid_qtype(m->type)) return MOE_ERR_UNSUPPORTED;
  if (m->rows <= 0 || m->cols <= 0 || m->n_expert <= 0 || expert < 0 || expert >= m->n_expert)
    return MOE_ERR_INVALID_ARG;
  if (m->cols % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (!m->codes || !m->scales || (m->type == MOE_NVFP4 && !m->tensor_scale)) return MOE_ERR_INVALID_ARG;
  if (!aligned(m->codes, 16) || !aligned(m->scales, 16) || !aligned(dst, 4)) return MOE_ERR_ALIGNMENT;
  if (out_dtype == MOE_F16) return hip_status(launch_dequant_pf(qmat_dev(*m), expert, dst, (hipStream_t)stream));
  return hip_status(launch_dequant(qmat_dev(*m), expert, out_dtype, dst, (hipStream_t)stream));
}

size_t moe_decode_stack_workspace_size(const moe_layer* layer, int32_t T_max) {
  if (check_dims(layer) != MOE_OK || T_max < 1 || T_max > kFusedMaxT) return 0;
  if (layer->d % 1024 != 0 || layer->d > 4096) return 0;
  return fused_ws_bytes(T_max, layer->d, layer->f, layer->k, layer->E);
}

// The layers of a fused decode stack: each valid, all of one shape and format
// set, d within the fused step's coverage.
static moe_status check_stack(const moe_layer* layers, int32_t n_layers) {
  const moe_layer& L0 = layers[0];
  for (int l = 0; l < n_layers; ++l) {
    const moe_layer& L = layers[l];
    moe_status st = check_layer(&L);
    if (st != MOE_OK) return st;
    if ((st = check_router(&L)) != MOE_OK) return st;
    if (L.d != L0.d || L.f != L0.f || L.E != L0.E || L.k != L0.k || L.has_shared != L0.has_shared ||
        L.gate.type != L0.gate.type || L.down.type != L0.down.type)
      return MOE_ERR_UNSUPPORTED;
  }
  if (L0.d % 1024 != 0 || L0.d > 4096) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status moe_decode_stack(const moe_layer* layers, int32_t n_layers, float* h, int32_t T, float eps,
                            const moe_stack_record* rec, void* ws, size_t ws_bytes, void* stream) {
  if (!layers || n_layers < 1 || !h || T < 1 || !(eps >= 0.0f)) return MOE_ERR_INVALID_ARG;
  if (T > kFusedMaxT) return MOE_ERR_UNSUPPORTED;
  const moe_layer& L0 = layers[0];
  moe_status st = check_stack(layers, n_layers);
  if (st != MOE_OK) return st;
  if (!aligned(h, 16)) return MOE_ERR_ALIGNMENT;
  FusedRecord r{};
  r.eps = eps;
  if (rec) {
    r.logits = rec->logits;
    r.topk_idx = rec->topk_idx;
    r.topk_w = rec->topk_w;
    r.x = (uint16_t*)rec->x;
    r.y = rec->y;
    r.error = rec->error;
    r.events = (hipEvent_t*)rec->events;
    if ((r.logits && !aligned(r.logits, 4)) || (r.topk_idx && !aligned(r.topk_idx, 4)) ||
        (r.topk_w && !aligned(r.topk_w, 4)) || (r.x && !aligned(r.x, 16)) || (r.y && !aligned(r.y, 16)) ||
        (r.error && !aligned(r.error, 4)))
      return MOE_ERR_ALIGNMENT;
  }
  if (!ws || ws_bytes < fused_ws_bytes(T, L0.d, L0.f, L0.k, L0.E)) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return MOE_ERR_ALIGNMENT;
  return hip_status(launch_fused_step(layers, n_layers, h, T, r, ws, (hipStream_t)stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free variant of moe_decode_stack: its workspace is a file-scope
// device array, one per GPU the library runs on (each device holds its own
// copy at its own address).  The array's name is a host-side stand-in: host
// code uses only the device address hipGetSymbolAddress returns, taken once
// per device on the first call with that device current.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = (size_t)8 << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, or null on failure.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t moe_decode_stack_scratch_bytes(void) { return kScratchBytes; }

moe_status moe_decode_stack_noalloc(const moe_layer* layers, int32_t n_layers, float* h, int32_t T, float eps,
                                    const moe_stack_record* rec, void* stream) {
  if (!layers || n_layers < 1 || T < 1) return MOE_ERR_INVALID_ARG;
  const size_t need = moe_decode_stack_workspace_size(&layers[0], T);
  // an invalid or unsupported shape: moe_decode_stack's own validation names it
  if (need == 0) return moe_decode_stack(layers, n_layers, h, T, eps, rec, nullptr, 0, stream);
  if (need > kScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = scratch_address();
  if (!ws) return MOE_ERR_HIP;
  return moe_decode_stack(layers, n_layers, h, T, eps, rec, ws, kScratchBytes, stream);
}

int32_t moe_decode_stack_persistent(const moe_layer* layers, int32_t n_layers, int32_t T) {
  if (!layers || n_layers < 1 || T < 1 || T > kFusedMaxT || check_stack(layers, n_layers) != MOE_OK) return 0;
  return fused_step_persistent(layers[0], n_layers, T) ? 1 : 0;
}

moe_status moe_residual_rmsnorm(float* h, const void* y, int32_t y_dtype, int32_t T, int32_t d, float eps,
                                void* x_out, void* stream) {
  if (!h || !x_out || T < 1 || d < 1 || !valid_dtype(y_dtype) || !(eps >= 0.0f)) return MOE_ERR_INVALID_ARG;
  if (d % 4 != 0) return MOE_ERR_UNSUPPORTED;  // the kernel moves 4 columns at a time
  if (!aligned(h, 16) || !aligned(x_out, 8) || (y && !aligned(y, y_dtype == MOE_BF16 ? 8 : 16)))
    return MOE_ERR_ALIGNMENT;
  return hip_status(launch_residual_rmsnorm(h, y, y_dtype, T, d, eps, x_out, (hipStream_t)stream));
}

}  // extern "C"
