// Internal launchers: one host function per kernel family, each defined in the
// translation unit that holds its kernels.  All return the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace qre {

// Device view of one projection of one layer (pointers to expert 0).
struct QMatDev {
  int type;
  int rows, cols;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* ts;
};

inline QMatDev qmat_dev(const moe_qmatrix& m) {
  return QMatDev{m.type, m.rows, m.cols, (const uint8_t*)m.codes, (const uint8_t*)m.scales, m.tensor_scale};
}

// Plan arrays (device).
struct PlanDev {
  int32_t* counts;
  int32_t* offsets;
  int32_t* row_token;
  int32_t* row_slot;
  int32_t* slot_row;
  int32_t* active;
  int32_t* n_active;
  int32_t* error;
};

inline PlanDev plan_dev(const moe_plan_buf& p) {
  return PlanDev{p.counts, p.offsets, p.row_token, p.row_slot, p.slot_row, p.active, p.n_active, p.error};
}

// moe_small.hip
hipError_t launch_dequant(const QMatDev& m, int expert, int out_dtype, void* dst, hipStream_t s);
hipError_t launch_router_logits(const float* W, const float* b, const void* x, int x_dtype, int T, int E, int d,
                                float* logits, hipStream_t s);
hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w, hipStream_t s);
// Router logits + top-k for the per-layer path; partials: device scratch of
// router_partials_bytes (the K-split router's slices; unused when that is 0).
size_t router_partials_bytes(int T, int E, int d, int x_dtype);
hipError_t launch_route(const float* W, const float* b, const void* x, int x_dtype, int T, int E, int d, int k,
                        float* logits, float* partials, int32_t* idx, float* w, hipStream_t s);
size_t plan_ws_bytes(int T, int E);
hipError_t launch_plan(const int32_t* idx, int T, int k, int E, const PlanDev& p, void* ws, hipStream_t s);
hipError_t launch_combine(const void* o, int o_bf16, const float* topk_w, const int32_t* slot_row, int T, int k,
                          int d, int has_shared, void* y, int y_dtype, hipStream_t s);
hipError_t launch_residual_rmsnorm(float* h, const void* y, int y_dtype, int T, int d, float eps, void* x_out,
                                   hipStream_t s);

// Expert stages (decode path for T <= kDecodeMaxT, prefill path above).
constexpr int kDecodeMaxT = 64;
enum FfnStage { kStagePrepare = 0, kStageGateUp = 1, kStageDown = 2, kStageCombine = 3 };

struct FfnCall {
  const moe_layer* L;
  const void* x;
  int x_dtype;
  int T;
  const float* topk_w;
  PlanDev p;
  void* y;
  int y_dtype;
  void* ws;
};

// moe_decode.hip
size_t decode_ws_bytes(int T, int d, int f, int k, int x_dtype);
hipError_t launch_decode_stage(int stage, const FfnCall& c, hipStream_t s);

// moe_prefill.hip
size_t prefill_ws_bytes(int T, int d, int f, int k);
// exact mode of the prefill GEMMs for batches of the per-layer path (see moe_prefill.hip)
bool prefill_exact(const moe_layer& L, int T, int x_dtype);
size_t prefill_exact_ws_bytes(int T, int d, int f, int k);
// One expert's prefill weight tile as fp16 (the GEMM's own decode), [rows][cols].
hipError_t launch_dequant_pf(const QMatDev& m, int expert, void* dst, hipStream_t s);
hipError_t launch_prefill_stage(int stage, const FfnCall& c, hipStream_t s);

// Down pass of the fused decode step over its slot table (moe_decode.hip).
struct DecodeArgs;
hipError_t launch_dq_down_table(const DecodeArgs& a, int fmt, int items, hipStream_t s);

// Fused decode step over a stack of layers (moe_fused.hip).  Optional
// per-layer records (null to skip).
constexpr int kFusedMaxT = 8;
struct FusedRecord {
  float* logits;      // [L][T][E]
  int32_t* topk_idx;  // [L][T][k]
  float* topk_w;      // [L][T][k]
  uint16_t* x;        // [L][T][d] bf16 layer inputs
  float* y;           // [L][T][d] layer outputs
  int32_t* error;     // [L] plan / overflow flags
  hipEvent_t* events; // [L][2] attached to each layer's gate/up launch (its start and end)
  float eps;
};
size_t fused_ws_bytes(int T, int d, int f, int k, int E);
hipError_t launch_fused_step(const moe_layer* layers, int n_layers, float* h, int T, const FusedRecord& rec,
                             void* ws, hipStream_t s);

// Persistent single-token decode step (moe_persist.hip): the whole stack in
// one launch after a set-up launch per 16 layers.  persist_covers says whether
// a stack shape takes it; its workspace is persist_ws_bytes from offset 0.
constexpr int kPsMaxLayers = 128;
bool fused_step_persistent(const moe_layer& L0, int n_layers, int T);
bool persist_covers(const moe_layer& L, int n_layers, int T);
size_t persist_ws_bytes(int d, int f, int E);
hipError_t launch_persist_step(const moe_layer* layers, int n_layers, float* h, const FusedRecord& rec, void* ws,
                               hipStream_t s);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace qre
