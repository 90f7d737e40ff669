// Fused decode step (moe_decode_stack): per layer the glue and router
// (k_fz_glue / k_fz_route), top-k + plan + grouped gate/up (k_fz_gateup), and
// the down pass over the slot table (k_ffn_dq in moe_decode.hip).  The routing
// and the plan are recomputed in each gate/up workgroup's LDS so that no
// launch waits on a separate plan kernel (the "device-planned MoE tail" with
// "grouped kernels", UD-IQ2_XS (L4 fix) page, "What was changed").
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>

#include "moe_dq.h"

namespace qre {

struct FusedPlan {  // plan of the current layer, written by k_fz_gateup's workgroup 0
  int32_t* pair_of_row;  // [T*k] pair t*k + j of each plan row (expert-major, token order)
  int32_t* error;
  int32_t* topk_idx;     // [T][k]
  float* topk_w;         // [T][k]
  SlotEnt* slots;        // [T*k + 1]: shared expert first, then the active experts ascending
  int32_t* n_slots;
};

// (1) Layer input and router.
//
// The residual r_l entering layer l is complete when the layer starts: the
// previous layer's down pass formed its combine, y = o[T*k + t] + sum_j
// topk_w[t][j] * o[t*k + j] (shared row, then the routed slots in order j),
// and wrote r_l = r_{l-1} + y together with each 64-column tile's sum of
// squares.  The glue forms the layer input x = bf16(r_l / sqrt(mean(r_l^2) +
// eps)) from r_l and those tile sums (the first layer sums the squares
// itself), writes x (bf16, and as power-of-two scaled fp16 for the expert
// products) and an optional record of x, and clears the layer's error word
// and down-pass tile counters.
struct FzGlueArgs {
  int d, T;
  const float* r;            // residual entering the layer [T][d]
  const float* ss_part;      // [T][d/64] tile sums of squares of r, or null (first layer)
  uint16_t* x_out;           // bf16 layer input
  uint16_t* rec_x;           // optional record of the same
  f16* x16;
  float* xs;
  int gate_fmt;
  float eps;
  int32_t* error_reset;      // the plan's error word, cleared for this layer
  int32_t* tile_cnt;         // [d/64] down-pass tile counters, cleared for this layer
};

constexpr int kGlueMaxQ = 4;  // d <= 4096: float4 chunks per thread

// Glue for one token, by one workgroup, in two parts so that a caller can put
// other loads in flight between them: glue_load issues the token's residual
// and tile sums; glue_finish forms the bf16 input, which it returns in v[]
// (as floats).
struct GlueLoads {
  f32x4 v[kGlueMaxQ];  // residual
  float ssp;           // tile sum of squares of lane (lanes past the tiles: 0)
};

__device__ __forceinline__ void glue_load(const FzGlueArgs& a, int t, GlueLoads& g) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int d = a.d;
  const int nq = d / 1024;
#pragma unroll
  for (int q = 0; q < kGlueMaxQ; ++q) {
    if (q < nq) g.v[q] = *(const f32x4*)(a.r + (long)t * d + (q * 256 + tid) * 4);
  }
  const int n_ct = d / 64;
  g.ssp = (a.ss_part && lane < n_ct) ? a.ss_part[t * n_ct + lane] : 0.0f;
}

__device__ __forceinline__ void glue_finish(const FzGlueArgs& a, int t, bool writer, GlueLoads& g,
                                            f32x4 (&v)[kGlueMaxQ]) {
  __shared__ float red[2][4];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int d = a.d;
  const int nq = d / 1024;
#pragma unroll
  for (int q = 0; q < kGlueMaxQ; ++q) v[q] = g.v[q];
  float tot;
  if (a.ss_part) {
    tot = wave_sum(g.ssp);  // every wavefront sums the tiles in the same order
  } else {
    float ss = 0.0f;
#pragma unroll
    for (int q = 0; q < kGlueMaxQ; ++q)
      if (q < nq) ss += v[q].x * v[q].x + v[q].y * v[q].y + v[q].z * v[q].z + v[q].w * v[q].w;
    ss = wave_sum(ss);
    if (lane == 0) red[0][wid] = ss;
    __syncthreads();
    tot = red[0][0] + red[0][1] + red[0][2] + red[0][3];
  }
  const float inv = 1.0f / sqrtf(tot / (float)d + a.eps);
  float mx = 0.0f;
#pragma unroll
  for (int q = 0; q < kGlueMaxQ; ++q) {
    if (q < nq) {
      const int i = (q * 256 + tid) * 4;
      const uint32_t p0 = pack_bf16x2(v[q].x * inv, v[q].y * inv);
      const uint32_t p1 = pack_bf16x2(v[q].z * inv, v[q].w * inv);
      v[q] = f32x4{bf16_bits_to_f32(p0 & 0xffffu), bf16_bits_to_f32(p0 >> 16), bf16_bits_to_f32(p1 & 0xffffu),
                   bf16_bits_to_f32(p1 >> 16)};
      if (writer) {
        const u32x2 pk = {p0, p1};
        *(u32x2*)(a.x_out + (long)t * d + i) = pk;
        if (a.rec_x) *(u32x2*)(a.rec_x + (long)t * d + i) = pk;
      }
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[q].x), fabsf(v[q].y)), fmaxf(fabsf(v[q].z), fabsf(v[q].w))));
    }
  }
  if (writer) {
    // fp16 activations (power-of-two scaled) for the expert products
    mx = wave_max(mx);
    if (lane == 0) red[1][wid] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
    const int ex = x16_exponent(mx);
    const float down = ldexpf(1.0f, -ex);
#pragma unroll
    for (int q = 0; q < kGlueMaxQ; ++q) {
      if (q < nq) {
        const int i = (q * 256 + tid) * 4;
        a.x16[(long)t * d + act_pos(a.gate_fmt, i + 0)] = (f16)(v[q].x * down);
        a.x16[(long)t * d + act_pos(a.gate_fmt, i + 1)] = (f16)(v[q].y * down);
        a.x16[(long)t * d + act_pos(a.gate_fmt, i + 2)] = (f16)(v[q].z * down);
        a.x16[(long)t * d + act_pos(a.gate_fmt, i + 3)] = (f16)(v[q].w * down);
      }
    }
    if (tid == 0) a.xs[t] = ldexpf(1.0f, ex);
  }
  __syncthreads();
}

__device__ __forceinline__ void glue_token(const FzGlueArgs& a, int t, bool writer, f32x4 (&v)[kGlueMaxQ]) {
  GlueLoads g;
  glue_load(a, t, g);
  glue_finish(a, t, writer, g, v);
}

// Clears of the layer's error word and down-pass tile counters (block 0).
__device__ __forceinline__ void glue_clear(const FzGlueArgs& a) {
  if (blockIdx.x != 0) return;
  if (threadIdx.x == 0 && a.error_reset) *a.error_reset = 0;
  if (a.tile_cnt && (int)threadIdx.x < a.d / 64) a.tile_cnt[threadIdx.x] = 0;
}

__device__ __forceinline__ void glue_pin_args(const FzGlueArgs& a) {
  pin_arg(a.d);
  pin_arg(a.T);
  pin_arg(a.r);
  pin_arg(a.ss_part);
  pin_arg(a.x_out);
  pin_arg(a.rec_x);
  pin_arg(a.x16);
  pin_arg(a.xs);
  pin_arg(a.gate_fmt);
  pin_arg(a.eps);
  pin_arg(a.error_reset);
  pin_arg(a.tile_cnt);
}

// Glue for T tokens: one workgroup per token.
__global__ __launch_bounds__(256) void k_fz_glue(const FzGlueArgs a) {
  glue_pin_args(a);
  glue_clear(a);
  f32x4 v[kGlueMaxQ];
  glue_token(a, blockIdx.x, true, v);
}

// Router: logits[t][e] for T tokens, one wavefront per expert row, fp64
// accumulation (exact products of fp32 weights and bf16 inputs).  INLINE (a
// single token): every workgroup forms the token's input itself with the glue
// (workgroup 0 writes it out), so the layer needs no separate glue launch.
// Otherwise x is read from the glue kernel's output.
struct FzRouteArgs {
  FzGlueArgs g;
  const float* Wr;
  const float* bias;
  int E;
  const uint16_t* x;  // bf16 [T][d] (not INLINE)
  float* logits;      // [T][E]
};

// Experts per workgroup: one, split over the four wavefronts along d, so
// that the router rows stream through every CU and each wavefront's fp64
// products cover a quarter of the row for every token (two experts per
// workgroup measured 2.4% slower at eight tokens).
template <bool INLINE>
constexpr int route_experts_per_wg() {
  return 1;
}

template <bool INLINE>
__global__ __launch_bounds__(256) void k_fz_route(const FzRouteArgs a) {
  __shared__ uint16_t sx[kFusedMaxT * 4096];  // bf16 layer inputs
  __shared__ double pr[4][kFusedMaxT];        // partial sums of the other wavefronts of an expert
  glue_pin_args(a.g);
  pin_arg(a.Wr);
  pin_arg(a.bias);
  pin_arg(a.E);
  pin_arg(a.x);
  pin_arg(a.logits);
  constexpr int WPE = 4 / route_experts_per_wg<INLINE>();  // wavefronts per expert
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int d = a.g.d, T = a.g.T;
  const int e = blockIdx.x * (4 / WPE) + wid / WPE;
  const int half = wid % WPE;
  const int nj = d / 256;
  const int jlo = half * nj / WPE, jhi = (half + 1) * nj / WPE;

  // INLINE: the glue's loads go first, so that forming the input waits for
  // them alone while the router row streams in
  GlueLoads gl;
  if constexpr (INLINE) glue_load(a.g, 0, gl);
  // router row part of this wave: lane holds elements (j*64 + lane)*4 .. +3
  f32x4 wv[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j >= jlo && j < jhi && e < a.E)
      wv[j] = __builtin_nontemporal_load((const f32x4*)(a.Wr + (long)e * d + (j * 64 + lane) * 4));
  // the bias with the weights, so that the end of the product waits for nothing
  const float bias_e = (a.bias && e < a.E) ? a.bias[e] : 0.0f;

  if constexpr (INLINE) {
    glue_clear(a.g);
    f32x4 v[kGlueMaxQ];
    glue_finish(a.g, 0, blockIdx.x == 0, gl, v);
    const int nq = d / 1024;
#pragma unroll
    for (int q = 0; q < kGlueMaxQ; ++q) {
      if (q < nq) {
        const int i = (q * 256 + tid) * 4;
        const u32x2 pk = {pack_bf16x2(v[q].x, v[q].y), pack_bf16x2(v[q].z, v[q].w)};
        *(u32x2*)&sx[i] = pk;
      }
    }
  } else {
    const int nch = T * d / 8;
    for (int c0 = tid; c0 < nch; c0 += 8 * 256) {
      u32x4 bv[8];
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int c = min(c0 + b * 256, nch - 1);
        bv[b] = *(const u32x4*)(a.x + (long)c * 8);
      }
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int c = c0 + b * 256;
        if (c < nch) {
          const int t = (c * 8) / d, i = (c * 8) % d;
          *(u32x4*)&sx[t * 4096 + i] = bv[b];
        }
      }
    }
  }
  __syncthreads();
  // all tokens' partial sums first, then their wave reductions together
  double r[kFusedMaxT];
  if (e < a.E) {
    double acc[kFusedMaxT];
#pragma unroll
    for (int t = 0; t < kFusedMaxT; ++t) acc[t] = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j >= jlo && j < jhi) {
        const int i = (j * 64 + lane) * 4;
        const double w0 = wv[j].x, w1 = wv[j].y, w2 = wv[j].z, w3 = wv[j].w;
#pragma unroll
        for (int t = 0; t < kFusedMaxT; ++t) {
          if (t < T) {
            const u32x2 xb = *(const u32x2*)&sx[t * 4096 + i];
            acc[t] += w0 * (double)bf16_bits_to_f32(xb.x & 0xffffu) + w1 * (double)bf16_bits_to_f32(xb.x >> 16) +
                      w2 * (double)bf16_bits_to_f32(xb.y & 0xffffu) + w3 * (double)bf16_bits_to_f32(xb.y >> 16);
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kFusedMaxT; ++t)
      if (t < T) r[t] = wave_sum_f64(acc[t]);
  }
  if constexpr (WPE > 1) {
    if (half != 0 && lane == 0 && e < a.E)
      for (int t = 0; t < T; ++t) pr[wid][t] = r[t];
    __syncthreads();
    if (half == 0 && e < a.E)
      for (int q = 1; q < WPE; ++q)
        for (int t = 0; t < T; ++t) r[t] += pr[wid + q][t];
  }
  if (half == 0 && lane == 0 && e < a.E) {
    const double b = (double)bias_e;
    for (int t = 0; t < T; ++t) a.logits[(long)t * a.E + e] = (float)(r[t] + b);
  }
}

// (2) Top-k + plan (in LDS, recomputed by every workgroup that needs it) +
// grouped gate/up.  Slot 0 is the shared expert (it needs no routing, so its
// items start streaming at once); slots 1.. are the active experts in
// ascending id order.  Workgroup 0 publishes the plan for the down pass and
// the next layer's combine.
struct FzGateArgs {
  DecodeArgs a;  // gate/up pass arguments (in16 = x16, in_scale = xs, hf, hmax, error)
  const float* logits;
  int E;
  FusedPlan plan;
};

constexpr int kFusedTK = kFusedMaxT * 32;  // token-slot pairs at most

// Single-tile passes (one N-tile of columns, the batch-1 case) are held to two
// waves per SIMD so that one grid of a decode step is resident at once.
template <int FMT, int NT, int NPL, bool ROLL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NT == 1 ? 2 : 1))) void k_fz_gateup(
    const FzGateArgs g) {
  __shared__ __align__(16) int32_t sidx[kFusedTK];
  __shared__ float sw[kFusedTK];
  __shared__ __align__(16) int32_t sfirst[kFusedTK];
  __shared__ uint32_t tk_key[4][64];  // top-k scratch, one row per wavefront
  __shared__ int32_t tk_idx[4][64];
  __shared__ __align__(16) uint32_t tk_max[32];      // workgroup top-k (one token): group maxima,
  __shared__ __align__(16) uint64_t tk_list[4][64];  // per-wavefront candidate lists,
  __shared__ int32_t tk_cnt[4];                      // and their lengths
  __shared__ int32_t srow_token[kFusedTK];
  __shared__ SlotEnt sslot[kFusedTK];
  extern __shared__ __align__(16) f16 sA[];

  const DecodeArgs& a = g.a;
  dq_pin_args(a);
  pin_arg(g.logits);
  pin_arg(g.plan.pair_of_row);
  pin_arg(g.plan.topk_idx);
  pin_arg(g.plan.topk_w);
  pin_arg(g.plan.slots);
  pin_arg(g.plan.n_slots);
  pin_arg(g.E);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int T = a.T, k = a.k, E = g.E;
  const int TK = T * k;
  const int ksplit = a.ksplit;
  const int rt_per_wg = 4 / ksplit;
  const int rows = a.mat[0].rows;
  const int wg_per_slot = (rows / 16) / rt_per_wg;
  const int hs = a.has_shared;
  const int max_slots = min(E, TK) + hs;
  const int n_items = max_slots * wg_per_slot;
  // The plan is needed by workgroup 0 (which publishes it) and by every
  // workgroup with a routed item; it is built before the item loop so that
  // none of its state stays live during the expert products.
  const int last_item = blockIdx.x + ((n_items - 1 - (int)blockIdx.x) / (int)gridDim.x) * (int)gridDim.x;
  int n_act = 0;
  if (blockIdx.x == 0 || last_item >= hs * wg_per_slot) {
    // ---- every token's logits into LDS (the activation buffer, unused until
    // the item loop) with all loads in flight together
    float* slog = (float*)sA;
    if (((uintptr_t)g.logits & 15) != 0) {
      // (a per-layer record slice that is not 16-byte aligned: scalar loads)
      for (int c0 = tid; c0 < T * E; c0 += 8 * 256) {
        float lv1[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) lv1[b] = g.logits[min(c0 + b * 256, T * E - 1)];
#pragma unroll
        for (int b = 0; b < 8; ++b)
          if (c0 + b * 256 < T * E) slog[c0 + b * 256] = lv1[b];
      }
    } else {
      const int n4 = (T * E) >> 2;
      for (int c0 = tid; c0 < n4; c0 += 8 * 256) {
        f32x4 lv4[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) lv4[b] = *(const f32x4*)(g.logits + 4 * min(c0 + b * 256, n4 - 1));
#pragma unroll
        for (int b = 0; b < 8; ++b)
          if (c0 + b * 256 < n4) *(f32x4*)&slog[4 * (c0 + b * 256)] = lv4[b];
      }
      const int tail = 4 * n4 + tid;
      if (tail < T * E) slog[tail] = g.logits[tail];
    }
    sidx[tid] = 0x7fffffff;  // padding of the pair list
    __syncthreads();
    // ---- top-k per token (one wavefront per token), renormalised weights
    auto topk_token = [&](int t) {
      wave_topk<NPL>(slog + t * E, E, k, lane, tk_key[wid], tk_idx[wid], sidx + t * k, sw + t * k);
      // (the same wavefront reads back what it wrote: its LDS accesses are in order)
      const float v = lane < k ? sw[t * k + lane] : 0.0f;
      const float vmax = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 0));
      const float ex = lane < k ? expf(v - vmax) : 0.0f;
      const float sum = wave_sum(ex);
      if (lane < k) sw[t * k + lane] = ex / sum;
    };
    if (T == 1) {
      // One token: top-k over the whole workgroup, then every wavefront forms
      // the weights and the plan itself (the same values, so no further
      // barrier): the plan is the order of the k distinct experts, row = slot
      // = the number of selected experts with a smaller id.
      wg_topk1<NPL>(slog, E, k, tk_max, tk_list, tk_cnt, tk_key[0], tk_idx[0], sidx, sw);
      const float v = lane < k ? sw[lane] : 0.0f;
      const float vmax = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 0));
      const float ex = lane < k ? expf(v - vmax) : 0.0f;
      const float sum = wave_sum(ex);
      const float w = ex / sum;
      const int e = lane < k ? sidx[lane] : 0x7fffffff;
      int less = 0;
      for (int i0 = 0; i0 < k; i0 += 4) {
        const i32x4 q = *(const i32x4*)&sidx[i0];
#pragma unroll
        for (int u = 0; u < 4; ++u) less += (i0 + u < k && q[u] < e) ? 1 : 0;
      }
      if (lane < k) {
        srow_token[less] = 0;
        sslot[less] = SlotEnt{e, less, 1, 0};
      }
      if (blockIdx.x == 0 && wid == 0) {
        const FusedPlan& P = g.plan;
        if (lane < k) {
          P.pair_of_row[less] = lane;
          P.topk_idx[lane] = e;
          P.topk_w[lane] = w;
          P.slots[hs + less] = SlotEnt{e, less, 1, 0};
        }
        if (lane == 0) {
          if (hs) P.slots[0] = SlotEnt{0, TK, T, 1};
          *P.n_slots = k + hs;
        }
      }
      n_act = k;
    } else {
      for (int t = wid; t < T; t += 4) topk_token(t);
      __syncthreads();
      // ---- plan: pair p (thread p) counts the pairs of smaller experts (its
      // expert's first plan row) and the earlier pairs of its own expert (its
      // rank); the first pair of each expert then counts the distinct smaller
      // experts (its slot).  Rows within an expert follow token order.
      // (the pair lists are padded to a multiple of 4 with an id above every
      // expert, which no count includes, and read four at a time)
      const int TK4 = (TK + 3) & ~3;
      int e = 0, less = 0, before = 0, same = 0;
      if (tid < TK) {
        e = sidx[tid];
  #pragma unroll 4
        for (int q0 = 0; q0 < TK4; q0 += 4) {
          const i32x4 eq = *(const i32x4*)&sidx[q0];
  #pragma unroll
          for (int u = 0; u < 4; ++u) {
            less += eq[u] < e ? 1 : 0;
            same += eq[u] == e ? 1 : 0;
            before += (eq[u] == e && q0 + u < tid) ? 1 : 0;
          }
        }
      }
      sfirst[tid] = (tid < TK && before == 0) ? e : 0x7fffffff;
      __syncthreads();
      if (tid < TK) {
        int dl = 0;
  #pragma unroll 4
        for (int q0 = 0; q0 < TK4; q0 += 4) {
          const i32x4 fq = *(const i32x4*)&sfirst[q0];
  #pragma unroll
          for (int u = 0; u < 4; ++u) dl += fq[u] < e ? 1 : 0;
        }
        srow_token[less + before] = tid / k;
        if (before == 0) sslot[dl] = SlotEnt{e, less, same, 0};
      }
      n_act = __syncthreads_count(tid < TK && before == 0);
      if (blockIdx.x == 0) {
        const FusedPlan& P = g.plan;
        if (tid < TK) {
          P.pair_of_row[less + before] = tid;
          P.topk_idx[tid] = e;
          P.topk_w[tid] = sw[tid];
        }
        for (int s = tid; s < n_act + hs; s += 256) P.slots[s] = s < hs ? SlotEnt{0, TK, T, 1} : sslot[s - hs];
        if (tid == 0) *P.n_slots = n_act + hs;
      }
    }
  }

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int slot = item / wg_per_slot;
    const int tile = (item % wg_per_slot) * rt_per_wg + wid / ksplit;
    SlotInfo si;
    if (slot < hs) {
      si = SlotInfo{0, true, TK, T};
    } else {
      if (slot - hs >= n_act) break;  // items are in slot order
      const SlotEnt se = sslot[slot - hs];
      si = SlotInfo{se.e, false, se.row0, se.cnt};
    }
    dq_item<FMT, NT, true, ROLL>(a, si, tile, wid % ksplit, srow_token, sA);
  }
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------

namespace {

// With timing events, the kernel is launched with them attached (they then
// carry the kernel's own start and end, as a profiler's kernel trace does).
template <int FMT, int NT, int NPL, bool ROLL>
hipError_t launch_fz_gate_npl(const FzGateArgs& g, int items, size_t lds, hipStream_t s, hipEvent_t e0,
                              hipEvent_t e1) {
  const int grid = fused_grid(k_fz_gateup<FMT, NT, NPL, ROLL>, lds, items);
  if (e0)
    hipExtLaunchKernelGGL((k_fz_gateup<FMT, NT, NPL, ROLL>), dim3(grid), dim3(256), (uint32_t)lds, s, e0, e1, 0, g);
  else
    hipLaunchKernelGGL((k_fz_gateup<FMT, NT, NPL, ROLL>), dim3(grid), dim3(256), lds, s, g);
  return hipGetLastError();
}

template <int FMT, int NT, bool ROLL>
hipError_t launch_fz_gate(const FzGateArgs& g, int items, size_t lds, int E, hipStream_t s, hipEvent_t e0,
                          hipEvent_t e1) {
  if (E <= 256) return launch_fz_gate_npl<FMT, NT, 4, ROLL>(g, items, lds, s, e0, e1);
  if (E <= 512) return launch_fz_gate_npl<FMT, NT, 8, ROLL>(g, items, lds, s, e0, e1);
  return launch_fz_gate_npl<FMT, NT, 16, ROLL>(g, items, lds, s, e0, e1);
}

template <int FMT, bool ROLL>
hipError_t launch_fz_gate_nt(const FzGateArgs& g, int nt, int items, size_t lds, int E, hipStream_t s,
                             hipEvent_t e0, hipEvent_t e1) {
  if (nt == 1) return launch_fz_gate<FMT, 1, ROLL>(g, items, lds, E, s, e0, e1);
  if (nt == 2) return launch_fz_gate<FMT, 2, ROLL>(g, items, lds, E, s, e0, e1);
  return launch_fz_gate<FMT, 4, ROLL>(g, items, lds, E, s, e0, e1);
}

template <int FMT>
hipError_t launch_fz_gate_fmt(const FzGateArgs& g, int items, int E, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  constexpr int CPT = cols_per_tile<FMT>();
  const int K = g.a.mat[0].cols;
  const int nt = pick_nt(CPT, g.a.T, K);
  // the activation buffer also holds the logits while the plan is built
  const size_t lds = std::max(dq_lds_bytes(FMT, CPT, nt, K, g.a.ksplit, 2), (size_t)g.a.T * E * 4);
  if (dq_nsteps(FMT, K, g.a.ksplit) > dq_pd(FMT, true))
    return launch_fz_gate_nt<FMT, true>(g, nt, items, lds, E, s, e0, e1);
  return launch_fz_gate_nt<FMT, false>(g, nt, items, lds, E, s, e0, e1);
}

}  // namespace

// ---------------------------------------------------------------- fused step

namespace {

struct FusedWs {
  float* hb[2];
  uint16_t* x;  // bf16 layer input [T][d]
  DecodeWs w;
  float* logits;
  FusedPlan plan;
  float* ss_part;     // [T][d/64] tile sums of squares of the residual
  int32_t* tile_cnt;  // [d/64] down-pass tile counters
};

FusedWs carve_fused(void* ws, int T, int d, int f, int k, int E) {
  const size_t TK = (size_t)T * k;
  char* p = (char*)ws;
  FusedWs F;
  F.hb[0] = (float*)p;
  p += align_up((size_t)T * d * 4, 256);
  F.hb[1] = (float*)p;
  p += align_up((size_t)T * d * 4, 256);
  F.x = (uint16_t*)p;
  p += align_up((size_t)T * d * 2, 256);
  F.w = carve(p, T, d, f, k, 1);
  p += decode_ws_bytes(T, d, f, k, MOE_BF16);
  F.logits = (float*)p;
  p += align_up((size_t)T * E * 4, 256);
  int32_t* ints = (int32_t*)p;
  p += 256;
  F.plan.n_slots = ints;
  F.plan.error = ints + 1;
  F.plan.pair_of_row = (int32_t*)p;
  p += align_up(TK * 4, 256);
  F.plan.topk_idx = (int32_t*)p;
  p += align_up(TK * 4, 256);
  F.plan.topk_w = (float*)p;
  p += align_up(TK * 4, 256);
  F.plan.slots = (SlotEnt*)p;
  p += align_up((TK + 1) * sizeof(SlotEnt), 256);
  F.ss_part = (float*)p;
  p += align_up((size_t)T * (d / 64) * 4, 256);
  F.tile_cnt = (int32_t*)p;
  return F;
}

}  // namespace

size_t fused_ws_bytes(int T, int d, int f, int k, int E) {
  const size_t TK = (size_t)T * k;
  const size_t launches = 2 * align_up((size_t)T * d * 4, 256) + align_up((size_t)T * d * 2, 256) +
                          decode_ws_bytes(T, d, f, k, MOE_BF16) + align_up((size_t)T * E * 4, 256) + 256 +
                          3 * align_up(TK * 4, 256) + align_up((TK + 1) * sizeof(SlotEnt), 256) +
                          align_up((size_t)T * (d / 64) * 4, 256) + align_up((size_t)(d / 64) * 4, 256);
  // a single-token call may take the persistent step, whose layout starts at offset 0 too
  const size_t ps = persist_ws_bytes(d, f, E);
  return launches > ps ? launches : ps;
}

// The persistent single-token step is taken where it covers the shape, unless
// the environment sets QRE_DECODE_LAUNCHES=1 (the per-layer launches, for
// comparison; read at every call).
static bool persist_enabled() {
  const char* v = getenv("QRE_DECODE_LAUNCHES");
  return !(v && v[0] == '1');
}

bool fused_step_persistent(const moe_layer& L0, int n_layers, int T) {
  return persist_enabled() && persist_covers(L0, n_layers, T);
}

hipError_t launch_fused_step(const moe_layer* layers, int n_layers, float* h, int T, const FusedRecord& rec,
                             void* ws, hipStream_t s) {
  const moe_layer& L0 = layers[0];
  if (fused_step_persistent(L0, n_layers, T)) return launch_persist_step(layers, n_layers, h, rec, ws, s);
  const int d = L0.d, f = L0.f, k = L0.k, E = L0.E;
  FusedWs F = carve_fused(ws, T, d, f, k, E);
  const int max_slots = (T * k < E ? T * k : E) + (L0.has_shared ? 1 : 0);
  const bool inline_glue = T == 1;
  for (int l = 0; l < n_layers; ++l) {
    const moe_layer& L = layers[l];
    int32_t* err_word = rec.error ? rec.error + l : F.plan.error;
    // residual entering the layer and leaving it (the down pass forms the latter)
    float* r_in = l == 0 ? h : F.hb[l & 1];
    float* r_out = l == n_layers - 1 ? h : F.hb[(l + 1) & 1];
    // (1) layer input (RMSNorm of the residual) and router
    FzGlueArgs g{};
    g.d = d;
    g.T = T;
    g.r = r_in;
    g.ss_part = l == 0 ? nullptr : F.ss_part;
    g.x_out = F.x;
    g.rec_x = rec.x ? rec.x + (size_t)l * T * d : nullptr;
    g.x16 = F.w.x16;
    g.xs = F.w.xs;
    g.gate_fmt = L.gate.type;
    g.eps = rec.eps;
    g.error_reset = err_word;
    g.tile_cnt = F.tile_cnt;
    FzRouteArgs ra{};
    ra.g = g;
    ra.Wr = L.router_w;
    ra.bias = L.router_bias;
    ra.E = E;
    ra.x = F.x;
    ra.logits = rec.logits ? rec.logits + (size_t)l * T * E : F.logits;
    if (inline_glue) {
      constexpr int epw = route_experts_per_wg<true>();
      hipLaunchKernelGGL(k_fz_route<true>, dim3((E + epw - 1) / epw), dim3(256), 0, s, ra);
    } else {
      constexpr int epw = route_experts_per_wg<false>();
      hipLaunchKernelGGL(k_fz_glue, dim3(T), dim3(256), 0, s, g);
      hipLaunchKernelGGL(k_fz_route<false>, dim3((E + epw - 1) / epw), dim3(256), 0, s, ra);
    }
    // (2) top-k + plan + gate/up
    FzGateArgs ga{};
    ga.a = gateup_args(L, T, 1, F.w);
    ga.a.error = err_word;
    ga.logits = ra.logits;
    ga.E = E;
    ga.plan = F.plan;
    ga.plan.error = err_word;
    if (rec.topk_idx) ga.plan.topk_idx = rec.topk_idx + (size_t)l * T * k;
    if (rec.topk_w) ga.plan.topk_w = rec.topk_w + (size_t)l * T * k;
    {
      const int wg_per_slot = (f / 16) / (4 / ga.a.ksplit);
      const int items = max_slots * wg_per_slot;
      hipEvent_t e0 = rec.events ? rec.events[2 * l] : nullptr, e1 = rec.events ? rec.events[2 * l + 1] : nullptr;
      hipError_t err;
      switch (L.gate.type) {
        case MOE_Q8_0: err = launch_fz_gate_fmt<MOE_Q8_0>(ga, items, E, s, e0, e1); break;
        case MOE_IQ4_NL: err = launch_fz_gate_fmt<MOE_IQ4_NL>(ga, items, E, s, e0, e1); break;
        default: err = launch_fz_gate_fmt<MOE_NVFP4>(ga, items, E, s, e0, e1); break;
      }
      if (err != hipSuccess) return err;
    }
    // (3) down over the slot table, rows written at their pair's position; the
    // last workgroup of each 64-column tile forms the combine and the residual
    {
      DecodeArgs da = down_args(L, T, F.w);
      da.slots = F.plan.slots;
      da.n_slots = F.plan.n_slots;
      da.pair_of_row = F.plan.pair_of_row;
      da.error = err_word;
      da.tile_cnt = F.tile_cnt;
      da.r_in = r_in;
      da.r_out = r_out;
      da.ss_part = F.ss_part;
      da.rec_y = rec.y ? rec.y + (size_t)l * T * d : nullptr;
      da.gate_w = ga.plan.topk_w;
      const int items = max_slots * ((d / 16) / 4);
      const hipError_t err = launch_dq_down_table(da, L.down.type, items, s);
      if (err != hipSuccess) return err;
    }
  }
  return hipGetLastError();
}

}  // namespace qre
