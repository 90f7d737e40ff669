// Persistent decode step for one token (moe_decode_stack at T = 1): every
// layer of the stack in one launch, the analogue of the pages' fused
// "device-planned MoE tail" with its "grouped kernels" (UD-IQ2_XS (L4 fix)
// page, "What was changed"), re-planned for one MI355X.
//
// Each workgroup runs the layer loop.  Per layer its phases are:
//   glue    the layer input x = bf16(r / sqrt(mean(r^2) + eps)) from the
//           residual r (complete once every 64-column tile of the previous
//           layer's combine has landed), kept in LDS as scaled fp16;
//   router  the logit of expert w (workgroup w), from a router row issued
//           before the wait for r;
//   gate/up the shared expert's 16-row tiles (no routing needed), then the
//           top-k over all logits (recomputed in LDS by each workgroup that
//           needs it) and the routed experts' tiles; h = silu(g) * u in fp32;
//   down    64 output rows of one slot (shared or routed pair j), once that
//           slot's h row is complete; h is scaled by a power of two per row
//           into fp16 hi/lo parts for the MFMA;
//   combine the workgroup with a tile's last-slot down item forms
//           y = o_shared + sum_j w_j o_j (slot order), the next residual and
//           its sum of squares, once the tile's down outputs are present.
// Dependencies between workgroups are monotonic counters in the workspace
// (zeroed by the set-up launch before the step): gate/up tiles per slot and
// combined tiles.  The router logits and the o rows carry their own
// readiness: each is stored as one 64-bit word holding the value and the
// layer's tag, and a workgroup that needs them polls the words themselves, so
// the poll that finds the last one present has also read them all (few
// workgroups poll each, so the polls cost little bandwidth).  Increments to
// one address serialise in the memory system (measured: about 40 ns each), so
// each event that many workgroups signal is counted on several sub-counters,
// one 256-byte line each, and a waiting wavefront polls all of them in one
// load instruction.  Waits poll with a bounded count; a wait that runs out
// sets error bit 16 and an abort word that ends every other wait, so the grid
// always drains.  The grid is at most the number of workgroups that fit on
// the device at once, so every workgroup a wait depends on is running.
//
// Other data passed between workgroups (h rows, residual tiles and their
// sums of squares) is written with agent-scope atomic stores and read
// with loads carrying the same cache-coherence bits as agent-scope atomic
// loads (sc1: they bypass the XCDs' private L2 caches; 16-byte buffer loads
// where the data is contiguous); a producer waits for its stores to complete
// (s_waitcnt) before its counter increment, and a consumer issues its loads
// after observing the counter.  Weight codes that do not depend on a wait
// (the next layer's router row and shared-expert tile, a down tile's codes)
// are issued before it.
#include <algorithm>
#include <cstdlib>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "moe_dq.h"

namespace qre {

namespace {

// Matrices of one layer in PsLayer::m
enum { kGate = 0, kUp = 1, kDown = 2, kSGate = 3, kSUp = 4, kSDown = 5 };

constexpr int kPsPD = 6;  // steps of weight codes issued up front per matrix (gate/up; down IQ4_NL / NVFP4)

// Counters, one per 256-byte line.  Events signalled by many workgroups are
// spread over sub-counters: arriver i of an event increments sub-counter
// i % (that event's sub-counter count).
constexpr int kLine = 64;  // int32 per line
constexpr int kMaxSlots = 33;             // k <= 32 routed + shared
constexpr int kSubTiles = 8;              // combined column tiles, by tile
constexpr int kSubSlot = 4;               // gate/up tiles of a slot, by tile
constexpr int kLnTiles = 0;
constexpr int kLnAbort = kLnTiles + kSubTiles;
constexpr int kLnSlot = kLnAbort + 1;                   // kSubSlot lines per slot
constexpr int kNumCnt = kLnSlot + kMaxSlots * kSubSlot;

constexpr uint32_t kSpinMax = 1u << 20;  // polls of one wait before it gives up (the default bound)

}  // namespace

struct PsMat {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* ts;
};

struct PsLayer {
  const float* router_w;
  const float* bias;
  PsMat m[6];
};

constexpr int kPsChunk = 16;  // layer descriptors per set-up launch

struct PsArgs {
  const PsLayer* layers;
  int n_layers, d, f, E, k, hs;
  float eps;
  float* h;            // residual entering the stack, and leaving it
  float* rbuf[2];      // residuals between layers (by parity)
  float* ss[2];        // [d / 64] tile sums of squares of a residual (by parity)
  uint64_t* lgt[2];    // [E] router logits tagged with layer + 1 (by parity; zeroed by the set-up)
  float* hrow;         // [k + hs][f] SwiGLU rows by slot (slot 0 = shared when present)
  uint64_t* otg;       // [k + 1][d] down outputs, tagged (layer + 1): pair j at row j, shared at row k
  int32_t* sync;       // kNumCnt lines of counters
  float* rec_logits;   // optional records (see moe_stack_record)
  int32_t* rec_idx;
  float* rec_w;
  uint16_t* rec_x;
  float* rec_y;
  int32_t* rec_err;
  int32_t* err_ws;     // the error word when there are no per-layer records
  uint32_t spin_max;   // polls of one wait before it gives up
};

__device__ __forceinline__ float ld_ag(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_ag(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every store of the workgroup has completed; then one increment of counter c
// (no value returned, so the workgroup does not wait for it).
__device__ __forceinline__ void ps_arrive(int32_t* c) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A value with its readiness: one 64-bit word, the tag in the high half (no
// tag is 0, so a zeroed word is never ready), stored in one access.
__device__ __forceinline__ void st_tag(uint64_t* p, uint32_t tag, float v) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup-wide poll of tagged words: thread t waits for the words
// p0[i * step] (i < NE, bit i of `pend` set) to carry `tag` and returns their
// values in v; a word already seen is not read again.  Bounded as ps_wait
// (error bit 16 and the abort word when it runs out; gives up when the abort
// word is set).  Returns false when it gave up.  Ends with a barrier.
template <int NE>
__device__ __forceinline__ bool ps_poll(const uint64_t* p0, int step, uint32_t pend, uint32_t tag, float (&v)[NE],
                                        int32_t* abort_w, int32_t* err, uint32_t spin) {
  __shared__ int s_stop[2];
  const int tid = threadIdx.x;
  for (uint32_t n = 1;; ++n) {
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      if ((pend >> i) & 1u) {
        const uint64_t w = __hip_atomic_load(p0 + i * step, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((uint32_t)(w >> 32) == tag) {
          v[i] = __uint_as_float((uint32_t)w);
          pend &= ~(1u << i);
        }
      }
    }
    // (two stop words, by round parity: a word is rewritten only after every
    // thread has passed the barrier that follows the reads of its last value)
    if (tid == 0) {
      int stop = 0;
      if ((n & 15u) == 0u && __hip_atomic_load(abort_w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) stop = 1;
      if (n > spin) {
        atomicOr(err, 16);
        __hip_atomic_store(abort_w, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        stop = 1;
      }
      s_stop[n & 1u] = stop;
    }
    const int np = __syncthreads_count(pend != 0u);
    if (np == 0) return true;
    if (s_stop[n & 1u]) return false;
    __builtin_amdgcn_s_sleep(2);
  }
}

// Wait until an event with narr arrivers per epoch, counted on nsub
// sub-counters (c + i * kLine, arriver j on sub-counter j % nsub), has reached
// `epoch` full rounds.  Wavefront 0 polls every sub-counter in one load
// instruction per round; the others wait at the barrier.  Returns false if the
// wait ran out (error bit 16, abort word set) or another workgroup's did.
__device__ __forceinline__ bool ps_wait(const int32_t* c, int nsub, int narr, int epoch, int32_t* abort_w,
                                        int32_t* err, uint32_t spin) {
  __shared__ int s_ok;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = lane < nsub ? max(0, (narr - lane + nsub - 1) / nsub) : 0;
    const int need = per * epoch;
    const int32_t* cl = c + min(lane, nsub - 1) * kLine;
    int ok = 1;
    uint32_t n = 0;
    while (true) {
      const int v = __hip_atomic_load(cl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__all(lane >= nsub || v >= need)) break;
      if ((n & 15u) == 15u && __hip_atomic_load(abort_w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
        ok = 0;
        break;
      }
      if (++n > spin) {
        if (lane == 0) {
          atomicOr(err, 16);
          __hip_atomic_store(abort_w, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (lane == 0) s_ok = ok;
  }
  __syncthreads();
  return s_ok != 0;
}

// Poll the E tagged logits of one layer until every one carries `tag`; thread
// t reads entries t + 256 i (i < PT) and, as each turns up, writes its value
// to slog.  Entries already seen are not read again.  Bounded like ps_wait;
// returns false if the poll ran out or another workgroup's wait did.  Ends
// with a barrier (slog complete and visible) on success.
template <int PT>
__device__ __forceinline__ bool ps_poll_logits(const uint64_t* lg, int E, uint32_t tag, float* slog,
                                               int32_t* abort_w, int32_t* err, uint32_t spin) {
  __shared__ int s_stop[2];
  const int tid = threadIdx.x;
  uint32_t pend = 0u;
#pragma unroll
  for (int i = 0; i < PT; ++i)
    if (tid + 256 * i < E) pend |= 1u << i;
  for (uint32_t n = 1;; ++n) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      if ((pend >> i) & 1u) {
        const uint64_t v = __hip_atomic_load(lg + tid + 256 * i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((uint32_t)(v >> 32) == tag) {
          slog[tid + 256 * i] = __uint_as_float((uint32_t)v);
          pend &= ~(1u << i);
        }
      }
    }
    // (two stop words, by round parity: a word is rewritten only after every
    // thread has passed the barrier that follows the reads of its last value)
    if (tid == 0) {
      int stop = 0;
      if ((n & 15u) == 0u && __hip_atomic_load(abort_w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) stop = 1;
      if (n > spin) {
        atomicOr(err, 16);
        __hip_atomic_store(abort_w, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        stop = 1;
      }
      s_stop[n & 1u] = stop;
    }
    const int np = __syncthreads_count(pend != 0u);
    if (np == 0) return true;
    if (s_stop[n & 1u]) return false;
    __builtin_amdgcn_s_sleep(2);
  }
}

// Weight loads (codes, scale rows, router rows) of this kernel are plain
// loads.  Unlike the per-layer decode tile, which streams far more bytes per
// launch, this kernel issues each layer's weights in short bursts right after
// a hand-off, and there the non-temporal form measured about 2% slower over
// the whole step (24- and 48-layer single-token stacks alike, so not an
// effect of the repeated steps' bytes staying in a cache).
template <typename T>
__device__ __forceinline__ T ps_ld(const T* p) {
  return *p;
}

// threadIdx.x, recomputed where it is used: values derived from it are then
// formed inside the layer loop instead of being hoisted out of it and held
// in registers for the whole kernel.
__device__ __forceinline__ int ps_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Workgroup LDS of the persistent kernel.
constexpr int kPsMaxD = 4096, kPsMaxF = 1024, kPsMaxE = 1024;
// scale rows of one item: a gate/up tile (16 rows of two matrices, K = d) or
// a down item (64 rows, K = f; Q5_1 records are the largest)
constexpr int kPsScGu = 2 * 16 * scale_row_bytes(MOE_Q8_0, kPsMaxD), kPsScDn = 64 * scale_row_bytes(MOE_Q5_1, kPsMaxF);
constexpr int kPsScBytes = kPsScGu > kPsScDn ? kPsScGu : kPsScDn;
struct PsLds {
  f16 x16[kPsMaxD];                 // layer input, scaled fp16, in the gate/up weights' decode order
  f16 hh[2][kPsMaxF];               // down: h of the slot as scaled fp16 hi / lo parts
  f16 zero[kPsMaxF];                // A-operand rows that hold no column
  uint8_t sc[kPsScBytes];           // scale rows of the current item
  float red[4][2][64];              // K-split partial sums (the token's column)
  float xsum[kPsMaxD / 16];         // sums of x16 over each EPS-element chunk (decode order)
  float hsum[2][kPsMaxF / 16];      // the same for the hi / lo parts of h
  float logit[kPsMaxE];
  float comb[kMaxSlots][64];        // the combine: the tile's down outputs, by o row
  uint32_t tk_key[64];              // top-k candidates
  int32_t tk_idx[64];
  int32_t idx[32];                  // this layer's top-k, slot order
  float wv[32];                     // ... their logits, then their gate weights
  double pr[4];
  float red1[8];
  float xs;
  int ex;
};

// One 16-row tile of the gate and up projections of one expert for the
// single token (x16 in LDS): four wavefronts split K, each lane row n of the
// tile and K slice G of every step; block-diagonal A operand (Q8_0, IQ4_NL)
// or a dense one (NVFP4-style), as in the per-layer decode tile.
// ps_gu_issue puts the tile's weight codes and scale rows in flight (they
// need no activation); ps_gu_compute writes h[tile * 16 + n] =
// silu(g) * u (fp32) of the rows.
template <int FMT>
struct GuCodes {
  u32x4 c[2][kPsPD];  // codes of every step, gate and up
  u32x4 s[2];         // 16-byte chunks of the tile's scale rows, this thread's
  float ts[2];        // NVFP4-style tensor scales
};

template <int FMT>
__device__ __forceinline__ void ps_gu_issue(const PsMat& Wg, const PsMat& Wu, int e, int tile, int K, int rows,
                                            GuCodes<FMT>& g) {
  constexpr int EPS = dq_eps(FMT);
  constexpr int STEP_B = FMT == MOE_Q8_0 ? 4 * EPS : 2 * EPS;  // code bytes per step and row
  const int tid = ps_tid(), lane = tid & 63, wid = tid >> 6;
  const int n = lane & 15, G = lane >> 4;
  const int kw = K / 4;
  const int nsteps = kw / (4 * EPS);
  const int crb = code_row_bytes(FMT, K), srb = scale_row_bytes(FMT, K);
  const int kbase = wid * kw + G * EPS;
  const long rw = (long)e * rows + tile * 16 + n;
  const PsMat* W[2] = {&Wg, &Wu};
  // scale rows first (16 * srb bytes per matrix, contiguous; at most two
  // chunks a thread), then the codes step by step, so that the compute can
  // start on the first steps while the later ones stream in
  const int sch = srb;  // 16-byte chunks per matrix
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int ch = min(tid + 256 * b, 2 * sch - 1);
    const int m = ch >= sch ? 1 : 0;
    g.s[b] = ps_ld(
        (const u32x4*)(W[m]->scales + ((long)e * rows + tile * 16) * srb + (ch - m * sch) * 16));
  }
  const uint8_t* cl[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    cl[m] = W[m]->codes + rw * crb + (FMT == MOE_Q8_0 ? kbase : (kbase >> 1));
    g.ts[m] = FMT == MOE_NVFP4 ? W[m]->ts[e] : 1.0f;
  }
#pragma unroll
  for (int u = 0; u < kPsPD; ++u)
#pragma unroll
    for (int m = 0; m < 2; ++m) g.c[m][u] = ps_ld((const u32x4*)(cl[m] + min(u, nsteps - 1) * STEP_B));
}

// Weights of MFMA i of a step: exact values (NVFP4-style), exact values plus
// 1152 (Q8_0, IQ4_NL; the caller subtracts 1152 times the activation sum), or
// the codes q (Q5_1, whose d and m the caller applies; qh: the high-bit word).
template <int FMT>
__device__ __forceinline__ f16x8 ps_decode(const u32x4& c, int i, uint32_t sraw, uint32_t qh = 0u) {
  if constexpr (FMT == MOE_IQ4_NL) return iq4_dword_to_f16x8_p1152(c[i]);
  else if constexpr (FMT == MOE_Q8_0) return q8_dwords_to_f16x8_p1152(c[2 * i], c[2 * i + 1]);
  else return decode_b<FMT>(c, i, sraw, qh);
}

template <int FMT>
__device__ __forceinline__ void ps_gu_compute(PsLds& S, const GuCodes<FMT>& g, int tile, int K, float* hout,
                                              int32_t* err) {
  constexpr int EPS = dq_eps(FMT);
  constexpr int NMF = EPS / 8;
  constexpr bool BD = FMT != MOE_NVFP4;
  const int tid = ps_tid(), lane = tid & 63, wid = tid >> 6;
  const int n = lane & 15, G = lane >> 4;
  const int kw = K / 4;
  const int nsteps = kw / (4 * EPS);
  const int srb = scale_row_bytes(FMT, K);
  const int kbase = wid * kw + G * EPS;
  const int sch = srb;
  __syncthreads();  // the previous item is done with S.sc and S.red
#pragma unroll
  for (int b = 0; b < 2; ++b)
    if (tid + 256 * b < 2 * sch) *(u32x4*)(S.sc + (tid + 256 * b) * 16) = g.s[b];
  __syncthreads();
  const bool valid = BD ? (n == 4 * G) : (n == 0);  // A rows holding the token's column
  const f16* ap = valid ? S.x16 + kbase : S.zero;
  const uint16_t* ssl[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) ssl[m] = (const uint16_t*)(S.sc + m * sch * 16 + n * srb) + (kbase >> 5);
  // the token's column is D row 0 (element x): with the block-diagonal
  // operand, lane (n, G) holds row n's partial sum over the step's chunk of
  // lane group G
  float acc[2] = {0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kPsPD; ++s) {
    if (s < nsteps) {
      f16x8 ac[NMF];
#pragma unroll
      for (int i = 0; i < NMF; ++i) ac[i] = *(const f16x8*)(ap + s * 4 * EPS + 8 * i);
      const float csum = BD ? 1152.0f * S.xsum[(kbase >> (EPS == 32 ? 5 : 4)) + 4 * s] : 0.0f;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint32_t ss = ssl[m][s * (4 * EPS / 32)];
        f32x4 D = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NMF; ++i)
          D = __builtin_amdgcn_mfma_f32_16x16x32_f16(ac[i], ps_decode<FMT>(g.c[m][s], i, ss), D, 0, 0, 0);
        if constexpr (FMT == MOE_NVFP4) {
          acc[m] += D.x;
        } else {
          acc[m] = fmaf(f16_bits_to_f32(ss), D.x - csum, acc[m]);
        }
      }
    }
    // one step's decoded weights at a time (the codes of every step are
    // already in registers; decoding ahead would only hold more registers)
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (BD) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      acc[m] += __shfl_xor(acc[m], 16, 64);
      acc[m] += __shfl_xor(acc[m], 32, 64);
    }
  }
  S.red[wid][0][lane] = acc[0];
  S.red[wid][1][lane] = acc[1];
  __syncthreads();
  if (wid == 0 && G == 0) {
    float gs = 0.f, us = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      gs += S.red[q][0][lane];
      us += S.red[q][1][lane];
    }
    const float xs = S.xs;
    gs = gs * g.ts[0] * xs;
    us = us * g.ts[1] * xs;
    const float hv = silu_f(gs) * us;
    if (!(fabsf(hv) <= 3.0e38f)) atomicOr(err, 2);
    st_ag(hout + tile * 16 + n, hv);
  }
}

// 64 output rows [ct * 64, ct * 64 + 64) of the down projection of one
// expert for the single token: h (staged in S.hh as hi / lo fp16 parts of
// h * 2^-ex) is the A operand's two columns; each wavefront 16 rows over all
// of K = f.  ps_dn_issue puts the codes and scale rows in flight;
// ps_dn_compute writes o = (hi + lo) * 2^ex of the rows.
// 16-byte chunks of the item's scale rows per thread (Q5_1: up to 64 rows x
// f / 32 records of 8 bytes)
constexpr int ps_dn_sch(int fmt) { return fmt == MOE_Q5_1 ? 4 : 1; }

template <int FMT>
struct DnCodes {
  u32x4 c[FMT == MOE_Q8_0 ? 2 * kPsPD : kPsPD];
  u32x4 s[ps_dn_sch(FMT)];
  float ts;
};

template <int FMT>
__device__ __forceinline__ void ps_dn_issue(const PsMat& Wd, int e, int ct, int K, int rows, DnCodes<FMT>& g) {
  constexpr int EPS = dq_eps(FMT);
  constexpr int PD = FMT == MOE_Q8_0 ? 2 * kPsPD : kPsPD;
  constexpr int STEP_B = FMT == MOE_Q8_0 ? 4 * EPS : 2 * EPS;
  const int tid = ps_tid(), lane = tid & 63, wid = tid >> 6;
  const int n = lane & 15, G = lane >> 4;
  const int nsteps = K / (4 * EPS);
  const int crb = code_row_bytes(FMT, K), srb = scale_row_bytes(FMT, K);
  const int kbase = G * EPS;
  const int row = ct * 64 + wid * 16 + n;
  const uint8_t* cl = Wd.codes + ((long)e * rows + row) * crb + (FMT == MOE_Q8_0 ? kbase : (kbase >> 1));
  const int sch = 64 * srb / 16;  // at most 256 * ps_dn_sch (issued first)
  const uint8_t* sbase = Wd.scales + ((long)e * rows + ct * 64) * srb;
#pragma unroll
  for (int j = 0; j < ps_dn_sch(FMT); ++j)
    g.s[j] = ps_ld((const u32x4*)(sbase + min(tid + 256 * j, sch - 1) * 16));
#pragma unroll
  for (int u = 0; u < PD; ++u) g.c[u] = ps_ld((const u32x4*)(cl + min(u, nsteps - 1) * STEP_B));
  g.ts = FMT == MOE_NVFP4 ? Wd.ts[e] : 1.0f;
}

template <int FMT>
__device__ __forceinline__ void ps_dn_compute(PsLds& S, const DnCodes<FMT>& g, int ct, int K, float hscale,
                                              uint64_t* oout, uint32_t tag) {
  constexpr int EPS = dq_eps(FMT);
  constexpr int NMF = EPS / 8;
  constexpr bool BD = FMT != MOE_NVFP4;
  constexpr int PD = FMT == MOE_Q8_0 ? 2 * kPsPD : kPsPD;
  const int tid = ps_tid(), lane = tid & 63, wid = tid >> 6;
  const int n = lane & 15, G = lane >> 4;
  const int nsteps = K / (4 * EPS);
  const int srb = scale_row_bytes(FMT, K);
  const int kbase = G * EPS;
  const int row = ct * 64 + wid * 16 + n;
  const int sch = 64 * srb / 16;
  // (S.sc is free: the caller's barrier after staging h)
#pragma unroll
  for (int j = 0; j < ps_dn_sch(FMT); ++j)
    if (tid + 256 * j < sch) *(u32x4*)(S.sc + (tid + 256 * j) * 16) = g.s[j];
  __syncthreads();
  // columns: hi (0) and lo (1)
  int c;
  bool valid;
  if constexpr (BD) {
    valid = (n >> 2) == G && (n & 3) < 2;
    c = n & 3;
  } else {
    valid = n < 2;
    c = n;
  }
  const f16* ap = valid ? S.hh[c] + kbase : S.zero;
  constexpr int SW = FMT == MOE_Q5_1 ? 4 : 1;  // 16-bit words per scale record
  const uint16_t* ssl = (const uint16_t*)(S.sc + (wid * 16 + n) * srb) + (kbase >> 5) * SW;
  // D rows 0 and 1 hold the hi and lo columns (elements x and y)
  f32x2 acc = {0.f, 0.f};
#pragma unroll
  for (int s = 0; s < PD; ++s) {
    if (s < nsteps) {
      uint32_t ss, qh = 0u;
      if constexpr (FMT == MOE_Q5_1) {
        const u32x2 rec = *(const u32x2*)(ssl + s * (4 * EPS / 32) * SW);
        ss = rec.x;
        qh = rec.y;
      } else {
        ss = ssl[s * (4 * EPS / 32)];
      }
      f32x4 D = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NMF; ++i) {
        const f16x8 a8 = *(const f16x8*)(ap + s * 4 * EPS + 8 * i);
        D = __builtin_amdgcn_mfma_f32_16x16x32_f16(a8, ps_decode<FMT>(g.c[s], i, ss, qh), D, 0, 0, 0);
      }
      if constexpr (FMT == MOE_NVFP4) {
        acc.x += D.x;
        acc.y += D.y;
      } else if constexpr (FMT == MOE_Q5_1) {
        // w = d q + m: d times the code product plus m times the chunk's activation sum
        const int chunk = (kbase >> 5) + 4 * s;
        const float dd = f16_bits_to_f32(ss & 0xffffu), mm = f16_bits_to_f32(ss >> 16);
        acc.x = fmaf(dd, D.x, fmaf(mm, S.hsum[0][chunk], acc.x));
        acc.y = fmaf(dd, D.y, fmaf(mm, S.hsum[1][chunk], acc.y));
      } else {
        const int chunk = (kbase >> (EPS == 32 ? 5 : 4)) + 4 * s;
        const float sc = f16_bits_to_f32(ss);
        acc.x = fmaf(sc, fmaf(-1152.0f, S.hsum[0][chunk], D.x), acc.x);
        acc.y = fmaf(sc, fmaf(-1152.0f, S.hsum[1][chunk], D.y), acc.y);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (BD) {
    acc.x += __shfl_xor(acc.x, 16, 64);
    acc.y += __shfl_xor(acc.y, 16, 64);
    acc.x += __shfl_xor(acc.x, 32, 64);
    acc.y += __shfl_xor(acc.y, 32, 64);
  }
  // D rows 0 and 1 (the hi and lo columns) of lanes n in group 0
  if (G == 0) st_tag(oout + row, tag, (acc.x * g.ts + acc.y * g.ts) * hscale);
}

// Glue of one token: x = bf16(r / sqrt(sum(r^2) / d + eps)), with the sum of
// squares from the previous layer's tile sums (or from r itself for the first
// layer).  Thread tid holds elements (q * 256 + tid) * 4 .. + 3 for q < d /
// 1024 (as floats of the bf16 values, for the router); writes the scaled fp16
// copy (gate weights' decode order) and its scale to LDS, and the bf16 record.
// Sum of v over aligned groups of LPC (4 or 8) consecutive lanes, in the
// group's last lane (row shifts within rows of 16 lanes).
template <int LPC>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_f32<kDppShr1, 0xf>(v);
  v += dpp_f32<kDppShr2, 0xf>(v);
  if constexpr (LPC == 8) v += dpp_f32<kDppShr4, 0xf>(v);
  return v;
}

__device__ __forceinline__ void ps_glue_x(PsLds& S, const float* r, const float* ssp, int d, float eps,
                                          uint16_t* rec_x, f32x4 (&xv)[4]) {
  const int tid = ps_tid(), lane = tid & 63, wid = tid >> 6;
  const int nq = d / 1024;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (q < nq) xv[q] = ld_ag4(r, (q * 256 + tid) * 16);
  float tot;
  if (ssp) {
    const float v = lane < d / 64 ? ld_ag(ssp + lane) : 0.0f;
    tot = wave_sum(v);  // every wavefront sums the tiles in the same order
  } else {
    float ss = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q < nq) ss += xv[q].x * xv[q].x + xv[q].y * xv[q].y + xv[q].z * xv[q].z + xv[q].w * xv[q].w;
    ss = wave_sum(ss);
    if (lane == 0) S.red1[wid] = ss;
    __syncthreads();
    tot = S.red1[0] + S.red1[1] + S.red1[2] + S.red1[3];
  }
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (q < nq) {
      const uint32_t p0 = pack_bf16x2(xv[q].x * inv, xv[q].y * inv);
      const uint32_t p1 = pack_bf16x2(xv[q].z * inv, xv[q].w * inv);
      xv[q] = f32x4{bf16_bits_to_f32(p0 & 0xffffu), bf16_bits_to_f32(p0 >> 16), bf16_bits_to_f32(p1 & 0xffffu),
                    bf16_bits_to_f32(p1 >> 16)};
      if (rec_x) *(u32x2*)(rec_x + (q * 256 + tid) * 4) = u32x2{p0, p1};
    }
  }
}

// The second half of the glue: x (as produced by ps_glue_x) as scaled fp16 in
// LDS, in the gate weights' decode order, with its scale and chunk sums.
template <int GF>
__device__ __forceinline__ void ps_glue_stage(PsLds& S, const f32x4 (&xv)[4], int d) {
  const int tid = ps_tid(), lane = tid & 63, wid = tid >> 6;
  const int nq = d / 1024;
  float mx = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (q < nq) mx = fmaxf(mx, fmaxf(fmaxf(fabsf(xv[q].x), fabsf(xv[q].y)), fmaxf(fabsf(xv[q].z), fabsf(xv[q].w))));
  mx = wave_max(mx);
  if (lane == 0) S.red1[4 + wid] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(S.red1[4], S.red1[5]), fmaxf(S.red1[6], S.red1[7]));
  const int ex = x16_exponent(mx);
  const float down = ldexpf(1.0f, -ex);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (q < nq) {
      const int i = (q * 256 + tid) * 4;
      f16 hv[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        hv[c] = (f16)(xv[q][c] * down);
        S.x16[act_pos(GF, i + c)] = hv[c];
      }
      if constexpr (GF != MOE_NVFP4) {
        // sum over each EPS-element chunk of the stored values (the weights
        // carry +1152, see ps_decode)
        constexpr int EPS = dq_eps(GF);
        const float cs = group_sum<EPS / 4>(((float)hv[0] + (float)hv[1]) + ((float)hv[2] + (float)hv[3]));
        if ((lane & (EPS / 4 - 1)) == EPS / 4 - 1) S.xsum[i / EPS] = cs;
      }
    }
  }
  if (tid == 0) S.xs = ldexpf(1.0f, ex);
  __syncthreads();
}

// Router row of expert e, the part this thread multiplies: elements
// (q * 256 + tid) * 4 .. + 3 (the glue's), one 16-byte load per q.
__device__ __forceinline__ void ps_router_load(const float* Wr, int e, int d, f32x4 (&wv)[4]) {
  const int nq = d / 1024;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (q < nq) wv[q] = ps_ld((const f32x4*)(Wr + (long)e * d + (q * 256 + ps_tid()) * 4));
}

// logit = fp32(sum_i W[e][i] x[i] + b[e]) with fp64 sums of the exact products.
__device__ __forceinline__ float ps_router_dot(PsLds& S, const f32x4 (&wv)[4], const f32x4 (&xv)[4], int d,
                                               float bias) {
  const int lane = ps_tid() & 63, wid = ps_tid() >> 6;
  const int nq = d / 1024;
  double acc = 0.0;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (q < nq)
      acc += (double)wv[q].x * (double)xv[q].x + (double)wv[q].y * (double)xv[q].y +
             (double)wv[q].z * (double)xv[q].z + (double)wv[q].w * (double)xv[q].w;
  acc = wave_sum_f64(acc);
  if (lane == 0) S.pr[wid] = acc;
  __syncthreads();
  const double r = ((S.pr[0] + S.pr[1]) + S.pr[2]) + S.pr[3];
  __syncthreads();  // S.pr may be reused
  return (float)(r + (double)bias);
}

// The combine of column tile ct (64 columns) of layer l: the nR = k + hs down
// outputs of every column (thread (q, c) polls o rows q, q + 4, ... of column
// c), then y = o_shared + sum_j w_j o_j (slot order), the new residual and
// the tile's sum of squares.  Returns false if the poll gave up.
__device__ __forceinline__ bool ps_combine(PsLds& S, const PsArgs& a, int l, int ct, const float* r_in, float* r_out,
                                           int32_t* abort_w, int32_t* err) {
  const int tid = ps_tid(), c = tid & 63, q = tid >> 6;
  const int d = a.d, k = a.k, nR = a.k + a.hs;
  constexpr int NE = (kMaxSlots + 3) / 4;
  uint32_t pend = 0u;
#pragma unroll
  for (int i = 0; i < NE; ++i)
    if (q + 4 * i < nR) pend |= 1u << i;
  float v[NE];
  if (!ps_poll<NE>(a.otg + (long)q * d + ct * 64 + c, 4 * d, pend, (uint32_t)(l + 1), v, abort_w, err, a.spin_max))
    return false;
#pragma unroll
  for (int i = 0; i < NE; ++i)
    if (q + 4 * i < nR) S.comb[q + 4 * i][c] = v[i];
  __syncthreads();
  if (q == 0) {
    const int col = ct * 64 + c;
    float y = a.hs ? S.comb[k][c] : 0.0f;
    for (int j = 0; j < k; ++j) y = fmaf(S.wv[j], S.comb[j][c], y);
    const float rn = ld_ag(r_in + col) + y;
    st_ag(r_out + col, rn);
    if (a.rec_y) a.rec_y[(long)l * d + col] = y;
    const float ss = wave_sum(rn * rn);
    if (c == 0) st_ag(a.ss[(l + 1) & 1] + ct, ss);
  }
  return true;
}

template <int GF, int DF, int PT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_ps_decode(const PsArgs a) {
  __shared__ PsLds S;
  pin_arg(a.layers);
  pin_arg(a.h);
  pin_arg(a.hrow);
  pin_arg(a.otg);
  pin_arg(a.sync);
  const int G = gridDim.x, w = blockIdx.x;
  const int d = a.d, f = a.f, E = a.E, k = a.k, hs = a.hs, L = a.n_layers;
  const int nS = k + hs;
  const int gu_per = f / 16, dn_per = d / 64;
  const int gu_total = nS * gu_per, dn_total = nS * dn_per;
  const bool has_gu = w < gu_total;
  const bool has_x = w < E || has_gu;
  const bool has_routed_gu = [&] {
    for (int it = w; it < gu_total; it += G)
      if (it / gu_per >= hs) return true;
    return false;
  }();
  const bool needs_topk = w == 0 || has_routed_gu || w < dn_total;
  // this workgroup's first gate/up item is a shared-expert tile (tile w): its
  // codes are issued before the wait for each layer's input
  const bool pre_sh = hs && w < gu_per;
  int32_t* sync = a.sync;
  int32_t* abort_w = sync + kLnAbort * kLine;

  for (int i = ps_tid(); i < kPsMaxF; i += 256) S.zero[i] = (f16)0.0f;

  f32x4 wv[4];
  if (w < E) ps_router_load(a.layers[0].router_w, w, d, wv);
  GuCodes<GF> gsh;
  if (pre_sh) ps_gu_issue<GF>(a.layers[0].m[kSGate], a.layers[0].m[kSUp], 0, w, d, f, gsh);

  for (int l = 0; l < L; ++l) {
    const int tid = ps_tid(), lane = tid & 63, wid = tid >> 6;
    const PsLayer& P = a.layers[l];
    int32_t* err = a.rec_err ? a.rec_err + l : a.err_ws;
    const float* r_in = l == 0 ? a.h : a.rbuf[l & 1];
    float* r_out = l == L - 1 ? a.h : a.rbuf[(l + 1) & 1];
    uint64_t* lg = a.lgt[l & 1];
    const uint32_t ltag = (uint32_t)(l + 1);

    // ---- glue and router (the logits first: they gate every routed item)
    if (has_x) {
      if (l > 0 && !ps_wait(sync + kLnTiles * kLine, kSubTiles, dn_per, l, abort_w, err, a.spin_max)) return;
      f32x4 xv[4];
      ps_glue_x(S, r_in, l == 0 ? nullptr : a.ss[l & 1], d, a.eps,
                (w == 0 && a.rec_x) ? a.rec_x + (long)l * d : nullptr, xv);
      for (int e = w; e < E; e += G) {
        if (e != w) ps_router_load(P.router_w, e, d, wv);  // (the first row is already in flight)
        const float bias = P.bias ? P.bias[e] : 0.0f;
        const float v = ps_router_dot(S, wv, xv, d, bias);
        if (tid == 0) {
          __hip_atomic_store(lg + e, ((uint64_t)ltag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
          if (a.rec_logits) a.rec_logits[(long)l * E + e] = v;
        }
      }
      if (has_gu) ps_glue_stage<GF>(S, xv, d);
    }

    // ---- gate/up of the shared expert (slot 0), which needs no routing
    for (int it = w; it < gu_total && it / gu_per < hs; it += G) {
      if (!(it == w && pre_sh)) ps_gu_issue<GF>(P.m[kSGate], P.m[kSUp], 0, it % gu_per, d, f, gsh);
      ps_gu_compute<GF>(S, gsh, it % gu_per, d, a.hrow, err);
      ps_arrive(sync + (kLnSlot + (it % gu_per) % kSubSlot) * kLine);
    }

    // ---- top-k and gate weights (every workgroup that needs them)
    if (needs_topk) {
      if (!ps_poll_logits<PT>(lg, E, ltag, S.logit, abort_w, err, a.spin_max)) return;
      // one wavefront selects (no barrier until the result is published)
      if (wid == 0) {
        wave_topk<PT * 4>(S.logit, E, k, lane, S.tk_key, S.tk_idx, S.idx, S.wv);
        const float v = lane < k ? S.wv[lane] : 0.0f;
        const float vmax = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 0));
        const float ex = lane < k ? expf(v - vmax) : 0.0f;
        const float sum = wave_sum(ex);
        if (lane < k) {
          S.wv[lane] = ex / sum;
          if (w == 0 && a.rec_idx) a.rec_idx[(long)l * k + lane] = S.idx[lane];
          if (w == 0 && a.rec_w) a.rec_w[(long)l * k + lane] = ex / sum;
        }
      }
      __syncthreads();
    }

    // ---- gate/up of the routed experts: slot hs + j holds pair j
    for (int it = w; it < gu_total; it += G) {
      const int slot = it / gu_per;
      if (slot < hs) continue;
      GuCodes<GF> g;
      ps_gu_issue<GF>(P.m[kGate], P.m[kUp], S.idx[slot - hs], it % gu_per, d, f, g);
      ps_gu_compute<GF>(S, g, it % gu_per, d, a.hrow + (long)slot * f, err);
      ps_arrive(sync + (kLnSlot + slot * kSubSlot + (it % gu_per) % kSubSlot) * kLine);
    }

    // the next layer's router row, in flight from here on (a workgroup that
    // issued it after its down work would wait for it at the next router)
    if (l + 1 < L && w < E) ps_router_load(a.layers[l + 1].router_w, w, d, wv);

    // ---- down, and the combine of each finished 64-column tile
    for (int it = w; it < dn_total; it += G) {
      const int slot = it / dn_per, ct = it % dn_per;
      const bool sh = slot < hs;
      DnCodes<DF> g;
      ps_dn_issue<DF>(sh ? P.m[kSDown] : P.m[kDown], sh ? 0 : S.idx[slot - hs], ct, f, d, g);
      if (!ps_wait(sync + (kLnSlot + slot * kSubSlot) * kLine, kSubSlot, gu_per, l + 1, abort_w, err, a.spin_max)) return;
      // the slot's h row, scaled by a power of two into fp16 hi / lo parts
      const float* hr = a.hrow + (long)slot * f;
      const f32x4 hv = tid * 4 < f ? ld_ag4(hr, tid * 16) : f32x4{0.f, 0.f, 0.f, 0.f};
      float mx = fmaxf(fmaxf(fabsf(hv.x), fabsf(hv.y)), fmaxf(fabsf(hv.z), fabsf(hv.w)));
      mx = wave_max(mx);
      __syncthreads();  // the previous item is done with S.hh, S.sc and S.red1
      if (lane == 0) S.red1[wid] = mx;
      __syncthreads();
      mx = fmaxf(fmaxf(S.red1[0], S.red1[1]), fmaxf(S.red1[2], S.red1[3]));
      const int ex = x16_exponent(mx);
      const float down = ldexpf(1.0f, -ex);
      if (tid * 4 < f) {
        float shi = 0.f, slo = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float sv = hv[c] * down;
          const f16 hi = (f16)sv;
          const f16 lo = (f16)(sv - (float)hi);
          const int pos = act_pos(DF, tid * 4 + c);
          S.hh[0][pos] = hi;
          S.hh[1][pos] = lo;
          shi += (float)hi;
          slo += (float)lo;
        }
        if constexpr (DF != MOE_NVFP4) {
          // chunk sums of the stored parts (Q8_0 / IQ4_NL: the weights carry
          // +1152; Q5_1: the block offset m multiplies them)
          constexpr int EPS = dq_eps(DF);
          shi = group_sum<EPS / 4>(shi);
          slo = group_sum<EPS / 4>(slo);
          if ((lane & (EPS / 4 - 1)) == EPS / 4 - 1) {
            S.hsum[0][tid * 4 / EPS] = shi;
            S.hsum[1][tid * 4 / EPS] = slo;
          }
        }
      }
      const int pair = sh ? k : slot - hs;
      ps_dn_compute<DF>(S, g, ct, f, ldexpf(1.0f, ex), a.otg + (long)pair * d, (uint32_t)(l + 1));
      // the workgroup with the tile's last-slot item combines the tile once
      // the tile's nS down outputs are present
      if (slot == nS - 1) {
        if (!ps_combine(S, a, l, ct, r_in, r_out, abort_w, err)) return;
        ps_arrive(sync + (kLnTiles + ct % kSubTiles) * kLine);
      }
    }

    // ---- the next layer's shared-expert tile, in flight while the residual forms
    if (l + 1 < L && pre_sh) ps_gu_issue<GF>(a.layers[l + 1].m[kSGate], a.layers[l + 1].m[kSUp], 0, w, d, f, gsh);
  }
}

// Set-up launch: the layer descriptors of one chunk into the workspace table;
// the first chunk also clears the counters and the error words.
struct PsSetupArgs {
  PsLayer L[kPsChunk];
  int l0, count;
  PsLayer* table;
  int32_t* sync;
  int32_t* rec_err;
  int n_layers;
  int32_t* err_ws;
  uint64_t* tags;  // every tagged word of the step (logits, o rows), contiguous
  int n_tags;
};

// One workgroup, or for the first chunk enough to zero the tagged words (no
// tag is 0, so a zeroed word reads as not yet written).
__global__ __launch_bounds__(256) void k_ps_setup(const PsSetupArgs s) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && tid < s.count) s.table[s.l0 + tid] = s.L[tid];
  if (s.l0 == 0 && blockIdx.x > 0) {
    for (long i = (long)(blockIdx.x - 1) * 256 + tid; i < s.n_tags; i += (long)(gridDim.x - 1) * 256) s.tags[i] = 0ull;
  }
  if (s.l0 == 0 && blockIdx.x == 0) {
    for (int i = tid; i < kNumCnt * kLine; i += 256) s.sync[i] = 0;  // (all counter lines)
    if (s.rec_err)
      for (int i = tid; i < s.n_layers; i += 256) s.rec_err[i] = 0;
    if (tid == 0) *s.err_ws = 0;
  }
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------

namespace {

struct PsWs {
  PsLayer* table;
  int32_t* sync;
  int32_t* err_ws;
  float* rbuf[2];
  float* ss[2];
  uint64_t* lgt[2];
  float* hrow;
  uint64_t* tags;  // lgt[0], lgt[1], otg: contiguous
  int n_tags;
  uint64_t* otg;
};

PsWs carve_ps(void* ws, int d, int f, int E, int k) {
  char* p = (char*)ws;
  PsWs W;
  W.table = (PsLayer*)p;
  p += align_up((size_t)kPsMaxLayers * sizeof(PsLayer), 256);
  W.sync = (int32_t*)p;
  p += align_up((size_t)kNumCnt * kLine * 4, 256);
  W.err_ws = (int32_t*)p;
  p += 256;
  for (int i = 0; i < 2; ++i) {
    W.rbuf[i] = (float*)p;
    p += align_up((size_t)d * 4, 256);
    W.ss[i] = (float*)p;
    p += align_up((size_t)(d / 64) * 4, 256);
  }
  W.hrow = (float*)p;
  p += align_up((size_t)kMaxSlots * f * 4, 256);
  // the tagged words, contiguous (the set-up zeroes them): the two logit
  // arrays, then the o rows
  W.tags = (uint64_t*)p;
  W.lgt[0] = W.tags;
  W.lgt[1] = W.lgt[0] + E;
  W.otg = W.lgt[1] + E;
  W.n_tags = 2 * E + (k + 1) * d;
  return W;
}

PsMat ps_mat(const moe_qmatrix& m) { return PsMat{(const uint8_t*)m.codes, (const uint8_t*)m.scales, m.tensor_scale}; }

// The grid is at most the workgroups resident at once, so that every
// workgroup a wait depends on is running.  With timing events, the launch
// carries them (its own start and end).
template <int GF, int DF, int PT>
hipError_t launch_ps_pt(const PsArgs& a, int need, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  auto kern = k_ps_decode<GF, DF, PT>;
  const int res = resident_wgs(kern, 0);
  if (res <= 0) return hipErrorInvalidConfiguration;
  const int grid = need < res ? need : res;
  if (e0)
    hipExtLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, s, e0, e1, 0, a);
  else
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

// logits per top-k thread: E <= 512 takes two, E <= 1024 four
template <int GF, int DF>
hipError_t launch_ps(const PsArgs& a, int need, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return a.E <= 512 ? launch_ps_pt<GF, DF, 2>(a, need, s, e0, e1) : launch_ps_pt<GF, DF, 4>(a, need, s, e0, e1);
}

template <int GF>
hipError_t launch_ps_d(int df, const PsArgs& a, int need, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (df) {
    case MOE_Q8_0: return launch_ps<GF, MOE_Q8_0>(a, need, s, e0, e1);
    case MOE_IQ4_NL: return launch_ps<GF, MOE_IQ4_NL>(a, need, s, e0, e1);
    case MOE_Q5_1: return launch_ps<GF, MOE_Q5_1>(a, need, s, e0, e1);
    default: return launch_ps<GF, MOE_NVFP4>(a, need, s, e0, e1);
  }
}

}  // namespace

size_t persist_ws_bytes(int d, int f, int E) {
  return align_up((size_t)kPsMaxLayers * sizeof(PsLayer), 256) + align_up((size_t)kNumCnt * kLine * 4, 256) + 256 +
         2 * (align_up((size_t)d * 4, 256) + align_up((size_t)(d / 64) * 4, 256)) +
         align_up((size_t)kMaxSlots * f * 4, 256) + ((size_t)2 * E + (size_t)kMaxSlots * d) * 8;
}

bool persist_covers(const moe_layer& L, int n_layers, int T) {
  if (T != 1 || n_layers > kPsMaxLayers) return false;
  if (L.d % 1024 != 0 || L.d > kPsMaxD || L.E > kPsMaxE || L.k > 32) return false;
  if (L.f % 128 != 0 || L.f > kPsMaxF) return false;
  // every step's codes issued up front: gate/up K / 4, down K = f
  const int eg = dq_eps(L.gate.type), ed = dq_eps(L.down.type);
  if (L.d / 4 / (4 * eg) > kPsPD) return false;
  if (L.f / (4 * ed) > (L.down.type == MOE_Q8_0 ? 2 * kPsPD : kPsPD)) return false;
  return true;
}

hipError_t launch_persist_step(const moe_layer* layers, int n_layers, float* h, const FusedRecord& rec, void* ws,
                               hipStream_t s) {
  const moe_layer& L0 = layers[0];
  PsWs W = carve_ps(ws, L0.d, L0.f, L0.E, L0.k);
  for (int l0 = 0; l0 < n_layers; l0 += kPsChunk) {
    PsSetupArgs sa{};
    sa.l0 = l0;
    sa.count = n_layers - l0 < kPsChunk ? n_layers - l0 : kPsChunk;
    for (int i = 0; i < sa.count; ++i) {
      const moe_layer& L = layers[l0 + i];
      PsLayer& P = sa.L[i];
      P.router_w = L.router_w;
      P.bias = L.router_bias;
      P.m[kGate] = ps_mat(L.gate);
      P.m[kUp] = ps_mat(L.up);
      P.m[kDown] = ps_mat(L.down);
      if (L.has_shared) {
        P.m[kSGate] = ps_mat(L.shared_gate);
        P.m[kSUp] = ps_mat(L.shared_up);
        P.m[kSDown] = ps_mat(L.shared_down);
      }
    }
    sa.table = W.table;
    sa.sync = W.sync;
    sa.rec_err = rec.error;
    sa.n_layers = n_layers;
    sa.err_ws = W.err_ws;
    sa.tags = W.tags;
    sa.n_tags = W.n_tags;
    // the first chunk: workgroup 0 and at least one more for the tagged words
    const int blocks = l0 == 0 ? 1 + std::min(256, (W.n_tags + 1023) / 1024) : 1;
    hipLaunchKernelGGL(k_ps_setup, dim3(blocks), dim3(256), 0, s, sa);
  }
  PsArgs a{};
  a.layers = W.table;
  a.n_layers = n_layers;
  a.d = L0.d;
  a.f = L0.f;
  a.E = L0.E;
  a.k = L0.k;
  a.hs = L0.has_shared ? 1 : 0;
  a.eps = rec.eps;
  a.h = h;
  for (int i = 0; i < 2; ++i) {
    a.rbuf[i] = W.rbuf[i];
    a.ss[i] = W.ss[i];
    a.lgt[i] = W.lgt[i];
  }
  a.hrow = W.hrow;
  a.otg = W.otg;
  a.sync = W.sync;
  a.rec_logits = rec.logits;
  a.rec_idx = rec.topk_idx;
  a.rec_w = rec.topk_w;
  a.rec_x = rec.x;
  a.rec_y = rec.y;
  a.rec_err = rec.error;
  a.err_ws = W.err_ws;
  // The poll bound of every wait; a test can lower it through the
  // environment (QRE_PERSIST_SPIN_MAX, read at every call) to drive the
  // give-up path from the host.
  a.spin_max = kSpinMax;
  if (const char* v = getenv("QRE_PERSIST_SPIN_MAX")) {
    const long n = strtol(v, nullptr, 10);
    if (n >= 1 && n <= (long)kSpinMax) a.spin_max = (uint32_t)n;
  }
  const int nS = L0.k + a.hs;
  int need = L0.E;
  need = need > nS * (L0.f / 16) ? need : nS * (L0.f / 16);
  need = need > nS * (L0.d / 64) ? need : nS * (L0.d / 64);
  hipEvent_t e0 = rec.events ? rec.events[0] : nullptr, e1 = rec.events ? rec.events[1] : nullptr;
  switch (L0.gate.type) {
    case MOE_Q8_0: return launch_ps_d<MOE_Q8_0>(L0.down.type, a, need, s, e0, e1);
    case MOE_IQ4_NL: return launch_ps_d<MOE_IQ4_NL>(L0.down.type, a, need, s, e0, e1);
    default: return launch_ps_d<MOE_NVFP4>(L0.down.type, a, need, s, e0, e1);
  }
}

}  // namespace qre
