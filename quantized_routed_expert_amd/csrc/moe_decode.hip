// Per-layer decode / verify path (T <= 64 tokens): the gate/up and down
// stages of moe_ffn_forward over an expert plan in global memory, the
// activation preparation, and the down pass of the fused decode step over its
// slot table.  The tile code is in moe_dq.h.
#include <hip/hip_runtime.h>

#include "moe_dq.h"

namespace qre {

// Fused step, down pass: the combine of one 64-column tile, by the last
// workgroup to finish the tile.  Wavefront w takes tokens w, w+4, ...; lane c
// column 64*ct + c.  y sums the shared row, then the routed slots in order j;
// the tile's sum of squares of the new residual is a wavefront reduction.
__device__ __forceinline__ void fz_combine_tile(const DecodeArgs& a, int ct) {
  const int d = a.mat[0].rows, T = a.T, k = a.k, TK = T * k;
  const int n_ct = d / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int col = ct * 64 + lane;
  auto ld_o = [&](long i) { return __hip_atomic_load(a.o + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  // tokens wid and wid + 4 together (T <= 8), all loads of a batch in flight
  // before any is used; rows past T or k repeat a valid one and are unused
  for (int t0 = wid; t0 < T; t0 += 8) {
    const int tt[2] = {t0, min(t0 + 4, T - 1)};
    float y[2], r[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      y[u] = a.has_shared ? ld_o((long)(TK + tt[u]) * d + col) : 0.0f;
      r[u] = a.r_in[(long)tt[u] * d + col];
    }
    for (int j0 = 0; j0 < k; j0 += 8) {
      float wj[2][8], oj[2][8];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int j = min(j0 + jj, k - 1);
          wj[u][jj] = a.gate_w[tt[u] * k + j];
          oj[u][jj] = ld_o((long)(tt[u] * k + j) * d + col);
        }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          if (j0 + jj < k) y[u] = fmaf(wj[u][jj], oj[u][jj], y[u]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u == 1 && t0 + 4 >= T) break;  // (wavefront-uniform)
      const int t = tt[u];
      const float rn = r[u] + y[u];
      a.r_out[(long)t * d + col] = rn;
      if (a.rec_y) a.rec_y[(long)t * d + col] = y[u];
      const float ss = wave_sum(rn * rn);
      if (lane == 0) a.ss_part[t * n_ct + ct] = ss;
    }
  }
}

// Stage kernel over a plan: global plan arrays, or (TABLE) the fused step's
// slot table, whose routed rows go to their pair's output row; there the
// workgroups of each 64-column tile count themselves done, and the last one
// forms the tile's combine.  The o rows are written and read with agent-scope
// atomic accesses, which bypass the XCDs' private L2 caches, and every store
// has completed (s_waitcnt) before the count: no cache-wide fence is needed
// (a __threadfence writes back and invalidates whole L2 caches, which costs
// more than the combine saves).
template <int FMT, int NT, bool GATEUP, bool ROLL, bool TABLE = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NT == 1 ? 2 : 1))) void k_ffn_dq(
    const DecodeArgs a) {
  extern __shared__ __align__(16) f16 sA[];  // activations of the current column pass, then scales

  dq_pin_args(a);
  const int wid = threadIdx.x >> 6;
  const int ksplit = a.ksplit;
  const int rt_per_wg = 4 / ksplit;
  const int rows = a.mat[0].rows;
  const int wg_per_slot = (rows / 16) / rt_per_wg;
  // the slot count and the first item's entry are read together (the table
  // has T*k + 1 entries at least; one past the count is read but not used)
  const SlotEnt se0 = a.slots[min((int)blockIdx.x / wg_per_slot, a.T * a.k)];
  const int total = *a.n_slots * wg_per_slot;

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int slot = item / wg_per_slot;
    const int tile = (item % wg_per_slot) * rt_per_wg + wid / ksplit;
    const SlotEnt se = item == (int)blockIdx.x ? se0 : a.slots[slot];
    const SlotInfo si{se.e, se.shared != 0, se.row0, se.cnt};
    dq_item<FMT, NT, GATEUP, ROLL, TABLE, !TABLE, !TABLE>(a, si, tile, wid % ksplit, a.row_token, sA);
    if constexpr (TABLE && !GATEUP) {
      if (a.tile_cnt) {
        __shared__ int s_last;
        const int ct = item % wg_per_slot;  // 64-column tile (four 16-row tiles)
        __builtin_amdgcn_s_waitcnt(0);      // this workgroup's o rows have landed
        __syncthreads();
        if (threadIdx.x == 0) s_last = atomicAdd(&a.tile_cnt[ct], 1) == total / wg_per_slot - 1;
        __syncthreads();
        if (s_last) {
          fz_combine_tile(a, ct);
          if (threadIdx.x == 0) a.tile_cnt[ct] = 0;
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Activation preparation: X16 rows (fp16, per-token power-of-two scale; fp32
// tokens as hi/lo pairs), in the block layout the gate/up weights decode to.
// ----------------------------------------------------------------------------

// The workgroup past the last token builds the slot table of the expert
// passes: the shared expert, then the active experts by descending token
// count (a counting sort over counts 0..T; the order within a count is
// immaterial), so that the passes start their longest items first and read
// an item's expert, rows and count in one load.
__global__ __launch_bounds__(256) void k_prep_x(const void* __restrict__ x, int x_bf16, int d, int P, int gate_fmt,
                                                f16* __restrict__ x16, float* __restrict__ xs,
                                                const int32_t* __restrict__ offsets,
                                                const int32_t* __restrict__ active,
                                                const int32_t* __restrict__ n_active, int has_shared, int k,
                                                SlotEnt* __restrict__ slots, int32_t* __restrict__ n_slots, int T,
                                                const int32_t* __restrict__ slot_row) {
  const int t = blockIdx.x;
  if (t == T) {
    __shared__ int32_t hist[kDecodeMaxT + 2];
    __shared__ int32_t start[kDecodeMaxT + 2];
    const int tid = threadIdx.x;
    const int n = *n_active;
    const int hs = has_shared ? 1 : 0;
    auto count_of = [&](int e) { return min(offsets[e + 1] - offsets[e], T); };
    if (tid <= T + 1) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += 256) atomicAdd(&hist[count_of(active[i])], 1);
    __syncthreads();
    if (tid == 0) {
      int run = hs;
      for (int c = T; c >= 0; --c) {
        start[c] = run;
        run += hist[c];
      }
      if (hs) slots[0] = SlotEnt{0, T * k, T, 1};
      *n_slots = run;
    }
    __syncthreads();
    for (int i = tid; i < n; i += 256) {
      const int e = active[i];
      const int c = count_of(e);
      slots[atomicAdd(&start[c], 1)] = SlotEnt{e, offsets[e], c, 0};
    }
    return;
  }
  __shared__ float red[4];
  float mx = 0.0f;
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    const float v = x_bf16 ? bf16_bits_to_f32(((const uint16_t*)x)[(long)t * d + i]) : ((const float*)x)[(long)t * d + i];
    mx = fmaxf(mx, fabsf(v));
  }
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int ex = x16_exponent(mx);
  const float down = ldexpf(1.0f, -ex);
  // the token's rows: its shared-expert row T*k + t, then the plan row of
  // each of its k pairs (the expert passes read a slot's rows consecutively)
  __shared__ int32_t rows[33];  // k <= 32
  if ((int)threadIdx.x <= k) rows[threadIdx.x] = threadIdx.x == 0 ? T * k + t : slot_row[t * k + threadIdx.x - 1];
  __syncthreads();
  // one 8-position output chunk per step: positions 8c .. 8c+7 hold two runs
  // of four consecutive elements (IQ4_NL block order: elements 4q.. and
  // 16+4q.. of the block for quarter q; other formats: in order), stored as
  // one 16-byte word per row
  for (int c = threadIdx.x; c < d / 8; c += blockDim.x) {
    const int e0 = gate_fmt == MOE_IQ4_NL ? (c >> 2) * 32 + 4 * (c & 3) : 8 * c;
    const int e1 = gate_fmt == MOE_IQ4_NL ? e0 + 16 : e0 + 4;
    float v[8];
    if (x_bf16) {
      const u32x2 a = *(const u32x2*)((const uint16_t*)x + (long)t * d + e0);
      const u32x2 b = *(const u32x2*)((const uint16_t*)x + (long)t * d + e1);
      const uint32_t w[4] = {a.x, a.y, b.x, b.y};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = bf16_bits_to_f32(w[q] & 0xffffu);
        v[2 * q + 1] = bf16_bits_to_f32(w[q] >> 16);
      }
    } else {
      const f32x4 a = *(const f32x4*)((const float*)x + (long)t * d + e0);
      const f32x4 b = *(const f32x4*)((const float*)x + (long)t * d + e1);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    f16x8 hi, lo;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float sv = v[q] * down;
      hi[q] = (f16)sv;
      lo[q] = (f16)(sv - (float)hi[q]);
    }
    // (a pair the plan dropped -- an invalid or repeated id -- has no row)
    for (int j = 0; j <= k; ++j) {
      const long r = rows[j];
      if (r < 0) continue;
      *(f16x8*)&x16[(r * P) * d + 8 * c] = hi;
      if (P == 2) *(f16x8*)&x16[(r * P + 1) * d + 8 * c] = lo;
    }
  }
  if ((int)threadIdx.x < (k + 1) * P) {
    const int j = threadIdx.x / P, part = threadIdx.x - j * P;
    if (rows[j] >= 0) xs[(long)rows[j] * P + part] = ldexpf(1.0f, ex);
  }
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------

namespace {

// One workgroup per item (up to 4096, which then loop): workgroups are
// dispatched in index order as earlier ones finish, so the items are balanced
// dynamically and the long items of the first slots (the shared expert, which
// carries every token) start at once.
template <int FMT, int NT, bool GATEUP, bool ROLL>
hipError_t launch_fmt_nt(const DecodeArgs& a, size_t lds, int items, hipStream_t s) {
  hipLaunchKernelGGL((k_ffn_dq<FMT, NT, GATEUP, ROLL>), dim3(items < 4096 ? items : 4096), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int FMT, bool GATEUP, bool ROLL>
hipError_t launch_fmt_roll(const DecodeArgs& a, int nt, size_t lds, int items, hipStream_t s) {
  if (nt == 1) return launch_fmt_nt<FMT, 1, GATEUP, ROLL>(a, lds, items, s);
  if (nt == 2) return launch_fmt_nt<FMT, 2, GATEUP, ROLL>(a, lds, items, s);
  return launch_fmt_nt<FMT, 4, GATEUP, ROLL>(a, lds, items, s);
}

template <int FMT, bool GATEUP>
hipError_t launch_fmt(const DecodeArgs& a, int ncols_max, int items, hipStream_t s) {
  constexpr int CPT = cols_per_tile<FMT>();
  const int K = a.mat[0].cols;
  const int nt = pick_nt(CPT, ncols_max, K);
  const size_t lds = dq_lds_bytes(FMT, CPT, nt, K, a.ksplit, GATEUP ? 2 : 1);
  if (dq_nsteps(FMT, K, a.ksplit) > dq_pd(FMT, GATEUP)) return launch_fmt_roll<FMT, GATEUP, true>(a, nt, lds, items, s);
  return launch_fmt_roll<FMT, GATEUP, false>(a, nt, lds, items, s);
}

template <bool GATEUP>
hipError_t launch_pass(int fmt, const DecodeArgs& a, int ncols_max, int items, hipStream_t s) {
  switch (fmt) {
    case MOE_Q8_0: return launch_fmt<MOE_Q8_0, GATEUP>(a, ncols_max, items, s);
    case MOE_IQ4_NL: return launch_fmt<MOE_IQ4_NL, GATEUP>(a, ncols_max, items, s);
    case MOE_Q5_1:
      if constexpr (!GATEUP) return launch_fmt<MOE_Q5_1, false>(a, ncols_max, items, s);
      return hipErrorInvalidValue;  // a down format only
    default: return launch_fmt<MOE_NVFP4, GATEUP>(a, ncols_max, items, s);
  }
}

}  // namespace

// Down pass of the fused step over the slot table: a grid of at most one
// resident wave of workgroups that loops over the items.
template <int FMT, int NT, bool ROLL>
static void launch_fz_down_nt(const DecodeArgs& a, size_t lds, int items, hipStream_t s) {
  auto kern = k_ffn_dq<FMT, NT, false, ROLL, true>;
  hipLaunchKernelGGL(kern, dim3(fused_grid(kern, lds, items)), dim3(256), lds, s, a);
}

template <int FMT, bool ROLL>
static hipError_t launch_fz_down_roll(const DecodeArgs& a, int nt, size_t lds, int items, hipStream_t s) {
  if (nt == 1)
    launch_fz_down_nt<FMT, 1, ROLL>(a, lds, items, s);
  else if (nt == 2)
    launch_fz_down_nt<FMT, 2, ROLL>(a, lds, items, s);
  else
    launch_fz_down_nt<FMT, 4, ROLL>(a, lds, items, s);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_fz_down_fmt(const DecodeArgs& a, int items, hipStream_t s) {
  constexpr int CPT = cols_per_tile<FMT>();
  const int K = a.mat[0].cols;
  const int nt = pick_nt(CPT, a.T * 2, K);
  const size_t lds = dq_lds_bytes(FMT, CPT, nt, K, a.ksplit, 1);
  if (dq_nsteps(FMT, K, a.ksplit) > dq_pd(FMT, false)) return launch_fz_down_roll<FMT, true>(a, nt, lds, items, s);
  return launch_fz_down_roll<FMT, false>(a, nt, lds, items, s);
}

hipError_t launch_dq_down_table(const DecodeArgs& a, int fmt, int items, hipStream_t s) {
  switch (fmt) {
    case MOE_Q8_0: return launch_fz_down_fmt<MOE_Q8_0>(a, items, s);
    case MOE_IQ4_NL: return launch_fz_down_fmt<MOE_IQ4_NL>(a, items, s);
    case MOE_Q5_1: return launch_fz_down_fmt<MOE_Q5_1>(a, items, s);
    default: return launch_fz_down_fmt<MOE_NVFP4>(a, items, s);
  }
}

size_t decode_ws_bytes(int T, int d, int f, int k, int x_dtype) {
  const int P = x_dtype == MOE_F32 ? 2 : 1;
  const size_t R = (size_t)T * k + T;
  return align_up(R * P * d * 2, 256) + align_up(R * P * 4, 256) + align_up(R * f * 4, 256) + align_up(R * (f / 16) * 4, 256) +
         align_up(R * d * 4, 256) + align_up(((size_t)T * k + 2) * sizeof(SlotEnt), 256) + 256;
}

hipError_t launch_decode_stage(int stage, const FfnCall& c, hipStream_t s) {
  const moe_layer& L = *c.L;
  const int T = c.T;
  const int P = c.x_dtype == MOE_F32 ? 2 : 1;
  DecodeWs w = carve(c.ws, T, L.d, L.f, L.k, P);
  if (stage == kStagePrepare) {
    hipLaunchKernelGGL(k_prep_x, dim3(T + 1), dim3(256), 0, s, c.x, c.x_dtype == MOE_BF16 ? 1 : 0, L.d, P,
                       L.gate.type, w.x16, w.xs, c.p.offsets, c.p.active, c.p.n_active, L.has_shared, L.k, w.slots,
                       w.n_slots, T, c.p.slot_row);
    return hipGetLastError();
  }
  if (stage == kStageCombine)
    return launch_combine(w.o, 0, c.topk_w, c.p.slot_row, T, L.k, L.d, L.has_shared, c.y, c.y_dtype, s);

  const int max_slots = (T * L.k < L.E ? T * L.k : L.E) + (L.has_shared ? 1 : 0);
  DecodeArgs a = stage == kStageGateUp ? gateup_args(L, T, P, w) : down_args(L, T, w);
  a.offsets = c.p.offsets;
  a.row_token = c.p.row_token;
  a.active = c.p.active;
  a.slots = w.slots;
  a.n_slots = w.n_slots;
  a.n_active = c.p.n_active;
  a.error = c.p.error;
  if (stage == kStageGateUp) {
    const int wg_per_slot = (L.f / 16) / (4 / a.ksplit);
    const long items = (long)max_slots * wg_per_slot;
    return launch_pass<true>(L.gate.type, a, T * P, (int)items, s);
  }
  const int wg_per_slot = (L.d / 16) / 4;
  const long items = (long)max_slots * wg_per_slot;
  return launch_pass<false>(L.down.type, a, T * 2, (int)items, s);
}

}  // namespace qre
