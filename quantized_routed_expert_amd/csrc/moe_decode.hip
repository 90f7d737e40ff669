// Decode / verify path of the routed experts (T <= 64 tokens): grouped
// dequantising GEMV-like products over the expert plan ("grouped kernels" of
// the device-planned MoE tail, UD-IQ2_XS (L4 fix) page, "What was changed").
//
// The work is HBM-bound: every weight byte of the active experts is read once.
// Weights are the B operand of v_mfma_f32_16x16x32_f16: each lane owns one
// weight row of a 16-row tile and one 16-byte chunk of codes per step (the
// four lane groups read a row's four consecutive chunks, 64 contiguous bytes),
// and decodes it in registers to exact fp16 values (IQ4_NL codebook entries,
// Q8_0 int8 codes, or e2m1 * e4m3 products for the NVFP4-style format).
// Activations are the A operand, staged in LDS as fp16 (with a per-token
// power-of-two scale) or as fp16 hi/lo pairs.  For the Q8_0 and IQ4_NL formats
// the A operand is block-diagonal: lane group G only multiplies the chunk it
// decoded, so each accumulator row group holds the partial sum of exactly one
// quant block and the block's fp16 scale is applied once per lane (fp32 FMA)
// after the MFMA.  The NVFP4-style block scale is folded into the fp16 weights
// (exact) and the tensor scale is applied at the end.  Accumulation is fp32.
//
// Two drivers share the tile code:
//  * k_ffn_dq: one stage of moe_ffn_forward (gate/up or down) over a plan in
//    global memory;
//  * the fused decode step (k_fz_route, k_fz_gateup, k_ffn_dq over a slot
//    table): three launches per layer, the routing and plan recomputed in each
//    workgroup's LDS so that no kernel waits on a chain of dependent loads.
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_launch.h"

namespace qre {

// Slot table entry (fused path): expert, first plan row, rows, 1 = shared.
struct SlotEnt {
  int32_t e, row0, cnt, shared;
};

struct DecodeArgs {
  QMatDev mat[2];   // routed: gate, up (gate/up pass) or down (down pass)
  QMatDev smat[2];  // shared expert, same roles
  int has_shared;
  // per-layer path: plan in global memory (routed slots first, shared last)
  const int32_t* offsets;
  const int32_t* row_token;
  const int32_t* active;
  const int32_t* n_active;
  // fused path: slot table (shared first) and its length
  const SlotEnt* slots;
  const int32_t* n_slots;
  int32_t* error;
  int T, k;
  int P;                   // fp16 parts per column: 1 (bf16 tokens), 2 (fp32 tokens, or h hi/lo)
  int ksplit;              // waves along K per 16-row tile (1, 2, 4)
  const f16* in16;         // gate/up: X16 [T*P][d]; down: H16 [(T*k+T)*2][f]
  const float* in_scale;   // gate/up: scale of each X16 row (a power of two)
  f16* h16;                // gate/up output H16 [(T*k+T)*2][f]
  int down_type;           // gate/up: layout of H16 rows (IQ4_NL: block-permuted)
  float* o;                // down output O [(T*k+T)][d]
  const int32_t* pair_of_row;  // fused down pass: O row of each plan row (t*k + j); null: the plan row
};

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

template <int FMT>
__device__ __forceinline__ f16x8 decode_b(const u32x4& c, int i, uint32_t sraw) {
  if constexpr (FMT == MOE_IQ4_NL) {
    return iq4_dword_to_f16x8(c[i]);
  } else if constexpr (FMT == MOE_Q8_0) {
    return q8_dwords_to_f16x8(c[2 * i], c[2 * i + 1]);
  } else {
    // dwords 0,1 hold the chunk's first 16-element block, 2,3 the second
    const uint32_t sbyte = (i < 2) ? (sraw & 0xffu) : ((sraw >> 8) & 0xffu);
    return fp4_dword_to_f16x8(c[i], (f16)e4m3_to_f32(sbyte));
  }
}

// Position of element i of a row in the activation layout matching the
// weight decode of format `fmt` (IQ4_NL reorders elements inside each block).
__device__ __forceinline__ int act_pos(int fmt, int i) {
  return fmt == MOE_IQ4_NL ? ((i & ~31) + iq4_pos(i & 31)) : i;
}

// Columns (token or hi/lo parts) per N-tile: block-diagonal formats use four
// (one per lane group's block); the NVFP4-style format uses the first eight
// rows of the dense 16-row A operand (the other eight stay zero).
template <int FMT>
constexpr int cols_per_tile() {
  return FMT == MOE_NVFP4 ? 8 : 4;
}

struct SlotInfo {
  int e;
  bool is_sh;
  int row0;
  int ncolt;  // tokens of the slot
};

// One workgroup item: rows [tile*16, tile*16+16) of slot `si` (gate + up, or
// down), this wave's K part, against all of the slot's columns.  sA: the
// workgroup's activation staging buffer; red: [4][NMAT][NT][64] partials.
template <int FMT, int NT, bool GATEUP>
__device__ __forceinline__ void dq_item(const DecodeArgs& a, const SlotInfo& si, int tile, int kpart,
                                        const int32_t* row_token, f16* sA, f32x4* red) {
  constexpr int EPS = (FMT == MOE_Q8_0) ? 16 : 32;  // elements per lane per step (one 16-byte load)
  constexpr int NMF = EPS / 8;                       // MFMAs per step
  constexpr bool BD = FMT != MOE_NVFP4;              // block-diagonal activations
  constexpr int CPT = cols_per_tile<FMT>();
  constexpr int CPP = NT * CPT;                      // columns staged per pass
  constexpr int NMAT = GATEUP ? 2 : 1;
  constexpr int PD = 6;                              // steps of codes in flight per matrix
  constexpr int AB = 2;                              // activation chunks per thread issued first

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = lane & 15, G = lane >> 4;
  const int ksplit = a.ksplit;
  const int rows = a.mat[0].rows, K = a.mat[0].cols;
  const int kw = K / ksplit;
  const int nsteps = kw / (4 * EPS);
  const int crb = code_row_bytes(FMT, K), srb = scale_row_bytes(FMT, K);
  const int P = a.P;
  const int ncol = si.ncolt * P;

  const uint8_t* crow[NMAT];
  const uint8_t* srow[NMAT];
  float tsc[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
    const QMatDev& W = si.is_sh ? a.smat[m] : a.mat[m];
    const long rw = (long)si.e * rows + tile * 16 + n;
    crow[m] = W.codes + rw * crb;
    srow[m] = W.scales + rw * srb;
    tsc[m] = (FMT == MOE_NVFP4) ? W.ts[si.e] : 1.0f;
  }
  // K position of this lane at step s: the four lane groups take four
  // consecutive EPS-element chunks, so a row's 16-byte code loads are
  // contiguous across the lane groups (64 bytes per row per step).
  const int kbase = kpart * kw + G * EPS;

  // input row of column `col` (a token, or one fp16 part of it)
  auto in_row_of = [&](int col) -> long {
    if constexpr (GATEUP) {
      const int tc = col / P, part = col - tc * P;
      const int t = si.is_sh ? tc : row_token[si.row0 + tc];
      return (long)t * P + part;
    } else {
      return (long)(si.row0 + col / 2) * 2 + (col & 1);
    }
  };

  const int chunks_per_col = K / 8;  // 16-byte activation chunks per column
  // All global loads below are unconditional (out-of-range ones repeat a valid
  // address and their result is discarded), so the waits that follow them are
  // exact: data issued earlier never waits for data issued later.
  // this lane's code and scale addresses at step 0; step s adds a constant
  // (4 * EPS elements: 64 code bytes, 4 * EPS / 32 scale words)
  const uint8_t* cl[NMAT];
  const uint16_t* sl[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
    cl[m] = crow[m] + (FMT == MOE_Q8_0 ? kbase : (kbase >> 1));
    sl[m] = (const uint16_t*)srow[m] + (kbase >> 5);
  }
  auto load_step = [&](int m, int s, u32x4& c, uint32_t& sc) {
    c = *(const u32x4*)(cl[m] + s * (FMT == MOE_Q8_0 ? 4 * EPS : 2 * EPS));
    // Q8_0 / IQ4_NL: the block's fp16 scale; NVFP4: the chunk's two E4M3 scales
    sc = sl[m][s * (4 * EPS / 32)];
  };
  for (int c0 = 0; c0 < ncol; c0 += CPP) {
    const int ncp = min(CPP, ncol - c0);
    const int nch = ncp * chunks_per_col;
    // ---- the first batch of this pass's activation chunks, issued before the
    // weight codes so that waiting for them does not wait for the codes
    u32x4 av[AB];
#pragma unroll
    for (int b = 0; b < AB; ++b) {
      const int ch = min(tid + b * 256, nch - 1);
      const int c = ch / chunks_per_col, kk = (ch - c * chunks_per_col) * 8;
      av[b] = *(const u32x4*)(a.in16 + in_row_of(c0 + c) * K + kk);
    }
    // ---- the first PD steps of weight codes (independent of the activations)
    u32x4 cb[NMAT][PD];
    uint32_t sb[NMAT][PD];
#pragma unroll
    for (int u = 0; u < PD; ++u)
#pragma unroll
      for (int m = 0; m < NMAT; ++m) load_step(m, min(u, nsteps - 1), cb[m][u], sb[m][u]);

    // ---- stage the activation columns into LDS.  Columns at or beyond ncp
    // are never read (their A rows are zero), so they are not written.
    __syncthreads();  // the previous pass has finished reading sA
#pragma unroll
    for (int b = 0; b < AB; ++b) {
      const int ch = tid + b * 256;
      if (ch < nch) {
        const int c = ch / chunks_per_col, kk = (ch - c * chunks_per_col) * 8;
        *(u32x4*)&sA[c * K + kk] = av[b];
      }
    }
    for (int ch = tid + AB * 256; ch < nch; ch += 256) {
      const int c = ch / chunks_per_col, kk = (ch - c * chunks_per_col) * 8;
      *(u32x4*)&sA[c * K + kk] = *(const u32x4*)(a.in16 + in_row_of(c0 + c) * K + kk);
    }
    __syncthreads();

    // A-operand LDS row for each N-tile (this lane is A row m = n, K slice G);
    // lanes without a column read column 0 and use zeros
    int acol[NT];
    bool aval[NT];
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
      int c;
      bool valid;
      if constexpr (BD) {
        valid = (n >> 2) == G;
        c = jt * CPT + (n & 3);
      } else {
        valid = n < CPT;
        c = jt * CPT + n;
      }
      aval[jt] = valid && c < ncp;
      acol[jt] = aval[jt] ? c : 0;
    }

    f32x4 acc[NMAT][NT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) acc[m][jt] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute_step = [&](const u32x4 (&cc)[NMAT], const uint32_t (&ss)[NMAT], int s) {
      f16x8 ac[NT][NMF];
#pragma unroll
      for (int jt = 0; jt < NT; ++jt)
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
          const f16x8 v = *(const f16x8*)&sA[acol[jt] * K + kbase + s * 4 * EPS + 8 * i];
          ac[jt][i] = aval[jt] ? v : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        f32x4 D[NT];
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) D[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
          const f16x8 bf = decode_b<FMT>(cc[m], i, ss[m]);
#pragma unroll
          for (int jt = 0; jt < NT; ++jt) D[jt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ac[jt][i], bf, D[jt], 0, 0, 0);
        }
        if constexpr (FMT == MOE_NVFP4) {
#pragma unroll
          for (int jt = 0; jt < NT; ++jt) acc[m][jt] += D[jt];
        } else {
          const float sc = f16_bits_to_f32(ss[m]);
#pragma unroll
          for (int jt = 0; jt < NT; ++jt) {
            acc[m][jt].x = fmaf(sc, D[jt].x, acc[m][jt].x);
            acc[m][jt].y = fmaf(sc, D[jt].y, acc[m][jt].y);
            acc[m][jt].z = fmaf(sc, D[jt].z, acc[m][jt].z);
            acc[m][jt].w = fmaf(sc, D[jt].w, acc[m][jt].w);
          }
        }
      }
    };

    if (nsteps <= PD) {
      // every step's codes are already in flight
#pragma unroll
      for (int u = 0; u < PD; ++u) {
        if (u < nsteps) {
          u32x4 cc[NMAT];
          uint32_t ss[NMAT];
#pragma unroll
          for (int m = 0; m < NMAT; ++m) {
            cc[m] = cb[m][u];
            ss[m] = sb[m][u];
          }
          compute_step(cc, ss, u);
        }
      }
    } else {
      // rolling prefetch, PD steps ahead (past the end it repeats the last step)
      for (int s0 = 0; s0 < nsteps; s0 += PD) {
#pragma unroll
        for (int u = 0; u < PD; ++u) {
          const int s = s0 + u;
          u32x4 cc[NMAT];
          uint32_t ss[NMAT];
#pragma unroll
          for (int m = 0; m < NMAT; ++m) {
            cc[m] = cb[m][u];
            ss[m] = sb[m][u];
            load_step(m, min(s + PD, nsteps - 1), cb[m][u], sb[m][u]);
          }
          if (s < nsteps) compute_step(cc, ss, s);
        }
      }
    }

    // block-diagonal: sum the four lane groups (one chunk each)
    if constexpr (BD) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) {
          f32x4& v = acc[m][jt];
          v.x += __shfl_xor(v.x, 16, 64);
          v.y += __shfl_xor(v.y, 16, 64);
          v.z += __shfl_xor(v.z, 16, 64);
          v.w += __shfl_xor(v.w, 16, 64);
          v.x += __shfl_xor(v.x, 32, 64);
          v.y += __shfl_xor(v.y, 32, 64);
          v.z += __shfl_xor(v.z, 32, 64);
          v.w += __shfl_xor(v.w, 32, 64);
        }
    }
    // reduce the K parts of this row tile through LDS
    if (ksplit > 1) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) red[((wid * NMAT + m) * NT + jt) * 64 + lane] = acc[m][jt];
      __syncthreads();
      if (kpart == 0) {
        for (int q = 1; q < ksplit; ++q)
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int jt = 0; jt < NT; ++jt) acc[m][jt] += red[(((wid + q) * NMAT + m) * NT + jt) * 64 + lane];
      }
      __syncthreads();
    }

    if (kpart == 0) {
      const int frow = tile * 16 + n;  // output feature of this lane
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) {
        // D row m = 4G + v.  Block-diagonal: the four lane groups hold the same
        // sums after the reduction; group G takes column slot v == G (P == 1)
        // or the pair v = 2G, 2G+1 (P == 2).  Dense: column 4G + v.
        float vals[NMAT][4];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          vals[m][0] = acc[m][jt].x * tsc[m];
          vals[m][1] = acc[m][jt].y * tsc[m];
          vals[m][2] = acc[m][jt].z * tsc[m];
          vals[m][3] = acc[m][jt].w * tsc[m];
        }
#pragma unroll
        for (int v = 0; v < 4; v += 1) {
          int cl;
          if constexpr (BD) {
            if (P == 1 ? (v != G) : (v != 2 * G)) continue;
            cl = jt * CPT + v;
          } else {
            if (P == 2 && (v & 1)) continue;
            cl = jt * CPT + 4 * G + v;
            if (4 * G + v >= CPT) continue;
          }
          if (cl >= ncp) continue;
          const int tc = (c0 + cl) / P;
          float val[NMAT];
#pragma unroll
          for (int m = 0; m < NMAT; ++m) val[m] = (P == 2) ? vals[m][v] + vals[m][v + 1] : vals[m][v];
          const int out_row = si.row0 + tc;
          if constexpr (GATEUP) {
            const int t = si.is_sh ? tc : row_token[si.row0 + tc];
            const float xs = a.in_scale[(long)t * P];
            const float g = val[0] * xs, u = val[1] * xs;
            const float h = silu_f(g) * u;
            if (!(fabsf(h) < 65504.0f)) atomicOr(a.error, 2);
            const f16 hi = (f16)h;
            const f16 lo = (f16)(h - (float)hi);
            const int f = rows;
            const int pos = act_pos(a.down_type, frow);
            a.h16[((long)out_row * 2 + 0) * f + pos] = hi;
            a.h16[((long)out_row * 2 + 1) * f + pos] = lo;
          } else {
            // fused path: routed rows go to their (token, slot) pair's row
            const int orow = (a.pair_of_row && !si.is_sh) ? a.pair_of_row[out_row] : out_row;
            a.o[(long)orow * rows + frow] = val[0];
          }
        }
      }
    }
  }
}

// Stage kernel over a plan (global plan arrays, or the fused path's slot table).
template <int FMT, int NT, bool GATEUP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NT == 1 ? 2 : 1))) void k_ffn_dq(
    const DecodeArgs a) {
  constexpr int NMAT = GATEUP ? 2 : 1;
  __shared__ f32x4 red[4 * NMAT * NT * 64];
  extern __shared__ f16 sA[];  // [CPP][K] activations of the current column pass

  const int wid = threadIdx.x >> 6;
  const int ksplit = a.ksplit;
  const int rt_per_wg = 4 / ksplit;
  const int rows = a.mat[0].rows;
  const int wg_per_slot = (rows / 16) / rt_per_wg;
  const bool table = a.slots != nullptr;
  const int n_act = table ? 0 : *a.n_active;
  const int total = (table ? *a.n_slots : n_act + a.has_shared) * wg_per_slot;

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int slot = item / wg_per_slot;
    const int tile = (item % wg_per_slot) * rt_per_wg + wid / ksplit;
    SlotInfo si;
    if (table) {
      const SlotEnt se = a.slots[slot];
      si = SlotInfo{se.e, se.shared != 0, se.row0, se.cnt};
    } else if (slot < n_act) {
      const int e = a.active[slot];
      si = SlotInfo{e, false, a.offsets[e], a.offsets[e + 1] - a.offsets[e]};
    } else {
      si = SlotInfo{0, true, a.T * a.k, a.T};
    }
    dq_item<FMT, NT, GATEUP>(a, si, tile, wid % ksplit, a.row_token, sA, red);
  }
}

// ----------------------------------------------------------------------------
// Activation preparation: X16 rows (fp16, per-token power-of-two scale; fp32
// tokens as hi/lo pairs), in the block layout the gate/up weights decode to.
// ----------------------------------------------------------------------------

// Exponent e such that max|x| * 2^-e lies in [2^14, 2^15) (0 for an all-zero row).
__device__ __forceinline__ int x16_exponent(float mx) {
  int ex = 0;
  if (mx > 0.0f && mx < __builtin_inff()) {
    int e2;
    frexpf(mx, &e2);  // mx = m * 2^e2, m in [0.5, 1)
    ex = max(-100, min(100, e2 - 15));
  }
  return ex;
}

__global__ __launch_bounds__(256) void k_prep_x(const void* __restrict__ x, int x_bf16, int d, int P, int gate_fmt,
                                                f16* __restrict__ x16, float* __restrict__ xs) {
  const int t = blockIdx.x;
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
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    const float v = x_bf16 ? bf16_bits_to_f32(((const uint16_t*)x)[(long)t * d + i]) : ((const float*)x)[(long)t * d + i];
    const float sv = v * down;
    const int pos = act_pos(gate_fmt, i);
    const f16 hi = (f16)sv;
    x16[((long)t * P) * d + pos] = hi;
    if (P == 2) x16[((long)t * P + 1) * d + pos] = (f16)(sv - (float)hi);
  }
  if (threadIdx.x < P) xs[(long)t * P + threadIdx.x] = ldexpf(1.0f, ex);
}

// ============================================================================
// Fused decode step (T <= kFusedMaxT tokens, bf16 layer inputs).
// ============================================================================

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
// Glue (layer l > 0): y = o[T*k + t] + sum_j topk_w[t][j] * o[t*k + j] (the
// previous layer's combine: shared row, then the routed slots in order j; the
// down pass writes routed rows at their pair's position), h_new = h + y, and
// the layer input x = bf16(h_new / sqrt(mean(h_new^2) + eps)).  The first
// layer takes x = bf16(rmsnorm(h)).  The glue writes the new residual, x (bf16,
// and as power-of-two scaled fp16 for the expert products) and optional
// records of the previous layer's y and this layer's x.
struct FzGlueArgs {
  int d, T, k, has_shared;
  const float* h_in;
  float* h_out;
  const float* o;            // previous layer's expert rows, or null (first layer)
  const float* topk_w;       // previous layer's gate weights
  float* rec_y;              // previous layer's y (optional)
  uint16_t* x_out;           // bf16 layer input (null: the final fold, no next layer)
  uint16_t* rec_x;           // optional record of the same
  f16* x16;
  float* xs;
  int gate_fmt;
  float eps;
  int32_t* error_reset;      // the plan's error word, cleared for the next layer
};

constexpr int kGlueMaxQ = 4;  // d <= 4096: float4 chunks per thread
constexpr int kGlueRB = 8;    // routed rows whose loads are in flight together

// Glue for one token, by one workgroup.  Returns the token's bf16 input in
// v[] (as floats) when the caller needs it.
__device__ __forceinline__ void glue_token(const FzGlueArgs& a, int t, bool writer, f32x4 (&v)[kGlueMaxQ]) {
  __shared__ float red[2][4];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int d = a.d, T = a.T, k = a.k;
  const int nq = d / 1024;
  // residual and shared row first; every routed row of a batch is in flight
  // before the first is used
  f32x4 y[kGlueMaxQ];
#pragma unroll
  for (int q = 0; q < kGlueMaxQ; ++q) {
    if (q < nq) {
      const int i = (q * 256 + tid) * 4;
      v[q] = *(const f32x4*)(a.h_in + (long)t * d + i);
      y[q] = (a.o && a.has_shared) ? *(const f32x4*)(a.o + (long)(T * k + t) * d + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  if (a.o) {
    for (int j0 = 0; j0 < k; j0 += kGlueRB) {
      float wj[kGlueRB];
      f32x4 ov[kGlueMaxQ][kGlueRB];
#pragma unroll
      for (int jj = 0; jj < kGlueRB; ++jj) wj[jj] = (j0 + jj < k) ? a.topk_w[t * k + j0 + jj] : 0.0f;
#pragma unroll
      for (int q = 0; q < kGlueMaxQ; ++q)
#pragma unroll
        for (int jj = 0; jj < kGlueRB; ++jj)
          if (q < nq && j0 + jj < k)
            ov[q][jj] = *(const f32x4*)(a.o + (long)(t * k + j0 + jj) * d + (q * 256 + tid) * 4);
#pragma unroll
      for (int q = 0; q < kGlueMaxQ; ++q)
#pragma unroll
        for (int jj = 0; jj < kGlueRB; ++jj)
          if (q < nq && j0 + jj < k) {
            y[q].x = fmaf(wj[jj], ov[q][jj].x, y[q].x);
            y[q].y = fmaf(wj[jj], ov[q][jj].y, y[q].y);
            y[q].z = fmaf(wj[jj], ov[q][jj].z, y[q].z);
            y[q].w = fmaf(wj[jj], ov[q][jj].w, y[q].w);
          }
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int q = 0; q < kGlueMaxQ; ++q) {
    if (q < nq) {
      const int i = (q * 256 + tid) * 4;
      if (a.o) {
        if (writer && a.rec_y) *(f32x4*)(a.rec_y + (long)t * d + i) = y[q];
        v[q] += y[q];
      }
      if (writer) *(f32x4*)(a.h_out + (long)t * d + i) = v[q];
      ss += v[q].x * v[q].x + v[q].y * v[q].y + v[q].z * v[q].z + v[q].w * v[q].w;
    }
  }
  if (!a.x_out) return;  // final fold: the residual is all that is needed
  ss = wave_sum(ss);
  if (lane == 0) red[0][wid] = ss;
  __syncthreads();
  const float inv = 1.0f / sqrtf((red[0][0] + red[0][1] + red[0][2] + red[0][3]) / (float)d + a.eps);
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

// Glue for T tokens: one workgroup per token.
__global__ __launch_bounds__(256) void k_fz_glue(const FzGlueArgs a) {
  f32x4 v[kGlueMaxQ];
  if (blockIdx.x == 0 && threadIdx.x == 0 && a.error_reset) *a.error_reset = 0;
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

template <bool INLINE>
__global__ __launch_bounds__(256) void k_fz_route(const FzRouteArgs a) {
  __shared__ uint16_t sx[kFusedMaxT * 4096];  // bf16 layer inputs
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int d = a.g.d, T = a.g.T;
  const int e = blockIdx.x * 4 + wid;

  // router row of this wave's expert: lane holds elements (j*64 + lane)*4 .. +3
  f32x4 wv[16];
  const int nj = d / 256;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j < nj && e < a.E) wv[j] = *(const f32x4*)(a.Wr + (long)e * d + (j * 64 + lane) * 4);

  if constexpr (INLINE) {
    if (blockIdx.x == 0 && tid == 0 && a.g.error_reset) *a.g.error_reset = 0;
    f32x4 v[kGlueMaxQ];
    glue_token(a.g, 0, blockIdx.x == 0, v);
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
    for (int c = tid; c < T * d / 8; c += 256) {
      const int t = (c * 8) / d, i = (c * 8) % d;
      *(u32x4*)&sx[t * 4096 + i] = *(const u32x4*)(a.x + (long)t * d + i);
    }
  }
  __syncthreads();
  if (e < a.E) {
    // all tokens' partial sums first, then their wave reductions together
    double acc[kFusedMaxT];
#pragma unroll
    for (int t = 0; t < kFusedMaxT; ++t) acc[t] = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < nj) {
        const int i = (j * 64 + lane) * 4;
#pragma unroll
        for (int t = 0; t < kFusedMaxT; ++t) {
          if (t < T) {
            const u32x2 xb = *(const u32x2*)&sx[t * 4096 + i];
            acc[t] += (double)wv[j].x * (double)bf16_bits_to_f32(xb.x & 0xffffu) +
                      (double)wv[j].y * (double)bf16_bits_to_f32(xb.x >> 16) +
                      (double)wv[j].z * (double)bf16_bits_to_f32(xb.y & 0xffffu) +
                      (double)wv[j].w * (double)bf16_bits_to_f32(xb.y >> 16);
          }
        }
      }
    }
    const double b = a.bias ? (double)a.bias[e] : 0.0;
#pragma unroll
    for (int t = 0; t < kFusedMaxT; ++t) {
      if (t < T) {
        const double r = wave_sum_f64(acc[t]);
        if (lane == 0) a.logits[(long)t * a.E + e] = (float)(r + b);
      }
    }
  }
}

// (2) Top-k + plan (in LDS, recomputed by every workgroup that needs it) +
// grouped gate/up.  Slot 0 is the shared expert (it needs no routing, so its
// items start streaming at once); slots 1.. are the active experts in
// ascending id order.  Workgroup 0 publishes the plan for the down pass and
// the next layer's combine.
struct FzGateArgs {
  DecodeArgs a;  // gate/up pass arguments (in16 = x16, in_scale = xs, h16, error)
  const float* logits;
  int E;
  FusedPlan plan;
};

constexpr int kFusedTK = kFusedMaxT * 32;  // token-slot pairs at most

template <int FMT, int NT, int NPL>
// Single-tile passes (one N-tile of columns, the batch-1 case) are held to two
// waves per SIMD so that one grid of a decode step is resident at once.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NT == 1 ? 2 : 1))) void k_fz_gateup(
    const FzGateArgs g) {
  constexpr int NMAT = 2;
  __shared__ f32x4 red[4 * NMAT * NT * 64];
  __shared__ int32_t sidx[kFusedTK];
  __shared__ float sw[kFusedTK];
  __shared__ int32_t sfirst[kFusedTK];
  __shared__ int32_t srow_token[kFusedTK];
  __shared__ SlotEnt sslot[kFusedTK];
  extern __shared__ f16 sA[];

  const DecodeArgs& a = g.a;
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
    // ---- top-k per token (one wavefront per token), renormalised weights
    for (int t = wid; t < T; t += 4) {
      int ix;
      float lv;
      wave_topk<NPL>(g.logits + (long)t * E, E, k, lane, ix, lv);
      const float vmax = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(lv), 0));
      const float ex = lane < k ? expf(lv - vmax) : 0.0f;
      const float sum = wave_sum(ex);
      if (lane < k) {
        sidx[t * k + lane] = ix;
        sw[t * k + lane] = ex / sum;
      }
    }
    __syncthreads();
    // ---- plan: pair p (thread p) counts the pairs of smaller experts (its
    // expert's first plan row) and the earlier pairs of its own expert (its
    // rank); the first pair of each expert then counts the distinct smaller
    // experts (its slot).  Rows within an expert follow token order.
    int e = 0, less = 0, before = 0, same = 0;
    if (tid < TK) {
      e = sidx[tid];
      for (int q = 0; q < TK; ++q) {
        const int eq = sidx[q];
        less += eq < e ? 1 : 0;
        same += eq == e ? 1 : 0;
        before += (eq == e && q < tid) ? 1 : 0;
      }
      sfirst[tid] = before == 0 ? e : 0x7fffffff;
    }
    __syncthreads();
    if (tid < TK) {
      int dl = 0;
      for (int q = 0; q < TK; ++q) dl += sfirst[q] < e ? 1 : 0;
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
    dq_item<FMT, NT, true>(a, si, tile, wid % ksplit, srow_token, sA, red);
  }
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------

namespace {

struct DecodeWs {
  f16* x16;
  float* xs;
  f16* h16;
  float* o;
};

DecodeWs carve(void* ws, int T, int d, int f, int k, int P) {
  char* p = (char*)ws;
  DecodeWs w;
  w.x16 = (f16*)p;
  p += align_up((size_t)T * P * d * 2, 256);
  w.xs = (float*)p;
  p += align_up((size_t)T * P * 4, 256);
  const size_t R = (size_t)T * k + T;
  w.h16 = (f16*)p;
  p += align_up(R * 2 * f * 2, 256);
  w.o = (float*)p;
  return w;
}

// Waves along K per 16-row tile: as many as divide the lane-group step count.
int pick_ksplit(int K, int eps) {
  const int S = K / (4 * eps);
  for (int ks : {4, 2})
    if (S % ks == 0) return ks;
  return 1;
}

// N-tiles per column pass: enough for the widest slot, within 48 KB of staged
// activations (columns x K x 2 bytes).
int pick_nt(int cpt, int ncols_max, int K) {
  const int fit = (48 * 1024) / (cpt * K * 2);
  int nt = (ncols_max + cpt - 1) / cpt;
  if (nt > fit) nt = fit;
  return nt >= 4 ? 4 : (nt >= 2 ? 2 : 1);
}

template <int FMT, bool GATEUP>
hipError_t launch_fmt(const DecodeArgs& a, int ncols_max, int grid, hipStream_t s) {
  constexpr int CPT = cols_per_tile<FMT>();
  const int K = a.mat[0].cols;
  const int nt = pick_nt(CPT, ncols_max, K);
  const size_t lds = (size_t)nt * CPT * K * 2;
  if (nt == 1)
    hipLaunchKernelGGL((k_ffn_dq<FMT, 1, GATEUP>), dim3(grid), dim3(256), lds, s, a);
  else if (nt == 2)
    hipLaunchKernelGGL((k_ffn_dq<FMT, 2, GATEUP>), dim3(grid), dim3(256), lds, s, a);
  else
    hipLaunchKernelGGL((k_ffn_dq<FMT, 4, GATEUP>), dim3(grid), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <bool GATEUP>
hipError_t launch_pass(int fmt, const DecodeArgs& a, int ncols_max, int grid, hipStream_t s) {
  switch (fmt) {
    case MOE_Q8_0: return launch_fmt<MOE_Q8_0, GATEUP>(a, ncols_max, grid, s);
    case MOE_IQ4_NL: return launch_fmt<MOE_IQ4_NL, GATEUP>(a, ncols_max, grid, s);
    default: return launch_fmt<MOE_NVFP4, GATEUP>(a, ncols_max, grid, s);
  }
}

DecodeArgs gateup_args(const moe_layer& L, int T, int P, const DecodeWs& w) {
  DecodeArgs a{};
  a.has_shared = L.has_shared;
  a.T = T;
  a.k = L.k;
  const int eps = L.gate.type == MOE_Q8_0 ? 16 : 32;
  a.mat[0] = qmat_dev(L.gate);
  a.mat[1] = qmat_dev(L.up);
  if (L.has_shared) {
    a.smat[0] = qmat_dev(L.shared_gate);
    a.smat[1] = qmat_dev(L.shared_up);
  }
  a.P = P;
  a.ksplit = pick_ksplit(L.d, eps);
  a.in16 = w.x16;
  a.in_scale = w.xs;
  a.h16 = w.h16;
  a.down_type = L.down.type;
  return a;
}

DecodeArgs down_args(const moe_layer& L, int T, const DecodeWs& w) {
  DecodeArgs a{};
  a.has_shared = L.has_shared;
  a.T = T;
  a.k = L.k;
  a.mat[0] = qmat_dev(L.down);
  if (L.has_shared) a.smat[0] = qmat_dev(L.shared_down);
  a.P = 2;
  a.ksplit = 1;
  a.in16 = w.h16;
  a.o = w.o;
  return a;
}

// Workgroups of `kern` (256 threads, `lds` dynamic bytes) resident at once on
// the current device, or 0 if the runtime cannot tell.
template <typename Kern>
int resident_wgs(Kern kern, size_t lds) {
  int dev = 0, ncu = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, lds) != hipSuccess) return 0;
  return ncu * per_cu;
}

// Grid of a fused expert pass over `items` items: all of them when they fit
// in one resident wave of workgroups, else one resident wave that loops.
template <typename Kern>
int fused_grid(Kern kern, size_t lds, int items) {
  const int res = resident_wgs(kern, lds);
  return (res > 0 && items > res) ? res : items;
}

template <int FMT, int NT, int NPL>
hipError_t launch_fz_gate_npl(const FzGateArgs& g, int items, size_t lds, hipStream_t s) {
  const int grid = fused_grid(k_fz_gateup<FMT, NT, NPL>, lds, items);
  hipLaunchKernelGGL((k_fz_gateup<FMT, NT, NPL>), dim3(grid), dim3(256), lds, s, g);
  return hipGetLastError();
}

template <int FMT, int NT>
hipError_t launch_fz_gate(const FzGateArgs& g, int items, size_t lds, int E, hipStream_t s) {
  if (E <= 256) return launch_fz_gate_npl<FMT, NT, 4>(g, items, lds, s);
  if (E <= 512) return launch_fz_gate_npl<FMT, NT, 8>(g, items, lds, s);
  return launch_fz_gate_npl<FMT, NT, 16>(g, items, lds, s);
}

template <int FMT>
hipError_t launch_fz_gate_fmt(const FzGateArgs& g, int items, int E, hipStream_t s) {
  constexpr int CPT = cols_per_tile<FMT>();
  const int K = g.a.mat[0].cols;
  const int nt = pick_nt(CPT, g.a.T, K);
  const size_t lds = (size_t)nt * CPT * K * 2;
  if (nt == 1) return launch_fz_gate<FMT, 1>(g, items, lds, E, s);
  if (nt == 2) return launch_fz_gate<FMT, 2>(g, items, lds, E, s);
  return launch_fz_gate<FMT, 4>(g, items, lds, E, s);
}

// Down pass of the fused step over the slot table.
template <int FMT>
hipError_t launch_fz_down_fmt(const DecodeArgs& a, int items, hipStream_t s) {
  constexpr int CPT = cols_per_tile<FMT>();
  const int K = a.mat[0].cols;
  const int nt = pick_nt(CPT, a.T * 2, K);
  const size_t lds = (size_t)nt * CPT * K * 2;
  if (nt == 1) {
    hipLaunchKernelGGL((k_ffn_dq<FMT, 1, false>), dim3(fused_grid(k_ffn_dq<FMT, 1, false>, lds, items)), dim3(256),
                       lds, s, a);
  } else if (nt == 2) {
    hipLaunchKernelGGL((k_ffn_dq<FMT, 2, false>), dim3(fused_grid(k_ffn_dq<FMT, 2, false>, lds, items)), dim3(256),
                       lds, s, a);
  } else {
    hipLaunchKernelGGL((k_ffn_dq<FMT, 4, false>), dim3(fused_grid(k_ffn_dq<FMT, 4, false>, lds, items)), dim3(256),
                       lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace

size_t decode_ws_bytes(int T, int d, int f, int k, int x_dtype) {
  const int P = x_dtype == MOE_F32 ? 2 : 1;
  const size_t R = (size_t)T * k + T;
  return align_up((size_t)T * P * d * 2, 256) + align_up((size_t)T * P * 4, 256) + align_up(R * 2 * f * 2, 256) +
         align_up(R * d * 4, 256);
}

hipError_t launch_decode_stage(int stage, const FfnCall& c, hipStream_t s) {
  const moe_layer& L = *c.L;
  const int T = c.T;
  const int P = c.x_dtype == MOE_F32 ? 2 : 1;
  DecodeWs w = carve(c.ws, T, L.d, L.f, L.k, P);
  if (stage == kStagePrepare) {
    hipLaunchKernelGGL(k_prep_x, dim3(T), dim3(256), 0, s, c.x, c.x_dtype == MOE_BF16 ? 1 : 0, L.d, P, L.gate.type,
                       w.x16, w.xs);
    return hipGetLastError();
  }
  if (stage == kStageCombine)
    return launch_combine(w.o, 0, c.topk_w, c.p.slot_row, T, L.k, L.d, L.has_shared, c.y, c.y_dtype, s);

  const int max_slots = (T * L.k < L.E ? T * L.k : L.E) + (L.has_shared ? 1 : 0);
  DecodeArgs a = stage == kStageGateUp ? gateup_args(L, T, P, w) : down_args(L, T, w);
  a.offsets = c.p.offsets;
  a.row_token = c.p.row_token;
  a.active = c.p.active;
  a.n_active = c.p.n_active;
  a.error = c.p.error;
  if (stage == kStageGateUp) {
    const int wg_per_slot = (L.f / 16) / (4 / a.ksplit);
    const long items = (long)max_slots * wg_per_slot;
    return launch_pass<true>(L.gate.type, a, T * P, (int)(items < 4096 ? items : 4096), s);
  }
  const int wg_per_slot = (L.d / 16) / 4;
  const long items = (long)max_slots * wg_per_slot;
  return launch_pass<false>(L.down.type, a, T * 2, (int)(items < 4096 ? items : 4096), s);
}

// ---------------------------------------------------------------- fused step

namespace {

struct FusedWs {
  float* hb[2];
  uint16_t* x;  // bf16 layer input [T][d]
  DecodeWs w;
  float* logits;
  FusedPlan plan;
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
  return F;
}

}  // namespace

size_t fused_ws_bytes(int T, int d, int f, int k, int E) {
  const size_t TK = (size_t)T * k;
  return 2 * align_up((size_t)T * d * 4, 256) + align_up((size_t)T * d * 2, 256) +
         decode_ws_bytes(T, d, f, k, MOE_BF16) + align_up((size_t)T * E * 4, 256) + 256 +
         3 * align_up(TK * 4, 256) + align_up((TK + 1) * sizeof(SlotEnt), 256);
}

hipError_t launch_fused_step(const moe_layer* layers, int n_layers, float* h, int T, const FusedRecord& rec,
                             void* ws, hipStream_t s) {
  const moe_layer& L0 = layers[0];
  const int d = L0.d, f = L0.f, k = L0.k, E = L0.E;
  FusedWs F = carve_fused(ws, T, d, f, k, E);
  const int max_slots = (T * k < E ? T * k : E) + (L0.has_shared ? 1 : 0);
  const bool inline_glue = T == 1;
  const float* prev_w = nullptr;  // topk weights of the previous layer
  for (int l = 0; l < n_layers; ++l) {
    const moe_layer& L = layers[l];
    int32_t* err_word = rec.error ? rec.error + l : F.plan.error;
    // (1) glue (previous layer's combine + residual + RMSNorm) and router
    FzGlueArgs g{};
    g.d = d;
    g.T = T;
    g.k = k;
    g.has_shared = L.has_shared;
    g.h_in = l == 0 ? h : F.hb[l & 1];
    g.h_out = F.hb[(l + 1) & 1];
    g.o = l == 0 ? nullptr : F.w.o;
    g.topk_w = prev_w;
    g.rec_y = (l > 0 && rec.y) ? rec.y + (size_t)(l - 1) * T * d : nullptr;
    g.x_out = F.x;
    g.rec_x = rec.x ? rec.x + (size_t)l * T * d : nullptr;
    g.x16 = F.w.x16;
    g.xs = F.w.xs;
    g.gate_fmt = L.gate.type;
    g.eps = rec.eps;
    g.error_reset = err_word;
    FzRouteArgs ra{};
    ra.g = g;
    ra.Wr = L.router_w;
    ra.bias = L.router_bias;
    ra.E = E;
    ra.x = F.x;
    ra.logits = rec.logits ? rec.logits + (size_t)l * T * E : F.logits;
    if (inline_glue) {
      hipLaunchKernelGGL(k_fz_route<true>, dim3((E + 3) / 4), dim3(256), 0, s, ra);
    } else {
      hipLaunchKernelGGL(k_fz_glue, dim3(T), dim3(256), 0, s, g);
      hipLaunchKernelGGL(k_fz_route<false>, dim3((E + 3) / 4), dim3(256), 0, s, ra);
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
    prev_w = ga.plan.topk_w;
    {
      const int wg_per_slot = (f / 16) / (4 / ga.a.ksplit);
      const int items = max_slots * wg_per_slot;
      if (rec.events) (void)hipEventRecord(rec.events[2 * l], s);
      hipError_t err;
      switch (L.gate.type) {
        case MOE_Q8_0: err = launch_fz_gate_fmt<MOE_Q8_0>(ga, items, E, s); break;
        case MOE_IQ4_NL: err = launch_fz_gate_fmt<MOE_IQ4_NL>(ga, items, E, s); break;
        default: err = launch_fz_gate_fmt<MOE_NVFP4>(ga, items, E, s); break;
      }
      if (err != hipSuccess) return err;
      if (rec.events) (void)hipEventRecord(rec.events[2 * l + 1], s);
    }
    // (3) down over the slot table, rows written at their pair's position
    {
      DecodeArgs da = down_args(L, T, F.w);
      da.slots = F.plan.slots;
      da.n_slots = F.plan.n_slots;
      da.pair_of_row = F.plan.pair_of_row;
      da.error = err_word;
      const int items = max_slots * ((d / 16) / 4);
      hipError_t err;
      switch (L.down.type) {
        case MOE_Q8_0: err = launch_fz_down_fmt<MOE_Q8_0>(da, items, s); break;
        case MOE_IQ4_NL: err = launch_fz_down_fmt<MOE_IQ4_NL>(da, items, s); break;
        default: err = launch_fz_down_fmt<MOE_NVFP4>(da, items, s); break;
      }
      if (err != hipSuccess) return err;
    }
  }
  // the last layer's combine, folded into h
  FzGlueArgs fg{};
  fg.d = d;
  fg.T = T;
  fg.k = k;
  fg.has_shared = layers[n_layers - 1].has_shared;
  fg.h_in = F.hb[n_layers & 1];
  fg.h_out = h;
  fg.o = F.w.o;
  fg.topk_w = prev_w;
  fg.rec_y = rec.y ? rec.y + (size_t)(n_layers - 1) * T * d : nullptr;
  fg.eps = rec.eps;
  hipLaunchKernelGGL(k_fz_glue, dim3(T), dim3(256), 0, s, fg);
  return hipGetLastError();
}

}  // namespace qre
