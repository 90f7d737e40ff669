// Decode / verify path of the routed experts (T <= 64 tokens): grouped
// dequantising GEMV-like products over the expert plan ("grouped kernels" of
// the device-planned MoE tail, UD-IQ2_XS (L4 fix) page, "What was changed").
//
// The work is HBM-bound: every weight byte of the active experts is read once.
// Weights are the B operand of v_mfma_f32_16x16x32_f16: each lane owns one
// weight row of a 16-row tile and a contiguous run of quant blocks, loads them
// with 128-bit loads and decodes them in registers to exact fp16 values
// (IQ4_NL codebook entries, Q8_0 int8 codes, or e2m1 * e4m3 products for the
// NVFP4-style format).  Activations are the A operand, carried as fp16 (with a
// per-token power-of-two scale) or as fp16 hi/lo pairs.  For the Q8_0 and
// IQ4_NL formats the A operand is block-diagonal: lane group G (16 lanes) only
// multiplies the block it decoded, so every 16x16 accumulator holds the partial
// sum of exactly one quant block per token and the block's fp16 scale is
// applied once per lane (fp32 FMA) after the MFMA.  The NVFP4-style block scale
// is folded into the fp16 weights (exact) and the tensor scale is applied at the
// end.  Accumulation is fp32 throughout.
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_launch.h"

namespace qre {

struct DecodeArgs {
  QMatDev mat[2];   // routed: gate, up (gate/up pass) or down (down pass)
  QMatDev smat[2];  // shared expert, same roles
  int has_shared;
  const int32_t* offsets;
  const int32_t* row_token;
  const int32_t* active;
  const int32_t* n_active;
  int32_t* error;
  int T, k;
  int P;                   // fp16 parts per column: 1 (bf16 tokens), 2 (fp32 tokens, or h hi/lo)
  int ksplit;              // waves along K per 16-row tile (1, 2, 4)
  const f16* in16;         // gate/up: X16 [T*P][d]; down: H16 [(T*k+T)*2][f]
  const float* in_scale;   // gate/up: scale of each X16 row (a power of two)
  f16* h16;                // gate/up output H16 [(T*k+T)*2][f]
  int down_type;           // gate/up: layout of H16 rows (IQ4_NL: block-permuted)
  float* o;                // down output O [(T*k+T)][d]
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

template <int FMT, int NT, bool GATEUP>
__global__ __launch_bounds__(256) void k_ffn_dq(const DecodeArgs a) {
  constexpr int EPS = (FMT == MOE_Q8_0) ? 16 : 32;  // elements per lane per step (one 16-byte load)
  constexpr int NMF = EPS / 8;                       // MFMAs per step
  constexpr bool BD = FMT != MOE_NVFP4;              // block-diagonal activations
  constexpr int CPT = BD ? 4 : 16;                   // columns per N-tile
  constexpr int NMAT = GATEUP ? 2 : 1;
  constexpr int PD = 4;                              // code loads in flight per matrix

  __shared__ f32x4 red[4][NMAT][NT][64];

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int n = lane & 15, G = lane >> 4;
  const int ksplit = a.ksplit;
  const int rt_per_wg = 4 / ksplit;
  const int rows = a.mat[0].rows, K = a.mat[0].cols;
  const int wg_per_slot = (rows / 16) / rt_per_wg;
  const int n_act = *a.n_active;
  const int total = (n_act + a.has_shared) * wg_per_slot;
  const int kpart = wid % ksplit;
  const int kw = K / ksplit;
  const int nsteps = kw / (4 * EPS);
  const int crb = code_row_bytes(FMT, K), srb = scale_row_bytes(FMT, K);
  const int P = a.P;

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int slot = item / wg_per_slot;
    const int tile = (item % wg_per_slot) * rt_per_wg + wid / ksplit;
    const bool is_sh = slot >= n_act;
    int e, row0, ncolt;
    if (!is_sh) {
      e = a.active[slot];
      row0 = a.offsets[e];
      ncolt = a.offsets[e + 1] - row0;
    } else {
      e = 0;
      row0 = a.T * a.k;
      ncolt = a.T;
    }
    const int ncol = ncolt * P;

    const uint8_t* crow[NMAT];
    const uint8_t* srow[NMAT];
    float tsc[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      const QMatDev& W = is_sh ? a.smat[m] : a.mat[m];
      const long rw = (long)e * rows + tile * 16 + n;
      crow[m] = W.codes + rw * crb;
      srow[m] = W.scales + rw * srb;
      tsc[m] = (FMT == MOE_NVFP4) ? W.ts[e] : 1.0f;
    }
    const int klane = kpart * kw + G * nsteps * EPS;  // first element of this lane's K run

    for (int c0 = 0; c0 < ncol; c0 += NT * CPT) {
      // A-operand source rows (this lane is A row m = n, K slice G)
      const f16* arow[NT];
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) {
        int col;
        bool valid;
        if constexpr (BD) {
          valid = (n >> 2) == G;
          col = c0 + jt * CPT + (n & 3);
        } else {
          valid = true;
          col = c0 + jt * CPT + n;
        }
        valid = valid && col < ncol;
        long in_row = 0;
        if (valid) {
          if constexpr (GATEUP) {
            const int tc = col / P, part = col - tc * P;
            const int t = is_sh ? tc : a.row_token[row0 + tc];
            in_row = (long)t * P + part;
          } else {
            in_row = (long)(row0 + col / 2) * 2 + (col & 1);
          }
        }
        arow[jt] = valid ? a.in16 + in_row * K + klane : nullptr;
      }

      f32x4 acc[NMAT][NT];
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) acc[m][jt] = f32x4{0.f, 0.f, 0.f, 0.f};

      // software pipeline: PD steps of codes and one step of activations ahead
      u32x4 cb[NMAT][PD];
      uint32_t sb[NMAT][PD];
      auto load_step = [&](int m, int s, u32x4& c, uint32_t& sc) {
        const int kel = klane + s * EPS;
        if constexpr (FMT == MOE_Q8_0) {
          c = *(const u32x4*)(crow[m] + kel);
          sc = ((const uint16_t*)srow[m])[kel >> 5];
        } else if constexpr (FMT == MOE_IQ4_NL) {
          c = *(const u32x4*)(crow[m] + (kel >> 1));
          sc = ((const uint16_t*)srow[m])[kel >> 5];
        } else {
          c = *(const u32x4*)(crow[m] + (kel >> 1));
          sc = ((const uint16_t*)srow[m])[kel >> 5];  // two E4M3 scales (blocks kel/16, kel/16+1)
        }
      };
      f16x8 an[NT][NMF];
      auto load_act = [&](int s, f16x8 (&dst)[NT][NMF]) {
#pragma unroll
        for (int jt = 0; jt < NT; ++jt)
#pragma unroll
          for (int i = 0; i < NMF; ++i) {
            if (arow[jt])
              dst[jt][i] = *(const f16x8*)(arow[jt] + s * EPS + 8 * i);
            else
              dst[jt][i] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
          }
      };
#pragma unroll
      for (int u = 0; u < PD; ++u)
        if (u < nsteps)
#pragma unroll
          for (int m = 0; m < NMAT; ++m) load_step(m, u, cb[m][u], sb[m][u]);
      load_act(0, an);

      for (int s0 = 0; s0 < nsteps; s0 += PD) {
#pragma unroll
        for (int u = 0; u < PD; ++u) {
          const int s = s0 + u;
          if (s < nsteps) {
            u32x4 cc[NMAT];
            uint32_t ss[NMAT];
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
              cc[m] = cb[m][u];
              ss[m] = sb[m][u];
              if (s + PD < nsteps) load_step(m, s + PD, cb[m][u], sb[m][u]);
            }
            f16x8 ac[NT][NMF];
#pragma unroll
            for (int jt = 0; jt < NT; ++jt)
#pragma unroll
              for (int i = 0; i < NMF; ++i) ac[jt][i] = an[jt][i];
            if (s + 1 < nsteps) load_act(s + 1, an);
#pragma unroll
            for (int m = 0; m < NMAT; ++m) {
              f32x4 D[NT];
#pragma unroll
              for (int jt = 0; jt < NT; ++jt) D[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int i = 0; i < NMF; ++i) {
                const f16x8 bf = decode_b<FMT>(cc[m], i, ss[m]);
#pragma unroll
                for (int jt = 0; jt < NT; ++jt)
                  D[jt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ac[jt][i], bf, D[jt], 0, 0, 0);
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
          }
        }
      }

      // block-diagonal: sum the four lane groups (one block each)
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
          for (int jt = 0; jt < NT; ++jt) red[wid][m][jt][lane] = acc[m][jt];
        __syncthreads();
        if (kpart == 0) {
          for (int q = 1; q < ksplit; ++q)
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
              for (int jt = 0; jt < NT; ++jt) acc[m][jt] += red[wid + q][m][jt][lane];
        }
        __syncthreads();
      }

      if (kpart == 0) {
        const int frow = tile * 16 + n;  // output feature of this lane
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) {
          // columns held by this lane: BD -> v = 0..3 (identical in all lane groups; group G takes
          // token slot G); dense -> 4G + v
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
            // each token column handled by exactly one lane of this row
            int col;
            if constexpr (BD) {
              if (P == 1 ? (v != G) : (v != 2 * G)) continue;
              col = c0 + jt * CPT + v;
            } else {
              if (P == 2 && (v & 1)) continue;
              col = c0 + jt * CPT + 4 * G + v;
            }
            if (col >= ncol) continue;
            const int tc = col / P;
            float val[NMAT];
#pragma unroll
            for (int m = 0; m < NMAT; ++m) val[m] = (P == 2) ? vals[m][v] + vals[m][v + 1] : vals[m][v];
            const int out_row = row0 + tc;
            if constexpr (GATEUP) {
              const int t = is_sh ? tc : a.row_token[row0 + tc];
              const float xs = a.in_scale[(long)t * P];
              const float g = val[0] * xs, u = val[1] * xs;
              const float h = silu_f(g) * u;
              if (!(fabsf(h) < 65504.0f)) atomicOr(a.error, 2);
              const f16 hi = (f16)h;
              const f16 lo = (f16)(h - (float)hi);
              const int f = rows;
              const int pos = (a.down_type == MOE_IQ4_NL) ? ((frow & ~31) + iq4_pos(frow & 31)) : frow;
              a.h16[((long)out_row * 2 + 0) * f + pos] = hi;
              a.h16[((long)out_row * 2 + 1) * f + pos] = lo;
            } else {
              a.o[(long)out_row * rows + frow] = val[0];
            }
          }
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Activation preparation: X16 rows (fp16, per-token power-of-two scale; fp32
// tokens as hi/lo pairs), in the block layout the gate/up weights decode to.
// ----------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_prep_x(const void* __restrict__ x, int x_bf16, int d, int P, int iq4_layout,
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
  // scale so that max |x| * 2^-e lies in [2^14, 2^15)
  int ex = 0;
  if (mx > 0.0f && mx < __builtin_inff()) {
    int e2;
    frexpf(mx, &e2);  // mx = m * 2^e2, m in [0.5, 1)
    ex = e2 - 15;
    ex = max(-100, min(100, ex));
  }
  const float down = ldexpf(1.0f, -ex);
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    const float v = x_bf16 ? bf16_bits_to_f32(((const uint16_t*)x)[(long)t * d + i]) : ((const float*)x)[(long)t * d + i];
    const float sv = v * down;
    const int pos = iq4_layout ? ((i & ~31) + iq4_pos(i & 31)) : i;
    const f16 hi = (f16)sv;
    x16[((long)t * P) * d + pos] = hi;
    if (P == 2) x16[((long)t * P + 1) * d + pos] = (f16)(sv - (float)hi);
  }
  if (threadIdx.x < P) xs[(long)t * P + threadIdx.x] = ldexpf(1.0f, ex);
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

template <int FMT, bool GATEUP>
hipError_t launch_fmt(const DecodeArgs& a, int ncols_max, int grid, hipStream_t s) {
  constexpr int CPT = (FMT == MOE_NVFP4) ? 16 : 4;
  const int nt = (ncols_max + CPT - 1) / CPT;
  if (nt <= 1)
    hipLaunchKernelGGL((k_ffn_dq<FMT, 1, GATEUP>), dim3(grid), dim3(256), 0, s, a);
  else if (nt <= 2)
    hipLaunchKernelGGL((k_ffn_dq<FMT, 2, GATEUP>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_ffn_dq<FMT, 4, GATEUP>), dim3(grid), dim3(256), 0, s, a);
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
  const int gate_fmt = L.gate.type, down_fmt = L.down.type;
  if (stage == kStagePrepare) {
    hipLaunchKernelGGL(k_prep_x, dim3(T), dim3(256), 0, s, c.x, c.x_dtype == MOE_BF16 ? 1 : 0, L.d, P,
                       gate_fmt == MOE_IQ4_NL ? 1 : 0, w.x16, w.xs);
    return hipGetLastError();
  }
  if (stage == kStageCombine)
    return launch_combine(w.o, 0, c.topk_w, c.p.slot_row, T, L.k, L.d, L.has_shared, c.y, c.y_dtype, s);

  const int max_slots = (T * L.k < L.E ? T * L.k : L.E) + (L.has_shared ? 1 : 0);
  DecodeArgs a{};
  a.has_shared = L.has_shared;
  a.offsets = c.p.offsets;
  a.row_token = c.p.row_token;
  a.active = c.p.active;
  a.n_active = c.p.n_active;
  a.error = c.p.error;
  a.T = T;
  a.k = L.k;
  if (stage == kStageGateUp) {
    const int eps = gate_fmt == MOE_Q8_0 ? 16 : 32;
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
    a.down_type = down_fmt;
    const int wg_per_slot = (L.f / 16) / (4 / a.ksplit);
    const long items = (long)max_slots * wg_per_slot;
    const int grid = (int)(items < 4096 ? items : 4096);
    return launch_pass<true>(gate_fmt, a, T * P, grid, s);
  }
  // down
  a.mat[0] = qmat_dev(L.down);
  if (L.has_shared) a.smat[0] = qmat_dev(L.shared_down);
  a.P = 2;
  a.ksplit = 1;
  a.in16 = w.h16;
  a.in_scale = nullptr;
  a.o = w.o;
  const int wg_per_slot = (L.d / 16) / 4;
  const long items = (long)max_slots * wg_per_slot;
  const int grid = (int)(items < 4096 ? items : 4096);
  return launch_pass<false>(down_fmt, a, T * 2, grid, s);
}

}  // namespace qre
