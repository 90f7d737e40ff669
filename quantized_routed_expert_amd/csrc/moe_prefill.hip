// Prefill path of the routed experts (T > 64): grouped GEMMs over the expert
// plan, the one place the layer is a dense contraction.  Tiles of quantised
// weights are dequantised to bf16 (round to nearest even of the exact value)
// into LDS and multiplied with bf16 activations on v_mfma_f32_16x16x32_bf16
// with fp32 accumulation.  The device-side tile list walks (slot, M-tile)
// pairs, one slot per active expert plus the shared expert, so hot experts get
// many tiles and cold ones a single ragged tile ("device-planned MoE tail" +
// "grouped kernels", UD-IQ2_XS (L4 fix) page, "What was changed").
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_launch.h"

namespace qre {

constexpr int kBM = 128;   // plan rows per tile
constexpr int kBK = 64;    // K per LDS stage (two quant blocks)
constexpr int kLdsK = kBK + 8;  // padded LDS row (bf16 elements)

struct PrefillArgs {
  QMatDev mat[2];
  QMatDev smat[2];
  int has_shared;
  const int32_t* offsets;
  const int32_t* row_token;
  const int32_t* active;
  const int32_t* n_active;
  const int32_t* mstart;   // [n_slots + 1] first M-tile of each slot
  int T, k;
  const void* x;           // gate/up: tokens [T][d] (bf16 or fp32)
  int x_bf16;
  const uint16_t* hin;     // down: H bf16 [(T*k+T)][f]
  uint16_t* hout;          // gate/up: H bf16
  uint16_t* o;             // down: O bf16 [(T*k+T)][d]
};

// Build the tile list: mstart[s] = sum over earlier slots of ceil(rows / kBM).
__global__ __launch_bounds__(1024) void k_pf_tiles(const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ active,
                                                   const int32_t* __restrict__ n_active, int has_shared, int T,
                                                   int32_t* __restrict__ mstart) {
  __shared__ int32_t part[1024];
  const int n_slots = *n_active + has_shared;
  const int per = (n_slots + blockDim.x - 1) / blockDim.x;
  const int s0 = threadIdx.x * per, s1 = min(n_slots, s0 + per);
  int sum = 0;
  for (int s = s0; s < s1; ++s) {
    const int cnt = (s < *n_active) ? offsets[active[s] + 1] - offsets[active[s]] : T;
    sum += (cnt + kBM - 1) / kBM;
  }
  part[threadIdx.x] = sum;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < (int)blockDim.x; ++i) {
      const int v = part[i];
      part[i] = run;
      run += v;
    }
    mstart[n_slots] = run;
  }
  __syncthreads();
  int run = part[threadIdx.x];
  for (int s = s0; s < s1; ++s) {
    mstart[s] = run;
    const int cnt = (s < *n_active) ? offsets[active[s] + 1] - offsets[active[s]] : T;
    run += (cnt + kBM - 1) / kBM;
  }
}

// Dequantise 32 elements (one 32-element group of a row) to bf16 (RNE of the
// exact value) and store them to LDS as 16 packed dwords.
template <int FMT>
__device__ __forceinline__ void dequant32_to_lds(const uint8_t* crow, const uint8_t* srow, float ts, int k0,
                                                 uint32_t* dst) {
  float v[32];
  if constexpr (FMT == MOE_IQ4_NL) {
    const u32x4 c = *(const u32x4*)(crow + (k0 >> 1));
    const float d = f16_bits_to_f32(((const uint16_t*)srow)[k0 >> 5]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x8 q = iq4_dword_to_f16x8(c[i]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[4 * i + t] = (float)q[t] * d;
        v[16 + 4 * i + t] = (float)q[4 + t] * d;
      }
    }
  } else if constexpr (FMT == MOE_Q8_0) {
    const u32x4 c0 = *(const u32x4*)(crow + k0);
    const u32x4 c1 = *(const u32x4*)(crow + k0 + 16);
    const float d = f16_bits_to_f32(((const uint16_t*)srow)[k0 >> 5]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        v[4 * i + b] = (float)(int8_t)((c0[i] >> (8 * b)) & 0xffu) * d;
        v[16 + 4 * i + b] = (float)(int8_t)((c1[i] >> (8 * b)) & 0xffu) * d;
      }
    }
  } else {
    const u32x4 c = *(const u32x4*)(crow + (k0 >> 1));
    const uint32_t sraw = ((const uint16_t*)srow)[k0 >> 5];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f16 sb = (f16)e4m3_to_f32((sraw >> (8 * h)) & 0xffu);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const f16x8 q = fp4_dword_to_f16x8(c[2 * h + i], sb);
#pragma unroll
        for (int t = 0; t < 8; ++t) v[16 * h + 8 * i + t] = (float)q[t] * ts;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) dst[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
}

__device__ __forceinline__ int find_slot(const int32_t* mstart, int n_slots, int mt) {
  int lo = 0, hi = n_slots - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mstart[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// GATEUP: N-tile = 64 gate rows + the same 64 up rows; waves split M (32 rows each).
// DOWN:   N-tile = 128 output rows; waves split M.
template <int FMT, bool GATEUP>
__global__ __launch_bounds__(256) void k_pf_gemm(const PrefillArgs a) {
  constexpr int BN = 128;  // weight rows staged per tile (gate/up: 64 + 64)
  __shared__ uint32_t sA[kBM * kLdsK / 2];
  __shared__ uint32_t sB[BN * kLdsK / 2];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = lane & 15, G = lane >> 4;
  const QMatDev& M0 = a.mat[0];
  const int rows = M0.rows, K = M0.cols;
  const int n_ntiles = GATEUP ? rows / 64 : rows / BN;
  const int n_act = *a.n_active;
  const int n_slots = n_act + a.has_shared;
  const int total = a.mstart[n_slots] * n_ntiles;
  const int crb = code_row_bytes(FMT, K), srb = scale_row_bytes(FMT, K);

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int mt = item / n_ntiles, nt = item % n_ntiles;
    const int slot = find_slot(a.mstart, n_slots, mt);
    const bool is_sh = slot >= n_act;
    int e, row0, cnt;
    if (!is_sh) {
      e = a.active[slot];
      row0 = a.offsets[e];
      cnt = a.offsets[e + 1] - row0;
    } else {
      e = 0;
      row0 = a.T * a.k;
      cnt = a.T;
    }
    const int m0 = (mt - a.mstart[slot]) * kBM;  // first row of this tile within the slot

    // ---- per-thread staging roles
    // A: 128 rows x 64 elements = 1024 chunks of 8 elements; 4 per thread
    // B: 128 weight rows x 2 groups of 32 elements; 1 per thread
    const int brow = tid >> 1, bgrp = tid & 1;
    const uint8_t* bcrow;
    const uint8_t* bsrow;
    float bts = 1.0f;
    {
      int mi = 0, wr;
      if constexpr (GATEUP) {
        mi = brow >> 6;
        wr = nt * 64 + (brow & 63);
      } else {
        wr = nt * BN + brow;
      }
      const QMatDev& W = is_sh ? a.smat[mi] : a.mat[mi];
      const long rw = (long)e * rows + wr;
      bcrow = W.codes + rw * crb;
      bsrow = W.scales + rw * srb;
      if (FMT == MOE_NVFP4) bts = W.ts[e];
    }
    // A source rows for this thread's 4 chunks
    long asrc[4];
    bool aval[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ch = tid + 256 * q;
      const int r = ch >> 3;
      const int rr = m0 + r;
      aval[q] = rr < cnt;
      long src = 0;
      if (aval[q]) {
        if constexpr (GATEUP) {
          const int t = is_sh ? rr : a.row_token[row0 + rr];
          src = (long)t * K;
        } else {
          src = (long)(row0 + rr) * K;
        }
      }
      asrc[q] = src;
    }

    f32x4 acc[2][2][4];  // [matrix or N half][M sub-tile][N sub-tile]
#pragma unroll
    for (int x0 = 0; x0 < 2; ++x0)
#pragma unroll
      for (int x1 = 0; x1 < 2; ++x1)
#pragma unroll
        for (int x2 = 0; x2 < 4; ++x2) acc[x0][x1][x2] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < K; k0 += kBK) {
      // stage A
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ch = tid + 256 * q;
        const int r = ch >> 3, c8 = (ch & 7) * 8;
        u32x4 v = {0, 0, 0, 0};
        if (aval[q]) {
          if constexpr (GATEUP) {
            if (a.x_bf16) {
              v = *(const u32x4*)((const uint16_t*)a.x + asrc[q] + k0 + c8);
            } else {
              const float* xf = (const float*)a.x + asrc[q] + k0 + c8;
              const f32x4 f0 = *(const f32x4*)xf, f1 = *(const f32x4*)(xf + 4);
              v = u32x4{pack_bf16x2(f0.x, f0.y), pack_bf16x2(f0.z, f0.w), pack_bf16x2(f1.x, f1.y),
                        pack_bf16x2(f1.z, f1.w)};
            }
          } else {
            v = *(const u32x4*)(a.hin + asrc[q] + k0 + c8);
          }
        }
        *(u32x4*)&sA[(r * kLdsK + c8) / 2] = v;
      }
      // stage B (dequantise)
      {
        uint32_t tmp[16];
        dequant32_to_lds<FMT>(bcrow, bsrow, bts, k0 + 32 * bgrp, tmp);
        uint32_t* dst = &sB[(brow * kLdsK + 32 * bgrp) / 2];
#pragma unroll
        for (int j = 0; j < 16; j += 4) *(u32x4*)&dst[j] = u32x4{tmp[j], tmp[j + 1], tmp[j + 2], tmp[j + 3]};
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < kBK; kk += 32) {
        bf16x8 af[2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
          const int r = wid * 32 + mi * 16 + n;
          af[mi] = __builtin_bit_cast(bf16x8, *(const u32x4*)&sA[(r * kLdsK + kk + 8 * G) / 2]);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) {
            const int br = h * 64 + ni * 16 + n;
            const bf16x8 bfr = __builtin_bit_cast(bf16x8, *(const u32x4*)&sB[(br * kLdsK + kk + 8 * G) / 2]);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
              acc[h][mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bfr, acc[h][mi][ni], 0, 0, 0);
          }
        }
      }
      __syncthreads();
    }

    // ---- epilogue: D row m = 4G + v of the 16x16 tile, column n
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int rr = m0 + wid * 32 + mi * 16 + 4 * G + v;
        if (rr >= cnt) continue;
        const long orow = row0 + rr;
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          if constexpr (GATEUP) {
            const float g = acc[0][mi][ni][v], u = acc[1][mi][ni][v];
            const float hv = g / (1.0f + __expf(-g)) * u;
            const int fcol = nt * 64 + ni * 16 + n;
            a.hout[orow * rows + fcol] = (uint16_t)f32_to_bf16_bits(hv);
          } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int dcol = nt * BN + h * 64 + ni * 16 + n;
              a.o[orow * rows + dcol] = (uint16_t)f32_to_bf16_bits(acc[h][mi][ni][v]);
            }
          }
        }
      }
    }
  }
}

namespace {

struct PrefillWs {
  int32_t* mstart;
  uint16_t* h;
  uint16_t* o;
};

PrefillWs carve(void* ws, int T, int d, int f, int k, int E) {
  char* p = (char*)ws;
  PrefillWs w;
  w.mstart = (int32_t*)p;
  p += align_up((size_t)(E + 2) * 4, 256);
  const size_t R = (size_t)T * k + T;
  w.h = (uint16_t*)p;
  p += align_up(R * f * 2, 256);
  w.o = (uint16_t*)p;
  return w;
}

template <bool GATEUP>
hipError_t launch_gemm(int fmt, const PrefillArgs& a, int grid, hipStream_t s) {
  switch (fmt) {
    case MOE_Q8_0: hipLaunchKernelGGL((k_pf_gemm<MOE_Q8_0, GATEUP>), dim3(grid), dim3(256), 0, s, a); break;
    case MOE_IQ4_NL: hipLaunchKernelGGL((k_pf_gemm<MOE_IQ4_NL, GATEUP>), dim3(grid), dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((k_pf_gemm<MOE_NVFP4, GATEUP>), dim3(grid), dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace

size_t prefill_ws_bytes(int T, int d, int f, int k) {
  const size_t R = (size_t)T * k + T;
  return align_up((size_t)(4096 + 2) * 4, 256) + align_up(R * f * 2, 256) + align_up(R * d * 2, 256);
}

hipError_t launch_prefill_stage(int stage, const FfnCall& c, hipStream_t s) {
  const moe_layer& L = *c.L;
  const int T = c.T;
  PrefillWs w = carve(c.ws, T, L.d, L.f, L.k, 4096);
  if (stage == kStagePrepare) {
    hipLaunchKernelGGL(k_pf_tiles, dim3(1), dim3(1024), 0, s, c.p.offsets, c.p.active, c.p.n_active, L.has_shared, T,
                       w.mstart);
    return hipGetLastError();
  }
  if (stage == kStageCombine)
    return launch_combine(w.o, 1, c.topk_w, c.p.slot_row, T, L.k, L.d, L.has_shared, c.y, c.y_dtype, s);
  PrefillArgs a{};
  a.has_shared = L.has_shared;
  a.offsets = c.p.offsets;
  a.row_token = c.p.row_token;
  a.active = c.p.active;
  a.n_active = c.p.n_active;
  a.mstart = w.mstart;
  a.T = T;
  a.k = L.k;
  const int max_slots = (T * L.k < L.E ? T * L.k : L.E) + (L.has_shared ? 1 : 0);
  const long max_mtiles = ((long)T * L.k + kBM - 1) / kBM + max_slots + (T + kBM - 1) / kBM;
  if (stage == kStageGateUp) {
    a.mat[0] = qmat_dev(L.gate);
    a.mat[1] = qmat_dev(L.up);
    if (L.has_shared) {
      a.smat[0] = qmat_dev(L.shared_gate);
      a.smat[1] = qmat_dev(L.shared_up);
    }
    a.x = c.x;
    a.x_bf16 = c.x_dtype == MOE_BF16 ? 1 : 0;
    a.hout = w.h;
    const long items = max_mtiles * (L.f / 64);
    const int grid = (int)(items < 8192 ? items : 8192);
    return launch_gemm<true>(L.gate.type, a, grid, s);
  }
  a.mat[0] = qmat_dev(L.down);
  if (L.has_shared) a.smat[0] = qmat_dev(L.shared_down);
  a.hin = w.h;
  a.o = w.o;
  const long items = max_mtiles * (L.d / 128);
  const int grid = (int)(items < 8192 ? items : 8192);
  return launch_gemm<false>(L.down.type, a, grid, s);
}

}  // namespace qre
