// Prefill path of the routed experts (T > 64): grouped GEMMs over the expert
// plan, the one place the layer is a dense contraction.  Tiles of quantised
// weights are dequantised to bf16 (round to nearest even of the exact value)
// into LDS and multiplied with bf16 activations on v_mfma_f32_16x16x32_bf16
// with fp32 accumulation.  The device-side tile list walks (slot, M-tile)
// pairs, one slot per active expert plus the shared expert, so hot experts get
// many tiles and cold ones a single ragged tile ("device-planned MoE tail" +
// "grouped kernels", UD-IQ2_XS (L4 fix) page, "What was changed").
#include <hip/hip_runtime.h>

#include <algorithm>

#include "moe_device.h"
#include "moe_launch.h"

namespace qre {

constexpr int kBM = 128;   // plan rows per tile

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

__device__ __forceinline__ int find_slot(const int32_t* mstart, int n_slots, int mt) {
  int lo = 0, hi = n_slots - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mstart[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ----------------------------------------------------------------------------
// Grouped GEMM tile: 128 plan rows (M) x 64 * NF weight rows (N), K in
// stages of 128.
//
// Activations (A operand of v_mfma_f32_16x16x32_bf16, bf16) are copied
// global -> LDS by 16-byte LDS-DMA loads (no registers), double-buffered: the
// next stage's copies are in flight while the current stage computes.  The
// LDS tile is [128 rows][16 chunks of 8 elements], chunk c of row r stored at
// c ^ (r & 15) so that the 16 rows a fragment read touches fall in distinct
// banks; each lane of a copy picks the source chunk that lands at its LDS slot.
//
// Weights (B operand) never pass through LDS: lane (n, G) of a wavefront loads,
// for each of its NF row fragments, the codes of quant block G of the stage
// (row n of the fragment) and decodes them in registers to bf16 = RNE(exact
// value); MFMA i of the stage takes elements 8i .. 8i+7 of each lane group's
// block, and the A fragment reads the matching activation chunk.  One MFMA
// thus reduces over four blocks; the K order of a sum is immaterial to the
// GEMM, so this is the plain product with exactly the oracle's bf16 weights.
//
// Eight wavefronts (two per SIMD, so that one's decode and LDS reads overlap
// the other's MFMAs) each hold all 128 M rows and NF weight-row fragments:
// GATEUP: wave w holds f-rows [16w, 16w+16) of the tile's 128, as a gate and
//         an up fragment (NF = 2), so SwiGLU is formed in registers.
// DOWN:   wave w holds 16 * NF consecutive d-rows.
// ----------------------------------------------------------------------------
constexpr int kPfBK = 128;                       // K per stage
constexpr int kPfMF = kBM / 16;                  // M fragments
constexpr int kPfBuf = kBM * kPfBK * 2;          // bytes of one activation buffer
constexpr int kXcds = 8;                         // accelerator complex dies of an MI355X
constexpr int kPfWaves = 8;                      // wavefronts per workgroup (two per SIMD)
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfCopies = kBM * kPfBK * 2 / (16 * kPfThreads);  // 16-byte copies per thread per stage

typedef __attribute__((address_space(3))) void lds_void;

// Code bytes of one lane's block-sized chunk per stage: IQ4_NL / NVFP4 16 (32
// elements), Q8_0 32.
template <int FMT>
struct PfCodes {
  u32x4 c[FMT == MOE_Q8_0 ? 2 : 1];
  uint32_t sc;  // fp16 block scale, or two E4M3 scales (NVFP4)
};

template <int FMT>
__device__ __forceinline__ void pf_load_codes(const uint8_t* crow, const uint8_t* srow, int kel, PfCodes<FMT>& pc) {
  // (non-temporal: each weight tile is read by few workgroups, close together)
  if constexpr (FMT == MOE_Q8_0) {
    pc.c[0] = __builtin_nontemporal_load((const u32x4*)(crow + kel));
    pc.c[1] = __builtin_nontemporal_load((const u32x4*)(crow + kel + 16));
  } else {
    pc.c[0] = __builtin_nontemporal_load((const u32x4*)(crow + (kel >> 1)));
  }
  pc.sc = __builtin_nontemporal_load((const uint16_t*)srow + (kel >> 5));
}

// Four biased bytes u (= value + 128) times scale d, rounded once to bf16: the
// products (u - 128) * d are exact in fp32 (at most 19 significant bits), so
// fma(u, d, -128 d) is exact and the bf16 rounding is the only one.
__device__ __forceinline__ u32x2 pf_biased4_to_bf16(uint32_t u, float d) {
  const float nd = -128.0f * d;
  const float v0 = fmaf((float)(u & 0xffu), d, nd);
  const float v1 = fmaf((float)((u >> 8) & 0xffu), d, nd);
  const float v2 = fmaf((float)((u >> 16) & 0xffu), d, nd);
  const float v3 = fmaf((float)(u >> 24), d, nd);
  return u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
}

// bf16 weights of MFMA i: elements 8i .. 8i+7 of the lane's 32-element chunk,
// in natural order.
template <int FMT>
__device__ __forceinline__ bf16x8 pf_decode(const PfCodes<FMT>& pc, int i, float ts) {
  if constexpr (FMT == MOE_IQ4_NL) {
    // elements 0..15 are the low nibbles of bytes 0..15, elements 16..31 the high ones
    const uint32_t w0 = pc.c[0][2 * (i & 1)], w1 = pc.c[0][2 * (i & 1) + 1];
    const int sh = (i >> 1) * 4;
    const float d = f16_bits_to_f32(pc.sc);
    const u32x2 a = pf_biased4_to_bf16(iq4_lookup4((w0 >> sh) & 0x0F0F0F0Fu), d);
    const u32x2 b = pf_biased4_to_bf16(iq4_lookup4((w1 >> sh) & 0x0F0F0F0Fu), d);
    return __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
  } else if constexpr (FMT == MOE_Q8_0) {
    const float d = f16_bits_to_f32(pc.sc);
    const u32x2 a = pf_biased4_to_bf16(pc.c[i >> 1][2 * (i & 1)] ^ 0x80808080u, d);
    const u32x2 b = pf_biased4_to_bf16(pc.c[i >> 1][2 * (i & 1) + 1] ^ 0x80808080u, d);
    return __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
  } else {
    // e2m1 * e4m3 is exact in fp16; times the tensor scale rounds once in fp32
    const uint32_t sbyte = (i < 2) ? (pc.sc & 0xffu) : ((pc.sc >> 8) & 0xffu);
    const f16x8 q = fp4_dword_to_f16x8(pc.c[0][i], (f16)e4m3_to_f32(sbyte));
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = pack_bf16x2((float)q[2 * j] * ts, (float)q[2 * j + 1] * ts);
    return __builtin_bit_cast(bf16x8, r);
  }
}

template <int FMT, bool GATEUP, int NF>
__global__ __launch_bounds__(kPfThreads) void k_pf_gemm(const PrefillArgs a) {
  extern __shared__ __align__(16) uint8_t sAbuf[];  // [2][kBM][16 chunks][16 B]
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = lane & 15, G = lane >> 4;
  const QMatDev& M0 = a.mat[0];
  const int rows = M0.rows, K = M0.cols;
  const int n_ntiles = GATEUP ? rows / (kPfWaves * 8 * NF) : rows / (kPfWaves * 16 * NF);
  const int n_act = *a.n_active;
  const int n_slots = n_act + a.has_shared;
  const int total = a.mstart[n_slots] * n_ntiles;
  const int crb = code_row_bytes(FMT, K), srb = scale_row_bytes(FMT, K);
  const int nstages = K / kPfBK;
  const uint16_t* act = GATEUP ? (const uint16_t*)a.x : a.hin;  // bf16 [rows][K]

  // Workgroups are dealt to the XCDs round-robin by index; each XCD takes a
  // contiguous run of items (the N-tiles of an M-tile, then the next M-tiles
  // of the same expert) so that activations and weights are shared in its L2.
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int grid_per_xcd = (int)gridDim.x / kXcds;
  const int xcd = blockIdx.x % kXcds, lane_in_xcd = blockIdx.x / kXcds;
  for (int it = lane_in_xcd; it < per_xcd; it += grid_per_xcd) {
    const int item = xcd * per_xcd + it;
    if (item >= total) break;
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

    // ---- this lane's weight rows (one per fragment)
    const uint8_t* bc[NF];
    const uint8_t* bs[NF];
    float ts[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      int mi = 0, wr;
      if constexpr (GATEUP) {
        mi = f / (NF / 2);                                                // gate, then up
        wr = nt * (kPfWaves * 8 * NF) + wid * (8 * NF) + (f % (NF / 2)) * 16 + n;   // same f-rows for both
      } else {
        wr = nt * (kPfWaves * 16 * NF) + wid * (16 * NF) + f * 16 + n;
      }
      const QMatDev& W = is_sh ? a.smat[mi] : a.mat[mi];
      const long rw = (long)e * rows + wr;
      bc[f] = W.codes + rw * crb;
      bs[f] = W.scales + rw * srb;
      ts[f] = (FMT == MOE_NVFP4) ? W.ts[e] : 1.0f;
    }

    // ---- activation copies: wave w, copy q covers LDS chunks (w*C+q)*64 + lane,
    // i.e. tile row (w*C+q)*4 + lane/16, stored chunk lane%16 = logical chunk ^ (row%16).
    int asrc[kPfCopies];   // element offset of the source row (rows past the slot's end copy its first row)
    int acol[kPfCopies];   // element offset of the logical chunk
#pragma unroll
    for (int q = 0; q < kPfCopies; ++q) {
      const int r = (wid * kPfCopies + q) * 4 + (lane >> 4);
      const int rr = m0 + r;
      const int rs = rr < cnt ? rr : 0;
      if constexpr (GATEUP) {
        const int t = is_sh ? rs : a.row_token[row0 + rs];
        asrc[q] = t * K;
      } else {
        asrc[q] = (row0 + rs) * K;
      }
      acol[q] = ((lane & 15) ^ (r & 15)) * 8;
    }
    auto copy_a = [&](int s, int buf) {
      uint8_t* base = sAbuf + buf * kPfBuf + (wid * kPfCopies) * 64 * 16;
#pragma unroll
      for (int q = 0; q < kPfCopies; ++q)
        __builtin_amdgcn_global_load_lds((const void*)(act + asrc[q] + s * kPfBK + acol[q]),
                                         (lds_void*)(base + q * 64 * 16), 16, 0, 0);
    };
    auto load_b = [&](int s, PfCodes<FMT> (&pc)[NF]) {
#pragma unroll
      for (int f = 0; f < NF; ++f) pf_load_codes<FMT>(bc[f], bs[f], s * kPfBK + 32 * G, pc[f]);
    };

    f32x4 acc[kPfMF][NF];
#pragma unroll
    for (int mi = 0; mi < kPfMF; ++mi)
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[mi][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    PfCodes<FMT> pc[NF], pn[NF];
    copy_a(0, 0);
    load_b(0, pc);
    for (int s = 0; s < nstages; ++s) {
      __builtin_amdgcn_s_waitcnt(0);  // this stage's copies and codes have landed
      __syncthreads();                // ... for every wave; the other buffer is free
      if (s + 1 < nstages) {
        copy_a(s + 1, (s + 1) & 1);
        load_b(s + 1, pn);
      }
      const uint8_t* sa = sAbuf + (s & 1) * kPfBuf;
      // Software pipeline over the stage's four MFMA steps: step i+1's A
      // fragments (LDS) and B fragments (decoded in registers) are produced
      // while step i's MFMAs run; the scheduling groups below interleave one
      // MFMA with a few VALU decode instructions and LDS reads.
      auto read_a = [&](int i, bf16x8 (&af)[kPfMF]) {
        const int c = 4 * G + i;  // logical chunk of MFMA step i
#pragma unroll
        for (int mi = 0; mi < kPfMF; ++mi)
          af[mi] = __builtin_bit_cast(bf16x8, *(const u32x4*)(sa + ((mi * 16 + n) * 16 + (c ^ n)) * 16));
      };
      bf16x8 afc[kPfMF], afn[kPfMF], bwc[NF], bwn[NF];
      read_a(0, afc);
#pragma unroll
      for (int f = 0; f < NF; ++f) bwc[f] = pf_decode<FMT>(pc[f], 0, ts[f]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < 3) {
          read_a(i + 1, afn);
#pragma unroll
          for (int f = 0; f < NF; ++f) bwn[f] = pf_decode<FMT>(pc[f], i + 1, ts[f]);
        }
#pragma unroll
        for (int mi = 0; mi < kPfMF; ++mi)
#pragma unroll
          for (int f = 0; f < NF; ++f)
            acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afc[mi], bwc[f], acc[mi][f], 0, 0, 0);
        if (i < 3) {
#pragma unroll
          for (int g = 0; g < kPfMF * NF; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // up to four VALU
            if (g % 4 == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
          }
#pragma unroll
          for (int mi = 0; mi < kPfMF; ++mi) afc[mi] = afn[mi];
#pragma unroll
          for (int f = 0; f < NF; ++f) bwc[f] = bwn[f];
        }
      }
#pragma unroll
      for (int f = 0; f < NF; ++f) pc[f] = pn[f];
    }
    __syncthreads();  // the next item's first copy must not overwrite a buffer still being read

    // ---- epilogue: D row (M) = mi*16 + 4G + v, column (N) = fragment row n
#pragma unroll
    for (int mi = 0; mi < kPfMF; ++mi) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int rr = m0 + mi * 16 + 4 * G + v;
        if (rr >= cnt) continue;
        const long orow = row0 + rr;
        if constexpr (GATEUP) {
#pragma unroll
          for (int f = 0; f < NF / 2; ++f) {
            const float g = acc[mi][f][v], u = acc[mi][f + NF / 2][v];
            const float hv = g / (1.0f + __expf(-g)) * u;
            const int fcol = nt * (kPfWaves * 8 * NF) + wid * (8 * NF) + f * 16 + n;
            a.hout[orow * rows + fcol] = (uint16_t)f32_to_bf16_bits(hv);
          }
        } else {
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            const int dcol = nt * (kPfWaves * 16 * NF) + wid * (16 * NF) + f * 16 + n;
            a.o[orow * rows + dcol] = (uint16_t)f32_to_bf16_bits(acc[mi][f][v]);
          }
        }
      }
    }
  }
}

// fp32 tokens -> bf16 (RNE), for the prefill products.
__global__ __launch_bounds__(256) void k_pf_x_bf16(const float* __restrict__ x, long n4, uint16_t* __restrict__ xb) {
  for (long i = blockIdx.x * 256L + threadIdx.x; i < n4; i += (long)gridDim.x * 256) {
    const f32x4 v = ((const f32x4*)x)[i];
    ((u32x2*)xb)[i] = u32x2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
  }
}

namespace {

struct PrefillWs {
  int32_t* mstart;
  uint16_t* h;
  uint16_t* o;
  uint16_t* xb;  // bf16 copy of fp32 tokens
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
  p += align_up(R * d * 2, 256);
  w.xb = (uint16_t*)p;
  return w;
}

constexpr size_t kPfLds = 2 * kPfBuf;  // double-buffered activation tile

template <int FMT, bool GATEUP, int NF>
hipError_t launch_gemm_nf(const PrefillArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((k_pf_gemm<FMT, GATEUP, NF>), dim3(grid), dim3(kPfThreads), kPfLds, s, a);
  return hipGetLastError();
}

template <int FMT, bool GATEUP>
hipError_t launch_gemm_fmt(int nf, const PrefillArgs& a, int grid, hipStream_t s) {
  if constexpr (GATEUP) return launch_gemm_nf<FMT, true, 2>(a, grid, s);  // a gate and an up fragment
  return nf == 2 ? launch_gemm_nf<FMT, false, 2>(a, grid, s) : launch_gemm_nf<FMT, false, 1>(a, grid, s);
}

template <bool GATEUP>
hipError_t launch_gemm(int fmt, int nf, const PrefillArgs& a, int grid, hipStream_t s) {
  switch (fmt) {
    case MOE_Q8_0: return launch_gemm_fmt<MOE_Q8_0, GATEUP>(nf, a, grid, s);
    case MOE_IQ4_NL: return launch_gemm_fmt<MOE_IQ4_NL, GATEUP>(nf, a, grid, s);
    default: return launch_gemm_fmt<MOE_NVFP4, GATEUP>(nf, a, grid, s);
  }
}

}  // namespace

size_t prefill_ws_bytes(int T, int d, int f, int k) {
  const size_t R = (size_t)T * k + T;
  return align_up((size_t)(4096 + 2) * 4, 256) + align_up(R * f * 2, 256) + align_up(R * d * 2, 256) +
         align_up((size_t)T * d * 2, 256);
}

hipError_t launch_prefill_stage(int stage, const FfnCall& c, hipStream_t s) {
  const moe_layer& L = *c.L;
  const int T = c.T;
  PrefillWs w = carve(c.ws, T, L.d, L.f, L.k, 4096);
  if (stage == kStagePrepare) {
    hipLaunchKernelGGL(k_pf_tiles, dim3(1), dim3(1024), 0, s, c.p.offsets, c.p.active, c.p.n_active, L.has_shared, T,
                       w.mstart);
    if (c.x_dtype == MOE_F32) {
      const long n4 = (long)T * L.d / 4;
      hipLaunchKernelGGL(k_pf_x_bf16, dim3((unsigned)std::min<long>((n4 + 255) / 256, 4096)), dim3(256), 0, s,
                         (const float*)c.x, n4, w.xb);
    }
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
    a.x = c.x_dtype == MOE_BF16 ? c.x : (const void*)w.xb;
    a.x_bf16 = 1;
    a.hout = w.h;
    // a gate and an up fragment per wavefront: a tile of 128 f-rows
    const long items = max_mtiles * (L.f / 128);
    const int grid = (int)(items < 8192 ? items : 8192) / kXcds * kXcds + kXcds;
    return launch_gemm<true>(L.gate.type, 2, a, grid, s);
  }
  a.mat[0] = qmat_dev(L.down);
  if (L.has_shared) a.smat[0] = qmat_dev(L.shared_down);
  a.hin = w.h;
  a.o = w.o;
  // 256 d-rows per tile where d allows, else 128
  const int nf = (L.d % 256 == 0) ? 2 : 1;
  const long items = max_mtiles * (L.d / (128 * nf));
  const int grid = (int)(items < 8192 ? items : 8192) / kXcds * kXcds + kXcds;
  return launch_gemm<false>(L.down.type, nf, a, grid, s);
}

}  // namespace qre
