// Prefill path of the routed experts (T > 64): grouped GEMMs over the expert
// plan, the one place the layer is a dense contraction.  Quantised weights are
// decoded in registers to fp16 (the exact code times the block scale, rounded
// once) and multiplied with fp16 activations (tokens scaled by a power of two
// per token, so bf16 tokens are exact) on v_mfma_f32_16x16x32_f16 with fp32
// accumulation.  The device-side tile list walks (slot, M-tile) pairs, one
// slot per active expert plus the shared expert, so hot experts get many tiles
// and cold ones a single ragged tile ("device-planned MoE tail" + "grouped
// kernels", UD-IQ2_XS (L4 fix) page, "What was changed").
#include <hip/hip_runtime.h>

#include <algorithm>

#include "moe_device.h"
#include "moe_launch.h"

namespace qre {

constexpr int kBM = 128;   // plan rows per tile

// One M-tile of the grouped GEMM: its expert (-1: the shared expert), the
// slot's first plan row and row count, and the tile's first row in the slot.
struct PfTile {
  int32_t e, row0, cnt, m0;
};
// M-tiles at most: one per kBM plan rows of the routed pairs, plus one
// partial tile per active expert, plus the shared expert's.
inline int pf_tile_cap(int T, int k, int E) {
  return (T * k + kBM - 1) / kBM + (T * k < E ? T * k : E) + (T + kBM - 1) / kBM + 1;
}

struct PrefillArgs {
  QMatDev mat[2];
  QMatDev smat[2];
  int has_shared;
  const int32_t* offsets;
  const int32_t* row_token;
  const int32_t* active;
  const int32_t* n_active;
  const int32_t* mstart;   // [n_slots + 1] first M-tile of each slot
  const PfTile* tiles;     // [M-tiles] the M-tile table
  const int32_t* n_mtiles; // its length
  int T, k;
  const f16* x16;          // gate/up: scaled fp16 tokens [T][d] (weight-decode layout)
  const float* xs;         // gate/up: scale of each token row (a power of two)
  int down_type;           // gate/up: layout of the H rows
  const f16* hin;          // down: H fp16 [(T*k+T)][f]
  f16* hout;               // gate/up: H
  uint16_t* o;             // down: O bf16 [(T*k+T)][d]
  int32_t* error;
};

// Preparation, one launch: workgroups 0 .. T-1 write the scaled fp16 copy of
// their token (max |x| scaled into [2^14, 2^15), elements in the layout the
// gate/up weights decode to); workgroup T builds the tile list,
// mstart[s] = sum over earlier slots of ceil(rows / kBM), and the M-tile
// table (so that a GEMM item finds its expert and rows in one load).
template <bool XB>
__global__ __launch_bounds__(256) void k_pf_prepare(const void* __restrict__ x, int T, int d, int gate_fmt,
                                                    f16* __restrict__ x16, float* __restrict__ xs,
                                                    const int32_t* __restrict__ offsets,
                                                    const int32_t* __restrict__ active,
                                                    const int32_t* __restrict__ n_active, int has_shared,
                                                    int32_t* __restrict__ mstart, PfTile* __restrict__ tiles,
                                                    int32_t* __restrict__ n_mtiles, int k) {
  __shared__ int32_t part[256 / 64 + 1];  // scan scratch
  __shared__ float red[4];
  const int tid = threadIdx.x;
  if ((int)blockIdx.x < T) {
    const long t = blockIdx.x;
    // groups of 4 consecutive elements (one 8- or 16-byte load); the IQ4_NL
    // layout moves whole groups: group g of a block (elements 4g .. 4g + 3) lands
    // at positions 8g .. 8g + 3 (g < 4) or 8(g - 4) + 4 .. 8(g - 4) + 7
    auto ld4 = [&](int i) -> f32x4 {
      if constexpr (XB) {
        const u32x2 u = *(const u32x2*)((const uint16_t*)x + t * d + i);
        return f32x4{bf16_bits_to_f32(u.x & 0xffffu), bf16_bits_to_f32(u.x >> 16), bf16_bits_to_f32(u.y & 0xffffu),
                     bf16_bits_to_f32(u.y >> 16)};
      } else {
        return *(const f32x4*)((const float*)x + t * d + i);
      }
    };
    auto st4 = [&](int i, f32x4 v, float down) {
      const int pos = gate_fmt == MOE_IQ4_NL ? (i & ~31) + iq4_pos(i & 31) : i;  // i and pos: multiples of 4
      const f16x2 lo = {(f16)(v[0] * down), (f16)(v[1] * down)}, hi = {(f16)(v[2] * down), (f16)(v[3] * down)};
      *(u32x2*)(x16 + t * d + pos) = u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
    };
    // the token is read once: d <= 4 * 4 * 256 elements stay in registers
    constexpr int kGroups = 4;
    f32x4 v[kGroups];
    float mx = 0.0f;
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
      const int i = (tid + j * 256) * 4;
      v[j] = i < d ? ld4(i) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) mx = fmaxf(mx, fabsf(v[j][c]));
    }
    for (int i = (tid + kGroups * 256) * 4; i < d; i += 256 * 4) {
      const f32x4 u = ld4(i);
#pragma unroll
      for (int c = 0; c < 4; ++c) mx = fmaxf(mx, fabsf(u[c]));
    }
    mx = wave_max(mx);
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const int ex = x16_exponent(mx);
    const float down = ldexpf(1.0f, -ex);
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
      const int i = (tid + j * 256) * 4;
      if (i < d) st4(i, v[j], down);
    }
    for (int i = (tid + kGroups * 256) * 4; i < d; i += 256 * 4) st4(i, ld4(i), down);
    if (tid == 0) xs[t] = ldexpf(1.0f, ex);
    return;
  }
  const int n_slots = *n_active + has_shared;
  const int per = (n_slots + 255) / 256;
  const int s0 = tid * per, s1 = min(n_slots, s0 + per);
  int sum = 0;
  for (int s = s0; s < s1; ++s) {
    const int cnt = (s < *n_active) ? offsets[active[s] + 1] - offsets[active[s]] : T;
    sum += (cnt + kBM - 1) / kBM;
  }
  int total;
  int run = block_exclusive_scan<256>(sum, part, total);
  if (tid == 0) {
    mstart[n_slots] = total;
    *n_mtiles = total;
  }
  for (int s = s0; s < s1; ++s) {
    mstart[s] = run;
    const bool routed = s < *n_active;
    const int e = routed ? active[s] : -1;
    const int row0 = routed ? offsets[e] : T * k;
    const int cnt = routed ? offsets[e + 1] - row0 : T;
    for (int m0 = 0; m0 < cnt; m0 += kBM) tiles[run++] = PfTile{e, row0, cnt, m0};
  }
}

// ----------------------------------------------------------------------------
// Grouped GEMM tile: kBM = 128 plan rows (M) x 64 * NF weight rows (N), K in
// stages of 128.
//
// Activations (A operand of v_mfma_f32_16x16x32_f16) are copied global -> LDS
// by 16-byte LDS-DMA loads (no registers), double-buffered: the next stage's
// copies are in flight while the current stage computes.  The LDS tile is
// [128 rows][16 chunks of 8 elements], chunk c of row r stored at c ^ (r & 15)
// so that the 16 rows a fragment read touches fall in distinct banks; each
// lane of a copy picks the source chunk that lands at its LDS slot.
//
// Weights (B operand) never pass through LDS: lane (n, G) of a wavefront loads,
// for each of its NF row fragments, the codes of quant block G of the stage
// (row n of the fragment) and decodes them in registers to fp16; MFMA i of the
// stage takes code dword i of each lane group's block, and the A fragment
// reads the activation chunk holding the same elements (the activation rows
// are stored in the order the weights decode to).  One MFMA thus reduces over
// four blocks; the K order of a sum is immaterial to the GEMM.
//
// Four wavefronts each hold all M rows of the tile and NF = 4 weight-row
// fragments, so a decoded weight fragment feeds up to eight MFMAs and an A
// fragment read from LDS feeds four; two workgroups share a CU (IQ4_NL: at
// most 256 registers per lane), so that one wavefront's MFMAs overlap the
// other's LDS reads and weight decode on each SIMD.  A tile is computed over
// its first NMF = 2, 4 or 8 M fragments only (enough for its rows): rows past
// the slot's end in the last fragments are copied from its first row and
// never stored.
// GATEUP: wave w holds f-rows [32w, 32w+32) of the tile's 128, as two gate and
//         two up fragments, so SwiGLU is formed in registers.
// DOWN:   wave w holds 16 * NF consecutive d-rows.
// ----------------------------------------------------------------------------
constexpr int kPfBK = 128;                       // K per stage
constexpr int kPfMF = kBM / 16;                  // M fragments of a full tile
constexpr int kPfBuf = kBM * kPfBK * 2;          // bytes of one activation buffer
constexpr int kXcds = 8;                         // accelerator complex dies of an MI355X
constexpr int kPfWaves = 4;                      // wavefronts per workgroup
constexpr int kPfThreads = 64 * kPfWaves;

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
  if constexpr (FMT == MOE_Q8_0) {
    pc.c[0] = *(const u32x4*)(crow + kel);
    pc.c[1] = *(const u32x4*)(crow + kel + 16);
  } else {
    pc.c[0] = *(const u32x4*)(crow + (kel >> 1));
  }
  pc.sc = ((const uint16_t*)srow)[kel >> 5];
}

// fp16 weights of MFMA i (code dword i of the lane's block-sized chunk):
// Q8_0 / IQ4_NL: the exact code values (fp16 integers) times the fp16 block
// scale, rounded once; NVFP4: e2m1 * e4m3, exact in fp16 (the tensor scale is
// applied to the fp32 result).
template <int FMT>
__device__ __forceinline__ f16x8 pf_decode(const PfCodes<FMT>& pc, int i) {
  if constexpr (FMT == MOE_NVFP4) {
    const float sc = i < 2 ? e4m3_byte_to_f32<0>(pc.sc) : e4m3_byte_to_f32<1>(pc.sc);
    return fp4_dword_to_f16x8(pc.c[0][i], (f16)sc);
  } else {
    const f16 d = __builtin_bit_cast(f16, (uint16_t)pc.sc);
    const f16x8 dd = {d, d, d, d, d, d, d, d};
    if constexpr (FMT == MOE_IQ4_NL) return iq4_dword_to_f16x8(pc.c[0][i]) * dd;
    return q8_dwords_to_f16x8(pc.c[i >> 1][2 * (i & 1)], pc.c[i >> 1][2 * (i & 1) + 1]) * dd;
  }
}

// One work item (M-tile x N-tile) over its first NMF M fragments.
template <int FMT, bool GATEUP, int NF, int NMF>
__device__ __forceinline__ void pf_item(const PrefillArgs& a, uint8_t* sAbuf, float* s_rsx, const PfTile tl,
                                        int nt, int rows, int K) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = lane & 15, G = lane >> 4;
  const int crb = code_row_bytes(FMT, K), srb = scale_row_bytes(FMT, K);
  const int nstages = K / kPfBK;
  const f16* act = GATEUP ? a.x16 : a.hin;  // fp16 [rows][K]
  const bool is_sh = tl.e < 0;
  const int e = is_sh ? 0 : tl.e, row0 = tl.row0, cnt = tl.cnt;
  const int m0 = tl.m0;  // first row of this tile within the slot

  // A fragment of step i: row mi*16 + n, logical chunk 4G + i, stored at
  // chunk (4G + i) ^ n; the fragment index adds mi * 4096 bytes
  int aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) aoff[i] = (n * 16 + ((4 * G + i) ^ n)) * 16;

  // ---- this lane's weight rows (one per fragment)
  const uint8_t* bc[NF];
  const uint8_t* bs[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    int mi = 0, wr;
    if constexpr (GATEUP) {
      mi = f / (NF / 2);                                                       // gate, then up
      wr = nt * (kPfWaves * 8 * NF) + wid * (8 * NF) + (f % (NF / 2)) * 16 + n;  // same f-rows for both
    } else {
      wr = nt * (kPfWaves * 16 * NF) + wid * (16 * NF) + f * 16 + n;
    }
    const QMatDev& W = is_sh ? a.smat[mi] : a.mat[mi];
    const long rw = (long)e * rows + wr;
    bc[f] = W.codes + rw * crb;
    bs[f] = W.scales + rw * srb;
  }
  float tsg = 1.0f, tsu = 1.0f;  // NVFP4 tensor scales (gate, up / down)
  if constexpr (FMT == MOE_NVFP4) {
    tsg = (is_sh ? a.smat[0] : a.mat[0]).ts[e];
    if constexpr (GATEUP) tsu = (is_sh ? a.smat[1] : a.mat[1]).ts[e];
  }

  // ---- activation copies: copy c = 4q + w (wave w, q < NMF) fills LDS bytes
  // [1024c, 1024c + 1024), i.e. tile row 4c + lane/16, stored chunk lane%16 =
  // logical chunk ^ (row%16).
  int asrc[NMF];  // element offset of the source row (rows past the slot's end copy its first row)
  int acol[NMF];  // element offset of the logical chunk
#pragma unroll
  for (int q = 0; q < NMF; ++q) {
    const int r = (q * kPfWaves + wid) * 4 + (lane >> 4);
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
    uint8_t* base = sAbuf + buf * kPfBuf + wid * 1024;
#pragma unroll
    for (int q = 0; q < NMF; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(act + asrc[q] + s * kPfBK + acol[q]),
                                       (lds_void*)(base + q * kPfWaves * 1024), 16, 0, 0);
  };
  auto load_b = [&](int s, PfCodes<FMT> (&pc)[NF]) {
#pragma unroll
    for (int f = 0; f < NF; ++f) pf_load_codes<FMT>(bc[f], bs[f], s * kPfBK + 32 * G, pc[f]);
  };

  f32x4 acc[NMF][NF];
#pragma unroll
  for (int mi = 0; mi < NMF; ++mi)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[mi][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  PfCodes<FMT> pc[NF], pn[NF];
  copy_a(0, 0);
  load_b(0, pc);
  // gate/up: the token scale of tile row tid, kept for the epilogue
  float rsx = 0.0f;
  if constexpr (GATEUP) {
    if (tid < NMF * 16) {
      const int rr = m0 + tid;
      const int rs = rr < cnt ? rr : 0;
      rsx = a.xs[is_sh ? rs : a.row_token[row0 + rs]];
    }
  }
  for (int s = 0; s < nstages; ++s) {
    __builtin_amdgcn_s_waitcnt(0);  // this stage's copies and codes have landed
    __syncthreads();                // ... for every wave; the other buffer is free
    if (s + 1 < nstages) {
      copy_a(s + 1, (s + 1) & 1);
      load_b(s + 1, pn);
    }
    const uint8_t* sa = sAbuf + (s & 1) * kPfBuf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint8_t* p = sa + aoff[i];
      f16x8 bw[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) bw[f] = pf_decode<FMT>(pc[f], i);
#pragma unroll
      for (int mi = 0; mi < NMF; ++mi) {
        const f16x8 af = __builtin_bit_cast(f16x8, *(const u32x4*)(p + mi * 4096));
#pragma unroll
        for (int f = 0; f < NF; ++f)
          acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bw[f], acc[mi][f], 0, 0, 0);
      }
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) pc[f] = pn[f];
  }
  if (GATEUP && tid < NMF * 16) s_rsx[tid] = rsx;
  __syncthreads();  // the next item's first copy must not overwrite a buffer still being read

  // ---- epilogue: D row (M) = mi*16 + 4G + v, column (N) = fragment row n
  bool bad = false;  // an h value beyond fp16 range
#pragma unroll
  for (int mi = 0; mi < NMF; ++mi) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int rr = m0 + mi * 16 + 4 * G + v;
      if (rr >= cnt) continue;
      const long orow = row0 + rr;
      if constexpr (GATEUP) {
        const float sx = s_rsx[mi * 16 + 4 * G + v];
#pragma unroll
        for (int f = 0; f < NF / 2; ++f) {
          const float g = acc[mi][f][v] * sx * tsg, u = acc[mi][f + NF / 2][v] * sx * tsu;
          // silu(g) * u with the hardware reciprocal (about 1 ulp); h is then
          // rounded to fp16
          const float hv = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
          bad |= !(fabsf(hv) < 65504.0f);
          const int fcol = nt * (kPfWaves * 8 * NF) + wid * (8 * NF) + f * 16 + n;
          a.hout[orow * rows + act_pos(a.down_type, fcol)] = (f16)hv;
        }
      } else {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int dcol = nt * (kPfWaves * 16 * NF) + wid * (16 * NF) + f * 16 + n;
          a.o[orow * rows + dcol] = (uint16_t)f32_to_bf16_bits(acc[mi][f][v] * tsg);
        }
      }
    }
  }
  if (GATEUP && bad) atomicOr(a.error, 2);
}

template <int FMT, bool GATEUP, int NF>
__global__ __launch_bounds__(kPfThreads, FMT == MOE_IQ4_NL ? 2 : 1) void k_pf_gemm(const PrefillArgs a) {
  __shared__ __align__(16) uint8_t sAbuf[2 * kPfBuf];  // [2][kBM][16 chunks][16 B]
  __shared__ float s_rsx[kBM];                         // gate/up: token scale of each tile row
  const QMatDev& M0 = a.mat[0];
  const int rows = M0.rows, K = M0.cols;
  const int n_ntiles = GATEUP ? rows / (kPfWaves * 8 * NF) : rows / (kPfWaves * 16 * NF);
  const int total = *a.n_mtiles * n_ntiles;

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
    const PfTile tl = a.tiles[mt];
    const int nrow = min(kBM, tl.cnt - tl.m0);  // rows of this tile, 1 .. kBM
    if (nrow > 64)
      pf_item<FMT, GATEUP, NF, 8>(a, sAbuf, s_rsx, tl, nt, rows, K);
    else if (nrow > 32)
      pf_item<FMT, GATEUP, NF, 4>(a, sAbuf, s_rsx, tl, nt, rows, K);
    else
      pf_item<FMT, GATEUP, NF, 2>(a, sAbuf, s_rsx, tl, nt, rows, K);
  }
}

namespace {

struct PrefillWs {
  int32_t* mstart;
  PfTile* tiles;
  int32_t* n_mtiles;
  f16* h;
  uint16_t* o;
  f16* x16;   // scaled fp16 tokens
  float* xs;  // their scales
};

PrefillWs carve(void* ws, int T, int d, int f, int k, int E) {
  char* p = (char*)ws;
  PrefillWs w;
  w.mstart = (int32_t*)p;
  p += align_up((size_t)(E + 2) * 4, 256);
  w.tiles = (PfTile*)p;
  p += align_up((size_t)pf_tile_cap(T, k, E) * sizeof(PfTile), 256);
  w.n_mtiles = (int32_t*)p;
  p += 256;
  const size_t R = (size_t)T * k + T;
  w.h = (f16*)p;
  p += align_up(R * f * 2, 256);
  w.o = (uint16_t*)p;
  p += align_up(R * d * 2, 256);
  w.x16 = (f16*)p;
  p += align_up((size_t)T * d * 2, 256);
  w.xs = (float*)p;
  return w;
}

template <int FMT, bool GATEUP, int NF>
hipError_t launch_gemm_nf(const PrefillArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((k_pf_gemm<FMT, GATEUP, NF>), dim3(grid), dim3(kPfThreads), 0, s, a);
  return hipGetLastError();
}

template <int FMT, bool GATEUP>
hipError_t launch_gemm_fmt(int nf, const PrefillArgs& a, int grid, hipStream_t s) {
  if constexpr (GATEUP) return launch_gemm_nf<FMT, true, 4>(a, grid, s);  // two gate and two up fragments
  return nf == 4 ? launch_gemm_nf<FMT, false, 4>(a, grid, s) : launch_gemm_nf<FMT, false, 2>(a, grid, s);
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
  return align_up((size_t)(4096 + 2) * 4, 256) + align_up((size_t)pf_tile_cap(T, k, 4096) * sizeof(PfTile), 256) +
         256 + align_up(R * f * 2, 256) + align_up(R * d * 2, 256) +
         align_up((size_t)T * d * 2, 256) + align_up((size_t)T * 4, 256);
}

hipError_t launch_prefill_stage(int stage, const FfnCall& c, hipStream_t s) {
  const moe_layer& L = *c.L;
  const int T = c.T;
  PrefillWs w = carve(c.ws, T, L.d, L.f, L.k, 4096);
  if (stage == kStagePrepare) {
    if (c.x_dtype == MOE_BF16)
      hipLaunchKernelGGL(k_pf_prepare<true>, dim3(T + 1), dim3(256), 0, s, c.x, T, L.d, L.gate.type, w.x16, w.xs,
                         c.p.offsets, c.p.active, c.p.n_active, L.has_shared, w.mstart, w.tiles, w.n_mtiles, L.k);
    else
      hipLaunchKernelGGL(k_pf_prepare<false>, dim3(T + 1), dim3(256), 0, s, c.x, T, L.d, L.gate.type, w.x16, w.xs,
                         c.p.offsets, c.p.active, c.p.n_active, L.has_shared, w.mstart, w.tiles, w.n_mtiles, L.k);
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
  a.tiles = w.tiles;
  a.n_mtiles = w.n_mtiles;
  a.T = T;
  a.k = L.k;
  a.error = c.p.error;
  const int max_slots = (T * L.k < L.E ? T * L.k : L.E) + (L.has_shared ? 1 : 0);
  const long max_mtiles = ((long)T * L.k + kBM - 1) / kBM + max_slots + (T + kBM - 1) / kBM;
  if (stage == kStageGateUp) {
    a.mat[0] = qmat_dev(L.gate);
    a.mat[1] = qmat_dev(L.up);
    if (L.has_shared) {
      a.smat[0] = qmat_dev(L.shared_gate);
      a.smat[1] = qmat_dev(L.shared_up);
    }
    a.x16 = w.x16;
    a.xs = w.xs;
    a.down_type = L.down.type;
    a.hout = w.h;
    // two gate and two up fragments per wavefront: a tile of 128 f-rows
    const long items = max_mtiles * (L.f / 128);
    const int grid = (int)(items < 8192 ? items : 8192) / kXcds * kXcds + kXcds;
    return launch_gemm<true>(L.gate.type, 4, a, grid, s);
  }
  a.mat[0] = qmat_dev(L.down);
  if (L.has_shared) a.smat[0] = qmat_dev(L.shared_down);
  a.hin = w.h;
  a.o = w.o;
  // 256 d-rows per tile where d allows, else 128
  const int nf = (L.d % 256 == 0) ? 4 : 2;
  const long items = max_mtiles * (L.d / (64 * nf));
  const int grid = (int)(items < 8192 ? items : 8192) / kXcds * kXcds + kXcds;
  return launch_gemm<false>(L.down.type, nf, a, grid, s);
}

}  // namespace qre
