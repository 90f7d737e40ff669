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
  // exact mode (batches of at most 64 tokens): gate/up writes h in fp32 and
  // the largest |h| of each row; the down pass reads h as scaled fp16 hi / lo
  // parts along a doubled K (hin rows of 2K: hi, then lo) and writes O in fp32
  float* hf;               // gate/up: h fp32 [(T*k+T)][f]
  uint32_t* hmax;          // gate/up: largest |h| of each row (float bits; zeroed by the preparation)
  const float* hx;         // down: the power of two each hin row was scaled down by
  float* of;               // down: O fp32 [(T*k+T)][d]
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
                                                    int32_t* __restrict__ n_mtiles, int k,
                                                    uint32_t* __restrict__ hmax) {
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
  if (hmax)  // exact mode: the row maxima of h start at zero
    for (int i = tid; i < T * k + T; i += 256) hmax[i] = 0u;
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
// fragment read from LDS feeds four; where the registers allow (see
// pf_min_blocks) two workgroups share a CU, so that one wavefront's MFMAs
// overlap the other's LDS reads and weight decode on each SIMD.  A tile is computed over
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

// Code bytes of one lane's block-sized chunk per stage: IQ4_NL / NVFP4 / Q5_1
// 16 (32 elements), Q8_0 32.
template <int FMT>
struct PfCodes {
  u32x4 c[FMT == MOE_Q8_0 ? 2 : 1];
  uint32_t sc;  // fp16 block scale, two E4M3 scales (NVFP4), or Q5_1's d | m << 16
  uint32_t qh;  // Q5_1: the block's high-bit word
};

// The codes and scale of element kel's block-sized chunk of a weight row:
// the row starts coff / soff bytes past the (workgroup-uniform) bases, and
// every offset is a 32-bit byte count, so that the loads can take the scalar
// base + 32-bit offset form.
template <int FMT>
__device__ __forceinline__ void pf_load_codes(const uint8_t* cbase, uint32_t coff, const uint8_t* sbase, uint32_t soff,
                                              int kel, PfCodes<FMT>& pc) {
  if constexpr (FMT == MOE_Q8_0) {
    pc.c[0] = *(const u32x4*)(cbase + (coff + (uint32_t)kel));
    pc.c[1] = *(const u32x4*)(cbase + (coff + (uint32_t)kel + 16u));
  } else {
    pc.c[0] = *(const u32x4*)(cbase + (coff + (uint32_t)(kel >> 1)));
  }
  if constexpr (FMT == MOE_Q5_1) {
    const u32x2 rec = *(const u32x2*)(sbase + (soff + (uint32_t)(kel >> 5) * 8u));
    pc.sc = rec.x;
    pc.qh = rec.y;
  } else {
    pc.sc = *(const uint16_t*)(sbase + (soff + (uint32_t)(kel >> 5) * 2u));
    pc.qh = 0u;
  }
}

// fp16 weights of MFMA i (code dword i of the lane's block-sized chunk):
// Q8_0 / IQ4_NL: the exact code values (fp16 integers) times the fp16 block
// scale, rounded once; NVFP4: e2m1 * e4m3, exact in fp16 (the tensor scale is
// applied to the fp32 result); Q5_1: d * q + m in fp16, one fused rounding.
template <int FMT>
__device__ __forceinline__ f16x8 pf_decode(const PfCodes<FMT>& pc, int i) {
  if constexpr (FMT == MOE_NVFP4) {
    const float sc = i < 2 ? e4m3_byte_to_f32<0>(pc.sc) : e4m3_byte_to_f32<1>(pc.sc);
    return fp4_dword_to_f16x8(pc.c[0][i], (f16)sc);
  } else if constexpr (FMT == MOE_Q5_1) {
    const f16 d = __builtin_bit_cast(f16, (uint16_t)(pc.sc & 0xffffu));
    const f16 m = __builtin_bit_cast(f16, (uint16_t)(pc.sc >> 16));
    const f16x8 dd = {d, d, d, d, d, d, d, d}, mm = {m, m, m, m, m, m, m, m};
    return __builtin_elementwise_fma(q5_1_dword_to_f16x8(pc.c[0][i], pc.qh, i), dd, mm);
  } else {
    const f16 d = __builtin_bit_cast(f16, (uint16_t)pc.sc);
    const f16x8 dd = {d, d, d, d, d, d, d, d};
    if constexpr (FMT == MOE_IQ4_NL) return iq4_dword_to_f16x8(pc.c[0][i]) * dd;
    return q8_dwords_to_f16x8(pc.c[i >> 1][2 * (i & 1)], pc.c[i >> 1][2 * (i & 1) + 1]) * dd;
  }
}

// The prefill weights are fp16 (code times block scale, rounded once).  A
// block scale of magnitude at or above kPfScaleMax<FMT> makes the product with
// the format's largest code magnitude (Q8_0: 128, IQ4_NL: 127) overflow fp16
// (it reaches 65520 and rounds to infinity); such scales, and non-finite ones,
// are reported through error bit 8.  NVFP4-style products (at most 6 * 448)
// are always finite.  A Q5_1 block's values d q + m lie between m (q = 0) and
// 31 d + m (q = 31); they overflow when either end reaches 65520 in
// magnitude (computed in fp32: exact, as 31 d and m are fp16 values whose sum
// near 65520 needs far fewer than 24 bits), or when d or m is not finite.
template <int FMT>
constexpr uint32_t kPfScaleMax = FMT == MOE_Q8_0 ? 0x6000u /* 512.0 */ : 0x6008u /* 516.0 */;

template <int FMT>
__device__ __forceinline__ bool pf_scale_out_of_range(const PfCodes<FMT>& pc) {
  if constexpr (FMT == MOE_NVFP4) {
    return false;
  } else if constexpr (FMT == MOE_Q5_1) {
    const float d = f16_bits_to_f32(pc.sc & 0xffffu), m = f16_bits_to_f32(pc.sc >> 16);
    return !(fmaxf(fabsf(m), fabsf(fmaf(31.0f, d, m))) < 65520.0f);
  } else {
    return (pc.sc & 0x7fffu) >= kPfScaleMax<FMT>;
  }
}

// Test hook: one expert's weights exactly as the prefill GEMM feeds them to
// the MFMA (pf_load_codes + pf_decode), one thread per 32-element chunk, in
// element order; NVFP4-style: e2m1 * e4m3 without the tensor scale.
template <int FMT>
__global__ void k_dequant_pf(QMatDev m, int expert, f16* __restrict__ dst) {
  const int rows = m.rows, cols = m.cols;
  const int nb = cols / 32;
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)rows * nb) return;
  const int r = (int)(i / nb), b = (int)(i % nb);
  const long rw = (long)expert * rows + r;
  PfCodes<FMT> pc;
  pf_load_codes<FMT>(m.codes + rw * code_row_bytes(FMT, cols), 0u, m.scales + rw * scale_row_bytes(FMT, cols), 0u,
                     b * 32, pc);
  f16* o = dst + (long)r * cols + b * 32;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f16x8 v = pf_decode<FMT>(pc, q);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      // IQ4_NL and Q5_1 decode elements 4q..4q+3 and 16+4q..16+4q+3; the others 8q..8q+7
      const int el = (FMT == MOE_IQ4_NL || FMT == MOE_Q5_1) ? (u < 4 ? 4 * q + u : 16 + 4 * q + (u - 4)) : 8 * q + u;
      o[el] = v[u];
    }
  }
}

hipError_t launch_dequant_pf(const QMatDev& m, int expert, void* dst, hipStream_t s) {
  const long total = (long)m.rows * (m.cols / 32);
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  switch (m.type) {
    case MOE_Q8_0: hipLaunchKernelGGL(k_dequant_pf<MOE_Q8_0>, grid, block, 0, s, m, expert, (f16*)dst); break;
    case MOE_IQ4_NL: hipLaunchKernelGGL(k_dequant_pf<MOE_IQ4_NL>, grid, block, 0, s, m, expert, (f16*)dst); break;
    case MOE_Q5_1: hipLaunchKernelGGL(k_dequant_pf<MOE_Q5_1>, grid, block, 0, s, m, expert, (f16*)dst); break;
    default: hipLaunchKernelGGL(k_dequant_pf<MOE_NVFP4>, grid, block, 0, s, m, expert, (f16*)dst); break;
  }
  return hipGetLastError();
}

// One work item (M-tile x N-tile) over its first NMF M fragments.
template <int FMT, bool GATEUP, int NF, int NMF, bool EXACT>
__device__ __forceinline__ void pf_item(const PrefillArgs& a, uint8_t* sA0, uint8_t* sA1, float* s_rsx,
                                        const PfTile tl, int nt, int rows, int K) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = lane & 15, G = lane >> 4;
  const int crb = code_row_bytes(FMT, K), srb = scale_row_bytes(FMT, K);
  // exact down pass: the activation rows are h's hi parts then its lo parts,
  // 2K long, against the same weights (stage s reads weight columns of
  // stage s mod K / kPfBK)
  constexpr bool KX2 = EXACT && !GATEUP;
  const int KA = KX2 ? 2 * K : K;
  const int nstages = KA / kPfBK;
  const f16* act = GATEUP ? a.x16 : a.hin;  // fp16 [rows][K]
  const bool is_sh = tl.e < 0;
  const int e = is_sh ? 0 : tl.e, row0 = tl.row0, cnt = tl.cnt;
  const int m0 = tl.m0;  // first row of this tile within the slot

  // A fragment of step i: row mi*16 + n, logical chunk 4G + i, stored at
  // chunk (4G + i) ^ n; the fragment index adds mi * 4096 bytes
  int aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) aoff[i] = (n * 16 + ((4 * G + i) ^ n)) * 16;

  // ---- this lane's weight rows (one per fragment): a workgroup-uniform base
  // per fragment (the expert, the N-tile, the fragment's first row) and one
  // per-lane row offset shared by all fragments, so that the loads take the
  // scalar base + 32-bit offset form (an expert's matrix is far below 4 GiB)
  const uint8_t* bc[NF];
  const uint8_t* bs[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    int mi = 0, wr0;
    if constexpr (GATEUP) {
      mi = f / (NF / 2);                                     // gate, then up
      wr0 = nt * (kPfWaves * 8 * NF) + (f % (NF / 2)) * 16;  // same f-rows for both
    } else {
      wr0 = nt * (kPfWaves * 16 * NF) + f * 16;
    }
    const QMatDev& W = is_sh ? a.smat[mi] : a.mat[mi];
    const long rw = (long)e * rows + wr0;
    bc[f] = W.codes + rw * crb;
    bs[f] = W.scales + rw * srb;
  }
  const int lrow = wid * (GATEUP ? 8 * NF : 16 * NF) + n;
  const uint32_t coff = (uint32_t)(lrow * crb), soff = (uint32_t)(lrow * srb);
  float tsg = 1.0f, tsu = 1.0f;  // NVFP4 tensor scales (gate, up / down)
  if constexpr (FMT == MOE_NVFP4) {
    tsg = (is_sh ? a.smat[0] : a.mat[0]).ts[e];
    if constexpr (GATEUP) tsu = (is_sh ? a.smat[1] : a.mat[1]).ts[e];
  }

  // ---- activation copies: copy c = 4q + w (wave w, q < NMF) fills LDS bytes
  // [1024c, 1024c + 1024), i.e. tile row 4c + lane/16, stored chunk lane%16 =
  // logical chunk ^ (row%16).
  // byte offset of the source row (rows past the slot's end copy its first
  // row) plus that of the lane's logical chunk, (lane % 16) ^ (r % 16), where
  // r % 16 is the same for every q
  uint32_t asrc[NMF];
  const uint32_t acol = (uint32_t)(((lane & 15) ^ ((wid * 4 + (lane >> 4)) & 15)) * 16);
#pragma unroll
  for (int q = 0; q < NMF; ++q) {
    const int r = (q * kPfWaves + wid) * 4 + (lane >> 4);
    const int rr = m0 + r;
    const int rs = rr < cnt ? rr : 0;
    if constexpr (GATEUP) {
      const int t = is_sh ? rs : a.row_token[row0 + rs];
      asrc[q] = (uint32_t)t * (uint32_t)(2 * K) + acol;
    } else {
      asrc[q] = (uint32_t)(row0 + rs) * (uint32_t)(2 * KA) + acol;
    }
  }
  auto copy_a = [&](int s, uint8_t* buf) {
    uint8_t* base = buf + wid * 1024;
#pragma unroll
    for (int q = 0; q < NMF; ++q)
      __builtin_amdgcn_global_load_lds((const void*)((const uint8_t*)act + (asrc[q] + (uint32_t)(s * 2 * kPfBK))),
                                       (lds_void*)(base + q * kPfWaves * 1024), 16, 0, 0);
  };
  auto load_b = [&](int s, PfCodes<FMT> (&pc)[NF]) {
#pragma unroll
    for (int f = 0; f < NF; ++f)
      pf_load_codes<FMT>(bc[f], coff, bs[f], soff, (KX2 ? (s * kPfBK) % K : s * kPfBK) + 32 * G, pc[f]);
  };

  f32x4 acc[NMF][NF];
#pragma unroll
  for (int mi = 0; mi < NMF; ++mi)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[mi][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  PfCodes<FMT> pc[NF], pn[NF];
  bool wbad = false;  // a block scale beyond the fp16 weight range
  copy_a(0, sA0);
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
  // One stage: its activations in `cur`, its codes in `pcur`; the next
  // stage's copies go to `nxt` and its codes to `pnxt`.  The two buffers are
  // distinct LDS objects and each call names them statically (the stage loop
  // runs in pairs), so the compiler sees that the copies in flight write the
  // other buffer and lets this stage's LDS reads run ahead of them.
  auto stage = [&](int s, const uint8_t* cur, uint8_t* nxt, PfCodes<FMT>(&pcur)[NF], PfCodes<FMT>(&pnxt)[NF]) {
    __builtin_amdgcn_s_waitcnt(0);  // this stage's copies and codes have landed
    __syncthreads();                // ... for every wave; the other buffer is free
    if (s + 1 < nstages) {
      copy_a(s + 1, nxt);
      load_b(s + 1, pnxt);
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) wbad |= pf_scale_out_of_range<FMT>(pcur[f]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint8_t* p = cur + aoff[i];
      f16x8 bw[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) bw[f] = pf_decode<FMT>(pcur[f], i);
#pragma unroll
      for (int mi = 0; mi < NMF; ++mi) {
        const f16x8 af = __builtin_bit_cast(f16x8, *(const u32x4*)(p + mi * 4096));
#pragma unroll
        for (int f = 0; f < NF; ++f)
          acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bw[f], acc[mi][f], 0, 0, 0);
      }
      // Q8_0: one sub-step's decoded weights at a time (decoding ahead holds
      // more registers than the kernel has)
      if constexpr (FMT == MOE_Q8_0) __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int s = 0; s < nstages; s += 2) {
    stage(s, sA0, sA1, pc, pn);
    if (s + 1 < nstages) stage(s + 1, sA1, sA0, pn, pc);
  }
  if (GATEUP && tid < NMF * 16) s_rsx[tid] = rsx;
  __syncthreads();  // every wave is done with the activation buffers: they stage the outputs now

  if constexpr (EXACT) {
    // ---- exact mode (few rows): fp32 outputs stored directly.  D row (M) =
    // mi*16 + 4G + v, column (N) = fragment row n.
    bool bad = false;  // an h value that is not finite
#pragma unroll
    for (int mi = 0; mi < NMF; ++mi) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int rr = m0 + mi * 16 + 4 * G + v;
        const bool valid = rr < cnt;
        const long orow = row0 + (valid ? rr : 0);
        if constexpr (GATEUP) {
          const float sx = s_rsx[mi * 16 + 4 * G + v];
          uint32_t mb = 0u;
#pragma unroll
          for (int f = 0; f < NF / 2; ++f) {
            const float g = acc[mi][f][v] * sx * tsg, u = acc[mi][f + NF / 2][v] * sx * tsu;
            const float hv = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
            const int fcol = nt * (kPfWaves * 8 * NF) + wid * (8 * NF) + f * 16 + n;
            if (valid) {
              bad |= !(fabsf(hv) <= 3.4028235e38f);
              a.hf[orow * rows + act_pos(a.down_type, fcol)] = hv;
              mb = max(mb, __float_as_uint(fabsf(hv)));
            }
          }
          // the row's largest |h| over this wavefront's 32 features (the 16
          // lanes of a row group), one atomic maximum per row and wavefront
          mb = max(mb, dpp_u32<kDppShr1, 0xf>(mb));
          mb = max(mb, dpp_u32<kDppShr2, 0xf>(mb));
          mb = max(mb, dpp_u32<kDppShr4, 0xf>(mb));
          mb = max(mb, dpp_u32<kDppShr8, 0xf>(mb));
          if (n == 15 && valid) atomicMax(&a.hmax[orow], mb);
        } else {
          const float hx = valid ? a.hx[orow] : 0.0f;
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            const int dcol = nt * (kPfWaves * 16 * NF) + wid * (16 * NF) + f * 16 + n;
            if (valid) a.of[orow * rows + dcol] = acc[mi][f][v] * tsg * hx;
          }
        }
      }
    }
    if (GATEUP && bad) atomicOr(a.error, 2);
    __syncthreads();  // the next item's first copy must not overwrite s_rsx still being read
    return;
  }

  // ---- epilogue: D row (M) = mi*16 + 4G + v, column (N) = fragment row n.
  // The item's outputs (tile rows x NC columns, 16-bit) are staged in the
  // activation buffers (rows [0, RPB) in sA0, the rest in sA1), then written
  // out as whole 16-byte pieces of rows: an output row's NC columns are
  // contiguous (h: positions of the down weights' decode order, which permutes
  // within blocks of 32 only; o: in order).
  constexpr int NC = GATEUP ? kPfWaves * 8 * NF : kPfWaves * 16 * NF;
  constexpr int RPB = kPfBuf / (NC * 2);
  // the lane's indices, formed here: positions derived from threadIdx.x
  // alone would otherwise be hoisted out of the item loop and held (spilled)
  // for the whole kernel
  int et = threadIdx.x;
  asm volatile("" : "+v"(et));
  const int en = et & 15, eG = (et & 63) >> 4, ewid = et >> 6;
  auto stage_at = [&](int r, int c) -> uint16_t* {
    uint8_t* b = r < RPB ? sA0 : sA1;
    return (uint16_t*)(b + ((r % RPB) * NC + c) * 2);
  };
  bool bad = false;  // an h value beyond fp16 range
#pragma unroll
  for (int mi = 0; mi < NMF; ++mi) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = mi * 16 + 4 * eG + v;
      const bool valid = m0 + r < cnt;
      if constexpr (GATEUP) {
        const float sx = s_rsx[r];
#pragma unroll
        for (int f = 0; f < NF / 2; ++f) {
          const float g = acc[mi][f][v] * sx * tsg, u = acc[mi][f + NF / 2][v] * sx * tsu;
          // silu(g) * u with the hardware reciprocal (about 1 ulp); h is then
          // rounded to fp16
          const float hv = g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
          bad |= valid && !(fabsf(hv) < 65504.0f);
          const int c = act_pos(a.down_type, ewid * (8 * NF) + f * 16 + en);
          *stage_at(r, c) = __builtin_bit_cast(uint16_t, (f16)hv);
        }
      } else {
#pragma unroll
        for (int f = 0; f < NF; ++f)
          *stage_at(r, ewid * (16 * NF) + f * 16 + en) = (uint16_t)f32_to_bf16_bits(acc[mi][f][v] * tsg);
      }
    }
  }
  __syncthreads();
  {
    constexpr int CPR = NC * 2 / 16;  // 16-byte pieces of an output row
    const int nvalid = min(NMF * 16, cnt - m0);
    uint16_t* out = GATEUP ? (uint16_t*)a.hout : a.o;
    for (int i = et; i < nvalid * CPR; i += kPfThreads) {
      const int r = i / CPR, c = i % CPR;
      *(u32x4*)(out + (long)(row0 + m0 + r) * rows + nt * NC + c * 8) = *(const u32x4*)stage_at(r, c * 8);
    }
  }
  __syncthreads();  // the next item's first copy must not overwrite a staging buffer still being read
  if (GATEUP && bad) atomicOr(a.error, 2);
  if (__any(wbad) && lane == 0) atomicOr(a.error, 8);
}

// Workgroups per CU the register budget is cut for: two where the kernel fits
// 256 registers a lane without spilling (IQ4_NL, NVFP4-style, Q5_1), else one
// (Q8_0: its 32-byte code records; the accumulators then live in AGPRs).
template <int FMT, bool GATEUP>
constexpr int pf_min_blocks() {
  return FMT == MOE_Q8_0 ? 1 : 2;
}

template <int FMT, bool GATEUP, int NF, bool EXACT>
__global__ __launch_bounds__(kPfThreads, (pf_min_blocks<FMT, GATEUP>())) void k_pf_gemm(const PrefillArgs a) {
  // the two activation buffers, [kBM][16 chunks][16 B] each
  __shared__ __align__(16) uint8_t sA0[kPfBuf];
  __shared__ __align__(16) uint8_t sA1[kPfBuf];
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
    PfTile tl = a.tiles[mt];
    // (the entry is the workgroup's: keep it in scalar registers)
    tl.e = __builtin_amdgcn_readfirstlane(tl.e);
    tl.row0 = __builtin_amdgcn_readfirstlane(tl.row0);
    tl.cnt = __builtin_amdgcn_readfirstlane(tl.cnt);
    tl.m0 = __builtin_amdgcn_readfirstlane(tl.m0);
    const int nrow = min(kBM, tl.cnt - tl.m0);  // rows of this tile, 1 .. kBM
    if (nrow > 64)
      pf_item<FMT, GATEUP, NF, 8, EXACT>(a, sA0, sA1, s_rsx, tl, nt, rows, K);
    else if (nrow > 32)
      pf_item<FMT, GATEUP, NF, 4, EXACT>(a, sA0, sA1, s_rsx, tl, nt, rows, K);
    else
      pf_item<FMT, GATEUP, NF, 2, EXACT>(a, sA0, sA1, s_rsx, tl, nt, rows, K);
  }
}

// Exact mode, between the passes: each h row scaled by a power of two (its
// largest |h| into [2^14, 2^15)) and split into fp16 hi and lo parts, hi
// then lo along a row of 2f (the down pass's activation row), and the power
// of two kept for the down pass's outputs.  Rows the plan left unused hold
// stale values and are never read.
__global__ __launch_bounds__(256) void k_pf_split_h(const float* __restrict__ hf, const uint32_t* __restrict__ hmax,
                                                    int f, f16* __restrict__ h2, float* __restrict__ hx) {
  const long r = blockIdx.x;
  const int ex = x16_exponent(__uint_as_float(hmax[r]));
  const float down = ldexpf(1.0f, -ex);
  for (int c = threadIdx.x; c < f; c += 256) {
    const float v = hf[r * f + c] * down;
    const f16 hi = (f16)v;
    h2[r * 2 * f + c] = hi;
    h2[r * 2 * f + f + c] = (f16)(v - (float)hi);
  }
  if (threadIdx.x == 0) hx[r] = ldexpf(1.0f, ex);
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
  // exact mode
  float* hf;       // h fp32 [R][f]
  uint32_t* hmax;  // [R]
  float* hx;       // [R]
  float* of;       // O fp32 [R][d]
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
  w.hf = nullptr;
  w.hmax = nullptr;
  w.hx = nullptr;
  w.of = nullptr;
  return w;
}

// Exact mode: the tile table, then h fp32, h as hi / lo fp16 rows of 2f (in
// the place of the fp16 H), the row maxima and scales, O fp32 (in the place
// of the bf16 O), the tokens.
PrefillWs carve_exact(void* ws, int T, int d, int f, int k, int E) {
  char* p = (char*)ws;
  PrefillWs w;
  w.mstart = (int32_t*)p;
  p += align_up((size_t)(E + 2) * 4, 256);
  w.tiles = (PfTile*)p;
  p += align_up((size_t)pf_tile_cap(T, k, E) * sizeof(PfTile), 256);
  w.n_mtiles = (int32_t*)p;
  p += 256;
  const size_t R = (size_t)T * k + T;
  w.hf = (float*)p;
  p += align_up(R * f * 4, 256);
  w.h = (f16*)p;
  p += align_up(R * f * 4, 256);
  w.hmax = (uint32_t*)p;
  p += align_up(R * 4, 256);
  w.hx = (float*)p;
  p += align_up(R * 4, 256);
  w.of = (float*)p;
  w.o = nullptr;
  p += align_up(R * d * 4, 256);
  w.x16 = (f16*)p;
  p += align_up((size_t)T * d * 2, 256);
  w.xs = (float*)p;
  return w;
}

template <int FMT, bool GATEUP, int NF, bool EXACT = false>
hipError_t launch_gemm_nf(const PrefillArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((k_pf_gemm<FMT, GATEUP, NF, EXACT>), dim3(grid), dim3(kPfThreads), 0, s, a);
  return hipGetLastError();
}

template <int FMT, bool GATEUP, bool EXACT = false>
hipError_t launch_gemm_fmt(int nf, const PrefillArgs& a, int grid, hipStream_t s) {
  // gate/up: two gate and two up fragments (NF = 4), or one of each (NF = 2)
  if constexpr (GATEUP && !EXACT)
    return launch_gemm_nf<FMT, true, 4, false>(a, grid, s);
  else
    return nf == 4 ? launch_gemm_nf<FMT, GATEUP, 4, EXACT>(a, grid, s) : launch_gemm_nf<FMT, GATEUP, 2, EXACT>(a, grid, s);
}

template <bool GATEUP>
hipError_t launch_gemm(int fmt, int nf, const PrefillArgs& a, int grid, hipStream_t s, bool exact) {
  if (exact) return launch_gemm_fmt<MOE_NVFP4, GATEUP, true>(nf, a, grid, s);  // (NVFP4-style only)
  switch (fmt) {
    case MOE_Q8_0: return launch_gemm_fmt<MOE_Q8_0, GATEUP>(nf, a, grid, s);
    case MOE_IQ4_NL: return launch_gemm_fmt<MOE_IQ4_NL, GATEUP>(nf, a, grid, s);
    case MOE_Q5_1:
      if constexpr (!GATEUP) return launch_gemm_fmt<MOE_Q5_1, false>(nf, a, grid, s);
      return hipErrorInvalidValue;  // a down format only
    default: return launch_gemm_fmt<MOE_NVFP4, GATEUP>(nf, a, grid, s);
  }
}

}  // namespace

// The exact mode of the prefill GEMMs serves batches of the per-layer path
// (at most kDecodeMaxT tokens) where it is faster than the decode kernels:
// NVFP4-style weights (exact in fp16, so the GEMMs' only roundings are the
// ones the decode path makes too), bf16 tokens (exact as scaled fp16), and
// more than kPfExactMinT tokens (measured crossover, 8-layer stacks of
// d = 3072, f = 768, E = 512, top-8 + shared, µs per layer, decode kernels /
// exact mode: 24 tokens 96.7 / 100.6, 32 tokens 107.8 / 105.9, 64 tokens
// 154.6 / 124.6).
constexpr int kPfExactMinT = 28;
bool prefill_exact(const moe_layer& L, int T, int x_dtype) {
  return T > kPfExactMinT && T <= kDecodeMaxT && x_dtype == MOE_BF16 && L.gate.type == MOE_NVFP4 &&
         L.up.type == MOE_NVFP4 && L.down.type == MOE_NVFP4 && L.d % 128 == 0 && L.f % 128 == 0;
}

size_t prefill_exact_ws_bytes(int T, int d, int f, int k) {
  const size_t R = (size_t)T * k + T;
  return align_up((size_t)(4096 + 2) * 4, 256) + align_up((size_t)pf_tile_cap(T, k, 4096) * sizeof(PfTile), 256) +
         256 + 2 * align_up(R * f * 4, 256) + 2 * align_up(R * 4, 256) + align_up(R * d * 4, 256) +
         align_up((size_t)T * d * 2, 256) + align_up((size_t)T * 4, 256);
}

size_t prefill_ws_bytes(int T, int d, int f, int k) {
  const size_t R = (size_t)T * k + T;
  return align_up((size_t)(4096 + 2) * 4, 256) + align_up((size_t)pf_tile_cap(T, k, 4096) * sizeof(PfTile), 256) +
         256 + align_up(R * f * 2, 256) + align_up(R * d * 2, 256) +
         align_up((size_t)T * d * 2, 256) + align_up((size_t)T * 4, 256);
}

hipError_t launch_prefill_stage(int stage, const FfnCall& c, hipStream_t s) {
  const moe_layer& L = *c.L;
  const int T = c.T;
  const bool exact = prefill_exact(L, T, c.x_dtype);
  PrefillWs w = exact ? carve_exact(c.ws, T, L.d, L.f, L.k, 4096) : carve(c.ws, T, L.d, L.f, L.k, 4096);
  if (stage == kStagePrepare) {
    if (c.x_dtype == MOE_BF16)
      hipLaunchKernelGGL(k_pf_prepare<true>, dim3(T + 1), dim3(256), 0, s, c.x, T, L.d, L.gate.type, w.x16, w.xs,
                         c.p.offsets, c.p.active, c.p.n_active, L.has_shared, w.mstart, w.tiles, w.n_mtiles, L.k,
                         w.hmax);
    else
      hipLaunchKernelGGL(k_pf_prepare<false>, dim3(T + 1), dim3(256), 0, s, c.x, T, L.d, L.gate.type, w.x16, w.xs,
                         c.p.offsets, c.p.active, c.p.n_active, L.has_shared, w.mstart, w.tiles, w.n_mtiles, L.k,
                         w.hmax);
    return hipGetLastError();
  }
  if (stage == kStageCombine) {
    if (exact) return launch_combine(w.of, 0, c.topk_w, c.p.slot_row, T, L.k, L.d, L.has_shared, c.y, c.y_dtype, s);
    return launch_combine(w.o, 1, c.topk_w, c.p.slot_row, T, L.k, L.d, L.has_shared, c.y, c.y_dtype, s);
  }
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
    a.hf = w.hf;
    a.hmax = w.hmax;
    // two gate and two up fragments per wavefront: a tile of 128 f-rows (exact
    // mode, few rows: one of each, 64 f-rows, twice the items)
    const int nfg = exact ? 2 : 4;
    const long items = max_mtiles * (L.f / (32 * nfg));
    const int grid = (int)(items < 8192 ? items : 8192) / kXcds * kXcds + kXcds;
    return launch_gemm<true>(L.gate.type, nfg, a, grid, s, exact);
  }
  if (exact) {
    hipLaunchKernelGGL(k_pf_split_h, dim3(T * L.k + T), dim3(256), 0, s, w.hf, w.hmax, L.f, w.h, w.hx);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  a.mat[0] = qmat_dev(L.down);
  if (L.has_shared) a.smat[0] = qmat_dev(L.shared_down);
  a.hin = w.h;
  a.o = w.o;
  a.hx = w.hx;
  a.of = w.of;
  // 256 d-rows per tile where d allows, else 128
  const int nf = (L.d % 256 == 0 && !exact) ? 4 : 2;
  const long items = max_mtiles * (L.d / (64 * nf));
  const int grid = (int)(items < 8192 ? items : 8192) / kXcds * kXcds + kXcds;
  return launch_gemm<false>(L.down.type, nf, a, grid, s, exact);
}

}  // namespace qre
