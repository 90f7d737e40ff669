// Decode tile code shared by the per-layer decode / verify path (T <= 64
// tokens, moe_decode.hip) and the fused decode step (moe_fused.hip): grouped
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
// Also here: the host-side workspace layout and launch-shape helpers.
#pragma once
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
  // per-layer path: plan in global memory
  const int32_t* offsets;
  const int32_t* row_token;
  const int32_t* active;
  const int32_t* n_active;
  // slot table (the shared expert first; per-layer path: then the active
  // experts by descending token count) and its length
  const SlotEnt* slots;
  const int32_t* n_slots;
  int32_t* error;
  int T, k;
  int P;                   // fp16 parts per column: 1 (bf16 tokens), 2 (fp32 tokens, or h hi/lo)
  int ksplit;              // waves along K per 16-row tile (1, 2, 4)
  const f16* in16;         // gate/up: X16 [T*P][d]
  const float* in_scale;   // gate/up: scale of each X16 row (a power of two)
  // SwiGLU rows: the gate/up pass writes h in fp32 (positions in the down
  // weights' decode order) and the largest |h| of each row over each of its
  // 16-feature tiles (float bits); the down pass stages h scaled by a power
  // of two per row as fp16 hi / lo parts and applies the power of two to its
  // result
  float* hf;               // [(T*k+T)][f]
  uint32_t* hmax;          // [(T*k+T)][f / 16]
  int down_type;           // gate/up: layout of the h rows (IQ4_NL, Q5_1: block-permuted)
  float* o;                // down output O [(T*k+T)][d]
  const int32_t* pair_of_row;  // fused down pass: O row of each plan row (t*k + j); null: the plan row
  // fused down pass: the combine, formed by the last workgroup of each
  // 64-column tile: r_out = r_in + y with y = o[T*k + t] + sum_j gate_w[t][j] *
  // o[t*k + j], and each tile's sum of squares of r_out
  int32_t* tile_cnt;       // [d/64] workgroups finished per tile (0 on entry, left 0)
  const float* r_in;
  float* r_out;
  float* ss_part;          // [T][d/64]
  float* rec_y;            // optional record of y
  const float* gate_w;     // [T][k]
};

// Kernel arguments are fetched through the scalar cache at their first use;
// a first use inside the item path puts a memory round trip on every item's
// critical path.  Touching every field the item path reads at kernel entry
// fetches them all together, once.
template <typename V>
__device__ __forceinline__ void pin_arg(V v) {
  asm volatile("" ::"s"(v));
}

__device__ __forceinline__ void dq_pin_args(const DecodeArgs& a) {
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    pin_arg(a.mat[m].codes);
    pin_arg(a.mat[m].scales);
    pin_arg(a.mat[m].ts);
    pin_arg(a.smat[m].codes);
    pin_arg(a.smat[m].scales);
    pin_arg(a.smat[m].ts);
  }
  pin_arg(a.mat[0].rows);
  pin_arg(a.mat[0].cols);
  pin_arg(a.has_shared);
  pin_arg(a.T);
  pin_arg(a.k);
  pin_arg(a.P);
  pin_arg(a.ksplit);
  pin_arg(a.down_type);
  pin_arg(a.in16);
  pin_arg(a.in_scale);
  pin_arg(a.hf);
  pin_arg(a.hmax);
  pin_arg(a.o);
  pin_arg(a.pair_of_row);
  pin_arg(a.error);
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// Weights of MFMA i of a step (code dword i of the lane's chunk): exact fp16
// values; for NVFP4-style with the block scale folded in (exact); for Q5_1
// the codes q (the block's d and m apply after the MFMA; qh: its high-bit word).
template <int FMT>
__device__ __forceinline__ f16x8 decode_b(const u32x4& c, int i, uint32_t sraw, uint32_t qh = 0u) {
  if constexpr (FMT == MOE_IQ4_NL) {
    return iq4_dword_to_f16x8(c[i]);
  } else if constexpr (FMT == MOE_Q8_0) {
    return q8_dwords_to_f16x8(c[2 * i], c[2 * i + 1]);
  } else if constexpr (FMT == MOE_Q5_1) {
    return q5_1_dword_to_f16x8(c[i], qh, i);
  } else {
    // dwords 0,1 hold the chunk's first 16-element block, 2,3 the second
    const float sc = i < 2 ? e4m3_byte_to_f32<0>(sraw) : e4m3_byte_to_f32<1>(sraw);
    return fp4_dword_to_f16x8(c[i], (f16)sc);
  }
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
// workgroup's dynamic LDS: the activation staging buffer (which also holds the
// [4][NMAT][NT][64] partial sums of the K reduction), then the scale rows.
// Steps of weight codes in flight per matrix (and per wave): the gate/up pass
// keeps two matrices' codes in registers, the down pass one (more steps for
// the 16-element steps of Q8_0).  A pass with more steps than that rolls the
// prefetch forward (ROLL); otherwise every code load is issued up front.
constexpr int dq_pd(int fmt, bool gateup) { return (!gateup && fmt == MOE_Q8_0) ? 12 : 6; }
constexpr int dq_eps(int fmt) { return fmt == MOE_Q8_0 ? 16 : 32; }  // elements per lane per step
inline int dq_nsteps(int fmt, int K, int ksplit) { return K / ksplit / (4 * dq_eps(fmt)); }

// PAIRS (down pass of the fused step): routed rows are written at the output
// row pair_of_row gives their plan row.
template <int FMT, int NT, bool GATEUP, bool ROLL, bool PAIRS = false, bool REUSE = false, bool GATHER = false>
__device__ __forceinline__ void dq_item(const DecodeArgs& a, const SlotInfo& si, int tile, int kpart,
                                        const int32_t* row_token, f16* sA) {
  // one word per column of a pass for the epilogue: the token's activation
  // scale (gate/up) or the output row (PAIRS)
  __shared__ uint32_t s_colw[4 * 8];
  __shared__ uint32_t s_colx[4 * 8];  // down pass: the power of two of each column's row
  __shared__ float s_tdown[4 * 4];    // ... and its inverse, by row of the pass (at most CPP / 2 = 16)
  constexpr int AST = GATEUP ? 1 : 2;  // down pass: hi / lo parts interleaved in 8-element runs
  constexpr int EPS = dq_eps(FMT);                   // elements per lane per step (one 16-byte load)
  constexpr int NMF = EPS / 8;                       // MFMAs per step
  constexpr bool BD = FMT != MOE_NVFP4;              // block-diagonal activations
  constexpr int CPT = cols_per_tile<FMT>();
  constexpr int CPP = NT * CPT;                      // columns staged per pass
  constexpr int NMAT = GATEUP ? 2 : 1;
  constexpr int PD = dq_pd(FMT, GATEUP);             // steps of codes in flight per matrix
  constexpr int AB = NT == 1 ? 2 : 12;               // activation chunks per thread issued first
  constexpr int RB = NT == 1 ? 2 : 8;                // later activation chunks in flight per thread

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
  const uint8_t* sreg[NMAT];  // the workgroup's scale rows (contiguous)
  float tsc[NMAT];
  const int wg_rows = 64 / ksplit;            // rows of the workgroup's tiles
  const int tile0 = tile - wid / ksplit;      // its first tile
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
    const QMatDev& W = si.is_sh ? a.smat[m] : a.mat[m];
    const long rw = (long)si.e * rows + tile * 16 + n;
    crow[m] = W.codes + rw * crb;
    sreg[m] = W.scales + ((long)si.e * rows + tile0 * 16) * srb;
    tsc[m] = (FMT == MOE_NVFP4) ? W.ts[si.e] : 1.0f;
  }
  // K position of this lane at step s: the four lane groups take four
  // consecutive EPS-element chunks, so a row's 16-byte code loads are
  // contiguous across the lane groups (64 bytes per row per step).
  const int kbase = kpart * kw + G * EPS;

  // gate/up input row of column `col` (a token, or one fp16 part of it).
  // GATHER (per-layer path): the preparation wrote the gate/up input in
  // plan-row order (rows T*k + t: the shared expert's), so a slot's rows are
  // consecutive; fused path: one row per token, found through the plan.
  auto in_row_of = [&](int col) -> long {
    const int tc = col / P, part = col - tc * P;
    if constexpr (GATHER) return (long)(si.row0 + tc) * P + part;
    const int t = si.is_sh ? tc : row_token[si.row0 + tc];
    return (long)t * P + part;
  };

  const int chunks_per_col = K / 8;  // 16-byte activation chunks per column
  // All global loads below are unconditional (out-of-range ones repeat a valid
  // address and their result is discarded), so the waits that follow them are
  // exact: data issued earlier never waits for data issued later.
  // this lane's code and scale addresses at step 0; step s adds a constant
  // (4 * EPS elements: 64 code bytes, 4 * EPS / 32 scale words)
  const uint8_t* cl[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m) cl[m] = crow[m] + (FMT == MOE_Q8_0 ? kbase : (kbase >> 1));
  // Weight codes are read once: non-temporal loads, which stream from HBM at a
  // far higher rate than loads that allocate for reuse.
  auto load_step = [&](int m, int s, u32x4& c) {
    c = __builtin_nontemporal_load((const u32x4*)(cl[m] + s * (FMT == MOE_Q8_0 ? 4 * EPS : 2 * EPS)));
  };

  // The scales of the workgroup's rows (wg_rows x srb bytes per matrix, one
  // contiguous region) go to LDS through coalesced 16-byte loads: per-step
  // scale loads of a few bytes per lane would cost as many memory requests
  // as the codes themselves.  sS follows the activation buffer.
  constexpr int RED_BYTES = 4 * NMAT * NT * 64 * 16;
  uint8_t* sS = (uint8_t*)sA + max(NT * CPT * K * 2, RED_BYTES);
  f32x4* red = (f32x4*)sA;
  const int s_chunks_m = wg_rows * srb / 16;  // per matrix (srb is a multiple of 8, wg_rows of 16)
  const int s_chunks = NMAT * s_chunks_m;
  constexpr int SB = 2;  // scale chunks per thread issued before the codes
  auto s_src = [&](int ch) -> const u32x4* {
    const int m = ch >= s_chunks_m ? 1 : 0;
    return (const u32x4*)(sreg[NMAT > 1 ? m : 0] + (ch - m * s_chunks_m) * 16);
  };
  u32x4 sv[SB];
#pragma unroll
  for (int b = 0; b < SB; ++b) sv[b] = __builtin_nontemporal_load(s_src(min(tid + b * 256, s_chunks - 1)));
  // A rows that hold no column read zeros from kw halves after the scales
  const int zoff = (int)(sS + s_chunks * 16 - (uint8_t*)sA) / 2;
  // this lane's scale words in LDS: row (wid / ksplit) * 16 + n, the step-0
  // block (Q5_1: 8-byte records, four 16-bit words each)
  constexpr int SW = FMT == MOE_Q5_1 ? 4 : 1;
  const uint16_t* ssl[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
    ssl[m] = (const uint16_t*)(sS + m * s_chunks_m * 16 + ((wid / ksplit) * 16 + n) * srb) + (kbase >> 5) * SW;
  // REUSE (without ROLL): the codes of every step, loaded in the first pass,
  // stay in registers for the later passes instead of being read again.
  u32x4 cb_keep[NMAT][PD];
  for (int c0 = 0; c0 < ncol; c0 += CPP) {
    const int ncp = min(CPP, ncol - c0);
    const int nch = ncp * chunks_per_col;
    // ---- the first batch of this pass's activation chunks, issued before the
    // weight codes so that waiting for them does not wait for the codes
    // (REUSE: the chunks go straight to LDS below instead)
    // 16-byte staging chunk ch lands at LDS byte 16 ch.  Gate/up: chunk kk / 8
    // of column c (column-major fp16).  Down: the pass's h rows, consecutive
    // fp32 rows of the workspace, copied as they are (row t of the pass at
    // bytes [4Kt, 4K(t+1)); converted in place below).
    const float* hsrc = GATEUP ? nullptr : a.hf + (long)(si.row0 + c0 / 2) * K;
    // down: the tile maxima of the pass's rows (wavefront w: rows w, w + 4,
    // ... of the pass), loaded first so that they land before everything else
    constexpr int QH = (CPP / 2 + 3) / 4;
    uint32_t hmb[QH];
#pragma unroll
    for (int q = 0; q < QH; ++q) hmb[q] = 0u;
    if constexpr (!GATEUP) {
      const int nt16 = K / 16;
#pragma unroll
      for (int q = 0; q < QH; ++q) {
        const int t = wid + 4 * q;
        if (t * 2 < ncp) {
          const uint32_t* hm = a.hmax + (long)(si.row0 + c0 / 2 + t) * nt16;
          for (int i = lane; i < nt16; i += 64) hmb[q] = max(hmb[q], hm[i]);
        }
      }
    }
    auto chunk_src = [&](int ch) -> const u32x4* {
      if constexpr (GATEUP) {
        const int c = ch / chunks_per_col, kk = (ch - c * chunks_per_col) * 8;
        return (const u32x4*)(a.in16 + in_row_of(c0 + c) * K + kk);
      } else {
        return (const u32x4*)hsrc + ch;
      }
    };
    u32x4 av[REUSE ? 1 : AB];
    if constexpr (!REUSE) {
#pragma unroll
      for (int b = 0; b < AB; ++b) av[b] = *chunk_src(min(tid + b * 256, nch - 1));
    }
    uint32_t cw = 0;
    {
      const int c = min(tid, ncp - 1);
      if constexpr (GATEUP) {
        cw = __float_as_uint(a.in_scale[in_row_of(c0 + c)]);
      } else if constexpr (PAIRS) {
        // (the shared slot's rows are past the pair list; its value is unused)
        cw = (uint32_t)a.pair_of_row[min(si.row0 + (c0 + c) / 2, a.T * a.k - 1)];
      }
    }
    // ---- the first PD steps of weight codes (independent of the activations)
    u32x4 cb_pass[NMAT][PD];
    u32x4(&cb)[NMAT][PD] = (REUSE && !ROLL) ? cb_keep : cb_pass;
    if (!(REUSE && !ROLL) || c0 == 0) {
#pragma unroll
      for (int u = 0; u < PD; ++u)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) load_step(m, min(u, nsteps - 1), cb[m][u]);
    }

    // ---- stage the activation columns into LDS.  Columns at or beyond ncp
    // are never read (their A rows are zero), so they are not written.
    __syncthreads();  // the previous pass has finished reading sA
    if constexpr (REUSE) {
      // every chunk of the pass by LDS DMA (16 bytes a lane, 1 KB a wavefront
      // instruction, contiguous in LDS), all in flight at once and no registers
      typedef __attribute__((address_space(3))) void lds_void_t;
      for (int q = wid; q * 64 < nch; q += 4) {
        const int ch = q * 64 + lane;
        if (ch < nch) __builtin_amdgcn_global_load_lds((const void*)chunk_src(ch), (lds_void_t*)(sA + q * 512), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int b = 0; b < AB; ++b) {
        const int ch = tid + b * 256;
        if (ch < nch) *(u32x4*)&sA[ch * 8] = av[b];
      }
    }
    if (tid < ncp) s_colw[tid] = cw;
    if constexpr (!GATEUP) {
      // the power of two of each row of the pass: its largest |h| into
      // [2^14, 2^15)
#pragma unroll
      for (int q = 0; q < QH; ++q) {
        const int t = wid + 4 * q;
        const int ex = x16_exponent(__uint_as_float(wave_max_u32(hmb[q])));
        if (t * 2 < ncp) {
          if (lane < 2) s_colx[2 * t + lane] = __float_as_uint(ldexpf(1.0f, ex));
          if (lane == 0) s_tdown[t] = ldexpf(1.0f, -ex);
        }
      }
    }
    if (c0 == 0) {
      // the item's scales (the first chunks were loaded with the activations)
#pragma unroll
      for (int b = 0; b < SB; ++b)
        if (tid + b * 256 < s_chunks) *(u32x4*)(sS + (tid + b * 256) * 16) = sv[b];
      for (int ch = tid + SB * 256; ch < s_chunks; ch += 256) *(u32x4*)(sS + ch * 16) = *s_src(ch);
      for (int z = tid; z < AST * kw / 8; z += 256) *(u32x4*)&sA[zoff + z * 8] = u32x4{0u, 0u, 0u, 0u};
    }
    // the rest in batches of RB loads in flight per thread
    if constexpr (REUSE) __builtin_amdgcn_s_waitcnt(0);  // the DMA chunks (and the codes) have landed
    for (int ch0 = tid + AB * 256; !REUSE && ch0 < nch; ch0 += RB * 256) {
      u32x4 bv[RB];
#pragma unroll
      for (int b = 0; b < RB; ++b) bv[b] = *chunk_src(min(ch0 + b * 256, nch - 1));
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const int ch = ch0 + b * 256;
        if (ch < nch) *(u32x4*)&sA[ch * 8] = bv[b];
      }
    }
    __syncthreads();
    if constexpr (!GATEUP) {
      // h rows in place: each 32-byte run of eight fp32 values becomes the
      // eight scaled fp16 hi parts, then the eight lo parts (one thread reads
      // and rewrites its own run, so no run is read after another's write)
      uint8_t* sb = (uint8_t*)sA;
      const int runs = nch / 2, runs_per_row = K / 8;
      for (int j = tid; j < runs; j += 256) {
        const float dn = s_tdown[j / runs_per_row];
        const f32x4 v0 = *(const f32x4*)(sb + j * 32), v1 = *(const f32x4*)(sb + j * 32 + 16);
        f16x8 hi, lo;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float sv = (c < 4 ? v0[c] : v1[c - 4]) * dn;
          hi[c] = (f16)sv;
          lo[c] = (f16)(sv - (float)hi[c]);
        }
        *(f16x8*)(sb + j * 32) = hi;
        *(f16x8*)(sb + j * 32 + 16) = lo;
      }
      __syncthreads();
    }

    // A-operand LDS position for each N-tile (this lane is A row m = n, K
    // slice G); lanes without a column read the zero region instead
    int abase[NT];
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
      // (down: column c is part c & 1 of the pass's row c / 2)
      abase[jt] = (valid && c < ncp) ? (GATEUP ? c * K + kbase : (c >> 1) * 2 * K + (c & 1) * 8 + 2 * kbase) : zoff;
    }

    f32x4 acc[NMAT][NT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) acc[m][jt] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute_step = [&](const u32x4 (&cc)[NMAT], int s) {
      // Q8_0 / IQ4_NL: the block's fp16 scale; NVFP4: the chunk's two E4M3
      // scales; Q5_1: d and m (ss), the high-bit word (sh)
      uint32_t ss[NMAT], sh[NMAT];
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        if constexpr (FMT == MOE_Q5_1) {
          const u32x2 rec = *(const u32x2*)(ssl[m] + s * (4 * EPS / 32) * SW);
          ss[m] = rec.x;
          sh[m] = rec.y;
        } else {
          ss[m] = ssl[m][s * (4 * EPS / 32)];
          sh[m] = 0u;
        }
      }
      f16x8 ac[NT][NMF];
#pragma unroll
      for (int jt = 0; jt < NT; ++jt)
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
          ac[jt][i] = *(const f16x8*)&sA[abase[jt] + AST * (s * 4 * EPS + 8 * i)];
        }
      // Q5_1: the activation sum of each column over the lane group's chunk
      // (an MFMA against ones), which the block offset m multiplies
      f32x4 Dsum[NT];
      if constexpr (FMT == MOE_Q5_1) {
        const f16x8 ones = {(f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f};
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) {
          Dsum[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < NMF; ++i) Dsum[jt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ac[jt][i], ones, Dsum[jt], 0, 0, 0);
        }
      }
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
        f32x4 D[NT];
#pragma unroll
        for (int jt = 0; jt < NT; ++jt) D[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
          const f16x8 bf = decode_b<FMT>(cc[m], i, ss[m], sh[m]);
#pragma unroll
          for (int jt = 0; jt < NT; ++jt) D[jt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ac[jt][i], bf, D[jt], 0, 0, 0);
        }
        if constexpr (FMT == MOE_Q5_1) {
          const float dd = f16_bits_to_f32(ss[m] & 0xffffu), mm = f16_bits_to_f32(ss[m] >> 16);
#pragma unroll
          for (int jt = 0; jt < NT; ++jt) {
            acc[m][jt].x = fmaf(dd, D[jt].x, fmaf(mm, Dsum[jt].x, acc[m][jt].x));
            acc[m][jt].y = fmaf(dd, D[jt].y, fmaf(mm, Dsum[jt].y, acc[m][jt].y));
            acc[m][jt].z = fmaf(dd, D[jt].z, fmaf(mm, Dsum[jt].z, acc[m][jt].z));
            acc[m][jt].w = fmaf(dd, D[jt].w, fmaf(mm, Dsum[jt].w, acc[m][jt].w));
          }
        } else if constexpr (FMT == MOE_NVFP4) {
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

    if constexpr (!ROLL) {
      // every step's codes are already in flight
#pragma unroll
      for (int u = 0; u < PD; ++u) {
        if (u < nsteps) {
          u32x4 cc[NMAT];
#pragma unroll
          for (int m = 0; m < NMAT; ++m) cc[m] = cb[m][u];
          compute_step(cc, u);
        }
      }
    } else {
      // rolling prefetch, PD steps ahead (past the end it repeats the last step)
      for (int s0 = 0; s0 < nsteps; s0 += PD) {
#pragma unroll
        for (int u = 0; u < PD; ++u) {
          const int s = s0 + u;
          u32x4 cc[NMAT];
#pragma unroll
          for (int m = 0; m < NMAT; ++m) {
            cc[m] = cb[m][u];
            load_step(m, min(s + PD, nsteps - 1), cb[m][u]);
          }
          if (s < nsteps) compute_step(cc, s);
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
    // reduce the K parts of this row tile through LDS (over the activations,
    // once every wave has finished reading them)
    if (ksplit > 1) {
      __syncthreads();
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
          // column of this lane group (uniform across its 16 lanes, n = 0..15)
          int cl;
          bool ok;
          if constexpr (BD) {
            ok = P == 1 ? (v == G) : (v == 2 * G);
            cl = jt * CPT + v;
          } else {
            ok = !(P == 2 && (v & 1)) && 4 * G + v < CPT;
            cl = jt * CPT + 4 * G + v;
          }
          ok = ok && cl < ncp;
          const int tc = (c0 + cl) / P;
          float val[NMAT];
#pragma unroll
          for (int m = 0; m < NMAT; ++m) val[m] = (P == 2 && v < 3) ? vals[m][v] + vals[m][v + 1] : vals[m][v];
          const int out_row = si.row0 + tc;
          if constexpr (GATEUP) {
            float h = 0.0f;
            if (ok) {
              const float xs = __uint_as_float(s_colw[cl]);
              const float g = val[0] * xs, u = val[1] * xs;
              h = silu_f(g) * u;
              if (!(fabsf(h) <= 3.4028235e38f)) atomicOr(a.error, 2);
              a.hf[(long)out_row * rows + act_pos(a.down_type, frow)] = h;
            }
            // the row's largest |h| over the tile's 16 features (a row of 16
            // lanes)
            uint32_t hb = __float_as_uint(fabsf(h));
            hb = max(hb, dpp_u32<kDppShr1, 0xf>(hb));
            hb = max(hb, dpp_u32<kDppShr2, 0xf>(hb));
            hb = max(hb, dpp_u32<kDppShr4, 0xf>(hb));
            hb = max(hb, dpp_u32<kDppShr8, 0xf>(hb));
            if (ok && n == 15) a.hmax[(long)out_row * (rows / 16) + tile] = hb;
          } else if (ok) {
            val[0] *= __uint_as_float(s_colx[cl]);  // the row's power of two (exact)
            // fused path: routed rows go to their (token, slot) pair's row
            const int orow = (PAIRS && !si.is_sh) ? (int)s_colw[cl] : out_row;
            if constexpr (PAIRS) {
              // coherent across the XCDs' L2 caches: the tile's last
              // workgroup reads these rows in this launch
              __hip_atomic_store(a.o + (long)orow * rows + frow, val[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
              a.o[(long)orow * rows + frow] = val[0];
            }
          }
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// host-side helpers
// ----------------------------------------------------------------------------

struct DecodeWs {
  f16* x16;
  float* xs;
  float* hf;
  uint32_t* hmax;
  float* o;
  SlotEnt* slots;    // per-layer slot table (see DecodeArgs::slots), T*k + 2 entries
  int32_t* n_slots;
};

inline DecodeWs carve(void* ws, int T, int d, int f, int k, int P) {
  char* p = (char*)ws;
  DecodeWs w;
  // x16 / xs: per-layer path, one row per plan row and per token (the
  // shared expert's, after the plan rows); fused path: rows 0..T-1 only
  const size_t R = (size_t)T * k + T;
  w.x16 = (f16*)p;
  p += align_up(R * P * d * 2, 256);
  w.xs = (float*)p;
  p += align_up(R * P * 4, 256);
  w.hf = (float*)p;
  p += align_up(R * f * 4, 256);
  w.hmax = (uint32_t*)p;
  p += align_up(R * (f / 16) * 4, 256);
  w.o = (float*)p;
  p += align_up(R * d * 4, 256);
  w.slots = (SlotEnt*)p;
  p += align_up(((size_t)T * k + 2) * sizeof(SlotEnt), 256);
  w.n_slots = (int32_t*)p;
  return w;
}

// Dynamic LDS of a decode pass: nt N-tiles of staged activations (or the K
// reduction's partial sums), the scale rows of the workgroup's tiles for each
// of nmat matrices, and 2 K / ksplit zero halves.
inline size_t dq_lds_bytes(int fmt, int cpt, int nt, int K, int ksplit, int nmat) {
  const size_t act = (size_t)nt * cpt * K * 2, red = (size_t)4 * nmat * nt * 64 * 16;
  return (act > red ? act : red) + (size_t)nmat * (64 / ksplit) * scale_row_bytes(fmt, K) + (size_t)(K / ksplit) * 4;
}

// Waves along K per 16-row tile: as many as divide the lane-group step count.
inline int pick_ksplit(int K, int eps) {
  const int S = K / (4 * eps);
  for (int ks : {4, 2})
    if (S % ks == 0) return ks;
  return 1;
}

// N-tiles per column pass: enough for the widest slot, within 48 KB of staged
// activations (columns x K x 2 bytes).
inline int pick_nt(int cpt, int ncols_max, int K) {
  const int fit = (48 * 1024) / (cpt * K * 2);
  int nt = (ncols_max + cpt - 1) / cpt;
  if (nt > fit) nt = fit;
  return nt >= 4 ? 4 : (nt >= 2 ? 2 : 1);
}

inline DecodeArgs gateup_args(const moe_layer& L, int T, int P, const DecodeWs& w) {
  DecodeArgs a{};
  a.has_shared = L.has_shared;
  a.T = T;
  a.k = L.k;
  const int eps = dq_eps(L.gate.type);
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
  a.hf = w.hf;
  a.hmax = w.hmax;
  a.down_type = L.down.type;
  return a;
}

inline DecodeArgs down_args(const moe_layer& L, int T, const DecodeWs& w) {
  DecodeArgs a{};
  a.has_shared = L.has_shared;
  a.T = T;
  a.k = L.k;
  a.mat[0] = qmat_dev(L.down);
  if (L.has_shared) a.smat[0] = qmat_dev(L.shared_down);
  a.P = 2;
  a.ksplit = 1;
  a.hf = w.hf;
  a.hmax = w.hmax;
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

}  // namespace qre
