// Small kernels of the routed-expert layer: dequantisation (test hook),
// router logits, top-k + gate weights, the expert plan, the combine and the
// residual / RMSNorm glue between stacked layers.
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_launch.h"

namespace qre {

// ============================================================================
// Dequantisation (test hook).  Exact values; bf16 output is RNE of the exact
// value.  Formats: include/moe.h.
// ============================================================================

__global__ void k_dequant(QMatDev m, int expert, int out_bf16, void* dst) {
  const int rows = m.rows, cols = m.cols;
  const int nb32 = cols / 32;
  const long total = (long)rows * nb32;  // one thread per 32 elements
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int r = (int)(i / nb32), b = (int)(i % nb32);
  const long row_e = (long)expert * rows + r;
  const uint8_t* crow = m.codes + row_e * code_row_bytes(m.type, cols);
  const uint8_t* srow = m.scales + row_e * scale_row_bytes(m.type, cols);
  float v[32];
  if (m.type == MOE_Q8_0) {
    const float d = f16_bits_to_f32(((const uint16_t*)srow)[b]);
    const int8_t* c = (const int8_t*)crow + b * 32;
    for (int j = 0; j < 32; ++j) v[j] = (float)c[j] * d;
  } else if (m.type == MOE_IQ4_NL) {
    const float d = f16_bits_to_f32(((const uint16_t*)srow)[b]);
    const u32x4 c = *(const u32x4*)(crow + b * 16);
    // decode through the same helper the GEMV kernels use
    for (int i4 = 0; i4 < 4; ++i4) {
      const f16x8 q = iq4_dword_to_f16x8(c[i4]);
      for (int t = 0; t < 4; ++t) {
        v[4 * i4 + t] = (float)q[t] * d;
        v[16 + 4 * i4 + t] = (float)q[4 + t] * d;
      }
    }
  } else if (m.type == MOE_Q5_1) {
    // record: d, m, high-bit word; value fp32(d q + m), one rounding (fma)
    const u32x2 rec = *(const u32x2*)(srow + b * 8);
    const float d = f16_bits_to_f32(rec.x & 0xffffu), mo = f16_bits_to_f32(rec.x >> 16);
    const u32x4 c = *(const u32x4*)(crow + b * 16);
    for (int i4 = 0; i4 < 4; ++i4) {
      const f16x8 q = q5_1_dword_to_f16x8(c[i4], rec.y, i4);
      for (int t = 0; t < 4; ++t) {
        v[4 * i4 + t] = fmaf((float)q[t], d, mo);
        v[16 + 4 * i4 + t] = fmaf((float)q[4 + t], d, mo);
      }
    }
  } else {  // NVFP4: two 16-element blocks
    const float ts = m.ts[expert];
    const u32x4 c = *(const u32x4*)(crow + b * 16);
    for (int half = 0; half < 2; ++half) {
      const float sb = e4m3_to_f32(srow[2 * b + half]);
      const f16 sbh = (f16)sb;  // exact: E4M3 values are fp16 values
      for (int i2 = 0; i2 < 2; ++i2) {
        const f16x8 q = fp4_dword_to_f16x8(c[2 * half + i2], sbh);
        for (int t = 0; t < 8; ++t) v[16 * half + 8 * i2 + t] = (float)q[t] * ts;
      }
    }
  }
  if (out_bf16) {
    uint32_t* o = (uint32_t*)((uint16_t*)dst + (long)r * cols + b * 32);
    for (int j = 0; j < 16; ++j) o[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
  } else {
    float* o = (float*)dst + (long)r * cols + b * 32;
    for (int j = 0; j < 32; ++j) o[j] = v[j];
  }
}

hipError_t launch_dequant(const QMatDev& m, int expert, int out_dtype, void* dst, hipStream_t s) {
  const long total = (long)m.rows * (m.cols / 32);
  const int bs = 256;
  const long grid = (total + bs - 1) / bs;
  hipLaunchKernelGGL(k_dequant, dim3((unsigned)grid), dim3(bs), 0, s, m, expert, out_dtype == MOE_BF16 ? 1 : 0,
                     dst);
  return hipGetLastError();
}

// ============================================================================
// Router logits  L[t][e] = fp32( sum_i W[e][i] x[t][i] + b[e] ).
// ("RAM and VRAM Hold Different Parts of the Expert Weights": the router picks
// the experts each token uses.)
// ============================================================================

__device__ __forceinline__ float load_x(const void* x, int x_bf16, long i) {
  return x_bf16 ? bf16_bits_to_f32(((const uint16_t*)x)[i]) : ((const float*)x)[i];
}

// Four consecutive activations x[i .. i+3] (i a multiple of 4).
template <bool XB>
__device__ __forceinline__ f32x4 load4_x(const void* x, long i) {
  if constexpr (XB) {
    const u32x2 v = *(const u32x2*)((const uint16_t*)x + i);
    return f32x4{bf16_bits_to_f32(v.x & 0xffffu), bf16_bits_to_f32(v.x >> 16), bf16_bits_to_f32(v.y & 0xffffu),
                 bf16_bits_to_f32(v.y >> 16)};
  } else {
    return *(const f32x4*)((const float*)x + i);
  }
}

// T <= 64: one workgroup per expert row, fp64 accumulation (products of an
// fp32 weight and a bf16/fp32 activation are exact in fp64), up to 16 tokens
// per pass.  The row is streamed from HBM once (held in registers for
// d <= 4096); the activations are shared by every workgroup and come from L2.
constexpr int kRtTok = 16;
constexpr int kRtJ = 4;  // 1024-element chunks of the row held in registers

template <bool XB>
__global__ __launch_bounds__(256) void k_router_gemv_f64(const float* __restrict__ W, const float* __restrict__ bias,
                                                         const void* __restrict__ x, int T, int E, int d,
                                                         float* __restrict__ logits) {
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  __shared__ double red[4][kRtTok];
  const float* wr = W + (long)e * d;
  const int nj = (d + 1023) / 1024;
  const float bv = bias ? bias[e] : 0.0f;
  // elements j*1024 + 4*tid .. +3 (out-of-row lanes load a valid address and
  // leave it unused)
  f32x4 wv[kRtJ];
#pragma unroll
  for (int j = 0; j < kRtJ; ++j)
    wv[j] = __builtin_nontemporal_load((const f32x4*)(wr + min(j * 1024 + tid * 4, d - 4)));

  auto accumulate = [&](const f32x4& w4, int i, int t0, int nt, double (&acc)[kRtTok]) {
    f32x4 xv[kRtTok];
#pragma unroll
    for (int t = 0; t < kRtTok; ++t) xv[t] = load4_x<XB>(x, (long)(t0 + min(t, nt - 1)) * d + i);
#pragma unroll
    for (int t = 0; t < kRtTok; ++t)
      if (t < nt)
        acc[t] += (double)w4.x * (double)xv[t].x + (double)w4.y * (double)xv[t].y + (double)w4.z * (double)xv[t].z +
                  (double)w4.w * (double)xv[t].w;
  };

  for (int t0 = 0; t0 < T; t0 += kRtTok) {
    const int nt = min(kRtTok, T - t0);
    double acc[kRtTok];
#pragma unroll
    for (int t = 0; t < kRtTok; ++t) acc[t] = 0.0;
#pragma unroll
    for (int j = 0; j < kRtJ; ++j) {
      const int i = j * 1024 + tid * 4;
      if (j < nj && i < d) accumulate(wv[j], i, t0, nt, acc);
    }
    for (int j = kRtJ; j < nj; ++j) {  // rows longer than 4096: re-read per pass
      const int i = j * 1024 + tid * 4;
      if (i < d) accumulate(*(const f32x4*)(wr + i), i, t0, nt, acc);
    }
#pragma unroll
    for (int t = 0; t < kRtTok; ++t) {
      if (t < nt) {
        const double v = wave_sum_f64(acc[t]);
        if (lane == 0) red[wid][t] = v;
      }
    }
    __syncthreads();
    if (tid < nt) {
      const double v = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid] + (double)bv;
      logits[(long)(t0 + tid) * E + e] = (float)v;
    }
    __syncthreads();
  }
}

// T > 64: fp32 tiled GEMM, 64 experts x 64 tokens per workgroup, K chunks of 32.
__global__ __launch_bounds__(256) void k_router_gemm_f32(const float* __restrict__ W, const float* __restrict__ bias,
                                                         const void* __restrict__ x, int x_bf16, int T, int E, int d,
                                                         float* __restrict__ logits) {
  __shared__ float sW[32][65];
  __shared__ float sX[32][65];
  const int e0 = blockIdx.x * 64, t0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  const int te = tid & 15, tt = tid >> 4;  // 4x4 outputs each: e = e0 + te + 16*i, t = t0 + tt + 16*j
  float acc[4][4] = {};
  for (int k0 = 0; k0 < d; k0 += 32) {
    for (int idx = tid; idx < 64 * 32; idx += 256) {
      const int r = idx >> 5, c = idx & 31;
      const int e = e0 + r, t = t0 + r;
      sW[c][r] = (e < E) ? W[(long)e * d + k0 + c] : 0.0f;
      sX[c][r] = (t < T) ? load_x(x, x_bf16, (long)t * d + k0 + c) : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < 32; ++c) {
      float wv[4], xv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[i] = sW[c][te + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) xv[j] = sX[c][tt + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(wv[i], xv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + te + 16 * i;
    if (e >= E) continue;
    const float bv = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + tt + 16 * j;
      if (t < T) logits[(long)t * E + e] = acc[i][j] + bv;
    }
  }
}

// T > 64 with bf16 tokens: logits on bf16 MFMA.  Each fp32 router weight is
// the exact sum of three bf16 parts (its top 8 significand bits, the next 8,
// the last 8: each remainder is exact in fp32), and a bf16 token times a bf16
// part is exact in fp32, so three MFMAs per product give fp32-accumulated
// dot products of the fp32 weights with the bf16 tokens.  A workgroup covers
// 64 tokens x 128 experts; wavefront w holds all 64 tokens (four M fragments)
// and experts [32w, 32w+32) (two N fragments).  The token tile of each
// 128-element K group is copied once per workgroup into LDS (16-byte LDS
// DMA) and read from there by the four wavefronts; each wavefront loads its
// router words itself.  The next group's copies and loads are in flight while
// the current group's products run.
constexpr int kRmTok = 64, kRmExp = 128;

__device__ __forceinline__ void split_bf16x3(const f32x4 (&w)[2], bf16x8& p1, bf16x8& p2, bf16x8& p3) {
  uint32_t u[8], r1[8], r2[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    u[j] = __float_as_uint(w[j >> 2][j & 3]);
    const float a = __uint_as_float(u[j]) - __uint_as_float(u[j] & 0xffff0000u);
    r1[j] = __float_as_uint(a);
    r2[j] = __float_as_uint(a - __uint_as_float(r1[j] & 0xffff0000u));
  }
  u32x4 q1, q2, q3;
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // the upper halves of elements 2j, 2j+1
    q1[j] = __builtin_amdgcn_perm(u[2 * j + 1], u[2 * j], 0x07060302u);
    q2[j] = __builtin_amdgcn_perm(r1[2 * j + 1], r1[2 * j], 0x07060302u);
    q3[j] = __builtin_amdgcn_perm(r2[2 * j + 1], r2[2 * j], 0x07060302u);
  }
  p1 = __builtin_bit_cast(bf16x8, q1);
  p2 = __builtin_bit_cast(bf16x8, q2);
  p3 = __builtin_bit_cast(bf16x8, q3);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_router_mfma(
    const float* __restrict__ W, const float* __restrict__ bias, const uint16_t* __restrict__ x, int T, int E, int d,
    float* __restrict__ logits) {
  // the token tile of a 128-element K group: [64 rows][16 chunks of 8], chunk
  // c of row r at c ^ (r & 15) (the 16 rows of a fragment read fall in
  // distinct banks); two buffers, the next group's copy in flight.  The
  // buffers are distinct LDS objects, named statically at every use, so the
  // compiler sees that a copy in flight writes the other buffer and does not
  // hold this group's LDS reads until it lands.
  __shared__ __align__(16) uint8_t sx0[kRmTok * 16 * 16];
  __shared__ __align__(16) uint8_t sx1[kRmTok * 16 * 16];
  typedef __attribute__((address_space(3))) void lds_void_t;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = lane & 15, G = lane >> 4;
  const int t0 = blockIdx.y * kRmTok, e0 = blockIdx.x * kRmExp + wid * 32;
  // this thread's four 16-byte copies per group: LDS slot q*256 + tid holds
  // row (q*256 + tid) / 16, stored chunk (q*256 + tid) % 16, i.e. logical
  // chunk (stored ^ row % 16); rows past T repeat the last one
  const uint16_t* xsrc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int slot = q * 256 + tid, r = slot >> 4, c = (slot & 15) ^ (r & 15);
    xsrc[q] = x + (long)min(t0 + r, T - 1) * d + c * 8;
  }
  auto copy_x = [&](int kg, uint8_t* buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(xsrc[q] + kg), (lds_void_t*)(buf + (q * 256 + wid * 64) * 16),
                                       16, 0, 0);
  };
  // this lane's router rows (rows past the end repeat the last one and are not stored)
  const float* wr[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) wr[f] = W + (long)min(e0 + f * 16 + n, E - 1) * d + 8 * G;
  auto load_w = [&](int kg, f32x4 (&wb)[4][2][2]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        wb[j][f][0] = *(const f32x4*)(wr[f] + kg + 32 * j);
        wb[j][f][1] = *(const f32x4*)(wr[f] + kg + 32 * j + 4);
      }
  };

  f32x4 acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int f = 0; f < 2; ++f) acc[mi][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint8_t* buf, const f32x4 (&wb)[4][2][2]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 xa[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int r = mi * 16 + n;
        xa[mi] = *(const u32x4*)(buf + (r * 16 + ((4 * j + G) ^ n)) * 16);
      }
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        bf16x8 p1, p2, p3;
        split_bf16x3(wb[j][f], p1, p2, p3);
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, xa[mi]);
          acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, p1, acc[mi][f], 0, 0, 0);
          acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, p2, acc[mi][f], 0, 0, 0);
          acc[mi][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, p3, acc[mi][f], 0, 0, 0);
        }
      }
    }
  };
  // K in groups of 128 (d is a multiple of 128): the group's token tile and
  // router words were requested during the previous group
  f32x4 wb0[4][2][2], wb1[4][2][2];
  copy_x(0, sx0);
  load_w(0, wb0);
  for (int kg = 0; kg < d; kg += 256) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // group kg is in LDS for every wave; buffer 1 is free
    if (kg + 128 < d) {
      copy_x(kg + 128, sx1);
      load_w(kg + 128, wb1);
    }
    compute(sx0, wb0);
    if (kg + 128 >= d) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // group kg + 128 is in LDS; buffer 0 is free
    if (kg + 256 < d) {
      copy_x(kg + 256, sx0);
      load_w(kg + 256, wb0);
    }
    compute(sx1, wb1);
  }
  // D row 4G + v of fragment (mi, f): token t0 + mi*16 + 4G + v, expert e0 + f*16 + n
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int e = e0 + f * 16 + n;
    if (e >= E) continue;
    const float bv = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + mi * 16 + 4 * G + v;
        if (t < T) logits[(long)t * E + e] = acc[mi][f][v] + bv;
      }
  }
}

// 8 < T <= 64 with bf16 tokens: the same exact-product MFMA logits, shaped
// for few tokens and split along K so that the launch fills the chip: a
// workgroup takes 16 experts and one of KS slices of K (at most kRsMaxChunks
// chunks of 32), and its wavefront w the tokens 16w .. 16w + 15 with all of
// its chunks in flight at once.  Slice s of the sum goes to
// partials[s][t][e]; the top-k launch adds the slices in slice order (then the
// bias), so the result does not depend on scheduling.
constexpr int kRsMaxChunks = 12;
constexpr int kRsMaxSlices = 16;  // d <= 4096, a multiple of 512: 16 slices always fit

// Slices of K for this router, or 0 when the shape takes another kernel.
int router_ksplit(int T, int d, int x_dtype) {
  if (x_dtype != MOE_BF16 || T <= 8 || T > 64 || d % 512 != 0 || d > 4096) return 0;
  const int nch = d / 32;
  for (int ks = 1; ks <= kRsMaxSlices; ++ks)
    if (nch % ks == 0 && nch / ks <= kRsMaxChunks) return ks;
  return 0;
}

__global__ __launch_bounds__(256) void k_router_mfma_split(const float* __restrict__ W, const uint16_t* __restrict__ x,
                                                           int T, int E, int d, int kslice,
                                                           float* __restrict__ partials) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int n = lane & 15, G = lane >> 4;
  const int e0 = blockIdx.x * 16, t0 = wid * 16;
  if (t0 >= T) return;
  const int kb = blockIdx.y * kslice, nc = kslice / 32;
  const uint16_t* xr = x + (long)min(t0 + n, T - 1) * d + kb + 8 * G;
  const float* wr = W + (long)min(e0 + n, E - 1) * d + kb + 8 * G;
  u32x4 xa[kRsMaxChunks];
  f32x4 wb[kRsMaxChunks][2];
#pragma unroll
  for (int c = 0; c < kRsMaxChunks; ++c) {
    const int cc = min(c, nc - 1);  // past the end: a repeated chunk, unused
    wb[c][0] = __builtin_nontemporal_load((const f32x4*)(wr + cc * 32));
    wb[c][1] = __builtin_nontemporal_load((const f32x4*)(wr + cc * 32 + 4));
    xa[c] = *(const u32x4*)(xr + cc * 32);
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < kRsMaxChunks; ++c) {
    if (c < nc) {
      bf16x8 p1, p2, p3;
      split_bf16x3(wb[c], p1, p2, p3);
      const bf16x8 a = __builtin_bit_cast(bf16x8, xa[c]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, p1, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, p2, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, p3, acc, 0, 0, 0);
    }
  }
  // D layout: lane (n, G) holds token t0 + 4G + v, expert e0 + n
  const int e = e0 + n;
  float* out = partials + (long)blockIdx.y * T * E;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int t = t0 + 4 * G + v;
    if (t < T && e < E) out[(long)t * E + e] = acc[v];
  }
}

hipError_t launch_router_logits(const float* W, const float* b, const void* x, int x_dtype, int T, int E, int d,
                                float* logits, hipStream_t s) {
  const int xb = x_dtype == MOE_BF16 ? 1 : 0;
  if (T <= 64) {
    if (xb)
      hipLaunchKernelGGL(k_router_gemv_f64<true>, dim3(E), dim3(256), 0, s, W, b, x, T, E, d, logits);
    else
      hipLaunchKernelGGL(k_router_gemv_f64<false>, dim3(E), dim3(256), 0, s, W, b, x, T, E, d, logits);
  } else if (xb) {
    hipLaunchKernelGGL(k_router_mfma, dim3((E + kRmExp - 1) / kRmExp, (T + kRmTok - 1) / kRmTok), dim3(256), 0, s, W,
                       b, (const uint16_t*)x, T, E, d, logits);
  } else {
    hipLaunchKernelGGL(k_router_gemm_f32, dim3((E + 63) / 64, (T + 63) / 64), dim3(256), 0, s, W, b, x, xb, T, E, d,
                       logits);
  }
  return hipGetLastError();
}

// ============================================================================
// Top-k + gate weights: one wavefront per token.  Slot order: descending
// logit, lower expert id first on ties; weights = softmax over the k selected
// logits.  E <= 1024.
// ============================================================================

template <int NPL>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E, int k,
                                              int32_t* __restrict__ idx, float* __restrict__ w) {
  __shared__ uint32_t sk[4][64];
  __shared__ int32_t si[4][64];
  __shared__ int32_t oi[4][64];
  __shared__ float ov[4][64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wid;
  if (t >= T) return;
  wave_topk<NPL>(logits + (long)t * E, E, k, lane, sk[wid], si[wid], oi[wid], ov[wid]);
  // (the same wavefront reads back what it wrote: its LDS accesses are in order)
  const float v = lane < k ? ov[wid][lane] : 0.0f;
  const float vmax = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 0));
  const float ex = lane < k ? expf(v - vmax) : 0.0f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    idx[(long)t * k + lane] = oi[wid][lane];
    w[(long)t * k + lane] = ex / sum;
  }
}

// The same after the K-split router: logits[t][e] = (slice 0 + slice 1 + ...
// in slice order) + bias[e], written out, then the top-k of those values.
template <int NPL>
__global__ __launch_bounds__(256) void k_topk_slices(const float* __restrict__ partials, int ks,
                                                     const float* __restrict__ bias, int T, int E, int k,
                                                     float* __restrict__ logits, int32_t* __restrict__ idx,
                                                     float* __restrict__ w) {
  __shared__ uint32_t sk[4][64];
  __shared__ int32_t si[4][64];
  __shared__ int32_t oi[4][64];
  __shared__ float ov[4][64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wid;
  if (t >= T) return;
  // every slice's loads are issued before the (ordered) sums
  float lv[NPL], sl[NPL][kRsMaxSlices];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = min(lane + 64 * i, E - 1);
#pragma unroll
    for (int p = 0; p < kRsMaxSlices; ++p) sl[i][p] = p < ks ? partials[((long)p * T + t) * E + e] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = min(lane + 64 * i, E - 1);
    float sum = sl[i][0];
#pragma unroll
    for (int p = 1; p < kRsMaxSlices; ++p)
      if (p < ks) sum += sl[i][p];
    lv[i] = sum + (bias ? bias[e] : 0.0f);
    if (lane + 64 * i < E) logits[(long)t * E + e] = lv[i];
  }
  wave_topk_vals<NPL>(lv, E, k, lane, sk[wid], si[wid], oi[wid], ov[wid]);
  const float v = lane < k ? ov[wid][lane] : 0.0f;
  const float vmax = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 0));
  const float ex = lane < k ? expf(v - vmax) : 0.0f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    idx[(long)t * k + lane] = oi[wid][lane];
    w[(long)t * k + lane] = ex / sum;
  }
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w, hipStream_t s) {
  const dim3 g((T + 3) / 4), b(256);
  if (E <= 64)
    hipLaunchKernelGGL(k_topk<1>, g, b, 0, s, logits, T, E, k, idx, w);
  else if (E <= 256)
    hipLaunchKernelGGL(k_topk<4>, g, b, 0, s, logits, T, E, k, idx, w);
  else if (E <= 512)
    hipLaunchKernelGGL(k_topk<8>, g, b, 0, s, logits, T, E, k, idx, w);
  else
    hipLaunchKernelGGL(k_topk<16>, g, b, 0, s, logits, T, E, k, idx, w);
  return hipGetLastError();
}

size_t router_partials_bytes(int T, int E, int d, int x_dtype) {
  return (size_t)router_ksplit(T, d, x_dtype) * T * E * 4;
}

hipError_t launch_route(const float* W, const float* b, const void* x, int x_dtype, int T, int E, int d, int k,
                        float* logits, float* partials, int32_t* idx, float* w, hipStream_t s) {
  const int ks = router_ksplit(T, d, x_dtype);
  if (ks == 0) {
    const hipError_t e = launch_router_logits(W, b, x, x_dtype, T, E, d, logits, s);
    if (e != hipSuccess) return e;
    return launch_topk(logits, T, E, k, idx, w, s);
  }
  hipLaunchKernelGGL(k_router_mfma_split, dim3((E + 15) / 16, ks), dim3(256), 0, s, W, (const uint16_t*)x, T, E, d,
                     d / ks, partials);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g((T + 3) / 4), bl(256);
  if (E <= 64)
    hipLaunchKernelGGL(k_topk_slices<1>, g, bl, 0, s, partials, ks, b, T, E, k, logits, idx, w);
  else if (E <= 256)
    hipLaunchKernelGGL(k_topk_slices<4>, g, bl, 0, s, partials, ks, b, T, E, k, logits, idx, w);
  else if (E <= 512)
    hipLaunchKernelGGL(k_topk_slices<8>, g, bl, 0, s, partials, ks, b, T, E, k, logits, idx, w);
  else
    hipLaunchKernelGGL(k_topk_slices<16>, g, bl, 0, s, partials, ks, b, T, E, k, logits, idx, w);
  return hipGetLastError();
}

// ============================================================================
// Expert plan ("device-planned MoE tail", UD-IQ2_XS (L4 fix) page, "What was
// changed").  No global atomics and no dependence on scheduling: within a
// block of up to 64 tokens, each expert gets a 64-bit mask of the tokens that
// picked it (LDS atomic OR is order-independent); a pair's rank among the
// expert's rows is the number of earlier tokens in the mask, plus the rows of
// the same expert in earlier blocks.  Rows of an expert are therefore in
// ascending token order.
//   T <= 64: one kernel, one workgroup.
//   T  > 64: count (per-block histograms), scan (one workgroup), scatter.
// ============================================================================

constexpr int kPlanTB = 64;

size_t plan_ws_bytes(int T, int E) {
  const int nb = (T + kPlanTB - 1) / kPlanTB;
  return align_up((size_t)nb * E * 4 + (size_t)nb * 4, 256);
}

// Status of pair q (local index) of a block whose ids are staged in LDS
// sidx: its expert id if the pair is kept, -1 for an id outside [0, E), -2
// for an id already named at an earlier slot of the same token (a top-k
// selection names each expert once; of repeats the lowest slot is kept).
__device__ __forceinline__ int pair_status(const int32_t* sidx, int q, int k, int E) {
  const int e = sidx[q];
  if (e < 0 || e >= E) return -1;
  const int j = q % k, q0 = q - j;
  for (int jj = 0; jj < j; ++jj)
    if (sidx[q0 + jj] == e) return -2;
  return e;
}

// Ids of one block of <= 64 tokens into LDS sidx, then token masks into LDS
// mask[E]; returns the error bits of the block (1: an id out of range, 4: a
// repeated id).
__device__ __forceinline__ int block_token_masks(const int32_t* __restrict__ idx, int t0, int t1, int k, int E,
                                                 int32_t* sidx, unsigned long long* mask) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) mask[e] = 0ull;
  for (int q = threadIdx.x; q < (t1 - t0) * k; q += blockDim.x) sidx[q] = idx[t0 * k + q];
  __syncthreads();
  int err = 0;
  for (int q = threadIdx.x; q < (t1 - t0) * k; q += blockDim.x) {
    const int e = pair_status(sidx, q, k, E);
    if (e >= 0)
      atomicOr(&mask[e], 1ull << (q / k));
    else
      err |= e == -1 ? 1 : 4;
  }
  const int e1 = __syncthreads_or(err & 1);
  const int e4 = __syncthreads_or(err & 4);
  return (e1 ? 1 : 0) | (e4 ? 4 : 0);
}

__device__ __forceinline__ void plan_scatter_block(int t0, int t1, int k, int E, const int32_t* sidx,
                                                   const unsigned long long* mask, const int32_t* base,
                                                   const PlanDev& p) {
  for (int q = threadIdx.x; q < (t1 - t0) * k; q += blockDim.x) {
    const int e = pair_status(sidx, q, k, E);
    const int qg = t0 * k + q;
    if (e < 0) {
      p.slot_row[qg] = -1;
      continue;
    }
    const int tl = q / k;
    const int rank = __popcll(mask[e] & ((1ull << tl) - 1ull));
    const int r = base[e] + rank;
    p.row_token[r] = t0 + tl;
    p.row_slot[r] = q % k;
    p.slot_row[qg] = r;
  }
}

// T <= 64, E <= 1024: the whole plan in one workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void k_plan_small(const int32_t* __restrict__ idx, int T, int k, int E, PlanDev p) {
  __shared__ unsigned long long mask[1024];
  __shared__ int32_t base[1024];
  __shared__ int32_t sidx[kPlanTB * 32];
  __shared__ int32_t scratch[2][17];
  const int err = block_token_masks(idx, 0, T, k, E, sidx, mask);
  const int e = threadIdx.x;
  const int cnt = e < E ? __popcll(mask[e]) : 0;
  int n_valid, n_act;
  const int off = block_exclusive_scan<1024>(cnt, scratch[0], n_valid);
  const int aoff = block_exclusive_scan<1024>(cnt > 0 ? 1 : 0, scratch[1], n_act);
  if (e < E) {
    base[e] = off;
    p.counts[e] = cnt;
    p.offsets[e] = off;
    if (cnt > 0) p.active[aoff] = e;
    if (e >= n_act) p.active[e] = -1;
  }
  if (e == 0) {
    p.offsets[E] = n_valid;
    *p.n_active = n_act;
    *p.error = err;
  }
  for (int r = n_valid + threadIdx.x; r < T * k; r += blockDim.x) {
    p.row_token[r] = -1;
    p.row_slot[r] = -1;
  }
  __syncthreads();
  plan_scatter_block(0, T, k, E, sidx, mask, base, p);
}

__global__ __launch_bounds__(256) void k_plan_count(const int32_t* __restrict__ idx, int T, int k, int E,
                                                    int32_t* __restrict__ hist, int32_t* __restrict__ blk_err) {
  __shared__ unsigned long long mask[1024];
  __shared__ int32_t sidx[kPlanTB * 32];
  const int b = blockIdx.x;
  const int t0 = b * kPlanTB, t1 = min(T, t0 + kPlanTB);
  const int err = block_token_masks(idx, t0, t1, k, E, sidx, mask);
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(long)b * E + e] = __popcll(mask[e]);
  if (threadIdx.x == 0) blk_err[b] = err;
}

__global__ __launch_bounds__(1024) void k_plan_scan(int T, int k, int E, int nb, int32_t* __restrict__ hist,
                                                    const int32_t* __restrict__ blk_err, PlanDev p) {
  __shared__ int32_t scratch[2][17];
  __shared__ int32_t err_s;
  const int e = threadIdx.x;
  // The counts of the first kR blocks (T <= 4096) stay in registers between the
  // two passes, all loaded together; the blocks beyond are handled in batches
  // of kB, their prefixes written in the first pass and read back.
  constexpr int kR = 64, kB = 16;
  int cr[kR];
  int cnt = 0;
  if (e < E) {
#pragma unroll
    for (int u = 0; u < kR; ++u) cr[u] = u < nb ? hist[(long)u * E + e] : 0;
#pragma unroll
    for (int u = 0; u < kR; ++u) {
      const int c = cr[u];
      cr[u] = cnt;  // exclusive prefix within the expert
      cnt += c;
    }
    for (int b0 = kR; b0 < nb; b0 += kB) {
      int c[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) c[u] = b0 + u < nb ? hist[(long)(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        if (b0 + u < nb) hist[(long)(b0 + u) * E + e] = cnt;
        cnt += c[u];
      }
    }
  }
  int n_valid, n_act;
  const int off = block_exclusive_scan<1024>(cnt, scratch[0], n_valid);
  const int aoff = block_exclusive_scan<1024>(cnt > 0 ? 1 : 0, scratch[1], n_act);
  if (e < E) {
    p.counts[e] = cnt;
    p.offsets[e] = off;
    if (cnt > 0) p.active[aoff] = e;
    if (e >= n_act) p.active[e] = -1;
#pragma unroll
    for (int u = 0; u < kR; ++u)
      if (u < nb) hist[(long)u * E + e] = cr[u] + off;
    for (int b0 = kR; b0 < nb; b0 += kB) {
      int c[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) c[u] = b0 + u < nb ? hist[(long)(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kB; ++u)
        if (b0 + u < nb) hist[(long)(b0 + u) * E + e] = c[u] + off;
    }
  }
  if (threadIdx.x == 0) err_s = 0;
  __syncthreads();
  for (int b = threadIdx.x; b < nb; b += blockDim.x)
    if (blk_err[b]) atomicOr(&err_s, blk_err[b]);
  __syncthreads();
  if (e == 0) {
    p.offsets[E] = n_valid;
    *p.n_active = n_act;
    *p.error = err_s;
  }
  for (int r = n_valid + threadIdx.x; r < T * k; r += blockDim.x) {
    p.row_token[r] = -1;
    p.row_slot[r] = -1;
  }
}

__global__ __launch_bounds__(256) void k_plan_scatter(const int32_t* __restrict__ idx, int T, int k, int E,
                                                      const int32_t* __restrict__ base, PlanDev p) {
  __shared__ unsigned long long mask[1024];
  __shared__ int32_t sidx[kPlanTB * 32];
  const int b = blockIdx.x;
  const int t0 = b * kPlanTB, t1 = min(T, t0 + kPlanTB);
  block_token_masks(idx, t0, t1, k, E, sidx, mask);
  plan_scatter_block(t0, t1, k, E, sidx, mask, base + (long)b * E, p);
}

hipError_t launch_plan(const int32_t* idx, int T, int k, int E, const PlanDev& p, void* ws, hipStream_t s) {
  if (T <= kPlanTB) {
    hipLaunchKernelGGL(k_plan_small, dim3(1), dim3(1024), 0, s, idx, T, k, E, p);
    return hipGetLastError();
  }
  const int nb = (T + kPlanTB - 1) / kPlanTB;
  int32_t* hist = (int32_t*)ws;
  int32_t* blk_err = hist + (size_t)nb * E;
  hipLaunchKernelGGL(k_plan_count, dim3(nb), dim3(256), 0, s, idx, T, k, E, hist, blk_err);
  hipLaunchKernelGGL(k_plan_scan, dim3(1), dim3(1024), 0, s, T, k, E, nb, hist, blk_err, p);
  hipLaunchKernelGGL(k_plan_scatter, dim3(nb), dim3(256), 0, s, idx, T, k, E, hist, p);
  return hipGetLastError();
}

// ============================================================================
// Combine: y_t = s_t + sum_j w[t][j] * o[slot_row[t*k+j]], slots in order j,
// fp32 arithmetic, one rounding to the output type.  o rows: plan rows
// 0..T*k-1, then the shared expert's rows T*k + t.
// ============================================================================

// y[t] = (shared row) + sum_j topk_w[t][j] * o[slot_row[t][j]], the terms
// added in slot order j (fp32 FMAs).  Each thread takes 8 consecutive columns;
// the rows of up to kCombineBatch slots are loaded before they are added, so
// that the loads of a token are in flight together.
constexpr int kCombineBatch = 8;

__global__ __launch_bounds__(256) void k_combine(const void* __restrict__ o, int o_bf16,
                                                 const float* __restrict__ topk_w, const int32_t* __restrict__ slot_row,
                                                 int T, int k, int d, int has_shared, void* __restrict__ y,
                                                 int y_bf16) {
  const int t = blockIdx.y;
  const int i = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i >= d) return;
  auto row8 = [&](long r, float (&f)[8]) {
    if (o_bf16) {
      const u32x4 v = __builtin_nontemporal_load((const u32x4*)((const uint16_t*)o + r * d + i));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f[2 * q] = bf16_bits_to_f32(v[q] & 0xffffu);
        f[2 * q + 1] = bf16_bits_to_f32(v[q] >> 16);
      }
    } else {
      const f32x4 u = *(const f32x4*)((const float*)o + r * d + i);
      const f32x4 w = *(const f32x4*)((const float*)o + r * d + i + 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f[q] = u[q];
        f[4 + q] = w[q];
      }
    }
  };
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (has_shared) row8((long)T * k + t, acc);
  for (int j0 = 0; j0 < k; j0 += kCombineBatch) {
    float v[kCombineBatch][8];
    float wj[kCombineBatch];
    int rj[kCombineBatch];
#pragma unroll
    for (int b = 0; b < kCombineBatch; ++b) {
      const int j = j0 + b;
      rj[b] = j < k ? slot_row[(long)t * k + j] : -1;
      wj[b] = j < k ? topk_w[(long)t * k + j] : 0.0f;
    }
#pragma unroll
    for (int b = 0; b < kCombineBatch; ++b) {
      if (rj[b] >= 0) row8(rj[b], v[b]);
    }
#pragma unroll
    for (int b = 0; b < kCombineBatch; ++b) {
      if (rj[b] < 0) continue;
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = fmaf(wj[b], v[b][q], acc[q]);
    }
  }
  if (y_bf16) {
    u32x4 r = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
               pack_bf16x2(acc[6], acc[7])};
    *(u32x4*)((uint16_t*)y + (long)t * d + i) = r;
  } else {
    *(f32x4*)((float*)y + (long)t * d + i) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *(f32x4*)((float*)y + (long)t * d + i + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
}

hipError_t launch_combine(const void* o, int o_bf16, const float* topk_w, const int32_t* slot_row, int T, int k,
                          int d, int has_shared, void* y, int y_dtype, hipStream_t s) {
  const int per_blk = 256 * 8;
  hipLaunchKernelGGL(k_combine, dim3((d + per_blk - 1) / per_blk, T), dim3(256), 0, s, o, o_bf16, topk_w, slot_row,
                     T, k, d, has_shared, y, y_dtype == MOE_BF16 ? 1 : 0);
  return hipGetLastError();
}

// ============================================================================
// Stack glue: h += y; x = bf16(h / sqrt(mean(h^2) + eps)).  One workgroup per
// token.
// ============================================================================

// Each thread takes groups of 4 consecutive columns; the first kGlueVec
// groups per thread stay in registers between the two passes (d <= 4096 at 256
// threads), any further ones are read back.
constexpr int kGlueVec = 4;

__global__ __launch_bounds__(256) void k_residual_rmsnorm(float* __restrict__ h, const void* __restrict__ y, int y_bf16,
                                                          int d, float eps, uint16_t* __restrict__ x_out) {
  const int t = blockIdx.x;
  float* hr = h + (long)t * d;
  __shared__ float red[4];
  auto add_y = [&](int i, f32x4 v) -> f32x4 {
    if (!y) return v;
    if (y_bf16) {
      const u32x2 u = *(const u32x2*)((const uint16_t*)y + (long)t * d + i);
      v[0] += bf16_bits_to_f32(u.x & 0xffffu);
      v[1] += bf16_bits_to_f32(u.x >> 16);
      v[2] += bf16_bits_to_f32(u.y & 0xffffu);
      v[3] += bf16_bits_to_f32(u.y >> 16);
    } else {
      const f32x4 u = *(const f32x4*)((const float*)y + (long)t * d + i);
      v[0] += u[0];
      v[1] += u[1];
      v[2] += u[2];
      v[3] += u[3];
    }
    return v;
  };
  f32x4 keep[kGlueVec];
  float ss = 0.0f;
#pragma unroll
  for (int q = 0; q < kGlueVec; ++q) {
    const int i = (threadIdx.x + 256 * q) * 4;
    if (i < d) {
      const f32x4 v = add_y(i, *(const f32x4*)(hr + i));
      *(f32x4*)(hr + i) = v;
      keep[q] = v;
#pragma unroll
      for (int c = 0; c < 4; ++c) ss = fmaf(v[c], v[c], ss);
    }
  }
  for (int i = (threadIdx.x + 256 * kGlueVec) * 4; i < d; i += 256 * 4) {
    const f32x4 v = add_y(i, *(const f32x4*)(hr + i));
    *(f32x4*)(hr + i) = v;
#pragma unroll
    for (int c = 0; c < 4; ++c) ss = fmaf(v[c], v[c], ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
  auto put = [&](int i, f32x4 v) {
    const u32x2 r = {pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv)};
    *(u32x2*)(x_out + (long)t * d + i) = r;
  };
#pragma unroll
  for (int q = 0; q < kGlueVec; ++q) {
    const int i = (threadIdx.x + 256 * q) * 4;
    if (i < d) put(i, keep[q]);
  }
  for (int i = (threadIdx.x + 256 * kGlueVec) * 4; i < d; i += 256 * 4) put(i, *(const f32x4*)(hr + i));
}

hipError_t launch_residual_rmsnorm(float* h, const void* y, int y_dtype, int T, int d, float eps, void* x_out,
                                   hipStream_t s) {
  hipLaunchKernelGGL(k_residual_rmsnorm, dim3(T), dim3(256), 0, s, h, y, y_dtype == MOE_BF16 ? 1 : 0, d, eps,
                     (uint16_t*)x_out);
  return hipGetLastError();
}

}  // namespace qre
