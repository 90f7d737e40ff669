// Device-side helpers for the gfx950 routed-expert kernels.
//
// Format decoding follows the block formats declared in include/moe.h: GGUF
// blocks along a row's reduction dimension (model card, "Sources": tensors are
// GGUF tensors copied unchanged), Q8_0 / IQ4_NL / NVFP4-style as the covered
// expert formats ("Qwen3.8-Flash-Next UD-IQ2_XS (L4 fix) for Basalt", section
// "What was changed").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace qre {

typedef _Float16 f16;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) int32_t i32x4;

constexpr int kWave = 64;

// ---------------------------------------------------------------- scalars

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// OCP FP8 E4M3: bias 7, subnormal m * 2^-9, S.1111.111 = NaN, max 448.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
  float v = (e == 0) ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  if (e == 15u && m == 7u) v = __builtin_nanf("");
  return s ? -v : v;
}

// The same conversion of byte SEL of w in one instruction: gfx950's
// v_cvt_f32_fp8 reads the OCP E4M3 format, and gives the value above for all
// 256 codes (checked code by code on the device, NaN included).
template <int SEL>
__device__ __forceinline__ float e4m3_byte_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8((int)w, SEL);
}

// float -> bf16, round to nearest even (gfx950 converts in hardware:
// v_cvt_pk_bf16_f32).
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- IQ4_NL

// The IQ4_NL codebook biased by +128 so every entry is an unsigned byte:
// {-127,-104,-83,-65,-49,-35,-22,-10,1,13,25,38,53,69,89,113} + 128, four
// entries per dword, entry 0 in the low byte.
constexpr uint32_t kIq4U0 = 0x3F2D1801u;  // 1, 24, 45, 63
constexpr uint32_t kIq4U1 = 0x766A5D4Fu;  // 79, 93, 106, 118
constexpr uint32_t kIq4U2 = 0xA6998D81u;  // 129, 141, 153, 166
constexpr uint32_t kIq4U3 = 0xF1D9C5B5u;  // 181, 197, 217, 241

// Four nibble indices (one per byte, values 0..15) -> four biased codebook
// bytes.  Two 8-entry byte permutes cover entries 0..7 and 8..15; a third
// permute keeps, per byte, the half that bit 3 of the index selects.
__device__ __forceinline__ uint32_t iq4_lookup4(uint32_t q) {
  const uint32_t lo = __builtin_amdgcn_perm(kIq4U1, kIq4U0, q);
  const uint32_t hi = __builtin_amdgcn_perm(kIq4U3, kIq4U2, q ^ 0x08080808u);
  // ((q >> 1) & 0x04040404) | 0x03020100 in one v_bitop3 (truth table 0xEA =
  // (A & B) | C over the inputs 0xF0, 0xCC, 0xAA)
  const uint32_t sel = __builtin_amdgcn_bitop3_b32(q >> 1, 0x04040404u, 0x03020100u, 0xEA);
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Two biased bytes u (= value + 128, 0..255) of U -> an fp16 pair holding the
// exact signed values: the pattern 0x64uu is the fp16 number 1024 + u, and
// subtracting 1152 is exact.  `sel` picks the two bytes (0x04010400 bytes 0,1;
// 0x04030402 bytes 2,3).
__device__ __forceinline__ uint32_t biased_bytes_to_f16x2(uint32_t U, uint32_t sel) {
  const uint32_t p = __builtin_amdgcn_perm(0x64646464u, U, sel);
  f16x2 v = __builtin_bit_cast(f16x2, p);
  const f16x2 off = {(f16)-1152.0f, (f16)-1152.0f};
  return __builtin_bit_cast(uint32_t, v + off);
}

// One dword of IQ4_NL codes (bytes 4i..4i+3 of a block) -> eight exact fp16
// codebook values, in the element order
//   4i, 4i+1, 4i+2, 4i+3, 16+4i, 16+4i+1, 16+4i+2, 16+4i+3
// (the activations are stored in the same per-block order, see iq4_pos).
__device__ __forceinline__ f16x8 iq4_dword_to_f16x8(uint32_t w) {
  const uint32_t ulo = iq4_lookup4(w & 0x0F0F0F0Fu);
  const uint32_t uhi = iq4_lookup4((w >> 4) & 0x0F0F0F0Fu);
  u32x4 r;
  r.x = biased_bytes_to_f16x2(ulo, 0x04010400u);
  r.y = biased_bytes_to_f16x2(ulo, 0x04030402u);
  r.z = biased_bytes_to_f16x2(uhi, 0x04010400u);
  r.w = biased_bytes_to_f16x2(uhi, 0x04030402u);
  return __builtin_bit_cast(f16x8, r);
}

// The same eight values plus 1152, exactly (the fp16 numbers 1024 + u for the
// biased bytes u = value + 128): two operations fewer per pair.  A product sum
// over these weights exceeds the true one by 1152 times the sum of the
// activations it covers, which the caller subtracts once.
__device__ __forceinline__ f16x8 iq4_dword_to_f16x8_p1152(uint32_t w) {
  const uint32_t ulo = iq4_lookup4(w & 0x0F0F0F0Fu);
  const uint32_t uhi = iq4_lookup4((w >> 4) & 0x0F0F0F0Fu);
  u32x4 r;
  r.x = __builtin_amdgcn_perm(0x64646464u, ulo, 0x04010400u);
  r.y = __builtin_amdgcn_perm(0x64646464u, ulo, 0x04030402u);
  r.z = __builtin_amdgcn_perm(0x64646464u, uhi, 0x04010400u);
  r.w = __builtin_amdgcn_perm(0x64646464u, uhi, 0x04030402u);
  return __builtin_bit_cast(f16x8, r);
}

// Position of block element e (0..31) in the IQ4_NL activation layout that
// matches iq4_dword_to_f16x8: code dword i covers positions 8i..8i+7.
__device__ __forceinline__ int iq4_pos(int e) {
  return ((e & 15) >> 2) * 8 + (e >> 4) * 4 + (e & 3);
}

// Position of element i of a row in the activation layout matching the
// weight decode of format `fmt` (IQ4_NL and Q5_1, whose 4-bit codes share the
// byte order, reorder elements inside each block).
__device__ __forceinline__ int act_pos(int fmt, int i) {
  return (fmt == MOE_IQ4_NL || fmt == MOE_Q5_1) ? ((i & ~31) + iq4_pos(i & 31)) : i;
}

// ---------------------------------------------------------------- Q5_1

// Four bits (bit b of x, x < 16) moved to bit 4 of byte b: the fifth bits of
// four Q5_1 codes.  The four shifted copies of x occupy disjoint bit ranges,
// so the product has no carries.
__device__ __forceinline__ uint32_t q5_high4(uint32_t x) { return (x * 0x02040810u) & 0x10101010u; }

// One dword of Q5_1 low nibbles (bytes 4i..4i+3 of a block) and the block's
// high-bit word -> the eight codes q (0..31) as the exact fp16 values 1024 + q
// (the pattern 0x64qq), in the IQ4_NL element order 4i..4i+3, 16+4i..16+4i+3.
__device__ __forceinline__ f16x8 q5_1_dword_to_f16x8_p1024(uint32_t w, uint32_t qh, int i) {
  const uint32_t lo = (w & 0x0F0F0F0Fu) | q5_high4((qh >> (4 * i)) & 0xFu);
  const uint32_t hi = ((w >> 4) & 0x0F0F0F0Fu) | q5_high4((qh >> (16 + 4 * i)) & 0xFu);
  u32x4 r = {__builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u), __builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u),
             __builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u), __builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u)};
  return __builtin_bit_cast(f16x8, r);
}

// The same codes as the exact fp16 values q (subtracting 1024 is exact).
__device__ __forceinline__ f16x8 q5_1_dword_to_f16x8(uint32_t w, uint32_t qh, int i) {
  const f16x8 off = {(f16)-1024.0f, (f16)-1024.0f, (f16)-1024.0f, (f16)-1024.0f,
                     (f16)-1024.0f, (f16)-1024.0f, (f16)-1024.0f, (f16)-1024.0f};
  return q5_1_dword_to_f16x8_p1024(w, qh, i) + off;
}

// 16 bytes at byte offset `off` from the wavefront-uniform `base`, with the
// cache-coherence bits of an agent-scope atomic load (sc1: a raw buffer load
// that bypasses the XCDs' private L2 caches), for data another workgroup of
// the same launch stored with agent-scope atomic stores.
__device__ __forceinline__ f32x4 ld_ag4(const float* base, int off) {
  constexpr int kSc1 = 16;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7fffffff, 0x00020000);
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1));
}

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

// ---------------------------------------------------------------- Q8_0

// One dword of int8 codes -> four exact fp16 values (in order).
__device__ __forceinline__ u32x2 q8_dword_to_f16x4(uint32_t w) {
  const uint32_t u = w ^ 0x80808080u;  // int8 c -> c + 128
  u32x2 r;
  r.x = biased_bytes_to_f16x2(u, 0x04010400u);
  r.y = biased_bytes_to_f16x2(u, 0x04030402u);
  return r;
}

__device__ __forceinline__ f16x8 q8_dwords_to_f16x8(uint32_t a, uint32_t b) {
  const u32x2 x = q8_dword_to_f16x4(a), y = q8_dword_to_f16x4(b);
  u32x4 r = {x.x, x.y, y.x, y.y};
  return __builtin_bit_cast(f16x8, r);
}

// Eight int8 codes plus 1152, exactly (as iq4_dword_to_f16x8_p1152).
__device__ __forceinline__ f16x8 q8_dwords_to_f16x8_p1152(uint32_t a, uint32_t b) {
  const uint32_t ua = a ^ 0x80808080u, ub = b ^ 0x80808080u;
  u32x4 r = {__builtin_amdgcn_perm(0x64646464u, ua, 0x04010400u), __builtin_amdgcn_perm(0x64646464u, ua, 0x04030402u),
             __builtin_amdgcn_perm(0x64646464u, ub, 0x04010400u), __builtin_amdgcn_perm(0x64646464u, ub, 0x04030402u)};
  return __builtin_bit_cast(f16x8, r);
}

// ---------------------------------------------------------------- NVFP4

// E2M1 (sign bit 3, exponent bits 2..1 with bias 1, mantissa bit 0) ->
// float: magnitude index 0..7 maps to {0, .5, 1, 1.5, 2, 3, 4, 6}.
__device__ __forceinline__ float e2m1_to_f32(uint32_t n) {
  const uint32_t s = (n >> 3) & 1u, e = (n >> 1) & 3u, m = n & 1u;
  const float mag = (e == 0) ? 0.5f * (float)m : (float)(2u + m) * __uint_as_float((e + 125u) << 23);
  return s ? -mag : mag;
}

// One dword of E2M1 codes (8 elements; element 2i in the low nibble of byte i)
// times an fp16 block scale -> eight fp16 values e2m1 * scale, in element
// order.  The products have at most 6 significant bits and are exact.  gfx950
// converts a byte of two FP4 codes to two fp16 values in one instruction
// (v_cvt_scalef32_pk_f16_fp4, scale 1).
__device__ __forceinline__ f16x8 fp4_dword_to_f16x8(uint32_t w, f16 scale) {
  const f16x2 s2 = {scale, scale};
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  u32x4 o = {__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1), __builtin_bit_cast(uint32_t, p2),
             __builtin_bit_cast(uint32_t, p3)};
  return __builtin_bit_cast(f16x8, o);
}

// ---------------------------------------------------------------- wave ops

// Wavefront reductions with DPP row shifts and row broadcasts: an inclusive
// prefix within each 16-lane row (row_shr 1, 2, 4, 8), then the row results
// carried up (row_bcast 15 into rows 1 and 3, row_bcast 31 into rows 2 and 3),
// so lane 63 holds the reduction of the wave; it is read back as a scalar.
// Lanes without a source read the identity (zero bits).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, true);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL, ROW_MASK>(__float_as_uint(v)));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint64_t r = ((uint64_t)dpp_u32<CTRL, ROW_MASK>((uint32_t)(u >> 32)) << 32) | dpp_u32<CTRL, ROW_MASK>((uint32_t)u);
  return __longlong_as_double((long long)r);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return ((uint64_t)dpp_u32<CTRL, ROW_MASK>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL, ROW_MASK>((uint32_t)v);
}
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;

__device__ __forceinline__ float lane63_f32(float v) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 63));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<kDppShr1, 0xf>(v);
  v += dpp_f32<kDppShr2, 0xf>(v);
  v += dpp_f32<kDppShr4, 0xf>(v);
  v += dpp_f32<kDppShr8, 0xf>(v);
  v += dpp_f32<kDppBcast15, 0xa>(v);
  v += dpp_f32<kDppBcast31, 0xc>(v);
  return lane63_f32(v);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<kDppShr1, 0xf>(v);
  v += dpp_f64<kDppShr2, 0xf>(v);
  v += dpp_f64<kDppShr4, 0xf>(v);
  v += dpp_f64<kDppShr8, 0xf>(v);
  v += dpp_f64<kDppBcast15, 0xa>(v);
  v += dpp_f64<kDppBcast31, 0xc>(v);
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Maximum of non-negative values (zero bits are the identity).
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppShr1, 0xf>(v));
  v = fmaxf(v, dpp_f32<kDppShr2, 0xf>(v));
  v = fmaxf(v, dpp_f32<kDppShr4, 0xf>(v));
  v = fmaxf(v, dpp_f32<kDppShr8, 0xf>(v));
  v = fmaxf(v, dpp_f32<kDppBcast15, 0xa>(v));
  v = fmaxf(v, dpp_f32<kDppBcast31, 0xc>(v));
  return lane63_f32(v);
}

// ---------------------------------------------------------------- top-k keys

// 32-bit key whose unsigned order is the logit order: the logit's bits mapped
// to an order-preserving unsigned integer, -0 and +0 equal.  Every real value
// maps above 1; NaN maps to 1 (ranked below every real value, as a sort that
// puts NaN last does); 0 marks an empty or taken entry.
__device__ __forceinline__ uint32_t topk_key32(float v) {
  // (selects, not branches: callers convert many entries back to back)
  const uint32_t u = __float_as_uint(v), a = u & 0x7fffffffu;
  uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  key = a == 0u ? 0x80000000u : key;  // -0 as +0
  return a > 0x7f800000u ? 1u : key;  // NaN
}
__device__ __forceinline__ float topk_key32_value(uint32_t key) {
  if (key == 1u) return __uint_as_float(0x7fc00000u);
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppShr1, 0xf>(v));
  v = max(v, dpp_u32<kDppShr2, 0xf>(v));
  v = max(v, dpp_u32<kDppShr4, 0xf>(v));
  v = max(v, dpp_u32<kDppShr8, 0xf>(v));
  v = max(v, dpp_u32<kDppBcast15, 0xa>(v));
  v = max(v, dpp_u32<kDppBcast31, 0xc>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Top-k of one token's logits L[0..E) with one wavefront (E <= 64 * NPL,
// 1 <= k <= min(E, 64)).  Slot j < k of the result is written to out_idx[j]
// (expert id) and out_val[j] (logit): descending logit, the lower expert id
// first on ties.
//
// A threshold first: the lanes are split into at least k groups and tau is
// the smallest group maximum.  Those group maxima are at least k distinct
// entries no smaller than tau, so the k-th largest entry, and every selected
// one, is >= tau.  The entries >= tau (a few dozen for real logits) are packed
// in index order into sk/si (per-wave LDS scratch of 64 entries each) and each
// one's slot is its rank: the entries above it plus the equal ones with a
// lower index.  If more than 64 entries pass the threshold (heavy ties), the
// slots are taken one wave-wide maximum at a time instead.
// wave_topk_vals takes the logits in registers (lv[i] = L[lane + 64 i]; the
// entries at E and beyond are ignored).
template <int NPL>
__device__ __forceinline__ void wave_topk_vals(const float (&lv)[NPL], int E, int k, int lane, uint32_t* sk,
                                               int32_t* si, int32_t* out_idx, float* out_val) {
  uint32_t key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) key[i] = topk_key32(lv[i]) & (lane + 64 * i < E ? 0xffffffffu : 0u);

  // ---- threshold: the smallest of the group maxima (groups of g lanes, 64/g >= k groups)
  uint32_t gm = key[0];
#pragma unroll
  for (int i = 1; i < NPL; ++i) gm = max(gm, key[i]);
  int ng = 1;
  while (ng < k) ng <<= 1;
  const int g = 64 / ng;
  if (g >= 2) gm = max(gm, dpp_u32<kDppShr1, 0xf>(gm));
  if (g >= 4) gm = max(gm, dpp_u32<kDppShr2, 0xf>(gm));
  if (g >= 8) gm = max(gm, dpp_u32<kDppShr4, 0xf>(gm));
  if (g >= 16) gm = max(gm, dpp_u32<kDppShr8, 0xf>(gm));
  if (g >= 32) gm = max(gm, dpp_u32<kDppBcast15, 0xa>(gm));
  if (g >= 64) gm = max(gm, dpp_u32<kDppBcast31, 0xc>(gm));
  const bool rep = (lane & (g - 1)) == g - 1;  // this lane holds its group's maximum
  const uint32_t tau = ~wave_max_u32(rep ? ~gm : 0u);

  // ---- the entries >= tau, packed in index order (register i, then lane)
  int C = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const bool c = key[i] != 0u && key[i] >= tau;
    const uint64_t mk = __ballot(c);
    const int pos = C + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
    if (c && pos < 64) {
      sk[pos] = key[i];
      si[pos] = lane + 64 * i;
    }
    C += __popcll(mk);
  }

  if (C <= 64) {
    // ---- slot = rank among the candidates
    uint32_t kl = 0u;
    int il = 0;
    if (lane < C) {
      kl = sk[lane];
      il = si[lane];
    }
    int rank = 0;
#pragma unroll 4
    for (int j = 0; j < C; ++j) {
      const uint32_t kj = sk[j];
      rank += (kj > kl) ? 1 : 0;
      rank += (kj == kl && j < lane) ? 1 : 0;
    }
    if (lane < C && rank < k) {
      out_idx[rank] = il;
      out_val[rank] = topk_key32_value(kl);
    }
    return;
  }

  // ---- many equal entries: one wave-wide maximum per round, all its holders in index order
  int c = 0;
  while (c < k) {
    uint32_t m = key[0];
#pragma unroll
    for (int i = 1; i < NPL; ++i) m = max(m, key[i]);
    m = wave_max_u32(m);
    if (m == 0u) break;  // fewer than k entries (excluded by the callers' k <= E)
    const float v = topk_key32_value(m);
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const bool hit = key[i] == m;
      const uint64_t mk = __ballot(hit);
      const int pos = c + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
      if (hit && pos < k) {
        out_idx[pos] = lane + 64 * i;
        out_val[pos] = v;
      }
      c += __popcll(mk);
      key[i] = hit ? 0u : key[i];
    }
  }
}

template <int NPL>
__device__ __forceinline__ void wave_topk(const float* __restrict__ L, int E, int k, int lane, uint32_t* sk,
                                          int32_t* si, int32_t* out_idx, float* out_val) {
  float lv[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) lv[i] = L[min(lane + 64 * i, E - 1)];  // unconditional loads, all in flight
  wave_topk_vals<NPL>(lv, E, k, lane, sk, si, out_idx, out_val);
}

// Top-k of one token's logits L[0..E) by a whole workgroup of 256 threads
// (E <= 64 * NPL, 1 <= k <= 32), with the result of wave_topk: slot j < k in
// out_idx[j] / out_val[j], descending logit, the lower expert id first on
// ties.  Thread t holds entries t + 256 i.  The threshold tau is the smallest
// of ng >= k group maxima (groups of 256 / ng consecutive threads, never
// spanning two wavefronts), so every selected entry is >= tau.  Each wavefront
// packs its entries >= tau into its own list, and each list entry counts the
// entries of all lists above it (64-bit keys: the order-preserving logit key,
// then the complement of the expert id, so that no two keys are equal and the
// count is the slot).  If a list would exceed 64 entries (heavy ties),
// wavefront 0 runs wave_topk instead.  Ends with a barrier, after which the
// result is visible to every wavefront.
template <int NPL>
__device__ __forceinline__ void wg_topk1(const float* __restrict__ L, int E, int k, uint32_t* smax,
                                         uint64_t (*ck)[64], int32_t* cnt, uint32_t* tk_key, int32_t* tk_idx,
                                         int32_t* out_idx, float* out_val) {
  constexpr int PT = NPL / 4;  // entries per thread
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint32_t key[PT];
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int e = tid + 256 * i;
    key[i] = topk_key32(L[min(e, E - 1)]) & (e < E ? 0xffffffffu : 0u);
  }
  int ng = 4;
  while (ng < k) ng <<= 1;
  const int gs = 256 / ng;  // 64 .. 8 threads per group
  uint32_t gm = key[0];
#pragma unroll
  for (int i = 1; i < PT; ++i) gm = max(gm, key[i]);
  if (gs >= 2) gm = max(gm, dpp_u32<kDppShr1, 0xf>(gm));
  if (gs >= 4) gm = max(gm, dpp_u32<kDppShr2, 0xf>(gm));
  if (gs >= 8) gm = max(gm, dpp_u32<kDppShr4, 0xf>(gm));
  if (gs >= 16) gm = max(gm, dpp_u32<kDppShr8, 0xf>(gm));
  if (gs >= 32) gm = max(gm, dpp_u32<kDppBcast15, 0xa>(gm));
  if (gs >= 64) gm = max(gm, dpp_u32<kDppBcast31, 0xc>(gm));
  if ((lane & (gs - 1)) == gs - 1) smax[tid / gs] = gm;  // the group's last thread holds its maximum
  __syncthreads();
  uint32_t tau = 0xffffffffu;
  for (int j0 = 0; j0 < ng; j0 += 4) {
    const u32x4 q = *(const u32x4*)&smax[j0];
    tau = min(tau, min(min(q.x, q.y), min(q.z, q.w)));
  }
  // ---- this wavefront's entries >= tau, in index order
  int c = 0;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const bool in = key[i] != 0u && key[i] >= tau;
    const uint64_t mk = __ballot(in);
    const int pos = c + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
    if (in && pos < 64) ck[wid][pos] = ((uint64_t)key[i] << 32) | (uint32_t)~(uint32_t)(tid + 256 * i);
    c += __popcll(mk);
  }
  // zero keys pad the list to a multiple of 8 (they count for nothing)
  if (c <= 64 && lane >= c && lane < ((c + 7) & ~7)) ck[wid][lane] = 0ull;
  if (lane == 0) cnt[wid] = c;
  __syncthreads();
  const int c0 = cnt[0], c1 = cnt[1], c2 = cnt[2], c3 = cnt[3];
  const int cmax = max(max(c0, c1), max(c2, c3));
  if (cmax <= 64) {
    const int cw = cnt[wid];
    const uint64_t kl = lane < cw ? ck[wid][lane] : 0ull;
    int rank = 0;
    for (int j0 = 0; j0 < cmax; j0 += 8) {
      u32x4 q[4][4];
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          q[w2][u] = j0 < cnt[w2] ? *(const u32x4*)&ck[w2][j0 + 2 * u] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint64_t x0 = ((uint64_t)q[w2][u].y << 32) | q[w2][u].x;
          const uint64_t x1 = ((uint64_t)q[w2][u].w << 32) | q[w2][u].z;
          rank += (x0 > kl ? 1 : 0) + (x1 > kl ? 1 : 0);
        }
    }
    if (lane < cw && rank < k) {
      out_idx[rank] = (int32_t)~(uint32_t)kl;
      out_val[rank] = topk_key32_value((uint32_t)(kl >> 32));
    }
  } else if (wid == 0) {
    wave_topk<NPL>(L, E, k, lane, tk_key, tk_idx, out_idx, out_val);
  }
  __syncthreads();
}

// Top-k of one token's logits L[0..E) by a whole workgroup of 256 threads
// (E <= 256 * PT, 1 <= k <= 32), with the result of wave_topk: slot j < k in
// out_idx[j] / out_val[j], descending logit, the lower expert id first on
// ties.  Thread t holds entries t + 256 i.  The threshold tau is the k-th
// largest of 32 group maxima (groups of 8 threads), found by k rounds of a
// wavefront maximum that each remove one copy; the k group maxima at or
// above tau are k entries, so every selected entry is >= tau.  The entries >=
// tau (typically a few more than k) are compacted into one LDS list of
// 64-bit keys (the order-preserving logit key, then the complement of the
// expert id: no two keys are equal), and wavefront 0 ranks them.  If more
// than 64 entries pass (heavy ties), wavefront 0 runs wave_topk instead.
// Ends with a barrier, after which the result is visible to every wavefront.
template <int PT>
__device__ __forceinline__ void wg_topk_tau(const float* __restrict__ L, int E, int k, uint32_t* smax /*[32]*/,
                                           uint64_t* list /*[64]*/, int32_t* cnt /*[4]*/, uint32_t* tk_key,
                                           int32_t* tk_idx, int32_t* out_idx, float* out_val) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint32_t key[PT];
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int e = tid + 256 * i;
    key[i] = topk_key32(L[min(e, E - 1)]) & (e < E ? 0xffffffffu : 0u);
  }
  uint32_t gm = key[0];
#pragma unroll
  for (int i = 1; i < PT; ++i) gm = max(gm, key[i]);
  gm = max(gm, dpp_u32<kDppShr1, 0xf>(gm));
  gm = max(gm, dpp_u32<kDppShr2, 0xf>(gm));
  gm = max(gm, dpp_u32<kDppShr4, 0xf>(gm));
  if ((lane & 7) == 7) smax[tid >> 3] = gm;  // the group's last thread holds its maximum
  __syncthreads();
  // every wavefront finds tau itself (no further barrier)
  uint32_t v = lane < 32 ? smax[lane] : 0u;
  uint32_t tau = 0u;
  for (int r = 0; r < k; ++r) {
    tau = wave_max_u32(v);
    const uint64_t hm = __ballot(v == tau);
    if (lane == (int)__builtin_ctzll(hm)) v = 0u;
  }
  int c = 0;
  uint64_t mk[PT];
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    mk[i] = __ballot(key[i] != 0u && key[i] >= tau);
    c += __popcll(mk[i]);
  }
  if (lane == 0) cnt[wid] = c;
  __syncthreads();
  const int c0 = cnt[0], c1 = cnt[1], c2 = cnt[2], c3 = cnt[3];
  const int C = c0 + c1 + c2 + c3;
  if (C <= 64) {
    int pos = wid == 0 ? 0 : (wid == 1 ? c0 : (wid == 2 ? c0 + c1 : c0 + c1 + c2));
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int p = pos + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mk[i] >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)mk[i], 0u));
      if ((mk[i] >> lane) & 1ull) list[p] = ((uint64_t)key[i] << 32) | (uint32_t)~(uint32_t)(tid + 256 * i);
      pos += __popcll(mk[i]);
    }
    __syncthreads();
    if (wid == 0) {
      const uint64_t kl = lane < C ? list[lane] : 0ull;
      int rank = 0;
      for (int j = 0; j < C; ++j) {
        const uint64_t kj = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(kl >> 32), j) << 32) |
                            (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)kl, j);
        rank += kj > kl ? 1 : 0;
      }
      if (lane < C && rank < k) {
        out_idx[rank] = (int32_t)~(uint32_t)kl;
        out_val[rank] = topk_key32_value((uint32_t)(kl >> 32));
      }
    }
  } else if (wid == 0) {
    wave_topk<PT * 4>(L, E, k, lane, tk_key, tk_idx, out_idx, out_val);
  }
  __syncthreads();
}

// Exclusive prefix sum over a workgroup of NT threads (NT a multiple of 64,
// at most 1024); `tot` receives the sum.  `scratch` holds NT/64 + 1 ints.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int& tot) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += u;
  }
  if (lane == 63) scratch[wid] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < NT / 64; ++w) {
      const int t = scratch[w];
      scratch[w] = run;
      run += t;
    }
    scratch[NT / 64] = run;
  }
  __syncthreads();
  const int res = inc - v + scratch[wid];
  tot = scratch[NT / 64];
  __syncthreads();
  return res;
}

// ---------------------------------------------------------------- formats

__host__ __device__ constexpr int code_row_bytes(int type, int cols) {
  return type == MOE_Q8_0 ? cols : cols / 2;
}
// Q8_0 / IQ4_NL: one binary16 scale per 32; NVFP4: one E4M3 per 16; Q5_1: an
// 8-byte record (d, m, high-bit word) per 32
__host__ __device__ constexpr int scale_row_bytes(int type, int cols) {
  return type == MOE_NVFP4 ? cols / 16 : (type == MOE_Q5_1 ? (cols / 32) * 8 : (cols / 32) * 2);
}

}  // namespace qre
