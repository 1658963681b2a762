// device.hpp -- gfx950 device helpers for NVFP4 encoding: E4M3 block scales,
// E2M1 elements (nearest-even and stochastic), Philox4x32-10, the 16-point
// Hadamard butterfly.  The numerical definition is the one stated in
// include/nvfp4_amd.h; every float step is one binary32 operation (the
// library is built with -ffp-contract=off).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Largest magnitude of an E2M1 element times the largest E4M3 scale (6 * 448):
// the tensor amax is mapped onto it.
constexpr float kTensorRange = 2688.0f;

// Raw buffer descriptor for a wave-uniform base pointer p (its value is the same
// in every lane of the wave; it is made explicitly uniform so that the descriptor
// sits in scalar registers).  The range field is left at its maximum: callers keep
// every access inside the tensor.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void *p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a)), hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>((uint64_t(hi) << 32) | lo), short(0), 0x7FFFFFFF,
                                           0x00020000);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round a binary32 value to bf16, nearest-even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ float encode_scale(float amax) {
  float s = amax > 0.0f ? kTensorRange / amax : 1.0f;
  return __builtin_isinf(s) ? 3.402823466e38f : s;
}

__device__ __forceinline__ float decode_scale(float amax) { return amax / kTensorRange; }

// E4M3 (OCP "FN": bias 7, max 448) from a non-negative binary32, nearest-even on
// the bits, clamped to the largest finite code 0x7E.  gfx950's converter rounds
// exactly so for every binary32 in [0, 464) (checked bit for bit against a
// software encoder over all of them); at 464 and above it gives NaN instead of
// saturating, so the input is clamped to 448 first (every value in (448, 464)
// rounds to 448 either way).
__device__ __forceinline__ uint32_t e4m3_from_f32(float u) {
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fminf(u, 448.0f), 0.0f, 0, false)) & 0xFFu;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  uint32_t e = (code >> 3) & 15u, m = code & 7u;
  if (e == 0) return float(m) * 0.001953125f;  // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// x / 6 rounded to nearest-even.  For x >= 2^-125 the product with RN(1/6)
// corrected by one fused residual step is that quotient (checked for every
// binary32 in that range); below it the quotient is subnormal and the division
// is done as such.
__device__ __forceinline__ float div6(float x) {
  if (__builtin_expect(x >= 0x1p-125f, 1)) {
    const float r6 = 1.0f / 6.0f;
    const float q0 = x * r6;
    return __builtin_fmaf(__builtin_fmaf(-q0, 6.0f, x), r6, q0);
  }
  return x / 6.0f;
}

// Element multipliers by scale code: tab[c] = s_enc / decode(c), saturated at
// the largest finite float (as the encode scale is: for a tensor amax below about
// 1e-35 the quotient can overflow while the block's elements are tiny), 0 for
// c = 0.  A workgroup fills its table once (threads 0..127) and reads it per block.
constexpr int kMultTable = 128;

__device__ __forceinline__ void fill_mult_table(float *tab, float s_enc) {
  if (threadIdx.x < kMultTable) {
    const float sf = e4m3_to_f32(threadIdx.x);
    const float m = sf > 0.0f ? s_enc / sf : 0.0f;
    tab[threadIdx.x] = __builtin_isinf(m) ? 3.402823466e38f : m;
  }
}

// Scale code and element multiplier of one block from its amax:
// code = E4M3(RN(amax_b / 6) * s_enc), mult = s_enc / decode(code).
__device__ __forceinline__ void block_scale(float amax_b, float s_enc, const float *tab, uint32_t &code, float &mult) {
  code = e4m3_from_f32(div6(amax_b) * s_enc);
  mult = tab[code];
}

// Block scale and multiplier of a 16-block transformed without the Hadamard
// factor 1/4 (u = 4 v, see hadamard16_unscaled).  The block amax RN(max|u| / 4) is
// the maximum of the rounded v (rounding is monotone).  When max|u| >= 2^-90 and
// the multiplier is at least 2^-120, RN(u * (mult / 4)) equals RN(RN(u / 4) * mult)
// for every element: mult / 4 is exact; u / 4 is exact unless |u| < 2^-124, and
// such an element scales below 2^-30 either way (the multiplier is at most 12 over
// the block amax), which encodes to zero under nearest-even and under stochastic
// rounding with 16 random bits.  So the factor joins the multiplier, one product
// per element fewer.  Otherwise (tiny blocks) the factor is applied to the
// elements first, the arithmetic as defined.
__device__ __forceinline__ void block_scale_quarter(float u[16], float s_enc, const float *tab, uint32_t &code,
                                                    float &mult) {
  float amax_u = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) amax_u = fmaxf(amax_u, __builtin_fabsf(u[j]));
  block_scale(amax_u * 0.25f, s_enc, tab, code, mult);
  if (__builtin_expect(amax_u >= 0x1p-90f && mult >= 0x1p-120f, 1)) {
    mult *= 0.25f;
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) u[j] *= 0.25f;
  }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Codes 2 sel and 2 sel + 1 of a word of 8 E2M1 codes (element 2j in the low nibble
// of byte j) as two f16, unscaled: every E2M1 value is an f16 value.  gfx950's
// converter applies only the exponent of its f32 scale operand, so that operand is
// 1 and the E4M3 block scale is applied by a separate f16 multiply.
__device__ __forceinline__ f16x2 fp4x2_to_f16(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  }
}

// Two E4M3 scale codes (the low 16 bits of w) as two f16: every E4M3 value,
// subnormals included, is an f16 value, so the conversion is exact.
__device__ __forceinline__ f16x2 e4m3x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
}

// Codes 2 sel, 2 sel + 1 of w times the block scale s: E2M1 x E4M3 has at most 6
// significant bits and lies in [2^-10, 2688], so the f16 product is exact.
__device__ __forceinline__ f16x2 dequant2(uint32_t w, int sel, _Float16 s) {
  return fp4x2_to_f16(w, sel) * f16x2{s, s};
}

// Canonical zero: clear the sign bit of every code whose magnitude is 0 (the
// converters write -0 for negative values that round to zero).  Per nibble,
// magnitude + 7 sets bit 3 exactly when the magnitude is non-zero.
__device__ __forceinline__ uint32_t canon_zero(uint32_t w) {
  const uint32_t mag = w & 0x77777777u;
  return mag | (w & ((mag + 0x77777777u) & 0x88888888u));
}

// 8 scaled values -> 8 E2M1 codes (element 2j in the low nibble of byte j),
// nearest-even with ties to the even code, |s| >= 6 saturating to 6.  gfx950's
// converter rounds exactly this way (checked against the oracle's encoder over
// every grid midpoint +-64 ulps and a dense sweep of binary32 values); its scale
// operand is 1, the block multiplier having been applied already.
__device__ __forceinline__ uint32_t encode8_rne(const float s[8]) {
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, s[0], s[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, s[2], s[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, s[4], s[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, s[6], s[7], 1.0f, 3);
  return canon_zero(w);
}

// Two stochastically rounded E2M1 codes (element a in bits 0..3, b in bits 4..7 of
// the result; the bits above are not defined).  a uses the low 16 bits of r, b the
// high 16 bits.  With F = floor(2^16 * position of |s| between its grid
// neighbours), a value rounds up when u16 + F >= 2^16.  gfx950's SR converter adds
// its random operand's top bits (bits 31..10 for the first element of a pair,
// 30..9 for the second) below the kept precision and truncates; the two elements
// of a pair would share random bits, so each element gets its own call, with its
// 16 bits at the top of its window and zeros below, and the wanted nibbles are
// kept.  (Written to byte 0: this converter does not keep the other bytes of its
// destination operand.)
__device__ __forceinline__ uint32_t encode2_sr(float a, float b, uint32_t r) {
  const f32x2 p = {a, b};
  const uint32_t lo = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, p, r << 16, 1.0f, 0);
  const uint32_t hi = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, p, (r >> 1) & 0x7FFF8000u, 1.0f, 0);
  return (lo & 0x0Fu) | (hi & ~0x0Fu);  // one bit-field insert; hi is zero above byte 0
}

// 8 scaled values -> 8 stochastically rounded codes; elements 2j, 2j+1 use r[j].
__device__ __forceinline__ uint32_t encode8_sr(const float s[8], const uint32_t r[4]) {
  const uint32_t b0 = encode2_sr(s[0], s[1], r[0]), b1 = encode2_sr(s[2], s[3], r[1]);
  const uint32_t b2 = encode2_sr(s[4], s[5], r[2]), b3 = encode2_sr(s[6], s[7], r[3]);
  // byte 0 of b0..b3 into bytes 0..3 (selector 0x0c gives a zero byte)
  const uint32_t w = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u) | __builtin_amdgcn_perm(b3, b2, 0x04000c0cu);
  return canon_zero(w);
}

// Philox4x32-10 (Salmon et al., SC'11): counter (c0..c3), key (k0, k1).
struct Philox4 {
  uint32_t v[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                 uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = uint64_t(0xD2511F53u) * c0, p1 = uint64_t(0xCD9E8D57u) * c2;
    // three-input exclusive or (truth table 0x96) in one instruction
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32(uint32_t(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32(uint32_t(p0 >> 32), c3, k1, 0x96);
    c0 = n0;
    c1 = uint32_t(p1);
    c2 = n2;
    c3 = uint32_t(p0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return Philox4{{c0, c1, c2, c3}};
}

// Random bits for the 16 consecutive logical elements starting at index i0 (a
// multiple of 16): two Philox calls, 16 bits per element, element i using the
// half-word (i & 7) of call i >> 3.
__device__ __forceinline__ void sr_bits16(uint64_t i0, uint64_t seed, uint64_t offset, uint32_t r[8]) {
  const uint64_t g = i0 >> 3;
  const uint32_t k0 = uint32_t(seed), k1 = uint32_t(seed >> 32);
  const uint32_t o0 = uint32_t(offset), o1 = uint32_t(offset >> 32);
  Philox4 a = philox4x32_10(uint32_t(g), uint32_t(g >> 32), o0, o1, k0, k1);
  Philox4 b = philox4x32_10(uint32_t(g + 1), uint32_t((g + 1) >> 32), o0, o1, k0, k1);
  r[0] = a.v[0]; r[1] = a.v[1]; r[2] = a.v[2]; r[3] = a.v[3];
  r[4] = b.v[0]; r[5] = b.v[1]; r[6] = b.v[2]; r[7] = b.v[3];
}

// The 64 random signs of 64-group j of the 64-point transform (MS-EDEN's rotation):
// words 0 and 1 of Philox4x32-10 with counter (j as two words, 0, 0) and key (key, 0);
// element t of the group takes bit t % 32 of word t / 32.
__device__ __forceinline__ void rht64_signs(uint64_t group, uint32_t key, uint32_t &w0, uint32_t &w1) {
  const Philox4 p = philox4x32_10(uint32_t(group), uint32_t(group >> 32), 0u, 0u, key, 0u);
  w0 = p.v[0];
  w1 = p.v[1];
}

// The 16 bits of a 64-group's signs that belong to its quarter q (elements 16 q ..
// 16 q + 15), bit r for element 16 q + r.
__device__ __forceinline__ uint32_t rht64_quarter(uint32_t w0, uint32_t w1, int q) {
  return ((q & 2) ? w1 : w0) >> (16 * (q & 1)) & 0xFFFFu;
}

// The 16 random bits of logical block b (MS-EDEN's scale rounding): half-word b & 7
// of Philox4x32-10 with counter (b >> 3 as two words, offset as two words), key seed.
__device__ __forceinline__ uint32_t block_bits16(uint64_t b, uint64_t seed, uint64_t offset) {
  const uint64_t g = b >> 3;
  const Philox4 p = philox4x32_10(uint32_t(g), uint32_t(g >> 32), uint32_t(offset), uint32_t(offset >> 32),
                                  uint32_t(seed), uint32_t(seed >> 32));
  const uint32_t j = uint32_t(b & 7u);
  return (p.v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
}

// Stochastic rounding of a non-negative binary32 y onto the E4M3 grid: with F the
// first 16 bits of y's position between its neighbouring E4M3 values, y goes up one
// code when u16 + F >= 2^16 (the add-and-truncate rule of the elements).  E4M3 codes
// are consecutive in value, so going up is code + 1.  Normal range (y >= 2^-6): the
// code is y's exponent and top 3 mantissa bits, F the next 16 bits.  Subnormal range:
// y * 2^9 (exact) splits into the code (its integer part) and the position.  y >=
// 448 saturates to 0x7E; zero stays zero.
__device__ __forceinline__ uint32_t e4m3_sr(float y, uint32_t u16) {
  if (!(y > 0.0f)) return 0u;
  if (y >= 448.0f) return 0x7Eu;
  uint32_t lo, F;
  if (y >= 0x1p-6f) {
    const uint32_t b = __float_as_uint(y);
    lo = ((((b >> 23) & 0xFFu) - 120u) << 3) | ((b >> 20) & 7u);
    F = (b >> 4) & 0xFFFFu;
  } else {
    const float t = y * 512.0f;
    const float fl = __builtin_floorf(t);
    lo = uint32_t(fl);
    F = uint32_t(__builtin_floorf((t - fl) * 65536.0f));
  }
  return lo + ((u16 + F) >> 16);
}

typedef float f32x2v __attribute__((ext_vector_type(2)));

// MS-EDEN's correction of one block: s the 16 scaled values, codes their
// nearest-even E2M1 codes (two words), sc the block's scale code.  With e the grid
// values of the codes, c = sum s^2 / sum s e (1 when the second sum is not positive),
// each sum over the 16 elements in order, one binary32 operation per step; the new
// scale code is decode(sc) * c rounded stochastically with the block's 16 bits.
// The E2M1 grid values come from gfx950's FP4 -> f32 converter (exact: every E2M1
// value is a binary32 value).
__device__ __forceinline__ uint32_t eden_scale(const float s[16], uint2 codes, uint32_t sc, uint32_t u16) {
  float e[16];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t w = h == 0 ? codes.x : codes.y;
    const f32x2v e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const f32x2v e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const f32x2v e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const f32x2v e3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    e[8 * h + 0] = e0[0]; e[8 * h + 1] = e0[1]; e[8 * h + 2] = e1[0]; e[8 * h + 3] = e1[1];
    e[8 * h + 4] = e2[0]; e[8 * h + 5] = e2[1]; e[8 * h + 6] = e3[0]; e[8 * h + 7] = e3[1];
  }
  float n = 0.0f, d = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) n = n + s[j] * s[j];
#pragma unroll
  for (int j = 0; j < 16; ++j) d = d + s[j] * e[j];
  const float c = d > 0.0f ? n / d : 1.0f;
  return e4m3_sr(e4m3_to_f32(sc) * c, u16);
}

// Butterflies of the 16-point Hadamard transform (distances 1, 2, 4, 8), without
// its factor 1/4: for a maximum of |v| the factor is applied once to the result,
// which gives the same value (multiplying by 1/4 and rounding is monotone, so the
// largest element stays the largest).
__device__ __forceinline__ void hadamard16_unscaled(float v[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

// Scale a 16-block by its multiplier (one binary32 product per element) and
// encode it into 8 bytes (two words), nearest-even or stochastic (r: the 8
// random words of sr_bits16).
__device__ __forceinline__ uint2 encode16_rne(const float v[16], float mult) {
  float s[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) s[j] = v[j] * mult;
  return make_uint2(encode8_rne(s), encode8_rne(s + 8));
}

__device__ __forceinline__ uint2 encode16_sr(const float v[16], float mult, const uint32_t r[8]) {
  float s[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) s[j] = v[j] * mult;
  return make_uint2(encode8_sr(s, r), encode8_sr(s + 8, r + 4));
}

}  // namespace nvfp4
