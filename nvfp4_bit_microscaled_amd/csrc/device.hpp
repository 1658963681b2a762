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
// the bits, clamped to the largest finite code 0x7E.
__device__ __forceinline__ uint32_t e4m3_from_f32(float u) {
  if (!(u > 0.0f)) return 0u;
  if (u < 0.015625f) {                          // below 2^-6: subnormal spacing 2^-9
    return uint32_t(__builtin_rintf(u * 512.0f));  // exact scaling; 8 means 2^-6 = code 0x08
  }
  uint32_t b = __float_as_uint(u);
  // keep 3 fraction bits: add half an output ulp minus one, plus the kept lsb (ties to even)
  b += 0x7FFFFu + ((b >> 20) & 1u);
  int32_t e = int32_t(b >> 23) - 127 + 7;       // E4M3 exponent field
  uint32_t code = (uint32_t(e) << 3) | ((b >> 20) & 7u);
  return (e > 15 || code > 0x7Eu) ? 0x7Eu : code;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  uint32_t e = (code >> 3) & 15u, m = code & 7u;
  if (e == 0) return float(m) * 0.001953125f;  // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// E2M1 magnitude code by counting the midpoints below |s|; a value exactly on a
// midpoint goes to the even code (so the comparisons alternate between > and >=).
__device__ __forceinline__ uint32_t e2m1_rne(float s) {
  float a = __builtin_fabsf(s);
  uint32_t mag = uint32_t(a > 0.25f) + uint32_t(a >= 0.75f) + uint32_t(a > 1.25f) + uint32_t(a >= 1.75f) +
                 uint32_t(a > 2.5f) + uint32_t(a >= 3.5f) + uint32_t(a > 5.0f);
  uint32_t sign = (__float_as_uint(s) >> 31) & (mag != 0u);
  return (sign << 3) | mag;
}

// Stochastic E2M1: lower neighbour by counting the grid points <= |s|, then up when
// r16 < 2^16 * (|s| - lower) / step.  Both sides of that comparison are exact.
__device__ __forceinline__ uint32_t e2m1_sr(float s, uint32_t r16) {
  float a = __builtin_fabsf(s);
  uint32_t mag;
  if (a >= 6.0f) {
    mag = 7u;
  } else {
    uint32_t lo = uint32_t(a >= 0.5f) + uint32_t(a >= 1.0f) + uint32_t(a >= 1.5f) + uint32_t(a >= 2.0f) +
                  uint32_t(a >= 3.0f) + uint32_t(a >= 4.0f);
    // grid point and 2^16 / step for each lower neighbour (codes 0..6)
    float base = lo < 4u ? 0.5f * float(lo) : (lo == 4u ? 2.0f : (lo == 5u ? 3.0f : 4.0f));
    float inv_step_2p16 = lo < 4u ? 131072.0f : (lo < 6u ? 65536.0f : 32768.0f);
    float thresh = (a - base) * inv_step_2p16;  // exact: Sterbenz difference times a power of two
    mag = lo + uint32_t(float(r16) < thresh);
  }
  uint32_t sign = (__float_as_uint(s) >> 31) & (mag != 0u);
  return (sign << 3) | mag;
}

// Philox4x32-10 (Salmon et al., SC'11): counter (c0..c3), key (k0, k1).
struct Philox4 {
  uint32_t v[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                 uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2), lo1 = 0xCD9E8D57u * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
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

// In-place orthonormal random Hadamard transform of a 16-vector.
__device__ __forceinline__ void rht16(float v[16], uint32_t signs) {
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = ((signs >> j) & 1u) ? -v[j] : v[j];
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
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] *= 0.25f;
}

// Scale code and element multiplier of one block from its amax.
__device__ __forceinline__ void block_scale(float amax_b, float s_enc, uint32_t &code, float &mult) {
  const float t = amax_b / 6.0f;
  code = e4m3_from_f32(t * s_enc);
  const float sf = e4m3_to_f32(code);
  mult = sf > 0.0f ? s_enc / sf : 0.0f;
}

// Encode a 16-block into 8 bytes (two uint32 words), nearest-even.
__device__ __forceinline__ uint2 encode16_rne(const float v[16], float mult) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 16; ++j) w[j >> 3] |= e2m1_rne(v[j] * mult) << (4 * (j & 7));
  return make_uint2(w[0], w[1]);
}

// Encode a 16-block stochastically; r holds the 8 random words of sr_bits16.
__device__ __forceinline__ uint2 encode16_sr(const float v[16], float mult, const uint32_t r[8]) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t r16 = (r[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
    w[j >> 3] |= e2m1_sr(v[j] * mult, r16) << (4 * (j & 7));
  }
  return make_uint2(w[0], w[1]);
}

}  // namespace nvfp4
