// hw_converters.hip -- test-only library: the product's own device conversion
// helpers (nvfp4_bit_microscaled_amd/csrc/device.hpp), run over exhaustive and
// dense input sweeps on the GPU so that tests can check them against tables the
// oracle defines.  Not part of the product; nothing in the product loads it.
//
// Every kernel is a grid-stride loop over an explicit element count, writes only
// within the buffers its caller sized, and counts mismatches with one atomic per
// mismatching element (plus the smallest mismatching index, for the report).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../nvfp4_bit_microscaled_amd/csrc/device.hpp"

using namespace nvfp4;

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void report(unsigned long long *bad, unsigned long long *first_bad, uint64_t idx) {
  atomicAdd(bad, 1ull);
  atomicMin(first_bad, static_cast<unsigned long long>(idx));
}

// Number of entries of the ascending table t[0..n) that are <= b (the oracle's
// code of b when t[c] is the first bit pattern the oracle encodes to code c).
__device__ __forceinline__ uint32_t rank(const uint32_t *t, int n, uint32_t b) {
  uint32_t r = 0;
  for (int c = 0; c < n; ++c) r += (t[c] <= b) ? 1u : 0u;
  return r;
}

// E4M3 block-scale codes of every non-negative binary32 with bit pattern in
// [first, first + count), against the oracle's code boundaries: starts[c] is the
// smallest bit pattern the oracle encodes to code c (c = 1..126; code 0 starts at 0).
__global__ __launch_bounds__(kThreads) void e4m3_sweep_kernel(uint32_t first, uint64_t count,
                                                              const uint32_t *__restrict__ starts,
                                                              unsigned long long *bad,
                                                              unsigned long long *first_bad) {
  __shared__ uint32_t t[126];
  for (int c = threadIdx.x; c < 126; c += kThreads) t[c] = starts[c + 1];
  __syncthreads();
  for (uint64_t i = uint64_t(blockIdx.x) * kThreads + threadIdx.x; i < count; i += uint64_t(gridDim.x) * kThreads) {
    const uint32_t b = first + uint32_t(i);
    const uint32_t got = e4m3_from_f32(__uint_as_float(b));
    if (got != rank(t, 126, b)) report(bad, first_bad, b);
  }
}

__global__ __launch_bounds__(kThreads) void e4m3_encode_kernel(const float *__restrict__ x, uint8_t *__restrict__ out,
                                                               int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n; i += int64_t(gridDim.x) * kThreads)
    out[i] = uint8_t(e4m3_from_f32(x[i]));
}

// Nearest-even E2M1 codes (encode8_rne, canonical zero included) of every binary32
// bit pattern in [first, first + count) whose exponent field is not all ones (no
// infinities or NaNs), 8 consecutive patterns per call, against the oracle's
// magnitude boundaries: starts[m] is the smallest non-negative bit pattern the
// oracle encodes to magnitude m (m = 1..7).  Expected code: magnitude of |x| from
// the table, the sign bit of x on top unless the magnitude is 0.
__global__ __launch_bounds__(kThreads) void fp4_rne_sweep_kernel(uint64_t first, uint64_t count,
                                                                 const uint32_t *__restrict__ starts,
                                                                 unsigned long long *bad,
                                                                 unsigned long long *first_bad) {
  uint32_t t[7];
#pragma unroll
  for (int m = 0; m < 7; ++m) t[m] = starts[m + 1];
  const uint64_t groups = count / 8;
  for (uint64_t g = uint64_t(blockIdx.x) * kThreads + threadIdx.x; g < groups; g += uint64_t(gridDim.x) * kThreads) {
    const uint64_t b0 = first + 8 * g;
    if (((b0 >> 23) & 0xFFu) == 0xFFu) continue;  // 8 consecutive patterns share the exponent field
    float s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = __uint_as_float(uint32_t(b0 + j));
    const uint32_t w = encode8_rne(s);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t b = uint32_t(b0 + j);
      uint32_t mag = 0;
#pragma unroll
      for (int m = 0; m < 7; ++m) mag += ((b & 0x7FFFFFFFu) >= t[m]) ? 1u : 0u;
      const uint32_t want = mag == 0 ? 0u : (mag | ((b >> 28) & 8u));
      if (((w >> (4 * j)) & 0xFu) != want) report(bad, first_bad, b);
    }
  }
}

// Stochastic E2M1 codes (encode8_sr, as the quantizers call it) of each value
// vals[i] for every one of the 2^16 random 16-bit values: the value sits in all 8
// element positions of a call, position j drawing u16 = 8 k + j in call k, so that
// every position and every half-word of the random words is exercised.  Expected
// (from the oracle): code lo[i] for u16 < thresh[i], code hi[i] from thresh[i] on
// (thresh = 65536: never rounds up).  A mismatch index is i * 65536 + u16.
__global__ __launch_bounds__(kThreads) void fp4_sr_sweep_kernel(const float *__restrict__ vals,
                                                                const uint32_t *__restrict__ thresh,
                                                                const uint8_t *__restrict__ lo,
                                                                const uint8_t *__restrict__ hi, int64_t n,
                                                                unsigned long long *bad,
                                                                unsigned long long *first_bad) {
  const uint64_t total = uint64_t(n) * 8192u;  // (value, call k) pairs
  for (uint64_t q = uint64_t(blockIdx.x) * kThreads + threadIdx.x; q < total; q += uint64_t(gridDim.x) * kThreads) {
    const uint64_t i = q >> 13;
    const uint32_t k = uint32_t(q & 8191u);
    const float v = vals[i];
    float s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = v;
    uint32_t r[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) r[h] = (8u * k + 2u * h) | ((8u * k + 2u * h + 1u) << 16);
    const uint32_t w = encode8_sr(s, r);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t u = 8u * k + j;
      const uint32_t want = u < thresh[i] ? lo[i] : hi[i];
      if (((w >> (4 * j)) & 0xFu) != want) report(bad, first_bad, i * 65536u + u);
    }
  }
}

// Stochastic codes of n values with given 16-bit random values (elements in pairs
// through encode2_sr, the quantizers' two-element step; n even).
__global__ __launch_bounds__(kThreads) void fp4_sr_encode_kernel(const float *__restrict__ x,
                                                                 const uint16_t *__restrict__ u16,
                                                                 uint8_t *__restrict__ codes, int64_t n) {
  for (int64_t p = int64_t(blockIdx.x) * kThreads + threadIdx.x; 2 * p < n; p += int64_t(gridDim.x) * kThreads) {
    const uint32_t r = uint32_t(u16[2 * p]) | (uint32_t(u16[2 * p + 1]) << 16);
    const uint32_t w = canon_zero(encode2_sr(x[2 * p], x[2 * p + 1], r) & 0xFFu);
    codes[2 * p] = uint8_t(w & 0xFu);
    codes[2 * p + 1] = uint8_t((w >> 4) & 0xFu);
  }
}

// The GEMM's operand dequantization, exhaustively: for scale-code pair index p
// (scale codes 2p & 127 and (2p + 1) & 127 in the low two bytes of the scale
// word), code byte c and selector sel, dequant2 of byte c placed at byte sel of the
// code word, times the f16 of the first scale code of the pair (sel even) or the
// second (sel odd), as the GEMM pairs them.  Selectors are compile-time constants,
// as in the GEMM, and each pair leaves as one 32-bit word.  out[(p * 256 + c) * 4 +
// sel]: the two f16 of the pair, element 0 in the low half.
__global__ __launch_bounds__(kThreads) void dequant_table_kernel(uint32_t *__restrict__ out) {
  const int p = blockIdx.x;  // 64 scale pairs
  const uint32_t sw = uint32_t((2 * p) & 127) | (uint32_t((2 * p + 1) & 127) << 8);
  const f16x2 sc = e4m3x2_to_f16(sw);
  for (int c = threadIdx.x; c < 256; c += kThreads) {
    const int o = (p * 256 + c) * 4;
    out[o + 0] = __builtin_bit_cast(uint32_t, dequant2(uint32_t(c), 0, sc[0]));
    out[o + 1] = __builtin_bit_cast(uint32_t, dequant2(uint32_t(c) << 8, 1, sc[1]));
    out[o + 2] = __builtin_bit_cast(uint32_t, dequant2(uint32_t(c) << 16, 2, sc[0]));
    out[o + 3] = __builtin_bit_cast(uint32_t, dequant2(uint32_t(c) << 24, 3, sc[1]));
  }
}

// The FP4 -> f32 converter MS-EDEN reads its grid values with (scale operand 1):
// out[(c * 4 + sel) * 2 + e] = element e of byte c placed at byte sel.
__global__ __launch_bounds__(kThreads) void fp4_f32_table_kernel(float *__restrict__ out) {
  for (int c = threadIdx.x; c < 256; c += kThreads) {
    const f32x2v a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(uint32_t(c), 1.0f, 0);
    const f32x2v b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(uint32_t(c) << 8, 1.0f, 1);
    const f32x2v d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(uint32_t(c) << 16, 1.0f, 2);
    const f32x2v g = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(uint32_t(c) << 24, 1.0f, 3);
    const int o = c * 8;
    out[o + 0] = a[0]; out[o + 1] = a[1]; out[o + 2] = b[0]; out[o + 3] = b[1];
    out[o + 4] = d[0]; out[o + 5] = d[1]; out[o + 6] = g[0]; out[o + 7] = g[1];
  }
}

// The FP4 -> f16 converter with an f32 scale operand other than 1 (the property
// that makes the GEMM apply the E4M3 scale by a separate multiply): the two
// elements of code byte bytes[i] (at byte 0) with scale operand scales[i], as one
// 32-bit word (element 0 in the low half).
__global__ __launch_bounds__(kThreads) void fp4_cvt_scaled_kernel(const uint8_t *__restrict__ bytes,
                                                                  const float *__restrict__ scales,
                                                                  uint32_t *__restrict__ out, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n; i += int64_t(gridDim.x) * kThreads) {
    out[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(uint32_t(bytes[i]), scales[i], 0));
  }
}

unsigned grid(uint64_t work) {
  const uint64_t g = (work + kThreads - 1) / kThreads;
  return unsigned(g < 1 ? 1 : (g > 65536 ? 65536 : g));
}

}  // namespace

extern "C" {

// Each call enqueues one kernel on `stream`; `bad` and `first_bad` are device
// counters the caller zeroes / sets to ~0 beforehand.  Returns the launch status.
__attribute__((visibility("default"))) int hwc_e4m3_sweep(uint32_t first, uint64_t count, const uint32_t *starts,
                                                          unsigned long long *bad, unsigned long long *first_bad,
                                                          hipStream_t stream) {
  hipLaunchKernelGGL(e4m3_sweep_kernel, dim3(grid(count)), dim3(kThreads), 0, stream, first, count, starts, bad,
                     first_bad);
  return int(hipPeekAtLastError());
}

__attribute__((visibility("default"))) int hwc_e4m3_encode(const float *x, uint8_t *out, int64_t n,
                                                           hipStream_t stream) {
  hipLaunchKernelGGL(e4m3_encode_kernel, dim3(grid(uint64_t(n))), dim3(kThreads), 0, stream, x, out, n);
  return int(hipPeekAtLastError());
}

__attribute__((visibility("default"))) int hwc_fp4_rne_sweep(uint64_t first, uint64_t count, const uint32_t *starts,
                                                             unsigned long long *bad, unsigned long long *first_bad,
                                                             hipStream_t stream) {
  hipLaunchKernelGGL(fp4_rne_sweep_kernel, dim3(grid(count / 8)), dim3(kThreads), 0, stream, first, count, starts,
                     bad, first_bad);
  return int(hipPeekAtLastError());
}

__attribute__((visibility("default"))) int hwc_fp4_sr_sweep(const float *vals, const uint32_t *thresh,
                                                            const uint8_t *lo, const uint8_t *hi, int64_t n,
                                                            unsigned long long *bad, unsigned long long *first_bad,
                                                            hipStream_t stream) {
  hipLaunchKernelGGL(fp4_sr_sweep_kernel, dim3(grid(uint64_t(n) * 8192u)), dim3(kThreads), 0, stream, vals, thresh,
                     lo, hi, n, bad, first_bad);
  return int(hipPeekAtLastError());
}

__attribute__((visibility("default"))) int hwc_fp4_sr_encode(const float *x, const uint16_t *u16, uint8_t *codes,
                                                             int64_t n, hipStream_t stream) {
  hipLaunchKernelGGL(fp4_sr_encode_kernel, dim3(grid(uint64_t(n / 2))), dim3(kThreads), 0, stream, x, u16, codes,
                     n);
  return int(hipPeekAtLastError());
}

__attribute__((visibility("default"))) int hwc_dequant_table(uint32_t *out, hipStream_t stream) {
  hipLaunchKernelGGL(dequant_table_kernel, dim3(64), dim3(kThreads), 0, stream, out);
  return int(hipPeekAtLastError());
}

__attribute__((visibility("default"))) int hwc_fp4_cvt_scaled(const uint8_t *bytes, const float *scales,
                                                              uint32_t *out, int64_t n, hipStream_t stream) {
  hipLaunchKernelGGL(fp4_cvt_scaled_kernel, dim3(grid(uint64_t(n))), dim3(kThreads), 0, stream, bytes, scales, out,
                     n);
  return int(hipPeekAtLastError());
}

__attribute__((visibility("default"))) int hwc_fp4_f32_table(float *out, hipStream_t stream) {
  hipLaunchKernelGGL(fp4_f32_table_kernel, dim3(1), dim3(kThreads), 0, stream, out);
  return int(hipPeekAtLastError());
}

}  // extern "C"
