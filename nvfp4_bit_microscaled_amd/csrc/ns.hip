// ns.hip -- the element-wise and reduction kernels of the NVFP4 Newton-Schulz
// iteration (Full-Stack FP4 pages, paragraph 1: the Muon optimizer's
// Newton-Schulz iterations run natively in NVFP4).  The iteration's products are
// fp4_gemm calls on quantized operands; what runs here is binary32 arithmetic
// between them, one IEEE operation per step (built with -ffp-contract=off):
//   y = alpha x + beta y          (fl(fl(alpha x) + fl(beta y))), optionally with max |y|
//   x0 = g * s, s = RN32(1 / (sqrt(sum g^2) + eps)), the sum of squares in binary64
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.hpp"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;
constexpr int kSumBlocks = 1024;  // workgroups of the sum of squares (and binary64 partials)

// y[i] = alpha * x[i] + beta * y[i], four elements per thread-step (n % 4 == 0,
// both 16-byte aligned).  With AMAX, workgroup b also stores the maximum |y| over
// the elements it wrote at partial[b] (max_finish_kernel reduces those): the
// amax that the quantization of y would otherwise take in a pass of its own.
template <bool AMAX>
__global__ __launch_bounds__(kThreads) void axpby_kernel(float alpha, const float4 *__restrict__ x, float beta,
                                                         float4 *__restrict__ y, int64_t n4, float *partial) {
  float m = 0.0f;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n4; i += int64_t(gridDim.x) * kThreads) {
    const float4 a = x[i], b = y[i];
    const float va[4] = {a.x, a.y, a.z, a.w}, vb[4] = {b.x, b.y, b.z, b.w};
    float r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float p = alpha * va[k];
      const float q = beta * vb[k];
      r[k] = p + q;
      if (AMAX) m = fmaxf(m, __builtin_fabsf(r[k]));
    }
    y[i] = make_float4(r[0], r[1], r[2], r[3]);
  }
  if constexpr (AMAX) {
    __shared__ float part[kThreads / 64];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
      for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, part[w]);
      partial[blockIdx.x] = m;
    }
  }
}

// *out0 (and *out1 when given) = max of partial[0 .. n) (one workgroup).
__global__ __launch_bounds__(kThreads) void max_finish_kernel(const float *__restrict__ partial, int n, float *out0,
                                                              float *out1) {
  __shared__ float part[kThreads / 64];
  float m = 0.0f;
  for (int i = threadIdx.x; i < n; i += kThreads) m = fmaxf(m, partial[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, part[w]);
    *out0 = m;
    if (out1) *out1 = m;
  }
}

// Per-workgroup binary64 partial sums of g[i]^2 (each square exact in binary64),
// in a fixed order: thread t of workgroup b sums the 16-byte vectors
// i = b * T + t + k * G * T in k order (their four squares in element order), then
// the workgroup sums its threads pairwise by a fixed tree.
__global__ __launch_bounds__(kThreads) void sumsq_kernel(const float4 *__restrict__ g, int64_t n4,
                                                         double *__restrict__ partial) {
  __shared__ double part[kThreads];
  double s = 0.0;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n4; i += int64_t(gridDim.x) * kThreads) {
    const float4 v = g[i];
    const double a = v.x, b = v.y, c = v.z, d = v.w;
    s += a * a;
    s += b * b;
    s += c * c;
    s += d * d;
  }
  part[threadIdx.x] = s;
  __syncthreads();
  for (int h = kThreads / 2; h > 0; h >>= 1) {
    if (int(threadIdx.x) < h) part[threadIdx.x] += part[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = part[0];
}

// s = RN32(1 / (sqrt(sum of the partials) + eps)) into *scale (one wave, a fixed
// order: lane l sums partials l, l + 64, ... in index order, then the lanes are
// summed by a fixed butterfly).
__global__ __launch_bounds__(64) void inv_norm_kernel(const double *__restrict__ partial, int nparts, float eps,
                                                      float *scale) {
  double ss = 0.0;
  for (int i = threadIdx.x; i < nparts; i += 64) ss += partial[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if (threadIdx.x == 0) *scale = float(1.0 / (sqrt(ss) + double(eps)));
}

// x = g * s, 16-byte vectors (g and x may be the same array).
__global__ __launch_bounds__(kThreads) void scale_kernel(const float4 *g, const float *__restrict__ scale, float4 *x,
                                                         int64_t n4) {
  const float s = *scale;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n4; i += int64_t(gridDim.x) * kThreads) {
    const float4 v = g[i];
    x[i] = make_float4(v.x * s, v.y * s, v.z * s, v.w * s);
  }
}

unsigned grid_of(int64_t n) {
  const int64_t g = (n + kThreads - 1) / kThreads;
  return unsigned(g < 1 ? 1 : (g > 4096 ? 4096 : g));
}

}  // namespace

hipError_t launch_axpby(float alpha, const float *x, float beta, float *y, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  return launch(axpby_kernel<false>, dim3(grid_of(n / 4)), dim3(kThreads), stream, alpha,
                reinterpret_cast<const float4 *>(x), beta, reinterpret_cast<float4 *>(y), n / 4,
                static_cast<float *>(nullptr));
}

int axpby_parts(int64_t n) { return int(grid_of(n / 4)); }

hipError_t launch_axpby_amax(float alpha, const float *x, float beta, float *y, int64_t n, float *partial,
                             hipStream_t stream) {
  if (n == 0) return hipSuccess;
  return launch(axpby_kernel<true>, dim3(grid_of(n / 4)), dim3(kThreads), stream, alpha,
                reinterpret_cast<const float4 *>(x), beta, reinterpret_cast<float4 *>(y), n / 4, partial);
}

hipError_t launch_max_finish(const float *partial, int n, float *out0, float *out1, hipStream_t stream) {
  return launch(max_finish_kernel, dim3(1), dim3(kThreads), stream, partial, n, out0, out1);
}

size_t normalize_scratch_bytes() { return kSumBlocks * sizeof(double) + sizeof(float); }

size_t axpby_partial_bytes() { return 4096 * sizeof(float); }  // grid_of's cap

// x = g / (|g|_F + eps); n % 4 == 0 and g, x 16-byte aligned (else hipErrorInvalidValue);
// scratch: normalize_scratch_bytes(), 8-byte aligned.
hipError_t launch_normalize(const float *g, float *x, int64_t n, float eps, void *scratch, hipStream_t stream) {
  if (n % 4 != 0 || (reinterpret_cast<uintptr_t>(g) & 15) != 0 || (reinterpret_cast<uintptr_t>(x) & 15) != 0)
    return hipErrorInvalidValue;
  double *partial = static_cast<double *>(scratch);
  float *scale = reinterpret_cast<float *>(partial + kSumBlocks);
  const int64_t n4 = n / 4, blocks = (n4 + kThreads - 1) / kThreads;
  const int nparts = int(blocks < 1 ? 1 : (blocks > kSumBlocks ? kSumBlocks : blocks));
  hipError_t e = launch(sumsq_kernel, dim3(nparts), dim3(kThreads), stream, reinterpret_cast<const float4 *>(g), n4,
                        partial);
  if (e == hipSuccess) e = launch(inv_norm_kernel, dim3(1), dim3(64), stream, static_cast<const double *>(partial),
                                  nparts, eps, scale);
  if (e == hipSuccess && n > 0)
    e = launch(scale_kernel, dim3(grid_of(n4)), dim3(kThreads), stream, reinterpret_cast<const float4 *>(g),
               static_cast<const float *>(scale), reinterpret_cast<float4 *>(x), n4);
  return e;
}

}  // namespace nvfp4
