// quantize.hip -- tensor amax and NVFP4 quantization kernels for gfx950.
//
// Layouts (NVFP4-12B page, paragraph 2: 16-element blocks with an E4M3 scale
// each and an FP32 scale per tensor; 2D scaling for weights; 16x16 random
// Hadamard transforms for the weight-gradient operands; stochastic rounding for
// gradients):
//   rowwise  : the logical tensor is x [R][C]; a block is 16 consecutive
//              elements of a row.  One thread owns one block, so the block amax
//              needs no cross-lane traffic.  A contiguous tensor is walked as a
//              flat array of blocks (two per thread in flight); a strided one row
//              by row.
//   colwise  : the logical tensor is x^T [C][R]; a block is 16 consecutive rows
//              of one column of x.  A workgroup covers 256 columns x 256 rows: a
//              thread owns 8 adjacent columns of a 16-row slab (every load is a
//              16-byte row segment, a wave reads 2 x 512 contiguous bytes per row)
//              and runs the transform down its registers; codes and scales are
//              gathered in LDS and leave as 128-byte runs of each logical row.
//   2D       : 16x16 tiles of x; 16 lanes own one tile (a lane per row), the tile
//              amax is a 16-lane butterfly reduction, and the transposed codes
//              are regrouped through LDS.
// Elements are encoded by gfx950's FP4 converters (nearest-even, or stochastic
// with 16 Philox bits per element), see device.hpp.
// The tensor amax is a separate reduction pass.  Each workgroup's maximum goes to
// the codes buffer of the tensor being quantized and a one-workgroup kernel
// reduces them (fp4_amax alone, or a tensor under 8 KB of codes: an atomicMax on
// the bit pattern of the non-negative float into an output zeroed by a one-thread
// kernel).  No memset node either way.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"
#include "internal.hpp"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;

// Load 8 consecutive elements (16 bytes of bf16, 32 bytes of fp32) as floats.
template <typename T>
__device__ __forceinline__ void load8(const T *p, float v[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t *p, float v[8]) {
  const uint4 q = *reinterpret_cast<const uint4 *>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(w[j] << 16);
    v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
  }
}

template <>
__device__ __forceinline__ void load8<float>(const float *p, float v[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// load8 with every element negated when `neg` (the row's random sign of the
// Hadamard transform): one exclusive or per 32-bit word, i.e. per two bf16.
template <typename T>
__device__ __forceinline__ void load8_neg(const T *p, float v[8], bool neg);

template <>
__device__ __forceinline__ void load8_neg<uint16_t>(const uint16_t *p, float v[8], bool neg) {
  const uint4 q = *reinterpret_cast<const uint4 *>(p);
  const uint32_t f = neg ? 0x80008000u : 0u;
  const uint32_t w[4] = {q.x ^ f, q.y ^ f, q.z ^ f, q.w ^ f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(w[j] << 16);
    v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
  }
}

template <>
__device__ __forceinline__ void load8_neg<float>(const float *p, float v[8], bool neg) {
  load8(p, v);
  const uint32_t f = neg ? 0x80000000u : 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = __uint_as_float(__float_as_uint(v[j]) ^ f);
}

// 16 rows x 8 adjacent columns of x (one 16-row slab), loaded as 16-byte row
// segments and kept as loaded; column j is widened to binary32 when it is used,
// so bf16 data takes half the registers.  Row r is negated when bit r of `neg`
// is set (the random signs of the Hadamard transform down the columns).
template <typename T>
struct Slab8;

template <>
struct Slab8<uint16_t> {
  uint4 w[16];
  __device__ __forceinline__ void load(const uint16_t *p, int64_t ld, uint32_t neg) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint4 q = *reinterpret_cast<const uint4 *>(p + r * ld);
      const uint32_t f = ((neg >> r) & 1u) ? 0x80008000u : 0u;
      w[r] = make_uint4(q.x ^ f, q.y ^ f, q.z ^ f, q.w ^ f);
    }
  }
  __device__ __forceinline__ float at(int r, int j) const {
    const uint32_t v = j >> 1 == 0 ? w[r].x : j >> 1 == 1 ? w[r].y : j >> 1 == 2 ? w[r].z : w[r].w;
    return __uint_as_float((j & 1) ? (v & 0xFFFF0000u) : (v << 16));
  }
};

template <>
struct Slab8<float> {
  float v[16][8];
  __device__ __forceinline__ void load(const float *p, int64_t ld, uint32_t neg) {
#pragma unroll
    for (int r = 0; r < 16; ++r) load8_neg(p + r * ld, v[r], (neg >> r) & 1u);
  }
  __device__ __forceinline__ float at(int r, int j) const { return v[r][j]; }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide max of non-negative values.  With `partial`, workgroup b stores it
// at partial[b] (amax_finish_kernel reduces those); otherwise it is folded into
// *out with one atomic (its bit pattern orders like the value).  The atomics of
// all workgroups serialise on one cache line, about 10 ns each on the MI355X, so
// the partial form is used wherever the caller's output gives room for it.
__device__ __forceinline__ void block_max_to(float v, float *out, float *partial, unsigned slot = blockIdx.x) {
  __shared__ float part[kThreads / 64];
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) part[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = part[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) m = fmaxf(m, part[i]);
    if (partial) partial[slot] = m;
    else atomicMax(reinterpret_cast<unsigned int *>(out), __float_as_uint(m));
  }
  __syncthreads();  // part[] is reused by a second reduction in the same kernel
}

// out[t] = factor * (max of partial[t * n .. t * n + n)) for t < nout (one
// workgroup; factor 1, or MS-EDEN's headroom 7/4).
__global__ __launch_bounds__(kThreads) void amax_finish_kernel(const float *__restrict__ partial, int n, int nout,
                                                               float *out0, float *out1, float factor) {
  __shared__ float part[kThreads / 64];
  for (int t = 0; t < nout; ++t) {
    float m = 0.0f;
    for (int i = threadIdx.x; i < n; i += kThreads) m = fmaxf(m, partial[t * n + i]);
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int i = 1; i < kThreads / 64; ++i) m = fmaxf(m, part[i]);
      *(t == 0 ? out0 : out1) = factor * m;
    }
    __syncthreads();
  }
}

__global__ void zero_f32_kernel(float *p) { *p = 0.0f; }
__global__ void scale_f32_kernel(float *p, float factor) { *p = factor * *p; }
__global__ void copy_scale_f32_kernel(const float *src, float *dst, float factor) { *dst = factor * *src; }
__global__ void zero2_f32_kernel(float *p, float *q) {
  *p = 0.0f;
  *q = 0.0f;
}

// Plain |x| max over [R][C] (row stride ld); 8 elements per thread-step.
template <typename T>
__global__ __launch_bounds__(kThreads) void amax_plain_kernel(const T *__restrict__ x, int64_t R, int64_t C,
                                                             int64_t ld, float *out, float *partial) {
  const int64_t chunks_per_row = C / 8;
  const int64_t total = R * chunks_per_row;
  float m = 0.0f;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < total; i += int64_t(gridDim.x) * kThreads) {
    const int64_t r = i / chunks_per_row, c = (i - r * chunks_per_row) * 8;
    float v[8];
    load8(x + r * ld + c, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, __builtin_fabsf(v[j]));
  }
  block_max_to(m, out, partial);
}

// Plain |x| max of a contiguous tensor: four 16-byte loads in flight per thread.
// The thread's maximum over its chunks of 8 when the tensor is spread over nblk
// workgroups and this is workgroup blk.
template <typename T>
__device__ __forceinline__ float flat_max(const T *__restrict__ x, int64_t nchunks, int64_t blk, int64_t nblk) {
  float m = 0.0f;
  const int64_t stride = nblk * kThreads;
  for (int64_t i = blk * kThreads + threadIdx.x; i < nchunks; i += 4 * stride) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = i + u * stride;
      if (j < nchunks) load8(x + j * 8, v[u]);
      else
#pragma unroll
        for (int e = 0; e < 8; ++e) v[u][e] = 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, __builtin_fabsf(v[u][e]));
  }
  return m;
}

// bf16: the bit patterns of non-negative finite values order like the values, so
// the maximum of |x| is taken on the raw 16-bit patterns with the sign bits
// cleared (one packed integer max per two elements) and widened once at the end.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

template <>
__device__ __forceinline__ float flat_max<uint16_t>(const uint16_t *__restrict__ x, int64_t nchunks, int64_t blk,
                                                    int64_t nblk) {
  u16x2 m = {0, 0};
  const int64_t stride = nblk * kThreads;
  for (int64_t i = blk * kThreads + threadIdx.x; i < nchunks; i += 4 * stride) {
    uint4 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = i + u * stride;
      q[u] = j < nchunks ? *reinterpret_cast<const uint4 *>(x + j * 8) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t w[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[k] & 0x7FFF7FFFu));
    }
  }
  const uint32_t top = m[0] > m[1] ? m[0] : m[1];
  return __uint_as_float(top << 16);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void amax_flat_kernel(const T *__restrict__ x, int64_t nchunks, float *out,
                                                            float *partial) {
  block_max_to(flat_max<T>(x, nchunks, blockIdx.x, gridDim.x), out, partial);
}

// amax after the Hadamard transform along rows (16 contiguous elements).
template <typename T>
__global__ __launch_bounds__(kThreads) void amax_rht_rows_kernel(const T *__restrict__ x, int64_t R, int64_t C,
                                                                int64_t ld, uint32_t signs, float *out,
                                                                float *partial) {
  const int64_t nkb = C / 16;
  const int64_t total = R * nkb;
  float m = 0.0f;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < total; i += int64_t(gridDim.x) * kThreads) {
    const int64_t r = i / nkb, c = (i - r * nkb) * 16;
    float v[16];
    load8(x + r * ld + c, v);
    load8(x + r * ld + c + 8, v + 8);
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = ((signs >> j) & 1u) ? -v[j] : v[j];
    hadamard16_unscaled(v);
#pragma unroll
    for (int j = 0; j < 16; ++j) m = fmaxf(m, __builtin_fabsf(v[j]));
  }
  block_max_to(m * 0.25f, out, partial);  // the transform's factor, once (see hadamard16_unscaled)
}

// amax after the Hadamard transform down columns (16 consecutive rows of x).
// A thread owns 8 adjacent columns of one 16-row slab.
template <typename T>
__global__ __launch_bounds__(kThreads) void amax_rht_cols_kernel(const T *__restrict__ x, int64_t R, int64_t C,
                                                                int64_t ld, uint32_t signs, float *out,
                                                                float *partial) {
  const int64_t cchunks = C / 8, slabs = R / 16;
  const int64_t total = cchunks * slabs;
  float m = 0.0f;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < total; i += int64_t(gridDim.x) * kThreads) {
    const int64_t s = i / cchunks, c = (i - s * cchunks) * 8;
    Slab8<T> sl;
    sl.load(x + s * 16 * ld + c, ld, signs);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float col[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) col[r] = sl.at(r, j);
      hadamard16_unscaled(col);
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, __builtin_fabsf(col[r]));
    }
  }
  block_max_to(m * 0.25f, out, partial);  // the transform's factor, once (see hadamard16_unscaled)
}

// One rowwise block: (optional transform,) block amax, scale, encode.  i0 is the
// block's first logical index (row * C + 16 * kb), which seeds its random bits.
template <bool RHT, bool SR>
__device__ __forceinline__ void quant_block_rows(float v[16], uint32_t signs, uint64_t i0, uint64_t seed,
                                                 uint64_t offset, float s_enc, const float *tab, uint2 &codes,
                                                 uint32_t &sc) {
  float mult;
  if (RHT) {
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = ((signs >> j) & 1u) ? -v[j] : v[j];
    hadamard16_unscaled(v);
    block_scale_quarter(v, s_enc, tab, sc, mult);
  } else {
    float amax_b = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) amax_b = fmaxf(amax_b, __builtin_fabsf(v[j]));
    block_scale(amax_b, s_enc, tab, sc, mult);
  }
  if (SR) {
    uint32_t rb[8];
    sr_bits16(i0, seed, offset, rb);
    codes = encode16_sr(v, mult, rb);
  } else {
    codes = encode16_rne(v, mult);
  }
}

// Rowwise 1D quantization of a contiguous tensor (row stride == C): block b covers
// elements [16 b, 16 b + 16) of the flat array, its codes bytes [8 b, 8 b + 8) and
// scale byte b, and its logical index is 16 b.  Each thread has two blocks in
// flight per step of a grid-stride loop.
template <typename T, bool RHT, bool SR>
__global__ __launch_bounds__(kThreads) void quant_rows_flat_kernel(const T *__restrict__ x, int64_t nblocks,
                                                                  uint32_t signs, uint64_t seed, uint64_t offset,
                                                                  const float *__restrict__ amax_p,
                                                                  uint8_t *__restrict__ codes,
                                                                  uint8_t *__restrict__ scales) {
  __shared__ float tab[kMultTable];
  const float s_enc = encode_scale(*amax_p);
  fill_mult_table(tab, s_enc);
  __syncthreads();
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t b0 = int64_t(blockIdx.x) * kThreads + threadIdx.x; b0 < nblocks; b0 += 2 * stride) {
    const int64_t b1 = b0 + stride;
    float v0[16], v1[16];
    load8(x + b0 * 16, v0);
    load8(x + b0 * 16 + 8, v0 + 8);
    if (b1 < nblocks) {
      load8(x + b1 * 16, v1);
      load8(x + b1 * 16 + 8, v1 + 8);
    }
    uint2 c;
    uint32_t sc;
    quant_block_rows<RHT, SR>(v0, signs, uint64_t(b0) * 16u, seed, offset, s_enc, tab, c, sc);
    *reinterpret_cast<uint2 *>(codes + b0 * 8) = c;
    scales[b0] = uint8_t(sc);
    if (b1 < nblocks) {
      quant_block_rows<RHT, SR>(v1, signs, uint64_t(b1) * 16u, seed, offset, s_enc, tab, c, sc);
      *reinterpret_cast<uint2 *>(codes + b1 * 8) = c;
      scales[b1] = uint8_t(sc);
    }
  }
}

// Two rowwise stochastic layouts of one contiguous tensor that differ only in
// their random draws (offsets off_a and off_b): the transform, the block amax and
// the scale are taken once, and each layout encodes with its own bits.  Both
// layouts share the tensor amax *amax_p.  Bit-identical to two quant_rows_flat_kernel
// launches.
template <typename T, bool RHT>
__global__ __launch_bounds__(kThreads) void quant_rows_flat_pair_kernel(
    const T *__restrict__ x, int64_t nblocks, uint32_t signs, uint64_t seed, uint64_t off_a, uint64_t off_b,
    const float *__restrict__ amax_p, uint8_t *__restrict__ codes_a, uint8_t *__restrict__ scales_a,
    uint8_t *__restrict__ codes_b, uint8_t *__restrict__ scales_b) {
  __shared__ float tab[kMultTable];
  const float s_enc = encode_scale(*amax_p);
  fill_mult_table(tab, s_enc);
  __syncthreads();
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t b = int64_t(blockIdx.x) * kThreads + threadIdx.x; b < nblocks; b += stride) {
    float v[16];
    load8(x + b * 16, v);
    load8(x + b * 16 + 8, v + 8);
    float mult;
    uint32_t sc;
    if (RHT) {
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = ((signs >> j) & 1u) ? -v[j] : v[j];
      hadamard16_unscaled(v);
      block_scale_quarter(v, s_enc, tab, sc, mult);
    } else {
      float amax_b = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) amax_b = fmaxf(amax_b, __builtin_fabsf(v[j]));
      block_scale(amax_b, s_enc, tab, sc, mult);
    }
    uint32_t rb[8];
    sr_bits16(uint64_t(b) * 16u, seed, off_a, rb);
    *reinterpret_cast<uint2 *>(codes_a + b * 8) = encode16_sr(v, mult, rb);
    scales_a[b] = uint8_t(sc);
    sr_bits16(uint64_t(b) * 16u, seed, off_b, rb);
    *reinterpret_cast<uint2 *>(codes_b + b * 8) = encode16_sr(v, mult, rb);
    scales_b[b] = uint8_t(sc);
  }
}

// Rowwise 1D quantization of a strided tensor: one thread per 16-block.  grid.x
// covers the blocks of a row, grid.y strides over rows.
template <typename T, bool RHT, bool SR>
__global__ __launch_bounds__(kThreads) void quant_rows_kernel(const T *__restrict__ x, int64_t R, int64_t C,
                                                             int64_t ld, uint32_t signs, uint64_t seed,
                                                             uint64_t offset, const float *__restrict__ amax_p,
                                                             uint8_t *__restrict__ codes,
                                                             uint8_t *__restrict__ scales) {
  __shared__ float tab[kMultTable];
  const float s_enc = encode_scale(*amax_p);
  fill_mult_table(tab, s_enc);
  __syncthreads();
  const int64_t nkb = C / 16;
  const int64_t kb = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (kb >= nkb) return;
  for (int64_t r = blockIdx.y; r < R; r += gridDim.y) {
    float v[16];
    load8(x + r * ld + kb * 16, v);
    load8(x + r * ld + kb * 16 + 8, v + 8);
    uint2 packed;
    uint32_t sc;
    quant_block_rows<RHT, SR>(v, signs, uint64_t(r) * uint64_t(C) + uint64_t(kb) * 16u, seed, offset, s_enc, tab,
                              packed, sc);
    *reinterpret_cast<uint2 *>(codes + r * (C / 2) + kb * 8) = packed;
    scales[r * nkb + kb] = uint8_t(sc);
  }
}

// Columnwise 1D quantization (logical tensor x^T, blocks down the columns of x),
// the form for rows too long for quant_cols4_kernel's 32-bit row offsets.
// A workgroup covers kColTile columns of x and kColSlabs 16-row slabs of it.
// Thread (wave w, lane l) owns columns 8 (l % 32) .. +7 of the tile and slabs
// 2 w + l / 32 + 8 i (i < kColSlabs / 8).  Codes go to LDS as [column][slab]
// (8 bytes each; the 16-byte slab pairs of a row XOR-swizzled by bits 3..5 of the
// row), scales as [column][slab] bytes, then each logical row leaves as
// contiguous 16-byte stores.
constexpr int kColTile = 256;   // columns of x (logical rows) per workgroup
constexpr int kColSlabs = 16;   // 16-row slabs of x (logical blocks) per workgroup
constexpr int kColRowBytes = kColSlabs * 8;

// Store a columnwise tile gathered in LDS (see quant_cols_kernel): row `row` of the
// tile is logical row c0 + row; its kColSlabs * 8 code bytes start at byte
// slab0 * 8 of that row, a 16-byte chunk holding two slabs; its scales are
// kColSlabs bytes from scale slab0.
__device__ __forceinline__ void store_col_tile(const uint8_t *lcodes, const uint8_t *lscales, int64_t R, int64_t C,
                                               int64_t c0, int64_t slab0, uint8_t *__restrict__ codes,
                                               uint8_t *__restrict__ scales) {
  const int64_t nslab = R / 16;
  const int64_t nvalid = min<int64_t>(int64_t(kColSlabs), nslab - slab0);  // slabs of this tile inside x
  for (int idx = threadIdx.x; idx < kColTile * (kColRowBytes / 16); idx += kThreads) {
    const int row = idx / (kColRowBytes / 16), part = idx % (kColRowBytes / 16);
    const int64_t c = c0 + row;
    if (c >= C || 2 * part >= nvalid) continue;
    const int pair = part ^ ((row >> 3) & 7);
    const uint4 v = *reinterpret_cast<const uint4 *>(&lcodes[row * kColRowBytes + pair * 16]);
    uint8_t *dst = codes + c * (R / 2) + (slab0 + 2 * part) * 8;
    if (2 * part + 1 < nvalid) {
      if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
        *reinterpret_cast<uint4 *>(dst) = v;
      } else {
        *reinterpret_cast<uint2 *>(dst) = make_uint2(v.x, v.y);
        *reinterpret_cast<uint2 *>(dst + 8) = make_uint2(v.z, v.w);
      }
    } else {
      *reinterpret_cast<uint2 *>(dst) = make_uint2(v.x, v.y);
    }
  }
  // scales: kColSlabs bytes per logical row
  for (int row = threadIdx.x; row < kColTile; row += kThreads) {
    const int64_t c = c0 + row;
    if (c >= C) continue;
    uint8_t *dst = scales + c * nslab + slab0;
    const uint8_t *src = &lscales[row * kColSlabs];
    if (nvalid == kColSlabs && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
      *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
    } else {
      for (int k = 0; k < nvalid; ++k) dst[k] = src[k];
    }
  }
}
// At most 168 registers (three waves per SIMD); held to four waves (128) the
// stochastic variant spilled to scratch memory and measured 250 us instead of 212
// per 12B step.
template <typename T, bool RHT, bool SR>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void quant_cols_kernel(
    const T *__restrict__ x, int64_t R, int64_t C, int64_t ld, uint32_t signs, uint64_t seed, uint64_t offset,
    const float *__restrict__ amax_p, uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
  __shared__ __attribute__((aligned(16))) uint8_t lcodes[kColTile * kColRowBytes];
  __shared__ uint8_t lscales[kColTile * kColSlabs];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cg = lane & 31;
  const int64_t c0 = int64_t(blockIdx.x) * kColTile;          // first column of the tile
  const int64_t slab0 = int64_t(blockIdx.y) * kColSlabs;      // first slab of the tile
  const int64_t nslab = R / 16;                                // logical blocks per logical row
  const int64_t cfirst = c0 + 8 * cg;                          // this thread's first column
  __shared__ float tab[kMultTable];
  const float s_enc = encode_scale(*amax_p);
  fill_mult_table(tab, s_enc);
  __syncthreads();

#pragma unroll 1
  for (int i = 0; i < kColSlabs / 8; ++i) {
    const int sl = 2 * wave + (lane >> 5) + 8 * i;             // slab within the tile
    const int64_t s = slab0 + sl;
    if (s >= nslab || cfirst >= C) continue;                   // lanes 2k, 2k + 1 skip together (C % 16 == 0)
    Slab8<T> slab;
    slab.load(x + s * 16 * ld + cfirst, ld, RHT ? signs : 0u);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float col[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) col[r] = slab.at(r, j);
      uint32_t sc;
      float mult;
      if (RHT) {
        hadamard16_unscaled(col);
        block_scale_quarter(col, s_enc, tab, sc, mult);
      } else {
        float amax_b = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) amax_b = fmaxf(amax_b, __builtin_fabsf(col[r]));
        block_scale(amax_b, s_enc, tab, sc, mult);
      }
      const int row = 8 * cg + j;  // logical row within the tile
      uint2 packed;
      if (SR) {
        uint32_t rb[8];
        sr_bits16(uint64_t(cfirst + j) * uint64_t(R) + uint64_t(s) * 16u, seed, offset, rb);
        packed = encode16_sr(col, mult, rb);
      } else {
        packed = encode16_rne(col, mult);
      }
      const int pair = (sl >> 1) ^ ((row >> 3) & 7);
      *reinterpret_cast<uint2 *>(&lcodes[row * kColRowBytes + pair * 16 + (sl & 1) * 8]) = packed;
      lscales[row * kColSlabs + sl] = uint8_t(sc);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();

  store_col_tile(lcodes, lscales, R, C, c0, slab0, codes, scales);
}


// Raw buffer access from a wave-uniform base (wave_rsrc): the descriptor sits in
// scalar registers, each row's byte offset in a scalar register, and only the
// lane's column offset in a vector register, so 16 rows cost no vector address
// arithmetic.

// 16 rows x 4 adjacent columns of x (one 16-row slab), as loaded; row r negated
// when bit r of `neg` is set.  Column j is widened to binary32 when it is used.
// rs: a buffer whose row 0 is the slab's first row; ldb: the row stride in bytes;
// voff: the byte offset of the lane's first element from the buffer's base.
template <typename T>
struct Slab4;

template <>
struct Slab4<uint16_t> {
  uint2 w[16];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t ldb, uint32_t voff, uint32_t neg) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const auto q = __builtin_amdgcn_raw_buffer_load_b64(rs, int(voff), int(uint32_t(r) * ldb), 0);
      const uint32_t f = ((neg >> r) & 1u) ? 0x80008000u : 0u;
      w[r] = make_uint2(q[0] ^ f, q[1] ^ f);
    }
  }
  __device__ __forceinline__ float at(int r, int j) const {
    const uint32_t v = (j >> 1) ? w[r].y : w[r].x;
    return __uint_as_float((j & 1) ? (v & 0xFFFF0000u) : (v << 16));
  }
};

template <>
struct Slab4<float> {
  float v[16][4];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t ldb, uint32_t voff, uint32_t neg) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const auto q = __builtin_amdgcn_raw_buffer_load_b128(rs, int(voff), int(uint32_t(r) * ldb), 0);
      const uint32_t f = ((neg >> r) & 1u) ? 0x80000000u : 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[r][j] = __uint_as_float(q[j] ^ f);
    }
  }
  __device__ __forceinline__ float at(int r, int j) const { return v[r][j]; }
};

// v of quad lane o, in every lane of the quad (DPP quad_perm [o, o, o, o]); o is a
// constant once the caller's loop is unrolled.
template <int O>
__device__ __forceinline__ float quad_bcast_c(float v) {
  return __uint_as_float(uint32_t(__builtin_amdgcn_mov_dpp(int(__float_as_uint(v)), O * 0x55, 0xF, 0xF, false)));
}

__device__ __forceinline__ float quad_bcast(float v, int o) {
  switch (o) {
    case 0: return quad_bcast_c<0>(v);
    case 1: return quad_bcast_c<1>(v);
    case 2: return quad_bcast_c<2>(v);
    default: return quad_bcast_c<3>(v);
  }
}

// Column j of a 4-column slab as one columnwise 16-block (logical row `row` of the
// workgroup's tile, logical block `sl`): the transform down the slab when RHT,
// block scale, then nearest-even or stochastic codes (the 16 random half-words of
// logical index i0) into the LDS tile, swizzled as in quant_cols_kernel.
template <typename T, bool RHT, bool SR>
__device__ __forceinline__ void col_block4(const Slab4<T> &slab, int j, float s_enc, const float *tab, int row, int sl,
                                           uint64_t i0, uint64_t seed, uint64_t offset, uint8_t *lcodes,
                                           uint8_t *lscales) {
  float col[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) col[r] = slab.at(r, j);
  uint32_t sc;
  float mult;
  if (RHT) {
    hadamard16_unscaled(col);
    block_scale_quarter(col, s_enc, tab, sc, mult);
  } else {
    float amax_b = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) amax_b = fmaxf(amax_b, __builtin_fabsf(col[r]));
    block_scale(amax_b, s_enc, tab, sc, mult);
  }
  uint2 packed;
  if (SR) {
    uint32_t rb[8];
    sr_bits16(i0, seed, offset, rb);
    packed = encode16_sr(col, mult, rb);
  } else {
    packed = encode16_rne(col, mult);
  }
  const int pair = (sl >> 1) ^ ((row >> 3) & 7);
  *reinterpret_cast<uint2 *>(&lcodes[row * kColRowBytes + pair * 16 + (sl & 1) * 8]) = packed;
  lscales[row * kColSlabs + sl] = uint8_t(sc);
}

// Columnwise 1D quantization with a thread owning 4 columns of a 16-row slab (the
// tile, LDS gathering and stores of quant_cols_kernel): half the registers of
// that kernel's 8 columns, so four waves share a SIMD, and rows read through
// buffer descriptors with scalar row offsets.  The launcher keeps 16 rows of x
// within 2^31 bytes (beyond that, quant_cols_kernel).  Bit-identical to it.
template <typename T, bool RHT, bool SR>
__global__ __launch_bounds__(kThreads) void quant_cols4_kernel(
    const T *__restrict__ x, int64_t R, int64_t C, int64_t ld, uint32_t signs, uint64_t seed, uint64_t offset,
    const float *__restrict__ amax_p, uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
  __shared__ __attribute__((aligned(16))) uint8_t lcodes[kColTile * kColRowBytes];
  __shared__ uint8_t lscales[kColTile * kColSlabs];
  __shared__ float tab[kMultTable];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c0 = int64_t(blockIdx.x) * kColTile;      // first column of the tile
  const int64_t slab0 = int64_t(blockIdx.y) * kColSlabs;  // first slab of the tile
  const int64_t nslab = R / 16;
  const int64_t cfirst = c0 + 4 * lane;                    // this thread's first column
  const float s_enc = encode_scale(*amax_p);
  fill_mult_table(tab, s_enc);
  __syncthreads();

#pragma unroll 1
  for (int i = 0; i < kColSlabs / 4; ++i) {
    const int sl = wave + 4 * i;  // slab within the tile
    const int64_t s = slab0 + sl;
    if (s >= nslab || cfirst >= C) continue;  // a lane quad skips together (C % 16 == 0)
    Slab4<T> slab;
    slab.load(wave_rsrc(x + s * 16 * ld + c0), uint32_t(ld * int64_t(sizeof(T))), uint32_t(lane * 4 * sizeof(T)),
              RHT ? signs : 0u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      col_block4<T, RHT, SR>(slab, j, s_enc, tab, 4 * lane + j, sl, uint64_t(cfirst + j) * uint64_t(R) + uint64_t(s) * 16u,
                             seed, offset, lcodes, lscales);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();

  store_col_tile(lcodes, lscales, R, C, c0, slab0, codes, scales);
}

// Both nearest-even layouts of x from one read: the columnwise layout (x^T, with
// the transform down 16-row slabs when RHT) and x's rowwise layout (no transform;
// codes [R][C/2], scales [R][C/16], tensor amax *ramax_p).  The tile of a
// workgroup is that of quant_cols_kernel (kColTile columns, kColSlabs slabs), with
// the columnwise codes gathered in LDS the same way and leaving as whole lines.
// Thread (wave w, lane l) owns columns 4 l .. 4 l + 3 of the tile and slabs
// w + 4 i (i < kColSlabs / 4): 16 x 4 elements per step, half of what
// quant_cols_kernel's threads hold, so that four waves share a SIMD (126
// registers; the LDS tile allows no more).  Rows are addressed through buffer
// descriptors with scalar row offsets, which keeps 16 row pointers out of the
// vector registers.
//  * Columnwise: each of the thread's 4 columns is a whole 16-block.
//  * Rowwise: a 16-column block is 4 lanes (a DPP quad); its amax takes two lane
//    exchanges, lane q of the quad computes the scales of rows q, q + 4, q + 8 and
//    q + 12 (and stores their bytes), and each row's multiplier is broadcast from
//    its lane.  The codes leave as 2 bytes per lane, 128 contiguous bytes per row
//    and wave.  A row whose transform sign is set holds -x in the slab; its
//    multiplier is negated, so the products are those of x (nearest-even is
//    symmetric).
// Bit-identical to the separate rowwise and columnwise kernels, and tested so.
// On the MI355X it takes 55 us for the 12B MLP's X (16384 x 5120 bf16, with the
// transform), where the 8-column form with both layouts took 60 us.
template <typename T, bool RHT>
__global__ __launch_bounds__(kThreads) void quant_dual_ne_kernel(
    const T *__restrict__ x, int64_t R, int64_t C, int64_t ld, uint32_t signs, const float *__restrict__ amax_p,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, const float *__restrict__ ramax_p,
    uint8_t *__restrict__ rcodes, uint8_t *__restrict__ rscales) {
  __shared__ __attribute__((aligned(16))) uint8_t lcodes[kColTile * kColRowBytes];
  __shared__ uint8_t lscales[kColTile * kColSlabs];
  __shared__ float tab[kMultTable], rtab[kMultTable];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c0 = int64_t(blockIdx.x) * kColTile;      // first column of the tile
  const int64_t slab0 = int64_t(blockIdx.y) * kColSlabs;  // first slab of the tile
  const int64_t nslab = R / 16;
  const int64_t cfirst = c0 + 4 * lane;                    // this thread's first column
  const float s_enc = encode_scale(*amax_p), rs_enc = encode_scale(*ramax_p);
  fill_mult_table(tab, s_enc);
  fill_mult_table(rtab, rs_enc);
  __syncthreads();

#pragma unroll 1
  for (int i = 0; i < kColSlabs / 4; ++i) {
    const int sl = wave + 4 * i;  // slab within the tile
    const int64_t s = slab0 + sl;
    if (s >= nslab || cfirst >= C) continue;  // a lane quad skips together (C % 16 == 0)
    // wave-uniform bases (the launcher keeps 16 rows of x within 2^31 bytes)
    Slab4<T> slab;
    slab.load(wave_rsrc(x + s * 16 * ld + c0), uint32_t(ld * int64_t(sizeof(T))), uint32_t(lane * 4 * sizeof(T)),
              RHT ? signs : 0u);
    const __amdgpu_buffer_rsrc_t rc = wave_rsrc(rcodes + s * 16 * (C / 2) + c0 / 2);
    const __amdgpu_buffer_rsrc_t rs = wave_rsrc(rscales + s * 16 * (C / 16) + c0 / 16);
    // Rowwise.  Block maxima of the 16 rows: the lane's 4 columns, then the quad's
    // other lanes (DPP quad_perm [1, 0, 3, 2], then [2, 3, 0, 1]), as integers (the
    // bit patterns of non-negative floats order like the values).
    uint32_t mb[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) m = fmaxf(m, __builtin_fabsf(slab.at(r, j)));
      uint32_t u = __float_as_uint(m);
      u = max(u, uint32_t(__builtin_amdgcn_mov_dpp(int(u), 0xB1, 0xF, 0xF, true)));
      u = max(u, uint32_t(__builtin_amdgcn_mov_dpp(int(u), 0x4E, 0xF, 0xF, true)));
      mb[r] = u;
    }
    // Lane q of a quad takes the scales of rows q, q + 4, q + 8 and q + 12, and
    // stores their scale bytes; each row's multiplier comes from its lane (DPP
    // quad_perm broadcast).
    const int q = lane & 3;
    float multk[4];
    uint32_t sck[4], w = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t mq = q == 0 ? mb[4 * k] : q == 1 ? mb[4 * k + 1] : q == 2 ? mb[4 * k + 2] : mb[4 * k + 3];
      block_scale(__uint_as_float(mq), rs_enc, rtab, sck[k], multk[k]);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float mult = quad_bcast(multk[r >> 2], r & 3);
      if (RHT) mult = __uint_as_float(__float_as_uint(mult) ^ (((signs >> r) & 1u) << 31));
      // bytes 0 and 1 of w; the others are not stored (canon_zero works per nibble)
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, slab.at(r, 0) * mult, slab.at(r, 1) * mult, 1.0f, 0);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, slab.at(r, 2) * mult, slab.at(r, 3) * mult, 1.0f, 1);
      __builtin_amdgcn_raw_buffer_store_b16(uint16_t(canon_zero(w)), rc, 2 * lane, int(r * (C / 2)), 0);
      if (q == (r & 3)) __builtin_amdgcn_raw_buffer_store_b8(uint8_t(sck[r >> 2]), rs, lane >> 2, int(r * (C / 16)), 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      col_block4<T, RHT, false>(slab, j, s_enc, tab, 4 * lane + j, sl, 0, 0, 0, lcodes, lscales);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();

  store_col_tile(lcodes, lscales, R, C, c0, slab0, codes, scales);
}

// Both tensor amaxes of a dual quantization in one read: |x| (rowwise layout) and
// |x| after the transform down 16-row slabs (columnwise layout).  A thread owns 8
// adjacent columns of one slab.
template <typename T, bool RHT>
__global__ __launch_bounds__(kThreads) void amax_dual_kernel(const T *__restrict__ x, int64_t R, int64_t C, int64_t ld,
                                                            uint32_t signs, float *out_rows, float *out_cols,
                                                            float *partial) {
  const int64_t cchunks = C / 8, slabs = R / 16;
  const int64_t total = cchunks * slabs;
  float mr = 0.0f, mc = 0.0f;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < total; i += int64_t(gridDim.x) * kThreads) {
    const int64_t sl = i / cchunks, c = (i - sl * cchunks) * 8;
    Slab8<T> slab;
    slab.load(x + sl * 16 * ld + c, ld, RHT ? signs : 0u);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float col[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        col[r] = slab.at(r, j);
        mr = fmaxf(mr, __builtin_fabsf(col[r]));  // the signs do not change |x|
      }
      if (RHT) hadamard16_unscaled(col);
#pragma unroll
      for (int r = 0; r < 16; ++r) mc = fmaxf(mc, __builtin_fabsf(col[r]));
    }
  }
  // partials: rows at [0, grid), columns at [grid, 2 grid)
  block_max_to(mr, out_rows, partial);
  block_max_to(RHT ? mc * 0.25f : mc, out_cols, partial ? partial + gridDim.x : nullptr);  // the transform's
                                                                                            // factor, once
}

// The thread's maxima for amax_dual4_kernel when the units are spread over nblk
// workgroups and this is workgroup blk (mr: x, mc: x^T after the transform,
// without its factor 1/4).
template <typename T, bool RHT, bool ROWS>
__device__ __forceinline__ void dual4_max(const T *__restrict__ x, int64_t R, int64_t C, int64_t ld, uint32_t signs,
                                          int64_t blk, int64_t nblk, float &mr, float &mc) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t cblocks = (C + 255) / 256, units = (R / 16) * cblocks;
  const uint32_t ldb = uint32_t(ld * int64_t(sizeof(T)));
  mr = 0.0f;
  mc = 0.0f;
  for (int64_t u = blk * 4 + wave; u < units; u += nblk * 4) {
    const int64_t sl = u / cblocks, cw = (u - sl * cblocks) * 256;
    if (cw + 4 * lane >= C) continue;  // a lane quad skips together (C % 16 == 0)
    Slab4<T> slab;
    slab.load(wave_rsrc(x + sl * 16 * ld + cw), ldb, uint32_t(lane * 4 * sizeof(T)), RHT ? signs : 0u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float col[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        col[r] = slab.at(r, j);
        if (ROWS) mr = fmaxf(mr, __builtin_fabsf(col[r]));  // the signs do not change |x|
      }
      if (RHT) hadamard16_unscaled(col);
#pragma unroll
      for (int r = 0; r < 16; ++r) mc = fmaxf(mc, __builtin_fabsf(col[r]));
    }
  }
}

// amax_dual_kernel with wave units of one 16-row slab x 256 columns, 4 columns per
// lane and rows read through buffer descriptors (scalar row offsets); the launcher
// keeps 16 rows of x within 2^31 bytes.  Without ROWS only the columnwise amax is
// taken (out_rows unused; partials of the columns at [grid, 2 grid)).
template <typename T, bool RHT, bool ROWS = true>
__global__ __launch_bounds__(kThreads) void amax_dual4_kernel(const T *__restrict__ x, int64_t R, int64_t C,
                                                             int64_t ld, uint32_t signs, float *out_rows,
                                                             float *out_cols, float *partial) {
  float mr, mc;
  dual4_max<T, RHT, ROWS>(x, R, C, ld, signs, blockIdx.x, gridDim.x, mr, mc);
  // partials: rows at [0, grid), columns at [grid, 2 grid)
  if (ROWS) block_max_to(mr, out_rows, partial);
  block_max_to(RHT ? mc * 0.25f : mc, out_cols, partial ? partial + gridDim.x : nullptr);  // the transform's
                                                                                            // factor, once
}

// The forward call's amax passes in one launch: workgroups [0, gx) take x [R][C]
// (contiguous; with XDUAL both of its amaxes as amax_dual4_kernel with the
// transform, partials at xp[0, gx) and xp[gx, 2 gx); otherwise its plain amax as
// amax_flat_kernel, partials at xp[0, gx)), the rest w's plain amax (wchunks
// chunks of 8, partials at wp[0, grid - gx)).
template <typename T, bool XDUAL>
__global__ __launch_bounds__(kThreads) void amax_xw_kernel(const T *__restrict__ x, int64_t R, int64_t C,
                                                          uint32_t signs, unsigned gx, float *xp,
                                                          const T *__restrict__ w, int64_t wchunks, float *wp) {
  if (blockIdx.x < gx) {
    if (XDUAL) {
      float mr, mc;
      dual4_max<T, true, true>(x, R, C, C, signs, blockIdx.x, gx, mr, mc);
      block_max_to(mr, nullptr, xp, blockIdx.x);
      block_max_to(mc * 0.25f, nullptr, xp + gx, blockIdx.x);  // the transform's factor, once
    } else {
      block_max_to(flat_max<T>(x, R * (C / 8), blockIdx.x, gx), nullptr, xp, blockIdx.x);
    }
  } else {
    const unsigned b = blockIdx.x - gx;
    block_max_to(flat_max<T>(w, wchunks, b, gridDim.x - gx), nullptr, wp, b);
  }
}

// The weight gradient's amax passes in one launch: workgroups [0, ga) take a [Ra][Ca]
// (dY) as amax_dual4_kernel with the transform (with A_ROWS its plain amax too:
// partials of the rows at ap[0, ga), of the columns at ap[ga, 2 ga); without, the
// columns at ap[0, ga)), the rest the transformed columnwise amax of b [Rb][Cb] (x),
// partials at bp[0, grid - ga).  Both contiguous.
template <typename T, bool A_ROWS>
__global__ __launch_bounds__(kThreads) void amax_wgrad_kernel(const T *__restrict__ a, int64_t Ra, int64_t Ca,
                                                             unsigned ga, float *ap, const T *__restrict__ b,
                                                             int64_t Rb, int64_t Cb, float *bp, uint32_t signs) {
  float mr, mc;
  if (blockIdx.x < ga) {
    dual4_max<T, true, A_ROWS>(a, Ra, Ca, Ca, signs, blockIdx.x, ga, mr, mc);
    if (A_ROWS) block_max_to(mr, nullptr, ap, blockIdx.x);
    block_max_to(mc * 0.25f, nullptr, A_ROWS ? ap + ga : ap, blockIdx.x);  // the transform's factor, once
  } else {
    const unsigned k = blockIdx.x - ga;
    dual4_max<T, true, false>(b, Rb, Cb, Cb, signs, k, gridDim.x - ga, mr, mc);
    block_max_to(mc * 0.25f, nullptr, bp, k);
  }
}

// Up to three partial-maximum sets reduced at once, one workgroup each: workgroup
// b writes factor[b] times the maximum of p[b][0, n[b]) to *out[b].
struct FinishSets {
  const float *p[3];
  int n[3];
  float *out[3];
  float factor[3];
};

__global__ __launch_bounds__(kThreads) void amax_finish_sets_kernel(FinishSets f) {
  const int b = blockIdx.x;
  float m = 0.0f;
  for (int i = threadIdx.x; i < f.n[b]; i += kThreads) m = fmaxf(m, f.p[b][i]);
  __shared__ float part[kThreads / 64];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < kThreads / 64; ++i) m = fmaxf(m, part[i]);
    *f.out[b] = f.factor[b] * m;
  }
}

// ---------------------------------------------------------------------------
// The 64-point transform (MS-EDEN's rotation) and the kernels that use it.  A
// 64-group is four 16-blocks; each block sits in one thread, and the butterflies at
// distance 16 and 32 pair the block with the group's other blocks held by other
// lanes: lanes 4k .. 4k+3 (rowwise, DPP quad exchanges) or lanes l, l ^ 16, l ^ 32,
// l ^ 48 (columnwise, a 16-row slab per lane).  The butterflies run in the order
// 1, 2, 4, 8 (in registers), then 16 and 32; the factor 1/8 comes last.

// Partner exchange inside a DPP quad: lane ^ 1 (quad_perm [1,0,3,2]) or lane ^ 2
// ([2,3,0,1]).  Every lane of the quad is active whenever one is.
template <int XOR>
__device__ __forceinline__ float quad_xor(float v) {
  constexpr int ctrl = XOR == 1 ? 0xB1 : 0x4E;
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false));
}

// One butterfly stage across lanes: the lane holding the group's lower half keeps
// a + b, the upper one a - b (a from the lower half, b from the upper).
__device__ __forceinline__ float butterfly(float own, float partner, bool upper) {
  return upper ? partner - own : own + partner;
}

// Rowwise: v holds quarter q (= lane & 3 of its quad) of a 64-group, its signs
// (the quarter's 16 bits) not yet applied.
__device__ __forceinline__ void rotate64_quad(float v[16], uint32_t sign16, int q) {
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = ((sign16 >> j) & 1u) ? -v[j] : v[j];
  hadamard16_unscaled(v);
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = butterfly(v[j], quad_xor<1>(v[j]), q & 1);
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = butterfly(v[j], quad_xor<2>(v[j]), q & 2);
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = v[j] * 0.125f;
}

// Columnwise: col holds one column of the 16-row slab that is quarter q (= lane >> 4)
// of its 64-group, signs already applied; partners are lanes ^ 16 and ^ 32, reached
// through the LDS crossbar (ds_bpermute), which runs beside the vector ALU this
// kernel is bound by.  gfx950's permlane swaps (vector-ALU moves) measured 6% slower.
__device__ __forceinline__ void rotate64_cols(float col[16], int q) {
  hadamard16_unscaled(col);
#pragma unroll
  for (int r = 0; r < 16; ++r) col[r] = butterfly(col[r], __shfl_xor(col[r], 16, 64), q & 1);
#pragma unroll
  for (int r = 0; r < 16; ++r) col[r] = butterfly(col[r], __shfl_xor(col[r], 32, 64), q & 2);
#pragma unroll
  for (int r = 0; r < 16; ++r) col[r] = col[r] * 0.125f;
}

// One transformed block: scale, then the elements nearest-even (with EDEN, the
// scale code then corrected), or stochastically.  eb: the block's logical index
// (EDEN's random bits); i0: its first element's logical index (element SR).
template <bool EDEN, bool SR>
__device__ __forceinline__ void quant_block64(const float v[16], float s_enc, const float *tab, uint64_t eb, uint64_t i0,
                                              uint64_t seed, uint64_t offset, uint2 &codes, uint32_t &sc) {
  float amax_b = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) amax_b = fmaxf(amax_b, __builtin_fabsf(v[j]));
  float mult;
  block_scale(amax_b, s_enc, tab, sc, mult);
  float s[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) s[j] = v[j] * mult;
  if (SR) {
    uint32_t rb[8];
    sr_bits16(i0, seed, offset, rb);
    codes = make_uint2(encode8_sr(s, rb), encode8_sr(s + 8, rb + 4));
  } else {
    codes = make_uint2(encode8_rne(s), encode8_rne(s + 8));
    if (EDEN) sc = eden_scale(s, codes, sc, block_bits16(eb, seed, offset));
  }
}

// Rowwise quantization with the 64-point transform, x [R][C] with row stride ld
// (C a multiple of 64): thread q of the grid-stride loop owns logical block q (row
// q / (C/16), block q % (C/16)); quads of lanes hold whole 64-groups.
template <typename T, bool EDEN, bool SR>
__global__ __launch_bounds__(kThreads) void quant_rows64_kernel(const T *__restrict__ x, int64_t R, int64_t C,
                                                               int64_t ld, uint32_t key, uint64_t seed,
                                                               uint64_t offset, const float *__restrict__ amax_p,
                                                               uint8_t *__restrict__ codes,
                                                               uint8_t *__restrict__ scales) {
  __shared__ float tab[kMultTable];
  const float s_enc = encode_scale(*amax_p);
  fill_mult_table(tab, s_enc);
  __syncthreads();
  const int64_t nkb = C / 16, total = R * nkb;
  for (int64_t q = int64_t(blockIdx.x) * kThreads + threadIdx.x; q < total; q += int64_t(gridDim.x) * kThreads) {
    const int64_t r = q / nkb, kb = q - r * nkb;
    float v[16];
    load8(x + r * ld + kb * 16, v);
    load8(x + r * ld + kb * 16 + 8, v + 8);
    uint32_t w0, w1;
    rht64_signs(uint64_t(kb >> 2), key, w0, w1);
    rotate64_quad(v, rht64_quarter(w0, w1, int(kb & 3)), int(kb & 3));
    uint2 c;
    uint32_t sc;
    quant_block64<EDEN, SR>(v, s_enc, tab, uint64_t(q), uint64_t(r) * uint64_t(C) + uint64_t(kb) * 16u, seed, offset,
                            c, sc);
    *reinterpret_cast<uint2 *>(codes + q * 8) = c;
    scales[q] = uint8_t(sc);
  }
}

// MS-EDEN and nearest-even rowwise layouts of one tensor with the same 64-point
// transform, from one read: each block is loaded and rotated once, then quantized
// against each layout's tensor scale (MS-EDEN's amax *amax_e is 7/4 of the
// nearest-even one's, *amax_n).  Bit-identical to two quant_rows64_kernel launches.
template <typename T>
__global__ __launch_bounds__(kThreads) void quant_rows64_pair_kernel(
    const T *__restrict__ x, int64_t R, int64_t C, int64_t ld, uint32_t key, uint64_t seed, uint64_t offset_e,
    const float *__restrict__ amax_e, uint8_t *__restrict__ codes_e, uint8_t *__restrict__ scales_e,
    const float *__restrict__ amax_n, uint8_t *__restrict__ codes_n, uint8_t *__restrict__ scales_n) {
  __shared__ float tab_e[kMultTable], tab_n[kMultTable];
  const float s_enc_e = encode_scale(*amax_e), s_enc_n = encode_scale(*amax_n);
  fill_mult_table(tab_e, s_enc_e);
  fill_mult_table(tab_n, s_enc_n);
  __syncthreads();
  const int64_t nkb = C / 16, total = R * nkb;
  for (int64_t q = int64_t(blockIdx.x) * kThreads + threadIdx.x; q < total; q += int64_t(gridDim.x) * kThreads) {
    const int64_t r = q / nkb, kb = q - r * nkb;
    float v[16];
    load8(x + r * ld + kb * 16, v);
    load8(x + r * ld + kb * 16 + 8, v + 8);
    uint32_t w0, w1;
    rht64_signs(uint64_t(kb >> 2), key, w0, w1);
    rotate64_quad(v, rht64_quarter(w0, w1, int(kb & 3)), int(kb & 3));
    const uint64_t i0 = uint64_t(r) * uint64_t(C) + uint64_t(kb) * 16u;
    uint2 c;
    uint32_t sc;
    quant_block64<true, false>(v, s_enc_e, tab_e, uint64_t(q), i0, seed, offset_e, c, sc);
    *reinterpret_cast<uint2 *>(codes_e + q * 8) = c;
    scales_e[q] = uint8_t(sc);
    quant_block64<false, false>(v, s_enc_n, tab_n, uint64_t(q), i0, seed, 0, c, sc);
    *reinterpret_cast<uint2 *>(codes_n + q * 8) = c;
    scales_n[q] = uint8_t(sc);
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void amax_rht64_rows_kernel(const T *__restrict__ x, int64_t R, int64_t C,
                                                                  int64_t ld, uint32_t key, float *out,
                                                                  float *partial) {
  const int64_t nkb = C / 16, total = R * nkb;
  float m = 0.0f;
  for (int64_t q = int64_t(blockIdx.x) * kThreads + threadIdx.x; q < total; q += int64_t(gridDim.x) * kThreads) {
    const int64_t r = q / nkb, kb = q - r * nkb;
    float v[16];
    load8(x + r * ld + kb * 16, v);
    load8(x + r * ld + kb * 16 + 8, v + 8);
    uint32_t w0, w1;
    rht64_signs(uint64_t(kb >> 2), key, w0, w1);
    rotate64_quad(v, rht64_quarter(w0, w1, int(kb & 3)), int(kb & 3));
#pragma unroll
    for (int j = 0; j < 16; ++j) m = fmaxf(m, __builtin_fabsf(v[j]));
  }
  block_max_to(m, out, partial);
}

// Columnwise quantization with the 64-point transform (logical tensor x^T, groups
// of 64 rows of x; R a multiple of 64).  A workgroup covers kColTile columns and
// kColSlabs 16-row slabs (four groups), as quant_cols_kernel, and leaves through the
// same LDS gather.  Thread (wave w, lane l): columns 128 (w & 1) + 8 (l & 15) .. +7
// of the tile, slab 4 g + (l >> 4) of group g = (w >> 1) + 2 i (i = 0, 1), so the
// four slabs of a group sit in lanes l, l ^ 16, l ^ 32, l ^ 48 of one wave.
template <typename T, bool EDEN, bool SR>
__global__ __launch_bounds__(kThreads) void quant_cols64_kernel(const T *__restrict__ x, int64_t R, int64_t C,
                                                               int64_t ld, uint32_t key, uint64_t seed,
                                                               uint64_t offset, const float *__restrict__ amax_p,
                                                               uint8_t *__restrict__ codes,
                                                               uint8_t *__restrict__ scales) {
  __shared__ __attribute__((aligned(16))) uint8_t lcodes[kColTile * kColRowBytes];
  __shared__ uint8_t lscales[kColTile * kColSlabs];
  __shared__ float tab[kMultTable];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cg = lane & 15, sq = lane >> 4;
  const int64_t c0 = int64_t(blockIdx.x) * kColTile;
  const int64_t slab0 = int64_t(blockIdx.y) * kColSlabs;
  const int64_t nslab = R / 16;
  const int64_t cfirst = c0 + 128 * (wave & 1) + 8 * cg;
  const float s_enc = encode_scale(*amax_p);
  fill_mult_table(tab, s_enc);
  __syncthreads();
#pragma unroll 1
  for (int i = 0; i < 2; ++i) {
    const int sl = 4 * ((wave >> 1) + 2 * i) + sq;  // slab within the tile
    const int64_t s = slab0 + sl;
    // a group is inside or outside x whole (nslab % 4 == 0); lanes l ^ 16, l ^ 32
    // own the same columns, so exchange partners are active together
    if (s >= nslab || cfirst >= C) continue;
    uint32_t w0, w1;
    rht64_signs(uint64_t(s >> 2), key, w0, w1);
    Slab8<T> slab;
    slab.load(x + s * 16 * ld + cfirst, ld, rht64_quarter(w0, w1, sq));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float col[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) col[r] = slab.at(r, j);
      rotate64_cols(col, sq);
      const int64_t c = cfirst + j;  // logical row
      uint2 packed;
      uint32_t sc;
      quant_block64<EDEN, SR>(col, s_enc, tab, uint64_t(c) * uint64_t(nslab) + uint64_t(s),
                              uint64_t(c) * uint64_t(R) + uint64_t(s) * 16u, seed, offset, packed, sc);
      const int row = 128 * (wave & 1) + 8 * cg + j;  // logical row within the tile
      const int pair = (sl >> 1) ^ ((row >> 3) & 7);
      *reinterpret_cast<uint2 *>(&lcodes[row * kColRowBytes + pair * 16 + (sl & 1) * 8]) = packed;
      lscales[row * kColSlabs + sl] = uint8_t(sc);
    }
  }
  __syncthreads();
  store_col_tile(lcodes, lscales, R, C, c0, slab0, codes, scales);
}

// quant_cols64_kernel with a thread owning 4 columns (half the registers, four
// waves per SIMD) and rows read through buffer descriptors.  Wave w takes columns
// 64 w .. 64 w + 63 of the tile and, in step i, group i (slabs 4 i .. 4 i + 3);
// lane l owns columns 64 w + 4 (l & 15) .. +3 of slab 4 i + (l >> 4), so a group's
// four slabs sit in lanes l, l ^ 16, l ^ 32, l ^ 48 as there.  The launcher keeps
// 64 rows of x within 2^31 bytes (beyond that, quant_cols64_kernel).  Bit-identical
// to it.
template <typename T, bool EDEN, bool SR>
__global__ __launch_bounds__(kThreads) void quant_cols64q_kernel(const T *__restrict__ x, int64_t R, int64_t C,
                                                                int64_t ld, uint32_t key, uint64_t seed,
                                                                uint64_t offset, const float *__restrict__ amax_p,
                                                                uint8_t *__restrict__ codes,
                                                                uint8_t *__restrict__ scales) {
  __shared__ __attribute__((aligned(16))) uint8_t lcodes[kColTile * kColRowBytes];
  __shared__ uint8_t lscales[kColTile * kColSlabs];
  __shared__ float tab[kMultTable];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cg = lane & 15, sq = lane >> 4;
  const int64_t c0 = int64_t(blockIdx.x) * kColTile;
  const int64_t slab0 = int64_t(blockIdx.y) * kColSlabs;
  const int64_t nslab = R / 16;
  const int64_t cw = c0 + 64 * wave;  // the wave's first column
  const int64_t cfirst = cw + 4 * cg;
  const uint32_t ldb = uint32_t(ld * int64_t(sizeof(T)));
  const float s_enc = encode_scale(*amax_p);
  fill_mult_table(tab, s_enc);
  __syncthreads();
#pragma unroll 1
  for (int i = 0; i < kColSlabs / 4; ++i) {
    const int sl = 4 * i + sq;  // slab within the tile
    const int64_t s = slab0 + sl;
    // a group is inside or outside x whole (nslab % 4 == 0); lanes l ^ 16, l ^ 32
    // own the same columns, so exchange partners are active together
    if (s >= nslab || cfirst >= C) continue;
    const int64_t g = (slab0 >> 2) + i;  // the group
    uint32_t w0, w1;
    rht64_signs(uint64_t(g), key, w0, w1);
    // the group's first row is the wave-uniform base; the lane's slab is 16 sq rows on
    Slab4<T> slab;
    slab.load(wave_rsrc(x + g * 64 * ld + cw), ldb, 16u * uint32_t(sq) * ldb + uint32_t(cg * 4 * sizeof(T)),
              rht64_quarter(w0, w1, sq));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float col[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) col[r] = slab.at(r, j);
      rotate64_cols(col, sq);
      const int64_t c = cfirst + j;  // logical row
      uint2 packed;
      uint32_t sc;
      quant_block64<EDEN, SR>(col, s_enc, tab, uint64_t(c) * uint64_t(nslab) + uint64_t(s),
                              uint64_t(c) * uint64_t(R) + uint64_t(s) * 16u, seed, offset, packed, sc);
      const int row = 64 * wave + 4 * cg + j;  // logical row within the tile
      const int pair = (sl >> 1) ^ ((row >> 3) & 7);
      *reinterpret_cast<uint2 *>(&lcodes[row * kColRowBytes + pair * 16 + (sl & 1) * 8]) = packed;
      lscales[row * kColSlabs + sl] = uint8_t(sc);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();
  store_col_tile(lcodes, lscales, R, C, c0, slab0, codes, scales);
}

// amax after the 64-point transform down columns: each wave takes units of one
// group (64 rows) x 128 columns, lanes as in quant_cols64_kernel.
template <typename T>
__global__ __launch_bounds__(kThreads) void amax_rht64_cols_kernel(const T *__restrict__ x, int64_t R, int64_t C,
                                                                  int64_t ld, uint32_t key, float *out,
                                                                  float *partial) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cg = lane & 15, sq = lane >> 4;
  const int64_t cblocks = (C + 127) / 128, units = (R / 64) * cblocks;
  float m = 0.0f;
  for (int64_t u = int64_t(blockIdx.x) * 4 + wave; u < units; u += int64_t(gridDim.x) * 4) {
    const int64_t g = u / cblocks, cfirst = (u - g * cblocks) * 128 + 8 * cg;
    if (cfirst >= C) continue;  // lanes l ^ 16, l ^ 32 skip together
    uint32_t w0, w1;
    rht64_signs(uint64_t(g), key, w0, w1);
    Slab8<T> slab;
    slab.load(x + (4 * g + sq) * 16 * ld + cfirst, ld, rht64_quarter(w0, w1, sq));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float col[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) col[r] = slab.at(r, j);
      rotate64_cols(col, sq);
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, __builtin_fabsf(col[r]));
    }
  }
  block_max_to(m, out, partial);
}

// amax_rht64_cols_kernel with units of one group x 64 columns and 4 columns per
// lane (lanes as in quant_cols64q_kernel, rows through buffer descriptors); the
// launcher keeps 64 rows of x within 2^31 bytes.  With ROWS it also takes the plain
// amax of x (every element passes through a lane) into *out_rows, partials of the
// rows at [0, grid) and of the columns at [grid, 2 grid).
template <typename T, bool ROWS = false>
__global__ __launch_bounds__(kThreads) void amax_rht64_cols4_kernel(const T *__restrict__ x, int64_t R, int64_t C,
                                                                   int64_t ld, uint32_t key, float *out,
                                                                   float *partial, float *out_rows) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cg = lane & 15, sq = lane >> 4;
  const int64_t cblocks = (C + 63) / 64, units = (R / 64) * cblocks;
  const uint32_t ldb = uint32_t(ld * int64_t(sizeof(T)));
  float m = 0.0f, mr = 0.0f;
  for (int64_t u = int64_t(blockIdx.x) * 4 + wave; u < units; u += int64_t(gridDim.x) * 4) {
    const int64_t g = u / cblocks, cw = (u - g * cblocks) * 64;
    if (cw + 4 * cg >= C) continue;  // lanes l ^ 16, l ^ 32 skip together
    uint32_t w0, w1;
    rht64_signs(uint64_t(g), key, w0, w1);
    Slab4<T> slab;
    slab.load(wave_rsrc(x + g * 64 * ld + cw), ldb, 16u * uint32_t(sq) * ldb + uint32_t(cg * 4 * sizeof(T)),
              rht64_quarter(w0, w1, sq));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float col[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        col[r] = slab.at(r, j);
        if (ROWS) mr = fmaxf(mr, __builtin_fabsf(col[r]));  // the signs do not change |x|
      }
      rotate64_cols(col, sq);
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, __builtin_fabsf(col[r]));
    }
  }
  if (ROWS) {
    block_max_to(mr, out_rows, partial);
    block_max_to(m, out, partial ? partial + gridDim.x : nullptr);
  } else {
    block_max_to(m, out, partial);
  }
}

// 2D (16x16 tile) nearest-even quantization of x [R][C] (R, C multiples of 16).
// Writes the direct layout (codes [R][C/2], scales [R/16][C/16]) to d_* and/or the
// transposed layout (codes [C][R/2], scales [C/16][R/16]) to t_*; either may be null.
// A workgroup covers a 256x256 block of x (16x16 tiles); wave w takes the block's
// tile-rows w, w + 4, w + 8, w + 12.  Lane l owns tile-column l % 16 and rows
// 4 (l / 16) .. +3 of the current tile-row, so a tile's amax is a reduction over
// its four lanes.  Each element is encoded twice by the converter: paired along
// its row (the direct codes, stored at once as 128-byte runs of each row) and
// paired down its column (the transposed codes, gathered in LDS and stored as
// 128-byte runs of each row of x^T when the block is done).
constexpr int k2dBlock = 256;

template <typename T>
__global__ __launch_bounds__(kThreads) void quant_2d_kernel(const T *__restrict__ x, int64_t R, int64_t C,
                                                           int64_t ld, const float *__restrict__ amax_p,
                                                           uint8_t *__restrict__ d_codes,
                                                           uint8_t *__restrict__ d_scales,
                                                           uint8_t *__restrict__ t_codes,
                                                           uint8_t *__restrict__ t_scales,
                                                           float *__restrict__ amax_copy) {
  // transposed codes: [row of x^T in the block][16 tile-rows x 8 bytes]; the 8-byte
  // slot of tile-row t in row q sits at t ^ (q / 16 % 16), which spreads the 16
  // lanes that write one slot index over distinct banks
  __shared__ __attribute__((aligned(16))) uint8_t tcodes[k2dBlock * 128];
  __shared__ uint8_t tscales[16 * 16];  // [tile-column][tile-row]
  __shared__ float tab[kMultTable];
  const float s_enc = encode_scale(*amax_p);
  // the tensor amax into the other layout's descriptor, once
  if (amax_copy != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *amax_copy = *amax_p;
  fill_mult_table(tab, s_enc);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tcl = lane & 15, rq = lane >> 4;
  const int64_t tiles_r = R / 16, tiles_c = C / 16;
  const int64_t tr0 = int64_t(blockIdx.y) * 16, tc0 = int64_t(blockIdx.x) * 16;  // the block's first tile-row, -column
  const int64_t tc = tc0 + tcl;
#pragma unroll 1
  for (int it = 0; it < 4; ++it) {
    const int trl = wave + 4 * it;  // tile-row within the block
    const int64_t tr = tr0 + trl;
    const bool active = tc < tiles_c && tr < tiles_r;
    float v[4][16];
    float m = 0.0f;
    if (active) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const T *p = x + (tr * 16 + 4 * rq + k) * ld + tc * 16;
        load8(p, v[k]);
        load8(p + 8, v[k] + 8);
#pragma unroll
        for (int j = 0; j < 16; ++j) m = fmaxf(m, __builtin_fabsf(v[k][j]));
      }
    }
    // tile amax over the four lanes of this tile-column (lanes l, l ^ 16, l ^ 32, l ^ 48)
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    uint32_t sc;
    float mult;
    block_scale(m, s_enc, tab, sc, mult);
    if (!active) continue;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int j = 0; j < 16; ++j) v[k][j] *= mult;
    if (d_codes) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint2 c = make_uint2(encode8_rne(v[k]), encode8_rne(v[k] + 8));
        *reinterpret_cast<uint2 *>(d_codes + (tr * 16 + 4 * rq + k) * (C / 2) + tc * 8) = c;
      }
      if (rq == 0) d_scales[tr * tiles_c + tc] = uint8_t(sc);
    }
    if (t_codes) {
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        // columns j, j + 1 of the tile: rows 4rq, 4rq+1 -> byte 2rq of the column's
        // 8 code bytes, rows 4rq+2, 4rq+3 -> byte 2rq+1
        uint32_t w = 0u;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0][j], v[1][j], 1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2][j], v[3][j], 1.0f, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0][j + 1], v[1][j + 1], 1.0f, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2][j + 1], v[3][j + 1], 1.0f, 3);
        w = canon_zero(w);
        const int q = tcl * 16 + j;  // row of x^T within the block; q / 16 % 16 == tcl
        const int slot = (trl ^ tcl) * 8 + 2 * rq;
        *reinterpret_cast<uint16_t *>(&tcodes[q * 128 + slot]) = uint16_t(w);
        *reinterpret_cast<uint16_t *>(&tcodes[(q + 1) * 128 + slot]) = uint16_t(w >> 16);
      }
      if (rq == 0) tscales[tcl * 16 + trl] = uint8_t(sc);
    }
  }
  if (!t_codes) return;
  __syncthreads();
  // 256 rows of x^T x 128 bytes: thread chunk i * 256 + tid is row (i*256 + tid) / 8,
  // 16-byte chunk (tile-rows 2 ch, 2 ch + 1) (i*256 + tid) % 8
  const int64_t nrows_t = min<int64_t>(k2dBlock, C - tc0 * 16);  // rows of x^T in this block
  const int64_t ntr = min<int64_t>(16, tiles_r - tr0);             // tile-rows in this block
#pragma unroll 2
  for (int i = 0; i < 8; ++i) {
    const int q = i * kThreads + threadIdx.x, row = q >> 3, ch = q & 7;
    if (row >= nrows_t || 2 * ch >= ntr) continue;
    const int g = (row >> 4) & 15;
    uint4 v = *reinterpret_cast<const uint4 *>(&tcodes[row * 128 + ((2 * ch) ^ (g & ~1)) * 8]);
    if (g & 1) v = make_uint4(v.z, v.w, v.x, v.y);  // the two slots sit swapped
    uint8_t *dst = t_codes + (tc0 * 16 + row) * (R / 2) + (tr0 + 2 * ch) * 8;
    if (2 * ch + 1 < ntr) {
      if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
        *reinterpret_cast<uint4 *>(dst) = v;
      } else {
        *reinterpret_cast<uint2 *>(dst) = make_uint2(v.x, v.y);
        *reinterpret_cast<uint2 *>(dst + 8) = make_uint2(v.z, v.w);
      }
    } else {
      *reinterpret_cast<uint2 *>(dst) = make_uint2(v.x, v.y);
    }
  }
  if (threadIdx.x < 16 && tc0 + threadIdx.x < tiles_c) {
    uint8_t *dst = t_scales + (tc0 + threadIdx.x) * tiles_r + tr0;
    const uint8_t *src = &tscales[threadIdx.x * 16];
    if (ntr == 16 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
      *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
    } else {
      for (int k = 0; k < ntr; ++k) dst[k] = src[k];
    }
  }
}

unsigned grid_for(int64_t work, int64_t per_block, int64_t cap) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return unsigned(g);
}

// Partial maxima need one float per workgroup (two for the dual amax).  They are
// stored in the codes buffer of the tensor the call is about to quantize, which
// the encoding kernels overwrite afterwards (stream order keeps the reduction
// before them); a codes buffer smaller than this takes the atomic form instead.
constexpr size_t kPartialBytes = 2 * 1024 * sizeof(float);

float *partial_room(const fp4_tensor *t) {
  if (!t || !t->codes) return nullptr;
  const size_t bytes = size_t(t->rows) * size_t(t->cols / 2);
  return bytes >= kPartialBytes ? reinterpret_cast<float *>(t->codes) : nullptr;
}

// Tensor amax into *out.  With `partial` (room for 1024 floats), every workgroup
// stores its maximum there and amax_finish_kernel reduces them; without it, *out
// is zeroed and every workgroup folds its maximum in with an atomic.
// With FP4_Q_EDEN the stored amax is 7/4 of the pass's (MS-EDEN's headroom).
template <typename T>
hipError_t amax_impl(const T *x, int64_t R, int64_t C, int64_t ld, uint32_t flags, uint32_t signs, float *out,
                     float *partial, hipStream_t stream) {
  hipError_t e = hipSuccess;
  const float factor = (flags & FP4_Q_EDEN) ? 1.75f : 1.0f;
  if (R == 0 || C == 0 || !partial) e = launch(zero_f32_kernel, dim3(1), dim3(1), stream, out);
  if (e != hipSuccess || R == 0 || C == 0) return e;
  const int64_t cap = partial ? 1024 : 256 * 16;  // 16 workgroups per CU are plenty for a streaming reduction
  dim3 grid;
  if ((flags & FP4_Q_RHT64) && (flags & FP4_Q_COLWISE) && 64 * ld * int64_t(sizeof(T)) < (int64_t(1) << 31)) {
    grid = dim3(grid_for((R / 64) * ((C + 63) / 64), 4, cap));
    e = launch(amax_rht64_cols4_kernel<T>, grid, dim3(kThreads), stream, x, R, C, ld, signs, out, partial,
               static_cast<float *>(nullptr));
  } else if ((flags & FP4_Q_RHT64) && (flags & FP4_Q_COLWISE)) {
    grid = dim3(grid_for((R / 64) * ((C + 127) / 128), 4, cap));
    e = launch(amax_rht64_cols_kernel<T>, grid, dim3(kThreads), stream, x, R, C, ld, signs, out, partial);
  } else if (flags & FP4_Q_RHT64) {
    grid = dim3(grid_for(R * (C / 16), kThreads * 2, cap));
    e = launch(amax_rht64_rows_kernel<T>, grid, dim3(kThreads), stream, x, R, C, ld, signs, out, partial);
  } else if (!(flags & FP4_Q_RHT) && ld == C) {
    // four workgroups per CU: on the MI355X a 200 MB read-only stream took 37 us with
    // 1024 workgroups, 52 us with 512 (kernel time without the atomics)
    grid = dim3(grid_for(R * (C / 8), kThreads * 4, 1024));
    e = launch(amax_flat_kernel<T>, grid, dim3(kThreads), stream, x, R * (C / 8), out, partial);
  } else if (!(flags & FP4_Q_RHT)) {
    grid = dim3(grid_for(R * (C / 8), kThreads * 4, cap));
    e = launch(amax_plain_kernel<T>, grid, dim3(kThreads), stream, x, R, C, ld, out, partial);
  } else if ((flags & FP4_Q_COLWISE) && 16 * ld * int64_t(sizeof(T)) < (int64_t(1) << 31)) {
    // the dual amax kernel's columnwise half; its partials sit at [grid, 2 grid)
    grid = dim3(grid_for((R / 16) * ((C + 255) / 256), 4, partial ? 512 : cap));
    e = launch(amax_dual4_kernel<T, true, false>, grid, dim3(kThreads), stream, x, R, C, ld, signs,
               static_cast<float *>(nullptr), out, partial);
    if (partial) partial += grid.x;
  } else if (flags & FP4_Q_COLWISE) {
    grid = dim3(grid_for((R / 16) * (C / 8), kThreads, cap));
    e = launch(amax_rht_cols_kernel<T>, grid, dim3(kThreads), stream, x, R, C, ld, signs, out, partial);
  } else {
    grid = dim3(grid_for(R * (C / 16), kThreads * 2, cap));
    e = launch(amax_rht_rows_kernel<T>, grid, dim3(kThreads), stream, x, R, C, ld, signs, out, partial);
  }
  if (e == hipSuccess && partial)
    e = launch(amax_finish_kernel, dim3(1), dim3(kThreads), stream, partial, int(grid.x), 1, out, out, factor);
  else if (e == hipSuccess && factor != 1.0f)
    e = launch(scale_f32_kernel, dim3(1), dim3(1), stream, out, factor);
  return e;
}

template <typename T, bool RHT, bool SR>
hipError_t launch_rows(const T *x, int64_t R, int64_t C, int64_t ld, uint32_t signs, uint64_t seed, uint64_t offset,
                       const fp4_tensor *out, hipStream_t stream) {
  const int64_t nkb = C / 16;
  if (ld == C) {
    const int64_t nblocks = R * nkb;
    return launch(quant_rows_flat_kernel<T, RHT, SR>, dim3(grid_for(nblocks, 2 * kThreads, 1 << 20)), dim3(kThreads),
                  stream, x, nblocks, signs, seed, offset, out->amax, out->codes, out->scales);
  }
  dim3 grid(unsigned((nkb + kThreads - 1) / kThreads), unsigned(R < 65535 ? R : 65535));
  return launch(quant_rows_kernel<T, RHT, SR>, grid, dim3(kThreads), stream, x, R, C, ld, signs, seed, offset,
                out->amax, out->codes, out->scales);
}

template <typename T, bool RHT, bool SR>
hipError_t launch_cols(const T *x, int64_t R, int64_t C, int64_t ld, uint32_t signs, uint64_t seed, uint64_t offset,
                       const fp4_tensor *out, hipStream_t stream) {
  const int64_t nslab = R / 16;
  dim3 grid(unsigned((C + kColTile - 1) / kColTile), unsigned((nslab + kColSlabs - 1) / kColSlabs));
  if (16 * ld * int64_t(sizeof(T)) < (int64_t(1) << 31))
    return launch(quant_cols4_kernel<T, RHT, SR>, grid, dim3(kThreads), stream, x, R, C, ld, signs, seed, offset,
                  out->amax, out->codes, out->scales);
  return launch(quant_cols_kernel<T, RHT, SR>, grid, dim3(kThreads), stream, x, R, C, ld, signs, seed, offset,
                out->amax, out->codes, out->scales);
}

template <typename T, bool EDEN, bool SR>
hipError_t launch_rht64(const T *x, int64_t R, int64_t C, int64_t ld, bool colwise, uint32_t key, uint64_t seed,
                        uint64_t offset, const fp4_tensor *out, hipStream_t stream) {
  if (colwise) {
    const int64_t nslab = R / 16;
    dim3 grid(unsigned((C + kColTile - 1) / kColTile), unsigned((nslab + kColSlabs - 1) / kColSlabs));
    if (64 * ld * int64_t(sizeof(T)) < (int64_t(1) << 31))
      return launch(quant_cols64q_kernel<T, EDEN, SR>, grid, dim3(kThreads), stream, x, R, C, ld, key, seed, offset,
                    out->amax, out->codes, out->scales);
    return launch(quant_cols64_kernel<T, EDEN, SR>, grid, dim3(kThreads), stream, x, R, C, ld, key, seed, offset,
                  out->amax, out->codes, out->scales);
  }
  return launch(quant_rows64_kernel<T, EDEN, SR>, dim3(grid_for(R * (C / 16), kThreads, 1 << 20)), dim3(kThreads),
                stream, x, R, C, ld, key, seed, offset, out->amax, out->codes, out->scales);
}

// Both nearest-even layouts of x in one kernel: cols (x^T, transformed when RHT)
// and rows (x).  Each takes its own tensor amax from its descriptor.
template <typename T, bool RHT>
hipError_t launch_cols_rows(const T *x, int64_t R, int64_t C, int64_t ld, uint32_t signs, const fp4_tensor *cols,
                            const fp4_tensor *rows, hipStream_t stream) {
  const int64_t nslab = R / 16;
  if (16 * ld * int64_t(sizeof(T)) >= (int64_t(1) << 31)) {
    // rows too long for the fused kernel's 32-bit offsets: one kernel per layout
    hipError_t e = launch_cols<T, RHT, false>(x, R, C, ld, signs, 0, 0, cols, stream);
    return e == hipSuccess ? launch_rows<T, false, false>(x, R, C, ld, signs, 0, 0, rows, stream) : e;
  }
  dim3 grid(unsigned((C + kColTile - 1) / kColTile), unsigned((nslab + kColSlabs - 1) / kColSlabs));
  return launch(quant_dual_ne_kernel<T, RHT>, grid, dim3(kThreads), stream, x, R, C, ld, signs, cols->amax,
                cols->codes, cols->scales, rows->amax, rows->codes, rows->scales);
}

template <typename T>
hipError_t quantize_impl(const T *x, int64_t R, int64_t C, int64_t ld, uint32_t flags, uint32_t signs, uint64_t seed,
                         uint64_t offset, const fp4_tensor *out, const fp4_tensor *out_t, hipStream_t stream) {
  if (!(flags & FP4_Q_AMAX_GIVEN)) {
    hipError_t e = amax_impl(x, R, C, ld, flags, signs, out->amax, partial_room(out), stream);
    if (e != hipSuccess) return e;
  }
  if (R == 0 || C == 0) return hipSuccess;
  const bool rht = flags & FP4_Q_RHT, sr = flags & FP4_Q_SR;
  if (flags & FP4_Q_RHT64) {
    const bool cw = flags & FP4_Q_COLWISE;
    if (flags & FP4_Q_EDEN) return launch_rht64<T, true, false>(x, R, C, ld, cw, signs, seed, offset, out, stream);
    if (sr) return launch_rht64<T, false, true>(x, R, C, ld, cw, signs, seed, offset, out, stream);
    return launch_rht64<T, false, false>(x, R, C, ld, cw, signs, seed, offset, out, stream);
  }
  if (flags & FP4_Q_2D) {
    // direct layout is x's; with COLWISE the logical tensor is x^T, so `out` takes
    // the transposed layout and `out_t` the direct one.
    uint8_t *dc = nullptr, *ds = nullptr, *tcp = nullptr, *tsp = nullptr;
    const fp4_tensor *direct = (flags & FP4_Q_COLWISE) ? out_t : out;
    const fp4_tensor *transp = (flags & FP4_Q_COLWISE) ? out : out_t;
    if (direct) { dc = direct->codes; ds = direct->scales; }
    if (transp) { tcp = transp->codes; tsp = transp->scales; }
    const int64_t tiles_c = C / 16, tiles_r = R / 16;
    const dim3 grid(unsigned((tiles_c + 15) / 16), unsigned((tiles_r + 15) / 16));
    float *amax_copy = (out_t && out_t->amax != out->amax) ? out_t->amax : nullptr;
    return launch(quant_2d_kernel<T>, grid, dim3(kThreads), stream, x, R, C, ld, out->amax, dc, ds, tcp, tsp,
                  amax_copy);
  }
  if (flags & FP4_Q_COLWISE) {
    if (rht && sr) return launch_cols<T, true, true>(x, R, C, ld, signs, seed, offset, out, stream);
    if (rht) return launch_cols<T, true, false>(x, R, C, ld, signs, seed, offset, out, stream);
    if (sr) return launch_cols<T, false, true>(x, R, C, ld, signs, seed, offset, out, stream);
    return launch_cols<T, false, false>(x, R, C, ld, signs, seed, offset, out, stream);
  }
  if (rht && sr) return launch_rows<T, true, true>(x, R, C, ld, signs, seed, offset, out, stream);
  if (rht) return launch_rows<T, true, false>(x, R, C, ld, signs, seed, offset, out, stream);
  if (sr) return launch_rows<T, false, true>(x, R, C, ld, signs, seed, offset, out, stream);
  return launch_rows<T, false, false>(x, R, C, ld, signs, seed, offset, out, stream);
}

// Dual quantization: both amaxes in one read of x (unless given), then the layouts.
// Nearest-even: one kernel writes both from one read of x (quant_dual_ne_kernel),
// 18 us faster per 12B step than two kernels.  Stochastic: the rowwise and
// the columnwise kernels in turn; a single kernel measured slower there, since the
// stochastic encoders are bound by vector-ALU work, which fusion does not reduce.
template <typename T>
hipError_t dual_impl(const T *x, int64_t R, int64_t C, int64_t ld, uint32_t flags, uint32_t signs, uint64_t seed,
                     uint64_t off_rows, uint64_t off_cols, const fp4_tensor *rows, const fp4_tensor *cols,
                     hipStream_t stream) {
  const bool rht = flags & FP4_Q_RHT, sr = flags & FP4_Q_SR;
  hipError_t e = hipSuccess;
  if (!(flags & FP4_Q_AMAX_GIVEN)) {
    float *partial = partial_room(rows);  // the rowwise codes (as many bytes as the columnwise ones)
    if (R == 0 || C == 0 || !partial)
      e = launch(zero2_f32_kernel, dim3(1), dim3(1), stream, rows->amax, cols->amax);
    if (e == hipSuccess && R > 0 && C > 0) {
      // two workgroups per CU; with wave units of 256 columns (amax_dual4_kernel) dY of
      // the 12B layer (640 MB) reads in 114-117 us and X (160 MB) in 29-30 us on the
      // MI355X, where per-thread slabs of 8 columns took 123 and 33 us
      dim3 grid;
      if (16 * ld * int64_t(sizeof(T)) < (int64_t(1) << 31)) {
        grid = dim3(grid_for((R / 16) * ((C + 255) / 256), 4, 512));
        e = rht ? launch(amax_dual4_kernel<T, true>, grid, dim3(kThreads), stream, x, R, C, ld, signs, rows->amax,
                         cols->amax, partial)
                : launch(amax_dual4_kernel<T, false>, grid, dim3(kThreads), stream, x, R, C, ld, signs, rows->amax,
                         cols->amax, partial);
      } else {
        grid = dim3(grid_for((R / 16) * (C / 8), kThreads, 512));
        e = rht ? launch(amax_dual_kernel<T, true>, grid, dim3(kThreads), stream, x, R, C, ld, signs, rows->amax,
                         cols->amax, partial)
                : launch(amax_dual_kernel<T, false>, grid, dim3(kThreads), stream, x, R, C, ld, signs, rows->amax,
                         cols->amax, partial);
      }
      if (e == hipSuccess && partial)
        e = launch(amax_finish_kernel, dim3(1), dim3(kThreads), stream, partial, int(grid.x), 2, rows->amax,
                   cols->amax, 1.0f);
    }
  }
  if (e != hipSuccess || R == 0 || C == 0) return e;
  if (!sr) {
    // nearest-even: both layouts from one read of x
    return rht ? launch_cols_rows<T, true>(x, R, C, ld, signs, cols, rows, stream)
               : launch_cols_rows<T, false>(x, R, C, ld, signs, cols, rows, stream);
  }
  e = quantize_impl(x, R, C, ld, FP4_Q_SR | FP4_Q_AMAX_GIVEN, signs, seed, off_rows, rows, nullptr, stream);
  if (e != hipSuccess) return e;
  const uint32_t fc = FP4_Q_COLWISE | FP4_Q_AMAX_GIVEN | FP4_Q_SR | (rht ? FP4_Q_RHT : 0u);
  return quantize_impl(x, R, C, ld, fc, signs, seed, off_cols, cols, nullptr, stream);
}

}  // namespace

hipError_t launch_quantize_dual(const void *x, fp4_dtype dtype, int64_t R, int64_t C, int64_t ld, uint32_t flags,
                                uint32_t signs, uint64_t seed, uint64_t off_rows, uint64_t off_cols,
                                const fp4_tensor *rows, const fp4_tensor *cols, hipStream_t stream) {
  if (dtype == FP4_BF16)
    return dual_impl(static_cast<const uint16_t *>(x), R, C, ld, flags, signs, seed, off_rows, off_cols, rows, cols,
                     stream);
  return dual_impl(static_cast<const float *>(x), R, C, ld, flags, signs, seed, off_rows, off_cols, rows, cols,
                   stream);
}

template <typename T>
hipError_t pair_impl(const T *x, int64_t R, int64_t C, uint32_t flags, uint32_t signs, uint64_t seed, uint64_t off_a,
                     uint64_t off_b, const fp4_tensor *a, const fp4_tensor *b, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (!(flags & FP4_Q_AMAX_GIVEN)) e = amax_impl(x, R, C, C, flags, signs, a->amax, partial_room(a), stream);
  if (e == hipSuccess) e = launch(copy_scale_f32_kernel, dim3(1), dim3(1), stream, a->amax, b->amax, 1.0f);
  if (e != hipSuccess || R == 0 || C == 0) return e;
  const int64_t nblocks = R * (C / 16);
  const dim3 grid(grid_for(nblocks, kThreads, 1 << 20));
  return (flags & FP4_Q_RHT)
             ? launch(quant_rows_flat_pair_kernel<T, true>, grid, dim3(kThreads), stream, x, nblocks, signs, seed,
                      off_a, off_b, a->amax, a->codes, a->scales, b->codes, b->scales)
             : launch(quant_rows_flat_pair_kernel<T, false>, grid, dim3(kThreads), stream, x, nblocks, signs, seed,
                      off_a, off_b, a->amax, a->codes, a->scales, b->codes, b->scales);
}

hipError_t launch_quantize_rows_pair(const void *x, fp4_dtype dtype, int64_t R, int64_t C, uint32_t flags,
                                     uint32_t signs, uint64_t seed, uint64_t off_a, uint64_t off_b,
                                     const fp4_tensor *a, const fp4_tensor *b, hipStream_t stream) {
  if (dtype == FP4_BF16)
    return pair_impl(static_cast<const uint16_t *>(x), R, C, flags, signs, seed, off_a, off_b, a, b, stream);
  return pair_impl(static_cast<const float *>(x), R, C, flags, signs, seed, off_a, off_b, a, b, stream);
}

template <typename T>
hipError_t pair64_impl(const T *x, int64_t R, int64_t C, uint32_t key, uint64_t seed, uint64_t offset_e,
                       const fp4_tensor *eden, const fp4_tensor *ne, hipStream_t stream) {
  hipError_t e = amax_impl(x, R, C, C, FP4_Q_RHT64, key, ne->amax, partial_room(ne), stream);
  if (e == hipSuccess) e = launch(copy_scale_f32_kernel, dim3(1), dim3(1), stream, ne->amax, eden->amax, 1.75f);
  if (e != hipSuccess || R == 0 || C == 0) return e;
  const dim3 grid(grid_for(R * (C / 16), kThreads, 1 << 20));
  return launch(quant_rows64_pair_kernel<T>, grid, dim3(kThreads), stream, x, R, C, C, key, seed, offset_e,
                eden->amax, eden->codes, eden->scales, ne->amax, ne->codes, ne->scales);
}

hipError_t launch_quantize_rows64_pair(const void *x, fp4_dtype dtype, int64_t R, int64_t C, uint32_t key,
                                       uint64_t seed, uint64_t offset_e, const fp4_tensor *eden, const fp4_tensor *ne,
                                       hipStream_t stream) {
  if (dtype == FP4_BF16)
    return pair64_impl(static_cast<const uint16_t *>(x), R, C, key, seed, offset_e, eden, ne, stream);
  return pair64_impl(static_cast<const float *>(x), R, C, key, seed, offset_e, eden, ne, stream);
}

template <typename T>
hipError_t amax_rows_cols64_impl(const T *x, int64_t R, int64_t C, uint32_t key, const fp4_tensor *rows,
                                 const fp4_tensor *cols, hipStream_t stream) {
  if (R == 0 || C == 0 || 64 * C * int64_t(sizeof(T)) >= (int64_t(1) << 31)) {
    hipError_t e = amax_impl(x, R, C, C, 0u, 0u, rows->amax, partial_room(rows), stream);
    return e == hipSuccess ? amax_impl(x, R, C, C, FP4_Q_COLWISE | FP4_Q_RHT64 | FP4_Q_EDEN, key, cols->amax,
                                       partial_room(cols), stream)
                           : e;
  }
  float *partial = partial_room(rows);
  hipError_t e = hipSuccess;
  if (!partial) e = launch(zero2_f32_kernel, dim3(1), dim3(1), stream, rows->amax, cols->amax);
  const dim3 grid(grid_for((R / 64) * ((C + 63) / 64), 4, partial ? 512 : 256 * 16));
  if (e == hipSuccess)
    e = launch(amax_rht64_cols4_kernel<T, true>, grid, dim3(kThreads), stream, x, R, C, C, key, cols->amax, partial,
               rows->amax);
  if (e != hipSuccess) return e;
  if (!partial) return launch(scale_f32_kernel, dim3(1), dim3(1), stream, cols->amax, 1.75f);
  e = launch(amax_finish_kernel, dim3(1), dim3(kThreads), stream, static_cast<const float *>(partial), int(grid.x),
             1, rows->amax, rows->amax, 1.0f);
  return e == hipSuccess ? launch(amax_finish_kernel, dim3(1), dim3(kThreads), stream,
                                  static_cast<const float *>(partial + grid.x), int(grid.x), 1, cols->amax, cols->amax,
                                  1.75f)
                         : e;
}

hipError_t launch_amax_rows_cols64(const void *x, fp4_dtype dtype, int64_t R, int64_t C, uint32_t key,
                                   const fp4_tensor *rows, const fp4_tensor *cols, hipStream_t stream) {
  if (dtype == FP4_BF16)
    return amax_rows_cols64_impl(static_cast<const uint16_t *>(x), R, C, key, rows, cols, stream);
  return amax_rows_cols64_impl(static_cast<const float *>(x), R, C, key, rows, cols, stream);
}

template <typename T>
hipError_t amax_fprop_impl(const T *x, const T *w, int64_t M, int64_t N, int64_t K, uint32_t signs,
                           const fp4_tensor *xq, const fp4_tensor *xq_t, const fp4_tensor *wq, bool *merged,
                           hipStream_t stream) {
  *merged = false;
  float *xp = partial_room(xq), *wp = partial_room(wq);
  const bool dual = xq_t != nullptr;
  if (M == 0 || N == 0 || K == 0 || !xp || !wp || (dual && 16 * K * int64_t(sizeof(T)) >= (int64_t(1) << 31)))
    return hipSuccess;
  const unsigned gx = dual ? grid_for((M / 16) * ((K + 255) / 256), 4, 512) : grid_for(M * (K / 8), kThreads * 4, 1024);
  const unsigned gw = grid_for(N * (K / 8), kThreads * 4, 1024);
  hipError_t e = dual ? launch(amax_xw_kernel<T, true>, dim3(gx + gw), dim3(kThreads), stream, x, M, K, signs, gx, xp,
                               w, N * (K / 8), wp)
                      : launch(amax_xw_kernel<T, false>, dim3(gx + gw), dim3(kThreads), stream, x, M, K, signs, gx,
                               xp, w, N * (K / 8), wp);
  if (e != hipSuccess) return e;
  FinishSets f{};
  int n = 0;
  f.p[n] = xp, f.n[n] = int(gx), f.out[n] = xq->amax, f.factor[n++] = 1.0f;
  if (dual) f.p[n] = xp + gx, f.n[n] = int(gx), f.out[n] = xq_t->amax, f.factor[n++] = 1.0f;
  f.p[n] = wp, f.n[n] = int(gw), f.out[n] = wq->amax, f.factor[n++] = 1.0f;
  e = launch(amax_finish_sets_kernel, dim3(n), dim3(kThreads), stream, f);
  *merged = e == hipSuccess;
  return e;
}

hipError_t launch_amax_fprop(const void *x, const void *w, fp4_dtype dtype, int64_t M, int64_t N, int64_t K,
                             uint32_t signs, const fp4_tensor *xq, const fp4_tensor *xq_t, const fp4_tensor *wq,
                             bool *merged, hipStream_t stream) {
  if (dtype == FP4_BF16)
    return amax_fprop_impl(static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(w), M, N, K, signs, xq,
                           xq_t, wq, merged, stream);
  return amax_fprop_impl(static_cast<const float *>(x), static_cast<const float *>(w), M, N, K, signs, xq, xq_t, wq,
                         merged, stream);
}

template <typename T>
hipError_t amax_wgrad_impl(const T *dy, const T *x, int64_t M, int64_t N, int64_t K, uint32_t signs,
                           const fp4_tensor *dyq, const fp4_tensor *dyq_t, const fp4_tensor *xq_t, bool *merged,
                           hipStream_t stream) {
  *merged = false;
  float *ap = partial_room(dyq_t), *bp = partial_room(xq_t);
  const int64_t lim = int64_t(1) << 31;
  if (M == 0 || N == 0 || K == 0 || !ap || !bp || 16 * N * int64_t(sizeof(T)) >= lim ||
      16 * K * int64_t(sizeof(T)) >= lim)
    return hipSuccess;
  const unsigned ga = grid_for((M / 16) * ((N + 255) / 256), 4, 512);
  const unsigned gb = grid_for((M / 16) * ((K + 255) / 256), 4, 1024);
  hipError_t e = dyq ? launch(amax_wgrad_kernel<T, true>, dim3(ga + gb), dim3(kThreads), stream, dy, M, N, ga, ap, x,
                              M, K, bp, signs)
                     : launch(amax_wgrad_kernel<T, false>, dim3(ga + gb), dim3(kThreads), stream, dy, M, N, ga, ap, x,
                              M, K, bp, signs);
  if (e != hipSuccess) return e;
  FinishSets f{};
  int n = 0;
  if (dyq) f.p[n] = ap, f.n[n] = int(ga), f.out[n] = dyq->amax, f.factor[n++] = 1.0f;
  f.p[n] = dyq ? ap + ga : ap, f.n[n] = int(ga), f.out[n] = dyq_t->amax, f.factor[n++] = 1.0f;
  f.p[n] = bp, f.n[n] = int(gb), f.out[n] = xq_t->amax, f.factor[n++] = 1.0f;
  e = launch(amax_finish_sets_kernel, dim3(n), dim3(kThreads), stream, f);
  *merged = e == hipSuccess;
  return e;
}

hipError_t launch_amax_wgrad(const void *dy, const void *x, fp4_dtype dtype, int64_t M, int64_t N, int64_t K,
                             uint32_t signs, const fp4_tensor *dyq, const fp4_tensor *dyq_t, const fp4_tensor *xq_t,
                             bool *merged, hipStream_t stream) {
  if (dtype == FP4_BF16)
    return amax_wgrad_impl(static_cast<const uint16_t *>(dy), static_cast<const uint16_t *>(x), M, N, K, signs, dyq,
                           dyq_t, xq_t, merged, stream);
  return amax_wgrad_impl(static_cast<const float *>(dy), static_cast<const float *>(x), M, N, K, signs, dyq, dyq_t,
                         xq_t, merged, stream);
}

hipError_t launch_amax_copy(const float *src, float *dst, float factor, hipStream_t stream) {
  return launch(copy_scale_f32_kernel, dim3(1), dim3(1), stream, src, dst, factor);
}

hipError_t launch_amax(const void *x, fp4_dtype dtype, int64_t R, int64_t C, int64_t ld, uint32_t flags,
                       uint32_t signs, float *out, hipStream_t stream) {
  if (dtype == FP4_BF16)
    return amax_impl(static_cast<const uint16_t *>(x), R, C, ld, flags, signs, out, nullptr, stream);
  return amax_impl(static_cast<const float *>(x), R, C, ld, flags, signs, out, nullptr, stream);
}

hipError_t launch_quantize(const void *x, fp4_dtype dtype, int64_t R, int64_t C, int64_t ld, uint32_t flags,
                           uint32_t signs, uint64_t seed, uint64_t offset, const fp4_tensor *out,
                           const fp4_tensor *out_t, hipStream_t stream) {
  if (dtype == FP4_BF16)
    return quantize_impl(static_cast<const uint16_t *>(x), R, C, ld, flags, signs, seed, offset, out, out_t, stream);
  return quantize_impl(static_cast<const float *>(x), R, C, ld, flags, signs, seed, offset, out, out_t, stream);
}

}  // namespace nvfp4
