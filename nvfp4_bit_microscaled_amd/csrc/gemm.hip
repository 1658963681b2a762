// gemm.hip -- NVFP4 block-scaled GEMM for gfx950: C = deq(A) . deq(B)^T, FP32 accumulate.
//
// The GEMMs are the only NVFP4 operations of the layer (NVFP4-12B page,
// paragraph 2: NVFP4 applies to the GEMMs of linear layers only).
//
// How the 16-element E4M3 block scales meet CDNA4's matrix cores.  gfx950's
// block-scaled MFMA (v_mfma_scale_f32_*_f8f6f4) applies one power-of-two (E8M0)
// scale per 32 K-elements.  An NVFP4 pair of blocks inside such a span has two
// independent E4M3 scales, and an E4M3 scale carries 3 mantissa bits that no
// E8M0 scale can hold; folding the mantissa into the elements needs 6
// significant bits (e.g. 1.5 * 1.875), which FP8/FP6/FP4 element formats cannot
// store.  Every such mapping therefore either loses accuracy far beyond the
// 1e-5 acceptance bound or needs four or more passes.  This kernel instead
// dequantizes in registers: an E2M1 value times an E4M3 scale has at most 6
// significant bits and lies in [2^-10, 2688], so it is exact in f16, every
// product of two such values is exact in the f32 accumulator, and the per-tensor
// FP32 scales are applied once in the epilogue.  The products run on
// v_mfma_f32_32x32x16_f16.  FP4 stays FP4 in HBM and in LDS (a quarter of the
// bytes of an f16 GEMM); the conversion is v_cvt_scalef32_pk_f16_fp4 followed by
// a packed f16 multiply by the block scale.
//
// Data flow per workgroup (256 threads, 4 waves in a WAVES_M x WAVES_N grid):
//   K advances in stages of 128 elements = 64 code bytes + 8 scale bytes per row.
//   Global -> registers (next stage, 16-byte loads) while the current stage is
//   consumed from LDS; LDS is double-buffered with one barrier per stage.
//   LDS rows are 64 bytes; the four 16-byte chunks of a row are XOR-swizzled by
//   row bits 1..2 so that 8 consecutive lanes reading one chunk index of 8
//   consecutive rows hit distinct bank groups.
// MFMA operand mapping: a 32x32x16 MFMA takes 8 f16 per lane for A (row l%32) and
// 8 for B (column l%32), lane half g = l/32 supplying one 8-element K group.  Any
// assignment of K values to (g, slot) works as long as A and B use the same one;
// here lane half g of sub-step s (of 4) in half-stage h takes the 8 codes
// [32*(2h+g) + 8s, +8), i.e. one 16-byte chunk per lane serves four MFMAs and
// each lane's 8 values share one block scale.
// Workgroup -> tile order: consecutive workgroup ids go to different XCDs, so ids
// are renumbered to give each XCD a contiguous range, then walked in groups of
// 8 tile-rows so that neighbouring tiles share A rows and B columns in L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"
#include "internal.hpp"

namespace nvfp4 {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 128;       // K elements per stage
constexpr int kRowBytes = 64;  // code bytes per row per stage
constexpr int kGroupM = 8;

struct GemmParams {
  const uint8_t *a_codes, *a_scales, *b_codes, *b_scales;
  const float *a_amax, *b_amax;
  int64_t M, N, K;
  int a_shift, b_shift;  // log2 of rows per scale row: 0 (1D) or 4 (2D)
  void *c;
  int64_t ldc;
  int c_bf16;
};

// 8 E2M1 codes (one 32-bit word, element 2j in the low nibble of byte j) times the
// block scale, as 8 f16.  Exact: see the header comment.
__device__ __forceinline__ half8 dequant8(uint32_t w, half2v sc) {
  const half2v h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sc;
  const half2v h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sc;
  const half2v h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sc;
  const half2v h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sc;
  return half8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

__device__ __forceinline__ half2v scale_h2(uint32_t code) {
  const _Float16 h = _Float16(e4m3_to_f32(code));  // exact: E4M3 values are f16 values
  return half2v{h, h};
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ ((row >> 1) & 3)) << 4); }

template <int BM, int BN, bool FAST>
struct StageRegs {
  uint4 a[BM / 64];
  uint4 b[BN / 64];
  uint2 s[(BM + BN + 255) / 256];
};

// Load the code chunk for (row, byte offset kbyte) of a [rows][kbytes] code matrix.
template <bool FAST>
__device__ __forceinline__ uint4 load_chunk(const uint8_t *base, int64_t row, int64_t rows, int64_t kbytes,
                                            int64_t kbyte) {
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < rows) {
    const uint8_t *p = base + row * kbytes + kbyte;
    if (FAST) {
      v = *reinterpret_cast<const uint4 *>(p);
    } else {
      // rows are only guaranteed 8-byte aligned (K a multiple of 16): two 8-byte loads
      if (kbyte + 8 <= kbytes) {
        const uint2 lo = *reinterpret_cast<const uint2 *>(p);
        v.x = lo.x;
        v.y = lo.y;
      }
      if (kbyte + 16 <= kbytes) {
        const uint2 hi = *reinterpret_cast<const uint2 *>(p + 8);
        v.z = hi.x;
        v.w = hi.y;
      }
    }
  }
  return v;
}

template <bool FAST>
__device__ __forceinline__ uint2 load_scales8(const uint8_t *base, int64_t row, int64_t rows, int shift,
                                              int64_t nkb, int64_t kb0) {
  uint2 v = make_uint2(0u, 0u);
  if (row < rows) {
    const uint8_t *p = base + (row >> shift) * nkb + kb0;
    if (FAST) {
      v = *reinterpret_cast<const uint2 *>(p);
    } else {
      uint32_t w[2] = {0u, 0u};
      for (int j = 0; j < 8; ++j)
        if (kb0 + j < nkb) w[j >> 2] |= uint32_t(p[j]) << (8 * (j & 3));
      v = make_uint2(w[0], w[1]);
    }
  }
  return v;
}

template <int BM, int BN, int WM, int WN, bool FAST>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams p) {
  constexpr int WAVES_N = BN / WN;
  static_assert((BM / WM) * (BN / WN) == 4, "four waves per workgroup");
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int NS = (BM + BN + 255) / 256;

  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BN * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds_s[2][(BM + BN) * 8];

  const int t = threadIdx.x;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int num_m = int((M + BM - 1) / BM), num_n = int((N + BN - 1) / BN);
  int pid = blockIdx.x;
  const int total = gridDim.x;
  if ((total & 7) == 0) pid = (pid & 7) * (total >> 3) + (pid >> 3);
  const int per_group = kGroupM * num_n;
  const int grp = pid / per_group, first_m = grp * kGroupM;
  const int gsz = min(num_m - first_m, kGroupM);
  const int tm = first_m + (pid % per_group) % gsz;
  const int tn = (pid % per_group) / gsz;
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;

  const int64_t kbytes = K / 2, nkb = K / 16;
  const int nstages = int((K + kBK - 1) / kBK);

  StageRegs<BM, BN, FAST> st;
  auto gload = [&](int kt) {
    const int64_t kbyte = int64_t(kt) * kRowBytes + 16 * (t & 3);
#pragma unroll
    for (int i = 0; i < BM / 64; ++i) st.a[i] = load_chunk<FAST>(p.a_codes, m0 + (t >> 2) + 64 * i, M, kbytes, kbyte);
#pragma unroll
    for (int i = 0; i < BN / 64; ++i) st.b[i] = load_chunk<FAST>(p.b_codes, n0 + (t >> 2) + 64 * i, N, kbytes, kbyte);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int r = t + 256 * i;
      const int64_t kb0 = int64_t(kt) * (kBK / 16);
      if (r < BM) st.s[i] = load_scales8<FAST>(p.a_scales, m0 + r, M, p.a_shift, nkb, kb0);
      else if (r < BM + BN) st.s[i] = load_scales8<FAST>(p.b_scales, n0 + (r - BM), N, p.b_shift, nkb, kb0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < BM / 64; ++i)
      *reinterpret_cast<uint4 *>(&lds_a[buf][swz((t >> 2) + 64 * i, t & 3)]) = st.a[i];
#pragma unroll
    for (int i = 0; i < BN / 64; ++i)
      *reinterpret_cast<uint4 *>(&lds_b[buf][swz((t >> 2) + 64 * i, t & 3)]) = st.b[i];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int r = t + 256 * i;
      if (r < BM + BN) *reinterpret_cast<uint2 *>(&lds_s[buf][r * 8]) = st.s[i];
    }
  };

  const int wave = t >> 6, lane = t & 63;
  const int wm = (wave / WAVES_N) * WM, wn = (wave % WAVES_N) * WN;
  const int lr = lane & 31, g = lane >> 5;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  if (nstages > 0) {
    gload(0);
    lstore(0);
    __syncthreads();
  }
  for (int kt = 0; kt < nstages; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nstages) gload(kt + 1);

    uint2 sa[TM], sb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) sa[i] = *reinterpret_cast<const uint2 *>(&lds_s[buf][(wm + 32 * i + lr) * 8]);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      sb[j] = *reinterpret_cast<const uint2 *>(&lds_s[buf][(BM + wn + 32 * j + lr) * 8]);

#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int chunk = 2 * h + g;
      uint4 qa[TM], qb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) qa[i] = *reinterpret_cast<const uint4 *>(&lds_a[buf][swz(wm + 32 * i + lr, chunk)]);
#pragma unroll
      for (int j = 0; j < TN; ++j) qb[j] = *reinterpret_cast<const uint4 *>(&lds_b[buf][swz(wn + 32 * j + lr, chunk)]);
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const int blk = 2 * chunk + pr;  // block (0..7) of this stage
        half2v sca[TM], scb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) sca[i] = scale_h2(((blk < 4 ? sa[i].x : sa[i].y) >> (8 * (blk & 3))) & 0xFFu);
#pragma unroll
        for (int j = 0; j < TN; ++j) scb[j] = scale_h2(((blk < 4 ? sb[j].x : sb[j].y) >> (8 * (blk & 3))) & 0xFFu);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int s = 2 * pr + s2;
          half8 fa[TM], fb[TN];
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            const uint32_t w = s == 0 ? qa[i].x : s == 1 ? qa[i].y : s == 2 ? qa[i].z : qa[i].w;
            fa[i] = dequant8(w, sca[i]);
          }
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const uint32_t w = s == 0 ? qb[j].x : s == 1 ? qb[j].y : s == 2 ? qb[j].z : qb[j].w;
            fb[j] = dequant8(w, scb[j]);
          }
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < nstages) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: apply the two per-tensor decode scales and store.
  const float gscale = decode_scale(*p.a_amax) * decode_scale(*p.b_amax);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t n = n0 + wn + 32 * j + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
        if (m < M && n < N) {
          const float v = acc[i][j][r] * gscale;
          if (p.c_bf16)
            reinterpret_cast<uint16_t *>(p.c)[m * p.ldc + n] = f32_to_bf16(v);
          else
            reinterpret_cast<float *>(p.c)[m * p.ldc + n] = v;
        }
      }
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const GemmParams &p, bool fast, hipStream_t stream) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  if (fast)
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, true>), dim3(unsigned(tiles)), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, false>), dim3(unsigned(tiles)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const fp4_tensor *a, const fp4_tensor *b, void *c, fp4_dtype c_dtype, int64_t ldc,
                       hipStream_t stream) {
  GemmParams p;
  p.a_codes = a->codes;
  p.a_scales = a->scales;
  p.b_codes = b->codes;
  p.b_scales = b->scales;
  p.a_amax = a->amax;
  p.b_amax = b->amax;
  p.M = a->rows;
  p.N = b->rows;
  p.K = a->cols;
  p.a_shift = a->two_d ? 4 : 0;
  p.b_shift = b->two_d ? 4 : 0;
  p.c = c;
  p.ldc = ldc;
  p.c_bf16 = c_dtype == FP4_BF16;
  if (p.M == 0 || p.N == 0) return hipSuccess;
  const bool fast = (p.K % kBK == 0) && (reinterpret_cast<uintptr_t>(a->codes) % 16 == 0) &&
                    (reinterpret_cast<uintptr_t>(b->codes) % 16 == 0) &&
                    (reinterpret_cast<uintptr_t>(a->scales) % 8 == 0) &&
                    (reinterpret_cast<uintptr_t>(b->scales) % 8 == 0);
  return launch_cfg<128, 128, 64, 64>(p, fast, stream);
}

}  // namespace nvfp4
