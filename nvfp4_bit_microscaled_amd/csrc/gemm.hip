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
// 1e-5 acceptance bound or needs four or more passes.  These kernels instead
// dequantize in registers: an E2M1 value times an E4M3 scale has at most 6
// significant bits and lies in [2^-10, 2688], so it is exact in f16, every
// product of two such values is exact in the f32 accumulator, and the per-tensor
// FP32 scales are applied once in the epilogue.  The products run on
// v_mfma_f32_32x32x16_f16.  FP4 stays FP4 in HBM and in LDS (a quarter of the
// bytes of an f16 GEMM); the conversion is v_cvt_scalef32_pk_f16_fp4 followed by
// a packed f16 multiply by the block scale (the converter's own f32 scale
// operand applies only its exponent, so it is left at 1).
//
// MFMA operand mapping (both kernels): a 32x32x16 MFMA takes 8 f16 per lane for A
// (row l%32) and 8 for B (column l%32), lane half g = l/32 supplying one group of
// 8 K values.  Any assignment of K values to (g, slot) is valid as long as A and
// B use the same one.  Here a lane reads one 16-byte chunk (32 codes, two scale
// blocks) per operand tile and feeds it to four consecutive MFMAs, 8 codes each,
// so the 8 values of one MFMA slot always share one block scale.
//
// Two kernels:
//   gemm_kernel       the main path (K a multiple of 256, aligned operands):
//                     256x256 output tile, four waves of 128x128, K stages of 256
//                     elements; global -> LDS by direct DMA loads
//                     (global_load_lds_dwordx4) into a double buffer, two barriers
//                     per stage.  Per wave and 16 K it dequantizes 8 operand tiles
//                     (64 VALU ops) for 16 MFMAs, so the conversions fit under the
//                     matrix-core time.
//                     A second instance with 128x128 tiles (four waves of 64x64)
//                     takes, as quarters, the few 256x256 tiles that would
//                     otherwise run as a mostly idle last round.  Other
//                     instances, each with its own registers: CLAMP (tiles that
//                     stick out of C), ACC (C = alpha v + beta S, an addend read in
//                     the epilogue), SK (stream-K runs) and MIRROR (a symmetric
//                     product's tiles above the diagonal also stored transposed).
//   gemm_edge_kernel  any K multiple of 16, any 8-byte-aligned operands: 128x128
//                     tile, register-staged loads with zero fill.
// Workgroup -> tile order (both): consecutive workgroup ids go to different XCDs,
// so ids are renumbered to give each XCD a contiguous range, then walked in
// groups of 8 tile-rows so that neighbouring tiles share A rows and B columns in
// that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <type_traits>
#include <utility>

#include "device.hpp"
#include "internal.hpp"

namespace nvfp4 {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGroupM = 8;

struct GemmParams {
  const uint8_t *a_codes, *a_scales, *b_codes, *b_scales;
  const float *a_amax, *b_amax;
  int64_t M, N, K;
  int a_shift, b_shift;  // log2 of rows per scale row: 0 (1D) or 4 (2D)
  void *c;
  int64_t ldc;
  int c_bf16;
  int tiles_main;  // gemm_kernel, 256x256: tiles [0, tiles_main) of the grouped order
  int tail_first;  // gemm_kernel, quarters: the quarters of 256x256 tiles tail_first .. last
  int ksplit;      // gemm_kernel, 256x256: K splits per tile (1: none)
  int split_first; // ksplit > 1: the first split tile (the tiles before it run unsplit)
  float *ws;       // ksplit > 1: raw partial tiles [tiles_main][256][256], item t * ksplit + s
  int acc_c;       // fp32 output only: 0 stores the product v; 1 stores
                   // C = fl(fl(alpha * v) + fl(beta * S)), S the addend (acc_src, or C itself)
  float alpha, beta;
  const float *acc_src;  // acc_c: the addend S, with C's row stride (null: C)
  unsigned *amax_bits;  // acc_c only, or null: atomic max of |C| over the stored elements, as the
                        // bits of a non-negative float (those order as unsigned integers)
  int64_t sk_total;     // stream-K: stages of the stream-K tiles (tiles split_first .. + sk_tiles)
  int sk_tiles;
  int sym;              // C = A B^T is symmetric (M = N, the same operand on both sides): only the
                        // tiles on and above the diagonal, in the triangle order of tri_at
  int mirror;           // sym, plain fp32 epilogue: each tile above the diagonal also stores its
                        // transpose below it
};

// Wave-wide maximum of a non-negative lane value, merged into *bits by an atomic
// integer max of its bit pattern.  Every lane of the wave calls it.
__device__ __forceinline__ void wave_amax(unsigned *bits, float m, int lane) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (lane == 0) atomicMax(bits, __float_as_uint(m));
}

// 8 E2M1 codes (one 32-bit word, element 2j in the low nibble of byte j) times the
// block scale, as 8 f16.  Exact: see the header comment.
__device__ __forceinline__ half8 dequant8(uint32_t w, _Float16 s) {
  const half2v h0 = dequant2(w, 0, s), h1 = dequant2(w, 1, s), h2 = dequant2(w, 2, s), h3 = dequant2(w, 3, s);
  return half8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

__device__ __forceinline__ half2v scales2(uint32_t w) { return e4m3x2_to_f16(w); }

__device__ __forceinline__ uint32_t word(const uint4 &v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

// Tile at position l of the grouped order: groups of kGroupM tile-rows, walked
// column by column, so that neighbouring positions share A rows and B columns.
__device__ __forceinline__ void tile_at(int l, int num_m, int num_n, int &tm, int &tn) {
  const int per_group = kGroupM * num_n;
  const int grp = l / per_group, first_m = grp * kGroupM;
  const int gsz = min(num_m - first_m, kGroupM);
  tm = first_m + (l % per_group) % gsz;
  tn = (l % per_group) / gsz;
}

// Position l of the triangle order: (r, c) with c <= r, row by row (r = 0: (0, 0);
// r = 1: (1, 0), (1, 1); ...).
__device__ __forceinline__ void tri_at(int64_t l, int &r, int &c) {
  int64_t i = int64_t((__builtin_sqrt(8.0 * double(l) + 1.0) - 1.0) * 0.5);
  while ((i + 1) * (i + 2) / 2 <= l) ++i;
  while (i * (i + 1) / 2 > l) --i;
  r = int(i);
  c = int(l - i * (i + 1) / 2);
}

// Tile (tm, tn) at position l of the launch's sequence: the grouped order, or for a
// symmetric C the upper triangle column by column (tn = r, tm = c of tri_at:
// neighbouring positions share B's tile).
__device__ __forceinline__ void seq_tile(const GemmParams &p, int l, int num_m, int num_n, int &tm, int &tn) {
  if (p.sym) {
    tri_at(l, tn, tm);
  } else {
    tile_at(l, num_m, num_n, tm, tn);
  }
}

// Tile coordinates of this workgroup (see the header comment).
__device__ __forceinline__ void tile_of(int num_m, int num_n, int &tm, int &tn) {
  int pid = blockIdx.x;
  const int total = gridDim.x;
  if ((total & 7) == 0) pid = (pid & 7) * (total >> 3) + (pid >> 3);
  const int per_group = kGroupM * num_n;
  const int grp = pid / per_group, first_m = grp * kGroupM;
  const int gsz = min(num_m - first_m, kGroupM);
  tm = first_m + (pid % per_group) % gsz;
  tn = (pid % per_group) / gsz;
}

// acc (one 32x32 MFMA tile per entry) times the product of the two tensor decode
// scales, stored at C[m0 + wm + 32 i + ...][n0 + wn + 32 j + lr].
template <int TM, int TN>
__device__ __forceinline__ void store_tiles(const GemmParams &p, const f32x16 (&acc)[TM][TN], int64_t m0, int64_t n0,
                                            int lr, int g) {
  const float gscale = decode_scale(*p.a_amax) * decode_scale(*p.b_amax);
  float mx = 0.0f;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t n = n0 + 32 * j + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + 32 * i + 8 * (r >> 2) + 4 * g + (r & 3);
        if (m < p.M && n < p.N) {
          const float v = acc[i][j][r] * gscale;
          if (p.c_bf16) {
            reinterpret_cast<uint16_t *>(p.c)[m * p.ldc + n] = f32_to_bf16(v);
          } else {
            float *dst = reinterpret_cast<float *>(p.c) + m * p.ldc + n;
            const float y = p.acc_c ? p.alpha * v + p.beta * (p.acc_src ? p.acc_src[m * p.ldc + n] : *dst) : v;
            *dst = y;
            mx = fmaxf(mx, __builtin_fabsf(y));
          }
        }
      }
    }
  if (p.amax_bits) wave_amax(p.amax_bits, mx, threadIdx.x & 63);
}

// Epilogue of the main kernel, whose MFMAs take the B tile as first operand so
// that acc[i][j] holds the 32x32 block C^T: lane l owns row m = 32 i + l % 32 of C
// and, in register group q, the 4 consecutive columns n = 32 j + 8 q + 4 (l / 32)
// .. +3.
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Cache-policy operand of the raw buffer builtins for a non-temporal store (the
// nt bit).
constexpr int kNontemporal = 2;

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0..N-1.
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Epilogue of the main kernel through LDS (C^T layout as above: a lane holds 4
// consecutive columns of a row per group of 4 accumulators).  A private 4 KB
// region per wave holds 32 rows of 128 bytes, the 16-byte chunks of a row
// XOR-swizzled by the row; each lane reads back whole chunks of rows and stores
// them, so every store writes whole 128-byte row runs of C.
//  * fp32 output: one 32x32 block at a time goes raw from the accumulator
//    registers into the region and is scaled after the read-back (gscale: the
//    product of the two tensor decode scales).
//  * bf16 output: two neighbouring blocks at a time, each scaled and rounded in
//    registers first: half the LDS traffic per block, and whole lines per store.
//    One block at a time wrote 64-byte half lines, which were not merged (fprop
//    wrote 860 MiB for 640 MiB of Y); pairing measured 0.4% faster per step.  The
//    next pair is converted while this pair's read-back is in flight (0.3% faster
//    GEMM).
// The region lies outside the two stage buffers, so the next tile's stages can
// land while this runs, and only one block's values pass through vector
// registers at a time.  The stores are non-temporal: the output is not read again
// by this kernel, and the quantizer that follows in a linear layer's step then
// reads its input from HBM without first evicting dirty output lines from the
// Infinity Cache (measured 5% faster quantization per step on the MI355X).
// CHECK: the tile may stick out of C (rows or columns past the edge are skipped;
// the launcher guarantees N % 4 == 0, a 16-byte aligned C and ldc % 4 == 0).
constexpr int kEpiBytes = 4096;

// fp32 accumulating epilogue, C = fl(fl(alpha * v) + fl(beta * S)) with S the addend
// (C itself, or another array of C's shape and stride), block by block as the plain
// fp32 path.  The addend of each block is loaded kAccAhead blocks ahead
// (kAccAheadCheck for partial tiles, whose bounds tests take registers) into
// a ring of registers: a load issued only when its block is stored waits a whole
// memory latency per block, with no other wave on the SIMD to cover it.  C is
// addressed as a raw buffer from the wave's corner: the lane's offset in one
// vector register, the block's row and column offsets in scalar ones (a wave's 128
// rows of C span less than 2^31 bytes, else the launcher takes the edge kernel).  mx takes the maximum of |C|
// over the lane's stored elements.
constexpr int kAccAhead = 8, kAccAheadCheck = 4;

template <int TM, int TN, bool CHECK>
__device__ __forceinline__ void store_tiles_lds_acc(const GemmParams &p, const f32x16 (&acc)[TM][TN], int64_t m0,
                                                    int64_t n0, int lane, uint8_t *region, float gscale, float &mx) {
  constexpr int NB = TM * TN, AH = CHECK ? kAccAheadCheck : kAccAhead, D = NB < AH ? NB : AH;
  const int lr = lane & 31, g = lane >> 5;
  const int wsw = (lr >> 1) & 7;  // swizzle of the row this lane writes
  const int rq = lane >> 3, ch = lane & 7;  // read-back: row 8k + rq of the block, columns 4 ch .. +3
  const uint32_t ldb = uint32_t(p.ldc) * 4u;
  const __amdgpu_buffer_rsrc_t rs = wave_rsrc(reinterpret_cast<float *>(p.c) + m0 * p.ldc + n0);
  const __amdgpu_buffer_rsrc_t rsrc =
      p.acc_src ? wave_rsrc(const_cast<float *>(p.acc_src) + m0 * p.ldc + n0) : rs;
  const uint32_t voff = uint32_t(rq) * ldb + 16u * uint32_t(ch);
  const int64_t mlim = p.M - m0, nlim = p.N - n0;
  // block b = (i, j): rows 32 i + 8 k + rq, columns 32 j + 4 ch
  auto inside = [&](int i, int j, int k) { return !CHECK || (32 * i + 8 * k + rq < mlim && 32 * j + 4 * ch < nlim); };
  auto soff = [&](int i, int j, int k) { return int(uint32_t(32 * i + 8 * k) * ldb + 128u * uint32_t(j)); };
  u32x4 old[D][4];
  auto fetch = [&](auto bc) {
    constexpr int b = decltype(bc)::value, i = b / TN, j = b % TN;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (inside(i, j, k)) old[b % D][k] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, int(voff), soff(i, j, k), 0);
  };
  static_for<D>(fetch);
  static_for<NB>([&](auto bc) {
    constexpr int b = decltype(bc)::value, i = b / TN, j = b % TN;
    // explicit moves out of the accumulator registers, one block at a time (else the
    // compiler may move them all at once, next to the ring of old values)
    float a[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) a[r] = acc[i][j][r];
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // columns 8q + 4g .. +3 of the block: chunk 2q + g
      const float4 v = make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
      *reinterpret_cast<float4 *>(region + lr * 128 + (((2 * q + g) ^ wsw) << 4)) = v;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 8 * k + rq;
      const float4 x = *reinterpret_cast<const float4 *>(region + r * 128 + ((ch ^ ((r >> 1) & 7)) << 4));
      if (inside(i, j, k)) {
        const u32x4 o = old[b % D][k];
        const float y0 = p.alpha * (x.x * gscale) + p.beta * __uint_as_float(o[0]);
        const float y1 = p.alpha * (x.y * gscale) + p.beta * __uint_as_float(o[1]);
        const float y2 = p.alpha * (x.z * gscale) + p.beta * __uint_as_float(o[2]);
        const float y3 = p.alpha * (x.w * gscale) + p.beta * __uint_as_float(o[3]);
        const u32x4 y = {__float_as_uint(y0), __float_as_uint(y1), __float_as_uint(y2), __float_as_uint(y3)};
        __builtin_amdgcn_raw_buffer_store_b128(y, rs, int(voff), soff(i, j, k), kNontemporal);
        mx = fmaxf(fmaxf(mx, fmaxf(__builtin_fabsf(y0), __builtin_fabsf(y1))),
                   fmaxf(__builtin_fabsf(y2), __builtin_fabsf(y3)));
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the region is rewritten by the next block
    if constexpr (b + D < NB) fetch(std::integral_constant<int, b + D>{});
    __builtin_amdgcn_sched_barrier(0);
  });
}

// ACC: the accumulating fp32 path (p.acc_c set), a kernel instantiation of its own
// so that the plain kernels keep their registers.
template <int TM, int TN, bool CHECK, bool ACC, bool MIRROR = false>
__device__ __forceinline__ void store_tiles_lds(const GemmParams &p, const f32x16 (&acc)[TM][TN], int64_t m0,
                                                int64_t n0, int lane, uint8_t *region, float gscale, float &mx) {
  static_assert(TN % 2 == 0, "bf16 blocks go in pairs");
  const int lr = lane & 31, g = lane >> 5;
  const int wsw = (lr >> 1) & 7;  // swizzle of the row this lane writes
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  if (p.c_bf16) {
    // Blocks (i, j) and (i, j + 1), j even, together: scaled and rounded in registers
    // first, so the pair passes through the region as 32 rows of 128 bytes: row lr,
    // 16-byte chunk 4 jj + q (columns 8q .. 8q+7 of block j + jj) at
    // chunk ^ ((lr / 2) % 8), lane half g writing its 8 bytes.  The next pair is
    // converted while this pair's read-back is in flight.  The explicit moves keep
    // the compiler from moving all the accumulators out of the accumulator
    // registers at once.
    constexpr int NP = TM * TN / 2;
    bf16x4 cur[2][4];
    auto convert = [&](auto pc) {
      constexpr int P = decltype(pc)::value, i = P / (TN / 2), j = 2 * (P % (TN / 2));
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        float a[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
          asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(a[r]) : "a"(acc[i][j + jj][r]));
#pragma unroll
        for (int q = 0; q < 4; ++q)
          cur[jj][q] = bf16x4{(__bf16)(a[4 * q] * gscale), (__bf16)(a[4 * q + 1] * gscale),
                              (__bf16)(a[4 * q + 2] * gscale), (__bf16)(a[4 * q + 3] * gscale)};
      }
    };
    convert(std::integral_constant<int, 0>{});
    static_for<NP>([&](auto pc) {
      constexpr int P = decltype(pc)::value, i = P / (TN / 2), j = 2 * (P % (TN / 2));
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<bf16x4 *>(region + lr * 128 + (((4 * jj + q) ^ wsw) << 4) + 8 * g) = cur[jj][q];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // lane: rows 8k + lane / 8 (k = 0..3), chunk lane % 8 (8 columns): whole lines
      bf16x8 h[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = 8 * k + (lane >> 3), c = lane & 7;
        h[k] = *reinterpret_cast<const bf16x8 *>(region + r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
      }
      if constexpr (P + 1 < NP) convert(std::integral_constant<int, P + 1>{});
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the region is rewritten by the next pair
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = 8 * k + (lane >> 3), c = lane & 7;
        const int64_t m = m0 + 32 * i + r, n = n0 + 32 * j + 8 * c;
        uint16_t *dst = reinterpret_cast<uint16_t *>(p.c) + m * p.ldc + n;
        if (!CHECK || (m < p.M && n + 8 <= p.N)) {
          __builtin_nontemporal_store(h[k], reinterpret_cast<bf16x8 *>(dst));
        } else if (m < p.M && n < p.N) {
          const bf16x4 lo = {h[k][0], h[k][1], h[k][2], h[k][3]};
          __builtin_nontemporal_store(lo, reinterpret_cast<bf16x4 *>(dst));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    return;
  }
  if constexpr (ACC) {
    store_tiles_lds_acc<TM, TN, CHECK>(p, acc, m0, n0, lane, region, gscale, mx);
    return;
  }
  // MIRROR (a symmetric C in whole tiles): a tile above the diagonal (m0 and n0 in
  // different 256-row tiles) also stores its transpose below the diagonal, straight
  // from the accumulators.  Lane (lr, g) holds row m0 + 32 i + lr, columns
  // 8q + 4g + t of block (i, j): column m0 + 32 i + lr of rows n0 + 32 j + 8q + 4g + t
  // of the lower tile, so for each (q, t) the 32 lanes of a half store 128
  // contiguous bytes of one row.  Addressed as a raw buffer from the wave's corner of
  // the lower tile (the launcher keeps 128 rows of C within 2^31 bytes).  Ordinary
  // stores: the amax pass that reads C next found them in the cache (84-93 us for
  // 5120^2 against 124 us when every line was written non-temporally).
  static_assert(!MIRROR || !CHECK, "the mirrored epilogue takes whole tiles");
  const bool mirror = MIRROR && p.mirror && (m0 >> 8) != (n0 >> 8);
  const uint32_t ldb = uint32_t(p.ldc) * 4u;
  const __amdgpu_buffer_rsrc_t rt = wave_rsrc(reinterpret_cast<float *>(p.c) + n0 * p.ldc + m0);  // MIRROR only
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      // fp32: one block, raw from the accumulator registers (explicit moves when the
      // block is also mirrored: else the compiler moves every accumulator out at once)
      float a[16];
      if constexpr (MIRROR) {
#pragma unroll
        for (int r = 0; r < 16; ++r) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(a[r]) : "a"(acc[i][j][r]));
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) a[r] = acc[i][j][r];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // columns 8q + 4g .. +3 of the block: chunk 2q + g
        const float4 v = make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
        *reinterpret_cast<float4 *>(region + lr * 128 + (((2 * q + g) ^ wsw) << 4)) = v;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // lane: rows 8k + lane / 8 (k = 0..3), chunk lane % 8 (4 columns)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = 8 * k + (lane >> 3), c = lane & 7;
        const float4 x = *reinterpret_cast<const float4 *>(region + r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
        const int64_t m = m0 + 32 * i + r, n = n0 + 32 * j + 4 * c;
        if (!CHECK || (m < p.M && n < p.N)) {
          const f32x4 y = {x.x * gscale, x.y * gscale, x.z * gscale, x.w * gscale};
          f32x4 *dst = reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(p.c) + m * p.ldc + n);
          __builtin_nontemporal_store(y, dst);
        }
      }
      if (mirror) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a[4 * q + t] * gscale), rt,
                                                  int(4u * uint32_t(32 * i + lr) + uint32_t(4 * g) * ldb),
                                                  int(uint32_t(32 * j + 8 * q + t) * ldb), 0);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the region is rewritten by the next block
      __builtin_amdgcn_sched_barrier(0);
    }
}

// ---------------------------------------------------------------------------
// Main kernel.
// LDS stage layout: A codes [BM][128 B], B codes [BN][128 B], then scales
// [BM + BN][16 B] (A rows first).  A row's eight 16-byte chunks are stored at
// chunk ^ swz(row): the 32 lanes that read one chunk index of 32 consecutive rows
// then touch every 16-byte bank group once per 8 (or 16) lanes.

__device__ __forceinline__ int swz8(int row) { return (row ^ (row >> 1)) & 7; }

typedef __attribute__((address_space(3))) void lds_void;


// Buffer resource for `bytes` bytes at p: raw and untyped (stride 0; dword 3 as
// for gfx9 raw buffers).  Loads whose per-lane offset is at or past `bytes`
// return zero.
__device__ __forceinline__ u32x4 make_rsrc(const void *p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return u32x4{uint32_t(a), uint32_t(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}

// 16-byte DMA from a buffer into LDS: lane l reads voffset + soffset and writes
// dst + 16 l (dst is wave-uniform; M0 carries it).  Issued as inline assembly on
// purpose: the compiler then keeps no count of these loads, so it does not stall
// later LDS reads of the other stage buffer on them (it cannot tell the two buffers
// apart).  The kernel orders them itself, with vmcnt(0) before every barrier that
// precedes a read of the buffer they fill and before it exits.
// M0 is a reserved register: the compiler allocates no value to it, and a clobber
// of it would not be honoured.  No compiler-generated instruction of this file's
// kernels reads or writes M0 (tests/test_lib_abi.py checks the assembly), so these
// statements are its only users.  A scalar write of M0 needs one wait state before
// an LDS DMA reads it (the compiler inserts one after its own M0 writes; inside one
// asm statement its hazard recognizer cannot), hence the s_nop between the two.
__device__ __forceinline__ void dma16(const u32x4 &rsrc, void *dst, uint32_t voffset, uint32_t soffset) {
  const uint32_t lds_addr = uint32_t(reinterpret_cast<uintptr_t>(dst));  // low half of a flat LDS address = offset
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voffset), "s"(rsrc), "s"(soffset));
}

// SK: stream-K.  Workgroup r (in the order that gives each XCD a contiguous share)
// takes stages [r T/G, (r+1) T/G) of the tile-by-stage sequence of the stream-K
// tiles (T = sk_total, G = grid), as segments of at most one tile each.  A segment
// that is a whole tile is stored as usual; any other is stored raw (no decode
// scales) into workspace slot r + t (t: the tile's position among the stream-K
// tiles), and streamk_reduce_kernel sums each split tile's segments in order.
template <int BM, int BN, int WAVES_M, int WAVES_N, bool CLAMP, bool QUARTERS, bool ACC, bool SK = false,
          bool MIRROR = false>
__global__ __launch_bounds__(64 * WAVES_M *WAVES_N) void gemm_kernel(GemmParams p) {
  static_assert(!SK || (!QUARTERS && !ACC), "stream-K runs 256x256 tiles without an accumulated C");
  static_assert(!QUARTERS || (BM == 128 && BN == 128), "quarters of 256x256 tiles");
  constexpr int NW = WAVES_M * WAVES_N, NT = 64 * NW;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 32, TN = WN / 32, T = TM + TN;
  constexpr int kRow = 128;  // code bytes per row per stage (256 K)
  constexpr int kSc = 16;    // scale bytes per row per stage (16 blocks)
  constexpr int B_OFF = BM * kRow, S_OFF = (BM + BN) * kRow;
  constexpr int STAGE = (BM + BN) * (kRow + kSc);
  static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "code DMA: whole instructions per wave");
  static_assert((BM + BN) % 64 == 0, "scale DMA: whole instructions");
  static_assert(STAGE % 1024 == 0, "stage alignment");
  static_assert(2 * STAGE + NW * kEpiBytes <= 160 * 1024, "stage buffers and epilogue regions fit in LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE + NW * kEpiBytes];

  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int64_t M = p.M, N = p.N;
  const uint32_t kbytes = uint32_t(p.K / 2), nkb = uint32_t(p.K / 16);
  const int zst = int(p.K / 256);                                 // K stages of a tile
  int nst_new = zst / (QUARTERS ? 1 : p.ksplit);  // K stages of the work item set_tile last set

  // Persistent tiles.  The grid has at most one workgroup per CU; with a grid that
  // is a multiple of 8 and smaller than the tile count, workgroup w runs on XCD
  // w % 8, which owns the contiguous eighth of the tile sequence; its j-th
  // workgroup takes tiles j, j + G/8, ... of that range, so the XCD's workgroups
  // always work on neighbouring tiles.  Otherwise workgroup w takes w, w + G, ...
  // 256x256 tiles: a prefix of the grouped order.  Quarters: the four 128x128
  // quarters of each later 256x256 tile, in that order.
  const int num_m = int((M + 255) / 256), num_n = int((N + 255) / 256);
  const int all_tiles = p.sym ? num_m * (num_m + 1) / 2 : num_m * num_n;
  const int ntiles = QUARTERS ? 4 * (all_tiles - p.tail_first) : p.tiles_main;
  int L, Lend, Lstride;
  int sk_r = 0;  // stream-K: this workgroup's range
  if constexpr (SK) {
    const int G = gridDim.x;
    sk_r = (G & 7) == 0 ? int(blockIdx.x & 7) * (G >> 3) + int(blockIdx.x >> 3) : int(blockIdx.x);
    L = int(p.sk_total * sk_r / G);
    Lend = int(p.sk_total * (sk_r + 1) / G);
    Lstride = 0;
  } else if ((gridDim.x & 7) == 0 && int(gridDim.x) < ntiles) {
    const int x = blockIdx.x & 7;
    L = int(int64_t(ntiles) * x / 8) + int(blockIdx.x >> 3);
    Lend = int(int64_t(ntiles) * (x + 1) / 8);
    Lstride = int(gridDim.x >> 3);
  } else {
    L = blockIdx.x;
    Lend = ntiles;
    Lstride = gridDim.x;
  }
  if (L >= Lend) return;
  const float gscale = decode_scale(*p.a_amax) * decode_scale(*p.b_amax);  // loaded before any DMA is in flight
  int64_t m0, n0;

  // DMA sources.  Unit u (16 bytes) of a wave's instruction j sits at row
  // (j*NW + wave)*8 + lane/8 of the tile, physical chunk lane%8, and holds that
  // row's logical chunk (lane%8) ^ swz8(row); swz8 depends only on the row's low
  // 4 bits, so it is the same for every j.  The loads are buffer loads whose
  // range check (on the per-lane offset) returns zeros for rows past the matrix
  // edge; those rows' outputs are not stored.  Offsets are 32-bit: the launcher
  // checks (rows + 256) * K/2 < 2^32.  Without CLAMP (M, N multiples of the
  // tile) the row step between instructions rides in the scalar offset.
  constexpr int JA = BM * 8 / NT, JB = BN * 8 / NT;
  constexpr int NSC = ((BM + BN) / 64 + NW - 1) / NW;
  static_assert(JA % 4 == 0 && JB % 4 == 0, "DMA split over four substeps");
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // scalar copy: LDS destinations stay scalar
  const int row0 = wave * 8 + (lane >> 3);
  const uint32_t lchunk = uint32_t(((lane & 7) ^ swz8(row0)) << 4);
  const uint32_t rstride = uint32_t(NW * 8) * kbytes;  // bytes between instruction j and j+1
  const u32x4 rsa = make_rsrc(p.a_codes, uint32_t(M) * kbytes);
  const u32x4 rsb = make_rsrc(p.b_codes, uint32_t(N) * kbytes);
  const u32x4 rssa = make_rsrc(p.a_scales, uint32_t((M + (1 << p.a_shift) - 1) >> p.a_shift) * nkb);
  const u32x4 rssb = make_rsrc(p.b_scales, uint32_t((N + (1 << p.b_shift) - 1) >> p.b_shift) * nkb);
  uint32_t va[CLAMP ? JA : 1], vb[CLAMP ? JB : 1], vs[NSC];
  int ks0 = 0;   // first K stage of the current item's split (0 without splits)
  int sk_t = 0;  // stream-K: the item's tile, as a position among the stream-K tiles
  // tile coordinates of sequence position l (groups of 8 tile-rows) and its DMA offsets
  auto set_tile = [&](int l) {
    int tm, tn;
    if constexpr (SK) {
      // stream-K: l is a stage of the sequence; the segment runs to its tile's end or
      // to the end of this workgroup's range
      sk_t = l / zst;
      ks0 = l - sk_t * zst;
      nst_new = min(zst - ks0, Lend - l);
      seq_tile(p, p.split_first + sk_t, num_m, num_n, tm, tn);
      m0 = int64_t(tm) * BM;
      n0 = int64_t(tn) * BN;
    } else if constexpr (QUARTERS) {
      seq_tile(p, p.tail_first + (l >> 2), num_m, num_n, tm, tn);
      m0 = int64_t(tm) * 256 + BM * ((l >> 1) & 1);
      n0 = int64_t(tn) * 256 + BN * (l & 1);
    } else {
      static_assert(QUARTERS || (BM == 256 && BN == 256), "tile grid of 256x256");
      // work item l: K split l % ksplit of tile l / ksplit, its first stage ks0
      const int t = l / p.ksplit;
      ks0 = (l - t * p.ksplit) * nst_new;
      seq_tile(p, p.split_first + t, num_m, num_n, tm, tn);
      m0 = int64_t(tm) * BM;
      n0 = int64_t(tn) * BN;
    }
    const uint32_t kc = uint32_t(ks0) * kRow, ksb = uint32_t(ks0) * kSc;  // the split's first K byte
#pragma unroll
    for (int j = 0; j < (CLAMP ? JA : 1); ++j) va[j] = uint32_t(m0 + row0 + NW * 8 * j) * kbytes + lchunk + kc;
#pragma unroll
    for (int j = 0; j < (CLAMP ? JB : 1); ++j) vb[j] = uint32_t(n0 + row0 + NW * 8 * j) * kbytes + lchunk + kc;
#pragma unroll
    for (int j = 0; j < NSC; ++j) {
      const int u = (j * NW + wave) * 64 + lane;
      vs[j] = (u < BM ? uint32_t((m0 + u) >> p.a_shift) * nkb : uint32_t((n0 + (u - BM)) >> p.b_shift) * nkb) + ksb;
    }
  };

  // global -> LDS: DMA instruction d (0 .. NDMA-1) of stage kt into buffer buf:
  // A code rows for d < JA, then B code rows, then the scale rows.  Asynchronous:
  // completion is awaited with vmcnt before the barrier that precedes the first
  // read.
  constexpr int NDMA = JA + JB + NSC;
  auto dma = [&](int kt, int buf, int d) {
    uint8_t *base = lds + buf * STAGE;
    const uint32_t kofs = uint32_t(kt) * kRow;
    if (d < JA) {
      dma16(rsa, base + (d * NW + wave_s) * 1024, CLAMP ? va[d] : va[0], CLAMP ? kofs : kofs + d * rstride);
    } else if (d < JA + JB) {
      const int j = d - JA;
      dma16(rsb, base + B_OFF + (j * NW + wave_s) * 1024, CLAMP ? vb[j] : vb[0], CLAMP ? kofs : kofs + j * rstride);
    } else {
      const int j = d - JA - JB;
      const int u0 = (j * NW + wave_s) * 64;  // scalar
      if ((BM + BN) % (64 * NW) == 0 || u0 < BM + BN)
        dma16(u0 < BM ? rssa : rssb, base + S_OFF + u0 * kSc, vs[j], uint32_t(kt) * kSc);
    }
  };
  auto issue = [&](int kt, int buf) {
#pragma unroll
    for (int d = 0; d < NDMA; ++d) dma(kt, buf, d);
  };

  const int wm = (wave / WAVES_N) * WM, wn = (wave % WAVES_N) * WN;
  const int lr = lane & 31, g = lane >> 5;
  const int sw = swz8(lr);  // = swz8(row) for every row this lane reads (rows differ by multiples of 32)
  // LDS byte offsets of this lane's first A and B rows; tile i adds 32*i rows
  const int rowa = (wm + lr) * kRow, rowb = B_OFF + (wn + lr) * kRow;
  const int sca = S_OFF + (wm + lr) * kSc + 2 * g, scb = S_OFF + (BM + wn + lr) * kSc + 2 * g;

  // A stage is 4 quarters of 64 K; in quarter q lane half g reads 32-element chunk
  // 2q+g of each of its rows (16 bytes) and that chunk's two block scales.
  // Registers hold two quarters (ring of 2) and the f16 operands of two 16-K
  // substeps: the substep after the current one is dequantized while the current
  // one's MFMAs run.  Tiles 0..TM-1 are A's, TM..T-1 are B's.
  uint4 ch[2][T];
  uint32_t scw[2][T];
  half2v scd[2][T];
  half8 op[2][T];
  // LDS read r (0 .. 2T-1) of quarter q into ring slot `slot`: the chunk of tile r
  // for r < T, else the two scale codes of tile r - T
  auto lds_read = [&](int buf, int q, int slot, int r) {
    const uint8_t *base = lds + buf * STAGE;
    if (r < T) {
      const int chunk = ((2 * q + g) ^ sw) << 4;
      const int row = r < TM ? rowa + 32 * kRow * r : rowb + 32 * kRow * (r - TM);
      ch[slot][r] = *reinterpret_cast<const uint4 *>(base + row + chunk);
    } else {
      const int i = r - T;
      const int sc = i < TM ? sca + 32 * kSc * i : scb + 32 * kSc * (i - TM);
      scw[slot][i] = *reinterpret_cast<const uint16_t *>(base + sc + 4 * q);
    }
  };
  // half h (codes 4h..4h+3) of tile i of substep s, from ring slot `slot` into
  // operand set dst: two conversions and two multiplies
  auto dequant_half = [&](int slot, int s, int dst, int i, int h) {
    const uint32_t w = word(ch[slot][i], s);
    const _Float16 sv = scd[slot][i][s >> 1];
    const half2v lo = dequant2(w, 2 * h, sv);
    const half2v hi = dequant2(w, 2 * h + 1, sv);
    op[dst][i][4 * h + 0] = lo[0];
    op[dst][i][4 * h + 1] = lo[1];
    op[dst][i][4 * h + 2] = hi[0];
    op[dst][i][4 * h + 3] = hi[1];
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Explicit issue order.  A substep is NMF slots; slot k issues MFMA k of the
  // current operand set, its share of the 2T half-tile conversions for the next
  // substep (4 VALU each: with 128x128 per wave, one per MFMA, whose 32 cycles
  // leave room for them), of the LDS reads and of the DMA loads; sched_barrier
  // keeps the compiler from regrouping slots.
  constexpr int NMF = TM * TN;
  // items [K * C, (K + 1) * C) of TOTAL, C = ceil(TOTAL / NMF), for slot K
  auto slot_items = [&](auto kc, auto total_c, auto &&f) {
    constexpr int K = decltype(kc)::value, TOTAL = decltype(total_c)::value;
    constexpr int C = (TOTAL + NMF - 1) / NMF;
    static_for<C>([&](auto ic) {
      constexpr int x = K * C + decltype(ic)::value;
      if constexpr (x < TOTAL) f(std::integral_constant<int, x>{});
    });
  };
  using HalfTiles = std::integral_constant<int, 2 * T>;
  using Tiles = std::integral_constant<int, T>;

  // after_epi: the previous tile's epilogue stores were issued after this tile's
  // second-stage DMA.  Vector memory operations retire in issue order on this
  // chip, so a wait that leaves that many stores (plus any newer DMA) outstanding
  // still waits for the second-stage DMA.  Without CLAMP every store is issued:
  // per 32x32 block, 2 (bf16) or 4 (fp32) per lane; with CLAMP some may be
  // skipped, so the stores are not counted.
  constexpr int kStoresBf16 = TM * TN * 2, kStoresF32 = TM * TN * 4;
  // One stage, in buffer (kt + par) & 1.  Quarters 0..2 read the next quarter of
  // this buffer during their first substep, so after quarter 2's first substep no
  // wave reads this buffer again.  A first barrier opens quarter 2's last substep
  // (by then a wave's reads have long landed, so its wait for them costs nothing;
  // at the second substep it waited for the read just issued: measured 1% slower
  // per GEMM), and the DMA of stage kt_dma (of the tile whose offsets va/vb/vs hold)
  // into this buffer is spread over that substep and quarter 3's first three.  At
  // quarter 3 every wave waits for stage kt+1's DMA (issued one stage earlier) and
  // passes a second barrier, then reads stage kt+1's first quarter from the other
  // buffer.  The last stage has none of that.  The wait at quarter 3 lets the newer
  // operations stay in flight: this stage's DMA issued so far and, after a tile
  // change, the epilogue stores.  (One barrier, at quarter 3 only, measured 0.8%
  // slower.)
  constexpr int kDmaPer = (NDMA + 3) / 4;
  static_assert(kDmaPer <= NMF, "DMA loads fit the slots");
  constexpr int kBarrierSub = 3;  // quarter 2's substep that opens with the first barrier
  // DMA loads of this stage issued before the second barrier
  constexpr int kDmaBeforeB = ((4 - kBarrierSub) * kDmaPer < NDMA) ? (4 - kBarrierSub) * kDmaPer : NDMA;
  auto stage = [&](int kt, auto last_tag, int par, int kt_dma, bool after_epi, auto zero_tag) {
    constexpr bool LAST = decltype(last_tag)::value;
    constexpr bool ZERO = decltype(zero_tag)::value;  // a tile's first stage: its first MFMAs start from C = 0
    const int buf = (kt + par) & 1;
    static_for<4>([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      constexpr int slot = q & 1;
      constexpr bool next_q = q < 3 || !LAST;  // is there a quarter after this one?
      static_for<4>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        constexpr int cur = s & 1;
        if constexpr (q == 2 && s == kBarrierSub && !LAST) {
          // every wave has read all of this buffer (quarter 3 was read at quarter 2, substep 0)
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          __syncthreads();
        }
        if constexpr (q == 3 && s == 0 && !LAST) {
          // stage kt+1's DMA has landed: the newer operations (this stage's DMA issued so
          // far, and the previous tile's epilogue stores) may stay in flight
          if (!CLAMP && after_epi && p.c_bf16 && p.ksplit == 1)  // split partials are stored as fp32
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(kStoresBf16 + kDmaBeforeB < 63 ? kStoresBf16 + kDmaBeforeB : 63) : "memory");
          else if (!CLAMP && after_epi)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(kStoresF32 + kDmaBeforeB < 63 ? kStoresF32 + kDmaBeforeB : 63) : "memory");
          else
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(kDmaBeforeB) : "memory");
          __syncthreads();
        }
        constexpr bool has_next = s < 3 || next_q;
        constexpr int nslot = s < 3 ? slot : slot ^ 1, ns = s < 3 ? s + 1 : 0;
        constexpr int dslot = (q == 2 && s >= kBarrierSub) ? s - kBarrierSub : (q == 3 && s < kBarrierSub) ? s + 4 - kBarrierSub : -1;
        static_for<NMF>([&](auto kc) {
          constexpr int k = decltype(kc)::value;
          constexpr int i = k / TN, j = k % TN;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(op[cur][TM + j], op[cur][i],
                                                              (ZERO && q == 0 && s == 0) ? f32x16{} : acc[i][j], 0,
                                                              0, 0);
          if constexpr (has_next)
            slot_items(kc, HalfTiles{}, [&](auto hc) {
              constexpr int h = decltype(hc)::value;
              dequant_half(nslot, ns, cur ^ 1, h / 2, h % 2);
            });
          if constexpr (s == 0 && next_q)
            slot_items(kc, HalfTiles{}, [&](auto rc) {
              lds_read(q < 3 ? buf : buf ^ 1, q < 3 ? q + 1 : 0, slot ^ 1, decltype(rc)::value);
            });
          if constexpr (s == 2 && next_q)
            slot_items(kc, Tiles{}, [&](auto tc) {
              constexpr int x = decltype(tc)::value;
              scd[slot ^ 1][x] = scales2(scw[slot ^ 1][x]);
            });
          if constexpr (!LAST && dslot >= 0 && k < kDmaPer && dslot * kDmaPer + k < NDMA)
            dma(kt_dma, buf, dslot * kDmaPer + k);
          __builtin_amdgcn_sched_barrier(0);
        });
      });
    });
  };

  // Tile loop.  A tile's first stage lands before its loop starts (its DMA runs
  // during the previous tile's stage before last, in place of a stage past the
  // end) and its second is issued as the previous tile's epilogue starts; the
  // epilogue stages through its own LDS regions, so it overlaps both.  Tile
  // buffers alternate with par, the buffer of the tile's stage 0, when the stage
  // count is odd.
  set_tile(L);
  int nst_cur = nst_new;  // K stages of the current item (the tile's, or the split's, or the segment's)
  int par = 0;
  bool first = true;  // no epilogue stores in flight yet
  float amx = 0.0f;   // with p.amax_bits: max |C| over this lane's stored elements
  issue(0, 0);
  issue(min(1, nst_cur - 1), 1);
  // the first stage's DMA has landed; the second stage's NDMA loads (issued last,
  // vector memory operations retire in order) stay in flight until quarter 3's wait
  if (nst_cur >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NDMA) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (;;) {
    // stage 0 of this tile is in buffer par and visible to every wave
    const int64_t mc = m0, nc = n0;
    const int Lcur = L, ks0c = ks0, tc = sk_t;
    const int nst = nst_cur;
    const int Lnext = SK ? L + nst : L + Lstride;
    const bool more = Lnext < Lend;
    // quarter 0 of stage 0 and the operands of its first substep
#pragma unroll
    for (int r = 0; r < 2 * T; ++r) lds_read(par, 0, 0, r);
#pragma unroll
    for (int i = 0; i < T; ++i) scd[0][i] = scales2(scw[0][i]);
#pragma unroll
    for (int i = 0; i < T; ++i) {
      dequant_half(0, 0, 0, i, 0);
      dequant_half(0, 0, 0, i, 1);
    }
    // the first stage starts the accumulators (C = 0) when it is a plain one; for
    // one- and two-stage tiles the accumulators were cleared after the last tile
    int kt0 = 0;
    if (nst >= 3) {
      stage(0, std::false_type{}, par, 2, !first, std::true_type{});
      kt0 = 1;
    }
    for (int kt = kt0; kt + 2 < nst; ++kt) stage(kt, std::false_type{}, par, kt + 2, false, std::false_type{});
    if (nst >= 2) {
      // the stage before last loads the next tile's first stage; without a next
      // tile it re-loads this tile's last stage into a buffer that is not read
      // again (drained below)
      if (more) set_tile(Lnext);
      stage(nst - 2, std::false_type{}, par, more ? 0 : nst - 1, nst == 2 && !first, std::false_type{});
    }
    stage(nst - 1, std::true_type{}, par, 0, false, std::false_type{});

    // every wave is done with this tile's stage buffers, and the DMA issued in the
    // stage before last has landed
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int par_next = (par + nst) & 1;
    if (more) {
      if (nst >= 2) {
        issue(1, par_next ^ 1);
      } else {
        // a one-stage item loaded nothing ahead: the next item's first stage, and its
        // second when it has one (a stream-K segment after a one-stage segment)
        set_tile(Lnext);
        issue(0, par_next);
        if (nst_new >= 2) issue(1, par_next ^ 1);
      }
    }
    const bool raw = SK ? !(ks0c == 0 && nst == zst) : (!QUARTERS && p.ksplit > 1);
    if (raw) {
      // raw partial tile (no decode scales) into the item's 256x256 slot of the workspace
      // (stream-K: slot r + t of this workgroup's range r and the segment's tile t)
      GemmParams pp = p;
      pp.c = p.ws + int64_t(SK ? sk_r + tc : Lcur) * (256 * 256);
      pp.ldc = 256;
      pp.c_bf16 = 0;
      pp.acc_c = 0;
      pp.amax_bits = nullptr;
      pp.mirror = 0;
      store_tiles_lds<TM, TN, false, false>(pp, acc, wm, wn, lane, lds + 2 * STAGE + wave * kEpiBytes, 1.0f, amx);
    } else {
      store_tiles_lds<TM, TN, CLAMP, ACC, MIRROR>(p, acc, mc + wm, nc + wn, lane, lds + 2 * STAGE + wave * kEpiBytes,
                                                  gscale, amx);
    }
    if (!more) break;
    if (nst == 1) {
      // a one-stage tile's first stage (and second) was only just issued
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    L = Lnext;
    par = par_next;
    first = false;
    nst_cur = nst_new;
    if (nst_cur < 3) {  // the next item's first stage does not start its accumulators
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};
    }
  }
  if (ACC && p.amax_bits) wave_amax(p.amax_bits, amx, lane);
}

// ---------------------------------------------------------------------------
// Edge kernel: any K (multiple of 16), operands only 8-byte aligned.
// K advances in stages of 128 elements = 64 code bytes + 8 scale bytes per row,
// register-staged (zero-filled past the edges), LDS double-buffered.  LDS rows are
// 64 bytes; the four 16-byte chunks of a row are XOR-swizzled by row bits 1..2.

constexpr int kEdgeBK = 128;
constexpr int kEdgeRow = 64;

__device__ __forceinline__ int swz4(int row, int chunk) { return row * kEdgeRow + ((chunk ^ ((row >> 1) & 3)) << 4); }

__device__ __forceinline__ uint4 load_chunk(const uint8_t *base, int64_t row, int64_t rows, int64_t kbytes,
                                            int64_t kbyte) {
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < rows) {
    const uint8_t *q = base + row * kbytes + kbyte;
    if (kbyte + 8 <= kbytes) {
      const uint2 lo = *reinterpret_cast<const uint2 *>(q);
      v.x = lo.x;
      v.y = lo.y;
    }
    if (kbyte + 16 <= kbytes) {
      const uint2 hi = *reinterpret_cast<const uint2 *>(q + 8);
      v.z = hi.x;
      v.w = hi.y;
    }
  }
  return v;
}

__device__ __forceinline__ uint2 load_scales8(const uint8_t *base, int64_t row, int64_t rows, int shift, int64_t nkb,
                                              int64_t kb0) {
  uint32_t w[2] = {0u, 0u};
  if (row < rows) {
    const uint8_t *q = base + (row >> shift) * nkb + kb0;
    for (int j = 0; j < 8; ++j)
      if (kb0 + j < nkb) w[j >> 2] |= uint32_t(q[j]) << (8 * (j & 3));
  }
  return make_uint2(w[0], w[1]);
}

__global__ __launch_bounds__(256) void gemm_edge_kernel(GemmParams p) {
  constexpr int BM = 128, BN = 128, WM = 64, WN = 64, WAVES_N = BN / WN;
  constexpr int TM = WM / 32, TN = WN / 32;

  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * kEdgeRow];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BN * kEdgeRow];
  __shared__ __attribute__((aligned(16))) uint8_t lds_s[2][(BM + BN) * 8];

  const int t = threadIdx.x;
  const int64_t M = p.M, N = p.N, K = p.K;
  int tm, tn;
  tile_of(int((M + BM - 1) / BM), int((N + BN - 1) / BN), tm, tn);
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;
  const int64_t kbytes = K / 2, nkb = K / 16;
  const int nstages = int((K + kEdgeBK - 1) / kEdgeBK);

  uint4 ra[BM / 64], rb[BN / 64];
  uint2 rs;
  auto gload = [&](int kt) {
    const int64_t kbyte = int64_t(kt) * kEdgeRow + 16 * (t & 3);
#pragma unroll
    for (int i = 0; i < BM / 64; ++i) ra[i] = load_chunk(p.a_codes, m0 + (t >> 2) + 64 * i, M, kbytes, kbyte);
#pragma unroll
    for (int i = 0; i < BN / 64; ++i) rb[i] = load_chunk(p.b_codes, n0 + (t >> 2) + 64 * i, N, kbytes, kbyte);
    const int64_t kb0 = int64_t(kt) * (kEdgeBK / 16);
    if (t < BM) rs = load_scales8(p.a_scales, m0 + t, M, p.a_shift, nkb, kb0);
    else rs = load_scales8(p.b_scales, n0 + (t - BM), N, p.b_shift, nkb, kb0);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < BM / 64; ++i) *reinterpret_cast<uint4 *>(&lds_a[buf][swz4((t >> 2) + 64 * i, t & 3)]) = ra[i];
#pragma unroll
    for (int i = 0; i < BN / 64; ++i) *reinterpret_cast<uint4 *>(&lds_b[buf][swz4((t >> 2) + 64 * i, t & 3)]) = rb[i];
    *reinterpret_cast<uint2 *>(&lds_s[buf][t * 8]) = rs;
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
    for (int j = 0; j < TN; ++j) sb[j] = *reinterpret_cast<const uint2 *>(&lds_s[buf][(BM + wn + 32 * j + lr) * 8]);

#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int chunk = 2 * h + g;
      uint4 qa[TM], qb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) qa[i] = *reinterpret_cast<const uint4 *>(&lds_a[buf][swz4(wm + 32 * i + lr, chunk)]);
#pragma unroll
      for (int j = 0; j < TN; ++j) qb[j] = *reinterpret_cast<const uint4 *>(&lds_b[buf][swz4(wn + 32 * j + lr, chunk)]);
      // blocks 2*chunk and 2*chunk+1 of this stage: bytes 4h+2g, +1 of the 8 scale bytes
      half2v sca[TM], scb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) sca[i] = scales2((h == 0 ? sa[i].x : sa[i].y) >> (16 * g));
#pragma unroll
      for (int j = 0; j < TN; ++j) scb[j] = scales2((h == 0 ? sb[j].x : sb[j].y) >> (16 * g));
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        half8 fa[TM], fb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[i] = dequant8(word(qa[i], s), sca[i][s >> 1]);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[j] = dequant8(word(qb[j], s), scb[j][s >> 1]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
    }
    if (kt + 1 < nstages) lstore(buf ^ 1);
    __syncthreads();
  }

  store_tiles<TM, TN>(p, acc, m0 + wm, n0 + wn, lr, g);
}

// Compute units of the current device (queried once per device; concurrent first
// calls store the same value).
unsigned compute_units() {
  static std::atomic<unsigned> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  unsigned n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int q = 0;
    if (hipDeviceGetAttribute(&q, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || q <= 0) q = 256;
    n = unsigned(q);
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Stream-K reduction: the workgroups of the stream-K launch (G = tiles_main of them)
// own ranges [r T/G, (r+1) T/G) of the T = sk_total stages of the stream-K tiles;
// tile t (stages [t Z, (t+1) Z)) whose stages one range holds was stored by that
// workgroup, any other is the sum, in range order, of the raw segments in slots
// r + t of the ranges r that share it, times the two tensor decode scales.
// Workgroup b covers 16 rows of tile b / 16; each thread four groups of 4 columns.
__global__ __launch_bounds__(256) void streamk_reduce_kernel(GemmParams p) {
  const int t = blockIdx.x >> 4, r0 = (blockIdx.x & 15) * 16;
  const int64_t G = p.tiles_main, Z = p.K / 256, total = p.sk_total;
  auto start = [&](int64_t r) { return total * r / G; };
  auto find = [&](int64_t u) {  // the range holding stage u
    int64_t r = u * G / total;
    while (r + 1 < G && start(r + 1) <= u) ++r;
    while (start(r) > u) --r;
    return r;
  };
  const int64_t lo = find(int64_t(t) * Z), hi = find(int64_t(t + 1) * Z - 1);
  if (lo == hi) return;
  const int num_m = int((p.M + 255) / 256), num_n = int((p.N + 255) / 256);
  int tm, tn;
  seq_tile(p, p.split_first + t, num_m, num_n, tm, tn);
  const float gscale = decode_scale(*p.a_amax) * decode_scale(*p.b_amax);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = threadIdx.x + 256 * i;  // float4 index within the 16 x 256 block
    const int r = r0 + (f >> 6), c = (f & 63) * 4;
    const int64_t m = int64_t(tm) * 256 + r, n = int64_t(tn) * 256 + c;
    float4 v = *reinterpret_cast<const float4 *>(p.ws + (lo + t) * (256 * 256) + r * 256 + c);
    for (int64_t rr = lo + 1; rr <= hi; ++rr) {
      const float4 w = *reinterpret_cast<const float4 *>(p.ws + (rr + t) * (256 * 256) + r * 256 + c);
      v.x += w.x;
      v.y += w.y;
      v.z += w.z;
      v.w += w.w;
    }
    if (m >= p.M || n >= p.N) continue;  // N % 4 == 0: a group of 4 columns is inside or outside
    if (p.c_bf16) {
      const bf16x4 h = {(__bf16)(v.x * gscale), (__bf16)(v.y * gscale), (__bf16)(v.z * gscale),
                        (__bf16)(v.w * gscale)};
      *reinterpret_cast<bf16x4 *>(reinterpret_cast<uint16_t *>(p.c) + m * p.ldc + n) = h;
    } else {
      *reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.c) + m * p.ldc + n) =
          make_float4(v.x * gscale, v.y * gscale, v.z * gscale, v.w * gscale);
    }
  }
}

// The lower triangle of an n x n symmetric product, whose tiles on and above the
// diagonal hold C, copied from the upper one through LDS.  Workgroup b takes the
// 64x64 block (bi, bj) at position b of tri_at (bj <= bi): it reads the upper block
// (bj, bi) as rows of 16-byte vectors, and writes its transpose below the
// diagonal, whole vectors off the diagonal.  Needs n, ldc multiples of 4 and c
// 16-byte aligned (the launcher checks).
__global__ __launch_bounds__(256) void mirror_lower_kernel(float *c, int64_t n, int64_t ldc) {
  __shared__ float t[64][65];
  int bi, bj;
  tri_at(blockIdx.x, bi, bj);
  const int x = threadIdx.x & 15, y0 = threadIdx.x >> 4;  // 16 vectors per row, 16 rows per pass
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int y = y0 + 16 * k;
    const int64_t r = int64_t(bj) * 64 + y, col = int64_t(bi) * 64 + 4 * x;  // the upper block (bj, bi)
    if (r < n && col < n) {
      const float4 v = *reinterpret_cast<const float4 *>(c + r * ldc + col);
      t[y][4 * x] = v.x;
      t[y][4 * x + 1] = v.y;
      t[y][4 * x + 2] = v.z;
      t[y][4 * x + 3] = v.w;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int y = y0 + 16 * k;
    const int64_t r = int64_t(bi) * 64 + y, col = int64_t(bj) * 64 + 4 * x;  // the lower block (bi, bj)
    if (r >= n || col >= n) continue;
    const float4 v = {t[4 * x][y], t[4 * x + 1][y], t[4 * x + 2][y], t[4 * x + 3][y]};
    float *dst = c + r * ldc + col;
    if (col + 3 < r) {
      *reinterpret_cast<float4 *>(dst) = v;
    } else {  // on the diagonal block: only the elements below it
      if (col < r) dst[0] = v.x;
      if (col + 1 < r) dst[1] = v.y;
      if (col + 2 < r) dst[2] = v.z;
    }
  }
}

// Split-K reduction: C tile split_first + t = (sum over s of partial tile
// t * ksplit + s, in split order) times the two tensor decode scales, converted and
// stored.  Workgroup b
// covers 16 rows of tile b / 16; each thread four groups of 4 columns.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmParams p) {
  const int num_m = int((p.M + 255) / 256), num_n = int((p.N + 255) / 256);
  const int t = blockIdx.x >> 4, r0 = (blockIdx.x & 15) * 16;  // t: the t-th split tile
  int tm, tn;
  seq_tile(p, p.split_first + t, num_m, num_n, tm, tn);
  const float gscale = decode_scale(*p.a_amax) * decode_scale(*p.b_amax);
  const float *part = p.ws + int64_t(t) * p.ksplit * (256 * 256);
  float mx = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int f = threadIdx.x + 256 * i;  // float4 index within the 16 x 256 block
    const int r = r0 + (f >> 6), c = (f & 63) * 4;
    const int64_t m = int64_t(tm) * 256 + r, n = int64_t(tn) * 256 + c;
    float4 v = *reinterpret_cast<const float4 *>(part + r * 256 + c);
    for (int sp = 1; sp < p.ksplit; ++sp) {
      const float4 w = *reinterpret_cast<const float4 *>(part + int64_t(sp) * (256 * 256) + r * 256 + c);
      v.x += w.x;
      v.y += w.y;
      v.z += w.z;
      v.w += w.w;
    }
    if (m >= p.M || n >= p.N) continue;  // N % 4 == 0: a group of 4 columns is inside or outside
    if (p.c_bf16) {
      const bf16x4 h = {(__bf16)(v.x * gscale), (__bf16)(v.y * gscale), (__bf16)(v.z * gscale),
                        (__bf16)(v.w * gscale)};
      *reinterpret_cast<bf16x4 *>(reinterpret_cast<uint16_t *>(p.c) + m * p.ldc + n) = h;
    } else {
      float4 *dst = reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.c) + m * p.ldc + n);
      float4 y = make_float4(v.x * gscale, v.y * gscale, v.z * gscale, v.w * gscale);
      if (p.acc_c) {
        const float4 old = p.acc_src ? *reinterpret_cast<const float4 *>(p.acc_src + m * p.ldc + n) : *dst;
        const float4 q = make_float4(p.beta * old.x, p.beta * old.y, p.beta * old.z, p.beta * old.w);
        y = make_float4(p.alpha * y.x + q.x, p.alpha * y.y + q.y, p.alpha * y.z + q.z, p.alpha * y.w + q.w);
      }
      *dst = y;
      mx = fmaxf(fmaxf(mx, fmaxf(__builtin_fabsf(y.x), __builtin_fabsf(y.y))),
                 fmaxf(__builtin_fabsf(y.z), __builtin_fabsf(y.w)));
    }
  }
  if (p.amax_bits) wave_amax(p.amax_bits, mx, threadIdx.x & 63);
}

// *w = 0 ahead of a GEMM that merges its output's maximum into *w.
__global__ __launch_bounds__(64) void zero_word_kernel(unsigned *w) {
  if (threadIdx.x == 0) *w = 0u;
}

template <int BM, int BN>
unsigned tiles_for(const GemmParams &p) {
  return unsigned(((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN));
}


// Split-K plan of the main path for an M x N x K product on `cus` CUs, in units of
// one 256-K stage of one 256x256 tile on one CU (about 5.7 us on the MI355X).
// Without splits a tile takes Z = K/256 stages and the tiles run in rounds of
// `cus`; a last round at most half full runs as 128x128 quarters, at about 60% of
// the main kernel's rate.  A split runs a tile as S work items of Z/S stages (at
// least 4), plus the partial tiles' traffic (S written and read again, the output
// written, at about 4 TB/s).  Two splits are weighed: of every tile (few tiles, long
// K), or of the last round's tiles only, after the whole rounds (in place of the
// quarters).  A split is taken when it saves at least 5% of the time it replaces.
struct SplitPlan {
  int ksplit = 1;        // S (1: no split)
  int64_t first = 0;     // first split tile, in the grouped tile order
  int64_t tiles = 0;     // split tiles
  bool streamk = false;  // the split tiles run as stream-K instead (ksplit 1)
  int64_t sk_grid = 0;   // stream-K: workgroups (ranges)
};

SplitPlan splitk_plan(int64_t M, int64_t N, int64_t K, unsigned cus, bool allow_sk = true, bool sym = false) {
  SplitPlan none;
  if (K < 256 || K % 256 != 0 || M <= 0 || N <= 0) return none;
  const int64_t nm = (M + 255) / 256;
  const int64_t tiles = sym ? nm * (nm + 1) / 2 : nm * ((N + 255) / 256), z = K / 256;
  const int64_t full = tiles / cus, rest = tiles % cus;
  const bool quarters = full > 0 && rest > 0 && rest <= int64_t(cus) / 2;
  const double tail = rest == 0 ? 0.0 : quarters ? double((4 * rest + cus - 1) / cus) * (double(z) / 4.0) / 0.6
                                                 : double(z);
  const double base = double(full * z) + tail;
  const double stage_s = 5.7e-6, bw = 4.0e12, tile_bytes = 256.0 * 256.0 * 4.0;
  auto split_cost = [&](int64_t n, int sp) {
    return double((n * sp + cus - 1) / cus) * double(z / sp) + double(n) * tile_bytes * (2 * sp + 1) / bw / stage_s;
  };
  SplitPlan best;
  double best_cost = base;
  for (int sp = 2; sp <= 16; sp *= 2) {
    if (z % sp != 0 || z / sp < 4) continue;
    const double whole = split_cost(tiles, sp);
    if (whole < 0.95 * base && whole < best_cost) {
      best_cost = whole;
      best.ksplit = sp;
      best.first = 0;
      best.tiles = tiles;
    }
    if (full > 0 && rest > 0) {
      const double t = split_cost(rest, sp);
      if (t < 0.95 * tail && double(full * z) + t < best_cost) {
        best_cost = double(full * z) + t;
        best.ksplit = sp;
        best.first = full * cus;
        best.tiles = rest;
      }
    }
  }
  // Stream-K over the tiles after the whole rounds: every CU an equal run of their
  // stages (at least 8), about 2.5 stages of restarts per run, and the partial tiles
  // (at most one per run and tile boundary) written and read back.
  if (allow_sk && rest > 0 && z >= 8 && rest * z >= 8 * int64_t(cus)) {
    const int64_t total = rest * z, g = cus;
    const double c = double((total + g - 1) / g) + 2.5 + double(g + rest) * tile_bytes * 2.0 / bw / stage_s;
    if (double(full * z) + c < 0.95 * best_cost) {
      best = SplitPlan{};
      best.streamk = true;
      best.first = full * cus;
      best.tiles = rest;
      best.sk_grid = g;
    }
  }
  return best;
}

// The persistent kernel for p: CLAMP unless M and N are whole tiles (exact), the
// accumulating instantiation for an accumulated C stored by the kernel itself
// (split items store raw partial tiles; the reduction accumulates).
template <int BM, int BN, bool QUARTERS>
hipError_t launch_tiles(bool exact, const dim3 &grid, hipStream_t stream, const GemmParams &p) {
  if (p.mirror) return launch(gemm_kernel<BM, BN, 2, 2, false, QUARTERS, false, false, true>, grid, dim3(256), stream, p);
  if (p.acc_c && (QUARTERS || p.ksplit == 1))
    return exact ? launch(gemm_kernel<BM, BN, 2, 2, false, QUARTERS, true>, grid, dim3(256), stream, p)
                 : launch(gemm_kernel<BM, BN, 2, 2, true, QUARTERS, true>, grid, dim3(256), stream, p);
  return exact ? launch(gemm_kernel<BM, BN, 2, 2, false, QUARTERS, false>, grid, dim3(256), stream, p)
               : launch(gemm_kernel<BM, BN, 2, 2, true, QUARTERS, false>, grid, dim3(256), stream, p);
}

size_t splitk_ws_bytes(const SplitPlan &sp) {
  if (sp.streamk) return size_t(sp.sk_grid + sp.tiles) * 256 * 256 * sizeof(float);  // slots r + t
  return sp.ksplit <= 1 ? 0 : size_t(sp.tiles) * size_t(sp.ksplit) * 256 * 256 * sizeof(float);
}

hipError_t launch_gemm_impl(const fp4_tensor *a, const fp4_tensor *b, void *c, fp4_dtype c_dtype, int64_t ldc,
                            void *ws, size_t ws_bytes, hipStream_t stream, bool acc_c = false,
                            float beta = 0.0f, unsigned *amax_bits = nullptr, bool *sym = nullptr,
                            float alpha = 1.0f, const float *acc_src = nullptr, bool *mirrored = nullptr) {
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
  p.tiles_main = 0;
  p.tail_first = -1;
  p.ksplit = 1;
  p.split_first = 0;
  p.ws = nullptr;
  p.sk_total = 0;
  p.sk_tiles = 0;
  p.sym = 0;
  p.mirror = 0;
  if (mirrored) *mirrored = false;
  p.acc_c = acc_c && !p.c_bf16;
  p.alpha = alpha;
  p.beta = beta;
  p.acc_src = p.acc_c ? acc_src : nullptr;
  p.amax_bits = p.acc_c ? amax_bits : nullptr;
  if (p.M == 0 || p.N == 0) return hipSuccess;
  auto al = [](const void *q, uintptr_t n) { return reinterpret_cast<uintptr_t>(q) % n == 0; };
  // main path: whole 256-element K stages, 16-byte aligned codes and scale rows,
  // every DMA offset within 32 bits, and an output whose rows the 16-byte stores
  // can write (16-byte aligned C and rows; an accumulated C within the buffer
  // offsets of its epilogue)
  const bool main_path = p.K >= 256 && p.K % 256 == 0 && al(a->codes, 16) && al(b->codes, 16) &&
                         al(a->scales, 16) && al(b->scales, 16) && (p.M + 256) * (p.K / 2) < (int64_t(1) << 32) &&
                         (p.N + 256) * (p.K / 2) < (int64_t(1) << 32) &&
                         al(c, 16) && ldc % (p.c_bf16 ? 8 : 4) == 0 && p.N % 4 == 0 &&
                         (!p.acc_c || ldc * 4 * 128 < (int64_t(1) << 31)) && al(p.acc_src, 16);
  // a symmetric C: the main path computes the tiles on and above the diagonal (the
  // caller mirrors the rest); elsewhere the whole product
  p.sym = sym && *sym && main_path && p.M == p.N && !p.c_bf16;
  if (sym) *sym = p.sym;
  if (main_path && ws) {
    const unsigned cus = compute_units();
    // stream-K stores raw segments and sums them afterwards; an accumulated C takes
    // the split plan
    SplitPlan sp = splitk_plan(p.M, p.N, p.K, cus, !p.acc_c, p.sym);
    if (sp.streamk && ws_bytes < splitk_ws_bytes(sp)) sp = splitk_plan(p.M, p.N, p.K, cus, false, p.sym);  // too small
    if (sp.streamk && (reinterpret_cast<uintptr_t>(ws) & 15) == 0) {
      // whole rounds of tiles in the usual persistent launch, then the rest as
      // stream-K, and one reduction launch for the tiles that runs share
      const bool exact = p.M % 256 == 0 && p.N % 256 == 0;
      hipError_t e = hipSuccess;
      if (sp.first > 0) {
        p.tiles_main = int(sp.first);
        e = launch_tiles<256, 256, false>(exact, dim3(cus), stream, p);
      }
      p.split_first = int(sp.first);
      p.ws = static_cast<float *>(ws);
      p.sk_tiles = int(sp.tiles);
      p.sk_total = sp.tiles * (p.K / 256);
      p.tiles_main = int(sp.sk_grid);
      const dim3 grid(unsigned(sp.sk_grid));
      if (e == hipSuccess)
        e = exact ? launch(gemm_kernel<256, 256, 2, 2, false, false, false, true>, grid, dim3(256), stream, p)
                  : launch(gemm_kernel<256, 256, 2, 2, true, false, false, true>, grid, dim3(256), stream, p);
      if (e == hipSuccess) e = launch(streamk_reduce_kernel, dim3(unsigned(sp.tiles) * 16), dim3(256), stream, p);
      return e;
    }
    if (sp.ksplit > 1 && ws_bytes >= splitk_ws_bytes(sp) && (reinterpret_cast<uintptr_t>(ws) & 15) == 0) {
      // whole tiles before the split ones (if any) in the usual persistent launch; then
      // every split tile as ksplit work items of K / ksplit writing partial tiles into
      // ws, and one reduction launch writing their part of C
      const bool exact = p.M % 256 == 0 && p.N % 256 == 0;
      auto main = [&](const GemmParams &q, unsigned items) {
        const dim3 grid(items < cus ? items : cus);
        return launch_tiles<256, 256, false>(exact, grid, stream, q);
      };
      hipError_t e = hipSuccess;
      if (sp.first > 0) {
        p.tiles_main = int(sp.first);
        e = main(p, unsigned(sp.first));
      }
      p.ksplit = sp.ksplit;
      p.split_first = int(sp.first);
      p.ws = static_cast<float *>(ws);
      p.tiles_main = int(sp.tiles) * sp.ksplit;
      if (e == hipSuccess) e = main(p, unsigned(p.tiles_main));
      if (e == hipSuccess) e = launch(splitk_reduce_kernel, dim3(unsigned(sp.tiles) * 16), dim3(256), stream, p);
      return e;
    }
  }
  if (main_path) {
    // persistent: one workgroup per CU (its 160 KB of LDS admit no second one).
    // When the tiles overrun whole rounds of the CUs by at most half a round,
    // those last tiles would keep some CUs busy for a full tile time while the
    // rest idle; they go instead, as four 128x128 quarters each (one or two per
    // CU, a quarter of the time each), to a second persistent launch.
    const int64_t nm = (p.M + 255) / 256;
    const unsigned tiles = p.sym ? unsigned(nm * (nm + 1) / 2) : tiles_for<256, 256>(p), cus = compute_units();
    const unsigned rest = tiles % cus;
    const bool split = tiles > cus && rest > 0 && rest <= cus / 2;
    p.tiles_main = int(split ? tiles - rest : tiles);
    const dim3 grid(tiles < cus ? tiles : cus);
    const bool exact = p.M % 256 == 0 && p.N % 256 == 0;
    // a symmetric plain fp32 C: every tile reaches its final store here, so the
    // epilogue writes the lower triangle too
    p.mirror = p.sym && !p.acc_c && exact && p.ldc * 4 * 128 < (int64_t(1) << 31);
    if (mirrored) *mirrored = p.mirror != 0;
    hipError_t e = launch_tiles<256, 256, false>(exact, grid, stream, p);
    if (e == hipSuccess && split) {
      p.tail_first = p.tiles_main;
      const dim3 qgrid(4 * rest < cus ? 4 * rest : cus);
      e = launch_tiles<128, 128, true>(exact, qgrid, stream, p);
    }
    return e;
  }
  return launch(gemm_edge_kernel, dim3(tiles_for<128, 128>(p)), dim3(256), stream, p);
}

}  // namespace

// The library's own split-K scratch, for callers that cannot allocate: a
// file-scope device array (one copy per GPU, at that GPU's own address, held from
// module load until the process ends).  Host code never passes the array's name to
// a kernel -- on the host it is only a stand-in for the symbol -- but the device
// address hipGetSymbolAddress returns, looked up once per device with that device
// current.  Every work item writes its whole partial tile before the reduction
// reads it, so nothing in it needs clearing between calls.
__device__ __attribute__((aligned(256))) uint8_t scratch[kStaticScratchBytes];

hipError_t static_scratch(void **ptr) {
  static std::mutex mu;
  static void *addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_gemm(const fp4_tensor *a, const fp4_tensor *b, void *c, fp4_dtype c_dtype, int64_t ldc,
                       hipStream_t stream) {
  return launch_gemm_impl(a, b, c, c_dtype, ldc, nullptr, 0, stream);
}

hipError_t launch_gemm_ws(const fp4_tensor *a, const fp4_tensor *b, void *c, fp4_dtype c_dtype, int64_t ldc, void *ws,
                          size_t ws_bytes, hipStream_t stream) {
  return launch_gemm_impl(a, b, c, c_dtype, ldc, ws, ws_bytes, stream);
}

hipError_t launch_gemm_ws_acc(const fp4_tensor *a, const fp4_tensor *b, float *c, int64_t ldc, float beta,
                              float *amax, void *ws, size_t ws_bytes, hipStream_t stream, float alpha,
                              const float *src) {
  unsigned *bits = reinterpret_cast<unsigned *>(amax);
  if (bits && a->rows > 0 && b->rows > 0) {
    const hipError_t e = launch(zero_word_kernel, dim3(1), dim3(64), stream, bits);
    if (e != hipSuccess) return e;
  }
  return launch_gemm_impl(a, b, c, FP4_FP32, ldc, ws, ws_bytes, stream, true, beta, bits, nullptr, alpha, src);
}

size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K) {
  return splitk_ws_bytes(splitk_plan(M, N, K, compute_units()));
}

size_t gemm_ws_bytes_sym(int64_t M, int64_t K) {
  return splitk_ws_bytes(splitk_plan(M, M, K, compute_units(), true, true));
}

hipError_t launch_gemm_sym_ws(const fp4_tensor *a, const fp4_tensor *b, float *c, int64_t ldc, void *ws,
                              size_t ws_bytes, hipStream_t stream) {
  // the mirror moves 16-byte vectors: a symmetric product only where they line up.
  // The persistent launch stores the lower triangle itself; after split or stream-K
  // plans a mirror kernel copies it.
  bool sym = a->rows % 4 == 0 && ldc % 4 == 0 && (reinterpret_cast<uintptr_t>(c) & 15) == 0, mirrored = false;
  hipError_t e = launch_gemm_impl(a, b, c, FP4_FP32, ldc, ws, ws_bytes, stream, false, 0.0f, nullptr, &sym, 1.0f,
                                  nullptr, &mirrored);
  if (e != hipSuccess || !sym || mirrored) return e;
  const int64_t nb = (a->rows + 63) / 64;
  return launch(mirror_lower_kernel, dim3(unsigned(nb * (nb + 1) / 2)), dim3(256), stream, c, a->rows, ldc);
}

hipError_t launch_gemm_sym_ws_acc(const fp4_tensor *a, const fp4_tensor *b, float *c, int64_t ldc, float alpha,
                                  float beta, const float *src, float *amax, void *ws, size_t ws_bytes,
                                  hipStream_t stream) {
  unsigned *bits = reinterpret_cast<unsigned *>(amax);
  if (bits && a->rows > 0 && b->rows > 0) {
    const hipError_t e = launch(zero_word_kernel, dim3(1), dim3(64), stream, bits);
    if (e != hipSuccess) return e;
  }
  bool sym = a->rows % 4 == 0 && ldc % 4 == 0 && (reinterpret_cast<uintptr_t>(c) & 15) == 0;
  hipError_t e = launch_gemm_impl(a, b, c, FP4_FP32, ldc, ws, ws_bytes, stream, true, beta, bits, &sym, alpha, src);
  if (e != hipSuccess || !sym) return e;
  const int64_t nb = (a->rows + 63) / 64;
  return launch(mirror_lower_kernel, dim3(unsigned(nb * (nb + 1) / 2)), dim3(256), stream, c, a->rows, ldc);
}

size_t gemm_ws_bytes_plan(int64_t M, int64_t N, int64_t K, bool allow_sk, bool sym) {
  return splitk_ws_bytes(splitk_plan(M, N, K, compute_units(), allow_sk, sym));
}

size_t gemm_ws_bytes_within(int64_t M, int64_t N, int64_t K, size_t limit) {
  const unsigned cus = compute_units();
  const size_t b = splitk_ws_bytes(splitk_plan(M, N, K, cus));
  return b <= limit ? b : splitk_ws_bytes(splitk_plan(M, N, K, cus, false));
}

}  // namespace nvfp4
