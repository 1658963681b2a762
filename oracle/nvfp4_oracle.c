/*
 * nvfp4_oracle.c -- plain CPU oracle for the NVFP4 quantize + block-scaled GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The product path (the
 * HIP library under nvfp4_bit_microscaled_amd/) never links, imports or calls
 * it, and shares no source with it.
 *
 * What is computed, and where the pages fix it (page names are the q2bstudio
 * blog titles; "NVFP4-12B page" is the one on NVIDIA's 4-bit pretraining of a
 * 12B Mamba-Transformer, "Quartet II page" the one on Quartet II / MS-EDEN):
 *   - the element format is a 4-bit microscaling format (NVFP4-12B page,
 *     paragraph 2, the sentence introducing NVFP4 on Blackwell Tensor Cores);
 *   - blocks of 16 elements, one E4M3 scale per block, one FP32 scale per
 *     tensor (NVFP4-12B page, paragraph 2, the sentence on the design of NVFP4);
 *   - 2D block scaling for weights, 16x16 random Hadamard transforms on the
 *     weight-gradient operands, stochastic rounding on gradients only
 *     (NVFP4-12B page, paragraph 2, the four-part recipe sentence);
 *   - stochastic rounding is used because it is unbiased (Quartet II page,
 *     paragraph 1, the sentence on earlier quantized training);
 *   - MS-EDEN, an unbiased quantization routine for microscale formats with
 *     more than 2x lower error than stochastic rounding (Quartet II page,
 *     paragraph 1, the MS-EDEN sentence).  The page names the method only; the
 *     reading here follows EDEN (Vargaftik et al., ICML 2022): a random rotation,
 *     deterministic rounding, then a scale correction that makes the estimate
 *     unbiased over the rotation.  The rotation is a random-sign Hadamard over
 *     64-element groups (orthonormal with the exact factor 1/8), the rounding is
 *     nearest-even, and each 16-block's correction factor is folded into its
 *     E4M3 scale by stochastic rounding.
 * The pages print no formula for any step.  Every step below follows one plain
 * reading (the E2M1 grid {0,0.5,1,1.5,2,3,4,6}, OCP E4M3, s_enc = 2688/amax,
 * Philox4x32-10 counters, Sylvester H16 scaled by 1/4); each reading is listed
 * in the design notes together with the pins that check it.
 *
 * Arithmetic: every float operation below is one IEEE binary32 operation with
 * round-to-nearest-even (built with -ffp-contract=off, no fast-math); the
 * dequantized values and the GEMM reference are binary64.
 *
 * Pins (tests/test_oracle_*.py): E2M1 and E4M3 codecs against brute-force
 * nearest-value search over the enumerated grids; the Hadamard against
 * H*H^T = 16 I and the Kronecker construction of H16; Philox against the
 * published known-answer vectors; stochastic rounding against its expectation;
 * the scale recipe against the "one value per block at near-FP8 precision"
 * property; dequantization against exact small cases; the 64-point transform
 * against the Kronecker H64 on integers; MS-EDEN's scale rounding against its
 * exact expectation, its correction against EDEN's projection identity, and its
 * unbiasedness and its error against stochastic rounding statistically.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define NVO_EXPORT __attribute__((visibility("default")))

/* flag bits, the same meaning as the product library's (restated here on purpose:
 * the oracle includes no header of the product). */
#define NVO_2D (1u << 0)      /* one scale per 16x16 tile of the logical tensor */
#define NVO_COLWISE (1u << 1) /* logical tensor is x^T: blocks run down the columns of x */
#define NVO_RHT (1u << 2)     /* random Hadamard transform of each 16-block before quantizing */
#define NVO_SR (1u << 3)      /* stochastic rounding of the elements (else nearest-even) */
#define NVO_RHT64 (1u << 5)   /* random Hadamard transform of each 64-group before quantizing */
#define NVO_EDEN (1u << 6)    /* MS-EDEN: EDEN scale correction, stochastically rounded block scales */

/* ------------------------------------------------------------------------- */
/* E2M1 element format.                                                        */
/* Magnitude code n (0..7) stands for the n-th point of the grid              */
/* {0, 0.5, 1, 1.5, 2, 3, 4, 6}; bit 3 is the sign.  Consecutive grid points   */
/* have consecutive codes, which is what "ties to even" refers to below.       */
/* ------------------------------------------------------------------------- */
static const float E2M1_GRID[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

NVO_EXPORT double nvo_e2m1_value(unsigned code) {
  double m = E2M1_GRID[code & 7u];
  return (code & 8u) ? -m : m;
}

/* Encode one scaled value s.  Nearest-even: nearest grid point, a tie going to the
 * even code.  Stochastic: between the two neighbouring grid points lo <= |s| < hi,
 * the position f = (|s| - lo) / (hi - lo) in [0, 1) is cut to 16 fraction bits,
 * F = floor(f * 2^16), and the 16 random bits u16 are added to it: the value goes
 * up when the sum carries out of 16 bits (u16 + F >= 2^16), i.e. with probability
 * F / 2^16 -- within 2^-16 of a grid step of unbiased.  |s| >= 6 saturates to 6 in
 * both modes.  Zero is always written as the +0 code. */
NVO_EXPORT unsigned nvo_e2m1_encode(float s, int stochastic, uint32_t u16) {
  float a = fabsf(s);
  unsigned mag;
  if (a >= 6.0f) {
    mag = 7;
  } else {
    unsigned lo = 0; /* walk up the grid to the largest point <= a */
    while (lo < 7 && E2M1_GRID[lo + 1] <= a) lo++;
    float step = E2M1_GRID[lo + 1] - E2M1_GRID[lo]; /* 0.5, 1 or 2 */
    float frac = (a - E2M1_GRID[lo]) / step;        /* exact: a power-of-two divide of an exact difference */
    int up;
    if (!stochastic)
      up = (frac > 0.5f) || (frac == 0.5f && (lo & 1u));
    else {
      uint32_t F = (uint32_t)floorf(frac * 65536.0f); /* exact: frac < 1 scaled by a power of two */
      up = (u16 & 0xFFFFu) + F >= 65536u;
    }
    mag = lo + (unsigned)up;
  }
  if (mag == 0) return 0;
  return (signbit(s) ? 8u : 0u) | mag;
}

/* ------------------------------------------------------------------------- */
/* E4M3 scale format (OCP FP8 E4M3, the "FN" variant: bias 7, no infinity,      */
/* 0x7F/0xFF are NaN, largest finite value 448).                               */
/* ------------------------------------------------------------------------- */
NVO_EXPORT double nvo_e4m3_value(unsigned code) {
  unsigned e = (code >> 3) & 15u, m = code & 7u;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9); /* subnormal: m/8 * 2^-6 */
  else
    v = ldexp(1.0 + m / 8.0, (int)e - 7);
  return (code & 0x80u) ? -v : v;
}

/* Round a non-negative binary32 value to E4M3, nearest-even, then clamp to the
 * largest finite value 448 ("satfinite").  Returns the 7-bit code. */
NVO_EXPORT unsigned nvo_e4m3_encode(float u) {
  if (!(u > 0.0f)) return 0; /* zero (and anything not positive) */
  if (isinf(u)) return 0x7E;
  double x = u;
  int e2;
  frexp(x, &e2);  /* x = f * 2^e2, f in [0.5, 1) */
  int E = e2 - 1; /* floor(log2 x) */
  if (E < -6) E = -6; /* below 2^-6 the spacing stays that of the subnormals, 2^-9 */
  double quantum = ldexp(1.0, E - 3); /* three fraction bits */
  double n = rint(x / quantum);       /* current rounding mode is nearest-even */
  double v = n * quantum;
  if (v > 448.0) v = 448.0;
  if (v == 0.0) return 0;
  if (v < ldexp(1.0, -6)) return (unsigned)(v / ldexp(1.0, -9)); /* subnormal code = m */
  frexp(v, &e2);
  E = e2 - 1;
  unsigned m = (unsigned)(v / ldexp(1.0, E - 3)) - 8u;
  return ((unsigned)(E + 7) << 3) | m;
}

/* Stochastic rounding of a non-negative binary32 y onto the E4M3 grid (MS-EDEN's
 * corrected block scales): between the neighbouring E4M3 values lo <= y < hi, the
 * position f = (y - lo) / (hi - lo) is cut to 16 fraction bits, F = floor(f 2^16),
 * and the value goes up when u16 + F >= 2^16 -- the same add-and-truncate rule as
 * the elements' stochastic rounding, unbiased to 2^-16 of a step.  y >= 448
 * saturates to 448 (code 0x7E); zero stays zero. */
NVO_EXPORT unsigned nvo_e4m3_sr(float y, uint32_t u16) {
  if (!(y > 0.0f)) return 0;
  if (y >= 448.0f) return 0x7E;
  unsigned lo = 0; /* walk up the grid to the largest value <= y */
  while (lo < 0x7E && nvo_e4m3_value(lo + 1) <= (double)y) lo++;
  double step = nvo_e4m3_value(lo + 1) - nvo_e4m3_value(lo); /* a power of two */
  double frac = ((double)y - nvo_e4m3_value(lo)) / step;      /* exact */
  uint32_t F = (uint32_t)floor(frac * 65536.0);
  return lo + (((u16 & 0xFFFFu) + F >= 65536u) ? 1u : 0u);
}

/* ------------------------------------------------------------------------- */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy  */
/* as 1, 2, 3", SC'11): ten rounds of two 32x32->64 multiplies, the key bumped  */
/* by the Weyl constants between rounds.                                        */
/* ------------------------------------------------------------------------- */
NVO_EXPORT void nvo_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    uint32_t n1 = (uint32_t)p1;
    uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    uint32_t n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The 16 random bits used by element i (its row-major index in the logical
 * output tensor): one Philox call serves 8 consecutive elements. */
static uint32_t sr_bits(uint64_t i, uint64_t seed, uint64_t offset) {
  uint64_t g = i >> 3;
  uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), (uint32_t)offset, (uint32_t)(offset >> 32)};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t w[4];
  nvo_philox4x32_10(ctr, key, w);
  unsigned j = (unsigned)(i & 7u);
  return (w[j >> 1] >> (16u * (j & 1u))) & 0xFFFFu;
}

/* ------------------------------------------------------------------------- */
/* Random Hadamard transform of one 16-element block: flip the signs picked by  */
/* the 16-bit mask, apply the Sylvester-ordered H16 by the fast Walsh-Hadamard  */
/* butterflies (pair distance 1, 2, 4, 8), multiply by 1/4 so that the         */
/* transform is orthonormal.                                                    */
/* ------------------------------------------------------------------------- */
NVO_EXPORT void nvo_rht16(float v[16], uint32_t signs) {
  for (int j = 0; j < 16; ++j)
    if ((signs >> j) & 1u) v[j] = -v[j];
  for (int h = 1; h < 16; h <<= 1)
    for (int i = 0; i < 16; ++i)
      if ((i & h) == 0) {
        float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
  for (int j = 0; j < 16; ++j) v[j] = v[j] * 0.25f;
}

/* ------------------------------------------------------------------------- */
/* Random Hadamard transform of one 64-element group (the rotation of MS-EDEN): */
/* the 64 random signs of group j are the first two words of Philox4x32-10 with */
/* counter (j as two words, 0, 0) and key (the caller's 32-bit key, 0), element */
/* t taking bit t % 32 of word t / 32; then the Sylvester-ordered H64 by the    */
/* butterflies at distance 1, 2, 4, 8, 16, 32, and the factor 1/8 that makes it */
/* orthonormal (exact: a power of two).                                          */
/* ------------------------------------------------------------------------- */
NVO_EXPORT void nvo_rht64_signs(uint64_t group, uint32_t key, uint32_t out[2]) {
  uint32_t ctr[4] = {(uint32_t)group, (uint32_t)(group >> 32), 0u, 0u};
  uint32_t k[2] = {key, 0u};
  uint32_t w[4];
  nvo_philox4x32_10(ctr, k, w);
  out[0] = w[0];
  out[1] = w[1];
}

NVO_EXPORT void nvo_rht64(float v[64], const uint32_t signs[2]) {
  for (int t = 0; t < 64; ++t)
    if ((signs[t >> 5] >> (t & 31)) & 1u) v[t] = -v[t];
  for (int h = 1; h < 64; h <<= 1)
    for (int i = 0; i < 64; ++i)
      if ((i & h) == 0) {
        float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
  for (int t = 0; t < 64; ++t) v[t] = v[t] * 0.125f;
}

/* ------------------------------------------------------------------------- */
/* The logical tensor.  Without COLWISE it is x itself ([R][C], row stride ld,  */
/* K = C); with COLWISE it is x^T ([C][R], K = R).  Blocks are 16 consecutive  */
/* elements along K; with RHT each block is transformed before anything else.  */
/* ------------------------------------------------------------------------- */
typedef struct {
  const float *x;
  int64_t R, C, ld;
  unsigned flags;
  uint32_t signs;
  int64_t rows, K;
} logical_t;

static logical_t make_logical(const float *x, int64_t R, int64_t C, int64_t ld, unsigned flags, uint32_t signs) {
  logical_t L = {x, R, C, ld, flags, signs, 0, 0};
  if (flags & NVO_COLWISE) { L.rows = C; L.K = R; }
  else { L.rows = R; L.K = C; }
  return L;
}

static float load_elem(const logical_t *L, int64_t r, int64_t k) {
  return (L->flags & NVO_COLWISE) ? L->x[k * L->ld + r] : L->x[r * L->ld + k];
}

/* Block kb of logical row r, transformed: with RHT its 16 elements, with RHT64 its
 * quarter of the transformed 64-group it belongs to (the group is transformed
 * whole for each of its blocks). */
static void load_block(const logical_t *L, int64_t r, int64_t kb, float v[16]) {
  if (L->flags & NVO_RHT64) {
    float g[64];
    uint32_t sg[2];
    int64_t j = kb / 4;
    for (int t = 0; t < 64; ++t) g[t] = load_elem(L, r, j * 64 + t);
    nvo_rht64_signs((uint64_t)j, L->signs, sg);
    nvo_rht64(g, sg);
    for (int t = 0; t < 16; ++t) v[t] = g[(kb % 4) * 16 + t];
    return;
  }
  for (int j = 0; j < 16; ++j) v[j] = load_elem(L, r, kb * 16 + j);
  if (L->flags & NVO_RHT) nvo_rht16(v, L->signs);
}

/* Tensor amax of the (transformed) logical tensor. */
NVO_EXPORT float nvo_amax(const float *x, int64_t R, int64_t C, int64_t ld, unsigned flags, uint32_t signs,
                          int nthreads) {
  logical_t L = make_logical(x, R, C, ld, flags, signs);
  float amax = 0.0f;
  int64_t nkb = L.K / 16;
  if (L.K % 16 != 0 || ((flags & NVO_RHT64) && L.K % 64 != 0)) return -1.0f; /* no such blocks */
  /* with RHT64 each transformed block is read once: block 4 j + q of a group is
   * quarter q of the group's transform, so taking whole groups covers every block */
  int64_t step = (flags & NVO_RHT64) ? 4 : 1, width = 16 * step;
#pragma omp parallel for schedule(static) reduction(max : amax) num_threads(nthreads)
  for (int64_t r = 0; r < L.rows; ++r)
    for (int64_t kb = 0; kb < nkb; kb += step) {
      float v[64];
      if (flags & NVO_RHT64) {
        uint32_t sg[2];
        for (int t = 0; t < 64; ++t) v[t] = load_elem(&L, r, kb * 16 + t);
        nvo_rht64_signs((uint64_t)(kb / 4), L.signs, sg);
        nvo_rht64(v, sg);
      } else {
        load_block(&L, r, kb, v);
      }
      for (int j = 0; j < width; ++j)
        if (fabsf(v[j]) > amax) amax = fabsf(v[j]);
    }
  return amax;
}

/* Per-tensor encode scale: the tensor amax is mapped onto 448 * 6 = 2688, the
 * largest value an E4M3 scale times an E2M1 element can hold. */
static float encode_scale(float amax) {
  float s = (amax > 0.0f) ? 2688.0f / amax : 1.0f;
  if (isinf(s)) s = FLT_MAX;
  return s;
}

NVO_EXPORT float nvo_decode_scale(float amax) { return amax / 2688.0f; }

/* Block scale: the block amax divided by 6 (the largest element), times the
 * tensor encode scale, rounded to E4M3; the per-block multiplier is the tensor
 * encode scale divided by the decoded block scale (0 when the scale is 0).
 * Like the encode scale, the multiplier saturates at the largest finite float:
 * for a tensor whose amax is below about 1e-35 the quotient can overflow while
 * the block's elements are tiny, and the scaled values must stay finite (an
 * infinite multiplier would turn a zero element into NaN). */
static void block_scale(float amax_b, float s_enc, unsigned *code, float *mult) {
  float t = amax_b / 6.0f;
  float u = t * s_enc;
  unsigned c = nvo_e4m3_encode(u);
  float sf = (float)nvo_e4m3_value(c);
  *code = c;
  float m = (sf > 0.0f) ? s_enc / sf : 0.0f;
  if (isinf(m)) m = FLT_MAX;
  *mult = m;
}

static void encode_block(const float v[16], float mult, int sr, int64_t i0, uint64_t seed, uint64_t offset,
                         uint8_t *codes_out /* 8 bytes */) {
  for (int j = 0; j < 16; j += 2) {
    float s0 = v[j] * mult, s1 = v[j + 1] * mult;
    uint32_t r0 = sr ? sr_bits((uint64_t)(i0 + j), seed, offset) : 0;
    uint32_t r1 = sr ? sr_bits((uint64_t)(i0 + j + 1), seed, offset) : 0;
    unsigned c0 = nvo_e2m1_encode(s0, sr, r0), c1 = nvo_e2m1_encode(s1, sr, r1);
    codes_out[j / 2] = (uint8_t)(c0 | (c1 << 4)); /* element 2j in the low nibble */
  }
}

/* MS-EDEN on one (transformed) block, after its scale code sc and multiplier are
 * set: the elements are encoded nearest-even; with s the scaled values and e the
 * grid values they round to, EDEN's correction factor is c = sum s^2 / sum s e (1
 * when the second sum is not positive), so that the corrected block c e has the
 * block's own projection onto s; c is folded into the block scale, whose decoded
 * value times c is rounded back to E4M3 stochastically with the block's 16 random
 * bits u16.  Sums run over the 16 elements in order, one binary32 operation per
 * step.  Writes the 8 code bytes and returns the new scale code. */
static unsigned eden_block(const float v[16], float mult, unsigned sc, uint32_t u16, uint8_t *codes_out) {
  float s[16], e[16];
  for (int j = 0; j < 16; ++j) {
    s[j] = v[j] * mult;
    unsigned c = nvo_e2m1_encode(s[j], 0, 0);
    e[j] = (float)nvo_e2m1_value(c);
    if (j & 1) codes_out[j / 2] |= (uint8_t)(c << 4);
    else codes_out[j / 2] = (uint8_t)c;
  }
  float n = 0.0f, d = 0.0f;
  for (int j = 0; j < 16; ++j) n = n + s[j] * s[j];
  for (int j = 0; j < 16; ++j) d = d + s[j] * e[j];
  float c = (d > 0.0f) ? n / d : 1.0f;
  float y = (float)nvo_e4m3_value(sc) * c;
  return nvo_e4m3_sr(y, u16);
}

/* Quantize logical rows [row0, row0 + nrows) of x.
 *   codes:  [nrows][K/2] bytes, two elements per byte, low nibble first
 *   scales: 1D [nrows][K/16]; 2D [nrows/16][K/16] (row0, nrows multiples of 16)
 * amax_in: the tensor amax to use (NULL: computed here over the whole tensor).
 * amax_out (nullable) receives the amax used.  Returns 0, or -1 on a bad shape. */
NVO_EXPORT int nvo_quantize(const float *x, int64_t R, int64_t C, int64_t ld, unsigned flags, uint32_t signs,
                            uint64_t seed, uint64_t offset, const float *amax_in, int64_t row0, int64_t nrows,
                            uint8_t *codes, uint8_t *scales, float *amax_out, int nthreads) {
  logical_t L = make_logical(x, R, C, ld, flags, signs);
  int two_d = (flags & NVO_2D) != 0, sr = (flags & NVO_SR) != 0, eden = (flags & NVO_EDEN) != 0;
  if (L.K % 16 != 0 || row0 < 0 || nrows < 0 || row0 + nrows > L.rows) return -1;
  if (two_d && (row0 % 16 != 0 || nrows % 16 != 0)) return -1;
  if ((flags & NVO_RHT64) && (L.K % 64 != 0 || (flags & NVO_RHT) || two_d)) return -1;
  if (eden && (!(flags & NVO_RHT64) || sr)) return -1;
  float amax = amax_in ? *amax_in : nvo_amax(x, R, C, ld, flags, signs, nthreads);
  /* MS-EDEN keeps 7/4 of headroom in the tensor scale: the stored amax is 7/4 of the
   * transformed tensor's, so that a block scale times its correction factor (about
   * 1 +- 0.3) stays below the largest E4M3 value */
  if (eden && !amax_in) amax = 1.75f * amax;
  if (amax_out) *amax_out = amax;
  float s_enc = encode_scale(amax);
  int64_t nkb = L.K / 16;

  if (!two_d) {
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t rr = 0; rr < nrows; ++rr) {
      int64_t r = row0 + rr;
      for (int64_t kb = 0; kb < nkb; ++kb) {
        float v[16], amax_b = 0.0f, mult;
        unsigned sc;
        load_block(&L, r, kb, v);
        for (int j = 0; j < 16; ++j)
          if (fabsf(v[j]) > amax_b) amax_b = fabsf(v[j]);
        block_scale(amax_b, s_enc, &sc, &mult);
        if (eden) {
          sc = eden_block(v, mult, sc, sr_bits((uint64_t)(r * nkb + kb), seed, offset),
                          codes + rr * (L.K / 2) + kb * 8);
        } else {
          encode_block(v, mult, sr, r * L.K + kb * 16, seed, offset, codes + rr * (L.K / 2) + kb * 8);
        }
        scales[rr * nkb + kb] = (uint8_t)sc;
      }
    }
  } else {
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t tr = 0; tr < nrows / 16; ++tr) {
      for (int64_t kb = 0; kb < nkb; ++kb) {
        float v[16][16], amax_b = 0.0f, mult;
        unsigned sc;
        for (int i = 0; i < 16; ++i) {
          load_block(&L, row0 + tr * 16 + i, kb, v[i]);
          for (int j = 0; j < 16; ++j)
            if (fabsf(v[i][j]) > amax_b) amax_b = fabsf(v[i][j]);
        }
        block_scale(amax_b, s_enc, &sc, &mult);
        scales[tr * nkb + kb] = (uint8_t)sc;
        for (int i = 0; i < 16; ++i) {
          int64_t r = row0 + tr * 16 + i;
          encode_block(v[i], mult, sr, r * L.K + kb * 16, seed, offset,
                       codes + (tr * 16 + i) * (L.K / 2) + kb * 8);
        }
      }
    }
  }
  return 0;
}

/* Dequantize a quantized tensor of `rows` rows and K columns (arrays laid out as
 * nvo_quantize writes them, starting at its first row):
 * value = E2M1(code) * E4M3(scale) * g, where g = amax / 2688 in binary32.
 * out: [rows][K] binary64 (every product is exact in binary64).  For 2D scales
 * the scale of row r is row r/16 of the scale array. */
NVO_EXPORT void nvo_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K, int two_d,
                               float amax, double *out, int nthreads) {
  double g = (double)nvo_decode_scale(amax);
  int64_t nkb = K / 16;
#pragma omp parallel for schedule(static) num_threads(nthreads)
  for (int64_t r = 0; r < rows; ++r) {
    int64_t srow = two_d ? r / 16 : r;
    for (int64_t k = 0; k < K; ++k) {
      uint8_t byte = codes[r * (K / 2) + k / 2];
      unsigned code = (k & 1) ? (byte >> 4) : (byte & 15u);
      double s = nvo_e4m3_value(scales[srow * nkb + k / 16]);
      out[r * K + k] = nvo_e2m1_value(code) * s * g;
    }
  }
}

/* Array forms of the two encoders, so that tests can sweep millions of inputs. */
NVO_EXPORT void nvo_e2m1_encode_n(const float *s, int64_t n, int stochastic, const uint32_t *u16, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)nvo_e2m1_encode(s[i], stochastic, u16 ? u16[i] : 0u);
}

NVO_EXPORT void nvo_e4m3_encode_n(const float *u, int64_t n, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)nvo_e4m3_encode(u[i]);
}

NVO_EXPORT void nvo_e4m3_sr_n(const float *y, int64_t n, const uint32_t *u16, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)nvo_e4m3_sr(y[i], u16[i]);
}
