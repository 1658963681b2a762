/*
 * nvfp4_amd.h -- C ABI of the MI355X (gfx950) NVFP4 linear-layer library.
 *
 * Sources, cited by page and paragraph throughout (q2bstudio blog pages):
 *   NVFP4-12B page   -- NVIDIA's 4-bit NVFP4 pretraining of a 12B hybrid
 *                       Mamba-Transformer; paragraph 2 holds the format
 *                       sentence (16-element blocks, one E4M3 scale per block,
 *                       one FP32 scale per tensor), the GEMM-only sentence
 *                       (NVFP4 is applied to the GEMMs of linear layers alone),
 *                       the four-part recipe sentence (about 16% of linears kept
 *                       in BF16, 16x16 random Hadamard transforms on the
 *                       weight-gradient operands, 2D block scaling for weights,
 *                       stochastic rounding on gradients only) and the
 *                       throughput sentence (FP4 GEMMs at 2x / 3x FP8 on
 *                       GB200 / GB300, half the operand bytes);
 *   Quartet II page  -- "Quartet II: Pre-entrenamiento de LLMs en NVFP4";
 *                       paragraph 1 holds the sentence on stochastic rounding
 *                       as the way to unbiased gradient estimates, the MS-EDEN
 *                       sentence (an unbiased routine for microscale formats
 *                       with more than 2x lower error than stochastic rounding)
 *                       and the sentence on linear layers quantized fully to
 *                       NVFP4, forward and backward.
 *
 * Numerical definition (the pages give no formulas; this is the reading the
 * library implements, bit for bit):
 *   amax     = max |v| over the tensor (v after the Hadamard transform if any)
 *   s_enc    = 2688 / amax (1 if amax == 0; FLT_MAX if the quotient overflows)
 *   per block: S = E4M3_rne_satfinite((amax_b / 6) * s_enc),
 *              m = s_enc / decode(S) (0 when S == 0; FLT_MAX if the quotient
 *              overflows, as only a tensor amax below about 1e-35 can make it)
 *   element  = E2M1(v * m), nearest-even or stochastic, saturating at 6;
 *              zero is always the +0 code; two codes per byte, low nibble first
 *   decode   = E2M1 * decode(S) * (amax / 2688)
 * All of it in binary32, one IEEE operation per step.
 * Stochastic rounding: element i (row-major index in the logical output) uses
 * the 16 bits (16*(i&1)) of word ((i&7)>>1) of Philox4x32-10 with counter
 * (i>>3 as two 32-bit words, offset as two words) and key (seed as two words);
 * with F = floor(2^16 * (distance to the lower grid point / grid step)) it rounds
 * up when that 16-bit value plus F reaches 2^16 (the random bits are added below
 * the kept precision and the sum is truncated).
 * Random Hadamard transform: in each 16-block, negate the elements whose bit is
 * set in the 16-bit sign mask, apply Sylvester's H16 (butterflies at distance
 * 1, 2, 4, 8), multiply by 1/4.
 *
 * Memory: every pointer argument of the compute calls is a device pointer the
 * caller owns (allocated on the current HIP device); the library allocates no
 * device memory and keeps no per-call state.  All work is enqueued on the given
 * stream in stream order; no call synchronizes with the host.  The tensor amax
 * stays on the device.
 *
 * Errors: arguments are checked before anything is enqueued; a failed check
 * returns a non-zero fp4_status and enqueues nothing.  A launch that fails
 * reports FP4_ERR_HIP (each launch's own status: an error left pending by the
 * caller's earlier HIP work is neither reported nor cleared); the launches
 * already enqueued by that call stay enqueued.  Faults that occur later on the
 * device surface at the caller's next synchronization.  Non-finite inputs are
 * outside the contract: their results are unspecified.
 */
#ifndef NVFP4_AMD_H
#define NVFP4_AMD_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Marks the library's exported entry points (everything else is hidden). */
#define FP4_API __attribute__((visibility("default")))

typedef enum fp4_status {
  FP4_OK = 0,
  FP4_ERR_NULL = 1,        /* a required pointer is NULL */
  FP4_ERR_SHAPE = 2,       /* a size is negative, or not a multiple of 16 where blocks need it */
  FP4_ERR_ALIGN = 3,       /* a pointer or leading dimension breaks the stated alignment */
  FP4_ERR_DTYPE = 4,       /* unknown input or output dtype */
  FP4_ERR_MODE = 5,        /* unsupported combination of quantization flags */
  FP4_ERR_MISMATCH = 6,    /* descriptor sizes do not agree with the call */
  FP4_ERR_HIP = 7,         /* a HIP launch or runtime call failed */
  FP4_ERR_WORKSPACE = 8    /* the shape's split-K plan needs more scratch than the static buffer holds */
} fp4_status;

typedef enum fp4_dtype {
  FP4_BF16 = 0,
  FP4_FP32 = 1
} fp4_dtype;

/* quantization flags (fp4_quantize, fp4_amax) */
#define FP4_Q_2D (1u << 0)         /* one scale per 16x16 tile (weights), else per 16 elements */
#define FP4_Q_COLWISE (1u << 1)    /* the logical tensor is x^T: blocks run down the columns of x */
#define FP4_Q_RHT (1u << 2)        /* random Hadamard transform of every 16-block first */
#define FP4_Q_SR (1u << 3)         /* stochastic rounding (Philox4x32-10), else nearest-even */
#define FP4_Q_AMAX_GIVEN (1u << 4) /* *out->amax already holds the tensor amax: skip its pass */
#define FP4_Q_RHT64 (1u << 5)      /* random Hadamard transform of every 64-group first (MS-EDEN's rotation) */
#define FP4_Q_EDEN (1u << 6)       /* MS-EDEN (with FP4_Q_RHT64): EDEN-corrected, stochastically rounded scales */

/* A quantized logical tensor of `rows` x `cols`; cols is the blocked (contraction) dimension.
 *   codes : [rows][cols/2] bytes, element 2j in the low nibble of byte j
 *   scales: E4M3 codes; 1D: [rows][cols/16]; 2D: [ceil(rows/16)][cols/16]
 *   amax  : one float, the tensor amax (decode scale = amax / 2688)
 * codes and scales may be NULL when rows or cols is 0; amax may not. */
typedef struct fp4_tensor {
  uint8_t *codes;
  uint8_t *scales;
  float *amax;
  int64_t rows;
  int64_t cols;
  int32_t two_d;
} fp4_tensor;

/* Bytes of the codes and scales of a rows x cols quantized tensor (the layout of
 * fp4_tensor above: 0.5 B per element plus one E4M3 byte per 16-block, or per 16x16
 * tile with two_d; NVFP4-12B page, paragraph 2, format and throughput sentences).
 * Pure host arithmetic.  FP4_ERR_NULL for a NULL output, FP4_ERR_SHAPE for a
 * negative size or cols not a multiple of 16. */
FP4_API fp4_status fp4_tensor_bytes(int64_t rows, int64_t cols, int32_t two_d, size_t *codes_bytes, size_t *scales_bytes);

/* Tensor amax -- the magnitude the per-tensor FP32 scale is taken from (NVFP4-12B
 * page, paragraph 2, format sentence) -- of the logical tensor of x ([rows][cols]
 * with row stride ld elements): x itself, or x^T with FP4_Q_COLWISE; with
 * FP4_Q_RHT the amax is taken after the 16-point transform of the recipe sentence
 * (blocks along the logical rows).  Writes one float at amax_out (device).
 * Needs: the blocked dimension (cols, or rows with COLWISE) a multiple of 16 when
 * FP4_Q_RHT is set (of 64 with FP4_Q_RHT64, the 64-point transform of fp4_quantize,
 * keyed by the 32-bit rht_signs); ld >= cols; x 16-byte aligned and ld a multiple of
 * 8 elements.  Errors: FP4_ERR_MODE (other flags, or RHT with RHT64), FP4_ERR_DTYPE, FP4_ERR_SHAPE, FP4_ERR_ALIGN,
 * FP4_ERR_NULL (x with elements, or amax_out). */
FP4_API fp4_status fp4_amax(const void *x, fp4_dtype dtype, int64_t rows, int64_t cols, int64_t ld, uint32_t flags,
                    uint32_t rht_signs, float *amax_out, hipStream_t stream);

/* NVFP4 quantization (NVFP4-12B page, paragraph 2: format sentence for the
 * blocks and scales; recipe sentence for 2D weight scaling, the 16x16 random
 * Hadamard transform of weight-gradient operands and stochastic rounding of
 * gradients; Quartet II page, paragraph 1, for the unbiasedness stochastic
 * rounding provides).  Quantizes the logical tensor L of x (L = x, or x^T with
 * FP4_Q_COLWISE) into *out (out->rows x out->cols must equal L's shape;
 * out->two_d must match FP4_Q_2D).
 * Without FP4_Q_AMAX_GIVEN the tensor amax is computed first into out->amax (the
 * amax pass keeps its per-workgroup maxima in out->codes, at most 8 KB, before the
 * codes are written; x must not overlap out->codes, as for any output).
 * out_t (FP4_Q_2D only, nullable) also receives L^T quantized with the same tile
 * scales: its codes and scales are the exact transposes of out's.
 * rht_signs: the transform's 16-bit sign mask (FP4_Q_RHT), or the 32-bit key of the
 * 64-point transform's signs (FP4_Q_RHT64); seed, offset: the Philox stream of
 * stochastic rounding (FP4_Q_SR) or of MS-EDEN's scale rounding (FP4_Q_EDEN).
 * MS-EDEN (Quartet II page, paragraph 1, MS-EDEN sentence: an unbiased routine for
 * microscale formats with more than 2x lower error than stochastic rounding),
 * read after EDEN's rotate - round - correct scheme:
 *   FP4_Q_RHT64: in each 64-group along the blocked dimension, negate the elements
 *     whose sign bit is set (group j's 64 bits: words 0 and 1 of Philox4x32-10 with
 *     counter (j as two words, 0, 0) and key (rht_signs, 0), element t at bit t % 32
 *     of word t / 32), apply Sylvester's H64 (butterflies at distance 1 .. 32) and
 *     multiply by 1/8;
 *   FP4_Q_EDEN (needs RHT64, excludes SR): elements nearest-even; per block, with
 *     s the scaled values and e their grid values, c = sum s^2 / sum s e (in element
 *     order; 1 if the second sum is not positive) and the scale code becomes
 *     decode(S) * c rounded stochastically onto E4M3 (block b of the logical tensor
 *     draws half-word b & 7 of Philox with counter (b >> 3, offset), key seed; it
 *     goes up when those 16 bits plus the first 16 bits of the position between the
 *     two E4M3 neighbours reach 2^16; 448 and above saturate); the stored tensor amax
 *     is RN(7/4 * max |v|) -- with FP4_Q_AMAX_GIVEN, *out->amax holds that value.
 * Modes: 1D with any of COLWISE, RHT, SR; 1D with RHT64 (and COLWISE, and SR or
 * EDEN); 2D with COLWISE only (no RHT, no SR).  RHT64 needs L's cols a multiple of
 * 64.
 * Needs: L's cols a multiple of 16 (and L's rows too for 2D); x 16-byte aligned,
 * ld a multiple of 8 elements; codes 16-byte and scales 8-byte aligned; with
 * COLWISE or 2D, x at most 16776960 rows (FP4_ERR_SHAPE otherwise).
 * Errors: FP4_ERR_MODE, FP4_ERR_DTYPE, FP4_ERR_SHAPE, FP4_ERR_ALIGN, FP4_ERR_NULL,
 * FP4_ERR_MISMATCH (descriptor shape or two_d), FP4_ERR_HIP. */
FP4_API fp4_status fp4_quantize(const void *x, fp4_dtype dtype, int64_t rows, int64_t cols, int64_t ld, uint32_t flags,
                        uint32_t rht_signs, uint64_t seed, uint64_t offset, const fp4_tensor *out,
                        const fp4_tensor *out_t, hipStream_t stream);

/* Both quantized layouts of one tensor x [rows][cols] in one call: the pair the
 * backward pass needs of dy (dgrad takes dy rowwise with stochastic rounding, wgrad
 * takes dy^T transformed with stochastic rounding) and the pair fprop and wgrad need
 * of x (rowwise nearest-even, and x^T transformed) -- NVFP4-12B page, paragraph 2,
 * recipe sentence, for which operand gets which treatment.  Both tensor amaxes are
 * taken in one read of x:
 *   out_rows: x quantized 1D along its rows ([rows][cols], as fp4_quantize with flags 0
 *             or FP4_Q_SR, Philox offset offset_rows);
 *   out_cols: x^T quantized 1D (blocks down the columns of x, [cols][rows]), after the
 *             16-point Hadamard transform if FP4_Q_RHT is set (as fp4_quantize with
 *             FP4_Q_COLWISE [| FP4_Q_RHT] [| FP4_Q_SR], Philox offset offset_cols).
 * Codes, scales and amaxes are bit-identical to those two fp4_quantize calls.
 * flags: FP4_Q_SR (both layouts stochastic), FP4_Q_RHT (columnwise layout
 * transformed), FP4_Q_AMAX_GIVEN (out_rows->amax and out_cols->amax already hold the
 * two tensor amaxes; otherwise both are computed first, in one read of x; the amax
 * pass keeps its per-workgroup maxima in out_rows->codes before the codes are
 * written).
 * Needs: rows and cols multiples of 16; x 16-byte aligned, ld a multiple of 8.
 * Errors: as fp4_quantize. */
FP4_API fp4_status fp4_quantize_dual(const void *x, fp4_dtype dtype, int64_t rows, int64_t cols, int64_t ld,
                                     uint32_t flags, uint32_t rht_signs, uint64_t seed, uint64_t offset_rows,
                                     uint64_t offset_cols, const fp4_tensor *out_rows, const fp4_tensor *out_cols,
                                     hipStream_t stream);

/* Block-scaled GEMM with FP32 accumulation -- the operation NVFP4 is applied to
 * (NVFP4-12B page, paragraph 2, GEMM-only sentence; the format sentence fixes the
 * per-block and per-tensor scales each operand carries):
 *   C[m][n] = sum_k deq(A)[m][k] * deq(B)[n][k]
 * for A [M][K] and B [N][K] (both K-major, M = a->rows, N = b->rows, K = a->cols =
 * b->cols, K a multiple of 16), written as fp32 or bf16 (nearest-even) with row
 * stride ldc elements into c (device, caller-owned).  The products of the
 * dequantized operands are exact; the accumulation is FP32.
 * Errors: FP4_ERR_NULL, FP4_ERR_MISMATCH (K differs), FP4_ERR_SHAPE (K % 16, ldc < N,
 * a 2D operand's rows not a multiple of 16), FP4_ERR_DTYPE, FP4_ERR_ALIGN (c not
 * aligned to its element), FP4_ERR_HIP. */
FP4_API fp4_status fp4_gemm(const fp4_tensor *a, const fp4_tensor *b, void *c, fp4_dtype c_dtype, int64_t ldc,
                    hipStream_t stream);

/* fp4_gemm (same definition; NVFP4-12B page, paragraph 2, GEMM-only sentence) with
 * a caller workspace for split-K.  When a product has few 256x256 output tiles for
 * the CUs and a long K (a weight-gradient GEMM over many tokens with a small
 * weight), each tile's K range is split into S parts that run as separate work
 * items writing raw fp32 partial tiles into ws, and a second kernel sums the S
 * partials of each tile in split order, applies the decode scales and writes C.
 * The split adds S-1 fp32 additions per output.  When under a round of tiles
 * remains, the plan may run them as stream-K instead: each CU an equal run of the
 * tiles' K stages, tiles held whole by one run stored directly, the others' raw
 * segments (one 256 KB slot per run and tile it touches) summed in run order by
 * the second kernel.  The plan is fixed for (M, N, K) on this GPU;
 * fp4_gemm_ws_bytes gives the workspace it needs (0 when it takes no split).  A
 * stream-K plan given less workspace than that runs the shape's fixed split when it
 * fits; with less than the plan needs, or a shape off the 256-K main path, this is
 * fp4_gemm.
 * ws: device memory, 16-byte aligned, owned by the caller, overwritten; calls that
 * share a workspace must be ordered on one stream.  Errors: as fp4_gemm, plus
 * FP4_ERR_NULL / FP4_ERR_ALIGN for a non-empty workspace that is NULL / misaligned. */
FP4_API fp4_status fp4_gemm_ws(const fp4_tensor *a, const fp4_tensor *b, void *c, fp4_dtype c_dtype, int64_t ldc,
                               void *ws, size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory -- code under HIP graph capture,
 * serving loops and harnesses that forbid hipMalloc: fp4_gemm_ws with the
 * library's own static scratch in place of a caller workspace.  The scratch is a
 * 64 MiB (FP4_STATIC_SCRATCH_BYTES) device array per GPU, held from the first call
 * on that GPU until the process ends; this call allocates nothing.  Every call on
 * one GPU shares that GPU's array, so calls that overlap on one GPU (different
 * streams, or different host threads without ordering) race; calls ordered on one
 * stream do not.  A stream-K plan whose slots exceed the maximum gives way to the
 * shape's fixed split; a shape whose plan still needs more than the maximum (see
 * fp4_gemm_ws_bytes) returns FP4_ERR_WORKSPACE and enqueues nothing (fp4_gemm runs
 * any shape without scratch).  Otherwise the result is that of fp4_gemm_ws with a
 * workspace of the maximum.  Errors: as fp4_gemm_ws, plus FP4_ERR_WORKSPACE. */
#define FP4_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
FP4_API fp4_status fp4_gemm_noalloc(const fp4_tensor *a, const fp4_tensor *b, void *c, fp4_dtype c_dtype, int64_t ldc,
                                    hipStream_t stream);

/* Workspace bytes fp4_gemm_ws uses for an M x N x K product (0: no split).  Pure
 * host arithmetic on the device's CU count.  FP4_ERR_NULL, FP4_ERR_SHAPE. */
FP4_API fp4_status fp4_gemm_ws_bytes(int64_t M, int64_t N, int64_t K, size_t *bytes);

/* Workspace bytes the linear-layer calls below need for a layer of M tokens, K
 * input and N output features: the largest split plan of its three GEMMs (fprop
 * M x N x K, dgrad M x K x N, wgrad N x K x M).  0 when none splits.  With less
 * workspace the linear calls still run, without the split.  FP4_ERR_NULL,
 * FP4_ERR_SHAPE. */
FP4_API fp4_status fp4_linear_ws_bytes(int64_t M, int64_t N, int64_t K, size_t *bytes);

/* The linear-layer calls: the recipe of the NVFP4-12B page, paragraph 2 (GEMM-only
 * sentence: NVFP4 is applied to the linear layers' GEMMs; recipe sentence: 2D block
 * scaling for weights, 16x16 random Hadamard transforms on the weight-gradient
 * operands, stochastic rounding on gradients only), with every operand of every
 * GEMM quantized to NVFP4, forward and backward (Quartet II page, paragraph 1, the
 * sentence on fully NVFP4 linear layers).  Common arguments:
 *   dtype        input element type (bf16 or fp32); all inputs contiguous row-major;
 *   ws, ws_bytes caller workspace for the GEMMs' split-K partial tiles
 *                (fp4_linear_ws_bytes; NULL / 0 runs without splits), overwritten;
 *   marks        nullable array of HIP events the call records on `stream` between
 *                its phases, for callers that time them (the count is given per
 *                call); the caller creates and owns them.
 * M, N, K must be multiples of 16.  Errors: as the quantize and GEMM calls they
 * compose; every check runs before the first launch. */

/* Forward: y = x . w^T with x [M][K], w [N][K], y [M][N] (y_dtype).
 *   x -> xq ([M][K]) 1D nearest-even; with xq_t (nullable, [K][M]) x^T is also
 *   quantized, after the 16-point transform with rht_signs, nearest-even -- the
 *   wgrad operand the backward pass then reads instead of x -- both layouts in one
 *   fp4_quantize_dual (one read of x);
 *   w -> wq ([N][K]) 2D (16x16) nearest-even, and wq_t (nullable, [K][N]) w^T with
 *   the same tile scales, for dgrad;
 *   y = gemm(xq, wq).
 * The amax passes of x (both of its amaxes with xq_t) and of w run as one launch,
 * in x's phase.
 * marks (2): after x's quantization, after w's (before the GEMM). */
FP4_API fp4_status fp4_linear_fprop(const void *x, const void *w, fp4_dtype dtype, void *y, fp4_dtype y_dtype, int64_t M,
                                    int64_t N, int64_t K, uint32_t rht_signs, const fp4_tensor *xq,
                                    const fp4_tensor *xq_t, const fp4_tensor *wq, const fp4_tensor *wq_t, void *ws,
                                    size_t ws_bytes, const hipEvent_t *marks, hipStream_t stream);

/* Input gradient dx = dy . w with dy [M][N], dx [M][K] (dx_dtype): dy is quantized
 * 1D with stochastic rounding (seed, offset) into dyq ([M][N]) and multiplied with
 * the forward pass's 2D-quantized w^T (wq_t, [K][N]).
 * marks (1): after dy's quantization (before the GEMM). */
FP4_API fp4_status fp4_linear_dgrad(const void *dy, fp4_dtype dtype, const fp4_tensor *wq_t, void *dx, fp4_dtype dx_dtype,
                                    int64_t M, int64_t N, int64_t K, uint64_t seed, uint64_t offset,
                                    const fp4_tensor *dyq, void *ws, size_t ws_bytes, const hipEvent_t *marks,
                                    hipStream_t stream);

/* Weight gradient dw = dy^T . x with dy [M][N], x [M][K], dw [N][K] (dw_dtype):
 * both operands are quantized transposed (blocks along the M tokens) after the
 * random Hadamard transform with the same signs; dy with stochastic rounding (seed,
 * offset) into dyq_t ([N][M]), x nearest-even into xq_t ([K][M]).
 * The amax passes of dy and x run as one launch, in dy's phase.
 * marks (2): after dy^T's quantization, after x^T's (before the GEMM). */
FP4_API fp4_status fp4_linear_wgrad(const void *dy, const void *x, fp4_dtype dtype, void *dw, fp4_dtype dw_dtype,
                                    int64_t M, int64_t N, int64_t K, uint32_t rht_signs, uint64_t seed,
                                    uint64_t offset, const fp4_tensor *dyq_t, const fp4_tensor *xq_t, void *ws,
                                    size_t ws_bytes, const hipEvent_t *marks, hipStream_t stream);

/* Backward pass of the linear layer y = x . w^T (x [M][K], w [N][K], dy [M][N]):
 *   dx = dy . w    (dx [M][K], dx_dtype)   and   dw = dy^T . x   (dw [N][K], dw_dtype).
 * dy is quantized once for both GEMMs (fp4_quantize_dual with FP4_Q_SR | FP4_Q_RHT):
 * rowwise with stochastic rounding at offset_dgrad into dyq ([M][N]), and transposed
 * with the 16-point transform (rht_signs) and stochastic rounding at offset_wgrad
 * into dyq_t ([N][M]).  wq_t ([K][N], 2D) is the forward pass's transposed weight.
 * x^T quantized with the same transform ([K][M], nearest-even) is read from xq_t;
 * if x is not NULL it is first quantized from x into xq_t, otherwise xq_t must
 * already hold it (fp4_linear_fprop with xq_t writes it).  The results equal
 * fp4_linear_dgrad and fp4_linear_wgrad with the same seeds, offsets and signs.
 * With x, the amax passes of dy and x run as one launch, in dy's phase.
 * marks (3): after dy's quantization, after x^T's (at the same point when x is
 * NULL), after the dgrad GEMM (before the wgrad GEMM). */
FP4_API fp4_status fp4_linear_backward(const void *dy, const void *x, fp4_dtype dtype, const fp4_tensor *wq_t,
                                       void *dx, fp4_dtype dx_dtype, void *dw, fp4_dtype dw_dtype, int64_t M, int64_t N,
                                       int64_t K, uint32_t rht_signs, uint64_t seed, uint64_t offset_dgrad,
                                       uint64_t offset_wgrad, const fp4_tensor *dyq, const fp4_tensor *dyq_t,
                                       const fp4_tensor *xq_t, void *ws, size_t ws_bytes, const hipEvent_t *marks,
                                       hipStream_t stream);

/* Backward pass with MS-EDEN on the weight gradient (Quartet II page, paragraph 1:
 * MS-EDEN, the unbiased alternative to stochastic rounding for microscale formats,
 * with lower quantization error; here the FP4_Q_RHT64 | FP4_Q_EDEN reading of
 * fp4_quantize).  As fp4_linear_backward, except for the two wgrad operands: both
 * take the 64-point rotation keyed by rht_key along the M tokens (M a multiple of
 * 64), which cancels in the product over tokens -- dy^T with MS-EDEN (seed,
 * offset_wgrad) into dyq_t ([N][M]), x^T nearest-even into xq_t ([K][M]).  dy for
 * dgrad is quantized rowwise with stochastic rounding (seed, offset_dgrad) into dyq
 * as in fp4_linear_backward.  dy's two amaxes (plain, and after the rotation) come
 * from one read of dy.  x non-NULL: x^T is quantized
 * from x; NULL: xq_t must already hold it (fp4_quantize of x with FP4_Q_COLWISE |
 * FP4_Q_RHT64 and the same key).  The results equal fp4_quantize of each operand
 * followed by fp4_gemm_ws.  marks (3): after dy's two quantizations, after x^T's,
 * after the dgrad GEMM.  Errors: as fp4_linear_backward; FP4_ERR_SHAPE also for
 * M not a multiple of 64. */
FP4_API fp4_status fp4_linear_backward_eden(const void *dy, const void *x, fp4_dtype dtype, const fp4_tensor *wq_t,
                                            void *dx, fp4_dtype dx_dtype, void *dw, fp4_dtype dw_dtype, int64_t M,
                                            int64_t N, int64_t K, uint32_t rht_key, uint64_t seed,
                                            uint64_t offset_dgrad, uint64_t offset_wgrad, const fp4_tensor *dyq,
                                            const fp4_tensor *dyq_t, const fp4_tensor *xq_t, void *ws,
                                            size_t ws_bytes, const hipEvent_t *marks, hipStream_t stream);

/* NVFP4 Newton-Schulz: the Muon optimizer's orthogonalising iteration with every
 * GEMM operand in NVFP4 (Full-Stack FP4 pages, paragraph 1, the optimizer
 * sentence: Newton-Schulz iterations native in NVFP4; the pages give no
 * polynomial, so the coefficients are the caller's -- Muon's quintic is
 * (3.4445, -4.7750, 2.0315)).  One iteration on X [m][n] (fp32, row-major):
 *   A = X X^T              fp4_gemm(X left, X right), fp32 [m][m]
 *   A2 = A A^T             fp4_gemm(A left, A right) (A is symmetric up to rounding)
 *   B = b A + c A2         fl(fl(b A) + fl(c A2)), in the A A^T product's epilogue
 *                          (A2 is never stored)
 *   BX = B X               fp4_gemm(B, X^T), X^T quantized columnwise
 *   X' = a X + BX          fl(fl(a X) + BX), in place of X
 * Operand quantization by variant (flags):
 *   0                        every operand 1D nearest-even (the two operands of
 *                            X X^T, and of A A^T, are then the same quantization:
 *                            x_left and a_left serve both sides, and x_right and
 *                            a_right are not written; x_left and xt come from one
 *                            read of X, and the amaxes of B and of the next X are
 *                            taken as the element-wise steps write them);
 *   FP4_Q_RHT | FP4_Q_SR     every operand with the 16-point transform (mask
 *                            rht_signs) and stochastic rounding;
 *   FP4_Q_RHT64 | FP4_Q_EDEN left operands (X left, A left, B) MS-EDEN, right
 *                            operands (X right, A right, X^T) the 64-point transform
 *                            (key rht_signs) nearest-even.
 * With either non-zero variant the left and right layouts of X (and of A) share
 * one amax pass: both transform the tensor alike; with FP4_Q_RHT | FP4_Q_SR they
 * differ only in their random draws and come from one read of the tensor.
 * In iteration t the operands draw Philox offsets offset + 8 t + k, k = 0 (X left),
 * 1 (X right), 2 (A left), 3 (A right), 4 (B), 5 (X^T), all with key seed. */
typedef struct fp4_ns_config {
  float a, b, c;      /* X' = a X + (b A + c A A^T) X */
  uint32_t flags;     /* operand variant, as above */
  uint32_t rht_signs; /* 16-bit mask (FP4_Q_RHT) or 32-bit key (FP4_Q_RHT64) */
  uint64_t seed, offset;
} fp4_ns_config;

/* The iteration's intermediates, all caller-owned device memory, overwritten; after
 * a call they hold the last iteration's values.  Descriptors as for fp4_quantize:
 * x_left, x_right [m][n]; a_left, a_right, b_q [m][m]; xt [n][m]; none 2D. */
typedef struct fp4_ns_buffers {
  float *a;  /* [m][m]: A */
  float *b;  /* [m][m]: B */
  float *bx; /* [m][n]: B X; or NULL: X' = a X + B X is then taken in the B X GEMM's epilogue
              * (C = fl(v + fl(a X)) for each product v, X updated in place; the same values;
              * with variant 0 that epilogue also takes the next X's amax) */
  fp4_tensor x_left, x_right, a_left, a_right, b_q, xt;
  void *ws;  /* GEMM split-K workspace and the element-wise steps' scratch (fp4_newton_schulz_ws_bytes), 16-byte
              * aligned */
  size_t ws_bytes;
} fp4_ns_buffers;

/* x = X_iters from X_0, where X_0 = g / (|g|_F + 1e-7) when normalize is non-zero
 * (|g|_F^2 summed in binary64 on the device, the scale 1 / (|g|_F + 1e-7) rounded
 * once to binary32, each element one product), else X_0 = g.  g and x [m][n] fp32,
 * device, may be the same buffer; m and n multiples of 16 (of 64 with
 * FP4_Q_RHT64).  iters >= 0.  Errors: FP4_ERR_NULL, FP4_ERR_SHAPE, FP4_ERR_MODE (an
 * unknown variant), FP4_ERR_MISMATCH (a descriptor's shape), FP4_ERR_ALIGN,
 * FP4_ERR_WORKSPACE (ws below fp4_newton_schulz_ws_bytes), FP4_ERR_HIP. */
FP4_API fp4_status fp4_newton_schulz(const float *g, float *x, int64_t m, int64_t n, int32_t iters, int32_t normalize,
                                     const fp4_ns_config *cfg, const fp4_ns_buffers *bufs, hipStream_t stream);

/* Workspace bytes fp4_newton_schulz needs for X [m][n]: the largest split-K plan of
 * its three GEMMs (m x m x n, m x m x m, m x n x m, in each form a variant runs them:
 * whole, symmetric, accumulating into their output), at least 16384 bytes (the
 * normalisation's binary64 partial sums, the per-workgroup maxima of the
 * element-wise steps), rounded up to 256, plus 256 (the next X's maximum from the
 * fused epilogue).  FP4_ERR_NULL, FP4_ERR_SHAPE. */
FP4_API fp4_status fp4_newton_schulz_ws_bytes(int64_t m, int64_t n, size_t *bytes);

/* A short static description of a status code (never NULL). */
FP4_API const char *fp4_status_string(fp4_status status);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_AMD_H */
