// api.hip -- the extern "C" surface declared in include/nvfp4_amd.h: argument
// checks (all before any enqueue), then the launchers.  The linear-layer calls
// compose quantize and gemm exactly as the NVFP4-12B page's recipe assigns the
// roles (paragraph 2): weights 2D-scaled, weight-gradient operands Hadamard
// transformed, gradients stochastically rounded, everything else nearest-even.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.hpp"

namespace {

fp4_status from_hip(hipError_t e) { return e == hipSuccess ? FP4_OK : FP4_ERR_HIP; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

fp4_status check_tensor(const fp4_tensor *t, int64_t rows, int64_t cols, int32_t two_d) {
  if (!t || !t->amax) return FP4_ERR_NULL;
  if ((!t->codes || !t->scales) && rows > 0 && cols > 0) return FP4_ERR_NULL;  // empty tensors need no storage
  if (t->rows != rows || t->cols != cols || (t->two_d != 0) != (two_d != 0)) return FP4_ERR_MISMATCH;
  if (!aligned(t->codes, 16) || !aligned(t->scales, 8) || !aligned(t->amax, 4)) return FP4_ERR_ALIGN;
  return FP4_OK;
}

fp4_status check_input(const void *x, fp4_dtype dtype, int64_t rows, int64_t cols, int64_t ld) {
  if (dtype != FP4_BF16 && dtype != FP4_FP32) return FP4_ERR_DTYPE;
  if (rows < 0 || cols < 0 || ld < cols) return FP4_ERR_SHAPE;
  if (!x && rows > 0 && cols > 0) return FP4_ERR_NULL;
  // vector loads: 8 elements of a row at a time
  if (cols % 8 != 0 || ld % 8 != 0 || !aligned(x, 16)) return FP4_ERR_ALIGN;
  return FP4_OK;
}

fp4_status check_quantize(const void *x, fp4_dtype dtype, int64_t rows, int64_t cols, int64_t ld, uint32_t flags,
                          const fp4_tensor *out, const fp4_tensor *out_t) {
  const uint32_t known = FP4_Q_2D | FP4_Q_COLWISE | FP4_Q_RHT | FP4_Q_SR | FP4_Q_AMAX_GIVEN | FP4_Q_RHT64 | FP4_Q_EDEN;
  if (flags & ~known) return FP4_ERR_MODE;
  const bool two_d = flags & FP4_Q_2D;
  if (two_d && (flags & (FP4_Q_RHT | FP4_Q_SR | FP4_Q_RHT64 | FP4_Q_EDEN))) return FP4_ERR_MODE;
  if ((flags & FP4_Q_RHT) && (flags & FP4_Q_RHT64)) return FP4_ERR_MODE;
  if ((flags & FP4_Q_EDEN) && (!(flags & FP4_Q_RHT64) || (flags & FP4_Q_SR))) return FP4_ERR_MODE;
  if (out_t && !two_d) return FP4_ERR_MODE;
  fp4_status s = check_input(x, dtype, rows, cols, ld);
  if (s != FP4_OK) return s;
  const bool colwise = flags & FP4_Q_COLWISE;
  const int64_t lrows = colwise ? cols : rows, lcols = colwise ? rows : cols;
  if (lcols % 16 != 0) return FP4_ERR_SHAPE;
  if (two_d && lrows % 16 != 0) return FP4_ERR_SHAPE;
  if ((flags & FP4_Q_RHT) && colwise && rows % 16 != 0) return FP4_ERR_SHAPE;
  if ((flags & FP4_Q_RHT64) && lcols % 64 != 0) return FP4_ERR_SHAPE;
  // columnwise and 2D launches give each 256 rows of x one grid row (at most 65535)
  if ((colwise || two_d) && (rows + 255) / 256 > 65535) return FP4_ERR_SHAPE;
  if ((s = check_tensor(out, lrows, lcols, two_d)) != FP4_OK) return s;
  if (out_t && (s = check_tensor(out_t, lcols, lrows, 1)) != FP4_OK) return s;
  return FP4_OK;
}

fp4_status check_gemm(const fp4_tensor *a, const fp4_tensor *b, const void *c, fp4_dtype c_dtype, int64_t ldc) {
  if (!a || !b) return FP4_ERR_NULL;
  if (c_dtype != FP4_BF16 && c_dtype != FP4_FP32) return FP4_ERR_DTYPE;
  if (a->rows < 0 || b->rows < 0 || a->cols < 0 || a->cols != b->cols) return FP4_ERR_MISMATCH;
  if (a->cols % 16 != 0) return FP4_ERR_SHAPE;
  fp4_status s;
  if ((s = check_tensor(a, a->rows, a->cols, a->two_d)) != FP4_OK) return s;
  if ((s = check_tensor(b, b->rows, b->cols, b->two_d)) != FP4_OK) return s;
  if ((a->two_d && a->rows % 16 != 0) || (b->two_d && b->rows % 16 != 0)) return FP4_ERR_SHAPE;
  if (ldc < b->rows) return FP4_ERR_SHAPE;
  if (!c && a->rows > 0 && b->rows > 0) return FP4_ERR_NULL;
  if (!aligned(c, c_dtype == FP4_BF16 ? 2 : 4)) return FP4_ERR_ALIGN;
  return FP4_OK;
}

// The transform's signs: a 16-bit mask (16-point transform) or a 32-bit key (64-point).
uint32_t sign_key(uint32_t flags, uint32_t rht_signs) { return (flags & FP4_Q_RHT64) ? rht_signs : rht_signs & 0xFFFFu; }

// The workspace of the GEMMs' split-K partial tiles: empty, or 16-byte aligned.
fp4_status check_ws(const void *ws, size_t ws_bytes) {
  if (ws_bytes > 0 && !ws) return FP4_ERR_NULL;
  if (ws_bytes > 0 && !aligned(ws, 16)) return FP4_ERR_ALIGN;
  return FP4_OK;
}

// Record the caller's phase event i (if the caller passed events) on the stream.
hipError_t mark(const hipEvent_t *marks, int i, hipStream_t stream) {
  return marks ? hipEventRecord(marks[i], stream) : hipSuccess;
}

}  // namespace

extern "C" {

fp4_status fp4_tensor_bytes(int64_t rows, int64_t cols, int32_t two_d, size_t *codes_bytes, size_t *scales_bytes) {
  if (!codes_bytes || !scales_bytes) return FP4_ERR_NULL;
  if (rows < 0 || cols < 0 || cols % 16 != 0) return FP4_ERR_SHAPE;
  *codes_bytes = size_t(rows) * size_t(cols / 2);
  *scales_bytes = size_t(two_d ? (rows + 15) / 16 : rows) * size_t(cols / 16);
  return FP4_OK;
}

fp4_status fp4_amax(const void *x, fp4_dtype dtype, int64_t rows, int64_t cols, int64_t ld, uint32_t flags,
                    uint32_t rht_signs, float *amax_out, hipStream_t stream) {
  if (flags & ~(FP4_Q_COLWISE | FP4_Q_RHT | FP4_Q_RHT64)) return FP4_ERR_MODE;
  if ((flags & FP4_Q_RHT) && (flags & FP4_Q_RHT64)) return FP4_ERR_MODE;
  fp4_status s = check_input(x, dtype, rows, cols, ld);
  if (s != FP4_OK) return s;
  if (!amax_out) return FP4_ERR_NULL;
  const int64_t blocked = (flags & FP4_Q_COLWISE) ? rows : cols;
  if ((flags & FP4_Q_RHT) && blocked % 16 != 0) return FP4_ERR_SHAPE;
  if ((flags & FP4_Q_RHT64) && blocked % 64 != 0) return FP4_ERR_SHAPE;
  return from_hip(nvfp4::launch_amax(x, dtype, rows, cols, ld, flags, sign_key(flags, rht_signs), amax_out, stream));
}

fp4_status fp4_quantize(const void *x, fp4_dtype dtype, int64_t rows, int64_t cols, int64_t ld, uint32_t flags,
                        uint32_t rht_signs, uint64_t seed, uint64_t offset, const fp4_tensor *out,
                        const fp4_tensor *out_t, hipStream_t stream) {
  fp4_status s = check_quantize(x, dtype, rows, cols, ld, flags, out, out_t);
  if (s != FP4_OK) return s;
  return from_hip(nvfp4::launch_quantize(x, dtype, rows, cols, ld, flags, sign_key(flags, rht_signs), seed, offset,
                                         out, out_t, stream));
}

fp4_status fp4_quantize_dual(const void *x, fp4_dtype dtype, int64_t rows, int64_t cols, int64_t ld, uint32_t flags,
                             uint32_t rht_signs, uint64_t seed, uint64_t offset_rows, uint64_t offset_cols,
                             const fp4_tensor *out_rows, const fp4_tensor *out_cols, hipStream_t stream) {
  if (flags & ~(FP4_Q_SR | FP4_Q_RHT | FP4_Q_AMAX_GIVEN)) return FP4_ERR_MODE;
  fp4_status s = check_input(x, dtype, rows, cols, ld);
  if (s != FP4_OK) return s;
  if (rows % 16 != 0 || cols % 16 != 0) return FP4_ERR_SHAPE;
  if ((s = check_tensor(out_rows, rows, cols, 0)) != FP4_OK) return s;
  if ((s = check_tensor(out_cols, cols, rows, 0)) != FP4_OK) return s;
  return from_hip(nvfp4::launch_quantize_dual(x, dtype, rows, cols, ld, flags, rht_signs & 0xFFFFu, seed, offset_rows,
                                              offset_cols, out_rows, out_cols, stream));
}

fp4_status fp4_gemm(const fp4_tensor *a, const fp4_tensor *b, void *c, fp4_dtype c_dtype, int64_t ldc,
                    hipStream_t stream) {
  fp4_status s = check_gemm(a, b, c, c_dtype, ldc);
  if (s != FP4_OK) return s;
  return from_hip(nvfp4::launch_gemm(a, b, c, c_dtype, ldc, stream));
}

fp4_status fp4_gemm_ws_bytes(int64_t M, int64_t N, int64_t K, size_t *bytes) {
  if (!bytes) return FP4_ERR_NULL;
  if (M < 0 || N < 0 || K < 0 || K % 16 != 0) return FP4_ERR_SHAPE;
  *bytes = nvfp4::gemm_ws_bytes(M, N, K);
  return FP4_OK;
}

fp4_status fp4_gemm_ws(const fp4_tensor *a, const fp4_tensor *b, void *c, fp4_dtype c_dtype, int64_t ldc, void *ws,
                       size_t ws_bytes, hipStream_t stream) {
  fp4_status s = check_gemm(a, b, c, c_dtype, ldc);
  if (s != FP4_OK) return s;
  if ((s = check_ws(ws, ws_bytes)) != FP4_OK) return s;
  return from_hip(nvfp4::launch_gemm_ws(a, b, c, c_dtype, ldc, ws, ws_bytes, stream));
}

fp4_status fp4_gemm_noalloc(const fp4_tensor *a, const fp4_tensor *b, void *c, fp4_dtype c_dtype, int64_t ldc,
                            hipStream_t stream) {
  fp4_status s = check_gemm(a, b, c, c_dtype, ldc);
  if (s != FP4_OK) return s;
  if (nvfp4::gemm_ws_bytes_within(a->rows, b->rows, a->cols, nvfp4::kStaticScratchBytes) >
      nvfp4::kStaticScratchBytes)
    return FP4_ERR_WORKSPACE;
  void *scratch = nullptr;
  hipError_t e = nvfp4::static_scratch(&scratch);
  if (e != hipSuccess) return FP4_ERR_HIP;
  return from_hip(nvfp4::launch_gemm_ws(a, b, c, c_dtype, ldc, scratch, nvfp4::kStaticScratchBytes, stream));
}

fp4_status fp4_linear_ws_bytes(int64_t M, int64_t N, int64_t K, size_t *bytes) {
  if (!bytes) return FP4_ERR_NULL;
  if (M < 0 || N < 0 || K < 0 || M % 16 || N % 16 || K % 16) return FP4_ERR_SHAPE;
  const size_t f = nvfp4::gemm_ws_bytes(M, N, K), d = nvfp4::gemm_ws_bytes(M, K, N), w = nvfp4::gemm_ws_bytes(N, K, M);
  *bytes = f > d ? (f > w ? f : w) : (d > w ? d : w);
  return FP4_OK;
}

fp4_status fp4_linear_fprop(const void *x, const void *w, fp4_dtype dtype, void *y, fp4_dtype y_dtype, int64_t M,
                            int64_t N, int64_t K, uint32_t rht_signs, const fp4_tensor *xq, const fp4_tensor *xq_t,
                            const fp4_tensor *wq, const fp4_tensor *wq_t, void *ws, size_t ws_bytes,
                            const hipEvent_t *marks, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0 || M % 16 || N % 16 || K % 16) return FP4_ERR_SHAPE;
  fp4_status s;
  if ((s = check_quantize(x, dtype, M, K, K, 0, xq, nullptr)) != FP4_OK) return s;
  if (xq_t && (s = check_tensor(xq_t, K, M, 0)) != FP4_OK) return s;
  if ((s = check_quantize(w, dtype, N, K, K, FP4_Q_2D, wq, wq_t)) != FP4_OK) return s;
  if ((s = check_gemm(xq, wq, y, y_dtype, N)) != FP4_OK) return s;
  if ((s = check_ws(ws, ws_bytes)) != FP4_OK) return s;
  // x's and w's amax passes in one launch (w's runs in x's phase), then the layouts
  // with their amax given
  bool merged = false;
  const uint32_t signs = rht_signs & 0xFFFFu;
  hipError_t e = nvfp4::launch_amax_fprop(x, w, dtype, M, N, K, signs, xq, xq_t, wq, &merged, stream);
  const uint32_t given = merged ? FP4_Q_AMAX_GIVEN : 0u;
  if (e == hipSuccess)
    e = xq_t ? nvfp4::launch_quantize_dual(x, dtype, M, K, K, FP4_Q_RHT | given, signs, 0, 0, 0, xq, xq_t, stream)
             : nvfp4::launch_quantize(x, dtype, M, K, K, given, 0, 0, 0, xq, nullptr, stream);
  if (e == hipSuccess) e = mark(marks, 0, stream);
  if (e == hipSuccess) e = nvfp4::launch_quantize(w, dtype, N, K, K, FP4_Q_2D | given, 0, 0, 0, wq, wq_t, stream);
  if (e == hipSuccess) e = mark(marks, 1, stream);
  if (e == hipSuccess) e = nvfp4::launch_gemm_ws(xq, wq, y, y_dtype, N, ws, ws_bytes, stream);
  return from_hip(e);
}

fp4_status fp4_linear_dgrad(const void *dy, fp4_dtype dtype, const fp4_tensor *wq_t, void *dx, fp4_dtype dx_dtype,
                            int64_t M, int64_t N, int64_t K, uint64_t seed, uint64_t offset, const fp4_tensor *dyq,
                            void *ws, size_t ws_bytes, const hipEvent_t *marks, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0 || M % 16 || N % 16 || K % 16) return FP4_ERR_SHAPE;
  fp4_status s;
  if ((s = check_quantize(dy, dtype, M, N, N, FP4_Q_SR, dyq, nullptr)) != FP4_OK) return s;
  if ((s = check_tensor(wq_t, K, N, 1)) != FP4_OK) return s;
  if ((s = check_gemm(dyq, wq_t, dx, dx_dtype, K)) != FP4_OK) return s;
  if ((s = check_ws(ws, ws_bytes)) != FP4_OK) return s;
  hipError_t e = nvfp4::launch_quantize(dy, dtype, M, N, N, FP4_Q_SR, 0, seed, offset, dyq, nullptr, stream);
  if (e == hipSuccess) e = mark(marks, 0, stream);
  if (e == hipSuccess) e = nvfp4::launch_gemm_ws(dyq, wq_t, dx, dx_dtype, K, ws, ws_bytes, stream);
  return from_hip(e);
}

fp4_status fp4_linear_wgrad(const void *dy, const void *x, fp4_dtype dtype, void *dw, fp4_dtype dw_dtype,
                            int64_t M, int64_t N, int64_t K, uint32_t rht_signs, uint64_t seed, uint64_t offset,
                            const fp4_tensor *dyq_t, const fp4_tensor *xq_t, void *ws, size_t ws_bytes,
                            const hipEvent_t *marks, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0 || M % 16 || N % 16 || K % 16) return FP4_ERR_SHAPE;
  const uint32_t fdy = FP4_Q_COLWISE | FP4_Q_RHT | FP4_Q_SR, fx = FP4_Q_COLWISE | FP4_Q_RHT;
  fp4_status s;
  if ((s = check_quantize(dy, dtype, M, N, N, fdy, dyq_t, nullptr)) != FP4_OK) return s;
  if ((s = check_quantize(x, dtype, M, K, K, fx, xq_t, nullptr)) != FP4_OK) return s;
  if ((s = check_gemm(dyq_t, xq_t, dw, dw_dtype, K)) != FP4_OK) return s;
  if ((s = check_ws(ws, ws_bytes)) != FP4_OK) return s;
  const uint32_t signs = rht_signs & 0xFFFFu;
  // dy's and x's amax passes in one launch (x's runs in dy's phase), then the layouts
  bool merged = false;
  hipError_t e = nvfp4::launch_amax_wgrad(dy, x, dtype, M, N, K, signs, nullptr, dyq_t, xq_t, &merged, stream);
  const uint32_t given = merged ? FP4_Q_AMAX_GIVEN : 0u;
  if (e == hipSuccess)
    e = nvfp4::launch_quantize(dy, dtype, M, N, N, fdy | given, signs, seed, offset, dyq_t, nullptr, stream);
  if (e == hipSuccess) e = mark(marks, 0, stream);
  if (e == hipSuccess) e = nvfp4::launch_quantize(x, dtype, M, K, K, fx | given, signs, 0, 0, xq_t, nullptr, stream);
  if (e == hipSuccess) e = mark(marks, 1, stream);
  if (e == hipSuccess) e = nvfp4::launch_gemm_ws(dyq_t, xq_t, dw, dw_dtype, K, ws, ws_bytes, stream);
  return from_hip(e);
}

fp4_status fp4_linear_backward(const void *dy, const void *x, fp4_dtype dtype, const fp4_tensor *wq_t, void *dx,
                               fp4_dtype dx_dtype, void *dw, fp4_dtype dw_dtype, int64_t M, int64_t N, int64_t K,
                               uint32_t rht_signs, uint64_t seed, uint64_t offset_dgrad, uint64_t offset_wgrad,
                               const fp4_tensor *dyq, const fp4_tensor *dyq_t, const fp4_tensor *xq_t, void *ws,
                               size_t ws_bytes, const hipEvent_t *marks, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0 || M % 16 || N % 16 || K % 16) return FP4_ERR_SHAPE;
  fp4_status s;
  if ((s = check_input(dy, dtype, M, N, N)) != FP4_OK) return s;
  if ((s = check_tensor(dyq, M, N, 0)) != FP4_OK) return s;
  if ((s = check_tensor(dyq_t, N, M, 0)) != FP4_OK) return s;
  if (x && (s = check_quantize(x, dtype, M, K, K, FP4_Q_COLWISE | FP4_Q_RHT, xq_t, nullptr)) != FP4_OK) return s;
  if ((s = check_tensor(xq_t, K, M, 0)) != FP4_OK) return s;
  if ((s = check_tensor(wq_t, K, N, 1)) != FP4_OK) return s;
  if ((s = check_gemm(dyq, wq_t, dx, dx_dtype, K)) != FP4_OK) return s;
  if ((s = check_gemm(dyq_t, xq_t, dw, dw_dtype, K)) != FP4_OK) return s;
  if ((s = check_ws(ws, ws_bytes)) != FP4_OK) return s;
  const uint32_t signs = rht_signs & 0xFFFFu;
  // with x, dy's two amaxes and x^T's in one launch (x's runs in dy's phase)
  bool merged = false;
  hipError_t e = x ? nvfp4::launch_amax_wgrad(dy, x, dtype, M, N, K, signs, dyq, dyq_t, xq_t, &merged, stream)
                   : hipSuccess;
  const uint32_t given = merged ? FP4_Q_AMAX_GIVEN : 0u;
  if (e == hipSuccess)
    e = nvfp4::launch_quantize_dual(dy, dtype, M, N, N, FP4_Q_SR | FP4_Q_RHT | given, signs, seed, offset_dgrad,
                                    offset_wgrad, dyq, dyq_t, stream);
  if (e == hipSuccess) e = mark(marks, 0, stream);
  if (e == hipSuccess && x)
    e = nvfp4::launch_quantize(x, dtype, M, K, K, FP4_Q_COLWISE | FP4_Q_RHT | given, signs, 0, 0, xq_t, nullptr,
                               stream);
  if (e == hipSuccess) e = mark(marks, 1, stream);
  if (e == hipSuccess) e = nvfp4::launch_gemm_ws(dyq, wq_t, dx, dx_dtype, K, ws, ws_bytes, stream);
  if (e == hipSuccess) e = mark(marks, 2, stream);
  if (e == hipSuccess) e = nvfp4::launch_gemm_ws(dyq_t, xq_t, dw, dw_dtype, K, ws, ws_bytes, stream);
  return from_hip(e);
}

// Newton-Schulz workspace: the normalisation's scratch, the axpby maxima and the
// three GEMMs' split-K partial tiles share its start; then one 256-byte slot whose
// first word takes the next X's maximum from the B X GEMM's fused epilogue.
static size_t ns_max_slot(int64_t m, int64_t n) {
  size_t w = nvfp4::normalize_scratch_bytes();
  if (nvfp4::axpby_partial_bytes() > w) w = nvfp4::axpby_partial_bytes();
  // every product's plan: X X^T, A A^T and B X whole, X X^T symmetric, and the
  // accumulated ones (no stream-K): A A^T into B (symmetric or whole), B X into X
  const size_t g[8] = {nvfp4::gemm_ws_bytes(m, m, n),
                       nvfp4::gemm_ws_bytes(m, m, m),
                       nvfp4::gemm_ws_bytes(m, n, m),
                       nvfp4::gemm_ws_bytes_sym(m, n),
                       nvfp4::gemm_ws_bytes_sym(m, m),
                       nvfp4::gemm_ws_bytes_plan(m, m, m, false, true),
                       nvfp4::gemm_ws_bytes_plan(m, m, m, false, false),
                       nvfp4::gemm_ws_bytes_plan(m, n, m, false, false)};
  for (size_t v : g) w = v > w ? v : w;
  return (w + 255) / 256 * 256;
}

fp4_status fp4_linear_backward_eden(const void *dy, const void *x, fp4_dtype dtype, const fp4_tensor *wq_t, void *dx,
                                    fp4_dtype dx_dtype, void *dw, fp4_dtype dw_dtype, int64_t M, int64_t N, int64_t K,
                                    uint32_t rht_key, uint64_t seed, uint64_t offset_dgrad, uint64_t offset_wgrad,
                                    const fp4_tensor *dyq, const fp4_tensor *dyq_t, const fp4_tensor *xq_t, void *ws,
                                    size_t ws_bytes, const hipEvent_t *marks, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0 || M % 64 || N % 16 || K % 16) return FP4_ERR_SHAPE;
  const uint32_t f_dyt = FP4_Q_COLWISE | FP4_Q_RHT64 | FP4_Q_EDEN, f_xt = FP4_Q_COLWISE | FP4_Q_RHT64;
  fp4_status s;
  if ((s = check_quantize(dy, dtype, M, N, N, FP4_Q_SR, dyq, nullptr)) != FP4_OK) return s;
  if ((s = check_quantize(dy, dtype, M, N, N, f_dyt, dyq_t, nullptr)) != FP4_OK) return s;
  if (x && (s = check_quantize(x, dtype, M, K, K, f_xt, xq_t, nullptr)) != FP4_OK) return s;
  if ((s = check_tensor(xq_t, K, M, 0)) != FP4_OK) return s;
  if ((s = check_tensor(wq_t, K, N, 1)) != FP4_OK) return s;
  if ((s = check_gemm(dyq, wq_t, dx, dx_dtype, K)) != FP4_OK) return s;
  if ((s = check_gemm(dyq_t, xq_t, dw, dw_dtype, K)) != FP4_OK) return s;
  if ((s = check_ws(ws, ws_bytes)) != FP4_OK) return s;
  // both of dy's amaxes from one read, then each layout with its amax given
  hipError_t e = nvfp4::launch_amax_rows_cols64(dy, dtype, M, N, rht_key, dyq, dyq_t, stream);
  if (e == hipSuccess)
    e = nvfp4::launch_quantize(dy, dtype, M, N, N, FP4_Q_SR | FP4_Q_AMAX_GIVEN, 0, seed, offset_dgrad, dyq, nullptr,
                               stream);
  if (e == hipSuccess)
    e = nvfp4::launch_quantize(dy, dtype, M, N, N, f_dyt | FP4_Q_AMAX_GIVEN, rht_key, seed, offset_wgrad, dyq_t,
                               nullptr, stream);
  if (e == hipSuccess) e = mark(marks, 0, stream);
  if (e == hipSuccess && x) e = nvfp4::launch_quantize(x, dtype, M, K, K, f_xt, rht_key, 0, 0, xq_t, nullptr, stream);
  if (e == hipSuccess) e = mark(marks, 1, stream);
  if (e == hipSuccess) e = nvfp4::launch_gemm_ws(dyq, wq_t, dx, dx_dtype, K, ws, ws_bytes, stream);
  if (e == hipSuccess) e = mark(marks, 2, stream);
  if (e == hipSuccess) e = nvfp4::launch_gemm_ws(dyq_t, xq_t, dw, dw_dtype, K, ws, ws_bytes, stream);
  return from_hip(e);
}

fp4_status fp4_newton_schulz_ws_bytes(int64_t m, int64_t n, size_t *bytes) {
  if (!bytes) return FP4_ERR_NULL;
  if (m < 0 || n < 0 || m % 16 || n % 16) return FP4_ERR_SHAPE;
  *bytes = ns_max_slot(m, n) + 256;
  return FP4_OK;
}

fp4_status fp4_newton_schulz(const float *g, float *x, int64_t m, int64_t n, int32_t iters, int32_t normalize,
                             const fp4_ns_config *cfg, const fp4_ns_buffers *bufs, hipStream_t stream) {
  if (!cfg || !bufs) return FP4_ERR_NULL;
  if (m < 0 || n < 0 || iters < 0 || m % 16 || n % 16) return FP4_ERR_SHAPE;
  uint32_t fl, fr;  // quantization flags of the left and right operands
  if (cfg->flags == 0) {
    fl = fr = 0;
  } else if (cfg->flags == (FP4_Q_RHT | FP4_Q_SR)) {
    fl = fr = FP4_Q_RHT | FP4_Q_SR;
  } else if (cfg->flags == (FP4_Q_RHT64 | FP4_Q_EDEN)) {
    fl = FP4_Q_RHT64 | FP4_Q_EDEN;
    fr = FP4_Q_RHT64;
    if (m % 64 || n % 64) return FP4_ERR_SHAPE;
  } else {
    return FP4_ERR_MODE;
  }
  if ((!g || !x) && m > 0 && n > 0) return FP4_ERR_NULL;
  if ((!bufs->a || !bufs->b) && m > 0 && n > 0) return FP4_ERR_NULL;
  if (!aligned(g, 16) || !aligned(x, 16) || !aligned(bufs->a, 16) || !aligned(bufs->b, 16) || !aligned(bufs->bx, 16))
    return FP4_ERR_ALIGN;
  // without bx, X' = a X + B X is taken in the B X GEMM's epilogue (X updated in place)
  const bool fused = bufs->bx == nullptr;
  fp4_status s;
  if ((s = check_quantize(x, FP4_FP32, m, n, n, fl, &bufs->x_left, nullptr)) != FP4_OK) return s;
  if ((s = check_quantize(x, FP4_FP32, m, n, n, fr, &bufs->x_right, nullptr)) != FP4_OK) return s;
  if ((s = check_quantize(bufs->a, FP4_FP32, m, m, m, fl, &bufs->a_left, nullptr)) != FP4_OK) return s;
  if ((s = check_quantize(bufs->a, FP4_FP32, m, m, m, fr, &bufs->a_right, nullptr)) != FP4_OK) return s;
  if ((s = check_quantize(bufs->b, FP4_FP32, m, m, m, fl, &bufs->b_q, nullptr)) != FP4_OK) return s;
  if ((s = check_quantize(x, FP4_FP32, m, n, n, fr | FP4_Q_COLWISE, &bufs->xt, nullptr)) != FP4_OK) return s;
  if ((s = check_ws(bufs->ws, bufs->ws_bytes)) != FP4_OK) return s;
  size_t need = 0;
  fp4_newton_schulz_ws_bytes(m, n, &need);
  if (bufs->ws_bytes < need) return FP4_ERR_WORKSPACE;
  if (m == 0 || n == 0) return FP4_OK;
  const uint32_t key = (fl & FP4_Q_RHT64) ? cfg->rht_signs : cfg->rht_signs & 0xFFFFu;
  hipError_t e = hipSuccess;
  if (normalize) e = nvfp4::launch_normalize(g, x, m * n, 1e-7f, bufs->ws, stream);
  else if (g != x) e = hipMemcpyAsync(x, g, size_t(m * n) * sizeof(float), hipMemcpyDeviceToDevice, stream);
  for (int32_t t = 0; t < iters && e == hipSuccess; ++t) {
    const uint64_t o = cfg->offset + 8u * uint64_t(t);
    auto q = [&](const float *src, int64_t r, int64_t c, uint32_t f, uint64_t off, const fp4_tensor *out) {
      return nvfp4::launch_quantize(src, FP4_FP32, r, c, c, f, key, cfg->seed, off, out, nullptr, stream);
    };
    // The left and right rowwise layouts of one tensor [m][c] (RHT + SR, or MS-EDEN
    // and the 64-point transform) transform it alike, so one amax pass serves both
    // (MS-EDEN stores 7/4 of the transformed values' amax), and both layouts come
    // from one read: with RHT + SR they differ only in their random draws (one
    // kernel transforms and scales each block once and encodes it twice); with
    // MS-EDEN and the 64-point transform each block is rotated once and quantized
    // against each layout's tensor scale.
    auto q_pair = [&](const float *src, int64_t c, uint64_t off_l, uint64_t off_r, const fp4_tensor *left,
                      const fp4_tensor *right) {
      (void)off_r;  // the right MS-EDEN partner is nearest-even: it draws no random bits
      if (fl & FP4_Q_EDEN)
        return nvfp4::launch_quantize_rows64_pair(src, FP4_FP32, m, c, key, cfg->seed, off_l, left, right, stream);
      return nvfp4::launch_quantize_rows_pair(src, FP4_FP32, m, c, fl, key, cfg->seed, off_l, off_r, left, right,
                                              stream);
    };
    // Nearest-even: both operands of X X^T (and of A A^T) are the same quantization,
    // X's rowwise and columnwise layouts come from one read of X (the dual
    // quantization), and the amaxes of B and of the next X are taken by the axpby
    // steps that write them (per-workgroup maxima in the workspace), so those
    // tensors are quantized with their amax given.  The next X's maxima are reduced
    // into X's descriptors at the start of the next iteration, so that after the
    // call every descriptor describes the operand it holds.
    // With the fused epilogue the B X GEMM leaves the next X's maximum in the
    // workspace's last slot instead.
    const bool same = cfg->flags == 0;
    const fp4_tensor *xr = same ? &bufs->x_left : &bufs->x_right, *ar = same ? &bufs->a_left : &bufs->a_right;
    float *partial = static_cast<float *>(bufs->ws);
    float *xmax = same && fused ? reinterpret_cast<float *>(static_cast<char *>(bufs->ws) + ns_max_slot(m, n)) : nullptr;
    if (same) {
      const bool given = t > 0;  // the previous iteration left X's maxima
      if (given)
        e = fused ? nvfp4::launch_max_finish(xmax, 1, bufs->x_left.amax, bufs->xt.amax, stream)
                  : nvfp4::launch_max_finish(partial, nvfp4::axpby_parts(m * n), bufs->x_left.amax, bufs->xt.amax,
                                             stream);
      if (e == hipSuccess)
        e = nvfp4::launch_quantize_dual(x, FP4_FP32, m, n, n, given ? FP4_Q_AMAX_GIVEN : 0u, key, cfg->seed, o + 0,
                                        o + 5, &bufs->x_left, &bufs->xt, stream);
    } else {
      e = q_pair(x, n, o + 0, o + 1, &bufs->x_left, &bufs->x_right);
    }
    // with one quantization on both sides X X^T and A A^T are exactly symmetric: the
    // GEMM computes the tiles on and above the diagonal and mirrors them
    if (e == hipSuccess)
      e = same ? nvfp4::launch_gemm_sym_ws(&bufs->x_left, xr, bufs->a, m, bufs->ws, bufs->ws_bytes, stream)
               : nvfp4::launch_gemm_ws(&bufs->x_left, xr, bufs->a, FP4_FP32, m, bufs->ws, bufs->ws_bytes, stream);
    if (e == hipSuccess) e = same ? q(bufs->a, m, m, fl, o + 2, &bufs->a_left)
                                  : q_pair(bufs->a, m, o + 2, o + 3, &bufs->a_left, &bufs->a_right);
    if (same) {
      // B = fl(fl(c A2) + fl(b A)) in the symmetric A A^T's epilogue (A2 = A A^T is
      // never stored; the sum is the axpby's, operands swapped), B's amax with it (with
      // the other variants B's amax is that of its transformed values: an amax pass)
      if (e == hipSuccess)
        e = nvfp4::launch_gemm_sym_ws_acc(&bufs->a_left, ar, bufs->b, m, cfg->c, cfg->b, bufs->a, bufs->b_q.amax,
                                          bufs->ws, bufs->ws_bytes, stream);
      if (e == hipSuccess) e = q(bufs->b, m, m, fl | FP4_Q_AMAX_GIVEN, o + 4, &bufs->b_q);
    } else {
      // B in A A^T's epilogue as above, the whole product (its two operands differ)
      if (e == hipSuccess)
        e = nvfp4::launch_gemm_ws_acc(&bufs->a_left, ar, bufs->b, m, cfg->b, nullptr, bufs->ws, bufs->ws_bytes, stream,
                                      cfg->c, bufs->a);
      if (e == hipSuccess) e = q(bufs->b, m, m, fl, o + 4, &bufs->b_q);
      if (e == hipSuccess) e = q(x, m, n, fr | FP4_Q_COLWISE, o + 5, &bufs->xt);
    }
    if (e == hipSuccess && fused) {
      e = nvfp4::launch_gemm_ws_acc(&bufs->b_q, &bufs->xt, x, n, cfg->a, xmax, bufs->ws, bufs->ws_bytes, stream);
    } else if (e == hipSuccess) {
      e = nvfp4::launch_gemm_ws(&bufs->b_q, &bufs->xt, bufs->bx, FP4_FP32, n, bufs->ws, bufs->ws_bytes, stream);
      if (e == hipSuccess)
        e = same ? nvfp4::launch_axpby_amax(1.0f, bufs->bx, cfg->a, x, m * n, partial, stream)
                 : nvfp4::launch_axpby(1.0f, bufs->bx, cfg->a, x, m * n, stream);
    }
  }
  return from_hip(e);
}

const char *fp4_status_string(fp4_status status) {
  switch (status) {
    case FP4_OK: return "ok";
    case FP4_ERR_NULL: return "a required pointer is NULL";
    case FP4_ERR_SHAPE: return "bad size: negative, or not a multiple of 16 where blocks need it";
    case FP4_ERR_ALIGN: return "a pointer or leading dimension breaks the required alignment";
    case FP4_ERR_DTYPE: return "unknown dtype";
    case FP4_ERR_MODE: return "unsupported combination of quantization flags";
    case FP4_ERR_MISMATCH: return "descriptor sizes do not agree with the call";
    case FP4_ERR_HIP: return "a HIP launch or runtime call failed";
    case FP4_ERR_WORKSPACE: return "the split-K plan of this shape needs more scratch than the static buffer holds";
  }
  return "unknown status";
}

}  // extern "C"
