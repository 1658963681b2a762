// internal.hpp -- launchers shared between the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/nvfp4_amd.h"

namespace nvfp4 {

template <typename T>
struct same_type {
  using type = T;
};

// Launch `kernel` on `stream` and return that launch's own status.  hipLaunchKernel
// reports the error of this launch alone, so a failure left behind by the caller's
// earlier HIP work is neither returned as ours nor cleared (hipGetLastError after a
// launch would do both).  The arguments are converted to the kernel's parameter
// types here, so the pointers below point at exactly what the kernel expects.
template <typename... P>
hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream,
                  typename same_type<P>::type... args) {
  void *ptrs[] = {static_cast<void *>(&args)..., nullptr};
  return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, ptrs, 0, stream);
}

hipError_t launch_amax(const void *x, fp4_dtype dtype, int64_t R, int64_t C, int64_t ld, uint32_t flags,
                       uint32_t signs, float *out, hipStream_t stream);

// The two amaxes of a contiguous x [R][C] (R a multiple of 64) that the MS-EDEN
// backward quantizes twice, from one read: x's plain amax into *rows->amax (its
// rowwise layout) and 7/4 of the amax of x^T after the 64-point rotation keyed by
// `key` into *cols->amax (its columnwise MS-EDEN layout, FP4_Q_COLWISE |
// FP4_Q_RHT64 | FP4_Q_EDEN).  Partial maxima go to rows' codes buffer.
hipError_t launch_amax_rows_cols64(const void *x, fp4_dtype dtype, int64_t R, int64_t C, uint32_t key,
                                   const fp4_tensor *rows, const fp4_tensor *cols, hipStream_t stream);

// The forward call's amax passes in one launch plus one reduction launch: x [M][K]
// (its plain amax into *xq->amax; with xq_t also the amax of x^T after the 16-point
// transform with `signs` into *xq_t->amax) and w [N][K] (plain, into *wq->amax),
// both contiguous.  *merged tells whether it ran: it does not when a tensor is
// empty or too small to hold its partial maxima in its codes buffer, or when x's
// rows exceed the 4-column kernel's offsets; the caller then lets the
// quantizations take their own amax passes.
hipError_t launch_amax_fprop(const void *x, const void *w, fp4_dtype dtype, int64_t M, int64_t N, int64_t K,
                             uint32_t signs, const fp4_tensor *xq, const fp4_tensor *xq_t, const fp4_tensor *wq,
                             bool *merged, hipStream_t stream);

// The weight gradient's amax passes in one launch plus one reduction launch: dy
// [M][N] (the amax of dy^T after the 16-point transform with `signs` into
// *dyq_t->amax, and with dyq non-NULL dy's plain amax into *dyq->amax) and x [M][K]
// (x^T after the transform, into *xq_t->amax), both contiguous.  *merged as for
// launch_amax_fprop.
hipError_t launch_amax_wgrad(const void *dy, const void *x, fp4_dtype dtype, int64_t M, int64_t N, int64_t K,
                             uint32_t signs, const fp4_tensor *dyq, const fp4_tensor *dyq_t, const fp4_tensor *xq_t,
                             bool *merged, hipStream_t stream);

// *dst = fl(factor * *src), one thread: an amax taken by one quantization handed to
// another of the same transformed values (factor 7/4 into an MS-EDEN one).
hipError_t launch_amax_copy(const float *src, float *dst, float factor, hipStream_t stream);

// Two rowwise stochastic layouts a, b of one contiguous tensor [R][C] (row stride C)
// with Philox offsets off_a, off_b, from one read: flags FP4_Q_SR with optional
// FP4_Q_RHT and FP4_Q_AMAX_GIVEN (then *a->amax holds the amax).  *b->amax
// receives a's amax.  The same codes and scales as two launch_quantize calls.
hipError_t launch_quantize_rows_pair(const void *x, fp4_dtype dtype, int64_t R, int64_t C, uint32_t flags,
                                     uint32_t signs, uint64_t seed, uint64_t off_a, uint64_t off_b,
                                     const fp4_tensor *a, const fp4_tensor *b, hipStream_t stream);

// The MS-EDEN layout `eden` (FP4_Q_RHT64 | FP4_Q_EDEN, Philox offset offset_e) and
// the nearest-even layout `ne` (FP4_Q_RHT64) of one contiguous tensor [R][C], rowwise
// with the 64-point transform of key `key`, from one read after one amax pass: the
// same codes, scales and amaxes as two launch_quantize calls.
hipError_t launch_quantize_rows64_pair(const void *x, fp4_dtype dtype, int64_t R, int64_t C, uint32_t key,
                                       uint64_t seed, uint64_t offset_e, const fp4_tensor *eden, const fp4_tensor *ne,
                                       hipStream_t stream);

hipError_t launch_quantize(const void *x, fp4_dtype dtype, int64_t R, int64_t C, int64_t ld, uint32_t flags,
                           uint32_t signs, uint64_t seed, uint64_t offset, const fp4_tensor *out,
                           const fp4_tensor *out_t, hipStream_t stream);

hipError_t launch_quantize_dual(const void *x, fp4_dtype dtype, int64_t R, int64_t C, int64_t ld, uint32_t flags,
                                uint32_t signs, uint64_t seed, uint64_t off_rows, uint64_t off_cols,
                                const fp4_tensor *rows, const fp4_tensor *cols, hipStream_t stream);

hipError_t launch_gemm(const fp4_tensor *a, const fp4_tensor *b, void *c, fp4_dtype c_dtype, int64_t ldc,
                       hipStream_t stream);

// launch_gemm with a caller workspace for split-K partial tiles (used only when the
// split plan for the shape wants one and ws holds gemm_ws_bytes of the shape)
hipError_t launch_gemm_ws(const fp4_tensor *a, const fp4_tensor *b, void *c, fp4_dtype c_dtype, int64_t ldc, void *ws,
                          size_t ws_bytes, hipStream_t stream);
// launch_gemm_ws into an fp32 C with an addend S: C = fl(fl(alpha * v) + fl(beta * S)),
// v the product as launch_gemm_ws stores it; S = src (C's shape and stride, not
// overlapping C), or C itself when src is null (each element read and written by the
// same thread, so C may be updated in place).  With amax non-null, *amax is set to
// max |C| over the new C (zeroed by a launch of its own first; it must not lie in
// the split-K partial tiles of ws).
hipError_t launch_gemm_ws_acc(const fp4_tensor *a, const fp4_tensor *b, float *c, int64_t ldc, float beta,
                              float *amax, void *ws, size_t ws_bytes, hipStream_t stream, float alpha = 1.0f,
                              const float *src = nullptr);

size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K);
// C = A B^T for a product known to be symmetric (M = N and the same quantized
// operand on both sides, so exactly symmetric): on the main path only the 256x256
// tiles on and above the diagonal are computed, each tile above the diagonal also
// stored transposed below it by the persistent launch's epilogue (after a split or
// stream-K plan a second kernel copies the upper triangle into the lower one instead);
// elsewhere the whole product.  fp32 C.
hipError_t launch_gemm_sym_ws(const fp4_tensor *a, const fp4_tensor *b, float *c, int64_t ldc, void *ws,
                              size_t ws_bytes, hipStream_t stream);
// Workspace of launch_gemm_sym_ws's plan for an M x M x K product.
size_t gemm_ws_bytes_sym(int64_t M, int64_t K);
// The symmetric product accumulated into an fp32 C: C = fl(fl(alpha * v) + fl(beta * S))
// with S = src (C's shape and stride, symmetric, not overlapping C unless src == c),
// on and above the diagonal, then mirrored; *amax (if non-null) = max |C|, zeroed
// first as in launch_gemm_ws_acc.
hipError_t launch_gemm_sym_ws_acc(const fp4_tensor *a, const fp4_tensor *b, float *c, int64_t ldc, float alpha,
                                  float beta, const float *src, float *amax, void *ws, size_t ws_bytes,
                                  hipStream_t stream);
// Workspace of the plan for an M x N x K product: stream-K allowed or not (an
// accumulated C takes no stream-K), symmetric or whole.
size_t gemm_ws_bytes_plan(int64_t M, int64_t N, int64_t K, bool allow_sk, bool sym);
// The workspace of the plan launch_gemm_ws runs with `limit` bytes: the stream-K
// plan's when it fits, else the fixed split's (which may still exceed the limit).
size_t gemm_ws_bytes_within(int64_t M, int64_t N, int64_t K, size_t limit);

// Size of the library's static split-K scratch (fp4_gemm_noalloc), per GPU.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;

// Device address of the static scratch on the current device (looked up once per
// device; allocates nothing).
hipError_t static_scratch(void **ptr);

// The Newton-Schulz iteration's binary32 steps (ns.hip).  n % 4 == 0 and 16-byte
// aligned vectors for the axpby launches.
hipError_t launch_axpby(float alpha, const float *x, float beta, float *y, int64_t n, hipStream_t stream);
// axpby that also leaves per-workgroup maxima of |y| in partial[0 .. axpby_parts(n))
// (axpby_partial_bytes() at most), reduced by launch_max_finish into *out0 (and *out1)
int axpby_parts(int64_t n);
size_t axpby_partial_bytes();
hipError_t launch_axpby_amax(float alpha, const float *x, float beta, float *y, int64_t n, float *partial,
                             hipStream_t stream);
hipError_t launch_max_finish(const float *partial, int n, float *out0, float *out1, hipStream_t stream);
size_t normalize_scratch_bytes();
hipError_t launch_normalize(const float *g, float *x, int64_t n, float eps, void *scratch, hipStream_t stream);

}  // namespace nvfp4
