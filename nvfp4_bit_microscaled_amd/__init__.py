"""Python binding of libnvfp4_amd.so, the gfx950 NVFP4 linear-layer library.

Argument marshalling only: every step runs in the library's HIP kernels.  Torch
supplies device memory and the current stream.  There is no fallback: if the
library is not built, load() raises.  The functions keep the C names and the
C argument order (see include/nvfp4_amd.h for the definitions).
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnvfp4_amd.so")

FP4_BF16 = 0
FP4_FP32 = 1

Q_2D = 1 << 0
Q_COLWISE = 1 << 1
Q_RHT = 1 << 2
Q_SR = 1 << 3
Q_AMAX_GIVEN = 1 << 4
Q_RHT64 = 1 << 5
Q_EDEN = 1 << 6

STATUS = {0: "FP4_OK", 1: "FP4_ERR_NULL", 2: "FP4_ERR_SHAPE", 3: "FP4_ERR_ALIGN", 4: "FP4_ERR_DTYPE",
          5: "FP4_ERR_MODE", 6: "FP4_ERR_MISMATCH", 7: "FP4_ERR_HIP", 8: "FP4_ERR_WORKSPACE"}
STATIC_SCRATCH_BYTES = 64 << 20

# every symbol the header declares
EXPORTS = ("fp4_tensor_bytes", "fp4_amax", "fp4_quantize", "fp4_quantize_dual", "fp4_gemm", "fp4_gemm_ws",
           "fp4_gemm_ws_bytes", "fp4_gemm_noalloc", "fp4_linear_ws_bytes", "fp4_linear_fprop", "fp4_linear_dgrad", "fp4_linear_wgrad",
           "fp4_linear_backward", "fp4_linear_backward_eden", "fp4_newton_schulz", "fp4_newton_schulz_ws_bytes", "fp4_status_string")


class Fp4Error(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({status_string(code)})")


class fp4_tensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("amax", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("two_d", ctypes.c_int32)]


class fp4_ns_config(ctypes.Structure):
    _fields_ = [("a", ctypes.c_float), ("b", ctypes.c_float), ("c", ctypes.c_float), ("flags", ctypes.c_uint32),
                ("rht_signs", ctypes.c_uint32), ("seed", ctypes.c_uint64), ("offset", ctypes.c_uint64)]


class fp4_ns_buffers(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("bx", ctypes.c_void_p), ("x_left", fp4_tensor),
                ("x_right", fp4_tensor), ("a_left", fp4_tensor), ("a_right", fp4_tensor), ("b_q", fp4_tensor),
                ("xt", fp4_tensor), ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t)]


_lib = None


def load():
    """Load the built library (raises if it is missing: build it with
    nvfp4_bit_microscaled_amd/build.py or __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, u32, u64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int32
    tp = ctypes.POINTER(fp4_tensor)
    sz = ctypes.POINTER(ctypes.c_size_t)
    szv = ctypes.c_size_t
    sigs = {
        "fp4_tensor_bytes": [i64, i64, i32, sz, sz],
        "fp4_amax": [vp, i32, i64, i64, i64, u32, u32, vp, vp],
        "fp4_quantize": [vp, i32, i64, i64, i64, u32, u32, u64, u64, tp, tp, vp],
        "fp4_quantize_dual": [vp, i32, i64, i64, i64, u32, u32, u64, u64, u64, tp, tp, vp],
        "fp4_gemm": [tp, tp, vp, i32, i64, vp],
        "fp4_gemm_ws": [tp, tp, vp, i32, i64, vp, ctypes.c_size_t, vp],
        "fp4_gemm_ws_bytes": [i64, i64, i64, sz],
        "fp4_gemm_noalloc": [tp, tp, vp, i32, i64, vp],
        "fp4_linear_ws_bytes": [i64, i64, i64, sz],
        "fp4_linear_fprop": [vp, vp, i32, vp, i32, i64, i64, i64, u32, tp, tp, tp, tp, vp, szv, vp, vp],
        "fp4_linear_dgrad": [vp, i32, tp, vp, i32, i64, i64, i64, u64, u64, tp, vp, szv, vp, vp],
        "fp4_linear_wgrad": [vp, vp, i32, vp, i32, i64, i64, i64, u32, u64, u64, tp, tp, vp, szv, vp, vp],
        "fp4_linear_backward": [vp, vp, i32, tp, vp, i32, vp, i32, i64, i64, i64, u32, u64, u64, u64, tp, tp, tp, vp,
                                szv, vp, vp],
        "fp4_linear_backward_eden": [vp, vp, i32, tp, vp, i32, vp, i32, i64, i64, i64, u32, u64, u64, u64, tp, tp, tp,
                                     vp, szv, vp, vp],
        "fp4_newton_schulz": [vp, vp, i64, i64, i32, i32, ctypes.POINTER(fp4_ns_config),
                              ctypes.POINTER(fp4_ns_buffers), vp],
        "fp4_newton_schulz_ws_bytes": [i64, i64, sz],
    }
    for name, args in sigs.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.fp4_status_string.argtypes = [ctypes.c_int]
    L.fp4_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def status_string(code: int) -> str:
    return load().fp4_status_string(code).decode()


def _check(fn, code):
    if code != 0:
        raise Fp4Error(fn, code)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FP4_BF16
    if t.dtype == torch.float32:
        return FP4_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ld(x: torch.Tensor) -> int:
    assert x.dim() == 2 and x.stride(1) == 1, "2D row-major input expected"
    return x.stride(0)


class QTensor:
    """Device buffers of one quantized logical tensor (codes, scales, amax)."""

    def __init__(self, rows: int, cols: int, two_d: bool = False, device="cuda"):
        nc, ns = tensor_bytes(rows, cols, two_d)
        self.rows, self.cols, self.two_d = rows, cols, bool(two_d)
        self.codes = torch.empty(nc, dtype=torch.uint8, device=device)
        self.scales = torch.empty(ns, dtype=torch.uint8, device=device)
        self.amax = torch.zeros(1, dtype=torch.float32, device=device)
        self._desc = fp4_tensor(self.codes.data_ptr(), self.scales.data_ptr(), self.amax.data_ptr(), rows, cols,
                                int(self.two_d))

    @property
    def desc(self):
        return ctypes.byref(self._desc)

    def codes_2d(self):
        return self.codes.view(self.rows, self.cols // 2)

    def scales_2d(self):
        r = (self.rows + 15) // 16 if self.two_d else self.rows
        return self.scales.view(r, self.cols // 16)


def tensor_bytes(rows: int, cols: int, two_d: bool = False):
    nc, ns = ctypes.c_size_t(), ctypes.c_size_t()
    _check("fp4_tensor_bytes", load().fp4_tensor_bytes(rows, cols, int(two_d), ctypes.byref(nc), ctypes.byref(ns)))
    return nc.value, ns.value


def fp4_amax(x: torch.Tensor, flags: int, rht_signs: int, amax_out: torch.Tensor, stream=None):
    _check("fp4_amax", load().fp4_amax(x.data_ptr(), _dtype(x), x.shape[0], x.shape[1], _ld(x), flags, rht_signs,
                                       amax_out.data_ptr(), _stream(stream)))


def fp4_quantize(x: torch.Tensor, flags: int, rht_signs: int, seed: int, offset: int, out: QTensor,
                 out_t: QTensor = None, stream=None):
    _check("fp4_quantize", load().fp4_quantize(x.data_ptr(), _dtype(x), x.shape[0], x.shape[1], _ld(x), flags,
                                               rht_signs, seed, offset, out.desc,
                                               out_t.desc if out_t is not None else None, _stream(stream)))


def fp4_quantize_dual(x: torch.Tensor, flags: int, rht_signs: int, seed: int, offset_rows: int, offset_cols: int,
                      out_rows: QTensor, out_cols: QTensor, stream=None):
    _check("fp4_quantize_dual", load().fp4_quantize_dual(x.data_ptr(), _dtype(x), x.shape[0], x.shape[1], _ld(x), flags,
                                                         rht_signs, seed, offset_rows, offset_cols, out_rows.desc,
                                                         out_cols.desc, _stream(stream)))


def fp4_gemm(a: QTensor, b: QTensor, c: torch.Tensor, stream=None):
    _check("fp4_gemm", load().fp4_gemm(a.desc, b.desc, c.data_ptr(), _dtype(c), c.stride(0), _stream(stream)))


def fp4_gemm_ws_bytes(M: int, N: int, K: int) -> int:
    n = ctypes.c_size_t()
    _check("fp4_gemm_ws_bytes", load().fp4_gemm_ws_bytes(M, N, K, ctypes.byref(n)))
    return n.value


def fp4_gemm_ws(a: QTensor, b: QTensor, c: torch.Tensor, ws: torch.Tensor = None, stream=None):
    """ws: a device byte tensor (at least fp4_gemm_ws_bytes(M, N, K) bytes for the split)."""
    wp = ws.data_ptr() if ws is not None else None
    wb = ws.numel() * ws.element_size() if ws is not None else 0
    _check("fp4_gemm_ws", load().fp4_gemm_ws(a.desc, b.desc, c.data_ptr(), _dtype(c), c.stride(0), wp, wb,
                                             _stream(stream)))


def fp4_gemm_noalloc(a: QTensor, b: QTensor, c: torch.Tensor, stream=None):
    """fp4_gemm_ws with the library's static split-K scratch (no allocation)."""
    _check("fp4_gemm_noalloc", load().fp4_gemm_noalloc(a.desc, b.desc, c.data_ptr(), _dtype(c), c.stride(0),
                                                       _stream(stream)))


def fp4_linear_ws_bytes(M: int, N: int, K: int) -> int:
    n = ctypes.c_size_t()
    _check("fp4_linear_ws_bytes", load().fp4_linear_ws_bytes(M, N, K, ctypes.byref(n)))
    return n.value


def _ws(ws):
    """(pointer, bytes) of an optional device byte tensor used as a workspace."""
    if ws is None:
        return None, 0
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _marks(marks):
    """An optional list of HIP event handles (ints) as a C array."""
    if marks is None:
        return None
    return (ctypes.c_void_p * len(marks))(*marks)


def fp4_linear_fprop(x, w, y, xq: QTensor, wq: QTensor, wq_t: QTensor = None, xq_t: QTensor = None, rht_signs: int = 0,
                     ws=None, marks=None, stream=None):
    """xq_t (optional): x^T quantized after the 16-point transform with rht_signs, in
    the same read of x as xq.  ws: optional device byte tensor (fp4_linear_ws_bytes).
    marks: optional list of 2 HIP event handles recorded between the phases."""
    M, K = x.shape
    N = w.shape[0]
    assert x.dtype == w.dtype and x.is_contiguous() and w.is_contiguous() and y.is_contiguous()
    wp, wb = _ws(ws)
    _check("fp4_linear_fprop", load().fp4_linear_fprop(
        x.data_ptr(), w.data_ptr(), _dtype(x), y.data_ptr(), _dtype(y), M, N, K, rht_signs, xq.desc,
        xq_t.desc if xq_t is not None else None, wq.desc, wq_t.desc if wq_t is not None else None, wp, wb,
        _marks(marks), _stream(stream)))


def fp4_linear_dgrad(dy, wq_t: QTensor, dx, seed: int, offset: int, dyq: QTensor, ws=None, marks=None, stream=None):
    M, N = dy.shape
    K = dx.shape[1]
    assert dy.is_contiguous() and dx.is_contiguous()
    wp, wb = _ws(ws)
    _check("fp4_linear_dgrad", load().fp4_linear_dgrad(dy.data_ptr(), _dtype(dy), wq_t.desc, dx.data_ptr(),
                                                       _dtype(dx), M, N, K, seed, offset, dyq.desc, wp, wb,
                                                       _marks(marks), _stream(stream)))


def fp4_linear_wgrad(dy, x, dw, rht_signs: int, seed: int, offset: int, dyq_t: QTensor, xq_t: QTensor, ws=None,
                     marks=None, stream=None):
    M, N = dy.shape
    K = x.shape[1]
    assert dy.dtype == x.dtype and dy.is_contiguous() and x.is_contiguous() and dw.is_contiguous()
    wp, wb = _ws(ws)
    _check("fp4_linear_wgrad", load().fp4_linear_wgrad(dy.data_ptr(), x.data_ptr(), _dtype(dy), dw.data_ptr(),
                                                       _dtype(dw), M, N, K, rht_signs, seed, offset, dyq_t.desc,
                                                       xq_t.desc, wp, wb, _marks(marks), _stream(stream)))


def fp4_linear_backward(dy, x, wq_t: QTensor, dx, dw, rht_signs: int, seed: int, offset_dgrad: int,
                        offset_wgrad: int, dyq: QTensor, dyq_t: QTensor, xq_t: QTensor, ws=None, marks=None,
                        stream=None):
    """x may be None when xq_t already holds the transformed, transposed x (for
    instance from fp4_linear_fprop with xq_t).  marks: optional list of 3 HIP event
    handles."""
    M, N = dy.shape
    K = dx.shape[1]
    assert dy.is_contiguous() and dx.is_contiguous() and dw.is_contiguous()
    if x is not None:
        assert x.dtype == dy.dtype and x.is_contiguous()
    wp, wb = _ws(ws)
    _check("fp4_linear_backward", load().fp4_linear_backward(
        dy.data_ptr(), x.data_ptr() if x is not None else None, _dtype(dy), wq_t.desc, dx.data_ptr(), _dtype(dx),
        dw.data_ptr(), _dtype(dw), M, N, K, rht_signs, seed, offset_dgrad, offset_wgrad, dyq.desc, dyq_t.desc,
        xq_t.desc, wp, wb, _marks(marks), _stream(stream)))


def fp4_linear_backward_eden(dy, x, wq_t: QTensor, dx, dw, rht_key: int, seed: int, offset_dgrad: int,
                             offset_wgrad: int, dyq: QTensor, dyq_t: QTensor, xq_t: QTensor, ws=None, marks=None,
                             stream=None):
    """As fp4_linear_backward with MS-EDEN on dy^T and the 64-point rotation (32-bit
    key rht_key) on both wgrad operands.  x may be None when xq_t already holds x^T
    with that rotation."""
    M, N = dy.shape
    K = dx.shape[1]
    assert dy.is_contiguous() and dx.is_contiguous() and dw.is_contiguous()
    if x is not None:
        assert x.dtype == dy.dtype and x.is_contiguous()
    wp, wb = _ws(ws)
    _check("fp4_linear_backward_eden", load().fp4_linear_backward_eden(
        dy.data_ptr(), x.data_ptr() if x is not None else None, _dtype(dy), wq_t.desc, dx.data_ptr(), _dtype(dx),
        dw.data_ptr(), _dtype(dw), M, N, K, rht_key, seed, offset_dgrad, offset_wgrad, dyq.desc, dyq_t.desc,
        xq_t.desc, wp, wb, _marks(marks), _stream(stream)))


MUON_QUINTIC = (3.4445, -4.7750, 2.0315)


def fp4_newton_schulz_ws_bytes(m: int, n: int) -> int:
    v = ctypes.c_size_t()
    _check("fp4_newton_schulz_ws_bytes", load().fp4_newton_schulz_ws_bytes(m, n, ctypes.byref(v)))
    return v.value


class NsBuffers:
    """Caller-owned intermediates of fp4_newton_schulz for X [m][n]; after a call
    they hold the last iteration's A, B (= b A + c A A^T), B X and quantized
    operands.  keep_bx=False leaves B X out: X' = a X + B X is then taken in the
    B X GEMM's epilogue (the same values, without B X's pass through memory; with
    nearest-even operands the epilogue also takes the next X's amax)."""

    def __init__(self, m: int, n: int, device="cuda", keep_bx: bool = True):
        f32 = dict(dtype=torch.float32, device=device)
        self.a = torch.empty(m, m, **f32)
        self.b = torch.empty(m, m, **f32)
        self.bx = torch.empty(m, n, **f32) if keep_bx else None
        self.x_left, self.x_right = QTensor(m, n, device=device), QTensor(m, n, device=device)
        self.a_left, self.a_right = QTensor(m, m, device=device), QTensor(m, m, device=device)
        self.b_q = QTensor(m, m, device=device)
        self.xt = QTensor(n, m, device=device)
        self.ws = torch.empty(max(fp4_newton_schulz_ws_bytes(m, n), 16), dtype=torch.uint8, device=device)
        self._s = fp4_ns_buffers(self.a.data_ptr(), self.b.data_ptr(), self.bx.data_ptr() if keep_bx else None,
                                 self.x_left._desc, self.x_right._desc, self.a_left._desc, self.a_right._desc,
                                 self.b_q._desc, self.xt._desc, self.ws.data_ptr(), self.ws.numel())


def fp4_newton_schulz(g: torch.Tensor, x: torch.Tensor, iters: int, bufs: NsBuffers, normalize: bool = True,
                      coeffs=MUON_QUINTIC, flags: int = 0, rht_signs: int = 0, seed: int = 0, offset: int = 0,
                      stream=None):
    """x = X_iters of the NVFP4 Newton-Schulz iteration from g (fp32 [m][n])."""
    m, n = g.shape
    assert g.dtype == torch.float32 and x.dtype == torch.float32 and g.is_contiguous() and x.is_contiguous()
    cfg = fp4_ns_config(coeffs[0], coeffs[1], coeffs[2], flags, rht_signs & 0xFFFFFFFF, seed, offset)
    _check("fp4_newton_schulz", load().fp4_newton_schulz(g.data_ptr(), x.data_ptr(), m, n, iters, int(normalize),
                                                         ctypes.byref(cfg), ctypes.byref(bufs._s), _stream(stream)))


class LinearBuffers:
    """Caller-owned quantized buffers for one linear layer y = x . w^T (M tokens,
    K in-features, N out-features)."""

    def __init__(self, M: int, N: int, K: int, device="cuda"):
        self.xq = QTensor(M, K, device=device)
        self.wq = QTensor(N, K, two_d=True, device=device)
        self.wq_t = QTensor(K, N, two_d=True, device=device)
        self.dyq = QTensor(M, N, device=device)
        self.dyq_t = QTensor(N, M, device=device)
        self.xq_t = QTensor(K, M, device=device)
