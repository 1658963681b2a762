"""CPU oracle for the NVFP4 quantize + block-scaled GEMM path.

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
the cpu_baseline leg of bench.py, never by the product package.  It shares no
code with the HIP library.

The quantization steps run in the C library next to this file (binary32, one
IEEE operation per step, in the order the steps are stated there); the GEMM
reference is the binary64 product of the dequantized operands, with numpy's
matmul as the library primitive.  What each step follows on the pages is cited
in nvfp4_oracle.c.
"""
import ctypes
import os

import numpy as np

from . import build as _build

# flag bits of nvo_quantize (same meaning as the product library's flags)
Q_2D = 1 << 0
Q_COLWISE = 1 << 1
Q_RHT = 1 << 2
Q_SR = 1 << 3
Q_RHT64 = 1 << 5
Q_EDEN = 1 << 6

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        i64 = ctypes.c_int64
        L.nvo_e2m1_value.restype = ctypes.c_double
        L.nvo_e2m1_value.argtypes = [ctypes.c_uint]
        L.nvo_e2m1_encode.restype = ctypes.c_uint
        L.nvo_e2m1_encode.argtypes = [ctypes.c_float, ctypes.c_int, ctypes.c_uint32]
        L.nvo_e4m3_value.restype = ctypes.c_double
        L.nvo_e4m3_value.argtypes = [ctypes.c_uint]
        L.nvo_e4m3_encode.restype = ctypes.c_uint
        L.nvo_e4m3_encode.argtypes = [ctypes.c_float]
        L.nvo_philox4x32_10.restype = None
        L.nvo_philox4x32_10.argtypes = [u32p, u32p, u32p]
        L.nvo_rht16.restype = None
        L.nvo_rht16.argtypes = [f32p, ctypes.c_uint32]
        L.nvo_amax.restype = ctypes.c_float
        L.nvo_amax.argtypes = [f32p, i64, i64, i64, ctypes.c_uint, ctypes.c_uint32, ctypes.c_int]
        L.nvo_decode_scale.restype = ctypes.c_float
        L.nvo_decode_scale.argtypes = [ctypes.c_float]
        L.nvo_quantize.restype = ctypes.c_int
        L.nvo_quantize.argtypes = [f32p, i64, i64, i64, ctypes.c_uint, ctypes.c_uint32, ctypes.c_uint64,
                                   ctypes.c_uint64, f32p, i64, i64, u8p, u8p, f32p, ctypes.c_int]
        L.nvo_dequantize.restype = None
        L.nvo_dequantize.argtypes = [u8p, u8p, i64, i64, ctypes.c_int, ctypes.c_float, f64p, ctypes.c_int]
        L.nvo_e2m1_encode_n.restype = None
        L.nvo_e2m1_encode_n.argtypes = [f32p, i64, ctypes.c_int, u32p, u8p]
        L.nvo_e4m3_encode_n.restype = None
        L.nvo_e4m3_encode_n.argtypes = [f32p, i64, u8p]
        L.nvo_e4m3_sr_n.restype = None
        L.nvo_e4m3_sr_n.argtypes = [f32p, i64, u32p, u8p]
        L.nvo_e4m3_sr.restype = ctypes.c_uint
        L.nvo_e4m3_sr.argtypes = [ctypes.c_float, ctypes.c_uint32]
        L.nvo_rht64_signs.restype = None
        L.nvo_rht64_signs.argtypes = [ctypes.c_uint64, ctypes.c_uint32, u32p]
        L.nvo_rht64.restype = None
        L.nvo_rht64.argtypes = [f32p, u32p]
        _lib = L
    return _lib


def default_threads() -> int:
    n = os.environ.get("NVO_THREADS") or os.environ.get("OMP_NUM_THREADS")
    return int(n) if n else min(16, os.cpu_count() or 1)


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


# ---------------------------------------------------------------- scalar codecs
def e2m1_value(code: int) -> float:
    return lib().nvo_e2m1_value(code)


def e2m1_encode(s: float, stochastic: bool = False, u16: int = 0) -> int:
    return lib().nvo_e2m1_encode(s, int(stochastic), u16)


def e2m1_encode_n(s, stochastic: bool = False, u16=None) -> np.ndarray:
    s = np.ascontiguousarray(s, dtype=np.float32).reshape(-1)
    out = np.empty(s.size, dtype=np.uint8)
    u = None if u16 is None else np.ascontiguousarray(u16, dtype=np.uint32).reshape(-1)
    lib().nvo_e2m1_encode_n(_ptr(s, ctypes.c_float), s.size, int(stochastic),
                            None if u is None else _ptr(u, ctypes.c_uint32), _ptr(out, ctypes.c_uint8))
    return out


def e4m3_encode_n(u) -> np.ndarray:
    u = np.ascontiguousarray(u, dtype=np.float32).reshape(-1)
    out = np.empty(u.size, dtype=np.uint8)
    lib().nvo_e4m3_encode_n(_ptr(u, ctypes.c_float), u.size, _ptr(out, ctypes.c_uint8))
    return out


def e4m3_value(code: int) -> float:
    return lib().nvo_e4m3_value(code)


def e4m3_encode(u: float) -> int:
    return lib().nvo_e4m3_encode(u)


def philox4x32_10(counter, key):
    c = (ctypes.c_uint32 * 4)(*[int(v) & 0xFFFFFFFF for v in counter])
    k = (ctypes.c_uint32 * 2)(*[int(v) & 0xFFFFFFFF for v in key])
    o = (ctypes.c_uint32 * 4)()
    lib().nvo_philox4x32_10(c, k, o)
    return [int(v) for v in o]


def rht16(v, signs: int) -> np.ndarray:
    a = np.ascontiguousarray(v, dtype=np.float32).copy()
    assert a.shape == (16,)
    lib().nvo_rht16(_ptr(a, ctypes.c_float), signs & 0xFFFF)
    return a


def e4m3_sr(y: float, u16: int) -> int:
    return lib().nvo_e4m3_sr(y, u16 & 0xFFFF)


def e4m3_sr_n(y, u16) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32).reshape(-1)
    u = np.ascontiguousarray(np.broadcast_to(np.asarray(u16, dtype=np.uint32), y.shape))
    out = np.empty(y.size, dtype=np.uint8)
    lib().nvo_e4m3_sr_n(_ptr(y, ctypes.c_float), y.size, _ptr(u, ctypes.c_uint32), _ptr(out, ctypes.c_uint8))
    return out


def rht64_signs(group: int, key: int):
    out = (ctypes.c_uint32 * 2)()
    lib().nvo_rht64_signs(group, key & 0xFFFFFFFF, out)
    return [int(out[0]), int(out[1])]


def rht64(v, group: int, key: int) -> np.ndarray:
    """The 64-point random Hadamard transform of group `group` under `key`."""
    a = np.ascontiguousarray(v, dtype=np.float32).copy()
    assert a.shape == (64,)
    sg = (ctypes.c_uint32 * 2)(*rht64_signs(group, key))
    lib().nvo_rht64(_ptr(a, ctypes.c_float), sg)
    return a


def decode_scale(amax: float) -> float:
    return lib().nvo_decode_scale(amax)


# ---------------------------------------------------------------- tensors
class QTensor:
    """A quantized logical tensor [rows, K]: codes [rows][K/2] (low nibble first),
    E4M3 scale codes (1D: [rows][K/16]; 2D: [rows/16][K/16]) and the tensor amax."""

    def __init__(self, codes, scales, amax, rows, K, two_d):
        self.codes, self.scales, self.amax = codes, scales, float(amax)
        self.rows, self.K, self.two_d = rows, K, bool(two_d)

    def row_slice(self, r0: int, r1: int) -> "QTensor":
        if self.two_d:
            assert r0 % 16 == 0 and (r1 % 16 == 0 or r1 == self.rows)
            sc = self.scales[r0 // 16:(r1 + 15) // 16]
        else:
            sc = self.scales[r0:r1]
        return QTensor(self.codes[r0:r1], sc, self.amax, r1 - r0, self.K, self.two_d)


def _as_f32(x) -> np.ndarray:
    x = np.asarray(x)
    assert x.ndim == 2
    return np.ascontiguousarray(x, dtype=np.float32)


def amax(x, colwise=False, rht=False, rht64=False, signs=0, threads=None) -> float:
    """Tensor amax of the logical tensor (after the 16-point transform with the 16-bit
    mask `signs`, or the 64-point one keyed by the 32-bit `signs`)."""
    x = _as_f32(x)
    flags = (Q_COLWISE if colwise else 0) | (Q_RHT if rht else 0) | (Q_RHT64 if rht64 else 0)
    a = float(lib().nvo_amax(_ptr(x, ctypes.c_float), x.shape[0], x.shape[1], x.shape[1], flags,
                             signs & 0xFFFFFFFF, threads or default_threads()))
    if a < 0:
        raise ValueError(f"oracle amax rejected shape {x.shape} flags {flags}")
    return a


def quantize(x, *, two_d=False, colwise=False, rht=False, sr=False, rht64=False, eden=False, signs=0, seed=0,
             offset=0, amax_in=None, rows=None, threads=None) -> QTensor:
    """Quantize the logical tensor (x, or x^T when colwise) of the fp32 array x.

    rht: the 16-point transform with the 16-bit mask `signs`; rht64: the 64-point
    transform keyed by the 32-bit `signs`; eden: MS-EDEN (needs rht64; the stored
    amax is 7/4 of the transformed tensor's); sr / eden draw from (seed, offset).
    rows: optional (row0, row1) range of logical rows to produce (amax is still
    that of the whole tensor)."""
    x = _as_f32(x)
    R, C = x.shape
    nrows_all, K = (C, R) if colwise else (R, C)
    r0, r1 = rows if rows is not None else (0, nrows_all)
    flags = (Q_2D if two_d else 0) | (Q_COLWISE if colwise else 0) | (Q_RHT if rht else 0) | (Q_SR if sr else 0) \
        | (Q_RHT64 if rht64 else 0) | (Q_EDEN if eden else 0)
    n = r1 - r0
    codes = np.zeros((n, K // 2), dtype=np.uint8)
    scales = np.zeros(((n // 16) if two_d else n, K // 16), dtype=np.uint8)
    a_out = np.zeros(1, dtype=np.float32)
    a_in = None if amax_in is None else np.array([amax_in], dtype=np.float32)
    rc = lib().nvo_quantize(_ptr(x, ctypes.c_float), R, C, C, flags, signs & 0xFFFFFFFF, seed, offset,
                            None if a_in is None else _ptr(a_in, ctypes.c_float), r0, n,
                            _ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8),
                            _ptr(a_out, ctypes.c_float), threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle quantize rejected shape {x.shape} flags {flags} rows {rows}")
    return QTensor(codes, scales, a_out[0], n, K, two_d)


def dequantize(q: QTensor, threads=None) -> np.ndarray:
    codes = np.ascontiguousarray(q.codes, dtype=np.uint8)
    scales = np.ascontiguousarray(q.scales, dtype=np.uint8)
    out = np.empty((q.rows, q.K), dtype=np.float64)
    lib().nvo_dequantize(_ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8), q.rows, q.K,
                         int(q.two_d), q.amax, _ptr(out, ctypes.c_double), threads or default_threads())
    return out


def gemm_ref(qa: QTensor, qb: QTensor):
    """Reference for C = deq(A) . deq(B)^T: the binary64 product and the bound
    sum_k |a_mk * b_nk| used by the acceptance test |y - y_ref| <= 1e-5 * bound."""
    assert qa.K == qb.K
    a = dequantize(qa)
    b = dequantize(qb)
    return a @ b.T, np.abs(a) @ np.abs(b).T


# ---------------------------------------------------------------- linear layer
def linear_fprop(x, w):
    """Y = X . W^T with X quantized 1D nearest-even and W 2D (16x16) nearest-even."""
    xq = quantize(x)
    wq = quantize(w, two_d=True)
    return xq, wq


def linear_dgrad(dy, w, seed, offset):
    """dX = dY . W: dY 1D stochastic rounding; W^T is the 2D quantization read transposed."""
    dyq = quantize(dy, sr=True, seed=seed, offset=offset)
    wtq = quantize(w, two_d=True, colwise=True)
    return dyq, wtq


def linear_wgrad(dy, x, signs, seed, offset):
    """dW = dY^T . X: both operands transposed (blocks along tokens), random Hadamard
    with the same signs on both, stochastic rounding on dY only."""
    dytq = quantize(dy, colwise=True, rht=True, sr=True, signs=signs, seed=seed, offset=offset)
    xtq = quantize(x, colwise=True, rht=True, signs=signs)
    return dytq, xtq


# ---------------------------------------------------------------- Newton-Schulz
# The Full-Stack FP4 pages (paragraph 1, optimizer sentence) run the Muon
# optimizer's Newton-Schulz iterations natively in NVFP4 and give no polynomial;
# the reading here is Muon's quintic X' = a X + (b A + c A A^T) X, A = X X^T, with
# every GEMM operand quantized (variants: nearest-even; 16-point transform + SR;
# MS-EDEN left operands with 64-point-rotated nearest-even right operands), the
# products the binary64 reference of the dequantized operands, the combinations in
# binary32 (one IEEE operation per step).

MUON_QUINTIC = (3.4445, -4.7750, 2.0315)


def ns_normalize(g, eps=1e-7):
    """X_0 = g * s, s = RN32(1 / (sqrt(sum g^2) + eps)), the sum in binary64."""
    g = _as_f32(g)
    ss = float(np.sum(g.astype(np.float64) ** 2))
    s = np.float32(1.0 / (np.sqrt(ss) + eps))
    return (g * s).astype(np.float32)


def ns_operand(x, variant, side, signs, seed, offset, colwise=False):
    """A GEMM operand of the iteration: x (or x^T) quantized per variant and side."""
    if variant == "rne":
        kw = {}
    elif variant == "rht_sr":
        kw = dict(rht=True, sr=True, signs=signs & 0xFFFF)
    elif variant == "eden":
        kw = dict(rht64=True, eden=(side == "left"), signs=signs)
    else:
        raise ValueError(variant)
    return quantize(x, colwise=colwise, seed=seed, offset=offset, **kw)


def ns_step(x, variant="rne", coeffs=MUON_QUINTIC, signs=0, seed=0, offset=0, a_in=None, b_in=None, bx_in=None):
    """One NVFP4 Newton-Schulz iteration on the fp32 array x [m][n]; operand k draws
    Philox offset `offset + k` (k = 0 X left, 1 X right, 2 A left, 3 A right, 4 B,
    5 X^T).  The products are the binary64 references rounded to binary32, unless
    a_in (A), b_in (B) or bx_in (B X) supply the values to continue from (a stage-wise
    comparison feeds the device's results in).  Returns every stage."""
    a_c, b_c, c_c = (np.float32(v) for v in coeffs)
    x = _as_f32(x)
    st = {"x": x}
    st["x_left"] = ns_operand(x, variant, "left", signs, seed, offset + 0)
    st["x_right"] = ns_operand(x, variant, "right", signs, seed, offset + 1)
    st["a_ref"], st["a_bound"] = gemm_ref(st["x_left"], st["x_right"])
    a = st["a_ref"].astype(np.float32) if a_in is None else _as_f32(a_in)
    st["a"] = a
    st["a_left"] = ns_operand(a, variant, "left", signs, seed, offset + 2)
    st["a_right"] = ns_operand(a, variant, "right", signs, seed, offset + 3)
    st["a2_ref"], st["a2_bound"] = gemm_ref(st["a_left"], st["a_right"])
    b = (b_c * a + c_c * st["a2_ref"].astype(np.float32)).astype(np.float32) if b_in is None else _as_f32(b_in)
    st["b"] = b
    st["b_q"] = ns_operand(b, variant, "left", signs, seed, offset + 4)
    st["xt"] = ns_operand(x, variant, "right", signs, seed, offset + 5, colwise=True)
    st["bx_ref"], st["bx_bound"] = gemm_ref(st["b_q"], st["xt"])
    bx = st["bx_ref"].astype(np.float32) if bx_in is None else _as_f32(bx_in)
    st["bx"] = bx
    st["x_next"] = (a_c * x + bx).astype(np.float32)
    return st


def newton_schulz(g, iters=5, variant="rne", coeffs=MUON_QUINTIC, signs=0, seed=0, offset=0, normalize=True):
    """The whole chain on the CPU: X_0 = g / (|g| + 1e-7), then `iters` iterations,
    iteration t with Philox offsets offset + 8 t + k."""
    x = ns_normalize(g) if normalize else _as_f32(g)
    for t in range(iters):
        x = ns_step(x, variant, coeffs, signs, seed, offset + 8 * t)["x_next"]
    return x
