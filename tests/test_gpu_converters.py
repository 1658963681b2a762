"""The hardware conversions the kernels rely on, checked against the oracle over
exhaustive or dense sweeps on the GPU (tests/hwprobe wraps the product's own
device helpers from nvfp4_bit_microscaled_amd/csrc/device.hpp):

* E4M3 block-scale encode (e4m3_from_f32: gfx950's f32 -> fp8 converter after a
  clamp at 448) on every non-negative binary32 up to +inf;
* nearest-even E2M1 encode (encode8_rne: the FP4 converter plus the canonical-zero
  fix) on every binary32 bit pattern that is not an infinity or NaN;
* stochastic E2M1 encode (encode8_sr, each element through its own SR-converter
  call) on ~4.5 million values spanning 34 binades of both signs, each for all 2^16
  random values -- the add-and-truncate rule of the stochastic-rounding reading,
  whose unbiasedness is what the Quartet II page (paragraph 1) asks of SR;
* the GEMM's operand dequantization (dequant2: FP4 -> f16 converter, times the f16
  of the E4M3 scale) for every code byte, byte position and scale code;
* the FP4 -> f16 converter's f32 scale operand acting as its power of two only;
* the FP4 -> f32 converter MS-EDEN reads grid values with, for every code byte and
  byte position.

The expected values come from the oracle alone: each encoder of the oracle is a
monotone step function of its input (nearest-even of a magnitude; for stochastic
rounding, of the random value), so the smallest input of each output code, found by
bisection with the oracle's own encoder, defines the oracle's result for every
input.  Each test also compares the GPU with the oracle element by element on a
random sample, which checks the tables themselves.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hwprobe", "libhwconv.so")
INF_BITS = 0x7F800000


@pytest.fixture(scope="module")
def hw(fp4):
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB)
    vp, u32, u64, i64 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int64
    sig = {
        "hwc_e4m3_sweep": [u32, u64, vp, vp, vp, vp],
        "hwc_e4m3_encode": [vp, vp, i64, vp],
        "hwc_fp4_rne_sweep": [u64, u64, vp, vp, vp, vp],
        "hwc_fp4_sr_sweep": [vp, vp, vp, vp, i64, vp, vp, vp],
        "hwc_fp4_sr_encode": [vp, vp, vp, i64, vp],
        "hwc_dequant_table": [vp, vp],
        "hwc_fp4_cvt_scaled": [vp, vp, vp, i64, vp],
        "hwc_fp4_f32_table": [vp, vp],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    return L


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Counters:
    """Device mismatch count and smallest mismatching index."""

    def __init__(self):
        self.bad = torch.zeros(1, dtype=torch.int64, device="cuda")
        self.first = torch.full((1,), -1, dtype=torch.int64, device="cuda")  # all ones: no mismatch yet

    def ptrs(self):
        return ctypes.c_void_p(self.bad.data_ptr()), ctypes.c_void_p(self.first.data_ptr())

    def result(self):
        torch.cuda.synchronize()
        return int(self.bad.cpu()[0]), int(self.first.cpu()[0]) & 0xFFFFFFFFFFFFFFFF


def as_f32(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def first_bits_of_codes(encode, codes, lo=0, hi=INF_BITS):
    """Smallest bit pattern b in [lo, hi] with encode(b) >= c, for each code c, by
    bisection (encode: a monotone map of non-negative bit patterns to codes)."""
    codes = np.asarray(codes, dtype=np.int64)
    a = np.full(codes.shape, lo, dtype=np.int64)
    b = np.full(codes.shape, hi, dtype=np.int64)
    while np.any(a < b):
        act = a < b
        mid = (a + b) // 2
        up = encode(mid.astype(np.uint32)).astype(np.int64) >= codes
        b = np.where(act & up, mid, b)
        a = np.where(act & ~up, mid + 1, a)
    return a.astype(np.uint32)


def test_oracle_encoders_are_monotone(oracle):
    """The premise of the boundary tables: on sorted non-negative inputs the oracle's
    E4M3 codes and E2M1 magnitudes never decrease (a sample of 4 million patterns
    plus every pattern near each boundary)."""
    rng = np.random.default_rng(11)
    bits = np.sort(rng.integers(0, INF_BITS + 1, size=4_000_000, dtype=np.uint64)).astype(np.uint32)
    e4 = oracle.e4m3_encode_n(as_f32(bits)).astype(np.int64)
    assert np.all(np.diff(e4) >= 0)
    e2 = oracle.e2m1_encode_n(as_f32(bits)).astype(np.int64) & 7
    assert np.all(np.diff(e2) >= 0)


def test_e4m3_scale_encoder_every_nonnegative_binary32(hw, oracle):
    enc = lambda b: oracle.e4m3_encode_n(as_f32(b))  # noqa: E731
    starts = first_bits_of_codes(enc, np.arange(127))
    assert starts[0] == 0 and enc(np.array([INF_BITS], np.uint32))[0] == 0x7E
    # the table reproduces the oracle on either side of every boundary
    for c in range(1, 127):
        assert enc(np.array([starts[c]], np.uint32))[0] == c
        assert enc(np.array([starts[c] - 1], np.uint32))[0] == c - 1
    st = torch.from_numpy(starts.astype(np.int64).astype(np.uint32).view(np.int32)).cuda()
    cnt = Counters()
    total = INF_BITS + 1
    chunk = 1 << 29
    for first in range(0, total, chunk):
        n = min(chunk, total - first)
        assert hw.hwc_e4m3_sweep(first, n, ctypes.c_void_p(st.data_ptr()), *cnt.ptrs(), _stream()) == 0
    bad, first_bad = cnt.result()
    assert bad == 0, f"{bad} E4M3 codes differ from the oracle; smallest input bits {first_bad:#010x}"
    # element by element on a random sample of values up to 500 and the boundary neighbourhoods
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.uniform(0, 500, 2_000_000).astype(np.float32),
                        as_f32((starts[1:, None].astype(np.int64) + np.arange(-64, 65)[None, :]).ravel())])
    xd = torch.from_numpy(x).cuda()
    out = torch.empty(x.size, dtype=torch.uint8, device="cuda")
    assert hw.hwc_e4m3_encode(ctypes.c_void_p(xd.data_ptr()), ctypes.c_void_p(out.data_ptr()), x.size, _stream()) == 0
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.e4m3_encode_n(x))


def test_fp4_nearest_even_encoder_every_finite_binary32(hw, oracle):
    enc = lambda b: oracle.e2m1_encode_n(as_f32(b)) & 7  # noqa: E731
    starts = first_bits_of_codes(enc, np.arange(8))
    assert starts[0] == 0 and enc(np.array([INF_BITS - 1], np.uint32))[0] == 7
    st = torch.from_numpy(starts.view(np.int32)).cuda()
    cnt = Counters()
    chunk = 1 << 30
    for first in range(0, 1 << 32, chunk):
        assert hw.hwc_fp4_rne_sweep(first, chunk, ctypes.c_void_p(st.data_ptr()), *cnt.ptrs(), _stream()) == 0
    bad, first_bad = cnt.result()
    assert bad == 0, f"{bad} nearest-even codes differ from the oracle; smallest input bits {first_bad:#010x}"


def sr_value_set(seed=13):
    """About 4.5 million values: in each binade 2^e, e = -30 .. 3, every pattern of the
    top 16 mantissa bits with random low bits, both signs; plus the E2M1 grid points,
    their midpoints and quarter points, zero, and values at and beyond 6."""
    rng = np.random.default_rng(seed)
    e = np.arange(-30, 4)
    top = np.arange(1 << 16, dtype=np.uint32)
    low = rng.integers(0, 1 << 7, size=(e.size, top.size), dtype=np.uint32)
    bits = ((e[:, None] + 127).astype(np.uint32) << 23) | (top[None, :] << 7) | low
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)
    mids = (grid[:-1] + grid[1:]) / 2
    quarters = np.concatenate([grid[:-1] + (grid[1:] - grid[:-1]) * f for f in (0.25, 0.75)]).astype(np.float32)
    extra = np.concatenate([grid, mids, quarters, np.float32([6.0, 6.25, 6.5, 7.0, 100.0, 1e30])])
    pos = np.concatenate([as_f32(bits.ravel()), extra.astype(np.float32)])
    return np.concatenate([pos, -pos])


def sr_table(oracle, v):
    """Per value (oracle): its code at u16 = 0, its code at u16 = 65535, and the
    smallest u16 from which it rounds up (65536: never)."""
    lo = oracle.e2m1_encode_n(v, True, np.zeros(v.size, np.uint32))
    hi = oracle.e2m1_encode_n(v, True, np.full(v.size, 65535, np.uint32))
    a = np.zeros(v.size, np.int64)
    b = np.full(v.size, 65536, np.int64)
    while np.any(a < b):
        act = a < b
        mid = (a + b) // 2  # below 65536 wherever a < b
        up = oracle.e2m1_encode_n(v, True, np.minimum(mid, 65535).astype(np.uint32)) != lo
        b = np.where(act & up, mid, b)
        a = np.where(act & ~up, mid + 1, a)
    return lo, hi, a


def test_fp4_stochastic_encoder_all_random_values(hw, oracle):
    v = sr_value_set()
    lo, hi, thresh = sr_table(oracle, v)
    # the oracle's rule, restated: rounding up from u16 = 2^16 - F, F = floor(2^16 frac)
    assert np.all((thresh == 65536) == (lo == hi))
    cnt = Counters()
    dv = torch.from_numpy(v).cuda()
    dt = torch.from_numpy(thresh.astype(np.uint32).view(np.int32)).cuda()
    dlo, dhi = torch.from_numpy(lo).cuda(), torch.from_numpy(hi).cuda()
    assert hw.hwc_fp4_sr_sweep(ctypes.c_void_p(dv.data_ptr()), ctypes.c_void_p(dt.data_ptr()),
                               ctypes.c_void_p(dlo.data_ptr()), ctypes.c_void_p(dhi.data_ptr()), v.size, *cnt.ptrs(),
                               _stream()) == 0
    bad, first_bad = cnt.result()
    if bad:
        i = first_bad >> 16
        pytest.fail(f"{bad} stochastic codes differ from the oracle; first at value {v[i]!r}, u16 {first_bad & 0xFFFF} "
                    f"(oracle: {lo[i]} below {thresh[i]}, {hi[i]} from there)")
    # element by element, random values and random bits, through the two-element step
    rng = np.random.default_rng(14)
    x = np.concatenate([rng.uniform(-7, 7, 3_000_000), rng.standard_normal(1_000_000) * 1e-3]).astype(np.float32)
    u = rng.integers(0, 1 << 16, size=x.size, dtype=np.uint16)
    xd, ud = torch.from_numpy(x).cuda(), torch.from_numpy(u.view(np.int16)).cuda()
    out = torch.empty(x.size, dtype=torch.uint8, device="cuda")
    assert hw.hwc_fp4_sr_encode(ctypes.c_void_p(xd.data_ptr()), ctypes.c_void_p(ud.data_ptr()),
                                ctypes.c_void_p(out.data_ptr()), x.size, _stream()) == 0
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.e2m1_encode_n(x, True, u.astype(np.uint32)))


def test_gemm_dequantization_every_code_and_scale(hw, oracle):
    out = torch.empty(64 * 256 * 4, dtype=torch.int32, device="cuda")
    assert hw.hwc_dequant_table(ctypes.c_void_p(out.data_ptr()), _stream()) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.float16).astype(np.float64).reshape(64, 256, 4, 2)
    e2 = np.array([oracle.e2m1_value(c) for c in range(16)])
    e4 = np.array([oracle.e4m3_value(c) for c in range(128)])
    checked = 0
    for p in range(64):
        for sel in range(4):
            s = (2 * p + (sel & 1)) & 127
            if s == 0x7F:  # the NaN code; the quantizers never write it
                continue
            for c in range(256):
                want = (e2[c & 15] * e4[s], e2[c >> 4] * e4[s])
                assert got[p, c, sel, 0] == want[0] and got[p, c, sel, 1] == want[1], (p, c, sel, s)
                checked += 1
    assert checked == 64 * 4 * 256 - 2 * 256  # all but the NaN scale code


def test_fp4_converter_scale_operand_is_a_power_of_two(hw, oracle):
    """With an f32 scale operand 2^k (1 + f), the FP4 -> f16 converter returns the
    E2M1 value times 2^k: the mantissa f is ignored.  That is why the GEMM leaves the
    operand at 1 and multiplies by the f16 E4M3 scale separately."""
    rng = np.random.default_rng(15)
    ks = np.arange(-14, 12)
    fracs = np.concatenate([[0.0, 0.125, 0.5, 0.875, 0.999], rng.uniform(0, 1, 11)])
    codes = np.arange(256, dtype=np.uint8)
    cb, kk, ff = np.meshgrid(codes, ks, fracs, indexing="ij")
    cb, kk, ff = cb.ravel(), kk.ravel(), ff.ravel()
    scales = (np.ldexp(1.0, kk) * (1.0 + ff)).astype(np.float32)
    db, ds = torch.from_numpy(cb).cuda(), torch.from_numpy(scales).cuda()
    out = torch.empty(cb.size, dtype=torch.int32, device="cuda")
    assert hw.hwc_fp4_cvt_scaled(ctypes.c_void_p(db.data_ptr()), ctypes.c_void_p(ds.data_ptr()),
                                 ctypes.c_void_p(out.data_ptr()), cb.size, _stream()) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.float16).astype(np.float64).reshape(-1, 2)
    e2 = np.array([oracle.e2m1_value(c) for c in range(16)])
    want = np.stack([e2[cb & 15], e2[cb >> 4]], axis=1) * np.ldexp(1.0, kk)[:, None]
    np.testing.assert_array_equal(got, want)


def test_fp4_to_f32_converter_every_code(hw, oracle):
    out = torch.empty(256 * 8, dtype=torch.float32, device="cuda")
    assert hw.hwc_fp4_f32_table(ctypes.c_void_p(out.data_ptr()), _stream()) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64).reshape(256, 4, 2)
    e2 = np.array([oracle.e2m1_value(c) for c in range(16)])
    for c in range(256):
        for sel in range(4):
            assert got[c, sel, 0] == e2[c & 15] and got[c, sel, 1] == e2[c >> 4], (c, sel)
