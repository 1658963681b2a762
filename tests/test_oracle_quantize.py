"""Pins of the oracle's tensor-level quantization and GEMM reference.

Facts used (none of them produced by the oracle itself):
* hand-derived quantizations of small blocks (closed form, derived in the comments);
* the NVFP4-12B page's format property that at least one value in sixteen (the
  block maximum) is held at FP8-like precision: under nearest-even the block
  maximum encodes to +-6 and dequantizes within 2^-4 relative error;
* the tensor maximum dequantizes to itself (scale 448, element 6);
* 2D 16x16 scales give identical quantized values for W and W^T (NVFP4-12B page,
  2D block scaling for weights, so that forward and backward see the same W);
* stochastic rounding is unbiased (Quartet II page, paragraph 1);
* the GEMM reference is a binary64 matrix product, checked against a brute-force
  triple loop and one-hot selections.
"""
import numpy as np
import pytest

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def unpack(codes: np.ndarray) -> np.ndarray:
    lo = codes & 15
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)


def e2m1(c):
    c = np.asarray(c)
    v = GRID[c & 7]
    return np.where(c & 8, -v, v)


def test_worked_block_exact(oracle):
    """Row 0: the grid itself with tensor amax 6.  s_enc = 2688/6 = 448; block amax
    6 gives t = 1, u = 448, scale code 0x7E (448), multiplier 448/448 = 1, so every
    element lands on its own code.  -0 is written as +0."""
    row = np.array([6, -4, 3, -2, 1.5, -1, 0.5, 0, 6, 4, -3, 2, -1.5, 1, -0.5, -0.0], dtype=np.float32)
    q = oracle.quantize(row[None, :])
    assert q.amax == 6.0
    assert q.scales[0, 0] == 0x7E
    assert list(q.codes[0]) == [0xE7, 0xC5, 0xA3, 0x01, 0x67, 0x4D, 0x2B, 0x09]
    deq = oracle.dequantize(q)[0]
    # g = fl32(6/2688) = fl32(1/448): dequantized values are x (1 + d), |d| <= 2^-24
    np.testing.assert_allclose(deq, row.astype(np.float64), rtol=2.0**-23, atol=0)


def test_worked_block_with_mantissa_scale(oracle):
    """Block 0 holds the tensor amax 6 (as above); block 1 has amax 3: t = 0.5,
    u = 224 = 1.75 * 2^7 exactly, scale code (7+7)<<3 | 6 = 0x76, multiplier
    448/224 = 2, so 3 -> 6, 1.5 -> 3, 0.75 -> 1.5, 0.25 -> 0.5."""
    row = np.zeros(32, dtype=np.float32)
    row[0] = 6.0
    row[16:20] = [3.0, -1.5, 0.75, -0.25]
    q = oracle.quantize(row[None, :])
    assert q.scales[0, 1] == 0x76
    codes = unpack(q.codes)[0]
    assert list(codes[16:20]) == [7, 8 | 5, 3, 8 | 1]
    assert np.all(codes[20:32] == 0)


def test_worked_block_rounding(oracle):
    """Tensor amax 6 (block 0); block 1 = [1, 0.3, 0, ...]: t = fl(1/6),
    u = fl(t * 448) = 74.666..., E4M3 spacing in [64, 128) is 8, so the scale
    is 72 (code (6+7)<<3 | 1 = 0x69); multiplier fl(448/72) = 6.2222...;
    1 -> 6.22 saturates to 6 (code 7); 0.3 -> 1.867 rounds to 2 (code 4)."""
    row = np.zeros(32, dtype=np.float32)
    row[0] = 6.0
    row[16] = 1.0
    row[17] = 0.3
    q = oracle.quantize(row[None, :])
    assert q.scales[0, 1] == 0x69
    codes = unpack(q.codes)[0]
    assert codes[16] == 7 and codes[17] == 4
    deq = oracle.dequantize(q)[0]
    g = np.float64(np.float32(6.0) / np.float32(2688.0))
    assert deq[16] == 6 * 72 * g and deq[17] == 2 * 72 * g


def test_worked_block_saturated_multiplier(oracle):
    """Block [2^-129, 0, ...]: amax 2^-129 makes 2688 / amax overflow, so s_enc =
    FLT_MAX = (1 - 2^-24) 2^128; t = fl(2^-129 / 6) = 174763 * 2^-149 (subnormal,
    174762.67 rounded), u = t * FLT_MAX = 0.08333 rounds to the E4M3 value
    1.375 * 2^-4 (code 3<<3 | 3 = 0x1B); s_enc / 0.0859375 overflows, so the
    multiplier saturates at FLT_MAX as well: 2^-129 * FLT_MAX = 0.5 - 2^-25 rounds
    to 0.5 (code 1) and the zeros stay 0.  (An infinite multiplier would give
    code 7 and turn the zeros into NaN.)"""
    row = np.zeros(16, dtype=np.float32)
    row[0] = np.float32(2.0**-129)
    q = oracle.quantize(row[None, :])
    assert q.amax == np.float32(2.0**-129)
    assert q.scales[0, 0] == 0x1B
    codes = unpack(q.codes)[0]
    assert codes[0] == 1 and np.all(codes[1:] == 0)
    # stochastic: 0.5 - 2^-25 sits 2^-24 of a step below 0.5, so it rounds up for
    # every 16-bit draw but 0; the zeros stay 0
    c = unpack(oracle.quantize(row[None, :], sr=True, seed=1, offset=0).codes)[0]
    assert c[0] in (0, 1) and np.all(c[1:] == 0)


def test_zero_tensor(oracle):
    x = np.zeros((32, 64), dtype=np.float32)
    for kw in (dict(), dict(two_d=True), dict(colwise=True, rht=True, sr=True, signs=0x1234, seed=5, offset=9)):
        q = oracle.quantize(x, **kw)
        assert q.amax == 0.0
        assert np.all(q.codes == 0) and np.all(q.scales == 0)
        assert np.all(oracle.dequantize(q) == 0.0)


def block_max_property(oracle, x, q):
    """Every block (1D: 16 elements of a row; 2D: a 16x16 tile) whose E4M3 scale is
    normal (code >= 8) has its maximum encoded as +-6 and dequantized within 2^-4
    (plus a few binary32 roundings) of the input."""
    deq = oracle.dequantize(q)
    R, K = deq.shape
    codes = unpack(q.codes)
    if q.two_d:
        def tiles(a):
            return a.reshape(R // 16, 16, K // 16, 16).transpose(0, 2, 1, 3).reshape(R // 16, K // 16, 256)
        xb, db, cb = tiles(x.astype(np.float64)), tiles(deq), tiles(codes)
    else:
        xb = x.astype(np.float64).reshape(R, K // 16, 16)
        db = deq.reshape(R, K // 16, 16)
        cb = codes.reshape(R, K // 16, 16)
    normal = q.scales >= 8
    jmax = np.abs(xb).argmax(axis=2)
    xm = np.take_along_axis(xb, jmax[..., None], 2)[..., 0]
    dm = np.take_along_axis(db, jmax[..., None], 2)[..., 0]
    cm = np.take_along_axis(cb, jmax[..., None], 2)[..., 0]
    assert np.all((cm[normal] & 7) == 7)
    rel = np.abs(dm[normal] - xm[normal]) / np.abs(xm[normal])
    assert rel.max() <= 2.0**-4 + 1e-6
    return normal.mean()


def test_block_max_near_fp8_precision(oracle):
    import workloads
    rng = np.random.default_rng(11)
    x = workloads.normal(rng, (128, 512), outlier_frac=0.001)
    frac_normal = block_max_property(oracle, x, oracle.quantize(x))
    assert frac_normal > 0.9


def test_tensor_max_round_trips(oracle):
    rng = np.random.default_rng(12)
    x = rng.standard_normal((64, 256)).astype(np.float32) * 3
    q = oracle.quantize(x)
    deq = oracle.dequantize(q)
    i = np.unravel_index(np.abs(x).argmax(), x.shape)
    assert q.scales[i[0], i[1] // 16] == 0x7E
    assert abs(deq[i] - x[i]) <= 2.0**-21 * abs(x[i])


def test_rne_error_bound(oracle):
    """Each element is within half a grid step (at most 1, between 4 and 6) of its
    scaled value: |deq - x| <= Sf * g * 1 (and <= 0.25 Sf g below 2)."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    q = oracle.quantize(x)
    deq = oracle.dequantize(q)
    sf = np.array([oracle.e4m3_value(int(c)) for c in range(127)])[q.scales]
    g = oracle.decode_scale(q.amax)
    unit = np.repeat(sf, 16, axis=1) * g
    err = np.abs(deq - x)
    assert np.all(err <= unit * (1.0 + 1e-6))
    small = np.abs(x) < unit * 1.75
    assert np.all(err[small] <= unit[small] * (0.25 + 1e-6))


def test_two_d_scales_are_tile_constant_and_transpose_exactly(oracle):
    rng = np.random.default_rng(14)
    w = (rng.standard_normal((96, 160)) * 0.02).astype(np.float32)
    q = oracle.quantize(w, two_d=True)
    qt = oracle.quantize(w, two_d=True, colwise=True)
    assert q.scales.shape == (6, 10) and qt.scales.shape == (10, 6)
    np.testing.assert_array_equal(qt.scales, q.scales.T)
    np.testing.assert_array_equal(unpack(qt.codes), unpack(q.codes).T)
    np.testing.assert_array_equal(oracle.dequantize(qt), oracle.dequantize(q).T)
    # the tile scale is the 1D scale of the row holding the tile maximum
    q1 = oracle.quantize(w)
    for tr in range(6):
        for kb in range(10):
            tile = np.abs(w[tr * 16:(tr + 1) * 16, kb * 16:(kb + 1) * 16])
            r = tr * 16 + np.unravel_index(tile.argmax(), tile.shape)[0]
            assert q.scales[tr, kb] == q1.scales[r, kb]
    block_max_property(oracle, w, q)


def test_colwise_is_rowwise_of_transpose(oracle):
    rng = np.random.default_rng(15)
    x = rng.standard_normal((48, 80)).astype(np.float32)
    for kw in (dict(), dict(rht=True, signs=0xBEEF), dict(sr=True, seed=3, offset=4)):
        a = oracle.quantize(x, colwise=True, **kw)
        b = oracle.quantize(np.ascontiguousarray(x.T), **kw)
        np.testing.assert_array_equal(a.codes, b.codes)
        np.testing.assert_array_equal(a.scales, b.scales)
        assert a.amax == b.amax


def test_rht_amax_and_inner_products(oracle):
    """With RHT on both operands and the same signs, deq(A) . deq(B)^T approximates
    A . B^T (the transform cancels); without quantization noise it is exact up to
    binary32 rounding of the butterflies."""
    rng = np.random.default_rng(16)
    dy = rng.laplace(0, 1e-3, (64, 48)).astype(np.float32)
    x = rng.standard_normal((64, 32)).astype(np.float32)
    a = oracle.quantize(dy, colwise=True, rht=True, signs=0x9A5F)
    b = oracle.quantize(x, colwise=True, rht=True, signs=0x9A5F)
    # amax of the transformed tensor, computed independently with numpy
    h2 = np.array([[1, 1], [1, -1]], dtype=np.float64)
    h = np.kron(np.kron(np.kron(h2, h2), h2), h2)
    d = np.array([-1.0 if (0x9A5F >> j) & 1 else 1.0 for j in range(16)])
    T = np.diag(d) @ h / 4
    blk = dy.T.astype(np.float64).reshape(48, 4, 16) @ T
    assert abs(a.amax - np.abs(blk).max()) <= 1e-6 * a.amax
    y, bound = oracle.gemm_ref(a, b)
    exact = dy.T.astype(np.float64) @ x.astype(np.float64)
    rel = np.linalg.norm(y - exact) / np.linalg.norm(exact)
    assert rel < 0.2  # 4-bit quantization noise only


def test_sr_unbiased_over_offsets(oracle):
    """Averaged over Philox offsets, stochastically rounded values converge to the
    input: the deviation of the mean stays within 5.5 binomial standard deviations
    (p = position of the scaled value between its grid neighbours) plus the 2^-16
    resolution bias."""
    rng = np.random.default_rng(17)
    x = rng.standard_normal((16, 128)).astype(np.float32)
    n = 400
    acc = np.zeros(x.shape)
    for off in range(n):
        acc += oracle.dequantize(oracle.quantize(x, sr=True, seed=1, offset=off))
    mean = acc / n
    q = oracle.quantize(x)  # scales do not depend on the rounding mode
    sf = np.array([oracle.e4m3_value(int(c)) for c in range(127)])[q.scales]
    unit = np.repeat(sf, 16, axis=1) * oracle.decode_scale(q.amax)
    a = np.abs(x) / unit
    sat = a >= 6.0  # saturated elements round to 6 deterministically
    lo_i = np.clip(np.searchsorted(GRID, a, side="right") - 1, 0, 6)
    step = GRID[lo_i + 1] - GRID[lo_i]
    p = np.clip((a - GRID[lo_i]) / step, 0, 1)
    sd = unit * step * np.sqrt(p * (1 - p) / n)
    tol = 5.5 * sd + unit * step * 2.0**-16 + 1e-6 * np.abs(x)
    assert np.all((np.abs(mean - x) <= tol) | sat)
    # and the empirical bias is not systematic
    assert abs(np.mean((mean - x)[~sat] / unit[~sat])) < 0.01


def test_sr_depends_on_offset_and_seed_only(oracle):
    rng = np.random.default_rng(18)
    x = rng.standard_normal((32, 64)).astype(np.float32)
    a = oracle.quantize(x, sr=True, seed=7, offset=1)
    b = oracle.quantize(x, sr=True, seed=7, offset=1)
    c = oracle.quantize(x, sr=True, seed=7, offset=2)
    e = oracle.quantize(x, sr=True, seed=8, offset=1)
    np.testing.assert_array_equal(a.codes, b.codes)
    assert (a.codes != c.codes).mean() > 0.2 and (a.codes != e.codes).mean() > 0.2
    # row subsets reproduce the same random stream (indices are global)
    part = oracle.quantize(x, sr=True, seed=7, offset=1, rows=(8, 24))
    np.testing.assert_array_equal(part.codes, a.codes[8:24])
    np.testing.assert_array_equal(part.scales, a.scales[8:24])


def test_gemm_ref_brute_force(oracle):
    rng = np.random.default_rng(19)
    xa = rng.standard_normal((5, 32)).astype(np.float32)
    xb = rng.standard_normal((7, 32)).astype(np.float32)
    qa, qb = oracle.quantize(xa), oracle.quantize(xb)
    y, bound = oracle.gemm_ref(qa, qb)
    A, B = oracle.dequantize(qa), oracle.dequantize(qb)
    for m in range(5):
        for n in range(7):
            s = 0.0
            t = 0.0
            for k in range(32):
                s += A[m, k] * B[n, k]
                t += abs(A[m, k] * B[n, k])
            assert abs(y[m, n] - s) <= 1e-15 * t
            assert abs(bound[m, n] - t) <= 1e-15 * t


def test_gemm_ref_one_hot_selects_rows(oracle):
    """A one-hot row of A (a single 6 at column k, so the element encodes exactly)
    picks column k of deq(B) times the dequantized 6."""
    rng = np.random.default_rng(20)
    xb = rng.standard_normal((9, 48)).astype(np.float32)
    xa = np.zeros((3, 48), dtype=np.float32)
    for m, k in enumerate((0, 17, 47)):
        xa[m, k] = 6.0
    qa, qb = oracle.quantize(xa), oracle.quantize(xb)
    y, _ = oracle.gemm_ref(qa, qb)
    B = oracle.dequantize(qb)
    a6 = oracle.dequantize(qa)
    for m, k in enumerate((0, 17, 47)):
        np.testing.assert_array_equal(y[m], a6[m, k] * B[:, k])


def test_sr_random_bit_mapping(oracle):
    """Element i (row-major in the logical output) uses bits 16*(i&1)..+15 of word
    (i&7)>>1 of Philox4x32-10(counter = (i>>3 as two words, offset as two words),
    key = seed as two words).  Values exactly half-way between grid points reveal
    the top bit of that 16-bit draw: they round up iff it is 1 (2^15 + u16 carries
    out of 16 bits).  Each block holds a 6 so that its scale is 448 and its
    multiplier exactly 1."""
    R, K = 4, 64
    x = np.full((R, K), 0.25, dtype=np.float32)
    x[:, ::16] = 6.0
    x[1, 1::16] = 5.0  # half-way between 4 and 6
    seed, offset = 0x1234_5678_9ABC, 0x0F0F_0000_0003
    q = oracle.quantize(x, sr=True, seed=seed, offset=offset)
    assert np.all(q.scales == 0x7E)
    codes = unpack(q.codes)
    key = [seed & 0xFFFFFFFF, seed >> 32]
    for r in range(R):
        for k in range(K):
            if k % 16 == 0:
                continue
            i = r * K + k
            g = i >> 3
            w = oracle.philox4x32_10([g & 0xFFFFFFFF, g >> 32, offset & 0xFFFFFFFF, offset >> 32], key)
            u16 = (w[(i & 7) >> 1] >> (16 * (i & 1))) & 0xFFFF
            lo, hi = (6, 7) if x[r, k] == 5.0 else (0, 1)
            assert codes[r, k] == (hi if u16 >= 0x8000 else lo), (r, k)
