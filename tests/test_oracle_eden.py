"""CPU pins of the oracle's 64-point random Hadamard transform and of MS-EDEN (the
unbiased microscale quantizer of the Quartet II page, paragraph 1, MS-EDEN
sentence), each against something other than the oracle's own formula:

* the transform against the Kronecker-built Sylvester H64 on integers (exact), and
  quantization with it against quantization of the exactly rotated input;
* the stochastic rounding of block scales against its exact expectation over all
  2^16 random values, with lo / hi found by brute force on the 127 E4M3 values;
* the EDEN correction: elements are the nearest-even codes of the usual scaled
  values, and each new block scale is a neighbour on the E4M3 grid of the old scale
  times sum s^2 / sum s e, recomputed here in binary64; over many blocks the
  stochastic scales average to that product;
* unbiasedness over the random rotations: the mean estimate over 3000 keys lies at
  the noise floor, while the same rotation without the correction (a control that
  proves the test can see a bias) does not;
* the page's error claim: MS-EDEN's mean squared error against that of stochastic
  rounding on the recipe's gradient-like and activation-like data.
"""
import numpy as np
import pytest

E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, 0, -0.5, -1, -1.5, -2, -3, -4, -6])


def sylvester(n):
    m = np.array([[1.0]])
    while m.shape[0] < n:
        m = np.block([[m, m], [m, -m]])
    return m


H64 = sylvester(64)


def e4m3_values():
    v = []
    for c in range(127):
        e, m = (c >> 3) & 15, c & 7
        v.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(v)


E4M3 = e4m3_values()


def sign_vector(oracle, group, key):
    s = oracle.rht64_signs(group, key)
    return np.array([-1.0 if (s[t >> 5] >> (t & 31)) & 1 else 1.0 for t in range(64)])


def unrotate(oracle, deq, key):
    """Inverse of the 64-point transform, group by group along each row (binary64)."""
    out = np.empty_like(deq)
    for j in range(deq.shape[1] // 64):
        out[:, 64 * j:64 * j + 64] = (deq[:, 64 * j:64 * j + 64] @ H64.T / 8) * sign_vector(oracle, j, key)
    return out


def test_h64_is_orthogonal():
    assert np.array_equal(H64 @ H64.T, 64 * np.eye(64))
    assert set(np.unique(H64)) == {-1.0, 1.0}


@pytest.mark.parametrize("key", [0, 1, 0xDEADBEEF])
def test_rht64_equals_kronecker_h64_on_integers(oracle, key):
    rng = np.random.default_rng(key & 0xFFFF)
    for group in (0, 1, 5, 2**33 + 7):
        x = rng.integers(-9, 10, 64).astype(np.float32)
        d = sign_vector(oracle, group, key)
        want = H64 @ (d * x) / 8  # exact: integers, then a power of two
        assert np.array_equal(oracle.rht64(x, group, key).astype(np.float64), want)
    # different groups and keys draw different signs
    assert not np.array_equal(sign_vector(oracle, 0, key), sign_vector(oracle, 1, key))
    assert not np.array_equal(sign_vector(oracle, 3, key), sign_vector(oracle, 3, key + 1))


@pytest.mark.parametrize("colwise", [False, True])
def test_rht64_quantize_is_quantize_of_the_rotated_tensor(oracle, colwise):
    """On integer data the rotation is exact, so quantizing with the transform
    equals quantizing the exactly rotated tensor without it (groups along the
    blocked dimension: rows of the logical tensor)."""
    rng = np.random.default_rng(3)
    key = 0x1234567
    x = rng.integers(-40, 41, (128, 192)).astype(np.float32)
    logical = x.T if colwise else x
    v = np.empty_like(logical, dtype=np.float64)
    for j in range(logical.shape[1] // 64):
        d = sign_vector(oracle, j, key)
        v[:, 64 * j:64 * j + 64] = (logical[:, 64 * j:64 * j + 64] * d) @ H64.T / 8
    q = oracle.quantize(x, colwise=colwise, rht64=True, signs=key)
    r = oracle.quantize(v.astype(np.float32))
    assert q.amax == r.amax
    assert np.array_equal(q.codes, r.codes) and np.array_equal(q.scales, r.scales)


def test_rht64_shape_rules(oracle):
    x = np.ones((16, 48), np.float32)
    with pytest.raises(ValueError):
        oracle.quantize(x, rht64=True)  # 48 is not a multiple of 64
    with pytest.raises(ValueError):
        oracle.quantize(np.ones((16, 64), np.float32), eden=True)  # MS-EDEN needs the 64-point transform
    with pytest.raises(ValueError):
        oracle.quantize(np.ones((16, 64), np.float32), rht64=True, eden=True, sr=True)


def brute_neighbours(y):
    i = np.searchsorted(E4M3, y, side="right") - 1
    return E4M3[i], E4M3[min(i + 1, 126)], i


@pytest.mark.parametrize("y", [0.0, 2.0 ** -12, 3 * 2.0 ** -11, 0.0123, 2.0 ** -6, 1.5, 1.5625, 1.59375, 3.3,
                               37.1, 255.9, 300.0, 415.5, 447.99, 448.0, 460.0, 1e9])
def test_e4m3_stochastic_rounding_expectation(oracle, y):
    u = np.arange(65536, dtype=np.uint32)
    codes = oracle.e4m3_sr_n(np.full(65536, y, np.float32), u)
    yf = float(np.float32(y))
    if yf >= 448.0:
        assert np.all(codes == 0x7E)
        return
    lo, hi, i = brute_neighbours(yf)
    assert set(np.unique(codes)) <= {i, i + 1}
    ups = int((codes == i + 1).sum())
    # exactly floor(2^16 frac) of the 2^16 draws go up, the last ones
    assert ups == int(np.floor((yf - lo) / (hi - lo) * 65536))
    assert np.all(codes[65536 - ups:] == i + 1) and np.all(codes[:65536 - ups] == i)
    mean = lo + (hi - lo) * ups / 65536
    assert abs(mean - yf) <= (hi - lo) * 2.0 ** -16
    if yf == lo:
        assert ups == 0  # grid points never move


def test_eden_blocks_follow_the_correction(oracle):
    """Recompute every block in binary64 from the oracle's own rotation: the codes
    are the nearest-even codes of the scaled values s, and the new scale is an E4M3
    neighbour of decode(S) * sum s^2 / sum s e; over all blocks the decoded new
    scales average to that product (unbiased stochastic rounding)."""
    rng = np.random.default_rng(5)
    x = rng.laplace(0, 1e-3, (128, 512)).astype(np.float32)
    key, seed, off = 99, 3, 4
    q = oracle.quantize(x, rht64=True, eden=True, signs=key, seed=seed, offset=off)
    vmax = oracle.amax(x, rht64=True, signs=key)
    assert q.amax == np.float32(1.75) * np.float32(vmax)
    s_enc = np.float32(2688.0) / np.float32(q.amax)
    ratios = []
    for r in range(x.shape[0]):
        v = np.concatenate([oracle.rht64(x[r, 64 * j:64 * j + 64], j, key) for j in range(x.shape[1] // 64)])
        for kb in range(x.shape[1] // 16):
            vb = v[16 * kb:16 * kb + 16]
            amax_b = np.float32(np.abs(vb).max())
            S = oracle.e4m3_encode(float(np.float32(np.float32(amax_b / np.float32(6.0)) * s_enc)))
            sf = np.float32(E4M3[S])
            mult = np.float32(s_enc / sf) if sf > 0 else np.float32(0.0)
            s = (vb * mult).astype(np.float32)
            byte = q.codes[r, 8 * kb:8 * kb + 8]
            code = np.stack([byte & 15, byte >> 4], axis=1).ravel()
            assert np.array_equal(code, oracle.e2m1_encode_n(s)), (r, kb)
            e = E2M1[code]
            d = float(np.dot(s.astype(np.float64), e))
            c = float(np.dot(s.astype(np.float64), s)) / d if d > 0 else 1.0
            y = float(sf) * c
            new = E4M3[q.scales[r, kb]]
            lo, hi, _ = brute_neighbours(y * (1 - 1e-6))
            _, hi2, _ = brute_neighbours(y * (1 + 1e-6))
            assert lo <= new <= hi2, (r, kb, y, new)
            if y > 0:
                ratios.append(new / y)
            assert 0.6 < c < 1.5 or d <= 0
    ratios = np.array(ratios)
    assert len(ratios) > 3000
    assert abs(ratios.mean() - 1.0) < 4 * ratios.std() / np.sqrt(len(ratios)) + 1e-4


def test_eden_is_unbiased_over_the_rotations(oracle):
    """Mean of the un-rotated MS-EDEN estimate over 3000 rotation keys (and scale
    draws): its distance from x is at the noise floor sqrt(E|err|^2 / N).  The same
    rotation with nearest-even and no correction stays biased, which shows the test
    can see a bias of that size."""
    rng = np.random.default_rng(0)
    x = rng.laplace(0, 1, (32, 128)).astype(np.float32)
    n = 3000
    nx = np.linalg.norm(x)
    ratio = {}
    for eden in (True, False):
        acc = np.zeros(x.shape)
        sq = 0.0
        for k in range(n):
            key = k * 7919 + 1
            q = oracle.quantize(x, rht64=True, eden=eden, signs=key, seed=k, offset=5, threads=1)
            xh = unrotate(oracle, oracle.dequantize(q, threads=1), key)
            acc += xh
            sq += ((xh - x) ** 2).sum()
        bias = np.linalg.norm(acc / n - x) / nx
        floor = np.sqrt(sq / n) / nx / np.sqrt(n)
        ratio[eden] = bias / floor
    assert ratio[True] < 1.35, ratio
    assert ratio[False] > 2.0, ratio


def test_eden_error_is_about_half_of_stochastic_rounding(oracle):
    """The page puts MS-EDEN's quantization error at more than 2x below stochastic
    rounding's.  Mean squared error relative to |x|^2, over 4 draws, on gradient-like
    (Laplace) and activation-like (Gaussian) data: against the recipe's own gradient
    quantizer (16-point transform + SR) this reading measures 2.03x and 2.01x;
    against plain SR 1.94x and 2.01x.  Asserted with margin below those figures."""
    rng = np.random.default_rng(1)
    data = {"laplace": rng.laplace(0, 1e-3, (256, 1024)).astype(np.float32),
            "gauss": rng.standard_normal((256, 1024)).astype(np.float32)}
    for name, x in data.items():
        nx2 = float((x.astype(np.float64) ** 2).sum())
        e_sr, e_eden = [], []
        for k in range(4):
            q = oracle.quantize(x, sr=True, seed=k, offset=1)
            e_sr.append(((oracle.dequantize(q) - x) ** 2).sum() / nx2)
            key = 1234 + k
            q = oracle.quantize(x, rht64=True, eden=True, signs=key, seed=k, offset=1)
            e_eden.append(((unrotate(oracle, oracle.dequantize(q), key) - x) ** 2).sum() / nx2)
        ratio = np.mean(e_sr) / np.mean(e_eden)
        assert ratio > 1.8, (name, ratio)
        assert np.mean(e_eden) < 0.011, (name, np.mean(e_eden))


def test_eden_zero_and_empty_blocks(oracle):
    x = np.zeros((16, 128), np.float32)
    q = oracle.quantize(x, rht64=True, eden=True, signs=5, seed=1, offset=1)
    assert q.amax == 0.0 and not q.codes.any() and not q.scales.any()
    # a zero row among non-zero rows: its blocks keep scale 0 and zero codes
    x = np.random.default_rng(2).standard_normal((16, 128)).astype(np.float32)
    x[3] = 0.0
    q = oracle.quantize(x, rht64=True, eden=True, signs=5, seed=1, offset=1)
    assert not q.codes[3].any() and not q.scales[3].any()
    assert q.scales[2].all()
