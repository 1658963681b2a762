"""Pins of the oracle's scalar building blocks against facts fixed outside the oracle.

* E2M1: the element grid {0, 0.5, 1, 1.5, 2, 3, 4, 6} (the 4-bit microscaling
  element format of the NVFP4-12B page, paragraph 2); encoding checked against a
  brute-force nearest-grid search written here in numpy.
* E4M3: the block-scale format (NVFP4-12B page, paragraph 2, format sentence);
  decode and encode checked against torch's float8_e4m3fn conversion, a library
  routine independent of the oracle.
* Philox4x32-10: the published known-answer vectors (tests/golden).
* Random Hadamard transform (NVFP4-12B page, paragraph 2, recipe sentence):
  checked against the Kronecker construction of Sylvester's H16 and H H^T = 16 I.
"""
import os

import numpy as np
import pytest
import torch

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
HERE = os.path.dirname(os.path.abspath(__file__))


# ----------------------------------------------------------------- E2M1
def test_e2m1_decode_table(oracle):
    for c in range(8):
        assert oracle.e2m1_value(c) == GRID[c]
        assert oracle.e2m1_value(c | 8) == -GRID[c]


def brute_e2m1_rne(s: np.ndarray) -> np.ndarray:
    """Nearest grid point by exhaustive distance; a tie goes to the even code."""
    # distances are exact in binary64 once |s| is clipped far above the grid
    a = np.minimum(np.abs(s.astype(np.float64)), 1e6)
    d = np.abs(a[:, None] - GRID[None, :])  # [n, 8]
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among equal-distance candidates take the even code (ties only ever involve two)
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    mag = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    sign = np.signbit(s) & (mag != 0)
    return (mag | (sign.astype(np.int64) << 3)).astype(np.uint8)


def e2m1_critical_points() -> np.ndarray:
    pts = list(GRID) + [(GRID[i] + GRID[i + 1]) / 2 for i in range(7)] + [6.5, 7.0, 8.0, 100.0, 1e30]
    pts = np.array(pts, dtype=np.float32)
    bits = pts.view(np.uint32).astype(np.int64)
    out = [pts]
    for d in (1, 2, 3, 17):
        out.append((bits + d).astype(np.uint32).view(np.float32))
        out.append(np.clip(bits - d, 0, None).astype(np.uint32).view(np.float32))
    v = np.concatenate(out)
    v = v[np.isfinite(v)]
    return np.concatenate([v, -v])


def test_e2m1_rne_critical_points(oracle):
    s = e2m1_critical_points()
    np.testing.assert_array_equal(oracle.e2m1_encode_n(s), brute_e2m1_rne(s))


def test_e2m1_rne_sweep(oracle):
    """Every 61st binary32 pattern in [0, 16), both signs."""
    bits = np.arange(0, 0x41800000, 61, dtype=np.uint32)
    s = bits.view(np.float32)
    np.testing.assert_array_equal(oracle.e2m1_encode_n(s), brute_e2m1_rne(s))
    np.testing.assert_array_equal(oracle.e2m1_encode_n(-s), brute_e2m1_rne(-s))


def test_e2m1_zero_is_canonical(oracle):
    assert oracle.e2m1_encode(-0.0) == 0
    assert oracle.e2m1_encode(-0.2) == 0  # rounds to zero: +0 code
    assert oracle.e2m1_encode(-0.2, True, 0) == 0  # u16 = 0 never rounds up


def test_e2m1_sr_exact_probabilities(oracle):
    """Stochastic rounding: over all 2^16 random values the number of "up" decisions
    is exactly floor(frac * 2^16), so the expectation is within 2^-16 of a step of
    the input (unbiased up to the 16-bit resolution; Quartet II page, paragraph 1)."""
    rng = np.random.default_rng(7)
    vals = np.concatenate([rng.uniform(0, 6, 40), GRID[:-1] + 1e-3, GRID, [5.999, 0.0001]]).astype(np.float32)
    u = np.arange(65536, dtype=np.uint32)
    for v in vals:
        codes = oracle.e2m1_encode_n(np.full(65536, v, dtype=np.float32), True, u)
        mags = codes & 7
        a = float(v)
        if a >= 6.0:
            assert np.all(mags == 7)
            continue
        lo = int(np.searchsorted(GRID, a, side="right") - 1)
        step = GRID[lo + 1] - GRID[lo]
        frac = (a - GRID[lo]) / step
        assert set(np.unique(mags)).issubset({lo, lo + 1})
        ups = int((mags == lo + 1).sum())
        assert ups == int(np.floor(frac * 65536)), (v, ups)
        mean = GRID[mags].mean()
        assert abs(mean - a) <= step * 2.0**-16 + 1e-12
        # the up decisions are exactly the random values whose sum with the 16-bit
        # position carries (a threshold rule: the largest draws go up)
        assert np.all((mags == lo + 1) == (u >= 65536 - np.floor(frac * 65536)))


def test_e2m1_sr_grid_points_never_move(oracle):
    u = np.arange(65536, dtype=np.uint32)
    for c in range(8):
        codes = oracle.e2m1_encode_n(np.full(65536, GRID[c], dtype=np.float32), True, u)
        assert np.all(codes == c)


# ----------------------------------------------------------------- E4M3
def torch_e4m3_values() -> np.ndarray:
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def test_e4m3_decode_matches_library(oracle):
    ref = torch_e4m3_values()
    for c in range(256):
        v = oracle.e4m3_value(c)
        if np.isnan(ref[c]):
            assert np.isnan(v)
        else:
            assert v == ref[c], c
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x01) == 2.0**-9


def test_e4m3_encode_matches_library(oracle):
    """Nearest-even rounding agrees with torch's float32 -> float8_e4m3fn cast wherever
    that cast is finite; where the cast overflows to NaN the oracle saturates to 448."""
    rng = np.random.default_rng(3)
    vals = [torch_e4m3_values()[:127]]
    v = vals[0]
    mids = (v[:-1] + v[1:]) / 2
    vals.append(mids)
    vals.append(rng.uniform(0, 500, 200000))
    vals.append(np.exp2(rng.uniform(-14, 9.5, 200000)))
    base = np.concatenate(vals).astype(np.float32)
    bits = base.view(np.uint32).astype(np.int64)
    allv = [base] + [(bits + d).astype(np.uint32).view(np.float32) for d in (-2, -1, 1, 2)]
    u = np.concatenate(allv)
    u = u[np.isfinite(u) & (u >= 0)]
    ours = oracle.e4m3_encode_n(u)
    ref = torch.from_numpy(u).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    fin = ~np.isnan(torch.from_numpy(u).to(torch.float8_e4m3fn).float().numpy())
    np.testing.assert_array_equal(ours[fin], ref[fin])
    assert np.all(ours[~fin] == 0x7E)
    assert oracle.e4m3_encode(float("inf")) == 0x7E
    assert oracle.e4m3_encode(1e30) == 0x7E


def test_e4m3_sweep_against_brute_force(oracle):
    """Every 101st binary32 pattern in [0, 2^10) against nearest-of-126 search."""
    vals = torch_e4m3_values()[:127]  # codes 0..0x7E, increasing
    bits = np.arange(0, 0x44800000, 101, dtype=np.uint32)
    u = bits.view(np.float32)
    ours = oracle.e4m3_encode_n(u)
    uu = u.astype(np.float64)
    idx = np.searchsorted(vals, uu)
    idx = np.clip(idx, 1, 126)
    lo, hi = vals[idx - 1], vals[idx]
    pick_hi = (uu - lo > hi - uu) | ((uu - lo == hi - uu) & (idx % 2 == 0))
    code = np.where(pick_hi, idx, idx - 1)
    code = np.where(uu >= 448.0, 126, code)
    np.testing.assert_array_equal(ours, code.astype(np.uint8))


# ----------------------------------------------------------------- Philox
def test_philox_known_answers(oracle):
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        vals = [int(t, 16) for t in r]
        assert oracle.philox4x32_10(vals[0:4], vals[4:6]) == vals[6:10]


def test_philox_bits_uniform(oracle):
    outs = np.array([oracle.philox4x32_10([i, 0, 5, 0], [11, 0]) for i in range(4096)], dtype=np.uint64)
    u16 = np.concatenate([outs & 0xFFFF, outs >> 16]).reshape(-1)
    # 16 bins of the top nibble: chi-square with 15 dof, loose 1e-4 level
    counts = np.bincount((u16 >> 12).astype(np.int64), minlength=16)
    exp = u16.size / 16
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert chi2 < 45.0


# ----------------------------------------------------------------- Hadamard
def sylvester_h16() -> np.ndarray:
    h2 = np.array([[1, 1], [1, -1]], dtype=np.float64)
    h = h2
    for _ in range(3):
        h = np.kron(h, h2)
    return h


def test_h16_orthogonality():
    h = sylvester_h16()
    np.testing.assert_array_equal(h @ h.T, 16 * np.eye(16))


@pytest.mark.parametrize("signs", [0x0000, 0xFFFF, 0xA5C3, 0x0001, 0x8000])
def test_rht_equals_matrix_on_integers(oracle, signs):
    """For small integers every butterfly is exact, so the transform must equal
    (x o d) H16 / 4 exactly; d_j = -1 where bit j of the mask is set."""
    h = sylvester_h16()
    d = np.array([-1.0 if (signs >> j) & 1 else 1.0 for j in range(16)])
    rng = np.random.default_rng(signs)
    for _ in range(50):
        x = rng.integers(-64, 65, 16).astype(np.float64)
        got = oracle.rht16(x, signs).astype(np.float64)
        np.testing.assert_array_equal(got, (x * d) @ h / 4.0)
    # unit vectors give the rows of D H / 4
    T = np.stack([oracle.rht16(np.eye(16)[j], signs) for j in range(16)]).astype(np.float64)
    np.testing.assert_array_equal(T, np.diag(d) @ h / 4.0)
    np.testing.assert_allclose(T @ T.T, np.eye(16), rtol=0, atol=0)


def test_rht_preserves_inner_products(oracle):
    """(a T) . (b T) = a . b: the transform cancels inside the weight-gradient GEMM."""
    rng = np.random.default_rng(1)
    for _ in range(100):
        a = rng.standard_normal(16).astype(np.float32)
        b = rng.standard_normal(16).astype(np.float32)
        ta = oracle.rht16(a, 0x3C5A).astype(np.float64)
        tb = oracle.rht16(b, 0x3C5A).astype(np.float64)
        ref = a.astype(np.float64) @ b.astype(np.float64)
        assert abs(ta @ tb - ref) <= 1e-5 * (np.abs(a) @ np.abs(b) + 1e-30)
