"""CPU pins of the oracle's NVFP4 Newton-Schulz chain (Muon's quintic, Full-Stack FP4
pages, paragraph 1, optimizer sentence), and the divergence it shows.

* Closed form: rows of a Hadamard matrix are orthogonal with equal norms, and NVFP4
  holds a matrix whose entries share one magnitude exactly, so the chain started
  there follows the scalar recursion s <- a s + b s^3 + c s^5 of its singular value
  (every singular value is the same).  That pins the polynomial's coefficients and
  powers, the products' orientation (X X^T, then B X) and the normalisation.
* Exact arithmetic on the same data (binary64 matmuls, no quantization) converges
  to singular values near 1, as Muon's quintic does; the NVFP4 chain on Gaussian
  data does not: after 5 iterations its largest singular value is far above it.
"""
import numpy as np
import pytest

A_, B_, C_ = 3.4445, -4.7750, 2.0315


def hadamard(n):
    m = np.array([[1.0]])
    while m.shape[0] < n:
        m = np.block([[m, m], [m, -m]])
    return m


def exact_chain(g, iters):
    x = g.astype(np.float64) / (np.linalg.norm(g.astype(np.float64)) + 1e-7)
    for _ in range(iters):
        a = x @ x.T
        x = A_ * x + (B_ * a + C_ * a @ a) @ x
    return x


def test_hadamard_rows_follow_the_scalar_recursion(oracle):
    """(Nearest-even operands only: a random rotation would spread the equal
    magnitudes, and the quantization would no longer be exact.)"""
    rng = np.random.default_rng(0)
    m, n = 64, 128
    h = hadamard(n)[rng.permutation(n)[:m]] * rng.choice([-1.0, 1.0], n)
    g = (0.37 * h).astype(np.float32)
    x = oracle.newton_schulz(g, iters=5, variant="rne")
    s = 1.0 / np.sqrt(m)  # |G/|G|_F| has m equal singular values of 1/sqrt(m)
    for _ in range(5):
        s = A_ * s + B_ * s ** 3 + C_ * s ** 5
    expect = s * np.sqrt(m) * g.astype(np.float64) / np.linalg.norm(g.astype(np.float64))
    assert np.abs(x - expect).max() <= 1e-5 * np.abs(expect).max()


def test_normalisation_is_the_frobenius_norm(oracle):
    g = np.random.default_rng(1).standard_normal((32, 64)).astype(np.float32)
    x0 = oracle.ns_normalize(g)
    assert abs(np.linalg.norm(x0.astype(np.float64)) - 1.0) < 1e-6


def test_nvfp4_chain_diverges_where_exact_arithmetic_converges(oracle):
    """The experiment behind the design notes' Newton-Schulz figures: a 256 x 512
    Gaussian G, 5 iterations.  Exact arithmetic ends with singular values in about
    [0.68, 1.13]; NVFP4 operands (nearest-even) end far outside: the quintic's
    a X + (b A + c A^2) X subtracts terms of size about 3 near sigma = 1, and each
    NVFP4 product carries about 13% relative error."""
    g = np.random.default_rng(0).standard_normal((256, 512)).astype(np.float32)
    sv_exact = np.linalg.svd(exact_chain(g, 5), compute_uv=False)
    assert 0.6 < sv_exact.min() and sv_exact.max() < 1.2
    sv_q = np.linalg.svd(oracle.newton_schulz(g, iters=5).astype(np.float64), compute_uv=False)
    assert sv_q.max() > 100.0, sv_q.max()
