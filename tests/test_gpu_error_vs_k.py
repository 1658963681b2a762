"""The error-versus-K analysis (bench.py --error-vs-k) against the oracle: the
GPU's relative error of the NVFP4 GEMM equals the one computed from the oracle's
quantization and binary64 product, for every quantization mode, on Gaussian and
outlier-heavy operands; and the quantized operands behind it are bit-exact."""
import numpy as np
import pytest
import torch

import bench
import workloads
from parity import assert_q_equal, check_gemm, host_q

pytestmark = pytest.mark.gpu

ORACLE_KW = {0: {}, "rht": {"rht": True}, "sr": {"sr": True}, "rht_sr": {"rht": True, "sr": True},
             "rht64": {"rht64": True}, "rht64_sr": {"rht64": True, "sr": True}, "eden": {"rht64": True, "eden": True}}


@pytest.mark.parametrize("K", [256, 2048])
@pytest.mark.parametrize("outliers", [False, True], ids=["gaussian", "outliers"])
@pytest.mark.parametrize("mode", list(bench.ERROR_MODES))
def test_error_matches_oracle(fp4, oracle, K, outliers, mode):
    M, N = 64, 48
    a, b, signs = workloads.error_operands(M, N, K, seed=K + outliers, outliers=outliers)
    err_gpu, c_gpu = bench.quantized_gemm_error(fp4, a.cuda(), b.cuda(), mode, signs)
    af, bf = workloads.widen(a), workloads.widen(b)
    fa, fb = bench.ERROR_MODES[mode]
    oa = oracle.quantize(af, signs=signs, seed=0, offset=1, **ORACLE_KW[fa])
    ob = oracle.quantize(bf, signs=signs, seed=0, offset=1, **ORACLE_KW[fb])
    # the operands the GPU quantized, bit for bit
    ga, gb = fp4.QTensor(M, K), fp4.QTensor(N, K)
    fp4.fp4_quantize(a.cuda(), bench.mode_flag(fp4, fa), signs, 0, 1, ga)
    fp4.fp4_quantize(b.cuda(), bench.mode_flag(fp4, fb), signs, 0, 1, gb)
    assert_q_equal(host_q(ga), oa, f"A {mode}")
    assert_q_equal(host_q(gb), ob, f"B {mode}")
    y_ref, bound = oracle.gemm_ref(oa, ob)
    c = c_gpu.cpu().numpy().astype(np.float64)
    check_gemm(c, y_ref, bound, False, f"error-vs-K GEMM {mode}")
    exact = af.astype(np.float64) @ bf.astype(np.float64).T
    err_ora = np.linalg.norm(y_ref - exact) / np.linalg.norm(exact)
    # the two errors differ by at most the GEMM tolerance's share of ||exact||
    slack = 1e-5 * np.linalg.norm(bound) / np.linalg.norm(exact)
    assert abs(err_gpu - err_ora) <= slack + 1e-12, (err_gpu, err_ora, slack)
    assert 1e-3 < err_ora < 0.5  # a quantization error, neither zero nor garbage


def test_error_flat_in_k_and_sr_costs_variance(fp4):
    """Properties the analysis must show on its own data: with independent
    rounding errors the error and the product both grow like sqrt(K), so the
    relative error stays flat from K = 256 to 8192; stochastic rounding, unbiased
    but of larger variance, costs more than nearest-even."""
    M = N = 128
    e = {}
    for K in (256, 8192):
        a, b, signs = workloads.error_operands(M, N, K, seed=K, outliers=False)
        a, b = a.cuda(), b.cuda()
        e[K] = {m: bench.quantized_gemm_error(fp4, a, b, m, signs)[0] for m in ("rne", "sr")}
    for m in ("rne", "sr"):
        assert 0.8 < e[8192][m] / e[256][m] < 1.25, e
    assert e[256]["sr"] > e[256]["rne"] and e[8192]["sr"] > e[8192]["rne"]


def sylvester(n):
    m = np.array([[1.0]])
    while m.shape[0] < n:
        m = np.block([[m, m], [m, -m]])
    return m


def oracle_estimate(oracle, af, mode, signs, seed, offset):
    """A's estimate in A's coordinates from the oracle: its dequantization, rotated
    back in binary64 (the 16-point transform per 16-block, the 64-point per group)."""
    kw = {"rne": {}, "sr": {"sr": True}, "rht_sr": {"rht": True, "sr": True}, "rht64_sr": {"rht64": True, "sr": True},
          "eden": {"rht64": True, "eden": True}}[mode]
    deq = oracle.dequantize(oracle.quantize(af, signs=signs, seed=seed, offset=offset, **kw))
    M, K = af.shape
    if mode in ("rne", "sr"):
        return deq
    n = 16 if mode == "rht_sr" else 64
    H = sylvester(n) / np.sqrt(n)
    out = np.empty_like(deq)
    for j in range(K // n):
        if n == 16:
            d = np.array([-1.0 if (signs >> t) & 1 else 1.0 for t in range(16)])
        else:
            w = oracle.rht64_signs(j, signs)
            d = np.array([-1.0 if (w[t >> 5] >> (t & 31)) & 1 else 1.0 for t in range(64)])
        out[:, n * j:n * j + n] = (deq[:, n * j:n * j + n] @ H.T) * d
    return out


@pytest.mark.parametrize("mode", ["rne", "sr", "rht_sr", "rht64_sr", "eden"])
def test_quantizer_estimate_through_the_identity_matches_oracle(fp4, oracle, mode):
    """The quantizer-error analysis reads A's estimate back through a GEMM with the
    identity quantized in A's rotation; that estimate equals the oracle's
    dequantization rotated back in binary64, within the GEMM tolerance."""
    M, K = 32, 512
    a = workloads.random_matrix((M, K), seed=9, kind="laplace", std=1e-3)
    signs = 0x1F2E3D4C & (0xFFFF if mode == "rht_sr" else 0xFFFFFFFF)
    ident = bench.identity_operand(fp4, K, mode, signs)
    c = bench.quantizer_estimate(fp4, a.cuda(), mode, signs, ident, seed=2, offset=1).double().cpu().numpy()
    est = oracle_estimate(oracle, workloads.widen(a), mode, signs, 2, 1)
    # every product is exact; the fp32 sums over K add at most K ulps of the largest term
    tol = 2.0 ** -22 * K * np.abs(est).max()
    assert np.abs(c - est).max() <= tol
    rel = float(((est - workloads.widen(a)) ** 2).sum() / (workloads.widen(a).astype(np.float64) ** 2).sum())
    assert 1e-3 < rel < 0.05, rel


def test_eden_bias_at_the_noise_floor_on_the_gpu(fp4):
    """The GPU's own demonstration (bench.py --error-vs-k, smaller): over 2048
    rotation keys the mean MS-EDEN estimate sits at the noise floor, while the same
    rotation without the correction does not."""
    r = bench.eden_bias(fp4, M=32, K=2048, draws=2048)
    assert r["modes"]["eden"]["ratio"] < 1.3, r
    assert r["modes"]["rht64"]["ratio"] > 1.8, r
