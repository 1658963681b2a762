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

ORACLE_KW = {0: {}, "rht": {"rht": True}, "sr": {"sr": True}, "rht_sr": {"rht": True, "sr": True}}


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
    flag = {0: 0, "rht": fp4.Q_RHT, "sr": fp4.Q_SR, "rht_sr": fp4.Q_RHT | fp4.Q_SR}
    fp4.fp4_quantize(a.cuda(), flag[fa], signs, 0, 1, ga)
    fp4.fp4_quantize(b.cuda(), flag[fb], signs, 0, 1, gb)
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
