"""GPU parity of the 64-point random Hadamard transform and MS-EDEN (Quartet II
page, paragraph 1, MS-EDEN sentence) against the oracle, through the C ABI:
codes, scales and the stored tensor amax bit for bit, rowwise and columnwise, with
nearest-even, stochastic rounding and MS-EDEN, in bf16 and fp32, at ragged sizes,
at the 12B MLP's dY size on sampled rows, and in a weight-gradient GEMM whose
operands are MS-EDEN dY^T and 64-point-rotated X^T."""
import numpy as np
import pytest
import torch

import workloads
from parity import assert_q_equal, check_gemm, dev, host_q

pytestmark = pytest.mark.gpu

KEY = 0x9E3779B9


def mode_flags(fp4, mode):
    return {"rne": fp4.Q_RHT64, "sr": fp4.Q_RHT64 | fp4.Q_SR, "eden": fp4.Q_RHT64 | fp4.Q_EDEN}[mode]


def oracle_kw(mode):
    return dict(rht64=True, sr=mode == "sr", eden=mode == "eden")


CASES = [((64, 192), False), ((48, 1024), False), ((1000, 320), False), ((192, 272), True), ((320, 1000), True),
         ((2048, 2048), True), ((4096, 768), False)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("mode", ["rne", "sr", "eden"])
@pytest.mark.parametrize("shape,colwise", CASES, ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else
                         ("cols" if v else "rows"))
def test_rht64_quantize_matches_oracle(fp4, oracle, shape, colwise, mode, dtype):
    R, C = shape
    x_cpu = workloads.random_matrix(shape, seed=R * 7 + C, kind="laplace" if mode != "rne" else "normal",
                                    std=1e-3 if mode != "rne" else 1.0, dtype=dtype)
    x = dev(x_cpu)
    lrows, lcols = (C, R) if colwise else (R, C)
    q = fp4.QTensor(lrows, lcols)
    flags = mode_flags(fp4, mode) | (fp4.Q_COLWISE if colwise else 0)
    fp4.fp4_quantize(x, flags, KEY, 11, 3, q)
    o = oracle.quantize(workloads.widen(x_cpu), colwise=colwise, signs=KEY, seed=11, offset=3, **oracle_kw(mode))
    assert_q_equal(host_q(q), o, f"{mode} {'cols' if colwise else 'rows'} {shape}")


@pytest.mark.parametrize("colwise", [False, True], ids=["rows", "cols"])
def test_rht64_amax_both_forms(fp4, oracle, colwise):
    """fp4_amax (atomic form) and the quantizer's amax pass (partial maxima) give the
    oracle's amax after the 64-point transform; with MS-EDEN the stored amax is
    RN(7/4 amax), also for a tensor small enough to take the atomic form."""
    for shape in ((128, 256), (64, 64), (1024, 2048)):
        x_cpu = workloads.random_matrix(shape, seed=shape[0], kind="outliers")
        x = dev(x_cpu)
        xf = workloads.widen(x_cpu)
        want = oracle.amax(xf, colwise=colwise, rht64=True, signs=KEY)
        a = torch.zeros(1, dtype=torch.float32, device="cuda")
        fp4.fp4_amax(x, fp4.Q_RHT64 | (fp4.Q_COLWISE if colwise else 0), KEY, a)
        torch.cuda.synchronize()
        assert float(a.cpu()[0]) == want
        lr, lc = (shape[1], shape[0]) if colwise else shape
        q = fp4.QTensor(lr, lc)
        fp4.fp4_quantize(x, fp4.Q_RHT64 | fp4.Q_EDEN | (fp4.Q_COLWISE if colwise else 0), KEY, 1, 1, q)
        torch.cuda.synchronize()
        assert float(q.amax.cpu()[0]) == float(np.float32(1.75) * np.float32(want))


def test_eden_amax_given_and_zero_tensor(fp4, oracle):
    x_cpu = workloads.random_matrix((256, 512), seed=5, kind="laplace", std=1e-3)
    x = dev(x_cpu)
    o = oracle.quantize(workloads.widen(x_cpu), signs=KEY, seed=2, offset=9, rht64=True, eden=True)
    q = fp4.QTensor(256, 512)
    q.amax.fill_(o.amax)
    fp4.fp4_quantize(x, fp4.Q_RHT64 | fp4.Q_EDEN | fp4.Q_AMAX_GIVEN, KEY, 2, 9, q)
    assert_q_equal(host_q(q), o, "amax given")
    z = torch.zeros(64, 128, dtype=torch.bfloat16, device="cuda")
    qz = fp4.QTensor(128, 64)
    fp4.fp4_quantize(z, fp4.Q_RHT64 | fp4.Q_EDEN | fp4.Q_COLWISE, KEY, 0, 0, qz)
    codes, scales, amax = host_q(qz)
    assert amax == 0.0 and not codes.any() and not scales.any()


def test_rht64_rejects_bad_shapes(fp4):
    x = torch.zeros(64, 96, dtype=torch.bfloat16, device="cuda")
    q = fp4.QTensor(64, 96)
    with pytest.raises(fp4.Fp4Error, match="SHAPE"):
        fp4.fp4_quantize(x, fp4.Q_RHT64, KEY, 0, 0, q)  # 96 is not a multiple of 64
    with pytest.raises(fp4.Fp4Error, match="MODE"):
        fp4.fp4_quantize(dev(torch.zeros(64, 128)), fp4.Q_EDEN, KEY, 0, 0, fp4.QTensor(64, 128))
    with pytest.raises(fp4.Fp4Error, match="MODE"):
        fp4.fp4_quantize(dev(torch.zeros(64, 128)), fp4.Q_RHT64 | fp4.Q_RHT, KEY, 0, 0, fp4.QTensor(64, 128))


def test_eden_full_size_dy_sampled_rows(fp4, oracle):
    """dY^T of the 12B MLP (dY 16384 x 20480, bf16 Laplace(0, 1e-3)) quantized with
    MS-EDEN columnwise, in the launch configuration of the bench's breakdown: the
    stored amax in full, and 48 sampled logical rows bit for bit."""
    M, N = 16384, 20480
    rng = np.random.default_rng(0)
    dy_cpu = workloads.to_bf16(workloads.laplace(rng, (M, N)))
    dy = dev(dy_cpu)
    q = fp4.QTensor(N, M)
    fp4.fp4_quantize(dy, fp4.Q_RHT64 | fp4.Q_EDEN | fp4.Q_COLWISE, KEY, 0, 2, q)
    codes, scales, amax = host_q(q)
    dyf = workloads.widen(dy_cpu)
    vmax = oracle.amax(dyf, colwise=True, rht64=True, signs=KEY)
    assert amax == float(np.float32(1.75) * np.float32(vmax))
    rows = np.sort(rng.choice(N, 48, replace=False))
    for r in rows:
        o = oracle.quantize(dyf, colwise=True, rht64=True, eden=True, signs=KEY, seed=0, offset=2, amax_in=amax,
                            rows=(int(r), int(r) + 1))
        assert np.array_equal(codes[r], o.codes[0]) and np.array_equal(scales[r], o.scales[0]), int(r)


@pytest.mark.parametrize("tokens", [1024, 4096])
def test_eden_wgrad_gemm(fp4, oracle, tokens):
    """dW = dY^T . X with dY^T quantized by MS-EDEN and X^T by the same 64-point
    rotation with nearest-even: operands bit-exact, dW within the GEMM tolerance of
    the binary64 product of the oracle's operands."""
    N, K = 384, 256
    inp = workloads.make_linear_inputs(workloads.Linear("w", tokens, N, K), seed=tokens)
    dy, x = dev(inp.dy), dev(inp.x)
    qd, qx = fp4.QTensor(N, tokens), fp4.QTensor(K, tokens)
    fp4.fp4_quantize(dy, fp4.Q_RHT64 | fp4.Q_EDEN | fp4.Q_COLWISE, KEY, 0, 2, qd)
    fp4.fp4_quantize(x, fp4.Q_RHT64 | fp4.Q_COLWISE, KEY, 0, 0, qx)
    dw = torch.empty(N, K, dtype=torch.float32, device="cuda")
    fp4.fp4_gemm(qd, qx, dw)
    dyf, xf = workloads.widen(inp.dy), workloads.widen(inp.x)
    od = oracle.quantize(dyf, colwise=True, rht64=True, eden=True, signs=KEY, seed=0, offset=2)
    ox = oracle.quantize(xf, colwise=True, rht64=True, signs=KEY)
    assert_q_equal(host_q(qd), od, "dY^T eden")
    assert_q_equal(host_q(qx), ox, "X^T rht64")
    ref, bound = oracle.gemm_ref(od, ox)
    check_gemm(dw.cpu().numpy(), ref, bound, False, "eden wgrad")
    # the rotation cancels in the product: the NVFP4 result stays close to the exact dW
    exact = dyf.astype(np.float64).T @ xf.astype(np.float64)
    rel = np.linalg.norm(dw.cpu().numpy() - exact) / np.linalg.norm(exact)
    assert rel < 0.2, rel


@pytest.mark.parametrize("mode", ["rne", "eden"])
def test_rht64_columns_with_a_row_stride_beyond_the_4_column_kernel(fp4, oracle, mode):
    """64 rows that span 2^31 bytes are beyond the 4-column kernel's 32-bit row
    offsets: the columnwise 64-point quantization takes the 8-column kernel and gives
    the oracle's bits (a 2 GiB strided bf16 view, 64 x 256)."""
    R, C = 64, 256
    ld = (1 << 31) // (64 * 2)
    x_cpu = workloads.random_matrix((R, C), seed=64, kind="laplace", std=1e-3)
    full = torch.empty((R, ld), dtype=torch.bfloat16, device="cuda")
    x = full[:, :C]
    x.copy_(x_cpu.to("cuda"))
    assert x.stride(0) == ld
    q = fp4.QTensor(C, R)
    fp4.fp4_quantize(x, mode_flags(fp4, mode) | fp4.Q_COLWISE, KEY, 4, 6, q)
    o = oracle.quantize(workloads.widen(x_cpu), colwise=True, signs=KEY, seed=4, offset=6, **oracle_kw(mode))
    assert_q_equal(host_q(q), o, f"wide-stride rht64 cols {mode}")
    del full, x
    torch.cuda.empty_cache()
