"""GPU parity of fp4_gemm: operands quantized by the oracle are uploaded, the GPU
GEMM runs through the C ABI, and every output is checked against the binary64
product of the oracle's dequantized operands within 1e-5 * sum|a b|."""
import numpy as np
import pytest
import torch

import workloads
from parity import check_gemm, upload_q

pytestmark = pytest.mark.gpu


def oracle_operands(oracle, M, N, K, seed, a2d=False, b2d=False, a_kind="normal", b_std=0.02):
    rng = np.random.default_rng(seed)
    if a_kind == "laplace":
        xa = workloads.laplace(rng, (M, K))
    else:
        xa = workloads.normal(rng, (M, K), outlier_frac=0.001 if a_kind == "outliers" else 0.0)
    xb = workloads.normal(rng, (N, K), std=b_std)
    return oracle.quantize(xa, two_d=a2d), oracle.quantize(xb, two_d=b2d)


def run_gemm(fp4, oracle, qa, qb, out_dtype):
    a, b = upload_q(fp4, qa), upload_q(fp4, qb)
    c = torch.full((qa.rows, qb.rows), float("nan"), dtype=out_dtype, device="cuda")
    fp4.fp4_gemm(a, b, c)
    torch.cuda.synchronize()
    return c.float().cpu().numpy()


CASES = [
    # (M, N, K, a2d, b2d): tile multiples, ragged M/N, K % 128 != 0, K % 32 == 16
    (256, 256, 256, False, False),
    (300, 200, 272, False, False),
    (512, 384, 1040, False, True),
    (129, 256, 4096, False, True),
    (129, 257, 4096, False, False),
    (1024, 1024, 4096, True, True),
    (64, 16, 16, False, False),
    # main path with ragged edges (rows/columns past M, N read as zeros, not stored)
    (300, 272, 512, False, True),
    (300, 260, 512, False, False),
    # bf16 output stores two neighbouring 32-column blocks together: N = 300 leaves the
    # second block of a pair with one whole and one half 8-column chunk inside C,
    # N = 288 the second block wholly outside
    (260, 300, 768, False, False),
    (96, 288, 256, False, True),
    # more 256x256 tiles than CUs: persistent loop; 17x16 = 272 tiles, 17x17 = 289
    # (an XCD split that is not even), ragged in both dimensions; on a 256-CU GPU
    # the tiles past the first 256 run as 128x128 quarters in a second launch
    # (64 and 132 quarters, one per workgroup; the ragged case has quarters wholly
    # past the edge)
    (4352, 4096, 256, False, True),
    (4100, 4100, 256, False, False),
    # 89x4 = 356 tiles: 100 past one round, 400 quarters, more than one per CU
    (22784, 1000, 256, False, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:3])) + ("_a2d" if c[3] else "") +
                         ("_b2d" if c[4] else ""))
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_gemm_parity(fp4, oracle, case, out_dtype):
    M, N, K, a2d, b2d = case
    qa, qb = oracle_operands(oracle, M, N, K, seed=M + N + K, a2d=a2d, b2d=b2d, a_kind="outliers")
    y = run_gemm(fp4, oracle, qa, qb, out_dtype)
    y_ref, bound = oracle.gemm_ref(qa, qb)
    check_gemm(y, y_ref, bound, out_dtype == torch.bfloat16, f"gemm {case}")


def test_tiny_config(fp4, oracle):
    """X, W 256x256 fp32 N(0,1) seed 0, both 1D nearest-even on the GPU (bit-exact
    against the oracle), Y = X . W^T in fp32."""
    from parity import assert_q_equal, dev, host_q
    x, w = workloads.make_tiny(0)
    qx, qw = fp4.QTensor(256, 256), fp4.QTensor(256, 256)
    fp4.fp4_quantize(dev(x), 0, 0, 0, 0, qx)
    fp4.fp4_quantize(dev(w), 0, 0, 0, 0, qw)
    y = torch.empty(256, 256, dtype=torch.float32, device="cuda")
    fp4.fp4_gemm(qx, qw, y)
    ox, ow = oracle.quantize(x.numpy()), oracle.quantize(w.numpy())
    assert_q_equal(host_q(qx), ox, "tiny X")
    assert_q_equal(host_q(qw), ow, "tiny W")
    y_ref, bound = oracle.gemm_ref(ox, ow)
    check_gemm(y.cpu().numpy(), y_ref, bound, False, "tiny")


def test_one_hot_and_exact_products(fp4, oracle):
    """K = 16, one block, A rows one-hot: the accumulator holds one exact product,
    so the only roundings are the epilogue's two (gA*gB, then acc*g): within 2 ulp."""
    xb = np.random.default_rng(4).standard_normal((48, 16)).astype(np.float32)
    xa = np.zeros((32, 16), dtype=np.float32)
    for m in range(32):
        xa[m, m % 16] = 6.0
    qa, qb = oracle.quantize(xa), oracle.quantize(xb)
    y = run_gemm(fp4, oracle, qa, qb, torch.float32)
    y_ref, _ = oracle.gemm_ref(qa, qb)
    assert np.all(np.abs(y - y_ref) <= 2.0**-22 * np.abs(y_ref))


def test_zero_k_and_zero_operands(fp4, oracle):
    qa, qb = oracle_operands(oracle, 64, 80, 128, seed=1)
    qa.codes[:] = 0
    y = run_gemm(fp4, oracle, qa, qb, torch.float32)
    assert np.all(y == 0.0)
    # K = 0: an empty sum
    a, b = fp4.QTensor(32, 0), fp4.QTensor(48, 0)
    c = torch.full((32, 48), 7.0, device="cuda")
    fp4.fp4_gemm(a, b, c)
    torch.cuda.synchronize()
    assert torch.all(c == 0)
    # M = 0: nothing to do
    e = fp4.QTensor(0, 64)
    c2 = torch.empty(0, 48, device="cuda")
    fp4.fp4_gemm(e, fp4.QTensor(48, 64), c2)


@pytest.mark.parametrize("ldc", [260, 264])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_row_stride_of_c(fp4, oracle, ldc, out_dtype):
    """C with a row stride beyond N on a main-path shape: rows of 260 bf16 are not
    16-byte multiples (the edge kernel takes that case), 264 are; the columns past
    N keep their contents."""
    M, N, K = 300, 256, 512
    qa, qb = oracle_operands(oracle, M, N, K, seed=5)
    a, b = upload_q(fp4, qa), upload_q(fp4, qb)
    big = torch.full((M, ldc), -1.0, dtype=out_dtype, device="cuda")
    from nvfp4_bit_microscaled_amd import load
    dt = 1 if out_dtype == torch.float32 else 0
    assert load().fp4_gemm(a.desc, b.desc, big.data_ptr(), dt, ldc, None) == 0
    torch.cuda.synchronize()
    y = big.float().cpu().numpy()
    assert np.all(y[:, N:] == -1.0)
    y_ref, bound = oracle.gemm_ref(qa, qb)
    check_gemm(y[:, :N], y_ref, bound, out_dtype == torch.bfloat16, f"ldc {ldc}")


def test_ldc_larger_than_n(fp4, oracle):
    qa, qb = oracle_operands(oracle, 100, 60, 256, seed=2)
    a, b = upload_q(fp4, qa), upload_q(fp4, qb)
    big = torch.full((100, 96), -1.0, device="cuda")
    c = big[:, :60]
    from nvfp4_bit_microscaled_amd import load
    st = load().fp4_gemm(a.desc, b.desc, c.data_ptr(), 1, 96, None)
    assert st == 0
    torch.cuda.synchronize()
    y = big.cpu().numpy()
    assert np.all(y[:, 60:] == -1.0)
    y_ref, bound = oracle.gemm_ref(qa, qb)
    check_gemm(y[:, :60], y_ref, bound, False, "ldc")


STREAMK_CASES = [
    # (M, N, K, a2d, sampled rows or None, stream-K tiles, tiles before them):
    (2560, 2560, 16384, False, None, 100, 0),     # 100 tiles, runs of 25 stages (some 1- and 2-stage segments)
    (384, 4224, 16384, True, None, 34, 0),        # ragged rows, 2D-scaled A
    (4224, 5760, 8192, False, 96, 135, 256),      # one whole round, then 135 tiles as stream-K
]


@pytest.mark.parametrize("case", STREAMK_CASES, ids=lambda c: "x".join(map(str, c[:3])))
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_gemm_stream_k(fp4, oracle, case, out_dtype):
    """fp4_gemm_ws with a stream-K plan: 256 workgroups each take an equal run of
    the stream-K tiles' stages, store the tiles they hold whole, and leave the rest
    as raw segments that a reduction sums in order.  Against the oracle within the
    GEMM tolerance (all rows, or sampled ones at the largest shape), twice on one
    workspace, and unsplit with too small a workspace."""
    M, N, K, a2d, nrows, sk_tiles, first = case
    need = fp4.fp4_gemm_ws_bytes(M, N, K)
    assert need == (256 + sk_tiles) * 256 * 256 * 4, need
    assert ((M + 255) // 256) * ((N + 255) // 256) == first + sk_tiles
    qa, qb = oracle_operands(oracle, M, N, K, seed=M + 2 * N + K, a2d=a2d, a_kind="laplace")
    a, b = upload_q(fp4, qa), upload_q(fp4, qb)
    rows = np.arange(M) if nrows is None else np.sort(np.random.default_rng(M).choice(M, nrows, replace=False))
    if nrows is not None:
        rows = np.union1d(rows, [0, M - 1])  # the first and last tile rows too
    qa_rows = oracle.QTensor(qa.codes[rows], qa.scales[rows // 16] if a2d else qa.scales[rows], qa.amax,
                             len(rows), qa.K, False)
    y_ref, bound = oracle.gemm_ref(qa_rows, qb)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        c = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
        fp4.fp4_gemm_ws(a, b, c, ws)
        torch.cuda.synchronize()
        check_gemm(c.float().cpu().numpy()[rows], y_ref, bound, out_dtype == torch.bfloat16,
                   f"stream-K {case} rep {rep}")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    c = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
    fp4.fp4_gemm_ws(a, b, c, small)
    torch.cuda.synchronize()
    check_gemm(c.float().cpu().numpy()[rows], y_ref, bound, out_dtype == torch.bfloat16, f"small workspace {case}")


SPLITK_CASES = [
    # (M, N, K, a2d, b2d, split tiles, splits): every tile split (few tiles, long K), or
    # only the tiles past the whole rounds of a 256-CU GPU (in place of quarters)
    (512, 512, 8192, False, True, 4, 8),      # 4 tiles, 8 splits of 1024
    (300, 200, 4096, False, False, 2, 4),     # ragged edges (rows/columns past M, N), 2 tiles
    (1024, 256, 16384, True, False, 4, 16),   # 4 tiles, 16 splits of 1024, 2D-scaled A
    (4352, 4096, 4096, False, True, 16, 4),   # 272 tiles: 256 whole, the last 16 split in 4
    (4100, 4100, 8192, False, False, 33, 4),  # 289 tiles, ragged: the last 33 split in 4
    (256, 256, 256, False, False, 0, 1),      # no split: the plain path
]


@pytest.mark.parametrize("case", SPLITK_CASES, ids=lambda c: "x".join(map(str, c[:3])) + f"_{c[5]}x{c[6]}")
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_gemm_split_k(fp4, oracle, case, out_dtype):
    """fp4_gemm_ws: the split plan for the shape, partial tiles in the caller's
    workspace, their sum against the oracle within the GEMM tolerance; run twice
    on one workspace (the second call overwrites the first's partials), and once
    with too small a workspace (the unsplit path)."""
    M, N, K, a2d, b2d, split_tiles, splits = case
    need = fp4.fp4_gemm_ws_bytes(M, N, K)
    assert need == split_tiles * splits * 256 * 256 * 4, need
    qa, qb = oracle_operands(oracle, M, N, K, seed=M + N + K, a2d=a2d, b2d=b2d, a_kind="laplace")
    a, b = upload_q(fp4, qa), upload_q(fp4, qb)
    ws = torch.full((max(need, 16),), 0xFF, dtype=torch.uint8, device="cuda")
    y_ref, bound = oracle.gemm_ref(qa, qb)
    for rep in range(2):
        c = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
        fp4.fp4_gemm_ws(a, b, c, ws)
        torch.cuda.synchronize()
        check_gemm(c.float().cpu().numpy(), y_ref, bound, out_dtype == torch.bfloat16, f"split-K {case} rep {rep}")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    c = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
    fp4.fp4_gemm_ws(a, b, c, small)
    torch.cuda.synchronize()
    check_gemm(c.float().cpu().numpy(), y_ref, bound, out_dtype == torch.bfloat16, f"small workspace {case}")


def random_shapes(n=16, seed=20261203, max_work=2e10):
    """Seeded (M, N, K, a2d, b2d) drawn across the paths: M, N from 1 to 4600 (each a
    multiple of 16 half the time, which 2D scales need), K a multiple of 256 (the main
    path) or of 16 (the edge kernel when K % 256 != 0) up to 8192, 2D scales on half
    of the operands whose rows allow them; shapes whose M N K exceeds max_work are
    drawn again (the binary64 reference stays within seconds)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M, N = (int(v) if rng.random() < 0.5 else 16 * max(1, int(v) // 16) for v in rng.integers(1, 4600, size=2))
        K = 256 * int(rng.integers(1, 33)) if rng.random() < 0.5 else 16 * int(rng.integers(1, 513))
        if float(M) * N * K > max_work:
            continue
        out.append((M, N, K, bool(M % 16 == 0 and rng.random() < 0.5), bool(N % 16 == 0 and rng.random() < 0.5)))
    return out


@pytest.mark.parametrize("case", random_shapes(), ids=lambda c: "x".join(map(str, c[:3])))
def test_gemm_random_shapes(fp4, oracle, case):
    """fp4_gemm and fp4_gemm_ws (with the workspace its plan asks for) on seeded random
    shapes, fp32 and bf16 outputs, against the oracle within the GEMM tolerance."""
    M, N, K, a2d, b2d = case
    qa, qb = oracle_operands(oracle, M, N, K, seed=M * 7 + N * 3 + K, a2d=a2d, b2d=b2d, a_kind="normal")
    a, b = upload_q(fp4, qa), upload_q(fp4, qb)
    y_ref, bound = oracle.gemm_ref(qa, qb)
    ws = torch.empty(max(fp4.fp4_gemm_ws_bytes(M, N, K), 16), dtype=torch.uint8, device="cuda")
    for out_dtype in (torch.float32, torch.bfloat16):
        for with_ws in (False, True):
            c = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
            if with_ws:
                fp4.fp4_gemm_ws(a, b, c, ws)
            else:
                fp4.fp4_gemm(a, b, c)
            torch.cuda.synchronize()
            check_gemm(c.float().cpu().numpy(), y_ref, bound, out_dtype == torch.bfloat16,
                       f"random {case} {out_dtype} ws={with_ws}")
