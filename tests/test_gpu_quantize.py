"""GPU parity of the quantizer: fp4_amax / fp4_quantize through the C ABI against
the oracle on the same seeded inputs, bit for bit (codes, E4M3 scales, amax)."""
import numpy as np
import pytest
import torch

import workloads
from parity import assert_q_equal, dev, host_q

pytestmark = pytest.mark.gpu


def make_x(shape, seed, kind="normal", std=1.0, dtype=torch.bfloat16):
    return workloads.random_matrix(shape, seed, kind=kind, std=std, dtype=dtype)


def run_case(fp4, oracle, x_cpu, flags, signs=0, seed=0, offset=0, with_t=True):
    colwise = bool(flags & fp4.Q_COLWISE)
    two_d = bool(flags & fp4.Q_2D)
    R, C = x_cpu.shape
    lrows, lcols = (C, R) if colwise else (R, C)
    x = dev(x_cpu)
    q = fp4.QTensor(lrows, lcols, two_d)
    q_t = fp4.QTensor(lcols, lrows, True) if two_d and with_t else None
    fp4.fp4_quantize(x, flags, signs, seed, offset, q, q_t)
    xf = workloads.widen(x_cpu)
    ora = oracle.quantize(xf, two_d=two_d, colwise=colwise, rht=bool(flags & fp4.Q_RHT), sr=bool(flags & fp4.Q_SR),
                          signs=signs, seed=seed, offset=offset)
    assert_q_equal(host_q(q), ora, f"flags={flags} shape={tuple(x_cpu.shape)}")
    if q_t is not None:
        ora_t = oracle.quantize(xf, two_d=True, colwise=not colwise)
        assert_q_equal(host_q(q_t), ora_t, f"transposed flags={flags} shape={tuple(x_cpu.shape)}")
    return q


ROW_SHAPES = [(1, 16), (333, 272), (64, 4096), (257, 1040)]
# 2048x2048: 8 column tiles x 8 slab groups, every tile whole
COL_SHAPES = [(16, 8), (784, 1000), (4096, 64), (272, 520), (2048, 2048)]
TILE_SHAPES = [(16, 16), (272, 400), (1024, 4096), (48, 2064)]


@pytest.mark.parametrize("shape", ROW_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("mode", ["rne", "sr", "rht", "rht_sr"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_rowwise(fp4, oracle, shape, mode, dtype):
    flags = {"rne": 0, "sr": fp4.Q_SR, "rht": fp4.Q_RHT, "rht_sr": fp4.Q_RHT | fp4.Q_SR}[mode]
    x = make_x(shape, seed=shape[0] * 7 + shape[1], dtype=dtype)
    run_case(fp4, oracle, x, flags, signs=0xA5C3, seed=0x1234_5678_9ABC_DEF0, offset=3)


@pytest.mark.parametrize("shape", COL_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("mode", ["rne", "sr", "rht", "rht_sr"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_colwise(fp4, oracle, shape, mode, dtype):
    flags = fp4.Q_COLWISE | {"rne": 0, "sr": fp4.Q_SR, "rht": fp4.Q_RHT, "rht_sr": fp4.Q_RHT | fp4.Q_SR}[mode]
    x = make_x(shape, seed=shape[0] * 3 + shape[1], kind="laplace", std=1e-3, dtype=dtype)
    run_case(fp4, oracle, x, flags, signs=0x5A3C, seed=7, offset=2)


@pytest.mark.parametrize("shape", TILE_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
@pytest.mark.parametrize("colwise", [False, True], ids=["direct", "colwise"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_two_d(fp4, oracle, shape, colwise, dtype):
    flags = fp4.Q_2D | (fp4.Q_COLWISE if colwise else 0)
    x = make_x(shape, seed=shape[0] + shape[1], std=0.02, dtype=dtype)
    run_case(fp4, oracle, x, flags)


@pytest.mark.parametrize("colwise", [False, True], ids=["direct", "colwise"])
def test_two_d_single_layout(fp4, oracle, colwise):
    """2D without the second layout: the kernel writes only the direct codes, or
    (COLWISE) only the transposed ones; ragged against its 256x256 blocks."""
    x = make_x((272, 528), seed=11, std=0.02)
    run_case(fp4, oracle, x, fp4.Q_2D | (fp4.Q_COLWISE if colwise else 0), with_t=False)


@pytest.mark.parametrize("flags_name", ["plain", "rht_rows", "rht_cols"])
def test_amax(fp4, oracle, flags_name):
    flags = {"plain": 0, "rht_rows": fp4.Q_RHT, "rht_cols": fp4.Q_RHT | fp4.Q_COLWISE}[flags_name]
    x_cpu = make_x((1008, 2064), seed=5, kind="outliers")
    out = torch.zeros(1, dtype=torch.float32, device="cuda")
    fp4.fp4_amax(dev(x_cpu), flags, 0x1357, out)
    got = float(out.cpu()[0])
    want = oracle.amax(workloads.widen(x_cpu), colwise=bool(flags & fp4.Q_COLWISE), rht=bool(flags & fp4.Q_RHT),
                       signs=0x1357)
    assert got == want


def test_amax_given_skips_the_pass(fp4, oracle):
    """With FP4_Q_AMAX_GIVEN the caller's amax is used as is (here: twice the true amax)."""
    x_cpu = make_x((128, 256), seed=9)
    xf = workloads.widen(x_cpu)
    a = 2.0 * oracle.amax(xf)
    q = fp4.QTensor(128, 256)
    q.amax.fill_(a)
    fp4.fp4_quantize(dev(x_cpu), fp4.Q_AMAX_GIVEN, 0, 0, 0, q)
    assert_q_equal(host_q(q), oracle.quantize(xf, amax_in=a), "amax given")


def test_zero_input(fp4, oracle):
    x_cpu = torch.zeros(64, 256, dtype=torch.bfloat16)
    for flags in (0, fp4.Q_SR, fp4.Q_COLWISE | fp4.Q_RHT | fp4.Q_SR, fp4.Q_2D):
        run_case(fp4, oracle, x_cpu, flags, signs=0xFFFF, seed=1, offset=1)


def test_scale_underflow_and_saturation(fp4, oracle):
    """Rows spanning 40 binades: blocks whose scale underflows to 0 (all codes 0),
    subnormal E4M3 scales, and the saturating tensor maximum."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((96, 512)).astype(np.float32)
    x *= np.exp2(rng.uniform(-30, 10, (96, 32))).repeat(16, axis=1).astype(np.float32)
    x[5, 7] = 3.0e4
    x_cpu = torch.from_numpy(x)
    qs = [run_case(fp4, oracle, x_cpu, flags, signs=0x0F0F, seed=2, offset=5)
          for flags in (0, fp4.Q_SR, fp4.Q_RHT, fp4.Q_COLWISE | fp4.Q_RHT | fp4.Q_SR)]
    codes, scales, _ = host_q(qs[0])  # the rowwise case holds both kinds of small block
    assert (scales == 0).any() and ((scales > 0) & (scales < 8)).any()


@pytest.mark.parametrize("top", [-110, -121], ids=["tiny", "scale_clamped"])
def test_tiny_and_subnormal_blocks(fp4, oracle, top):
    """fp32 tensors of tiny values: block amaxes log-uniform over [2^-149, 2^top],
    so many blocks sit below 2^-125 (their amax / 6 is subnormal) and, with
    top = -110, every E4M3 scale code occurs.  With top = -121 the tensor amax is
    so small that 2688 / amax overflows and the encode scale takes its clamped
    value."""
    rng = np.random.default_rng(-top)
    x = rng.uniform(-1.0, 1.0, (128, 1024)).astype(np.float64)
    x *= np.exp2(rng.uniform(-149, top, (128, 64))).repeat(16, axis=1)
    x_cpu = torch.from_numpy(x.astype(np.float32))
    for flags in (fp4.Q_SR, fp4.Q_RHT, fp4.Q_COLWISE | fp4.Q_RHT, fp4.Q_COLWISE | fp4.Q_RHT | fp4.Q_SR, fp4.Q_2D):
        run_case(fp4, oracle, x_cpu, flags, signs=0x3C5A, seed=9, offset=4)
    codes, scales, _ = host_q(run_case(fp4, oracle, x_cpu, 0))
    assert len(np.unique(scales)) > (100 if top == -110 else 50)


@pytest.mark.parametrize("signs", [0x3C5C, 0xF0F3])
def test_transform_with_cancelling_elements(fp4, oracle, signs):
    """Blocks (a, a, t, 0, ..., 0) along the transform's dimension, with the first
    two random signs equal: the transform cancels the two a's exactly in half of
    its outputs and leaves +-t there, so tiny elements (t down to a few times
    2^-149, where a quarter of t is inexact) sit in blocks whose amax is far larger
    (a from 2^-100 to 2^4).  Checks the transformed encoders bit for bit on blocks
    on both sides of their tiny-block threshold."""
    rng = np.random.default_rng(signs)
    nb = 64 * 32
    a = np.exp2(rng.uniform(-100, 4, nb)) * rng.choice([-1.0, 1.0], nb)
    t = np.where(rng.uniform(size=nb) < 0.5, rng.integers(1, 64, nb) * 2.0 ** -149,
                 np.exp2(rng.uniform(-149, -100, nb)) * rng.choice([-1.0, 1.0], nb))
    blocks = np.zeros((nb, 16))
    blocks[:, 0] = a
    blocks[:, 1] = a
    blocks[:, 2] = t
    rows = blocks.reshape(64, 32 * 16).astype(np.float32)       # blocks along rows
    cols = np.ascontiguousarray(rows.reshape(64, 32, 16).transpose(1, 2, 0).reshape(512, 64))  # down columns
    for flags in (fp4.Q_RHT, fp4.Q_RHT | fp4.Q_SR):
        run_case(fp4, oracle, torch.from_numpy(rows), flags, signs=signs, seed=11, offset=6)
        run_case(fp4, oracle, torch.from_numpy(cols), fp4.Q_COLWISE | flags, signs=signs, seed=11, offset=6)


def test_empty(fp4):
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    q = fp4.QTensor(0, 64)
    fp4.fp4_quantize(x, 0, 0, 0, 0, q)
    torch.cuda.synchronize()
    assert float(q.amax.cpu()[0]) == 0.0


def test_sr_offsets_decorrelate_on_gpu(fp4):
    x = dev(make_x((256, 1024), seed=3))
    a, b = fp4.QTensor(256, 1024), fp4.QTensor(256, 1024)
    fp4.fp4_quantize(x, fp4.Q_SR, 0, 11, 1, a)
    fp4.fp4_quantize(x, fp4.Q_SR, 0, 11, 2, b)
    torch.cuda.synchronize()
    frac = (a.codes != b.codes).float().mean().item()
    assert 0.2 < frac < 0.95


DUAL_CASES = [
    # (R, C, flags): the dy pair (SR, transformed columns), the x pair (RNE, transformed
    # columns), plain, ragged tiles (C not a multiple of 256, R not of 256)
    (256, 512, "sr_rht"),
    (512, 256, "rht"),
    (272, 400, "sr"),
    (48, 784, "none"),
    # the nearest-even pair at ragged tiles: a partial last column tile and slab tile
    (272, 400, "rht"),
    (48, 784, "rht"),
    # 8 x 8 whole tiles of the columnwise kernels
    (2048, 2048, "rht"),
    (2048, 2048, "sr_rht"),
]


@pytest.mark.parametrize("case", DUAL_CASES, ids=lambda c: f"{c[0]}x{c[1]}_{c[2]}")
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_quantize_dual_matches_two_single_quantizations(fp4, oracle, case, dtype):
    """One read of x, two layouts: each bit-exact against the oracle's own
    quantization of that layout (rowwise with offset_rows, columnwise with
    offset_cols), amaxes included."""
    R, C, mode = case
    sr, rht = "sr" in mode, "rht" in mode
    rng = np.random.default_rng(R * 7 + C)
    x = workloads.laplace(rng, (R, C)) if sr else workloads.normal(rng, (R, C), outlier_frac=0.01)
    xt = torch.from_numpy(x).to(dtype)
    xf = xt.float().numpy()
    signs, seed, o_r, o_c = 0xA5C3, 0x1234_5678_9ABC, 11, 12
    flags = (fp4.Q_SR if sr else 0) | (fp4.Q_RHT if rht else 0)
    qr, qc = fp4.QTensor(R, C), fp4.QTensor(C, R)
    fp4.fp4_quantize_dual(dev(xt), flags, signs, seed, o_r, o_c, qr, qc)
    ora_r = oracle.quantize(xf, sr=sr, seed=seed, offset=o_r)
    ora_c = oracle.quantize(xf, colwise=True, rht=rht, sr=sr, signs=signs, seed=seed, offset=o_c)
    assert_q_equal(host_q(qr), ora_r, f"dual rows {case}")
    assert_q_equal(host_q(qc), ora_c, f"dual cols {case}")
    # with the amaxes given, the same codes
    qr2, qc2 = fp4.QTensor(R, C), fp4.QTensor(C, R)
    qr2.amax.copy_(qr.amax)
    qc2.amax.copy_(qc.amax)
    fp4.fp4_quantize_dual(dev(xt), flags | fp4.Q_AMAX_GIVEN, signs, seed, o_r, o_c, qr2, qc2)
    assert_q_equal(host_q(qr2), ora_r, f"dual rows, amax given {case}")
    assert_q_equal(host_q(qc2), ora_c, f"dual cols, amax given {case}")


STRIDED_MODES = {
    "rows_rne": 0, "rows_sr": "SR", "rows_rht_sr": "RHT|SR", "cols_rne": "COLWISE", "cols_rht_sr": "COLWISE|RHT|SR",
    "two_d": "2D", "two_d_colwise": "2D|COLWISE",
}


@pytest.mark.parametrize("mode", list(STRIDED_MODES))
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_strided_input(fp4, oracle, mode, dtype):
    """x is a view of a wider matrix (row stride ld = cols + 40): the strided amax
    and encoding kernels against the oracle on the same values."""
    spec = STRIDED_MODES[mode]
    flags = 0
    for name in (spec.split("|") if spec else []):
        flags |= {"SR": fp4.Q_SR, "RHT": fp4.Q_RHT, "COLWISE": fp4.Q_COLWISE, "2D": fp4.Q_2D}[name]
    R, C = 272, 528
    wide = make_x((R, C + 40), seed=R + C, kind="laplace", std=1e-3, dtype=dtype)
    x = wide.to("cuda")[:, :C]
    assert x.stride(0) == C + 40
    colwise, two_d = bool(flags & fp4.Q_COLWISE), bool(flags & fp4.Q_2D)
    lrows, lcols = (C, R) if colwise else (R, C)
    q = fp4.QTensor(lrows, lcols, two_d)
    q_t = fp4.QTensor(lcols, lrows, True) if two_d else None
    fp4.fp4_quantize(x, flags, 0x6A95, 5, 9, q, q_t)
    xf = workloads.widen(wide)[:, :C]
    ora = oracle.quantize(xf, two_d=two_d, colwise=colwise, rht=bool(flags & fp4.Q_RHT), sr=bool(flags & fp4.Q_SR),
                          signs=0x6A95, seed=5, offset=9)
    assert_q_equal(host_q(q), ora, f"strided {mode}")
    if q_t is not None:
        assert_q_equal(host_q(q_t), oracle.quantize(xf, two_d=True, colwise=not colwise), f"strided {mode} (T)")
    # both layouts at once from the same strided view (stochastic: two kernels;
    # nearest-even: one kernel writing both)
    if mode == "rows_rne":
        for sr in (True, False):
            qr, qc = fp4.QTensor(R, C), fp4.QTensor(C, R)
            fp4.fp4_quantize_dual(x, (fp4.Q_SR if sr else 0) | fp4.Q_RHT, 0x6A95, 5, 9, 10, qr, qc)
            assert_q_equal(host_q(qr), oracle.quantize(xf, sr=sr, seed=5, offset=9), f"strided dual rows sr={sr}")
            assert_q_equal(host_q(qc), oracle.quantize(xf, colwise=True, rht=True, sr=sr, signs=0x6A95, seed=5,
                                                       offset=10), f"strided dual cols sr={sr}")


@pytest.mark.parametrize("shape", [(32, 512), (16, 496), (64, 256), (48, 320)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_amax_pass_both_forms(fp4, oracle, shape):
    """Tensors on both sides of 8 KB of codes: the amax pass keeps per-workgroup
    maxima in the codes buffer (reduced by one workgroup) at and above it, and
    folds them in with atomics below it.  Both give the oracle's amax and codes."""
    R, C = shape
    x_cpu = make_x(shape, seed=R * C, kind="outliers")
    for flags in (0, fp4.Q_RHT | fp4.Q_SR, fp4.Q_COLWISE | fp4.Q_RHT):
        run_case(fp4, oracle, x_cpu, flags, signs=0x1F2E, seed=3, offset=8)
    qr, qc = fp4.QTensor(R, C), fp4.QTensor(C, R)
    fp4.fp4_quantize_dual(dev(x_cpu), fp4.Q_RHT, 0x1F2E, 0, 0, 0, qr, qc)
    xf = workloads.widen(x_cpu)
    assert_q_equal(host_q(qr), oracle.quantize(xf), f"dual rows {shape}")
    assert_q_equal(host_q(qc), oracle.quantize(xf, colwise=True, rht=True, signs=0x1F2E), f"dual cols {shape}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_dual_with_a_row_stride_beyond_the_fused_kernel(fp4, oracle, dtype):
    """16 rows that span 2^31 bytes (row stride 2^31 / (16 * element size) elements)
    are beyond the one-kernel dual layouts' 32-bit row offsets: the call takes one
    kernel per layout and gives the same bits (a 2 GiB strided view, 16 x 256)."""
    R, C = 16, 256
    ld = (1 << 31) // (16 * torch.finfo(dtype).bits // 8)
    x_cpu = make_x((R, C), seed=77, dtype=dtype)
    full = torch.empty((R, ld), dtype=dtype, device="cuda")
    x = full[:, :C]
    x.copy_(x_cpu.to("cuda"))
    assert x.stride(0) == ld
    qr, qc = fp4.QTensor(R, C), fp4.QTensor(C, R)
    fp4.fp4_quantize_dual(x, fp4.Q_RHT, 0x2C4B, 0, 0, 0, qr, qc)
    xf = workloads.widen(x_cpu)
    assert_q_equal(host_q(qr), oracle.quantize(xf), "wide-stride dual rows")
    assert_q_equal(host_q(qc), oracle.quantize(xf, colwise=True, rht=True, signs=0x2C4B), "wide-stride dual cols")
    del full, x
    torch.cuda.empty_cache()


QUANT_MODES = ["rne", "sr", "rht", "rht_sr", "2d", "rht64", "rht64_sr", "eden"]


def random_quant_cases(n=24, seed=20261204, max_elems=6_000_000):
    """Seeded (R, C, mode, colwise, dtype, kind) over every quantizer mode and layout:
    the blocked dimension a multiple of 16 (64 for the 64-point transform and
    MS-EDEN; both for 2D), the other dimension free but for the row stride's multiple
    of 8 elements, ragged tiles in both, bf16 and fp32 inputs, Gaussian or Laplace
    values."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        mode = QUANT_MODES[len(out) % len(QUANT_MODES)]
        colwise = bool(rng.random() < 0.5)
        blk = 64 if mode.startswith("rht64") or mode == "eden" else 16
        nb = int(rng.integers(1, 4096 // blk + 1))
        other = int(rng.integers(1, 3000))
        if mode == "2d":
            other = 16 * max(1, other // 16)
        elif colwise:  # x's row stride: a multiple of 8 elements
            other = 8 * max(1, other // 8)
        R, C = (nb * blk, other) if colwise else (other, nb * blk)
        if R * C > max_elems:
            continue
        out.append((R, C, mode, colwise, "bf16" if rng.random() < 0.5 else "fp32",
                    "laplace" if rng.random() < 0.5 else "normal"))
    return out


@pytest.mark.parametrize("case", random_quant_cases(), ids=lambda c: f"{c[0]}x{c[1]}_{c[2]}_{'col' if c[3] else 'row'}_{c[4]}")
def test_quantize_random_cases(fp4, oracle, case):
    """fp4_quantize on seeded random shapes of every mode and layout, bit for bit
    against the oracle (codes, scales, amax; 2D also its transposed layout)."""
    R, C, mode, colwise, dtype, kind = case
    x_cpu = make_x((R, C), seed=R * 5 + C, kind=kind, std=1.0 if kind == "normal" else 1e-3,
                   dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    flags = {"rne": 0, "sr": fp4.Q_SR, "rht": fp4.Q_RHT, "rht_sr": fp4.Q_RHT | fp4.Q_SR, "2d": fp4.Q_2D,
             "rht64": fp4.Q_RHT64, "rht64_sr": fp4.Q_RHT64 | fp4.Q_SR, "eden": fp4.Q_RHT64 | fp4.Q_EDEN}[mode]
    if colwise:
        flags |= fp4.Q_COLWISE
    if mode in ("rne", "sr", "rht", "rht_sr", "2d"):
        run_case(fp4, oracle, x_cpu, flags, signs=0x6B1D, seed=0xC0FFEE, offset=5)
        return
    key = 0x9E3779B9
    lrows, lcols = (C, R) if colwise else (R, C)
    q = fp4.QTensor(lrows, lcols)
    fp4.fp4_quantize(dev(x_cpu), flags, key, 0xC0FFEE, 5, q)
    ora = oracle.quantize(workloads.widen(x_cpu), colwise=colwise, rht64=True, sr=mode == "rht64_sr",
                          eden=mode == "eden", signs=key, seed=0xC0FFEE, offset=5)
    assert_q_equal(host_q(q), ora, f"{case}")
