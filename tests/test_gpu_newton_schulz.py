"""GPU parity of the NVFP4 Newton-Schulz iteration (fp4_newton_schulz; Full-Stack FP4
pages, paragraph 1, optimizer sentence) against the oracle, stage by stage: each
iteration runs on the GPU, and the oracle redoes it from the GPU's own inputs to
that stage, so every quantized operand is compared bit for bit, every product
within the GEMM tolerance, and X' = a X + B X bit for bit given the GPU's B X."""
import numpy as np
import pytest
import torch

import workloads
from parity import assert_q_equal, check_gemm, dev, host_q

pytestmark = pytest.mark.gpu

SIGNS = 0x1234ACE1
A_, B_, C_ = 3.4445, -4.7750, 2.0315


def variant_flags(fp4, variant):
    return {"rne": 0, "rht_sr": fp4.Q_RHT | fp4.Q_SR, "eden": fp4.Q_RHT64 | fp4.Q_EDEN}[variant]


@pytest.mark.parametrize("variant", ["rne", "rht_sr", "eden"])
@pytest.mark.parametrize("shape", [(128, 256), (256, 768), (1024, 4096), (512, 128), (400, 512), (768, 512),
                                   (2560, 9984), (5888, 256)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
def test_newton_schulz_stagewise(fp4, oracle, variant, shape):
    """With nearest-even operands X X^T and A A^T take the symmetric GEMM (tiles on
    and above the diagonal, mirrored) when their K is whole 256-element stages: A and
    B come out exactly symmetric, each element within the GEMM tolerance; 400 x 512
    has ragged 256 x 256 tiles and a mirror whose 64 x 64 blocks overhang the edge.
    The plans differ by shape: 768 x 512 runs X X^T as one persistent launch whose
    epilogue also stores each upper tile's transpose below the diagonal; 5888 x 256
    does that for its first 256 of 276 upper tiles and the last 20 as 128 x 128
    quarters; 1024 x 4096 splits X X^T over K; 2560 x 9984 runs it as stream-K (55
    upper tiles of 39 stages, 100 whole ones for the other variants) and A A^T, with B
    in its epilogue, split over K in 2 (the reduction adds b A); after a split or
    stream-K, and after A A^T, the mirror kernel fills the lower triangle."""
    m, n = shape
    if variant == "eden" and (m % 64 or n % 64):
        pytest.skip("the 64-point transform needs multiples of 64")
    iters = 3 if m < 1024 else 1
    g_cpu = workloads.random_matrix((m, n), seed=m + n, dtype=torch.float32)
    g = dev(g_cpu)
    x = torch.empty_like(g)
    bufs = fp4.NsBuffers(m, n)
    flags = variant_flags(fp4, variant)
    fp4.fp4_newton_schulz(g, x, 0, bufs, normalize=True, flags=flags, rht_signs=SIGNS, seed=7, offset=100)
    torch.cuda.synchronize()
    xt = x.cpu().numpy()
    o0 = oracle.ns_normalize(workloads.widen(g_cpu))
    # the scale is rounded once to binary32 from a binary64 sum whose order differs
    # from the oracle's: equal unless that sum sits within 1e-16 of a rounding edge
    assert np.all(np.abs(xt - o0) <= np.spacing(np.abs(o0)))
    for t in range(iters):
        fp4.fp4_newton_schulz(x, x, 1, bufs, normalize=False, flags=flags, rht_signs=SIGNS, seed=7,
                              offset=100 + 8 * t)
        torch.cuda.synchronize()
        a, b, bx, xn = (v.cpu().numpy() for v in (bufs.a, bufs.b, bufs.bx, x))
        st = oracle.ns_step(xt, variant, signs=SIGNS, seed=7, offset=100 + 8 * t, a_in=a, b_in=b, bx_in=bx)
        names = ("x_left", "a_left", "b_q", "xt") if variant == "rne" else \
            ("x_left", "x_right", "a_left", "a_right", "b_q", "xt")
        for name in names:
            assert_q_equal(host_q(getattr(bufs, name)), st[name], f"{variant} iteration {t} {name}")
        check_gemm(a, st["a_ref"], st["a_bound"], False, f"{variant} iteration {t} A = X X^T")
        if variant == "rne" and n % 256 == 0:  # X X^T on the 256-K main path: the symmetric GEMM
            assert np.array_equal(a, a.T), f"iteration {t}: A not symmetric"
            if m % 256 == 0:  # A A^T too, so B = b A + c A2 is
                assert np.array_equal(b, b.T), f"iteration {t}: B not symmetric"
        # B = fl(fl(b A) + fl(c A2)) with the GPU's A2 within the GEMM tolerance
        b_ref = B_ * a.astype(np.float64) + C_ * st["a2_ref"]
        tol = abs(C_) * 1e-5 * st["a2_bound"] + 2.0 ** -22 * (np.abs(B_ * a) + np.abs(C_ * st["a2_ref"]))
        assert np.all(np.abs(b - b_ref) <= tol), f"{variant} iteration {t} B"
        check_gemm(bx, st["bx_ref"], st["bx_bound"], False, f"{variant} iteration {t} B X")
        assert np.array_equal(xn, st["x_next"]), f"{variant} iteration {t} X'"
        xt = xn
    if iters > 1:
        # several iterations in one call equal the same iterations one call each; the
        # last iteration's operands too (with nearest-even, a call's later iterations
        # take X's amax from the axpby that wrote X, the first from an amax pass)
        x2 = torch.empty_like(g)
        bufs2 = fp4.NsBuffers(m, n)
        fp4.fp4_newton_schulz(g, x2, iters, bufs2, normalize=True, flags=flags, rht_signs=SIGNS, seed=7, offset=100)
        torch.cuda.synchronize()
        assert torch.equal(x2, x)
        for name in names:
            c1, s1, a1 = host_q(getattr(bufs2, name))
            c2, s2, a2 = host_q(getattr(bufs, name))
            assert a1 == a2 and np.array_equal(s1, s2) and np.array_equal(c1, c2), f"{variant} one call, {name}"


def test_newton_schulz_rejects_bad_arguments(fp4):
    g = torch.zeros(64, 96, dtype=torch.float32, device="cuda")
    bufs = fp4.NsBuffers(64, 96)
    with pytest.raises(fp4.Fp4Error, match="SHAPE"):  # the 64-point transform needs multiples of 64
        fp4.fp4_newton_schulz(g, g, 1, bufs, flags=fp4.Q_RHT64 | fp4.Q_EDEN)
    with pytest.raises(fp4.Fp4Error, match="MODE"):
        fp4.fp4_newton_schulz(g, g, 1, bufs, flags=fp4.Q_SR)
    with pytest.raises(fp4.Fp4Error, match="MISMATCH"):
        fp4.fp4_newton_schulz(torch.zeros(64, 128, device="cuda"), torch.zeros(64, 128, device="cuda"), 1, bufs)


@pytest.mark.parametrize("variant", ["rne", "rht_sr", "eden"])
@pytest.mark.parametrize("shape", [(128, 256), (512, 400), (1024, 4096), (4096, 1024), (4400, 4000), (5120, 20480)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
def test_newton_schulz_fused_epilogue_equals_the_axpby(fp4, variant, shape):
    """Without B X, X' = a X + B X is taken in the B X GEMM's epilogue: the same
    binary32 operations, so X and every quantized operand (amax included: with
    nearest-even operands the epilogue's maximum gives the next X's) equal the call
    that writes B X and runs the axpby.  The shapes reach the edge kernel (K = 128),
    the partial-tile main kernel (N = 400), the whole-tile main kernel, its split-K
    form (4096 x 1024: B X is 4096 x 1024 x 4096, 64 tiles split over K), partial
    tiles with 128x128 quarters for the last 32 of 288 tiles (4400 x 4000), and the
    12B weight-gradient shape (1600 whole tiles, the last 64 as quarters)."""
    m, n = shape
    if variant == "eden" and (m % 64 or n % 64):
        pytest.skip("the 64-point transform needs multiples of 64")
    g = dev(workloads.random_matrix((m, n), seed=m * 3 + n, dtype=torch.float32))
    flags = variant_flags(fp4, variant)
    out = {}
    for keep in (True, False):
        x = torch.empty_like(g)
        bufs = fp4.NsBuffers(m, n, keep_bx=keep)
        fp4.fp4_newton_schulz(g, x, 3, bufs, normalize=True, flags=flags, rht_signs=SIGNS, seed=5, offset=40)
        torch.cuda.synchronize()
        out[keep] = (x, bufs)
    assert torch.equal(out[True][0], out[False][0]), f"{variant} {shape}: X"
    names = ("x_left", "a_left", "b_q", "xt") if variant == "rne" else \
        ("x_left", "x_right", "a_left", "a_right", "b_q", "xt")
    for name in names:
        c1, s1, a1 = host_q(getattr(out[True][1], name))
        c2, s2, a2 = host_q(getattr(out[False][1], name))
        assert a1 == a2 and np.array_equal(s1, s2) and np.array_equal(c1, c2), f"{variant} {shape}: {name}"
