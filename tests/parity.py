"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same seeded input, compare.

Acceptance (both fixed in advance, not tuned to results):
* quantized codes, scales and the tensor amax: bit-exact;
* GEMM outputs: |y - y_ref| <= 1e-5 * sum_k |a_mk b_nk| with y_ref the binary64
  product of the oracle's dequantized operands; for bf16 outputs the rounding of
  the output itself adds at most 2^-8 |y| (half a bf16 ulp is <= 2^-8 relative),
  so the bound becomes 1e-5 * (1 + 2^-8) * bound + 2^-8 * |y_ref|.
"""
import numpy as np
import torch

REL_TOL = 1e-5
BF16_REL = 2.0 ** -8


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.to("cuda").contiguous()


def host_q(q):
    """GPU QTensor -> numpy (codes [rows][cols/2], scales, amax)."""
    torch.cuda.synchronize()
    return q.codes_2d().cpu().numpy(), q.scales_2d().cpu().numpy(), float(q.amax.cpu()[0])


def assert_q_equal(gpu, ora, what=""):
    codes, scales, amax = gpu
    assert amax == ora.amax, f"{what}: amax {amax!r} != oracle {ora.amax!r}"
    assert scales.shape == ora.scales.shape, what
    bad_s = np.argwhere(scales != ora.scales)
    assert bad_s.size == 0, f"{what}: {len(bad_s)} scale mismatches, first at {bad_s[0].tolist()}"
    assert codes.shape == ora.codes.shape, what
    bad = np.argwhere(codes != ora.codes)
    assert bad.size == 0, f"{what}: {len(bad)} code-byte mismatches, first at {bad[0].tolist()}"


def check_gemm(y: np.ndarray, y_ref: np.ndarray, bound: np.ndarray, bf16: bool, what=""):
    y = y.astype(np.float64)
    if bf16:
        tol = REL_TOL * (1 + BF16_REL) * bound + BF16_REL * np.abs(y_ref)
    else:
        tol = REL_TOL * bound
    err = np.abs(y - y_ref)
    ok = err <= tol
    if not ok.all():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outputs out of tolerance; worst at {i}: "
                             f"y={y[i]!r} ref={y_ref[i]!r} bound={bound[i]!r}")
    return float((err / np.maximum(bound, 1e-300)).max())


def upload_q(fp4, ora, device="cuda"):
    """Copy an oracle-quantized tensor into device buffers (the oracle feeding the
    GPU GEMM, never the other way round)."""
    q = fp4.QTensor(ora.rows, ora.K, ora.two_d, device=device)
    q.codes.copy_(torch.from_numpy(np.ascontiguousarray(ora.codes).reshape(-1)))
    q.scales.copy_(torch.from_numpy(np.ascontiguousarray(ora.scales).reshape(-1)))
    q.amax.fill_(ora.amax)
    return q
