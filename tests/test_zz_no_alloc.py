"""GPU check of fp4_gemm_noalloc, the GEMM entry point that allocates nothing
(its split-K partial tiles go to the library's static scratch): two calls in a
row, the second on a smaller product, each bit-identical to fp4_gemm_ws with a
caller workspace of fp4_gemm_ws_bytes, and within the GEMM tolerance of the
oracle's binary64 product."""
import pytest
import torch

import workloads
from parity import check_gemm, upload_q

pytestmark = pytest.mark.gpu


def _operands(oracle, M, N, K, seed):
    a = workloads.widen(workloads.random_matrix((M, K), seed))
    b = workloads.widen(workloads.random_matrix((N, K), seed + 1, std=0.02))
    return oracle.quantize(a), oracle.quantize(b)


@pytest.mark.parametrize("c_dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_noalloc_equals_gemm_ws_twice(fp4, oracle, c_dtype):
    # (M, N, K): both plans split over K; the second product is smaller
    shapes = [(1024, 1024, 8192), (512, 768, 4096)]
    for M, N, K in shapes:
        need = fp4.fp4_gemm_ws_bytes(M, N, K)
        assert 0 < need <= fp4.STATIC_SCRATCH_BYTES, (M, N, K, need)
    results = []
    for i, (M, N, K) in enumerate(shapes):
        print(f"fp4_gemm_noalloc call {i}: {M}x{N}x{K} {c_dtype}", flush=True)
        qa, qb = _operands(oracle, M, N, K, seed=100 + i)
        ga, gb = upload_q(fp4, qa), upload_q(fp4, qb)
        c_na = torch.full((M, N), float("nan"), dtype=c_dtype, device="cuda")
        fp4.fp4_gemm_noalloc(ga, gb, c_na)
        ws = torch.empty(fp4.fp4_gemm_ws_bytes(M, N, K), dtype=torch.uint8, device="cuda")
        c_ws = torch.full((M, N), float("nan"), dtype=c_dtype, device="cuda")
        fp4.fp4_gemm_ws(ga, gb, c_ws, ws)
        torch.cuda.synchronize()
        assert torch.equal(c_na, c_ws), f"call {i}: noalloc differs from fp4_gemm_ws"
        ref, bound = oracle.gemm_ref(qa, qb)
        check_gemm(c_na.float().cpu().numpy(), ref, bound, c_dtype == torch.bfloat16, f"noalloc call {i}")
        results.append(c_na)
    assert results[1].shape != results[0].shape


def test_noalloc_takes_the_split_when_stream_k_does_not_fit(fp4, oracle):
    """2560 x 2560 x 16384 plans stream-K with a workspace of 256 + 100 slots (89 MiB),
    more than the 64 MiB static scratch: fp4_gemm_noalloc then runs the shape's fixed
    split, bit-identical to fp4_gemm_ws given a 64 MiB workspace (which makes the same
    choice), and within the GEMM tolerance of the oracle."""
    M, N, K = 2560, 2560, 16384
    assert fp4.fp4_gemm_ws_bytes(M, N, K) == (256 + 100) * 256 * 256 * 4 > fp4.STATIC_SCRATCH_BYTES
    print(f"fp4_gemm_noalloc {M}x{N}x{K}", flush=True)
    qa, qb = _operands(oracle, M, N, K, seed=7)
    ga, gb = upload_q(fp4, qa), upload_q(fp4, qb)
    c_na = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    fp4.fp4_gemm_noalloc(ga, gb, c_na)
    ws = torch.empty(fp4.STATIC_SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
    c_ws = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    fp4.fp4_gemm_ws(ga, gb, c_ws, ws)
    torch.cuda.synchronize()
    assert torch.equal(c_na, c_ws)
    ref, bound = oracle.gemm_ref(qa, qb)
    check_gemm(c_na.cpu().numpy(), ref, bound, False, "noalloc with the split plan")
