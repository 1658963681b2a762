"""CPU-side checks of the product library: it loads without a GPU, exports every
symbol include/nvfp4_amd.h declares, and rejects bad arguments before enqueuing
anything (argument checks run on the host, so they need no device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    with open(os.path.join(ROOT, "include", "nvfp4_amd.h")) as f:
        src = f.read()
    return sorted(set(re.findall(r"^\s*FP4_API\s+(?:fp4_status|const char \*)\s*(fp4_\w+)\s*\(", src, re.M)))


@pytest.fixture(scope="module")
def lib():
    import nvfp4_bit_microscaled_amd as m
    if not os.path.exists(m.LIB_PATH):
        from nvfp4_bit_microscaled_amd import build
        build.build()
    return m.load()


def test_header_lists_the_binding_exports():
    import nvfp4_bit_microscaled_amd as m
    assert header_functions() == sorted(m.EXPORTS)


def test_library_exports_every_header_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_library_does_not_export_internals():
    import nvfp4_bit_microscaled_amd as m
    out = os.popen(f"nm -D --defined-only {m.LIB_PATH}").read()
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert {n for n in exported if n.startswith("fp4_")} == set(m.EXPORTS)


def test_status_strings(lib):
    import nvfp4_bit_microscaled_amd as m
    for code in range(9):
        assert m.status_string(code)
    assert m.status_string(0) == "ok"


def test_tensor_bytes(lib):
    import nvfp4_bit_microscaled_amd as m
    assert m.tensor_bytes(8192, 4096) == (8192 * 2048, 8192 * 256)
    assert m.tensor_bytes(4096, 4096, True) == (4096 * 2048, 256 * 256)
    assert m.tensor_bytes(20, 32, True) == (20 * 16, 2 * 2)
    with pytest.raises(m.Fp4Error):
        m.tensor_bytes(16, 24)


def desc(rows, cols, two_d=0, base=0x10000):
    import nvfp4_bit_microscaled_amd as m
    return m.fp4_tensor(base, base + 0x100000, base + 0x200000, rows, cols, two_d)


def test_quantize_rejects_bad_arguments(lib):
    """Every call below fails its host-side checks, so no device pointer is touched."""
    import nvfp4_bit_microscaled_amd as m
    x = ctypes.c_void_p(0x1000)
    q = desc(64, 128)
    Q = ctypes.byref
    # unknown dtype
    assert lib.fp4_quantize(x, 7, 64, 128, 128, 0, 0, 0, 0, Q(q), None, None) == 4
    # K not a multiple of 16
    assert lib.fp4_quantize(x, 0, 64, 120, 120, 0, 0, 0, 0, Q(desc(64, 120)), None, None) in (2, 3)
    # descriptor shape mismatch
    assert lib.fp4_quantize(x, 0, 64, 128, 128, 0, 0, 0, 0, Q(desc(32, 128)), None, None) == 6
    # 2D with stochastic rounding is not a mode of the recipe
    assert lib.fp4_quantize(x, 0, 64, 128, 128, m.Q_2D | m.Q_SR, 0, 0, 0, Q(desc(64, 128, 1)), None, None) == 5
    # transposed output requested without 2D
    assert lib.fp4_quantize(x, 0, 64, 128, 128, 0, 0, 0, 0, Q(q), Q(desc(128, 64, 1)), None) == 5
    # null input
    assert lib.fp4_quantize(None, 0, 64, 128, 128, 0, 0, 0, 0, Q(q), None, None) == 1
    # misaligned input
    assert lib.fp4_quantize(ctypes.c_void_p(0x1002), 0, 64, 128, 128, 0, 0, 0, 0, Q(q), None, None) == 3
    # ld smaller than the row
    assert lib.fp4_quantize(x, 0, 64, 128, 64, 0, 0, 0, 0, Q(q), None, None) == 2
    # unknown flag bit
    assert lib.fp4_quantize(x, 0, 64, 128, 128, 1 << 9, 0, 0, 0, Q(q), None, None) == 5
    # colwise: logical tensor is [128][64]
    assert lib.fp4_quantize(x, 0, 64, 128, 128, m.Q_COLWISE, 0, 0, 0, Q(q), None, None) == 6


def test_gemm_rejects_bad_arguments(lib):
    c = ctypes.c_void_p(0x1000)
    Q = ctypes.byref
    a, b = desc(64, 128), desc(32, 128)
    assert lib.fp4_gemm(Q(a), Q(desc(32, 96)), c, 1, 32, None) == 6  # K mismatch
    assert lib.fp4_gemm(Q(a), Q(b), c, 9, 32, None) == 4  # dtype
    assert lib.fp4_gemm(Q(a), Q(b), c, 1, 16, None) == 2  # ldc < N
    assert lib.fp4_gemm(Q(a), Q(b), None, 1, 32, None) == 1
    assert lib.fp4_gemm(Q(a), Q(b), ctypes.c_void_p(0x1002), 1, 32, None) == 3
    assert lib.fp4_gemm(Q(a), Q(desc(24, 128, 1)), c, 1, 32, None) == 2  # 2D rows not tile multiple
    assert lib.fp4_gemm(None, Q(b), c, 1, 32, None) == 1


def test_gemm_ws_rejects_bad_arguments(lib):
    c = ctypes.c_void_p(0x1000)
    Q = ctypes.byref
    a, b = desc(64, 128), desc(32, 128)
    assert lib.fp4_gemm_ws(Q(a), Q(desc(32, 96)), c, 1, 32, ctypes.c_void_p(0x2000), 4096, None) == 6
    assert lib.fp4_gemm_ws(Q(a), Q(b), c, 1, 32, None, 4096, None) == 1  # bytes but no workspace
    assert lib.fp4_gemm_ws(Q(a), Q(b), c, 1, 32, ctypes.c_void_p(0x2008), 4096, None) == 3  # misaligned


def test_gemm_ws_bytes_follows_the_split_plan(lib):
    """The split plan on a 256-CU GPU (the host query falls back to 256 without a
    device): which products split, and the workspace = split tiles x splits x 256 KB;
    under a round of long-K tiles takes stream-K instead, whose workspace holds a
    256 KB slot per run (256) plus one per stream-K tile."""
    n = ctypes.c_size_t()
    tile = 256 * 256 * 4

    def need(M, N, K):
        assert lib.fp4_gemm_ws_bytes(M, N, K, ctypes.byref(n)) == 0
        return n.value
    assert need(3072, 3072, 32768) == (256 + 144) * tile  # 144 tiles: stream-K over all
    assert need(8192, 3072, 32768) == 128 * 2 * tile      # 384 tiles: the last 128 in 2
    assert need(9216, 3072, 32768) == (256 + 176) * tile  # 432 tiles: the last 176 as stream-K
    assert need(20480, 5120, 16384) == 64 * 4 * tile    # 1600 tiles: the last 64 in 4
    assert need(16384, 20480, 5120) == 0                # 20 whole rounds
    assert need(8192, 4096, 4096) == 0                  # 2 whole rounds
    assert need(256, 256, 256) == 0                     # one stage: nothing to split
    assert need(300, 200, 4096) == 2 * 4 * tile         # ragged, 2 tiles in 4
    assert lib.fp4_gemm_ws_bytes(64, 64, 40, ctypes.byref(n)) == 2  # K not a multiple of 16
    assert lib.fp4_gemm_ws_bytes(64, 64, 64, None) == 1


def test_linear_rejects_bad_arguments(lib):
    Q = ctypes.byref
    x, w, y = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000)
    ws = ctypes.c_void_p(0x5000)
    M, N, K = 64, 32, 48
    ok = lib.fp4_linear_fprop
    tail = (None, 0, None, None)  # ws, ws_bytes, marks, stream
    assert ok(x, w, 0, y, 0, M, N, 40, 0, Q(desc(M, 40)), None, Q(desc(N, 40, 1)), None, *tail) == 2
    assert ok(x, w, 0, y, 0, M, N, K, 0, Q(desc(M, K)), None, Q(desc(N, K, 0)), None, *tail) == 6  # W must be 2D
    assert ok(x, w, 0, y, 0, M, N, K, 0, Q(desc(M, K)), None, Q(desc(N, K, 1)), Q(desc(N, K, 1)), *tail) == 6  # W^T
    assert ok(x, w, 0, y, 0, M, N, K, 0, Q(desc(M, K)), Q(desc(M, K)), Q(desc(N, K, 1)), None, *tail) == 6  # X^T
    # workspace: bytes without a pointer, misaligned pointer
    assert ok(x, w, 0, y, 0, M, N, K, 0, Q(desc(M, K)), None, Q(desc(N, K, 1)), None, None, 64, None, None) == 1
    assert ok(x, w, 0, y, 0, M, N, K, 0, Q(desc(M, K)), None, Q(desc(N, K, 1)), None,
              ctypes.c_void_p(0x5004), 64, None, None) == 3
    assert lib.fp4_linear_dgrad(x, 0, Q(desc(N, K, 1)), y, 0, M, N, K, 0, 1, Q(desc(M, N)), *tail) == 6
    assert lib.fp4_linear_dgrad(x, 0, Q(desc(K, N, 1)), y, 0, M, N, K, 0, 1, Q(desc(M, N)), None, 16, None,
                                None) == 1
    assert lib.fp4_linear_wgrad(x, w, 0, y, 1, M, N, K, 0, 0, 2, Q(desc(N, M)), Q(desc(M, K)), *tail) == 6
    assert lib.fp4_linear_wgrad(x, w, 0, y, 1, M, N, K, 0, 0, 2, Q(desc(N, M)), Q(desc(K, M)),
                                ctypes.c_void_p(0x5008), 256, None, None) == 3
    del ws


def test_gemm_noalloc_rejects_before_touching_the_device(lib):
    """fp4_gemm_noalloc checks its arguments and the static scratch limit on the
    host: a shape whose split plan needs more than 64 MiB (the 3B block's O-projection
    wgrad, 144 tiles as stream-K over 256 runs = 100 MiB) is rejected with
    FP4_ERR_WORKSPACE."""
    import nvfp4_bit_microscaled_amd as m
    Q = ctypes.byref
    c = ctypes.c_void_p(0x100000)
    n = ctypes.c_size_t()
    assert lib.fp4_gemm_ws_bytes(3072, 3072, 32768, ctypes.byref(n)) == 0 and n.value > m.STATIC_SCRATCH_BYTES
    assert lib.fp4_gemm_noalloc(Q(desc(3072, 32768)), Q(desc(3072, 32768)), c, 1, 3072, None) == 8
    assert lib.fp4_gemm_noalloc(Q(desc(64, 128)), Q(desc(32, 96)), c, 1, 32, None) == 6  # K mismatch
    assert lib.fp4_gemm_noalloc(Q(desc(64, 128)), Q(desc(32, 128)), None, 1, 32, None) == 1
    # the 12B weight-gradient plan fits exactly
    assert lib.fp4_gemm_ws_bytes(20480, 5120, 16384, ctypes.byref(n)) == 0 and n.value == m.STATIC_SCRATCH_BYTES


def test_linear_ws_bytes_is_the_largest_gemm_plan(lib):
    """fp4_linear_ws_bytes = the largest split plan of fprop (M, N, K), dgrad
    (M, K, N) and wgrad (N, K, M)."""
    n = ctypes.c_size_t()

    def gemm(M, N, K):
        assert lib.fp4_gemm_ws_bytes(M, N, K, ctypes.byref(n)) == 0
        return n.value

    def linear(M, N, K):
        assert lib.fp4_linear_ws_bytes(M, N, K, ctypes.byref(n)) == 0
        return n.value
    for M, N, K in ((16384, 20480, 5120), (32768, 3072, 3072), (32768, 9216, 3072), (8192, 4096, 4096),
                    (32768, 3072, 8192), (256, 256, 256)):
        assert linear(M, N, K) == max(gemm(M, N, K), gemm(M, K, N), gemm(N, K, M))
    assert linear(16384, 20480, 5120) == 64 * 4 * 256 * 256 * 4  # the 12B wgrad tail
    assert lib.fp4_linear_ws_bytes(64, 40, 64, ctypes.byref(n)) == 2
    assert lib.fp4_linear_ws_bytes(64, 64, 64, None) == 1


def test_quantize_dual_rejects_bad_arguments(lib):
    import nvfp4_bit_microscaled_amd as m
    x = ctypes.c_void_p(0x1000)
    Q = ctypes.byref
    R, C = 64, 128
    rows, cols = desc(R, C), desc(C, R)
    f = lib.fp4_quantize_dual
    assert f(x, 0, R, C, C, 1 << 9, 0, 0, 0, 0, Q(rows), Q(cols), None) == 5  # unknown flag
    assert f(x, 0, R, C, C, m.Q_2D, 0, 0, 0, 0, Q(rows), Q(cols), None) == 5  # no 2D mode
    assert f(x, 0, 40, C, C, 0, 0, 0, 0, 0, Q(desc(40, C)), Q(desc(C, 40)), None) == 2  # rows % 16
    assert f(x, 0, R, C, C, 0, 0, 0, 0, 0, Q(cols), Q(cols), None) == 6  # rowwise descriptor shape
    assert f(x, 0, R, C, C, 0, 0, 0, 0, 0, Q(rows), Q(rows), None) == 6  # columnwise descriptor shape
    assert f(None, 0, R, C, C, 0, 0, 0, 0, 0, Q(rows), Q(cols), None) == 1
    assert f(x, 0, R, C, C, 0, 0, 0, 0, 0, None, Q(cols), None) == 1


def test_linear_backward_rejects_bad_arguments(lib):
    Q = ctypes.byref
    dy, x, dx, dw = (ctypes.c_void_p(a) for a in (0x1000, 0x2000, 0x3000, 0x4000))
    M, N, K = 64, 32, 48
    f = lib.fp4_linear_backward
    good = (Q(desc(K, N, 1)), dx, 1, dw, 0, M, N, K, 0, 0, 1, 2, Q(desc(M, N)), Q(desc(N, M)), Q(desc(K, M)),
            None, 0, None, None)
    assert f(dy, x, 0, *good[:5], M, N, 40, *good[8:]) == 2  # K % 16
    assert f(dy, x, 0, Q(desc(K, N, 0)), *good[1:]) == 6  # W^T must be 2D
    assert f(dy, x, 0, *good[:12], Q(desc(N, M)), *good[13:]) == 6  # dY rowwise shape
    assert f(dy, x, 0, *good[:14], Q(desc(M, K)), *good[15:]) == 6  # X^T shape
    assert f(None, x, 0, *good) == 1
    assert f(dy, x, 0, *good[:15], None, 32, None, None) == 1  # workspace bytes without a pointer


def test_linear_backward_eden_rejects_bad_arguments(lib):
    Q = ctypes.byref
    dy, x, dx, dw = (ctypes.c_void_p(a) for a in (0x1000, 0x2000, 0x3000, 0x4000))
    M, N, K = 128, 32, 48
    f = lib.fp4_linear_backward_eden
    good = (Q(desc(K, N, 1)), dx, 1, dw, 0, M, N, K, 0x9E3779B9, 0, 1, 2, Q(desc(M, N)), Q(desc(N, M)),
            Q(desc(K, M)), None, 0, None, None)
    assert f(dy, x, 0, *good[:5], 96, N, K, *good[8:]) == 2  # M % 64: the rotation runs along the tokens
    assert f(dy, x, 0, *good[:5], M, N, 40, *good[8:]) == 2  # K % 16
    assert f(dy, x, 0, Q(desc(K, N, 0)), *good[1:]) == 6  # W^T must be 2D
    assert f(dy, x, 0, *good[:13], Q(desc(M, N)), *good[14:]) == 6  # dY^T shape
    assert f(dy, x, 0, *good[:14], Q(desc(M, K)), *good[15:]) == 6  # X^T shape
    assert f(None, x, 0, *good) == 1
    assert f(dy, x, 0, *good[:15], None, 32, None, None) == 1  # workspace bytes without a pointer


def test_gemm_m0_is_only_written_by_the_lds_dma_statement(tmp_path):
    """The GEMM's LDS DMA sets M0 in inline assembly, which the compiler cannot see.
    That is sound only while no compiler-generated instruction of gemm.hip uses M0:
    compile its device code to assembly and check that every line naming m0 is the
    DMA statement's own write, followed by one wait state and the LDS DMA load."""
    import subprocess
    from nvfp4_bit_microscaled_amd import build
    out = tmp_path / "gemm.s"
    cmd = [build.HIPCC, *build.FLAGS, "--cuda-device-only", "-S", os.path.join(build.CSRC, "gemm.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    lines = [ln.strip() for ln in out.read_text().splitlines()]
    uses = [i for i, ln in enumerate(lines) if re.search(r"\bm0\b", ln) and not ln.startswith(";")]
    assert uses, "the DMA statement is expected in the assembly"
    for i in uses:
        assert re.fullmatch(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi|ttmp\d+)", lines[i]), lines[i]
        assert lines[i + 1] == "s_nop 0", lines[i + 1]
        assert lines[i + 2].startswith("buffer_load_dwordx4") and lines[i + 2].endswith("offen lds"), lines[i + 2]
