"""GPU parity of the three linear-layer passes, end to end through the C ABI:
every intermediate quantized operand bit-exact against the oracle, every output
within the GEMM tolerance of the binary64 reference built from the oracle's own
quantization.  Full-size workloads are checked on sampled output rows (and all
of their quantized operand rows); smaller ones in full."""
import numpy as np
import pytest
import torch

import workloads
from parity import assert_q_equal, check_gemm, dev, host_q

pytestmark = pytest.mark.gpu


def run_fprop(fp4, x_cpu, w_cpu, y_dtype):
    M, K = x_cpu.shape
    N = w_cpu.shape[0]
    bufs = fp4.LinearBuffers(M, N, K)
    y = torch.empty(M, N, dtype=y_dtype, device="cuda")
    fp4.fp4_linear_fprop(dev(x_cpu), dev(w_cpu), y, bufs.xq, bufs.wq, bufs.wq_t)
    torch.cuda.synchronize()
    return bufs, y


def sample_rows(n, count, seed):
    if n <= count:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(n, size=count, replace=False))


def pick(oracle, q, rows):
    """The given logical rows of an oracle-quantized 1D tensor."""
    return oracle.QTensor(q.codes[rows], q.scales[rows], q.amax, len(rows), q.K, False)


def check_rows(oracle, x_f32, gpu_q, rows, **kw):
    """Quantize only the chosen logical rows with the oracle (with the whole-tensor
    amax), compare them with the GPU's rows bit for bit, and return the oracle's."""
    amax = oracle.amax(x_f32, colwise=kw.get("colwise", False), rht=kw.get("rht", False), signs=kw.get("signs", 0))
    codes, scales, g_amax = gpu_q
    assert g_amax == amax
    parts = [oracle.quantize(x_f32, amax_in=amax, rows=(int(r), int(r) + 1), **kw) for r in rows]
    o_codes = np.concatenate([o.codes for o in parts])
    o_scales = np.concatenate([o.scales for o in parts])
    bad = [int(r) for i, r in enumerate(rows)
           if not (np.array_equal(codes[r], o_codes[i]) and np.array_equal(scales[r], o_scales[i]))]
    assert not bad, f"rows differing from the oracle: {bad[:8]}"
    return oracle.QTensor(o_codes, o_scales, amax, len(rows), parts[0].K, False)


@pytest.mark.parametrize("shape", [(32, 32, 64), (256, 128, 512), (1008, 272, 400)],
                         ids=lambda s: "x".join(map(str, s)))
def test_small_linear_all_passes(fp4, oracle, shape):
    """32 x 32 x 64: codes buffers too small for partial maxima, so the calls take
    their per-tensor amax passes (atomic form) instead of the merged launches."""
    M, N, K = shape
    inp = workloads.make_linear_inputs(workloads.Linear("t", M, N, K), seed=M + N + K)
    xf, wf, dyf = (workloads.widen(t) for t in (inp.x, inp.w, inp.dy))
    # fprop
    bufs, y = run_fprop(fp4, inp.x, inp.w, torch.bfloat16)
    oxq, owq = oracle.linear_fprop(xf, wf)
    assert_q_equal(host_q(bufs.xq), oxq, "xq")
    assert_q_equal(host_q(bufs.wq), owq, "wq")
    y_ref, bound = oracle.gemm_ref(oxq, owq)
    check_gemm(y.float().cpu().numpy(), y_ref, bound, True, "fprop")
    # dgrad
    dx = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    fp4.fp4_linear_dgrad(dev(inp.dy), bufs.wq_t, dx, workloads.SR_SEED, workloads.SR_OFFSET_DGRAD, bufs.dyq)
    odyq, owtq = oracle.linear_dgrad(dyf, wf, workloads.SR_SEED, workloads.SR_OFFSET_DGRAD)
    assert_q_equal(host_q(bufs.wq_t), owtq, "wq_t")
    assert_q_equal(host_q(bufs.dyq), odyq, "dyq")
    y_ref, bound = oracle.gemm_ref(odyq, owtq)
    check_gemm(dx.float().cpu().numpy(), y_ref, bound, True, "dgrad")
    # wgrad
    dw = torch.empty(N, K, dtype=torch.float32, device="cuda")
    fp4.fp4_linear_wgrad(dev(inp.dy), dev(inp.x), dw, inp.signs, workloads.SR_SEED, workloads.SR_OFFSET_WGRAD,
                         bufs.dyq_t, bufs.xq_t)
    odytq, oxtq = oracle.linear_wgrad(dyf, xf, inp.signs, workloads.SR_SEED, workloads.SR_OFFSET_WGRAD)
    assert_q_equal(host_q(bufs.dyq_t), odytq, "dyq_t")
    assert_q_equal(host_q(bufs.xq_t), oxtq, "xq_t")
    y_ref, bound = oracle.gemm_ref(odytq, oxtq)
    check_gemm(dw.cpu().numpy(), y_ref, bound, False, "wgrad")
    # the unquantized product, for the record (not a gate): relative Frobenius error
    exact = dyf.astype(np.float64).T @ xf.astype(np.float64)
    rel = np.linalg.norm(dw.cpu().numpy() - exact) / np.linalg.norm(exact)
    assert rel < 0.3


def test_fprop_8k_config(fp4, oracle):
    """X 8192x4096 N(0,1) with 0.1% x50 outliers, W 4096x4096 N(0, 0.02^2) 2D, Y bf16.
    Quantized operands in full; Y on 64 sampled rows."""
    wl = workloads.WORKLOADS["fprop_8k"]
    lin = wl.linears[0]
    inp = workloads.make_linear_inputs(lin, seed=0, x_outliers=True, with_dy=False)
    xf, wf = workloads.widen(inp.x), workloads.widen(inp.w)
    bufs, y = run_fprop(fp4, inp.x, inp.w, torch.bfloat16)
    oxq, owq = oracle.linear_fprop(xf, wf)
    assert_q_equal(host_q(bufs.xq), oxq, "xq")
    assert_q_equal(host_q(bufs.wq), owq, "wq")
    rows = sample_rows(lin.M, 64, 1)
    y_ref, bound = oracle.gemm_ref(pick(oracle, oxq, rows), owq)
    check_gemm(y.float().cpu().numpy()[rows], y_ref, bound, True, "fprop 8k")


def test_wgrad_8k_config(fp4, oracle):
    """dY 8192x4096 Laplace(0, 1e-3), X 8192x4096 N(0,1), RHT along the 8192 tokens,
    dY stochastically rounded, dW fp32 4096x4096; sampled dW rows."""
    lin = workloads.WORKLOADS["wgrad_8k"].linears[0]
    inp = workloads.make_linear_inputs(lin, seed=0)
    xf, dyf = workloads.widen(inp.x), workloads.widen(inp.dy)
    M, N, K = lin.M, lin.N, lin.K
    bufs = fp4.LinearBuffers(M, N, K)
    dw = torch.empty(N, K, dtype=torch.float32, device="cuda")
    fp4.fp4_linear_wgrad(dev(inp.dy), dev(inp.x), dw, inp.signs, workloads.SR_SEED, workloads.SR_OFFSET_WGRAD,
                         bufs.dyq_t, bufs.xq_t)
    torch.cuda.synchronize()
    odytq, oxtq = oracle.linear_wgrad(dyf, xf, inp.signs, workloads.SR_SEED, workloads.SR_OFFSET_WGRAD)
    assert_q_equal(host_q(bufs.dyq_t), odytq, "dyq_t")
    assert_q_equal(host_q(bufs.xq_t), oxtq, "xq_t")
    rows = sample_rows(N, 64, 2)
    y_ref, bound = oracle.gemm_ref(pick(oracle, odytq, rows), oxtq)
    check_gemm(dw.cpu().numpy()[rows], y_ref, bound, False, "wgrad 8k")


def test_mlp_up_12b_sampled(fp4, oracle):
    """The 12B-hybrid-like MLP up-projection at full size (X 16384x5120, W 20480x5120,
    dY 16384x20480): all three passes in the launch configuration the benchmark
    times (dual quantization of X and dY, fp4_linear_backward); quantized operands
    and outputs checked on sampled rows."""
    lin = workloads.WORKLOADS["mlp_up_12b"].linears[0]
    M, N, K = lin.M, lin.N, lin.K
    inp = workloads.make_linear_inputs(lin, seed=0)
    x, w, dy = dev(inp.x), dev(inp.w), dev(inp.dy)
    bufs = fp4.LinearBuffers(M, N, K)
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    dx = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    dw = torch.empty(N, K, dtype=torch.float32, device="cuda")
    # the benchmark's step: X's two layouts at once, W 2D (+W^T), Y; then the backward
    # pass with dY's two layouts at once and X^T from the forward pass
    fp4.fp4_quantize_dual(x, fp4.Q_RHT, inp.signs, 0, 0, 0, bufs.xq, bufs.xq_t)
    fp4.fp4_quantize(w, fp4.Q_2D, 0, 0, 0, bufs.wq, bufs.wq_t)
    fp4.fp4_gemm(bufs.xq, bufs.wq, y)
    fp4.fp4_linear_backward(dy, None, bufs.wq_t, dx, dw, inp.signs, workloads.SR_SEED, workloads.SR_OFFSET_DGRAD,
                            workloads.SR_OFFSET_WGRAD, bufs.dyq, bufs.dyq_t, bufs.xq_t)
    # the wgrad GEMM as the benchmark runs it: fp4_gemm_ws, whose plan splits the last
    # 64 of its 1600 tiles (dW rows 18432.., columns 3072..) over K instead of quarters
    ws = torch.empty(max(fp4.fp4_gemm_ws_bytes(N, K, M), 16), dtype=torch.uint8, device="cuda")
    dw2 = torch.empty(N, K, dtype=torch.float32, device="cuda")
    fp4.fp4_gemm_ws(bufs.dyq_t, bufs.xq_t, dw2, ws)
    torch.cuda.synchronize()
    del x, w, dy, ws
    xf, wf, dyf = (workloads.widen(t) for t in (inp.x, inp.w, inp.dy))
    sr, off_d, off_w = workloads.SR_SEED, workloads.SR_OFFSET_DGRAD, workloads.SR_OFFSET_WGRAD

    # fprop: sampled rows of X's quantization; W (2D) in full; sampled rows of Y
    rows = sample_rows(M, 24, 3)
    oxs = check_rows(oracle, xf, host_q(bufs.xq), rows)
    owq = oracle.quantize(wf, two_d=True)
    assert_q_equal(host_q(bufs.wq), owq, "wq")
    y_ref, bound = oracle.gemm_ref(oxs, owq)
    check_gemm(y.float().cpu().numpy()[rows], y_ref, bound, True, "fprop 12B")
    del owq, y

    # dgrad: sampled rows of dY's SR quantization; W^T (2D) in full; sampled dX rows
    ods = check_rows(oracle, dyf, host_q(bufs.dyq), rows, sr=True, seed=sr, offset=off_d)
    owtq = oracle.quantize(wf, two_d=True, colwise=True)
    assert_q_equal(host_q(bufs.wq_t), owtq, "wq_t")
    y_ref, bound = oracle.gemm_ref(ods, owtq)
    check_gemm(dx.float().cpu().numpy()[rows], y_ref, bound, True, "dgrad 12B")
    del owtq, dx

    # wgrad: sampled rows of dY^T (RHT+SR), some in the last tile-rows; X^T (RHT) in
    # full; sampled dW rows, from fp4_linear_backward and from fp4_gemm_ws
    wrows = np.union1d(sample_rows(N, 16, 4), sample_rows(N - 18432, 8, 5) + 18432)
    odt = check_rows(oracle, dyf, host_q(bufs.dyq_t), wrows, colwise=True, rht=True, sr=True, signs=inp.signs,
                     seed=sr, offset=off_w)
    oxtq = oracle.quantize(xf, colwise=True, rht=True, signs=inp.signs)
    assert_q_equal(host_q(bufs.xq_t), oxtq, "xq_t")
    y_ref, bound = oracle.gemm_ref(odt, oxtq)
    check_gemm(dw.cpu().numpy()[wrows], y_ref, bound, False, "wgrad 12B")
    check_gemm(dw2.cpu().numpy()[wrows], y_ref, bound, False, "wgrad 12B, fp4_gemm_ws")


def test_block_3b_sampled(fp4, oracle):
    """The 3B-like block at 32768 tokens: QKV, O, up and down projections, each with
    all three passes as the benchmark times them; every operand checked on sampled
    rows (codes and scales bit-exact with the whole-tensor amax), every output on a
    sampled block of rows and columns."""
    wl = workloads.WORKLOADS["block_3b"]
    sr, off_d, off_w = workloads.SR_SEED, workloads.SR_OFFSET_DGRAD, workloads.SR_OFFSET_WGRAD
    for li, lin in enumerate(wl.linears):
        M, N, K = lin.M, lin.N, lin.K
        inp = workloads.make_linear_inputs(lin, seed=li)
        x, w, dy = dev(inp.x), dev(inp.w), dev(inp.dy)
        bufs = fp4.LinearBuffers(M, N, K)
        y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        dx = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
        dw = torch.empty(N, K, dtype=torch.float32, device="cuda")
        fp4.fp4_quantize_dual(x, fp4.Q_RHT, inp.signs, 0, 0, 0, bufs.xq, bufs.xq_t)
        fp4.fp4_quantize(w, fp4.Q_2D, 0, 0, 0, bufs.wq, bufs.wq_t)
        fp4.fp4_gemm(bufs.xq, bufs.wq, y)
        fp4.fp4_linear_backward(dy, None, bufs.wq_t, dx, dw, inp.signs, sr, off_d, off_w, bufs.dyq, bufs.dyq_t,
                                bufs.xq_t)
        torch.cuda.synchronize()
        del x, w, dy
        xf, wf, dyf = (workloads.widen(t) for t in (inp.x, inp.w, inp.dy))
        owq = oracle.quantize(wf, two_d=True)
        assert_q_equal(host_q(bufs.wq), owq, f"{lin.name} wq")
        owtq = oracle.quantize(wf, two_d=True, colwise=True)
        assert_q_equal(host_q(bufs.wq_t), owtq, f"{lin.name} wq_t")
        rows = sample_rows(M, 12, 10 + li)
        # fprop: Y rows, all columns
        oxs = check_rows(oracle, xf, host_q(bufs.xq), rows)
        y_ref, bound = oracle.gemm_ref(oxs, owq)
        check_gemm(y.float().cpu().numpy()[rows], y_ref, bound, True, f"{lin.name} fprop")
        # dgrad: dX rows, all columns
        ods = check_rows(oracle, dyf, host_q(bufs.dyq), rows, sr=True, seed=sr, offset=off_d)
        y_ref, bound = oracle.gemm_ref(ods, owtq)
        check_gemm(dx.float().cpu().numpy()[rows], y_ref, bound, True, f"{lin.name} dgrad")
        # wgrad: a sampled block of dW (rows of dY^T, rows of X^T)
        nrows, kcols = sample_rows(N, 8, 20 + li), sample_rows(K, 48, 30 + li)
        odt = check_rows(oracle, dyf, host_q(bufs.dyq_t), nrows, colwise=True, rht=True, sr=True,
                         signs=inp.signs, seed=sr, offset=off_w)
        oxt = check_rows(oracle, xf, host_q(bufs.xq_t), kcols, colwise=True, rht=True, signs=inp.signs)
        y_ref, bound = oracle.gemm_ref(odt, oxt)
        check_gemm(dw.cpu().numpy()[np.ix_(nrows, kcols)], y_ref, bound, False, f"{lin.name} wgrad")
        # wgrad as the benchmark runs it: fp4_gemm_ws, split over K where the plan says so
        # (O: 144 tiles of 256x256 over K = 32768, 8 splits; up and down: 2)
        ws = torch.empty(max(fp4.fp4_gemm_ws_bytes(N, K, M), 16), dtype=torch.uint8, device="cuda")
        dw2 = torch.empty(N, K, dtype=torch.float32, device="cuda")
        fp4.fp4_gemm_ws(bufs.dyq_t, bufs.xq_t, dw2, ws)
        torch.cuda.synchronize()
        check_gemm(dw2.cpu().numpy()[np.ix_(nrows, kcols)], y_ref, bound, False, f"{lin.name} wgrad, fp4_gemm_ws")
        del y, dx, dw, dw2, ws, bufs


@pytest.mark.parametrize("quantize_x", [True, False], ids=["x_given", "xq_t_from_forward"])
def test_linear_backward_equals_dgrad_and_wgrad(fp4, oracle, quantize_x):
    """fp4_linear_backward (dY quantized once for both GEMMs) gives bit for bit the
    outputs and quantized operands of fp4_linear_dgrad + fp4_linear_wgrad, and both
    match the oracle."""
    M, N, K = 528, 272, 400
    inp = workloads.make_linear_inputs(workloads.Linear("t", M, N, K), seed=5)
    xf, wf, dyf = (workloads.widen(t) for t in (inp.x, inp.w, inp.dy))
    x, w, dy = dev(inp.x), dev(inp.w), dev(inp.dy)
    sr, off_d, off_w = workloads.SR_SEED, workloads.SR_OFFSET_DGRAD, workloads.SR_OFFSET_WGRAD
    a = fp4.LinearBuffers(M, N, K)
    fp4.fp4_quantize(w, fp4.Q_2D, 0, 0, 0, a.wq, a.wq_t)
    dx_a = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    dw_a = torch.empty(N, K, dtype=torch.float32, device="cuda")
    fp4.fp4_linear_dgrad(dy, a.wq_t, dx_a, sr, off_d, a.dyq)
    fp4.fp4_linear_wgrad(dy, x, dw_a, inp.signs, sr, off_w, a.dyq_t, a.xq_t)
    b = fp4.LinearBuffers(M, N, K)
    if not quantize_x:
        fp4.fp4_quantize_dual(x, fp4.Q_RHT, inp.signs, 0, 0, 0, b.xq, b.xq_t)
    dx_b = torch.empty_like(dx_a)
    dw_b = torch.empty_like(dw_a)
    fp4.fp4_linear_backward(dy, x if quantize_x else None, a.wq_t, dx_b, dw_b, inp.signs, sr, off_d, off_w, b.dyq,
                            b.dyq_t, b.xq_t)
    torch.cuda.synchronize()
    assert torch.equal(dx_a, dx_b) and torch.equal(dw_a, dw_b)
    for name, qa, qb in (("dyq", a.dyq, b.dyq), ("dyq_t", a.dyq_t, b.dyq_t), ("xq_t", a.xq_t, b.xq_t)):
        assert torch.equal(qa.codes, qb.codes) and torch.equal(qa.scales, qb.scales), name
        assert torch.equal(qa.amax, qb.amax), name
    odyq, owtq = oracle.linear_dgrad(dyf, wf, sr, off_d)
    odytq, oxtq = oracle.linear_wgrad(dyf, xf, inp.signs, sr, off_w)
    assert_q_equal(host_q(b.dyq), odyq, "dyq")
    assert_q_equal(host_q(b.dyq_t), odytq, "dyq_t")
    assert_q_equal(host_q(b.xq_t), oxtq, "xq_t")
    y_ref, bound = oracle.gemm_ref(odyq, owtq)
    check_gemm(dx_b.float().cpu().numpy(), y_ref, bound, True, "backward dgrad")
    y_ref, bound = oracle.gemm_ref(odytq, oxtq)
    check_gemm(dw_b.cpu().numpy(), y_ref, bound, False, "backward wgrad")


def test_linear_calls_equal_the_primitive_composition(fp4, oracle):
    """fp4_linear_fprop (with X^T) + fp4_linear_backward with a workspace give bit for
    bit the quantized operands and outputs of the same step composed from
    fp4_quantize_dual, fp4_quantize and fp4_gemm_ws, including a wgrad GEMM that
    takes the split-K path; the phase events they record complete in order; and the
    operands match the oracle (outputs within the GEMM tolerance)."""
    import bench

    M, N, K = 2048, 768, 1024
    assert fp4.fp4_gemm_ws_bytes(N, K, M) > 0, "the wgrad product is expected to split over K"
    inp = workloads.make_linear_inputs(workloads.Linear("t", M, N, K), seed=77)
    x, w, dy = dev(inp.x), dev(inp.w), dev(inp.dy)
    sr, od, ow = workloads.SR_SEED, workloads.SR_OFFSET_DGRAD, workloads.SR_OFFSET_WGRAD
    ws = torch.empty(fp4.fp4_linear_ws_bytes(M, N, K), dtype=torch.uint8, device="cuda")
    assert ws.numel() >= fp4.fp4_gemm_ws_bytes(N, K, M)
    outs = []
    for composed in (False, True):
        b = fp4.LinearBuffers(M, N, K)
        y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        dx = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
        dw = torch.empty(N, K, dtype=torch.float32, device="cuda")
        if composed:
            fp4.fp4_quantize_dual(x, fp4.Q_RHT, inp.signs, 0, 0, 0, b.xq, b.xq_t)
            fp4.fp4_quantize(w, fp4.Q_2D, 0, 0, 0, b.wq, b.wq_t)
            fp4.fp4_gemm_ws(b.xq, b.wq, y, ws)
            fp4.fp4_quantize_dual(dy, fp4.Q_SR | fp4.Q_RHT, inp.signs, sr, od, ow, b.dyq, b.dyq_t)
            fp4.fp4_gemm_ws(b.dyq, b.wq_t, dx, ws)
            fp4.fp4_gemm_ws(b.dyq_t, b.xq_t, dw, ws)
        else:
            stream = torch.cuda.current_stream()
            evs = [bench.HipTimingEvent() for _ in range(7)]
            evs[0].record(stream)
            fp4.fp4_linear_fprop(x, w, y, b.xq, b.wq, b.wq_t, xq_t=b.xq_t, rht_signs=inp.signs, ws=ws,
                                 marks=[evs[1].h.value, evs[2].h.value])
            fp4.fp4_linear_backward(dy, None, b.wq_t, dx, dw, inp.signs, sr, od, ow, b.dyq, b.dyq_t, b.xq_t, ws=ws,
                                    marks=[evs[3].h.value, evs[4].h.value, evs[5].h.value])
            evs[6].record(stream)
        torch.cuda.synchronize()
        if not composed:
            gaps = [evs[i].elapsed_time(evs[i + 1]) for i in range(6)]
            assert all(g >= 0.0 for g in gaps), gaps
            assert gaps[3] < 0.05 * sum(gaps), "the X^T phase of the backward call is empty when x is NULL"
        outs.append((b, y, dx, dw))
    (a, ya, dxa, dwa), (c, yc, dxc, dwc) = outs
    for name in ("xq", "xq_t", "wq", "wq_t", "dyq", "dyq_t"):
        qa, qc = getattr(a, name), getattr(c, name)
        assert torch.equal(qa.codes, qc.codes) and torch.equal(qa.scales, qc.scales), name
        assert torch.equal(qa.amax, qc.amax), name
    assert torch.equal(ya, yc) and torch.equal(dxa, dxc) and torch.equal(dwa, dwc)
    # and against the oracle
    xf, wf, dyf = (workloads.widen(t) for t in (inp.x, inp.w, inp.dy))
    oxq, owq = oracle.linear_fprop(xf, wf)
    odyq, owtq = oracle.linear_dgrad(dyf, wf, sr, od)
    odytq, oxtq = oracle.linear_wgrad(dyf, xf, inp.signs, sr, ow)
    for name, o in (("xq", oxq), ("wq", owq), ("wq_t", owtq), ("dyq", odyq), ("dyq_t", odytq), ("xq_t", oxtq)):
        assert_q_equal(host_q(getattr(a, name)), o, name)
    for name, out, qa, qb, bf16 in (("fprop", ya, oxq, owq, True), ("dgrad", dxa, odyq, owtq, True),
                                    ("wgrad", dwa, odytq, oxtq, False)):
        ref, bound = oracle.gemm_ref(qa, qb)
        check_gemm(out.float().cpu().numpy(), ref, bound, bf16, name)


@pytest.mark.parametrize("quantize_x", [True, False], ids=["x", "xq_t_given"])
@pytest.mark.parametrize("shape", [(64, 128, 64), (256, 128, 192), (1024, 272, 400), (2048, 768, 1024)],
                         ids=lambda s: "x".join(map(str, s)))
def test_linear_backward_eden(fp4, oracle, shape, quantize_x):
    """fp4_linear_backward_eden: dY rowwise with stochastic rounding for dgrad, dY^T
    with MS-EDEN and X^T nearest-even, both after the 64-point rotation along the
    tokens, for wgrad.  Every quantized operand bit-exact against the oracle, both
    outputs within the GEMM tolerance of the binary64 product of the oracle's
    operands; the rotation cancels, so dW stays close to the unquantized product.
    64 x 128 x 64 is small enough that dY's amaxes are merged by atomics (its codes
    buffer cannot hold the partial maxima); 2048 x 768 x 1024 takes the split-K path
    for wgrad."""
    M, N, K = shape
    inp = workloads.make_linear_inputs(workloads.Linear("t", M, N, K), seed=M + 3 * N + K)
    xf, wf, dyf = (workloads.widen(t) for t in (inp.x, inp.w, inp.dy))
    x, w, dy = dev(inp.x), dev(inp.w), dev(inp.dy)
    sr, od, ow = workloads.SR_SEED, workloads.SR_OFFSET_DGRAD, workloads.SR_OFFSET_WGRAD
    key = 0x9E3779B9
    b = fp4.LinearBuffers(M, N, K)
    fp4.fp4_quantize(w, fp4.Q_2D, 0, 0, 0, b.wq, b.wq_t)
    if not quantize_x:
        fp4.fp4_quantize(x, fp4.Q_COLWISE | fp4.Q_RHT64, key, 0, 0, b.xq_t)
    ws = torch.empty(max(fp4.fp4_linear_ws_bytes(M, N, K), 16), dtype=torch.uint8, device="cuda")
    dx = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    dw = torch.empty(N, K, dtype=torch.float32, device="cuda")
    fp4.fp4_linear_backward_eden(dy, x if quantize_x else None, b.wq_t, dx, dw, key, sr, od, ow, b.dyq, b.dyq_t,
                                 b.xq_t, ws=ws)
    torch.cuda.synchronize()
    odyq, owtq = oracle.linear_dgrad(dyf, wf, sr, od)
    odytq = oracle.quantize(dyf, colwise=True, rht64=True, eden=True, signs=key, seed=sr, offset=ow)
    oxtq = oracle.quantize(xf, colwise=True, rht64=True, signs=key)
    for name, o in (("dyq", odyq), ("wq_t", owtq), ("dyq_t", odytq), ("xq_t", oxtq)):
        assert_q_equal(host_q(getattr(b, name)), o, name)
    y_ref, bound = oracle.gemm_ref(odyq, owtq)
    check_gemm(dx.float().cpu().numpy(), y_ref, bound, True, "eden backward dgrad")
    y_ref, bound = oracle.gemm_ref(odytq, oxtq)
    check_gemm(dw.cpu().numpy(), y_ref, bound, False, "eden backward wgrad")
    exact = dyf.astype(np.float64).T @ xf.astype(np.float64)
    assert np.linalg.norm(dw.cpu().numpy() - exact) / np.linalg.norm(exact) < 0.3
