"""HIP graph capture of the library's calls: every launch is a kernel on the given
stream (no memset, no allocation, no host synchronisation), so a caller can capture
a training step, or a Newton-Schulz call, and replay it.  Each test captures once,
then replays several times with eager work (the outputs zeroed) and device
synchronisations between the replays, and checks every replay against the same
calls run eagerly, bit for bit."""
import pytest
import torch

import workloads
from parity import dev

pytestmark = pytest.mark.gpu


def capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def replay_and_check(g, outputs, expected, replays=3):
    for r in range(replays):
        for t in outputs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(outputs, expected)):
            assert torch.equal(got, want), f"replay {r}, output {i}"


def test_linear_step_in_a_graph(fp4):
    """fprop (with X^T) + backward with a workspace, the wgrad product split over K,
    and fp4_gemm_noalloc (the library's static scratch) on the step's operands."""
    M, N, K = 2048, 768, 1024
    assert fp4.fp4_gemm_ws_bytes(N, K, M) > 0
    inp = workloads.make_linear_inputs(workloads.Linear("t", M, N, K), seed=11)
    x, w, dy = dev(inp.x), dev(inp.w), dev(inp.dy)
    sr, od, ow = workloads.SR_SEED, workloads.SR_OFFSET_DGRAD, workloads.SR_OFFSET_WGRAD
    ws = torch.empty(fp4.fp4_linear_ws_bytes(M, N, K), dtype=torch.uint8, device="cuda")
    b = fp4.LinearBuffers(M, N, K)
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    dx = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    dw = torch.empty(N, K, dtype=torch.float32, device="cuda")
    dw2 = torch.empty(N, K, dtype=torch.float32, device="cuda")

    def step():
        fp4.fp4_linear_fprop(x, w, y, b.xq, b.wq, b.wq_t, xq_t=b.xq_t, rht_signs=inp.signs, ws=ws)
        fp4.fp4_linear_backward(dy, None, b.wq_t, dx, dw, inp.signs, sr, od, ow, b.dyq, b.dyq_t, b.xq_t, ws=ws)
        fp4.fp4_gemm_noalloc(b.dyq_t, b.xq_t, dw2)

    step()
    torch.cuda.synchronize()
    outputs = [y, dx, dw, dw2, b.xq.codes, b.xq_t.codes, b.wq.codes, b.dyq.codes, b.dyq_t.codes, b.dyq_t.amax]
    expected = [t.clone() for t in outputs]
    assert torch.equal(dw, dw2)
    g = capture(step)
    replay_and_check(g, outputs, expected)


@pytest.mark.parametrize("variant", ["rne", "rht_sr", "eden"])
def test_newton_schulz_in_a_graph(fp4, variant):
    """A 3-iteration NVFP4 Newton-Schulz call (normalisation included, X' taken in
    the B X GEMM's epilogue) captured and replayed."""
    m, n = 256, 512
    flags = {"rne": 0, "rht_sr": fp4.Q_RHT | fp4.Q_SR, "eden": fp4.Q_RHT64 | fp4.Q_EDEN}[variant]
    g_in = dev(workloads.random_matrix((m, n), seed=3, dtype=torch.float32))
    x = torch.empty_like(g_in)
    bufs = fp4.NsBuffers(m, n, keep_bx=False)

    def call():
        fp4.fp4_newton_schulz(g_in, x, 3, bufs, flags=flags, rht_signs=0x1234ACE1, seed=9, offset=0)

    call()
    torch.cuda.synchronize()
    outputs = [x, bufs.a, bufs.b, bufs.x_left.codes, bufs.xt.codes, bufs.b_q.codes, bufs.x_left.amax]
    expected = [t.clone() for t in outputs]
    graph = capture(call)
    replay_and_check(graph, outputs, expected)
