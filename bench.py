"""Benchmark: NVFP4 linear-layer step (fprop + dgrad + wgrad) on one MI355X.

One step is the whole hot path over one batch, through the library's linear-layer
calls: fp4_linear_fprop quantizes X (rowwise nearest-even, and X^T with the
16-point random Hadamard transform for wgrad, in one dual quantization) and W (2D
16x16 nearest-even, W^T emitted), then Y = X.W^T; fp4_linear_backward quantizes dY
once (rowwise stochastic for dgrad, dY^T transformed and stochastic for wgrad),
then dX = dY.W and dW = dY^T.X, reading the forward pass's W^T and X^T.  Each
quantization includes its amax pass; the GEMMs get the caller workspace sized by
fp4_linear_ws_bytes, so their split-K plans run.  Inputs are seeded synthetic
tensors (workloads/) already resident in HBM when the timed region starts.

Prints one JSON line.  `value` is whole-step NVFP4 linear TFLOP/s (3 GEMMs of
2*M*N*K flops each, divided by the step time including every quantization);
`roofline` is that of the dominant kernel, the block-scaled GEMM: its time comes
from HIP events the linear calls record between their phases inside the timed
steps (events without the system-scope fence, one per phase boundary, so that
timing does not slow the step); `quantize.kernels` times each quantize call of the
step, and its layout kernels alone, after the timed steps (input read from HBM),
with algorithmic bytes and the bound (HBM, or the vector ALU for the stochastic
encoders); `other_workloads` holds the same figures for the fprop 8k, wgrad 8k and
3B-block configurations (fewer steps each); `cpu_baseline` is the oracle timed on
the host cores this process may use, on a bounded sample of the same workload,
extrapolated to the step.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# published MI355X peaks (dense)
PEAK_HBM_GBS = 8000.0
PEAK_F16_MFMA_TFLOPS = 2500.0
PEAK_FP4_MFMA_TFLOPS = 10100.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mlp_up_12b",
                    choices=["mlp_up_12b", "fprop_8k", "wgrad_8k", "block_3b", "newton_schulz"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="measure only --workload (default: also the other full-size configurations, fewer steps)")
    ap.add_argument("--other-steps", type=int, default=10)
    ap.add_argument("--no-clocks", action="store_true",
                    help="skip the extra untimed steps that sample the driver's clocks (gpu_clocks: null)")
    ap.add_argument("--no-breakdown", action="store_true",
                    help="skip the per-kernel quantize breakdown (profiler runs that look at the steps only)")
    ap.add_argument("--cpu-sample-rows", type=int, default=8192)
    ap.add_argument("--error-vs-k", action="store_true",
                    help="instead of the benchmark: relative error of the NVFP4 GEMM against the unquantized binary64 "
                         "product for K from 256 to 32768, per quantization mode (one JSON line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy three times (the known-size reference that scales the "
                         "FETCH_SIZE / WRITE_SIZE counters into bytes) and exit")
    ap.add_argument("--ns-calls-only", choices=["rne", "rht_sr", "eden"],
                    help="with --workload newton_schulz: only run that operand variant's call (X' taken in the B X "
                         "GEMM's epilogue), warmup + steps times, and print its time per call (a short run for "
                         "kernel traces)")
    ap.add_argument("--stream-rates", action="store_true",
                    help="only measure streaming rates (the library's amax pass at 256 MiB to 2 GiB of bf16, and a "
                         "2 GiB device copy) and print one JSON line")
    return ap.parse_args()


ERROR_MODES = {  # operand A (activation- or gradient-like), operand B (weight-like)
    "rne": (0, 0),
    "rht": ("rht", "rht"),
    "sr": ("sr", 0),
    "rht_sr": ("rht_sr", "rht"),
    "rht64_sr": ("rht64_sr", "rht64"),
    "eden": ("eden", "rht64"),
}


def mode_flag(fp4, m):
    """fp4_quantize flags of an operand mode of ERROR_MODES (rht: the 16-point
    transform; rht64: the 64-point one; eden: MS-EDEN)."""
    return {0: 0, "rne": 0, "rht": fp4.Q_RHT, "sr": fp4.Q_SR, "rht_sr": fp4.Q_RHT | fp4.Q_SR, "rht64": fp4.Q_RHT64,
            "rht64_sr": fp4.Q_RHT64 | fp4.Q_SR, "eden": fp4.Q_RHT64 | fp4.Q_EDEN}[m]


def quantized_gemm_error(fp4, a, b, mode, signs, seed=0, offset=1):
    """Relative Frobenius error ||C_q - C|| / ||C|| of the NVFP4 GEMM of bf16 device
    tensors a [M, K], b [N, K] against their unquantized binary64 product.  Both
    operands are quantized 1D along K (rowwise); `mode` picks the random Hadamard
    transform (same signs on both operands, so the product is unchanged up to
    quantization) and stochastic rounding of A.  Returns (error, C_q)."""
    import torch
    fa, fb = ERROR_MODES[mode]
    M, K = a.shape
    N = b.shape[0]
    qa, qb = fp4.QTensor(M, K), fp4.QTensor(N, K)
    fp4.fp4_quantize(a, mode_flag(fp4, fa), signs, seed, offset, qa)
    fp4.fp4_quantize(b, mode_flag(fp4, fb), signs, seed, offset, qb)
    c = torch.empty(M, N, dtype=torch.float32, device=a.device)
    fp4.fp4_gemm(qa, qb, c)
    ref = a.double() @ b.double().T.contiguous()
    err = float(torch.linalg.norm(c.double() - ref) / torch.linalg.norm(ref))
    return err, c


QUANT_MODES = {  # A's mode -> the rotation of the identity that undoes A's
    "rne": 0, "sr": 0, "rht_sr": "rht", "rht64_sr": "rht64", "rht64": "rht64", "eden": "rht64"}


def identity_operand(fp4, K, mode, signs, device="cuda"):
    """The K x K identity quantized nearest-even with the rotation of `mode`'s
    operand A: its rows are the rotated unit vectors (entries 0, +-1/4 or +-1/8, all
    exact in NVFP4), so deq(A_q) . deq(I_q)^T is A's dequantized estimate rotated
    back -- the quantizer's output in A's own coordinates, from the product path."""
    import torch
    eye = torch.eye(K, dtype=torch.bfloat16, device=device)
    q = fp4.QTensor(K, K)
    fp4.fp4_quantize(eye, mode_flag(fp4, QUANT_MODES[mode]), signs, 0, 0, q)
    return q


def quantizer_estimate(fp4, a, mode, signs, ident, seed=0, offset=1):
    """A's NVFP4 estimate in A's coordinates (fp32 [M, K]): A quantized in `mode`,
    times the identity quantized with the same rotation."""
    import torch
    M, K = a.shape
    qa = fp4.QTensor(M, K)
    fp4.fp4_quantize(a, mode_flag(fp4, mode), signs, seed, offset, qa)
    c = torch.empty(M, K, dtype=torch.float32, device=a.device)
    fp4.fp4_gemm(qa, ident, c)
    return c


def quantizer_errors(fp4, data, K=4096, M=512, draws=4):
    """Relative mean squared error |A_hat - A|^2 / |A|^2 of each quantizer mode, over
    `draws` seeds and rotation keys, on activation-like, outlier-heavy and
    gradient-like data: the quantity the Quartet II page compares between MS-EDEN and
    stochastic rounding."""
    import torch

    import workloads
    rows = []
    for kind in data:
        if kind == "laplace":
            a = workloads.random_matrix((M, K), seed=K + 7, kind="laplace", std=1e-3)
        else:
            a = workloads.random_matrix((M, K), seed=K + 7, kind="outliers" if kind == "outliers" else "normal")
        a = a.cuda()
        ad = a.double()
        na = float((ad ** 2).sum())
        res = {}
        for mode in ("rne", "sr", "rht_sr", "rht64_sr", "eden"):
            errs = []
            for d in range(draws):
                key = 0x2545F491 * (d + 1) & 0xFFFFFFFF
                signs = key & 0xFFFF if mode == "rht_sr" else key
                ident = identity_operand(fp4, K, mode, signs)
                c = quantizer_estimate(fp4, a, mode, signs, ident, seed=d, offset=1)
                errs.append(float(((c.double() - ad) ** 2).sum()) / na)
            res[mode] = sum(errs) / len(errs)
        rows.append({"data": kind, "M": M, "K": K, "draws": draws, "rel_mse": {k: round(v, 6) for k, v in res.items()},
                     "sr_over_eden": round(res["sr"] / res["eden"], 3),
                     "rht_sr_over_eden": round(res["rht_sr"] / res["eden"], 3)})
        torch.cuda.synchronize()
    return rows


def eden_bias(fp4, M=64, K=4096, draws=4096):
    """The mean of the estimate over `draws` rotation keys (and scale draws), for
    MS-EDEN and for the same rotation with nearest-even and no correction: the
    distance of the mean from A relative to |A|, against the noise floor
    sqrt(E|A_hat - A|^2 / draws) / |A|.  An unbiased quantizer sits at the floor."""
    import torch

    import workloads
    a = workloads.random_matrix((M, K), seed=3, kind="laplace", std=1e-3).cuda()
    ad = a.double()
    na = float(torch.linalg.norm(ad))
    out = {}
    for mode in ("eden", "rht64"):
        acc = torch.zeros_like(ad)
        sq = 0.0
        for d in range(draws):
            key = (0x9E3779B1 * (d + 1)) & 0xFFFFFFFF
            c = quantizer_estimate(fp4, a, mode, key, identity_operand(fp4, K, mode, key), seed=d, offset=7).double()
            acc += c
            sq += float(((c - ad) ** 2).sum())
        bias = float(torch.linalg.norm(acc / draws - ad)) / na
        floor = (sq / draws) ** 0.5 / na / draws ** 0.5
        out[mode] = {"rel_bias": round(bias, 6), "noise_floor": round(floor, 6), "ratio": round(bias / floor, 3)}
    return {"M": M, "K": K, "draws": draws, "data": "Laplace(0, 1e-3)", "modes": out}


def error_vs_k():
    """Error accumulation of the NVFP4 GEMM versus K (the pages discuss how FP4
    errors grow along the reduction; they give no figures)."""
    import torch

    import nvfp4_bit_microscaled_amd as fp4
    import workloads

    fp4.load()
    M = N = 512
    rows = []
    for outliers in (False, True):
        for K in (256, 1024, 4096, 16384, 32768):
            a, b, signs = workloads.error_operands(M, N, K, seed=K, outliers=outliers)
            a, b = a.cuda(), b.cuda()
            for mode in ERROR_MODES:
                err, _ = quantized_gemm_error(fp4, a, b, mode, signs)
                rows.append({"K": K, "data": "outliers" if outliers else "gaussian", "mode": mode,
                             "rel_fro_error": round(err, 6)})
    torch.cuda.synchronize()
    quant = quantizer_errors(fp4, ("gaussian", "outliers", "laplace"))
    bias = eden_bias(fp4)
    print(json.dumps({"analysis": "NVFP4 GEMM relative Frobenius error vs K against the unquantized binary64 product",
                      "M": M, "N": N, "operands": "A ~ N(0,1) (optionally 0.1% x50 outliers), B ~ N(0, 0.02^2); bf16",
                      "modes": {k: f"A {v[0] or 'rne'}, B {v[1] or 'rne'}" for k, v in ERROR_MODES.items()},
                      "rows": rows,
                      "quantizer": quant,
                      "unbiasedness": bias}), flush=True)


def copy_calibration():
    """A plain device copy of known size, beyond the 256 MB Infinity Cache: each
    launch reads and writes exactly 512 MiB, so the HBM counters of these launches
    give the factor that turns counter readings into bytes."""
    import torch
    x = torch.ones(512 * 2**20 // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": x.numel() * 4, "launches": 3}), flush=True)



def stream_rates():
    """The practical HBM read rate by size: fp4_amax (a read-only pass, atomic form)
    over 256 MiB, 512 MiB and 2 GiB of bf16 (the 256 MB Infinity Cache holds at most
    the first), and a 2 GiB device copy; median of 10 launches each, after 3 warm-up
    launches, timed with HIP events on the current stream."""
    import torch

    import nvfp4_bit_microscaled_amd as fp4
    fp4.load()
    x = torch.randn(2**30 // 4096, 4096, dtype=torch.bfloat16, device="cuda")  # 2 GiB
    y = torch.empty_like(x)
    a = torch.zeros(1, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def med_ms(fn, reps=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = HipTimingEvent(), HipTimingEvent()
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[reps // 2]

    out = {"unit": "TB/s", "amax_read": {}}
    for mib in (256, 512, 2048):
        xs = x.view(-1)[:mib * 2**20 // 2].view(-1, 4096)
        ms = med_ms(lambda: fp4.fp4_amax(xs, 0, 0, a))
        out["amax_read"][f"{mib} MiB"] = {"ms": round(ms, 4), "rate": round(mib * 2**20 / (ms * 1e-3) / 1e12, 3)}
    ms = med_ms(lambda: y.copy_(x))
    out["copy_2GiB"] = {"ms": round(ms, 4), "rate": round(2 * 2**31 / (ms * 1e-3) / 1e12, 3),
                        "bytes": "read + written"}
    print(json.dumps(out), flush=True)


class HipTimingEvent:
    """A HIP event used only for timing, created with hipEventDisableSystemFence.  A
    default event record ends with a system-scope fence that writes back and
    invalidates the caches, which idled the GPU about 10 us at every recorded call
    boundary of the step and slowed the call after it.  With the flag, and one record
    per call boundary, the step measured as fast as with no per-call events at all
    (0.4-0.6% faster than with default events, two per boundary).  Elapsed times are
    read after a device synchronization."""
    _lib = None

    def __init__(self):
        import ctypes
        if HipTimingEvent._lib is None:
            lib = ctypes.CDLL("libamdhip64.so")
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            HipTimingEvent._lib = lib
        self._ct = ctypes
        self.h = ctypes.c_void_p()
        rc = HipTimingEvent._lib.hipEventCreateWithFlags(ctypes.byref(self.h), 0x20000000)  # hipEventDisableSystemFence
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")

    def record(self, stream):
        rc = HipTimingEvent._lib.hipEventRecord(self.h, self._ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_time(self, end):
        ms = self._ct.c_float()
        rc = HipTimingEvent._lib.hipEventElapsedTime(self._ct.byref(ms), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def __del__(self):
        if HipTimingEvent._lib is not None and self.h:
            HipTimingEvent._lib.hipEventDestroy(self.h)

def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel_src):
    """HBM bytes per fp4_gemm call (its launches together) from the committed
    rocprofv3 counter summary, if it was taken on the kernel source as it stands
    (same hash); else None."""
    p = os.path.join(ROOT, "profiles", "mlp_up_12b_hbm_traffic.md")
    if not os.path.exists(p):
        return None
    txt = open(p).read()
    h = re.search(r"source sha256\[:16\]: (\w+)", txt)
    t = re.search(r"bytes per step \(3 fp4_gemm calls\): ([0-9.eE+]+)", txt)
    if not h or not t or h.group(1) != source_hash(kernel_src):
        return None
    return float(t.group(1)) / 3.0


NS_SHAPE = (5120, 20480)  # X = G^T of the 12B MLP up-projection's weight gradient (20480 x 5120)
NS_ITERS = 5
NS_VARIANTS = ("rne", "rht_sr", "eden")


def ns_flags(fp4, variant):
    return {"rne": 0, "rht_sr": fp4.Q_RHT | fp4.Q_SR, "eden": fp4.Q_RHT64 | fp4.Q_EDEN}[variant]


def newton_schulz_timing(steps, warmup, dev, variants=NS_VARIANTS):
    """Muon's NVFP4 Newton-Schulz (5 iterations from X_0 = G / |G|) on a Gaussian G of
    the 12B MLP weight-gradient shape, per operand variant: time per call (HIP events
    on the stream) with X' = a X + B X taken in the B X GEMM's epilogue, the same with
    B X written out and a separate a X + B X pass, TFLOP/s over its 15 GEMMs, and each
    of its three GEMM shapes timed alone on the call's own quantized operands."""
    import torch

    import nvfp4_bit_microscaled_amd as fp4
    import workloads

    m, n = NS_SHAPE
    g = workloads.random_matrix((m, n), seed=0, dtype=torch.float32).to(dev)
    x = torch.empty_like(g)
    bufs = fp4.NsBuffers(m, n, device=dev, keep_bx=False)
    bufs_bx = fp4.NsBuffers(m, n, device=dev, keep_bx=True)
    stream = torch.cuda.current_stream()
    flops_iter = 2.0 * m * m * n + 2.0 * m * m * m + 2.0 * m * n * m

    def per_call(b, f):
        for _ in range(warmup):
            fp4.fp4_newton_schulz(g, x, NS_ITERS, b, flags=f, rht_signs=0x1234ACE1, seed=1, offset=0)
        evs = [HipTimingEvent() for _ in range(steps + 1)]
        torch.cuda.synchronize()
        evs[0].record(stream)
        for i in range(steps):
            fp4.fp4_newton_schulz(g, x, NS_ITERS, b, flags=f, rht_signs=0x1234ACE1, seed=1, offset=0)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        return sum(evs[i].elapsed_time(evs[i + 1]) for i in range(steps)) / steps

    out = {}
    for variant in variants:
        f = ns_flags(fp4, variant)
        ms_sep = per_call(bufs_bx, f)
        ms = per_call(bufs, f)
        # the three GEMM shapes alone (whole products through fp4_gemm_ws), on this call's
        # last operands: with nearest-even X X^T and A A^T take the left layout on both
        # sides (the right layouts are not written)
        same = variant == "rne"
        xr, ar = (bufs.x_left, bufs.a_left) if same else (bufs.x_right, bufs.a_right)
        gem = []
        for name, qa, qb, c, flops in (("A = X X^T", bufs.x_left, xr, bufs.a, 2.0 * m * m * n),
                                       ("A A^T", bufs.a_left, ar, bufs.b, 2.0 * m * m * m),
                                       ("B X", bufs.b_q, bufs.xt, bufs_bx.bx, 2.0 * m * n * m)):
            e0, e1 = HipTimingEvent(), HipTimingEvent()
            e0.record(stream)
            for _ in range(5):
                fp4.fp4_gemm_ws(qa, qb, c, bufs.ws)
            e1.record(stream)
            torch.cuda.synchronize()
            gms = e0.elapsed_time(e1) / 5
            gem.append({"gemm": name, "M": qa.rows, "N": qb.rows, "K": qa.cols, "ms": round(gms, 4),
                        "tflops": round(flops / (gms * 1e-3) / 1e12, 1),
                        "frac_f16_peak": round(flops / (gms * 1e-3) / 1e12 / PEAK_F16_MFMA_TFLOPS, 4)})
        out[variant] = {"ms_per_call": round(ms, 4), "ms_per_call_separate_axpby": round(ms_sep, 4),
                        "iters": NS_ITERS,
                        "tflops": round(NS_ITERS * flops_iter / (ms * 1e-3) / 1e12, 1), "gemms": gem}
    return {"X": [m, n], "flops_per_call": NS_ITERS * flops_iter, "variants": out}


def newton_schulz_divergence(dev, m=1024, n=4096):
    """Singular values after 5 iterations from the same Gaussian G, per variant, and in
    exact arithmetic (binary64 products, no quantization); the relative distance of each
    NVFP4 result from the exact one."""
    import torch

    import nvfp4_bit_microscaled_amd as fp4
    import workloads

    a_, b_, c_ = fp4.MUON_QUINTIC
    g = workloads.random_matrix((m, n), seed=1, dtype=torch.float32).to(dev)
    xe = g.double() / (torch.linalg.norm(g.double()) + 1e-7)
    for _ in range(NS_ITERS):
        a = xe @ xe.T
        xe = a_ * xe + (b_ * a + c_ * (a @ a)) @ xe
    sve = torch.linalg.svdvals(xe)
    res = {"G": [m, n], "exact": {"sigma_max": round(float(sve.max()), 4), "sigma_min": round(float(sve.min()), 4)}}
    bufs = fp4.NsBuffers(m, n, device=dev, keep_bx=False)
    x = torch.empty_like(g)
    for variant in NS_VARIANTS:
        fp4.fp4_newton_schulz(g, x, NS_ITERS, bufs, flags=ns_flags(fp4, variant), rht_signs=0x1234ACE1, seed=1,
                              offset=0)
        sv = torch.linalg.svdvals(x.double())
        res[variant] = {"sigma_max": round(float(sv.max()), 4), "sigma_min": round(float(sv.min()), 6),
                        "rel_distance_from_exact": round(float(torch.linalg.norm(x.double() - xe)
                                                               / torch.linalg.norm(xe)), 4)}
    return res


def newton_schulz_calls(variant, steps, warmup, dev):
    """Only the fused call of one operand variant on X 5120x20480: warmup + steps
    calls, the last steps timed with HIP events (one JSON line)."""
    import torch

    import nvfp4_bit_microscaled_amd as fp4
    import workloads

    m, n = NS_SHAPE
    g = workloads.random_matrix((m, n), seed=0, dtype=torch.float32).to(dev)
    x = torch.empty_like(g)
    bufs = fp4.NsBuffers(m, n, device=dev, keep_bx=False)
    f = ns_flags(fp4, variant)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fp4.fp4_newton_schulz(g, x, NS_ITERS, bufs, flags=f, rht_signs=0x1234ACE1, seed=1, offset=0)
    e0, e1 = HipTimingEvent(), HipTimingEvent()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        fp4.fp4_newton_schulz(g, x, NS_ITERS, bufs, flags=f, rht_signs=0x1234ACE1, seed=1, offset=0)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = NS_ITERS * (2.0 * m * m * n + 2.0 * m * m * m + 2.0 * m * n * m)
    print(json.dumps({"workload": "newton_schulz", "variant": variant, "X": [m, n], "iters": NS_ITERS,
                      "calls": warmup + steps, "timed_calls": steps, "ms_per_call": round(ms, 4),
                      "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}), flush=True)


def run_newton_schulz(args, dev):
    import torch
    if args.ns_calls_only:
        newton_schulz_calls(args.ns_calls_only, args.steps, args.warmup, dev)
        return
    t = newton_schulz_timing(args.steps, args.warmup, dev)
    torch.cuda.empty_cache()
    d = newton_schulz_divergence(dev)
    v = t["variants"]["rne"]
    gem = max(v["gemms"], key=lambda r: r["tflops"])
    out = {
        "metric": "NVFP4 linear TFLOPS (fprop/dgrad/wgrad) + quantize GB/s, % of roofline, 1 GPU",
        "value": v["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": v["ms_per_call"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "nvfp4 operands (e2m1 x e4m3 block scale), f16 MFMA products, f32 accumulate",
        "data": "synthetic (seeded: G ~ N(0,1) fp32)",
        "config": {"workload": f"Muon Newton-Schulz in NVFP4: quintic (3.4445, -4.7750, 2.0315), {NS_ITERS} "
                               f"iterations on X {t['X'][0]}x{t['X'][1]} (the 12B MLP up-projection's weight "
                               f"gradient, transposed), every GEMM operand quantized",
                   "name": "newton_schulz", "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": gem["tflops"], "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gem["tflops"] / PEAK_F16_MFMA_TFLOPS, 4), "traffic": None,
                     "kernel": f"block-scaled GEMM {gem['gemm']} ({gem['M']}x{gem['N']}x{gem['K']}) alone"},
        "newton_schulz": t, "divergence": d, "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def setup_workload(name, dev):
    """Device tensors and caller-owned buffers of every linear of workload `name`,
    plus one GEMM workspace sized by fp4_linear_ws_bytes for the largest layer."""
    import torch

    import nvfp4_bit_microscaled_amd as fp4
    import workloads

    wl = workloads.WORKLOADS[name]
    t_gen = time.time()
    layers = []
    for li, lin in enumerate(wl.linears):
        inp = workloads.make_linear_inputs(lin, seed=li, x_outliers=wl.x_outliers, with_dy="dgrad" in wl.passes
                                           or "wgrad" in wl.passes)
        x, w = inp.x.to(dev), inp.w.to(dev)
        dy = inp.dy.to(dev) if inp.dy is not None else None
        bufs = fp4.LinearBuffers(lin.M, lin.N, lin.K, device=dev)
        outs = {
            "y": torch.empty(lin.M, lin.N, dtype=torch.bfloat16, device=dev),
            "dx": torch.empty(lin.M, lin.K, dtype=torch.bfloat16, device=dev) if dy is not None else None,
            "dw": torch.empty(lin.N, lin.K, dtype=torch.float32, device=dev) if dy is not None else None,
        }
        layers.append((lin, inp, x, w, dy, bufs, outs))
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen
    ws_need = max(fp4.fp4_linear_ws_bytes(lin.M, lin.N, lin.K) for lin in wl.linears)
    ws = torch.empty(max(ws_need, 16), dtype=torch.uint8, device=dev)
    return wl, layers, ws, ws_need, t_gen


EDEN_KEY = 0x9E3779B9  # the 64-point rotation's key in the MS-EDEN backward


def step(wl, layers, ws, stream, record, backward="recipe"):
    """One pass of the whole hot path through the linear-layer calls.  `record`
    collects (kind, bytes or flops, ev0, ev1) per phase: each call records the phase
    events it documents, and a phase's start event is the previous phase's end event
    (one record per boundary).  With fprop and wgrad, fp4_linear_fprop also writes
    X^T transformed (one dual quantization of X) and the backward call reads it.
    backward="eden" (workloads with all three passes): fp4_linear_backward_eden, the
    wgrad operands with the 64-point rotation and dY^T with MS-EDEN; X^T is then
    quantized by the backward call from x."""
    import nvfp4_bit_microscaled_amd as Q
    import workloads

    ev = HipTimingEvent
    chain = [None]
    sd, od, ow = workloads.SR_SEED, workloads.SR_OFFSET_DGRAD, workloads.SR_OFFSET_WGRAD
    fprop, dgrad, wgrad = ("fprop" in wl.passes), ("dgrad" in wl.passes), ("wgrad" in wl.passes)

    def call(phases, fn):
        # phases: [(kind, amount)], one per interval between the call's events
        if chain[0] is None:
            chain[0] = ev()
            chain[0].record(stream)
        evs = [ev() for _ in phases]
        fn([e.h.value for e in evs[:-1]])
        evs[-1].record(stream)
        prev = chain[0]
        for (kind, amount), e in zip(phases, evs):
            if kind is not None:
                record.append((kind, amount, prev, e))
            prev = e
        chain[0] = evs[-1]

    for lin, inp, x, w, dy, b, o in layers:
        M, N, K = lin.M, lin.N, lin.K
        in_b = x.element_size()
        one_d = 0.5 + 1 / 16           # code + scale bytes per element of a 1D layout
        two_d = 2 * (0.5 + 1 / 256)    # W and W^T of a 2D quantization
        gflop = 2.0 * M * N * K
        eden = backward == "eden"
        if eden:
            assert fprop and dgrad and wgrad, "the MS-EDEN backward step needs all three passes"
        if fprop:
            xt = b.xq_t if wgrad and not eden else None
            call([("quant", M * K * (in_b + (2 if xt is not None else 1) * one_d)), ("quant", N * K * (in_b + two_d)),
                  ("gemm", gflop)],
                 lambda m: Q.fp4_linear_fprop(x, w, o["y"], b.xq, b.wq, b.wq_t, xq_t=xt, rht_signs=inp.signs, ws=ws,
                                              marks=m))
        if eden:
            call([("quant", M * N * (in_b + 2 * one_d)), ("quant", M * K * (in_b + one_d)), ("gemm", gflop),
                  ("gemm", gflop)],
                 lambda m: Q.fp4_linear_backward_eden(dy, x, b.wq_t, o["dx"], o["dw"], EDEN_KEY, sd, od, ow, b.dyq,
                                                      b.dyq_t, b.xq_t, ws=ws, marks=m))
        elif dgrad and wgrad:
            if fprop:  # X^T came with fprop's dual quantization: the X^T phase is empty
                phases = [("quant", M * N * (in_b + 2 * one_d)), (None, 0), ("gemm", gflop), ("gemm", gflop)]
            else:
                phases = [("quant", M * N * (in_b + 2 * one_d)), ("quant", M * K * (in_b + one_d)), ("gemm", gflop),
                          ("gemm", gflop)]
            call(phases, lambda m: Q.fp4_linear_backward(dy, None if fprop else x, b.wq_t, o["dx"], o["dw"],
                                                         inp.signs, sd, od, ow, b.dyq, b.dyq_t, b.xq_t, ws=ws,
                                                         marks=m))
        elif dgrad:
            call([("quant", M * N * (in_b + one_d)), ("gemm", gflop)],
                 lambda m: Q.fp4_linear_dgrad(dy, b.wq_t, o["dx"], sd, od, b.dyq, ws=ws, marks=m))
        elif wgrad:
            call([("quant", M * N * (in_b + one_d)), ("quant", M * K * (in_b + one_d)), ("gemm", gflop)],
                 lambda m: Q.fp4_linear_wgrad(dy, x, o["dw"], inp.signs, sd, ow, b.dyq_t, b.xq_t, ws=ws, marks=m))


def measure(wl, layers, ws, steps, warmup, backward="recipe"):
    """Warm up, then time `steps` steps (host clock between two device
    synchronizations) with the per-phase events; returns the step figures."""
    import torch

    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        step(wl, layers, ws, stream, [], backward)
    torch.cuda.synchronize()
    records = []
    t0 = time.perf_counter()
    for _ in range(steps):
        step(wl, layers, ws, stream, records, backward)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    gemm_ms = sum(e0.elapsed_time(e1) for k, _, e0, e1 in records if k == "gemm")
    gemm_flops = sum(f for k, f, _, _ in records if k == "gemm")
    n_gemm = sum(1 for k, *_ in records if k == "gemm")
    quant_ms = sum(e0.elapsed_time(e1) for k, _, e0, e1 in records if k == "quant")
    quant_bytes = sum(f for k, f, _, _ in records if k == "quant")
    step_flops = gemm_flops / steps
    return {
        "ms_per_step": ms_per_step,
        "step_flops": step_flops,
        "value": step_flops / (ms_per_step * 1e-3) / 1e12,
        "gemm_tflops": gemm_flops / (gemm_ms * 1e-3) / 1e12,
        "gemm_ms": gemm_ms,
        "gemm_flops": gemm_flops,
        "n_gemm": n_gemm,
        "quant_ms": quant_ms,
        "quant_gbs": quant_bytes / (quant_ms * 1e-3) / 1e9,
    }


def sysfs_clock_dir():
    """The sysfs directory of cuda:0's PCI device, which holds the driver's
    pp_dpm_sclk / pp_dpm_mclk tables; None when it cannot be found."""
    import glob

    import torch

    p = torch.cuda.get_device_properties(0)
    cand = []
    bus = getattr(p, "pci_bus_id", None)
    if bus is not None:
        cand.append("/sys/bus/pci/devices/%04x:%02x:%02x.0" % (getattr(p, "pci_domain_id", 0) or 0, bus,
                                                            getattr(p, "pci_device_id", 0) or 0))
    found = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if len(found) == 1:
        cand.append(os.path.dirname(found[0]))
    for d in cand:
        if os.access(os.path.join(d, "pp_dpm_sclk"), os.R_OK):
            return d
    return None


def sample_clocks(run, period_s=0.002):
    """Shader and memory clocks as the driver reports them while run() executes:
    the level marked current in pp_dpm_sclk / pp_dpm_mclk (its frequency is the
    measured one: it moves between the table's levels), read every period_s by a
    host thread.  Median, min and max in MHz, or None when sysfs is not readable."""
    import threading

    d = sysfs_clock_dir()
    if d is None:
        run()
        return None
    samples = {"sclk": [], "mclk": []}
    stop = threading.Event()

    def current(name):
        try:
            with open(os.path.join(d, "pp_dpm_" + name)) as f:
                for line in f:
                    if "*" in line:
                        return float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
        except (OSError, ValueError, IndexError):
            return None
        return None

    def loop():
        while not stop.is_set():
            for k in samples:
                v = current(k)
                if v is not None:
                    samples[k].append(v)
            time.sleep(period_s)

    t = threading.Thread(target=loop, daemon=True)
    t.start()
    try:
        run()
    finally:
        stop.set()
        t.join()
    out = {"source": "sysfs " + os.path.join(d, "pp_dpm_{sclk,mclk}") + ", the level marked current, sampled every "
                     f"{period_s * 1e3:g} ms"}
    for k, v in samples.items():
        if v:
            v = sorted(v)
            out[k + "_mhz"] = {"median": v[len(v) // 2], "min": v[0], "max": v[-1], "samples": len(v)}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the NVFP4 linear path here is measured "
              f"on one GPU's shard; sharding across GPUs is designed, not built", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.stream_rates:
        stream_rates()
        return
    if args.error_vs_k:
        error_vs_k()
        return

    import torch

    import nvfp4_bit_microscaled_amd as fp4

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    fp4.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "newton_schulz":
        run_newton_schulz(args, dev)
        return

    wl, layers, ws, ws_need, t_gen = setup_workload(args.workload, dev)
    r = measure(wl, layers, ws, args.steps, args.warmup)
    # the clocks the driver reports over as many steps again, after the timed ones (a
    # host thread reading sysfs stays out of the timed region)
    clocks = None if args.no_clocks else sample_clocks(lambda: measure(wl, layers, ws, args.steps, 0))
    gemm_shapes = []
    for lin in wl.linears:
        if "fprop" in wl.passes:
            gemm_shapes.append((lin.M, lin.N, lin.K))
        if "dgrad" in wl.passes:
            gemm_shapes.append((lin.M, lin.K, lin.N))
        if "wgrad" in wl.passes:
            gemm_shapes.append((lin.N, lin.K, lin.M))
    split_shapes = [sh for sh in gemm_shapes if fp4.fp4_gemm_ws_bytes(*sh) > 0]

    kernel_src = os.path.join(ROOT, "nvfp4_bit_microscaled_amd", "csrc", "gemm.hip")
    traffic = measured_traffic(kernel_src)
    gemm_tflops = r["gemm_tflops"]
    roofline = {
        "bound": "mfma",
        "achieved": round(gemm_tflops, 2),
        "peak": PEAK_F16_MFMA_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(gemm_tflops / PEAK_F16_MFMA_TFLOPS, 4),
        "traffic": traffic,
        "kernel": "nvfp4 block-scaled GEMM (f16 MFMA on exactly dequantized E2M1xE4M3 operands); the GEMM phase of "
                  "each linear-layer call: a persistent 256x256-tile launch, plus a 128x128-quarters launch when the "
                  "tiles overrun whole rounds of the CUs by at most half a round, or split over K into the caller "
                  "workspace and summed by a second launch when the plan for the shape takes a split",
        "split_k_shapes": split_shapes,
        "workspace_bytes": ws_need,
        "flops_per_call": r["gemm_flops"] / r["n_gemm"],
        "avg_call_ms": round(r["gemm_ms"] / r["n_gemm"], 4),
        "frac_of_fp4_dense_peak": round(gemm_tflops / PEAK_FP4_MFMA_TFLOPS, 4),
        "note": "exact NVFP4 products run on the f16 matrix path (one E8M0 scale per 32 K of the FP4/FP8 MFMAs cannot "
                "carry two E4M3 block scales), whose dense peak, 2.5 PFLOP/s, is half the MI355X's dense FP8 rate; "
                "the pages quote FP4 GEMMs at 2x (GB200) and 3x (GB300) the FP8 rate on Blackwell",
    }

    breakdown = [] if args.no_breakdown else quantize_breakdown(layers, wl)
    hbm_rows = [row for row in breakdown if row["bound"] == "hbm"]

    # the oracle runs last, on the host copies of these inputs: its thread pools keep
    # the host cores busy for a while after it returns, which delayed the launches of
    # GPU work timed after it (quantize phases of the other workloads measured up to
    # 1.5x their time)
    host_inputs = [(lin, inp) for lin, inp, *_ in layers]

    lin0 = wl.linears[0]
    out = {
        "metric": "NVFP4 linear TFLOPS (fprop/dgrad/wgrad) + quantize GB/s, % of roofline, 1 GPU",
        "value": round(r["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 operands (e2m1 x e4m3 block scale), f16 MFMA products, f32 accumulate",
        "data": "synthetic (seeded: X~N(0,1), W~N(0,0.02^2), dY~Laplace(0,1e-3); bf16)",
        "config": {
            "workload": wl.description,
            "name": wl.name,
            "linears": [[l.name, l.M, l.N, l.K] for l in wl.linears],
            "passes": list(wl.passes),
            "global_batch": lin0.M,
            "parallelism": "single GPU",
        },
        "quantize": {
            "achieved_gbs": round(r["quant_gbs"], 1),
            "peak_gbs": PEAK_HBM_GBS,
            "frac": round(r["quant_gbs"] / PEAK_HBM_GBS, 4),
            "note": "algorithmic bytes (input read once + codes + scales of every layout written) per quantize phase "
                    "of the linear calls; the time includes the amax pass",
            "ms_per_step": round(r["quant_ms"] / args.steps, 4),
            "kernels": breakdown,
            "hbm_bound_kernels_frac": round(sum(row["bytes"] for row in hbm_rows) / (sum(row["us"] for row in hbm_rows)
                                                                                     * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
            if hbm_rows else None,
        },
        "gemm_ms_per_step": round(r["gemm_ms"] / args.steps, 4),
        "roofline": roofline,
        "cpu_baseline": None,
        "gpu_clocks": clocks,
        "input_generation_s": round(t_gen, 1),
    }
    others = []
    if not args.no_other_workloads and all(p_ in wl.passes for p_ in ("fprop", "dgrad", "wgrad")):
        # the same layers with MS-EDEN in place of the 16-point transform + SR for dY^T
        # (and the 64-point rotation on X^T): fp4_linear_backward_eden
        o = measure(wl, layers, ws, args.other_steps, 2, backward="eden")
        others.append({
            "workload": wl.description + "; backward with MS-EDEN on dY^T and the 64-point rotation on both wgrad "
                                         "operands (fp4_linear_backward_eden)",
            "name": wl.name + "_eden_backward", "steps": args.other_steps,
            "ms_per_step": round(o["ms_per_step"], 4), "value": round(o["value"], 2), "unit": "TFLOP/s",
            "gemm_avg_call_ms": round(o["gemm_ms"] / o["n_gemm"], 4),
            "gemm_tflops": round(o["gemm_tflops"], 2),
            "quantize_ms_per_step": round(o["quant_ms"] / args.other_steps, 4),
        })
    del layers, ws
    torch.cuda.empty_cache()
    if not args.no_other_workloads:
        for name in ("fprop_8k", "wgrad_8k", "block_3b"):
            if name == args.workload:
                continue
            owl, olayers, ows, _, ogen = setup_workload(name, dev)
            o = measure(owl, olayers, ows, args.other_steps, 2)
            others.append({
                "workload": owl.description, "name": name, "steps": args.other_steps,
                "ms_per_step": round(o["ms_per_step"], 4), "value": round(o["value"], 2), "unit": "TFLOP/s",
                "gemm_avg_call_ms": round(o["gemm_ms"] / o["n_gemm"], 4),
                "gemm_tflops": round(o["gemm_tflops"], 2),
                "gemm_frac_f16_peak": round(o["gemm_tflops"] / PEAK_F16_MFMA_TFLOPS, 4),
                "quantize_ms_per_step": round(o["quant_ms"] / args.other_steps, 4),
                "quantize_gbs": round(o["quant_gbs"], 1),
                "quantize_frac_hbm": round(o["quant_gbs"] / PEAK_HBM_GBS, 4),
                "input_generation_s": round(ogen, 1),
            })
            del olayers, ows
            torch.cuda.empty_cache()
        nt = newton_schulz_timing(3, 1, dev, variants=("rne",))
        v = nt["variants"]["rne"]
        others.append({"workload": f"Muon Newton-Schulz in NVFP4, {NS_ITERS} iterations on X {nt['X'][0]}x{nt['X'][1]}",
                       "name": "newton_schulz", "steps": 3, "ms_per_step": v["ms_per_call"],
                       "ms_per_step_separate_axpby": v["ms_per_call_separate_axpby"], "value": v["tflops"],
                       "unit": "TFLOP/s", "gemms": v["gemms"]})
        torch.cuda.empty_cache()
        out["other_workloads"] = others
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(host_inputs, wl, args.cpu_sample_rows, r["step_flops"])
    print(json.dumps(out), flush=True)


def quantize_breakdown(layers, wl, reps=5):
    """The quantize calls of the step timed one at a time, each after a 512 MiB read
    so that its input comes from HBM, not from the 256 MB Infinity Cache: every call
    whole (its amax pass included), and its layout kernels alone (amax given).  Rates
    are algorithmic bytes over the median of `reps` calls: the input read once plus
    the outputs written once (so a whole call, which reads its input once for the
    amax and again for the layouts, is rated below its kernels).  The amax kernels'
    own times are in the step's kernel trace."""
    import torch

    import nvfp4_bit_microscaled_amd as Q
    import workloads

    stream = torch.cuda.current_stream()
    flush = torch.ones(512 * 2**20 // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")

    def med_ms(fn):
        ts = []
        for _ in range(reps):
            torch.sum(flush, dim=0, out=sink)
            e0, e1 = HipTimingEvent(), HipTimingEvent()
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[len(ts) // 2]

    G = Q.Q_AMAX_GIVEN
    one_d = 0.5 + 1 / 16
    two_d = 2 * (0.5 + 1 / 256)
    rows = []

    def add(name, kernel, nbytes, ms, bound):
        rows.append({"call": name, "kernel": kernel, "us": round(ms * 1e3, 1), "bytes": int(nbytes),
                     "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9
                                                                                    / PEAK_HBM_GBS, 3),
                     "bound": bound})

    for lin, inp, x, w, dy, b, o in layers:
        M, N, K = lin.M, lin.N, lin.K
        in_b = x.element_size()
        sd, od, ow = workloads.SR_SEED, workloads.SR_OFFSET_DGRAD, workloads.SR_OFFSET_WGRAD
        fprop, dgrad, wgrad = ("fprop" in wl.passes), ("dgrad" in wl.passes), ("wgrad" in wl.passes)
        if fprop and wgrad:
            xb = M * K * (in_b + 2 * one_d)
            add(f"{lin.name} X dual call (amax pass + both layouts)", "amax_dual4_kernel + quant_dual_ne_kernel", xb,
                med_ms(lambda: Q.fp4_quantize_dual(x, Q.Q_RHT, inp.signs, 0, 0, 0, b.xq, b.xq_t)), "call")
            add(f"{lin.name} X rowwise + X^T columnwise transformed, one kernel (amax given)", "quant_dual_ne_kernel",
                xb, med_ms(lambda: Q.fp4_quantize_dual(x, Q.Q_RHT | G, inp.signs, 0, 0, 0, b.xq, b.xq_t)), "hbm")
        elif fprop:
            add(f"{lin.name} X rowwise nearest-even (amax given)", "quant_rows_flat_kernel", M * K * (in_b + one_d),
                med_ms(lambda: Q.fp4_quantize(x, G, 0, 0, 0, b.xq)), "hbm")
        elif wgrad:
            add(f"{lin.name} X^T columnwise transformed (amax given)", "quant_cols4_kernel", M * K * (in_b + one_d),
                med_ms(lambda: Q.fp4_quantize(x, Q.Q_COLWISE | Q.Q_RHT | G, inp.signs, 0, 0, b.xq_t)), "hbm")
        if fprop or dgrad:
            wb = N * K * (in_b + two_d)
            add(f"{lin.name} W 2D call (amax pass + W and W^T)", "amax_flat_kernel + quant_2d_kernel", wb,
                med_ms(lambda: Q.fp4_quantize(w, Q.Q_2D, 0, 0, 0, b.wq, b.wq_t)), "call")
            add(f"{lin.name} W 2D + W^T nearest-even (amax given)", "quant_2d_kernel", wb,
                med_ms(lambda: Q.fp4_quantize(w, Q.Q_2D | G, 0, 0, 0, b.wq, b.wq_t)), "hbm")
            scratch = torch.zeros(1, dtype=torch.float32, device="cuda")
            add(f"{lin.name} W amax alone (fp4_amax: the same kernel, its atomic form)", "amax_flat_kernel",
                N * K * in_b, med_ms(lambda: Q.fp4_amax(w, 0, 0, scratch)), "hbm")
        if dgrad and wgrad:
            add(f"{lin.name} dY dual call (amax pass + two stochastic layouts)", "amax_dual4_kernel + quant_rows_flat_kernel + quant_cols4_kernel",
                M * N * (in_b + 2 * one_d),
                med_ms(lambda: Q.fp4_quantize_dual(dy, Q.Q_SR | Q.Q_RHT, inp.signs, sd, od, ow, b.dyq, b.dyq_t)),
                "call")
        if dgrad:
            add(f"{lin.name} dY rowwise stochastic (amax given)", "quant_rows_flat_kernel", M * N * (in_b + one_d),
                med_ms(lambda: Q.fp4_quantize(dy, Q.Q_SR | G, 0, sd, od, b.dyq)), "valu")
        if wgrad:
            add(f"{lin.name} dY^T columnwise transformed stochastic (amax given)", "quant_cols4_kernel",
                M * N * (in_b + one_d),
                med_ms(lambda: Q.fp4_quantize(dy, Q.Q_COLWISE | Q.Q_RHT | Q.Q_SR | G, inp.signs, sd, ow, b.dyq_t)),
                "valu")
            # MS-EDEN in place of the 16-point transform + SR for dY^T, and its GEMM
            # partner X^T with the same 64-point rotation (not in the timed step)
            key = 0x9E3779B9
            add(f"{lin.name} dY^T MS-EDEN call (64-point transform, amax pass + layout)",
                "amax_rht64_cols4_kernel + quant_cols64q_kernel", M * N * (in_b + one_d),
                med_ms(lambda: Q.fp4_quantize(dy, Q.Q_COLWISE | Q.Q_RHT64 | Q.Q_EDEN, key, sd, ow, b.dyq_t)), "call")
            add(f"{lin.name} dY^T columnwise 64-point transform + MS-EDEN (amax given)", "quant_cols64q_kernel",
                M * N * (in_b + one_d),
                med_ms(lambda: Q.fp4_quantize(dy, Q.Q_COLWISE | Q.Q_RHT64 | Q.Q_EDEN | G, key, sd, ow, b.dyq_t)),
                "valu")
            add(f"{lin.name} X^T columnwise 64-point transform nearest-even (amax given)", "quant_cols64q_kernel",
                M * K * (in_b + one_d),
                med_ms(lambda: Q.fp4_quantize(x, Q.Q_COLWISE | Q.Q_RHT64 | G, key, 0, 0, b.xq_t)), "hbm")
    del flush
    return rows


def host_cpu():
    """The host cores this process may use: its CPU affinity, further limited by a
    cgroup CPU quota when one is set; with nproc and the CPU model for the record."""
    n_all = os.cpu_count() or 1
    try:
        aff = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        aff = n_all
    quota = None
    try:
        q, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if q != "max":
            quota = int(q) / int(period)
    except (OSError, ValueError):
        pass
    usable = aff if quota is None else max(1, min(aff, int(quota)))
    model = None
    try:
        model = next((ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo") if ln.startswith("model name")),
                     None)
    except OSError:
        pass
    return {"usable": usable, "nproc": n_all, "affinity": aff, "cgroup_quota": quota, "model": model}


def cpu_baseline(layers, wl, sample_rows, step_flops):
    """The oracle, untuned, on the host cores this process may use (its own threads
    and the BLAS pool of the binary64 products both limited to that count):
    full-tensor amax passes, quantization of a sample of logical rows of every
    operand, and the binary64 GEMM reference on a sample x sample block of each pass;
    each part extrapolated linearly to the step."""
    from threadpoolctl import threadpool_limits

    cpu = host_cpu()
    with threadpool_limits(limits=cpu["usable"]):
        out = _cpu_baseline(layers, wl, sample_rows, step_flops, cpu["usable"])
    out["cores"] = cpu["usable"]
    out["host"] = cpu
    return out


def _cpu_baseline(layers, wl, sample_rows, step_flops, threads):
    import numpy as np

    import oracle
    import workloads

    _ = np.ones((256, 256)) @ np.ones((256, 256))  # start the BLAS thread pool outside the timed parts
    total_s = 0.0
    parts = []
    t_start = time.perf_counter()
    for lin, inp, *_ in layers:
        M, N, K = lin.M, lin.N, lin.K
        xf = workloads.widen(inp.x)
        wf = workloads.widen(inp.w)
        dyf = workloads.widen(inp.dy) if inp.dy is not None else None
        r = sample_rows
        jobs = []  # (array, kwargs, logical rows)
        if "fprop" in wl.passes:
            jobs += [("X", xf, dict(), M), ("W", wf, dict(two_d=True), N)]
        if "dgrad" in wl.passes:
            jobs += [("dY", dyf, dict(sr=True, seed=0, offset=1), M), ("W^T", wf, dict(two_d=True, colwise=True), K)]
        if "wgrad" in wl.passes:
            jobs += [("dY^T", dyf, dict(colwise=True, rht=True, sr=True, signs=inp.signs, seed=0, offset=2), N),
                     ("X^T", xf, dict(colwise=True, rht=True, signs=inp.signs), K)]
        qs = {}
        for name, arr, kw, rows in jobs:
            t = time.perf_counter()
            a = oracle.amax(arr, colwise=kw.get("colwise", False), rht=kw.get("rht", False), signs=kw.get("signs", 0),
                            threads=threads)
            t_amax = time.perf_counter() - t
            n = min(r, rows)
            t = time.perf_counter()
            qs[name] = oracle.quantize(arr, amax_in=a, rows=(0, n), threads=threads, **kw)
            t_q = time.perf_counter() - t
            total_s += t_amax + t_q * rows / n
        pairs = []
        if "fprop" in wl.passes:
            pairs.append(("X", "W", M, N))
        if "dgrad" in wl.passes:
            pairs.append(("dY", "W^T", M, K))
        if "wgrad" in wl.passes:
            pairs.append(("dY^T", "X^T", N, K))
        for a, b, rows_a, rows_b in pairs:
            # the oracle's GEMM reference is dequantize(A), dequantize(B), then the
            # binary64 products y = A.B^T and bound = |A|.|B|^T: the dequantizations
            # scale with the rows of each operand, the products with both
            qa, qb = qs[a], qs[b]
            t = time.perf_counter()
            da = oracle.dequantize(qa, threads=threads)
            t_da = time.perf_counter() - t
            t = time.perf_counter()
            db = oracle.dequantize(qb, threads=threads)
            t_db = time.perf_counter() - t
            t = time.perf_counter()
            _ = da @ db.T, np.abs(da) @ np.abs(db).T
            t_mm = time.perf_counter() - t
            total_s += t_da * rows_a / qa.rows + t_db * rows_b / qb.rows + t_mm * (rows_a / qa.rows) * (
                rows_b / qb.rows)
        del xf, wf, dyf
        parts.append(lin.name)
    wall = time.perf_counter() - t_start
    return {
        "value": round(step_flops / total_s / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"per operand: full-tensor amax + quantization of the first {sample_rows} logical rows; per pass: "
                   f"binary64 GEMM reference (dequantize both operands, y and sum|ab| products) on a "
                   f"{sample_rows}x{sample_rows} output block; amax passes at full size, every other part scaled to "
                   f"the full step by its own size law ({round(total_s, 1)} s extrapolated, {round(wall, 1)} s measured)"),
    }


if __name__ == "__main__":
    main()
