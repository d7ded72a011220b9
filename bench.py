"""Benchmark of the FP8 runtime chain on one MI355X.

Default workload (the prefill-shaped layer): X bf16 4096x8192 drawn as
0.5 * Student-t(3), quantized per tensor with a current (dynamic) E4M3 scale;
W bf16 29568x8192 ~ N(0, 0.02) quantized once at setup with a static
per-tensor E4M3 scale; Y = s_x s_w (X8 W8^T) in bf16.  One step = the per-batch
hot path: amax(X) -> scale -> saturating cast of X (with saturation/underflow
counters) -> scaled GEMM with FP32 accumulation and bf16 output.  Inputs are
resident in HBM before the timed region.  Prints one JSON line.

The other workload shapes (decode, delayed-scaling backward, block-scaled)
are parity-test cases; their quantize and GEMM kernels are timed as extra
components of the same line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 quantize GB/s + scaled-GEMM TFLOP/s, as % of MI355X HBM/FP8 peak"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="CPU budget of the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the other workload shapes' component timings")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run only a plain device copy of 1 GiB (read 1 GiB, write 1 GiB) three "
                        "times: the reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    return p.parse_args()


def src_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_from_profile(kernel_file: str):
    """HBM bytes per launch from a committed rocprofv3 PMC summary, if it was
    taken on the current kernel source (else None)."""
    prof = os.path.join(ROOT, "profiles", kernel_file)
    if not os.path.exists(prof):
        return None
    try:
        d = json.load(open(prof))
    except (OSError, ValueError):
        return None
    src = os.path.join(ROOT, d.get("source", ""))
    if not os.path.exists(src) or src_hash(src) != d.get("source_sha256_16"):
        return None
    return d.get("hbm_bytes_per_launch")


class Timer:
    """HIP events on torch's current stream, which is the stream the library
    launches on (the binding passes torch.cuda.current_stream())."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def start(self, name):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.setdefault(name, []).append([e, None])

    def stop(self, name):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs[name][-1][1] = e

    def ms(self, name):
        return [a.elapsed_time(b) for a, b in self.pairs.get(name, [])]


def cpu_baseline_prefill(x_bits, w_bits, M, N, K, budget_s):
    """The oracle as it stands, single-threaded, on a bounded sample of the
    same workload, extrapolated to one full step (TFLOP/s of the step).  All
    oracle inputs come from the seeded generators and the oracle itself."""
    import oracle

    oracle.build(force=False)
    # untimed setup: static weight scale and the codes of a sample of W rows
    g = np.random.default_rng(7)
    w_rows = np.sort(g.choice(N, size=256, replace=False))
    s_w, _ = oracle.compute_scale(oracle.amax(w_bits), oracle.E4M3)
    wq, _, _, _, _ = oracle.quantize(np.ascontiguousarray(w_bits[w_rows]), oracle.E4M3, (0, 0),
                                     mode=oracle.GIVEN, scale=s_w)
    # timed: full amax of X, then the cast of a sample of rows
    t0 = time.perf_counter()
    oracle.amax(x_bits)
    t_amax = time.perf_counter() - t0
    rows_done, tq, chunk = 0, 0.0, 64
    while tq < budget_s * 0.25 and rows_done + chunk <= M:
        t0 = time.perf_counter()
        xq, s_x, _, _, _ = oracle.quantize(np.ascontiguousarray(x_bits[rows_done:rows_done + chunk]),
                                           oracle.E4M3, (0, 0))
        tq += time.perf_counter() - t0
        rows_done += chunk
    quant_full_s = t_amax + tq * (M / rows_done)
    npts, tg = 0, 0.0
    while tg < budget_s * 0.75:
        m = g.integers(0, xq.shape[0], 256)
        n = g.integers(0, wq.shape[0], 256)
        t0 = time.perf_counter()
        oracle.gemm_points(xq, oracle.E4M3, s_x, (0, 0), wq, oracle.E4M3, s_w, (0, 0), m, n)
        tg += time.perf_counter() - t0
        npts += 256
    gemm_full_s = tg / npts * M * N
    step_s = quant_full_s + gemm_full_s
    return {"value": 2.0 * M * N * K / step_s / 1e12, "unit": "TFLOP/s", "cores": 1,
            "kind": "oracle",
            "sample": ("oracle amax of all of X (%.2f s), cast of %d of %d X rows (%.2f s) and %d "
                       "GEMM dot products of K=%d (%.2f s), extrapolated to one full step: %.1f s"
                       % (t_amax, rows_done, M, tq, npts, K, tg, step_s))}


def bench_prefill(args, torch, rt, wl):
    M, N, K = 4096, 29568, 8192
    w = wl.C3Prefill()
    t0 = time.time()
    x_bits = w.make_x()
    w_bits = w.make_w()
    print("inputs generated in %.1f s" % (time.time() - t0), file=sys.stderr, flush=True)
    from_bits = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    x = from_bits(x_bits)
    W = from_bits(w_bits)
    dev = "cuda"
    # setup (untimed): static weight scale from W's own amax, weight codes
    aw = torch.empty((1, 1), device=dev)
    rt.fp8_amax(W, (0, 0), aw)
    s_w = torch.empty((1, 1), device=dev)
    r_w = torch.empty((1, 1), device=dev)
    rt.fp8_compute_scale(aw, rt.E4M3, 1e-12, False, s_w, r_w)
    Wq = torch.empty((N, K), dtype=torch.uint8, device=dev)
    cnt_w = torch.zeros(2, dtype=torch.int64, device=dev)
    am_w = torch.empty((1, 1), device=dev)
    xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
    s_x = torch.empty((1, 1), device=dev)
    r_x = torch.empty((1, 1), device=dev)
    am_x = torch.empty((1, 1), device=dev)
    cnt = torch.zeros(2, dtype=torch.int64, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    timer = Timer(torch)

    def quant_w():
        rt.fp8_quantize(W, (0, 0), rt.E4M3, rt.GIVEN, 1e-12, False, s_w, r_w, Wq, am_w, cnt_w)

    def step(timed):
        if timed:
            timer.start("quant_x")
        rt.fp8_quantize(x, (0, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, s_x, r_x, xq, am_x, cnt)
        if timed:
            timer.stop("quant_x")
            timer.start("gemm")
        rt.fp8_scaled_gemm(xq, rt.E4M3, (0, 0), s_x, Wq, rt.E4M3, (0, 0), s_w, y)
        if timed:
            timer.stop("gemm")

    # the same GEMM with the output requantized to E4M3 in the epilogue (an
    # output scale given, as a delayed scale would be), amax of Y and counters
    s_y = torch.full((1, 1), 0.05, device=dev)
    am_y = torch.empty((1, 1), device=dev)
    cnt_y = torch.zeros(2, dtype=torch.int64, device=dev)
    yq = torch.empty((M, N), dtype=torch.uint8, device=dev)

    def gemm_fp8out():
        rt.fp8_scaled_gemm_fp8out(xq, rt.E4M3, (0, 0), s_x, Wq, rt.E4M3, (0, 0), s_w, yq, rt.E4M3, s_y, None,
                                  am_y, cnt_y)

    quant_w()
    for _ in range(3):
        timer.start("quant_w")
        quant_w()
        timer.stop("quant_w")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        step(True)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = ev0.elapsed_time(ev1)
    ms_step = total_ms / args.steps
    gemm_fp8out()
    for _ in range(3):
        timer.start("gemm_fp8out")
        gemm_fp8out()
        timer.stop("gemm_fp8out")
    torch.cuda.synchronize()
    go_ms = float(np.mean(timer.ms("gemm_fp8out")))
    fp8out = mfma_entry(go_ms * 1e3, 2.0 * M * N * K, M * K + N * K + M * N + 8)
    fp8out["kernels"] = "k_gemm_big (E4M3 out) + k_split_reduce (last wave) + k_finish"
    q_ms = float(np.mean(timer.ms("quant_x")))
    g_ms = float(np.mean(timer.ms("gemm")))
    qw_ms = float(np.mean(timer.ms("quant_w")))
    flops = 2.0 * M * N * K
    # algorithmic bytes: X read once (bf16) + codes written once + scale
    q_bytes = M * K * 2 + M * K * 1 + 4
    qw_bytes = N * K * 2 + N * K * 1 + 4
    g_bytes = M * K + N * K + M * N * 2 + 8
    g_tflops = flops / (g_ms * 1e-3) / 1e12
    sat = cnt.cpu().tolist()
    out = {
        "metric": METRIC, "value": flops / (ms_step * 1e-3) / 1e12, "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3",
        "data": "synthetic (seeded Philox; X = 0.5*t(3), W ~ N(0,0.02))",
        "config": {"workload": "prefill MLP up-projection: X[4096x8192] bf16 per-tensor dynamic "
                               "E4M3 x W[29568x8192] bf16 per-tensor static E4M3 -> Y bf16",
                   "M": M, "N": N, "K": K},
        "roofline": {"bound": "mfma", "achieved": g_tflops, "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": g_tflops / FP8_PEAK_TFLOPS,
                     "traffic": traffic_from_profile("gemm_prefill_traffic.json"),
                     "kernel": "k_gemm_big + k_split_reduce (one GEMM call: fp8 E4M3xE4M3, per-tensor scales, bf16 out)",
                     "avg_launch_us": g_ms * 1e3},
        "components": {
            "quantize_x_dynamic_per_tensor": {
                "us": q_ms * 1e3, "p95_us": float(np.percentile(timer.ms("quant_x"), 95)) * 1e3,
                "GB_s": q_bytes / (q_ms * 1e-3) / 1e9,
                "frac_hbm": q_bytes / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "algorithmic_bytes": q_bytes, "kernels": "k_tensor_amax + k_tensor_cast + k_finish"},
            "gemm": {"us": g_ms * 1e3, "p95_us": float(np.percentile(timer.ms("gemm"), 95)) * 1e3,
                     "TFLOP_s": g_tflops, "frac_fp8_peak": g_tflops / FP8_PEAK_TFLOPS,
                     "algorithmic_bytes": g_bytes},
            "quantize_w_given_per_tensor": {
                "us": qw_ms * 1e3, "GB_s": qw_bytes / (qw_ms * 1e-3) / 1e9,
                "frac_hbm": qw_bytes / (qw_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "algorithmic_bytes": qw_bytes},
            "gemm_fp8_out_e4m3": fp8out,
            "quant_over_gemm": q_ms / g_ms,
            "quant_over_gemm_context": "T(amax + scale + cast of X, with counters) / T(GEMM) on the prefill "
                                       "shape; the pages state under 0.5% on Hopper",
            "x_saturated_underflowed": sat,
        },
        "wall_s_timed": wall,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_prefill(x_bits, w_bits, M, N, K, args.cpu_seconds)
    return out


class Timing(float):
    """Median microseconds, carrying the 95th percentile as .p95."""

    def __new__(cls, med, p95):
        t = super().__new__(cls, med)
        t.p95 = p95
        return t


def time_op(torch, fn, reps=20, warmup=3, scrub=None):
    """Median and 95th percentile (linear interpolation) of fn() over reps
    event-timed runs on the current stream after warmup untimed calls; scrub
    (untimed) runs before each repeat to evict the caches."""
    for _ in range(warmup):
        fn()
    out = []
    for _ in range(reps):
        if scrub is not None:
            scrub()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        out.append(e0.elapsed_time(e1) * 1e3)
    return Timing(float(np.median(out)), float(np.percentile(out, 95)))


def hbm_entry(us, nbytes, kernels):
    gbs = nbytes / (us * 1e-6) / 1e9
    e = {"us": float(us), "GB_s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS, "algorithmic_bytes": nbytes,
         "kernels": kernels}
    if hasattr(us, "p95"):
        e["p95_us"] = us.p95
    return e


def mfma_entry(us, flops, nbytes):
    tf = flops / (us * 1e-6) / 1e12
    e = {"us": float(us), "TFLOP_s": tf, "frac_fp8_peak": tf / FP8_PEAK_TFLOPS, "algorithmic_bytes": nbytes}
    if hasattr(us, "p95"):
        e["p95_us"] = us.p95
    return e


def recipe_staleness(torch, rt, wl):
    """The delayed-scaling workload's 32-step sequence (spike included) at
    256 x 8192, quantized to E5M2 under each recipe: current scaling, and
    delayed scaling from the 16-entry history with the window maximum or the
    latest amax, with margins.  Per recipe: saturated and underflowed
    elements over the sequence, steps with any saturation, and the relative
    error energy sum_t sum e^2 / sum_t sum g^2 of the restored tensors."""
    dev = "cuda"
    c = wl.C4Delayed(M=256)
    gs = [torch.from_numpy(c.make_g(t).view(np.int16)).view(torch.bfloat16).to(dev) for t in range(c.steps)]
    _, spikes = c.sigmas()
    M, K = c.M, c.K
    recipes = [("current", None, 0), ("window_max", rt.HIST_MAX, 0), ("latest", rt.HIST_LATEST, 0),
               ("window_max_margin1", rt.HIST_MAX, 1), ("window_max_margin2", rt.HIST_MAX, 2)]
    out = {"workload": "delayed E5M2, %d steps of %dx%d bf16, spike x100 at step(s) %s, history %d"
                       % (c.steps, M, K, [int(x) for x in spikes], c.history)}
    q = torch.empty((M, K), dtype=torch.uint8, device=dev)
    s, r, am = (torch.empty((1, 1), dtype=torch.float32, device=dev) for _ in range(3))
    cnt = torch.zeros(2, dtype=torch.int64, device=dev)
    st = torch.empty(7, dtype=torch.float64, device=dev)
    for name, fn, margin in recipes:
        hist = torch.zeros(c.history, dtype=torch.float32, device=dev)
        head = torch.zeros(1, dtype=torch.int32, device=dev)
        sat = und = sat_steps = 0
        se = sg = 0.0
        for t, g in enumerate(gs):
            mode = rt.DYNAMIC if (fn is None or t == 0) else rt.GIVEN  # step 0: cold start
            rt.fp8_quantize(g, (0, 0), rt.E5M2, mode, 1e-12, False, s, r, q, am, cnt)
            rt.fp8_quant_error(g, q, rt.E5M2, (0, 0), s, st)
            if fn is not None:
                rt.fp8_delayed_scale_update(hist, head, am, rt.E5M2, fn, margin, 1e-12, False, s, r)
            cn, sv = cnt.tolist(), st.tolist()
            sat, und, sat_steps = sat + cn[0], und + cn[1], sat_steps + (cn[0] > 0)
            se, sg = se + sv[0], sg + sv[1]
        out[name] = {"saturated": sat, "underflowed": und, "steps_with_saturation": sat_steps,
                     "relative_error_energy": se / sg}
    return out


def extra_components(torch, rt, wl):
    """Quantize and GEMM kernels of the other workload shapes, each timed alone
    (3 untimed calls, then median and 95th percentile of 20, caches scrubbed
    between repeats by a 1 GiB fill)."""
    dev = "cuda"
    junk = torch.empty(2**28, dtype=torch.float32, device=dev)
    scrub = lambda: junk.fill_(1.0)
    from_bits = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
    u8 = lambda *shape: torch.empty(shape, dtype=torch.uint8, device=dev)
    comp = {}

    # decode-shaped linear: A 16x8192 per token, W 8192x8192 per output channel, bias, bf16 out
    c2 = wl.C2Decode()
    d = c2.make()
    M, N, K = c2.M, c2.N, c2.K
    A, W, bias = from_bits(d["a"]), from_bits(d["w"]), from_bits(d["bias"])
    Aq, Wq = u8(M, K), u8(N, K)
    sa, ra, sw, rw = f32(M, 1), f32(M, 1), f32(N, 1), f32(N, 1)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    qa = lambda: rt.fp8_quantize(A, (1, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, sa, ra, Aq)
    qw = lambda: rt.fp8_quantize(W, (1, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, sw, rw, Wq)
    gm = lambda: rt.fp8_scaled_gemm(Aq, rt.E4M3, (1, 0), sa, Wq, rt.E4M3, (1, 0), sw, y, bias=bias)
    qa(); qw()
    comp["decode_quantize_a_per_token"] = hbm_entry(time_op(torch, qa, scrub=scrub), M * K * 3 + M * 4,
                                                     "k_rowgroups")
    comp["decode_quantize_w_per_channel"] = hbm_entry(time_op(torch, qw, scrub=scrub), N * K * 3 + N * 4,
                                                       "k_rowgroups")
    g_bytes = M * K + N * K + M * N * 2 + (M + N) * 4 + N * 2
    e = hbm_entry(time_op(torch, gm, scrub=scrub), g_bytes, "k_gemm_skinny")
    e["TFLOP_s"] = 2.0 * M * N * K / (e["us"] * 1e-6) / 1e12
    comp["decode_gemm_bf16_bias"] = e
    # weight-only FP8: the same per-channel E4M3 weight codes, bf16 activations
    yw = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    wo = lambda: rt.fp8_weight_only_gemm(A, Wq, rt.E4M3, (1, 0), sw, yw, bias=bias)
    wo()
    wo_bytes = M * K * 2 + N * K + M * N * 2 + N * 4 + N * 2
    e = hbm_entry(time_op(torch, wo, scrub=scrub), wo_bytes, "k_gemm_wonly")
    e["TFLOP_s"] = 2.0 * M * N * K / (e["us"] * 1e-6) / 1e12
    comp["decode_weight_only_gemm_bf16_bias"] = e
    # the same two GEMMs on the fragment-ordered image of the weight codes
    # (packed once, as a weight is laid out offline; the pack is timed alone)
    P = rt.fp8_pack_weights16(Wq)
    pk = lambda: rt.fp8_pack_weights16(Wq, out=P.data)
    comp["decode_pack_weights16"] = hbm_entry(time_op(torch, pk, scrub=scrub), 2 * N * K, "k_pack_weights16")
    gmp = lambda: rt.fp8_scaled_gemm(Aq, rt.E4M3, (1, 0), sa, P, rt.E4M3, (1, 0), sw, y, bias=bias)
    gmp()
    e = hbm_entry(time_op(torch, gmp, scrub=scrub), g_bytes, "k_gemm_skinny (packed B)")
    e["TFLOP_s"] = 2.0 * M * N * K / (e["us"] * 1e-6) / 1e12
    comp["decode_gemm_bf16_bias_packed_w"] = e
    wop = lambda: rt.fp8_weight_only_gemm(A, P, rt.E4M3, (1, 0), sw, yw, bias=bias)
    wop()
    e = hbm_entry(time_op(torch, wop, scrub=scrub), wo_bytes, "k_gemm_wonly (packed W)")
    e["TFLOP_s"] = 2.0 * M * N * K / (e["us"] * 1e-6) / 1e12
    comp["decode_weight_only_gemm_bf16_bias_packed_w"] = e
    # one decode step (per-token quantize of A, then the GEMM on the weight
    # image: two launches), eager and as a replayed HIP graph, on a stream of
    # its own that holds the library's workspace before capture
    gs = torch.cuda.Stream()
    dstep = lambda: (qa(), gmp())
    with torch.cuda.stream(gs):
        dstep()
    gs.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=gs):
        dstep()
    step_bytes = M * K * 3 + M * 4 + g_bytes
    with torch.cuda.stream(gs):
        comp["decode_step_packed_eager"] = hbm_entry(time_op(torch, dstep, scrub=scrub), step_bytes,
                                                     "k_rowgroups + k_gemm_skinny (packed B)")
        comp["decode_step_packed_hip_graph"] = hbm_entry(time_op(torch, graph.replay, scrub=scrub), step_bytes,
                                                         "the same two kernels, one graph replay")
    gs.synchronize()
    del P, graph
    # granularity ledger: error statistics of the per-channel weight codes
    # against the bf16 weight, with the 16 activation rows
    stats = torch.empty(7, dtype=torch.float64, device=dev)
    le = lambda: rt.fp8_quant_error(W, Wq, rt.E4M3, (1, 0), sw, stats, x=A)
    le()
    e = hbm_entry(time_op(torch, le, scrub=scrub), N * K * 3 + N * 4 + M * K * 2, "k_quant_error + k_ledger_finish")
    e["TFLOP_s"] = 4.0 * M * N * K / (e["us"] * 1e-6) / 1e12  # x.e and x.w per (m, n, k)
    comp["ledger_quant_error_w_per_channel_x16"] = e
    # the ledger itself at this weight: scale metadata against error per granularity
    specs = [((0, 0), 0), ((1, 0), 0), ((1, 128), 0), ((128, 128), 0), ((1, 32), 1)]
    rows = rt.fp8_granularity_ledger(W, rt.E4M3, specs, x=A)
    ledger = {}
    for r in rows:
        key = "%dx%d%s" % (r["gran"][0], r["gran"][1], "_pow2" if r["pow2_round_up"] else "")
        ledger[key] = {k: r[k] for k in ("qparam_count", "qparam_bytes", "total_state_bytes", "weight_mse",
                                         "weight_max_abs_err", "output_mse", "output_cosine", "saturated",
                                         "underflowed")}
    comp["granularity_ledger_decode_w_e4m3"] = ledger
    del A, W, bias, Aq, Wq, y, yw, d, stats

    # delayed-scaling backward GEMM, one step: G 8192x8192 E5M2 with the scale of
    # the history window, W 8192x8192 E4M3 per tensor, fp32 out
    c4 = wl.C4Delayed()
    M, N, K = c4.M, c4.N, c4.K
    G = from_bits(c4.make_g(1))
    W = from_bits(c4.make_w())
    Gq, Wq = u8(M, K), u8(N, K)
    hist = torch.zeros(c4.history, dtype=torch.float32, device=dev)
    head = torch.zeros(1, dtype=torch.int32, device=dev)
    sg, rg, am, sw, rw = f32(1, 1), f32(1, 1), f32(1, 1), f32(1, 1), f32(1, 1)
    cnt = torch.zeros(2, dtype=torch.int64, device=dev)
    rt.fp8_quantize(G, (0, 0), rt.E5M2, rt.DYNAMIC, 1e-12, False, sg, rg, Gq, am, cnt)
    rt.fp8_amax_history_update(hist, head, am, rt.E5M2, 1e-12, False, sg, rg)
    rt.fp8_quantize(W, (0, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, sw, rw, Wq)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    qg = lambda: rt.fp8_quantize(G, (0, 0), rt.E5M2, rt.GIVEN, 1e-12, False, sg, rg, Gq, am, cnt)
    hu = lambda: rt.fp8_amax_history_update(hist, head, am, rt.E5M2, 1e-12, False, sg, rg)
    gm = lambda: rt.fp8_scaled_gemm(Gq, rt.E5M2, (0, 0), sg, Wq, rt.E4M3, (0, 0), sw, y)
    comp["delayed_quantize_g_given_e5m2"] = hbm_entry(time_op(torch, qg, scrub=scrub), M * K * 3 + 4,
                                                       "k_tensor_cast (given, amax + counts) + k_finish")
    comp["delayed_history_update_us"] = float(time_op(torch, hu))
    comp["delayed_gemm_e5m2_e4m3_f32"] = mfma_entry(time_op(torch, gm, scrub=scrub), 2.0 * M * N * K,
                                                    M * K + N * K + M * N * 4 + 8)
    # cast-transpose of the same G (the backward reads it in both orientations):
    # codes row-major and K-major in one pass, per-tensor GIVEN (+ amax, counters),
    # and per-column DYNAMIC (column amax pass, scales, then the pass)
    Gt = u8(K, M)
    ct = lambda: rt.fp8_quantize_transpose(G, (0, 0), rt.E5M2, rt.GIVEN, 1e-12, False, sg, rg, Gq, Gt, am, cnt)
    comp["cast_transpose_g_e5m2_given"] = hbm_entry(time_op(torch, ct, scrub=scrub), M * K * 4 + 4,
                                                    "k_cast_transpose + k_finish")
    sgc, rgc = f32(1, K), f32(1, K)
    ctc = lambda: rt.fp8_quantize_transpose(G, (0, 1), rt.E5M2, rt.DYNAMIC, 1e-12, False, sgc, rgc, Gq, Gt)
    comp["cast_transpose_g_e5m2_per_column_dynamic"] = hbm_entry(
        time_op(torch, ctc, scrub=scrub), M * K * 4 + K * 8,
        "k_col_amax + k_col_amax_finish + k_compute_scale + k_cast_transpose")
    del G, W, Gq, Wq, y, Gt

    # block-scaled GEMM: A 1x128 groups, W 128x128 blocks, bf16 out; variant 1x32 power-of-two
    c5 = wl.C5Block()
    M, N, K = c5.M, c5.N, c5.K
    A = from_bits(c5.make_a())
    W = from_bits(c5.make_w())
    Aq, Wq = u8(M, K), u8(N, K)
    sa, sw = f32(M, K // 128), f32(N // 128, K // 128)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    qa = lambda: rt.fp8_quantize(A, (1, 128), rt.E4M3, rt.DYNAMIC, 1e-12, False, sa, None, Aq)
    qw = lambda: rt.fp8_quantize(W, (128, 128), rt.E4M3, rt.DYNAMIC, 1e-12, False, sw, None, Wq)
    gm = lambda: rt.fp8_scaled_gemm(Aq, rt.E4M3, (1, 128), sa, Wq, rt.E4M3, (128, 128), sw, y)
    qa(); qw()
    comp["block_quantize_a_1x128"] = hbm_entry(time_op(torch, qa, scrub=scrub),
                                               M * K * 3 + sa.numel() * 4, "k_rowgroups")
    comp["block_quantize_w_128x128"] = hbm_entry(time_op(torch, qw, scrub=scrub),
                                                 N * K * 3 + sw.numel() * 4, "k_blocktile")
    comp["block_gemm_bf16"] = mfma_entry(time_op(torch, gm, scrub=scrub), 2.0 * M * N * K,
                                         M * K + N * K + M * N * 2 + (sa.numel() + sw.numel()) * 4)
    sa32, sw32 = f32(M, K // 32), f32(N, K // 32)
    qa = lambda: rt.fp8_quantize(A, (1, 32), rt.E4M3, rt.DYNAMIC, 1e-12, True, sa32, None, Aq)
    qw = lambda: rt.fp8_quantize(W, (1, 32), rt.E4M3, rt.DYNAMIC, 1e-12, True, sw32, None, Wq)
    gm = lambda: rt.fp8_scaled_gemm(Aq, rt.E4M3, (1, 32), sa32, Wq, rt.E4M3, (1, 32), sw32, y,
                                    flags=rt.POW2_SCALES)
    qa(); qw()
    comp["block_mx_quantize_a_1x32_pow2"] = hbm_entry(time_op(torch, qa, scrub=scrub),
                                                      M * K * 3 + sa32.numel() * 4, "k_rowgroups")
    comp["block_mx_gemm_bf16"] = mfma_entry(time_op(torch, gm, scrub=scrub), 2.0 * M * N * K,
                                            M * K + N * K + M * N * 2 + (sa32.numel() + sw32.numel()) * 4)
    del A, W, Aq, Wq, y, junk
    torch.cuda.empty_cache()
    return comp


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the FP8 chain is measured on a single MI355X "
              "(multi-GPU sharding is described, not built).", file=sys.stderr)
        sys.exit(2)
    import torch

    import dynamic_scaling_scaled_amd as rt
    import workloads as wl

    rt.lib()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        src = torch.ones(2**28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4,
                          "repeats": 3}), flush=True)
        return
    out = bench_prefill(args, torch, rt, wl)
    if not args.no_extra:
        out["components"].update(extra_components(torch, rt, wl))
        out["delayed_recipe_staleness"] = recipe_staleness(torch, rt, wl)
        fr = [v["frac_hbm"] for k, v in out["components"].items()
              if isinstance(v, dict) and "frac_hbm" in v and "quantize" in k and "decode_quantize_a" not in k]
        out["components"]["quantize_min_frac_hbm_large"] = min(fr)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
