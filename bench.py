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
    p.add_argument("--calibrate-mfma", action="store_true",
                   help="run only the register-only FP8 MFMA rate (32x32x64 and 16x16x128, zero and random "
                        "operands): the matrix cores' ceiling at the clock the chip holds for them")
    p.add_argument("--library-comparison", action="store_true",
                   help="run only a comparison of fp8_scaled_gemm with hipBLASLt (torch._scaled_mm) on "
                        "identical E4M3 codes and per-tensor scales at the large shapes, bf16 out")
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


def host_cpu():
    """CPU model and the logical CPUs this process may run on (capped at 16,
    the host share of one GPU on a shared node)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count() or 1
    return model, avail, max(1, min(16, avail))


def pick(n, k, seed):
    return np.sort(np.random.default_rng(seed).choice(n, size=min(k, n), replace=False))


def gather(torch, t, rows, cols=None):
    """Host copy of t[rows][:, cols] (or whole rows)."""
    r = torch.as_tensor(rows, device=t.device, dtype=torch.long)
    v = t.index_select(0, r)
    if cols is not None:
        v = v.index_select(1, torch.as_tensor(cols, device=t.device, dtype=torch.long))
    v = v.cpu()
    if v.dtype == torch.bfloat16:
        return v.view(torch.int16).numpy().view(np.uint16)
    return v.numpy()


def oracle_prefill_sample(oracle, x_bits, w_bits, M, N, K, budget_s, threads, plan=None):
    """One sample of the prefill step on the oracle, on `threads` host threads
    (the oracle's C calls run without the GIL, each on its own row range or
    point batch): the full amax of X, the cast of a sample of X rows under the
    resulting scale, and GEMM dot products between those rows and a sample of
    W rows.  With plan=None the sample grows until budget_s seconds (a quarter
    for the cast, the rest for the GEMM); otherwise the same amounts as plan.
    Returns (seconds for amax, rows cast, cast seconds, dot products, GEMM
    seconds, the amounts as a plan)."""
    import concurrent.futures as cf

    g = np.random.default_rng(7)
    w_rows = np.sort(g.choice(N, size=256, replace=False))
    s_w, _ = oracle.compute_scale(oracle.amax(w_bits), oracle.E4M3)  # untimed setup
    wq, _, _, _, _ = oracle.quantize(np.ascontiguousarray(w_bits[w_rows]), oracle.E4M3, (0, 0),
                                     mode=oracle.GIVEN, scale=s_w)
    ex = cf.ThreadPoolExecutor(threads)
    bounds = np.linspace(0, M, threads + 1).astype(int)
    t0 = time.perf_counter()
    parts = list(ex.map(lambda i: oracle.amax(x_bits[bounds[i]:bounds[i + 1]]), range(threads)))
    a_x = np.max(np.array(parts, np.float32))
    s_x, r_x = oracle.compute_scale(np.array([[a_x]], np.float32), oracle.E4M3)
    t_amax = time.perf_counter() - t0
    chunk = 64

    def cast(r0):
        return oracle.quantize(np.ascontiguousarray(x_bits[r0:r0 + chunk]), oracle.E4M3, (0, 0),
                               mode=oracle.GIVEN, scale=s_x, inv_scale=r_x)[0]

    rows_done, tq, xq = 0, 0.0, []
    while (rows_done < plan[0] if plan else tq < budget_s * 0.25) and rows_done + chunk * threads <= M:
        t0 = time.perf_counter()
        xq += list(ex.map(cast, range(rows_done, rows_done + chunk * threads, chunk)))
        tq += time.perf_counter() - t0
        rows_done += chunk * threads
    xq = np.concatenate(xq)
    npts, tg, batch = 0, 0.0, 256

    def dots(seed):
        gi = np.random.default_rng(seed)
        m, n = gi.integers(0, xq.shape[0], batch), gi.integers(0, wq.shape[0], batch)
        oracle.gemm_points(xq, oracle.E4M3, s_x, (0, 0), wq, oracle.E4M3, s_w, (0, 0), m, n)

    while npts < plan[1] if plan else tg < budget_s * 0.75:
        t0 = time.perf_counter()
        list(ex.map(dots, range(npts, npts + batch * threads, batch)))
        tg += time.perf_counter() - t0
        npts += batch * threads
    ex.shutdown()
    return t_amax, rows_done, tq, npts, tg, (rows_done, npts)


def cpu_baseline_prefill(x_bits, w_bits, M, N, K, budget_s):
    """The oracle as it stands (never tuned for speed) on a bounded sample of
    the prefill step, extrapolated to one full step (TFLOP/s of the step):
    first on one thread with about budget_s seconds of work, then the same
    sample on all the host threads this process may use.  All oracle inputs
    come from the seeded generators and the oracle itself."""
    import oracle

    oracle.build(force=False)
    model, avail, threads = host_cpu()
    res = {}
    plan = None
    for nt in (1, threads):
        t_amax, rows, tq, npts, tg, plan = oracle_prefill_sample(oracle, x_bits, w_bits, M, N, K, budget_s,
                                                                 nt, plan)
        step_s = t_amax + tq * (M / rows) + tg / npts * M * N
        res[nt] = {"value": 2.0 * M * N * K / step_s / 1e12, "unit": "TFLOP/s", "cores": nt,
                   "kind": "oracle",
                   "sample": ("oracle on %d thread(s): amax of all of X (%.2f s), cast of %d of %d X rows "
                              "(%.2f s), %d GEMM dot products of K=%d (%.2f s); extrapolated to one full "
                              "step: %.1f s" % (nt, t_amax, rows, M, tq, npts, K, tg, step_s))}
    out = dict(res[threads])
    out["cpu_model"] = model
    out["logical_cpus_available"] = avail
    out["single_thread"] = res[1]
    return out


def _pool_map(threads, fn, items):
    import concurrent.futures as cf

    with cf.ThreadPoolExecutor(threads) as ex:
        return list(ex.map(fn, items))


def _row_chunks(rows, threads):
    b = np.linspace(0, rows, threads * 4 + 1).astype(int)
    return [(b[i], b[i + 1]) for i in range(len(b) - 1) if b[i + 1] > b[i]]


def oracle_tensor_scale(oracle, x, fmt, threads):
    """Per-tensor amax (exact: max of row-range maxima) and (s, r) of x."""
    parts = _pool_map(threads, lambda r: oracle.amax(x[r[0]:r[1]]), _row_chunks(x.shape[0], threads))
    a = np.max(np.array(parts, np.float32)).reshape(1, 1)
    s, r = oracle.compute_scale(a, fmt)
    return a, s, r


def oracle_given_counts(oracle, x, fmt, s, r, threads):
    """Saturation / underflow counts of the GIVEN-mode cast of all of x (row
    ranges on threads; the counts add up exactly)."""
    parts = _pool_map(threads, lambda rr: oracle.quantize(np.ascontiguousarray(x[rr[0]:rr[1]]), fmt, (0, 0),
                                                          mode=oracle.GIVEN, scale=s, inv_scale=r)[4],
                      _row_chunks(x.shape[0], threads))
    return np.sum(np.array(parts, np.uint64), axis=0)


def _same(a, b):
    a, b = np.asarray(a), np.asarray(b)
    if a.shape != b.shape:
        return False
    if a.dtype == np.float32 or b.dtype == np.float32:
        a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
        na, nb = np.isnan(a), np.isnan(b)
        return bool(np.array_equal(na, nb) and np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32)))
    return bool(np.array_equal(a, b))


def _gemm_stats(oracle, y_gpu, aq, fa, sa, ga, bq, fb, sb, gb, out_bf16, bias=None):
    """The parity tests' per-element GEMM rule on every (row of aq, row of bq)
    pair: stats of |y - y_ref| against 1e-5 S and 1e-5 S + T_hw."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_helpers import check_gemm

    Ma, Nb = aq.shape[0], bq.shape[0]
    m, n = np.repeat(np.arange(Ma), Nb), np.tile(np.arange(Nb), Ma)
    yref, S = oracle.gemm_points(aq, fa, sa, ga, bq, fb, sb, gb, m, n, bias=bias)
    thw = oracle.dot_truncation_bound(aq, fa, sa, ga, bq, fb, sb, gb, m, n)
    bias_f = None if bias is None else oracle.bf16_bits_to_f32(bias)[n]
    ok, st = check_gemm(np.asarray(y_gpu).reshape(-1), yref, S, out_bf16, oracle, bias=bias_f, t_hw=thw)
    st["within_tolerance"] = ok
    return st


def parity_leg(oracle, keep, threads):
    """The oracle on the inputs of every workload the benchmark ran, compared
    with what the GPU produced at full size: per-tensor amax and scales over
    the whole tensors, codes of sampled rows, saturation / underflow counts
    over whole tensors, every step of the delayed chain, and the GEMM on all
    pairs of sampled rows under the parity tests' rule.  Bit-exact items are
    reported as true / false; GEMM items as the largest |y - y_ref| / S and
    the count above 1e-5 S."""
    E4, E5 = oracle.E4M3, oracle.E5M2
    out = {}
    if "tiny" in keep:
        k = keep["tiny"]
        xq, sx, rx, ax, cx = oracle.quantize(k["x"], E4, (0, 0))
        wq, sw, _, _, _ = oracle.quantize(k["w"], E4, (1, 0))
        M = k["y"].shape[0]
        exact = (_same(xq, k["xq"]) and _same(sx, k["s_x"]) and _same(rx, k["r_x"]) and _same(ax, k["am_x"])
                 and _same(cx.astype(np.int64), k["cnt_x"]) and _same(wq, k["wq"]) and _same(sw, k["s_w"]))
        out["tiny"] = {"codes_scales_counts_bit_exact": exact,
                       "gemm_f32_all_outputs": _gemm_stats(oracle, k["y"], xq[:M], E4, sx, (0, 0), wq, E4, sw,
                                                           (1, 0), False)}
    if "decode" in keep:
        k = keep["decode"]
        aq, sa, ra, _, _ = oracle.quantize(k["a_bits"], E4, (1, 0))
        wq, sw, rw, _, _ = oracle.quantize(k["w_rows"], E4, (1, 0))
        exact = (_same(aq, k["aq"]) and _same(sa, k["s_a"]) and _same(ra, k["r_a"]) and _same(wq, k["wq"])
                 and _same(sw, k["s_w"]) and _same(rw, k["r_w"]))
        out["decode"] = {"codes_scales_bit_exact": exact, "sample": "all 16 A rows x 256 W rows",
                         "gemm_bf16_bias": _gemm_stats(oracle, k["y"], aq, E4, sa, (1, 0), wq, E4, sw, (1, 0), True,
                                                       bias=k["bias"][k["rows_b"]])}
    if "prefill" in keep:
        k = keep["prefill"]
        ax, sx, rx = oracle_tensor_scale(oracle, k["x_bits"], E4, threads)
        cx = oracle_given_counts(oracle, k["x_bits"], E4, sx, rx, threads)
        aw, sw, rw = oracle_tensor_scale(oracle, k["w_bits"], E4, threads)
        cw = oracle_given_counts(oracle, k["w_bits"], E4, sw, rw, threads)
        xq = oracle.quantize(np.ascontiguousarray(k["x_bits"][k["rows_a"]]), E4, (0, 0), mode=oracle.GIVEN,
                             scale=sx, inv_scale=rx)[0]
        wq = oracle.quantize(np.ascontiguousarray(k["w_bits"][k["rows_b"]]), E4, (0, 0), mode=oracle.GIVEN,
                             scale=sw, inv_scale=rw)[0]
        exact = (_same(ax, k["am_x"]) and _same(sx, k["s_x"]) and _same(rx, k["r_x"])
                 and _same(cx.astype(np.int64), k["cnt_x"]) and _same(xq, k["xq"]) and _same(aw, k["am_w"])
                 and _same(sw, k["s_w"]) and _same(rw, k["r_w"]) and _same(cw.astype(np.int64), k["cnt_w"])
                 and _same(wq, k["wq"]))
        out["prefill"] = {"amax_scales_counts_bit_exact_whole_tensors_codes_sampled_rows": exact,
                          "sample": "64 X rows x 64 W rows",
                          "gemm_bf16": _gemm_stats(oracle, k["y"], xq, E4, sx, (0, 0), wq, E4, sw, (0, 0), True)}
    if "delayed" in keep:
        k = keep["delayed"]
        st = k["steps"]
        hist = np.zeros(16, np.float32)
        head, s_o, r_o = 0, None, None
        bad = []
        for t, g in enumerate(k["chain_g"]):
            a_t, s0, r0 = oracle_tensor_scale(oracle, g, E5, threads)
            if t == 0:
                s_o, r_o = s0[0, 0], r0[0, 0]
            s_arr, r_arr = np.array([[s_o]], np.float32), np.array([[r_o]], np.float32)
            cn = oracle_given_counts(oracle, g, E5, s_arr, r_arr, threads)
            if not (_same(np.float32(st["amax"][t]), a_t[0, 0]) and _same(np.float32(st["scale_used"][t]), s_o)
                    and [st["saturated"][t], st["underflowed"][t]] == cn.astype(np.int64).tolist()):
                bad.append(t)
            if t == len(k["chain_g"]) - 1:
                gq = oracle.quantize(np.ascontiguousarray(g[k["rows_a"]]), E5, (0, 0), mode=oracle.GIVEN,
                                     scale=s_arr, inv_scale=r_arr)[0]
            head, s_o, r_o = oracle.history_update(hist, head, float(a_t[0, 0]), E5)
        aw, sw, rw = oracle_tensor_scale(oracle, k["w_bits"], E4, threads)
        wq = oracle.quantize(np.ascontiguousarray(k["w_bits"][k["rows_b"]]), E4, (0, 0), mode=oracle.GIVEN,
                             scale=sw, inv_scale=rw)[0]
        out["delayed"] = {"steps_checked": len(k["chain_g"]), "steps_not_bit_exact": bad,
                          "last_step_codes_and_w_bit_exact": _same(gq, k["gq"]) and _same(wq, k["wq"])
                          and _same(sw, k["s_w"]) and _same(rw, k["r_w"]),
                          "sample": "amax, scale used and counts of every step over all of G_t; GEMM of the "
                                    "last step on 64 G rows x 64 W rows",
                          "gemm_f32_last_step": _gemm_stats(oracle, k["y"], gq, E5, np.float32(k["s_g"]).reshape(1, 1),
                                                            (0, 0), wq, E4, sw, (0, 0), False)}
    for name, ga, gb, pow2 in (("block", (1, 128), (128, 128), False), ("block_mx", (1, 32), (1, 32), True)):
        if name not in keep:
            continue
        k = keep[name]
        aq, sa, _, _, _ = oracle.quantize(k["a_rows"], E4, ga, pow2=pow2)
        wq, sw, _, _, _ = oracle.quantize(k["w_rows"], E4, gb, pow2=pow2)
        exact = _same(aq, k["aq"]) and _same(sa, k["s_a"]) and _same(wq, k["wq"]) and _same(sw, k["s_w"])
        out[name] = {"codes_scales_bit_exact": exact,
                     "sample": "64 A rows x %d W rows" % k["w_rows"].shape[0],
                     "gemm_bf16": _gemm_stats(oracle, k["y"], aq, E4, sa, ga, wq, E4, sw, gb, True)}
    return out


def bench_prefill(args, torch, rt, wl, keep):
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
    fp8out["kernels"] = "k_gemm_big16 (E4M3 out) + k_split_reduce (last wave) + k_finish"
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
                     "kernel": "k_gemm_big16 + k_split_reduce (one GEMM call: fp8 E4M3xE4M3, per-tensor scales, bf16 out)",
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
    # the practical streaming ceiling at the X quantize's size: a plain device
    # copy moving the same bytes (X read twice + codes written once = 168 MB,
    # as a 84 MB -> 84 MB copy), timed like the components (scrubbed, median of 20)
    moved_x = 2 * M * K * 2 + M * K
    junk = torch.empty(2**28, dtype=torch.float32, device=dev)
    src = torch.empty(moved_x // 2, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    copy_us = time_op(torch, lambda: dst.copy_(src), scrub=lambda: junk.fill_(1.0))
    qx = out["components"]["quantize_x_dynamic_per_tensor"]
    qx["moved_bytes"] = moved_x
    qx["moved_GB_s"] = moved_x / (q_ms * 1e-3) / 1e9
    qx["copy_same_bytes_GB_s"] = moved_x / (copy_us * 1e-6) / 1e9
    qx["frac_of_copy_rate"] = qx["moved_GB_s"] / qx["copy_same_bytes_GB_s"]
    qx["note"] = ("two passes by construction (X is read for amax, then again for the cast): 2 reads + 1 write; "
                  "the copy moves the same bytes with torch's device copy")
    # HBM bytes per call from the rocprofv3 FETCH_SIZE / WRITE_SIZE summary
    # (null once the kernels' source has changed since it was taken)
    qx["traffic"] = traffic_from_profile("quantize_x_prefill_traffic.json")
    del junk, src, dst
    # what the parity leg compares with the oracle: 64 rows of X and 64 rows of W
    ra, rb = pick(M, 64, 31), pick(N, 64, 32)
    keep["prefill"] = {"x_bits": x_bits, "w_bits": w_bits, "rows_a": ra, "rows_b": rb,
                       "xq": gather(torch, xq, ra), "wq": gather(torch, Wq, rb), "y": gather(torch, y, ra, rb),
                       "s_x": s_x.cpu().numpy(), "r_x": r_x.cpu().numpy(), "am_x": am_x.cpu().numpy(),
                       "cnt_x": cnt.cpu().numpy(), "s_w": s_w.cpu().numpy(), "r_w": r_w.cpu().numpy(),
                       "am_w": am_w.cpu().numpy(), "cnt_w": cnt_w.cpu().numpy()}
    del x, W, Wq, xq, y, yq
    torch.cuda.empty_cache()
    return out


def tiny_latency(torch, rt, wl, keep):
    """The tiny per-tensor workload end to end: dynamic E4M3 quantize of X
    (256 x 1024 fp32, with counters) and the GEMM X[0:64] W^T (K = 1024, fp32
    out, W per-channel codes from setup).  Launch-latency bound: absolute
    microseconds, warm (back to back) and with the caches scrubbed."""
    dev = "cuda"
    c = wl.C1Tiny()
    d = c.make()
    X = torch.from_numpy(d["x"]).to(dev)
    Wt = torch.from_numpy(d["w"]).to(dev)
    xq = torch.empty(X.shape, dtype=torch.uint8, device=dev)
    wq = torch.empty(Wt.shape, dtype=torch.uint8, device=dev)
    sx, rx, ax = (torch.empty((1, 1), device=dev) for _ in range(3))
    sw = torch.empty((c.N, 1), device=dev)
    cnt = torch.zeros(2, dtype=torch.int64, device=dev)
    y = torch.empty((c.M_gemm, c.N), device=dev)
    rt.fp8_quantize(Wt, (1, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, sw, None, wq)
    q = lambda: rt.fp8_quantize(X, (0, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, sx, rx, xq, ax, cnt)
    gm = lambda: rt.fp8_scaled_gemm(xq[:c.M_gemm], rt.E4M3, (0, 0), sx, wq, rt.E4M3, (1, 0), sw, y)
    step = lambda: (q(), gm())
    junk = torch.empty(2**26, dtype=torch.float32, device=dev)
    scrub = lambda: junk.fill_(1.0)
    out = {"workload": "X 256x1024 fp32 (4 entries +-400) per-tensor dynamic E4M3 -> GEMM 64x256x1024 "
                       "(W per-channel E4M3) -> fp32",
           "step_us_warm": float(time_op(torch, step, reps=200, warmup=10)),
           "step_us_scrubbed": float(time_op(torch, step, reps=50, warmup=3, scrub=scrub)),
           "quantize_us_warm": float(time_op(torch, q, reps=200, warmup=10)),
           "gemm_us_warm": float(time_op(torch, gm, reps=200, warmup=10)),
           "kernels": "k_tensor_amax + k_tensor_cast (counters added by atomics: a small grid); "
                      "k_gemm_skinny (exact products, a workgroup per 16-row tile of A)"}
    step()
    torch.cuda.synchronize()
    keep["tiny"] = {"x": d["x"], "w": d["w"], "xq": xq.cpu().numpy(), "wq": wq.cpu().numpy(),
                    "s_x": sx.cpu().numpy(), "r_x": rx.cpu().numpy(), "am_x": ax.cpu().numpy(),
                    "cnt_x": cnt.cpu().numpy(), "s_w": sw.cpu().numpy(), "y": y.cpu().numpy()}
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


def extra_components(torch, rt, wl, keep):
    """Quantize and GEMM kernels of the other workload shapes, each timed alone
    (3 untimed calls, then median and 95th percentile of 20, caches scrubbed
    between repeats by a 1 GiB fill); the delayed workload runs its 32-step
    chain.  keep: None, or a dict that receives what the parity leg checks."""
    check = keep is not None
    keep = keep if check else {}
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
                                                     "k_blocktile")
    comp["decode_quantize_w_per_channel"] = hbm_entry(time_op(torch, qw, scrub=scrub), N * K * 3 + N * 4,
                                                       "k_blocktile")
    g_bytes = M * K + N * K + M * N * 2 + (M + N) * 4 + N * 2
    e = hbm_entry(time_op(torch, gm, scrub=scrub), g_bytes, "k_gemm_skinny")
    e["TFLOP_s"] = 2.0 * M * N * K / (e["us"] * 1e-6) / 1e12
    comp["decode_gemm_bf16_bias"] = e
    # the same layer with an E4M3 output (GIVEN output scale, amax of y and counters)
    yq8 = u8(M, N)
    sy8 = torch.full((1, 1), 0.01, dtype=torch.float32, device=dev)
    amy, cnty = f32(1), torch.zeros(2, dtype=torch.int64, device=dev)
    g8 = lambda: rt.fp8_scaled_gemm_fp8out(Aq, rt.E4M3, (1, 0), sa, Wq, rt.E4M3, (1, 0), sw, yq8, rt.E4M3, sy8,
                                           None, amy, cnty, bias=bias)
    g8()
    e = hbm_entry(time_op(torch, g8, scrub=scrub), M * K + N * K + M * N + (M + N) * 4 + N * 2,
                  "k_gemm_skinny (E4M3 output) + k_finish")
    e["TFLOP_s"] = 2.0 * M * N * K / (e["us"] * 1e-6) / 1e12
    comp["decode_gemm_fp8_out_e4m3"] = e
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
    # or quantized straight into the image (one pass, no row-major codes)
    sw2 = f32(N, 1)
    qwp = lambda: rt.fp8_quantize_packed16(W, (1, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, sw2, None, out=P.data)
    qwp()
    comp["decode_quantize_w_per_channel_into_image"] = hbm_entry(time_op(torch, qwp, scrub=scrub),
                                                                  N * K * 3 + N * 4, "k_image_rows")
    gmp = lambda: rt.fp8_scaled_gemm(Aq, rt.E4M3, (1, 0), sa, P, rt.E4M3, (1, 0), sw, y, bias=bias)
    gmp()
    e = hbm_entry(time_op(torch, gmp, scrub=scrub), g_bytes, "k_gemm_skinny (packed B)")
    e["TFLOP_s"] = 2.0 * M * N * K / (e["us"] * 1e-6) / 1e12
    comp["decode_gemm_bf16_bias_packed_w"] = e
    g8p = lambda: rt.fp8_scaled_gemm_fp8out(Aq, rt.E4M3, (1, 0), sa, P, rt.E4M3, (1, 0), sw, yq8, rt.E4M3, sy8,
                                            None, amy, cnty, bias=bias)
    g8p()
    e = hbm_entry(time_op(torch, g8p, scrub=scrub), M * K + N * K + M * N + (M + N) * 4 + N * 2,
                  "k_gemm_skinny (packed B, E4M3 output) + k_finish")
    e["TFLOP_s"] = 2.0 * M * N * K / (e["us"] * 1e-6) / 1e12
    comp["decode_gemm_fp8_out_e4m3_packed_w"] = e
    wop = lambda: rt.fp8_weight_only_gemm(A, P, rt.E4M3, (1, 0), sw, yw, bias=bias)
    wop()
    e = hbm_entry(time_op(torch, wop, scrub=scrub), wo_bytes, "k_gemm_wonly (packed W)")
    e["TFLOP_s"] = 2.0 * M * N * K / (e["us"] * 1e-6) / 1e12
    comp["decode_weight_only_gemm_bf16_bias_packed_w"] = e
    # block-scaled decode: 1x128 token groups on A, 128x128 blocks on W (the
    # same bf16 operands), on the weight image
    Aqb, Wqb = u8(M, K), u8(N, K)
    sab, swb = f32(M, K // 128), f32(N // 128, K // 128)
    rt.fp8_quantize(A, (1, 128), rt.E4M3, rt.DYNAMIC, 1e-12, False, sab, None, Aqb)
    rt.fp8_quantize(W, (128, 128), rt.E4M3, rt.DYNAMIC, 1e-12, False, swb, None, Wqb)
    Pb = rt.fp8_pack_weights16(Wqb)
    gmb = lambda: rt.fp8_scaled_gemm(Aqb, rt.E4M3, (1, 128), sab, Pb, rt.E4M3, (128, 128), swb, y, bias=bias)
    gmb()
    gb_bytes = M * K + N * K + M * N * 2 + (M * K // 128 + N * K // 16384) * 4 + N * 2
    e = hbm_entry(time_op(torch, gmb, scrub=scrub), gb_bytes, "k_gemm_skinny (packed B, per-step scales)")
    e["TFLOP_s"] = 2.0 * M * N * K / (e["us"] * 1e-6) / 1e12
    comp["decode_gemm_block_scaled_bf16_bias_packed_w"] = e
    del Aqb, Wqb, Pb
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
    gm()
    torch.cuda.synchronize()
    rb = pick(N, 256, 21)
    keep["decode"] = {"a_bits": d["a"], "w_rows": d["w"][rb], "bias": d["bias"], "rows_b": rb,
                      "aq": Aq.cpu().numpy(), "wq": gather(torch, Wq, rb), "s_a": sa.cpu().numpy(),
                      "r_a": ra.cpu().numpy(), "s_w": gather(torch, sw, rb), "r_w": gather(torch, rw, rb),
                      "y": gather(torch, y, np.arange(M), rb)}
    del A, W, bias, Aq, Wq, y, yw, d, stats

    # delayed-scaling backward GEMM: the full 32-step chain at 8192 x 8192.  Step 0
    # uses current scaling (cold start), later steps the scale of the 16-entry
    # amax history; every step pushes its observed amax.  Per step: the E5M2
    # quantize of G_t (with observed amax and counters), the history update and
    # the GEMM G_t(E5M2) W^T(E4M3, per tensor) -> fp32, each event-timed after a
    # cache scrub.
    c4 = wl.C4Delayed()
    M, N, K = c4.M, c4.N, c4.K
    sig, spikes = c4.sigmas()
    w4 = c4.make_w()
    W = from_bits(w4)
    G = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    Gq, Wq = u8(M, K), u8(N, K)
    hist = torch.zeros(c4.history, dtype=torch.float32, device=dev)
    head = torch.zeros(1, dtype=torch.int32, device=dev)
    sg, rg, am, sw, rw = f32(1, 1), f32(1, 1), f32(1, 1), f32(1, 1), f32(1, 1)
    cnt = torch.zeros(2, dtype=torch.int64, device=dev)
    rt.fp8_quantize(W, (0, 0), rt.E4M3, rt.DYNAMIC, 1e-12, False, sw, rw, Wq)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    steps = {"sigma": [], "amax": [], "scale_used": [], "saturated": [], "underflowed": [],
             "quantize_us": [], "history_update_us": [], "gemm_us": []}

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        return e0, e1

    chain_g = [] if check else None
    for t in range(c4.steps):
        g_bits = c4.make_g(t)
        if chain_g is not None:
            chain_g.append(g_bits)           # kept for the oracle's check of every step
        G.copy_(torch.from_numpy(g_bits.view(np.int16)).view(torch.bfloat16))
        if t == 0:
            q = lambda: rt.fp8_quantize(G, (0, 0), rt.E5M2, rt.DYNAMIC, 1e-12, False, sg, rg, Gq, am, cnt)
        else:
            q = lambda: rt.fp8_quantize(G, (0, 0), rt.E5M2, rt.GIVEN, 1e-12, False, sg, rg, Gq, am, cnt)
        scrub()
        eq = timed(q)
        s_used = sg.clone()
        scrub()
        eg = timed(lambda: rt.fp8_scaled_gemm(Gq, rt.E5M2, (0, 0), sg, Wq, rt.E4M3, (0, 0), sw, y))
        eh = timed(lambda: rt.fp8_amax_history_update(hist, head, am, rt.E5M2, 1e-12, False, sg, rg))
        torch.cuda.synchronize()
        cn = cnt.tolist()
        steps["sigma"].append(float(sig[t]))
        steps["amax"].append(float(am.item()))
        steps["scale_used"].append(float(s_used.item()))
        steps["saturated"].append(int(cn[0]))
        steps["underflowed"].append(int(cn[1]))
        steps["quantize_us"].append(eq[0].elapsed_time(eq[1]) * 1e3)
        steps["gemm_us"].append(eg[0].elapsed_time(eg[1]) * 1e3)
        steps["history_update_us"].append(eh[0].elapsed_time(eh[1]) * 1e3)
        if t == c4.steps - 1 and check:
            ra, rb = pick(M, 64, 41), pick(N, 64, 42)
            keep["delayed"] = {"w_bits": w4, "rows_a": ra, "rows_b": rb, "gq": gather(torch, Gq, ra),
                               "wq": gather(torch, Wq, rb), "s_g": s_used.cpu().numpy(),
                               "s_w": sw.cpu().numpy(), "r_w": rw.cpu().numpy(), "y": gather(torch, y, ra, rb),
                               "steps": steps, "chain_g": chain_g}
    gus = Timing(float(np.median(steps["gemm_us"])), float(np.percentile(steps["gemm_us"], 95)))
    # the GIVEN-mode quantize of the last step's G with the history's next
    # scale, timed like every other component (the chain's per-step times
    # follow each step's host-side draw of G_t, half a second with the GPU
    # idle, so they also hold the clock's ramp back up)
    qg = lambda: rt.fp8_quantize(G, (0, 0), rt.E5M2, rt.GIVEN, 1e-12, False, sg, rg, Gq, am, cnt)
    comp["delayed_quantize_g_given_e5m2"] = hbm_entry(time_op(torch, qg, scrub=scrub), M * K * 3 + 4,
                                                       "k_tensor_cast (given, amax + counts) + k_finish")
    comp["delayed_history_update_us"] = float(np.median(steps["history_update_us"]))
    comp["delayed_gemm_e5m2_e4m3_f32"] = mfma_entry(gus, 2.0 * M * N * K, M * K + N * K + M * N * 4 + 8)
    comp["delayed_chain_32_steps"] = {
        "workload": "G_t bf16 8192x8192 = N(0,1) sigma_t, sigma_t = exp(z_t), x100 spike at step(s) %s; "
                    "E5M2, 16-entry amax history (step 0 current scaling); W 8192x8192 per-tensor E4M3; "
                    "fp32 out" % [int(v) for v in spikes],
        "per_step": steps,
        "per_step_timing": "event-timed after a cache scrub, right after the host draws G_t (GPU idle meanwhile)",
        "saturated_total": int(sum(steps["saturated"])), "underflowed_total": int(sum(steps["underflowed"])),
        "steps_with_saturation": int(sum(v > 0 for v in steps["saturated"]))}
    # cast-transpose of the last step's G (the backward reads it in both
    # orientations): codes row-major and K-major in one pass, per-tensor GIVEN
    # (+ amax, counters), and per-column DYNAMIC (column amax pass, scales, then the pass)
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
    a5, w5 = c5.make_a(), c5.make_w()  # host copies for the parity leg (same seeds)
    ra = pick(M, 64, 51)
    blocks = pick(N // 128, 2, 52)
    rb = np.concatenate([b * 128 + np.arange(128) for b in blocks])
    keep["block"] = {"a_rows": a5[ra], "w_rows": w5[rb], "rows_a": ra, "rows_b": rb, "blocks": blocks,
                     "aq": gather(torch, Aq, ra), "wq": gather(torch, Wq, rb), "s_a": gather(torch, sa, ra),
                     "s_w": gather(torch, sw, blocks), "y": gather(torch, y, ra, rb)}
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
    ra, rb = pick(M, 64, 53), pick(N, 64, 54)
    keep["block_mx"] = {"a_rows": a5[ra], "w_rows": w5[rb], "rows_a": ra, "rows_b": rb,
                        "aq": gather(torch, Aq, ra), "wq": gather(torch, Wq, rb), "s_a": gather(torch, sa32, ra),
                        "s_w": gather(torch, sw32, rb), "y": gather(torch, y, ra, rb)}
    del a5, w5
    del A, W, Aq, Wq, y, junk
    torch.cuda.empty_cache()
    return comp


def calibrate_mfma(torch):
    """FP8 MFMA rate with operands in registers (libfp8rt_calib.so): 16 MFMAs
    per wave and iteration, 4 waves per workgroup, 2048 workgroups, median of
    5 event-timed launches after 2 untimed ones, for each instruction shape on
    zero operands and on random bytes (finite E4M3 codes)."""
    import ctypes as C

    path = os.path.join(ROOT, "dynamic_scaling_scaled_amd", "libfp8rt_calib.so")
    if not os.path.exists(path):
        raise ImportError("libfp8rt_calib.so is not built: run __graft_entry__.build()")
    L = C.CDLL(path)
    L.fp8rt_calib_mfma_rate.restype = C.c_int
    L.fp8rt_calib_mfma_rate.argtypes = [C.c_int, C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_void_p]
    nops = L.fp8rt_calib_mfma_operand_ints()
    blocks, iters = 2048, 2000
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    g = np.random.default_rng(7)
    codes = g.integers(0, 256, nops * 4, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E          # no NaN codes
    operands = {"zero": torch.zeros(nops, dtype=torch.int32, device="cuda"),
                "random_e4m3": torch.from_numpy(codes.view(np.int32).copy()).cuda()}
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    rows = []
    for shape, flop in ((32, 2 * 32 * 32 * 64), (16, 2 * 16 * 16 * 128)):
        for name, ops in operands.items():
            run = lambda: L.fp8rt_calib_mfma_rate(shape, C.c_void_p(ops.data_ptr()), blocks, iters,
                                                  C.c_void_p(out.data_ptr()), st)
            ts = []
            for rep in range(7):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                rc = run()
                e1.record()
                e1.synchronize()
                if rc != 0:
                    raise RuntimeError("fp8rt_calib_mfma_rate returned %d" % rc)
                if rep >= 2:
                    ts.append(e0.elapsed_time(e1) * 1e-3)
            t = float(np.median(ts))
            pf = blocks * 4 * iters * 16 * flop / t / 1e15
            rows.append({"instruction": "v_mfma_f32_%s_f8f6f4" % ("32x32x64" if shape == 32 else "16x16x128"),
                         "operands": name, "ms": t * 1e3, "PFLOP_s": pf, "frac_fp8_peak": pf * 1e3 / FP8_PEAK_TFLOPS})
    return {"mfma_rate_registers_only": rows}


LIBRARY_SHAPES = [(4096, 29568, 8192), (4096, 28672, 8192), (8192, 8192, 8192), (8192, 18432, 7168)]


def library_comparison(torch, rt):
    """fp8_scaled_gemm against hipBLASLt (reached through torch._scaled_mm) on
    the same E4M3 codes (N(0,1)-shaped values cast by torch), per-tensor scales,
    bf16 out: median of 20 event-timed calls, caches scrubbed, interleaved so
    that both see the same clock; the largest |difference| relative to the
    output's scale.  Context for the kernels' rates, not part of the step."""
    g = torch.Generator(device="cuda")
    g.manual_seed(20261204)
    junk = torch.empty(2**28, dtype=torch.float32, device="cuda")
    rows = []
    for M, N, K in LIBRARY_SHAPES:
        a8 = torch.randn((M, K), device="cuda", generator=g).to(torch.float8_e4m3fn)
        b8 = (torch.randn((N, K), device="cuda", generator=g) * 4).to(torch.float8_e4m3fn)
        sa = torch.tensor([[0.01]], device="cuda")
        sb = torch.tensor([[0.005]], device="cuda")
        y_rt = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        held = [None]

        def lib():
            held[0] = torch._scaled_mm(a8, b8.t(), scale_a=sa.view(()), scale_b=sb.view(()),
                                       out_dtype=torch.bfloat16)

        ours = lambda: rt.fp8_scaled_gemm(a8.view(torch.uint8), rt.E4M3, (0, 0), sa, b8.view(torch.uint8),
                                          rt.E4M3, (0, 0), sb, y_rt)
        t_lib, t_rt = [], []
        for _ in range(3):
            lib()
            ours()
        for _ in range(20):
            for fn, acc in ((lib, t_lib), (ours, t_rt)):
                junk.fill_(1.0)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                e1.synchronize()
                acc.append(e0.elapsed_time(e1) * 1e3)
        y_lib = held[0]
        d = (y_lib.float() - y_rt.float()).abs().max().item() / max(y_lib.float().abs().max().item(), 1e-30)
        flops = 2.0 * M * N * K
        rows.append({"shape_MxNxK": [M, N, K], "hipblaslt_us": float(np.median(t_lib)),
                     "fp8_scaled_gemm_us": float(np.median(t_rt)),
                     "hipblaslt_frac_fp8_peak": flops / (np.median(t_lib) * 1e-6) / 1e12 / FP8_PEAK_TFLOPS,
                     "fp8_scaled_gemm_frac_fp8_peak": flops / (np.median(t_rt) * 1e-6) / 1e12 / FP8_PEAK_TFLOPS,
                     "max_abs_diff_over_max_abs_y": d})
        print("library comparison %dx%dx%d done" % (M, N, K), file=sys.stderr, flush=True)
        held[0] = None
        del a8, b8, y_lib, y_rt
        torch.cuda.empty_cache()
    return {"library_comparison": rows, "note": "hipBLASLt through torch._scaled_mm; same codes and scales; "
                                                "median of 20 scrubbed calls each, interleaved"}


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
    if args.calibrate_mfma:
        print(json.dumps(calibrate_mfma(torch)), flush=True)
        return
    if args.library_comparison:
        print(json.dumps(library_comparison(torch, rt)), flush=True)
        return
    keep = {}
    out = bench_prefill(args, torch, rt, wl, keep)
    print("prefill step timed", file=sys.stderr, flush=True)
    out["components"]["tiny_latency"] = tiny_latency(torch, rt, wl, keep)
    if not args.no_extra:
        out["components"].update(extra_components(torch, rt, wl, None if args.no_cpu_baseline else keep))
        print("other workloads timed", file=sys.stderr, flush=True)
        out["delayed_recipe_staleness"] = recipe_staleness(torch, rt, wl)
        fr = [v["frac_hbm"] for k, v in out["components"].items()
              if isinstance(v, dict) and "frac_hbm" in v and "quantize" in k and "decode_quantize_a" not in k]
        out["components"]["quantize_min_frac_hbm_large"] = min(fr)
    if not args.no_cpu_baseline:
        # the CPU-baseline leg: the oracle timed on a sample of the prefill
        # step, then run on every workload's inputs to check the GPU's results
        p = keep["prefill"]
        out["cpu_baseline"] = cpu_baseline_prefill(p["x_bits"], p["w_bits"], 4096, 29568, 8192, args.cpu_seconds)
        print("cpu baseline timed", file=sys.stderr, flush=True)
        import oracle

        t0 = time.perf_counter()
        out["parity_full_size"] = parity_leg(oracle, keep, host_cpu()[2])
        out["parity_full_size"]["oracle_seconds"] = time.perf_counter() - t0
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
