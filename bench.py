#!/usr/bin/env python3
"""Benchmark of the FP8 fine-grained quantisation + block-scaled GEMM path on one MI355X.

Default workload (one "step" = the whole hot path on one batch, inputs resident
in HBM): the dense projection  X bf16 [4096,7168] (N(0,1), 0.1% x100 outliers),
W bf16 [7168,7168] (N(0,0.02)):
    fp8_quant_act_weight(X, W) -> fp8_block_gemm -> Y bf16
(the first call quantises X per 1x128 and W per 128x128 in one launch).
The metric is GEMM TFLOP/s of the whole step (2*M*N*K / step time, host clock
over the timed steps); within those steps each GEMM launch sits between two HIP
events on its stream, and the quantisers are timed afterwards as batches.  X and
W are rotated over enough HBM copies (6 of X, 4 of W) that a pass over them
exceeds the 256 MB last-level cache, which so never serves a quantiser's reads.
The line also times, outside the step, the quantisers at the shapes their HBM
target is quoted on (activation [16384,7168], weight [7168,18432]) and the
dual weight quantiser, each rotated the same way.  Before the W warm-up steps
the step runs back to back for --settle seconds (default 1): a cold GPU's
clocks take ~100 GEMMs to come up, which a long training run never sees.

Other workloads (``--workload quant|moe|moe_ep|wgrad|dgrad|pow2|fused|tiny|pertensor``) measure the
remaining rows of the path and print their own JSON line; the default run prints exactly one line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle SECONDS]
                    [--workload dense|quant|moe|moe_ep|wgrad|dgrad|pow2|fused|tiny|pertensor] [--no-cpu-baseline]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 matrix-core peak
PEAK_FP16_TFLOPS = 2500.0  # dense fp16/bf16 matrix-core peak (exact accumulation path)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E


def _sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _traffic(record_name, kernel_src):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None.

    The summary records the sha256 of the kernel source it was taken with; if
    the source has changed since, the figure no longer applies and None is
    returned."""
    from fp8_fine_grained_amd.profile_summary import load_traffic

    rec = load_traffic(os.path.join(ROOT, "profiles", record_name))
    if not rec or rec.get("kernel_source_sha256") != _sha(kernel_src):
        return None
    return rec.get("per_launch_bytes")


def _mfma_counters(record_name):
    """Matrix-core utilisation of the GEMM from a committed rocprofv3 counter
    summary (MFMA-busy fraction of the active cycles, the average clock, and
    their product over the 2.4 GHz of the published peak), or None when the
    GEMM source has changed since the counters were taken."""
    from fp8_fine_grained_amd.profile_summary import load_traffic

    src = os.path.join(ROOT, "fp8_fine_grained_amd", "csrc", "gemm_fp8.hip")
    rec = load_traffic(os.path.join(ROOT, "profiles", record_name))
    if not rec or rec.get("kernel_source_sha256") != _sha(src):
        return None
    return {"mfma_busy_fraction": rec["mfma_busy_fraction"], "clock_ghz": rec["clock_ghz"],
            "fraction_of_peak_mfma_cycles": rec["fraction_of_peak_mfma_cycles"], "source": "profiles/" + record_name}


class Timer:
    """HIP-event timing of one kernel launch site on the stream it is launched on.

    The events are created with hipEventReleaseToDevice.  A default event
    performs a system-scope release when it is recorded, which writes the
    dirty L2 lines back to HBM (after the dense GEMM that is its whole bf16
    output) and so adds that write-back to the bracketed launch; a
    device-scope release times the launch alone."""

    _lib = None
    RELEASE_TO_DEVICE = 0x40000000

    def __init__(self, torch, n=64):
        """n: the most launches this timer will bracket (its events are created
        here, outside the timed region)."""
        import ctypes

        self.torch = torch
        self.ct = ctypes
        if Timer._lib is None:
            torch.cuda.init()
            lib = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch has already loaded
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            Timer._lib = lib
        self.lib = Timer._lib
        self.events = []
        for _ in range(2 * n):
            ev = ctypes.c_void_p()
            rc = self.lib.hipEventCreateWithFlags(ctypes.byref(ev), self.RELEASE_TO_DEVICE)
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self.events.append(ev)
        self.used = 0

    def _record(self):
        if self.used >= len(self.events):
            raise RuntimeError("Timer: more launches than events created")
        ev = self.events[self.used]
        self.used += 1
        rc = self.lib.hipEventRecord(ev, self.ct.c_void_p(self.torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def __enter__(self):
        self._record()
        return self

    def __exit__(self, *a):
        self._record()

    def times_ms(self):
        """Duration of every bracketed launch, in recording order."""
        self.torch.cuda.synchronize()
        ts = []
        for i in range(0, self.used, 2):
            ms = self.ct.c_float()
            rc = self.lib.hipEventElapsedTime(self.ct.byref(ms), self.events[i], self.events[i + 1])
            if rc != 0:
                raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
            ts.append(ms.value)
        return ts

    def mean_ms(self):
        ts = self.times_ms()
        return sum(ts) / len(ts) if ts else float("nan")

    def percentiles_ms(self):
        """p10, median and p90 of the bracketed launches (nearest rank)."""
        ts = sorted(self.times_ms())
        if not ts:
            return None
        pick = lambda q: ts[min(len(ts) - 1, int(q * len(ts)))]
        return {"p10": pick(0.10), "p50": pick(0.50), "p90": pick(0.90)}


LLC_BYTES = 256 << 20  # MI355X last-level (Infinity) cache


def _copies(nbytes, least=3):
    """Input copies to rotate over so that one pass over them exceeds the
    last-level cache by a margin: a launch never finds its input there."""
    return max(least, -(-int(1.25 * LLC_BYTES) // int(nbytes)))


def _cpu_info():
    """Host CPU model and the threads the oracle runs on: its quantisers use
    one thread per core this process may run on (sched_getaffinity), its GEMM
    the BLAS library's thread pool."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info

        blas = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:
        blas = None
    return model, len(os.sched_getaffinity(0)), blas


def settle_clocks(torch, step, seconds):
    """Run `step` back to back for `seconds` of wall time before the warm-up
    steps.  From a cold start the GPU's clocks take ~100 dense GEMMs (about a
    fifth of a second) to come up; what the timed steps measure is the steady
    rate of a long training run, which never sees that ramp."""
    t0 = time.perf_counter()
    n = 0
    while True:
        step(n, False)
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                return n


# ------------------------------------------------------------------ dense

def bench_dense(args, torch, fp8, workloads):
    M, N, K = 4096, 7168, 7168
    d = workloads.dense()
    nx, nw = _copies(M * K * 2), _copies(N * K * 2)
    xs = [d["x"].cuda() for _ in range(nx)]
    ws = [d["w"].cuda() for _ in range(nw)]
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    qb = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sb = torch.empty((N // 128, K // 128), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    t_gemm = Timer(torch, args.steps)
    t_aw, t_act, t_w = Timer(torch, 1), Timer(torch, 1), Timer(torch, 1)

    def step(i, timed):
        x, w = xs[i % nx], ws[i % nw]
        # X per 1x128 and W per 128x128 in one launch (one kernel ramp and tail)
        fp8.fp8_quant_act_weight(x, w, qa, sa, qb, sb)
        if timed:
            with t_gemm:
                fp8.fp8_block_gemm(qa, sa, qb, sb, accum="fp8", y=y)
        else:
            fp8.fp8_block_gemm(qa, sa, qb, sb, accum="fp8", y=y)

    settled = settle_clocks(torch, step, args.settle)
    for i in range(args.warmup):
        step(i, False)
    # The timed steps: the GEMM launch of each step sits between two events (the
    # roofline kernel's per-launch duration); the step rate is the host clock
    # over all steps.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    # The quantisers' own durations, each as one back-to-back batch of launches
    # over the rotated inputs (a per-launch bracket would add the event packets'
    # few microseconds to these short kernels): the step's one-launch pair, and
    # for comparison the two quantisers as separate launches.
    with t_aw:
        for i in range(args.steps):
            fp8.fp8_quant_act_weight(xs[i % nx], ws[i % nw], qa, sa, qb, sb)
    with t_act:
        for i in range(args.steps):
            fp8.fp8_quant_act_1x128(xs[i % nx], qa, sa)
    with t_w:
        for i in range(args.steps):
            fp8.fp8_quant_weight_128x128(ws[i % nw], qb, sb)
    torch.cuda.synchronize()
    extra = quantiser_lines(args, torch, fp8, workloads, d)
    flop = 2.0 * M * N * K
    gemm_ms = t_gemm.mean_ms()
    aw_ms = t_aw.mean_ms() / args.steps
    act_ms, w_ms = t_act.mean_ms() / args.steps, t_w.mean_ms() / args.steps
    act_bytes = M * K * (2 + 1) + M * (K // 128) * 4
    w_bytes = N * K * (2 + 1) + (N // 128) * (K // 128) * 4
    gemm_tflops = flop / (gemm_ms * 1e-3) / 1e12
    traffic = _traffic("block_gemm_dense_4096x7168x7168_traffic.md",
                       os.path.join(ROOT, "fp8_fine_grained_amd", "csrc", "gemm_fp8.hip"))
    out = {
        "metric": "FP8 block-scaled GEMM TFLOP/s (% dense FP8 peak); quantizer GB/s (% HBM peak)",
        "value": flop / dt / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dt * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "data": "synthetic",
        "config": {
            "workload": "dense projection: quantise X bf16 [4096,7168] per 1x128 and W bf16 [7168,7168] "
                        "per 128x128 to E4M3 (one launch), then block-scaled FP8 GEMM Y = X W^T, bf16 out, "
                        "FP8 matrix-core accumulation promoted to fp32 every 128 K",
            "M": M, "N": N, "K": K, "accum": "fp8_mfma", "input_copies_rotated": {"X": nx, "W": nw},
            "clock_settle_s": args.settle, "clock_settle_steps": settled,
        },
        "kernels": {
            "fp8_quant_act_weight (X + W, the step's launch)": {
                "ms": aw_ms, "GB/s": (act_bytes + w_bytes) / (aw_ms * 1e-3) / 1e9,
                "frac_hbm": (act_bytes + w_bytes) / (aw_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
            "fp8_quant_act_1x128 (separate launch)": {"ms": act_ms, "GB/s": act_bytes / (act_ms * 1e-3) / 1e9,
                                                      "frac_hbm": act_bytes / (act_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
            "fp8_quant_weight_128x128 (separate launch)": {
                "ms": w_ms, "GB/s": w_bytes / (w_ms * 1e-3) / 1e9,
                "frac_hbm": w_bytes / (w_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
            "fp8_block_gemm": {"ms": gemm_ms, "TFLOP/s": gemm_tflops,
                               "frac_fp8_peak": gemm_tflops / PEAK_FP8_TFLOPS,
                               "ms_percentiles": t_gemm.percentiles_ms()},
            **extra,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": gemm_tflops,
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": gemm_tflops / PEAK_FP8_TFLOPS,
            "traffic": traffic,
            "mfma_counters": _mfma_counters("block_gemm_dense_4096x7168x7168_mfma_util.md"),
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_dense(d)
    return out


def bench_pow2(args, torch, fp8, workloads):
    """The dense step with power-of-two scales: the quantisers write E8M0-valued
    scales and the matrix cores apply them inside the scaled MFMA (no separate
    promotion step)."""
    M, N, K = 4096, 7168, 7168
    d = workloads.dense()
    nx, nw = _copies(M * K * 2), _copies(N * K * 2)
    xs = [d["x"].cuda() for _ in range(nx)]
    ws = [d["w"].cuda() for _ in range(nw)]
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    qb = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sb = torch.empty((N // 128, K // 128), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    t_gemm = Timer(torch, args.steps)
    t_aw, t_act, t_w = Timer(torch, 1), Timer(torch, 1), Timer(torch, 1)

    def step(i, timed):
        fp8.fp8_quant_act_weight(xs[i % nx], ws[i % nw], qa, sa, qb, sb, pow2=True)
        if timed:
            with t_gemm:
                fp8.fp8_block_gemm(qa, sa, qb, sb, accum="scaled", y=y)
        else:
            fp8.fp8_block_gemm(qa, sa, qb, sb, accum="scaled", y=y)

    settle_clocks(torch, step, args.settle)
    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    with t_aw:
        for i in range(args.steps):
            fp8.fp8_quant_act_weight(xs[i % nx], ws[i % nw], qa, sa, qb, sb, pow2=True)
    with t_act:
        for i in range(args.steps):
            fp8.fp8_quant_act_1x128(xs[i % nx], qa, sa, pow2=True)
    with t_w:
        for i in range(args.steps):
            fp8.fp8_quant_weight_128x128(ws[i % nw], qb, sb, pow2=True)
    torch.cuda.synchronize()
    flop = 2.0 * M * N * K
    gemm_ms = t_gemm.mean_ms()
    act_bytes = M * K * (2 + 1) + M * (K // 128) * 4
    w_bytes = N * K * (2 + 1) + (N // 128) * (K // 128) * 4
    tf = flop / (gemm_ms * 1e-3) / 1e12
    return {
        "metric": "FP8 block-scaled GEMM TFLOP/s, power-of-two scales on the scaled MFMA", "value": flop / dt / 1e12,
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": dt * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "e4m3", "data": "synthetic",
        "config": {"workload": "dense projection with power-of-two (E8M0) group scales: quantise X bf16 [4096,7168] "
                               "per 1x128 and W bf16 [7168,7168] per 128x128 (one launch), scaled-MFMA GEMM "
                               "Y = X W^T, bf16 out",
                   "M": M, "N": N, "K": K, "accum": "scaled_mfma", "input_copies_rotated": {"X": nx, "W": nw}},
        "kernels": {
            "fp8_quant_act_weight, pow2 (X + W, the step's launch)": _hbm_line(
                "aw", t_aw.mean_ms() / args.steps, act_bytes + w_bytes, {}),
            "fp8_quant_act_1x128_pow2 (separate launch)": _hbm_line("act", t_act.mean_ms() / args.steps, act_bytes, {}),
            "fp8_quant_weight_128x128_pow2 (separate launch)": _hbm_line("w", t_w.mean_ms() / args.steps, w_bytes, {}),
            "fp8_block_gemm (scaled)": {"ms": gemm_ms, "TFLOP/s": tf, "frac_fp8_peak": tf / PEAK_FP8_TFLOPS,
                                        "ms_percentiles": t_gemm.percentiles_ms()},
        },
        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / PEAK_FP8_TFLOPS,
                     "traffic": _traffic("block_gemm_pow2_4096x7168x7168_traffic.md",
                                         os.path.join(ROOT, "fp8_fine_grained_amd", "csrc", "gemm_fp8.hip")),
                     "mfma_counters": _mfma_counters("block_gemm_pow2_4096x7168x7168_mfma_util.md")},
    }


def bench_fused(args, torch, fp8, workloads):
    """The dense step with the output cast fused into the GEMM: quantise X and W,
    then one GEMM that writes Y as E4M3 codes + 1x128 scales (the next layer's
    input).  The same work unfused -- fp32 Y to HBM, then the 1x128 quantiser --
    is timed afterwards; both give the same bytes."""
    M, N, K = 4096, 7168, 7168
    d = workloads.dense()
    nx, nw = _copies(M * K * 2), _copies(N * K * 2)
    xs = [d["x"].cuda() for _ in range(nx)]
    ws = [d["w"].cuda() for _ in range(nw)]
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    qb = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sb = torch.empty((N // 128, K // 128), dtype=torch.float32, device="cuda")
    qy = torch.empty((M, N), dtype=torch.uint8, device="cuda")
    sy = torch.empty((M, N // 128), dtype=torch.float32, device="cuda")
    y32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    t_f, t_g, t_q = Timer(torch, args.steps), Timer(torch, args.steps), Timer(torch, args.steps)

    def step(i, timed):
        fp8.fp8_quant_act_weight(xs[i % nx], ws[i % nw], qa, sa, qb, sb)
        if timed:
            with t_f:
                fp8.fp8_block_gemm_quant(qa, sa, qb, sb, q=qy, scales=sy)
        else:
            fp8.fp8_block_gemm_quant(qa, sa, qb, sb, q=qy, scales=sy)

    settle_clocks(torch, step, args.settle)
    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    # unfused: the same step with fp32 Y written, then quantised by the 1x128 quantiser
    t1 = time.perf_counter()
    for i in range(args.steps):
        fp8.fp8_quant_act_weight(xs[i % nx], ws[i % nw], qa, sa, qb, sb)
        with t_g:
            fp8.fp8_block_gemm(qa, sa, qb, sb, accum="fp8", y=y32)
        with t_q:
            fp8.fp8_quant_act_1x128(y32, qy, sy)
    torch.cuda.synchronize()
    dt_unfused = (time.perf_counter() - t1) / args.steps
    flop = 2.0 * M * N * K
    fms = t_f.mean_ms()
    tf = flop / (fms * 1e-3) / 1e12
    return {
        "metric": "FP8 block-scaled GEMM TFLOP/s, output cast to E4M3 1x128 in the epilogue", "value": flop / dt / 1e12,
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": dt * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "e4m3", "data": "synthetic",
        "config": {"workload": "dense projection with the output quantised for the next layer: quantise X bf16 "
                               "[4096,7168] 1x128 and W bf16 [7168,7168] 128x128, GEMM Y = X W^T whose epilogue "
                               "writes Y as E4M3 codes [4096,7168] + fp32 scales [4096,56]",
                   "M": M, "N": N, "K": K, "accum": "fp8_mfma", "input_copies_rotated": {"X": nx, "W": nw}},
        "kernels": {
            "fp8_block_gemm_quant": {"ms": fms, "TFLOP/s": tf, "frac_fp8_peak": tf / PEAK_FP8_TFLOPS},
            "unfused: fp8_block_gemm (fp32 out)": {"ms": t_g.mean_ms()},
            "unfused: fp8_quant_act_1x128 of Y (fp32)": {"ms": t_q.mean_ms()},
            "unfused step (ms)": {"ms": dt_unfused * 1e3},
        },
        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / PEAK_FP8_TFLOPS, "traffic": None},
    }


def quantiser_lines(args, torch, fp8, workloads, d):
    """The quantisers at the shapes their HBM target is quoted on (activation
    bf16 [16384,7168] Student-t, weight bf16 [7168,18432] N(0,0.02)), and the
    dual weight quantiser of the data gradient on W [7168,7168]; each timed as
    one back-to-back batch over enough rotated input copies that a pass over
    them exceeds the last-level cache.  Not part of the step or its value."""
    act = workloads.quant_act()
    w = workloads.quant_weight()
    M, K = act.shape
    N, KW = w.shape
    na, nw = _copies(act.numel() * 2, 2), _copies(w.numel() * 2, 2)
    acts = [act.cuda() for _ in range(na)]
    ws = [w.cuda() for _ in range(nw)]
    del act, w
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    qw = torch.empty((N, KW), dtype=torch.uint8, device="cuda")
    sw = torch.empty((N // 128, KW // 128), dtype=torch.float32, device="cuda")
    D = d["w"].shape[0]
    nd = _copies(D * D * 2)
    wd = [d["w"].cuda() for _ in range(nd)]
    q1 = torch.empty((D, D), dtype=torch.uint8, device="cuda")
    q2 = torch.empty((D, D), dtype=torch.uint8, device="cuda")
    s1 = torch.empty((D // 128, D // 128), dtype=torch.float32, device="cuda")
    s2 = torch.empty((D // 128, D // 128), dtype=torch.float32, device="cuda")
    n = max(args.steps, 20)
    for i in range(max(args.warmup, 4)):
        fp8.fp8_quant_act_1x128(acts[i % na], qa, sa)
        fp8.fp8_quant_weight_128x128(ws[i % nw], qw, sw)
        fp8.fp8_quant_weight_128x128_dual(wd[i % nd], q1, s1, q2, s2)
    ta, tw, tdl = Timer(torch, 1), Timer(torch, 1), Timer(torch, 1)
    with ta:
        for i in range(n):
            fp8.fp8_quant_act_1x128(acts[i % na], qa, sa)
    with tw:
        for i in range(n):
            fp8.fp8_quant_weight_128x128(ws[i % nw], qw, sw)
    with tdl:
        for i in range(n):
            fp8.fp8_quant_weight_128x128_dual(wd[i % nd], q1, s1, q2, s2)
    torch.cuda.synchronize()
    ab = M * K * 3 + M * (K // 128) * 4
    wb = N * KW * 3 + (N // 128) * (KW // 128) * 4
    db = D * D * 4 + 2 * (D // 128) ** 2 * 4
    return {
        "fp8_quant_act_1x128 [16384,7168] Student-t": _hbm_line("act", ta.mean_ms() / n, ab, {"copies": na}),
        "fp8_quant_weight_128x128 [7168,18432]": _hbm_line("w", tw.mean_ms() / n, wb, {"copies": nw}),
        "fp8_quant_weight_128x128_dual [7168,7168]": _hbm_line("dual", tdl.mean_ms() / n, db, {"copies": nd}),
    }


def cpu_baseline_dense(d, min_seconds=10.0, max_steps=10):
    """The oracle on the dense step itself (all 4096 rows of X, all of W),
    repeated until at least `min_seconds` of host time (at most `max_steps`
    steps): a few seconds per step, depending on the host's cores."""
    from oracle import gemm, quant

    rows = d["x"].shape[0]
    x = d["x"][:rows].float().numpy()
    w = d["w"].float().numpy()
    steps, dt = 0, 0.0
    while steps < max_steps and (steps == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        ra, rsa = quant.quant_1x128(x)
        rb, rsb = quant.quant_128x128(w)
        gemm.block_gemm(ra, rsa, rb, rsb)
        dt += time.perf_counter() - t0
        steps += 1
    flop = 2.0 * rows * w.shape[0] * w.shape[1] * steps
    model, cores, blas = _cpu_info()
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": model, "blas_threads": blas,
            "sample": f"{steps} dense step(s), X [{rows},{x.shape[1]}] and W [{w.shape[0]},{w.shape[1]}]: numpy 1x128 + "
                      f"128x128 quantisation ({quant.threads()} threads over row chunks) and fp64 GEMM (BLAS, "
                      f"{blas} threads); {dt:.1f} s in all"}


# ------------------------------------------------------------------ other rows

def _hbm_line(name, ms, nbytes, extra):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms": ms, "GB/s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS, "bytes": nbytes, **extra}


def bench_quant(args, torch, fp8, workloads):
    act = workloads.quant_act()
    w = workloads.quant_weight()
    acts = [act.cuda() for _ in range(3)]
    ws = [w.cuda() for _ in range(3)]
    M, K = act.shape
    N, KW = w.shape
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    qw = torch.empty((N, KW), dtype=torch.uint8, device="cuda")
    sw = torch.empty((N // 128, KW // 128), dtype=torch.float32, device="cuda")
    # Each quantiser is timed as one back-to-back batch of `steps` launches (inputs
    # rotated over three copies) inside a single event pair: a per-launch bracket
    # would add the event packets' few microseconds to a ~60 us kernel.
    ta, tw = Timer(torch, 1), Timer(torch, 1)
    for i in range(args.warmup):
        fp8.fp8_quant_act_1x128(acts[i % 3], qa, sa)
        fp8.fp8_quant_weight_128x128(ws[i % 3], qw, sw)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with ta:
        for i in range(args.steps):
            fp8.fp8_quant_act_1x128(acts[i % 3], qa, sa)
    with tw:
        for i in range(args.steps):
            fp8.fp8_quant_weight_128x128(ws[i % 3], qw, sw)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    ab = M * K * 3 + M * (K // 128) * 4
    wb = N * KW * 3 + (N // 128) * (KW // 128) * 4
    act_line = _hbm_line("act", ta.mean_ms() / args.steps, ab, {})
    w_line = _hbm_line("weight", tw.mean_ms() / args.steps, wb, {})
    return {
        "metric": "quantizer GB/s (% HBM peak)", "value": (ab + wb) / dt / 1e9, "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": dt * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "e4m3",
        "data": "synthetic",
        "config": {"workload": "quantiser bandwidth: activation bf16 [16384,7168] Student-t nu=3 per 1x128; "
                               "weight bf16 [7168,18432] N(0,0.02) per 128x128", "input_copies_rotated": 3},
        "kernels": {"fp8_quant_act_1x128": act_line, "fp8_quant_weight_128x128": w_line},
        "roofline": {"bound": "hbm", "achieved": act_line["GB/s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": act_line["frac_hbm"],
                     "traffic": _traffic("quant_act_1x128_16384x7168_traffic.md",
                                         os.path.join(ROOT, "fp8_fine_grained_amd", "csrc", "quant.hip"))},
    }


def bench_pertensor(args, torch, fp8, workloads):
    # The dense projection with ONE scale per tensor (the practice the 1x128 /
    # 128x128 grouping replaces): per-tensor quantisation of X and W (an amax
    # pass, then the cast: X and W are read twice), then the same block GEMM,
    # whose scales are then all equal.  The fine-grained quantisers are timed
    # on the same inputs beside it.
    d = workloads.dense()
    M, K = d["x"].shape
    N = d["w"].shape[0]
    nx, nw = _copies(M * K * 2), _copies(N * K * 2)
    xs = [d["x"].cuda() for _ in range(nx)]
    ws = [d["w"].cuda() for _ in range(nw)]
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    qb = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sb = torch.empty((N // 128, K // 128), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    tx, tw, tg = Timer(torch, args.steps), Timer(torch, args.steps), Timer(torch, args.steps)

    def step(i, timed):
        if timed:
            with tx:
                fp8.fp8_quant_per_tensor(xs[i % nx], "act", qa, sa)
            with tw:
                fp8.fp8_quant_per_tensor(ws[i % nw], "weight", qb, sb)
            with tg:
                fp8.fp8_block_gemm(qa, sa, qb, sb, accum="fp8", y=y)
        else:
            fp8.fp8_quant_per_tensor(xs[i % nx], "act", qa, sa)
            fp8.fp8_quant_per_tensor(ws[i % nw], "weight", qb, sb)
            fp8.fp8_block_gemm(qa, sa, qb, sb, accum="fp8", y=y)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    fa, fw = Timer(torch, 1), Timer(torch, 1)
    with fa:
        for i in range(args.steps):
            fp8.fp8_quant_act_1x128(xs[i % nx], qa, sa)
    with fw:
        for i in range(args.steps):
            fp8.fp8_quant_weight_128x128(ws[i % nw], qb, sb)
    flop = 2.0 * M * N * K
    gms = tg.mean_ms()
    tf = flop / (gms * 1e-3) / 1e12
    return {
        "metric": "FP8 block GEMM TFLOP/s, per-tensor scales (step incl. per-tensor quantisation)",
        "value": flop / dt / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": dt * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "e4m3",
        "data": "synthetic",
        "config": {"workload": "dense projection X bf16 [4096,7168] (0.1% x100), W bf16 [7168,7168], one scale per "
                               "tensor (amax pass + cast), block-scaled FP8 GEMM with uniform scales, bf16 out",
                   "M": M, "N": N, "K": K, "input_copies_rotated": {"X": nx, "W": nw}},
        "kernels": {
            "fp8_quant_per_tensor (X, 3 launches)": {"ms": tx.mean_ms()},
            "fp8_quant_per_tensor (W, 3 launches)": {"ms": tw.mean_ms()},
            "fp8_block_gemm": {"ms": gms, "TFLOP/s": tf, "frac_fp8_peak": tf / PEAK_FP8_TFLOPS},
            "for comparison: fp8_quant_act_1x128 (X)": {"ms": fa.mean_ms() / args.steps},
            "for comparison: fp8_quant_weight_128x128 (W)": {"ms": fw.mean_ms() / args.steps},
        },
        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / PEAK_FP8_TFLOPS, "traffic": None},
    }


def bench_tiny(args, torch, fp8, workloads):
    # The small configuration: X fp32 [128,256] (1% of entries x50), W fp32
    # [128,256]; quantise both, then the block-scaled GEMM with fp32 output and
    # exact accumulation.  It is latency-bound (8.4 MFLOP), so the step is timed
    # as one back-to-back batch inside a single event pair.
    t = workloads.tiny()
    x, w = t["x"].cuda(), t["w"].cuda()
    M, K = x.shape
    N = w.shape[0]
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    qb = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sb = torch.empty((N // 128, K // 128), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def step():
        fp8.fp8_quant_act_1x128(x, qa, sa)
        fp8.fp8_quant_weight_128x128(w, qb, sb)
        fp8.fp8_block_gemm(qa, sa, qb, sb, accum="exact", y=y)

    tb, tg = Timer(torch, 1), Timer(torch, 1)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with tb:
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    with tg:
        for _ in range(args.steps):
            fp8.fp8_block_gemm(qa, sa, qb, sb, accum="exact", y=y)
    # The same step captured once in a HIP graph and replayed: one submission
    # for the three kernels instead of three launches.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    tr = Timer(torch, 1)
    with tr:
        for _ in range(args.steps):
            graph.replay()
    step_ms, gemm_ms, replay_ms = tb.mean_ms() / args.steps, tg.mean_ms() / args.steps, tr.mean_ms() / args.steps
    flop = 2.0 * M * N * K
    tf = flop / (gemm_ms * 1e-3) / 1e12
    return {
        "metric": "small-case step latency (us)", "value": step_ms * 1e3, "unit": "us", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": dt * 1e3, "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "e4m3", "data": "synthetic",
        "config": {"workload": "small case: X fp32 [128,256] N(0,1) with 1% x50 outliers, W fp32 [128,256] "
                               "N(0,0.02); 1x128 and 128x128 quantisation, block-scaled GEMM, fp32 out, exact "
                               "accumulation", "M": M, "N": N, "K": K},
        "kernels": {"step (3 launches, event-timed batch)": {"us": step_ms * 1e3},
                    "step as one HIP graph replay": {"us": replay_ms * 1e3},
                    "fp8_block_gemm": {"us": gemm_ms * 1e3, "TFLOP/s": tf}},
        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / PEAK_FP16_TFLOPS, "traffic": None},
    }


def bench_moe(args, torch, fp8, workloads):
    # One step of the MoE up-projection: quantise the 8192 tokens 1x128, then the
    # grouped GEMM reads each routed row from its token (FP8 dispatch by index).
    # The same GEMM on a pre-permuted copy of the rows is timed afterwards.
    route = workloads.moe_routing()
    tokens = workloads.moe_tokens().cuda()
    offsets = torch.from_numpy(route["offsets"]).cuda()
    idx = torch.from_numpy(route["perm"].astype("int32")).cuda()
    G, N, K = 256, 2048, 7168
    T, Mt = tokens.shape[0], idx.numel()
    # Weights drawn on the GPU from a seeded generator: the benchmark needs no
    # oracle comparison, and 3.76e9 CPU draws would dominate the run time.
    gen = torch.Generator(device="cuda").manual_seed(4)
    w = (torch.randn((G * N, K), generator=gen, device="cuda", dtype=torch.float32) * 0.02).to(torch.bfloat16)
    qb, sb = fp8.fp8_quant_weight_128x128(w)
    del w
    qb, sb = qb.view(G, N, K), sb.view(G, N // 128, K // 128)
    qt = torch.empty((T, K), dtype=torch.uint8, device="cuda")
    st = torch.empty((T, K // 128), dtype=torch.float32, device="cuda")
    y = torch.empty((Mt, N), dtype=torch.bfloat16, device="cuda")
    tg = Timer(torch, args.steps)
    tq, tp = Timer(torch, 1), Timer(torch, args.steps)

    def step(timed):
        fp8.fp8_quant_act_1x128(tokens, qt, st)
        if timed:
            with tg:
                fp8.fp8_block_grouped_gemm_gather(qt, st, idx, offsets, qb, sb, accum="fp8", y=y)
        else:
            fp8.fp8_block_grouped_gemm_gather(qt, st, idx, offsets, qb, sb, accum="fp8", y=y)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    with tq:
        for _ in range(args.steps):
            fp8.fp8_quant_act_1x128(tokens, qt, st)
    # the same GEMM on routed rows copied out in advance (no gather)
    qa, sa = qt[idx.long()].contiguous(), st[idx.long()].contiguous()
    for _ in range(args.steps):
        with tp:
            fp8.fp8_block_grouped_gemm(qa, sa, offsets, qb, sb, accum="fp8", y=y)
    torch.cuda.synchronize()
    flop = 2.0 * Mt * N * K
    gms, pms = tg.mean_ms(), tp.mean_ms()
    gemm_bytes = T * K + T * (K // 128) * 4 + G * N * K + G * (N // 128) * (K // 128) * 4 + Mt * N * 2 + Mt * 4

    def gemm_line(ms):
        return {"ms": ms, "TFLOP/s": flop / (ms * 1e-3) / 1e12, "frac_fp8_peak": flop / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
                "GB/s": gemm_bytes / (ms * 1e-3) / 1e9, "frac_hbm": gemm_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}

    return {
        "metric": "grouped FP8 GEMM TFLOP/s", "value": flop / dt / 1e12, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": dt * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "e4m3", "data": "synthetic",
        "config": {"workload": "MoE up-projection: 8192 tokens x 7168, 256 experts top-8 -> 65536 routed rows; "
                               "per-expert W [2048,7168]; 1x128 quantisation of the tokens, grouped GEMM reading "
                               "each routed row from its token by index, bf16 out",
                   "T": T, "M_total": Mt, "N": N, "K": K, "G": G},
        "kernels": {
            "fp8_quant_act_1x128 (tokens)": _hbm_line("act", tq.mean_ms() / args.steps, T * K * 3 + T * (K // 128) * 4, {}),
            "fp8_block_grouped_gemm_gather": dict(gemm_line(gms), ms_percentiles=tg.percentiles_ms()),
            "fp8_block_grouped_gemm (pre-permuted rows)": gemm_line(pms),
        },
        "roofline": {"bound": "hbm", "achieved": gemm_bytes / (gms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": gemm_bytes / (gms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "traffic": _traffic("grouped_gemm_moe_65536x2048x7168_traffic.md",
                                         os.path.join(ROOT, "fp8_fine_grained_amd", "csrc", "gemm_fp8.hip")),
                     "mfma_counters": _mfma_counters("grouped_gemm_moe_65536x2048x7168_mfma_util.md")},
    }


def bench_moe_ep(args, torch, fp8, workloads):
    # One GPU's share of the MoE up-projection under expert parallelism over 8
    # GPUs: 32 consecutive experts and the rows routed to them (~8192 of the
    # 65536), the same gathering launch at G = 32.  The eight shares of the 256
    # experts run in turn, so consecutive launches read different weights (470 MB
    # each) from HBM, as each GPU's own share would be.
    import numpy as np

    route = workloads.moe_routing()
    tokens = workloads.moe_tokens().cuda()
    idx = torch.from_numpy(route["perm"].astype("int32")).cuda()
    G, N, K, GS = 256, 2048, 7168, 32
    T, Mt = tokens.shape[0], idx.numel()
    gen = torch.Generator(device="cuda").manual_seed(4)
    w = (torch.randn((G * N, K), generator=gen, device="cuda", dtype=torch.float32) * 0.02).to(torch.bfloat16)
    qb, sb = fp8.fp8_quant_weight_128x128(w)
    del w
    qb, sb = qb.view(G, N, K), sb.view(G, N // 128, K // 128)
    qt, st = fp8.fp8_quant_act_1x128(tokens)
    y = torch.empty((Mt, N), dtype=torch.bfloat16, device="cuda")
    off_np = route["offsets"].astype(np.int64)
    shares = []
    for e in range(G // GS):
        lo, hi = int(off_np[e * GS]), int(off_np[(e + 1) * GS])
        o = torch.from_numpy((off_np[e * GS:(e + 1) * GS + 1] - lo).astype(np.int32)).cuda()
        tok = int(np.unique(route["perm"][lo:hi]).size)  # distinct tokens the share reads
        nbytes = (tok * (K + (K // 128) * 4) + GS * (N * K + (N // 128) * (K // 128) * 4)
                  + (hi - lo) * (N * 2 + 4))
        shares.append((idx[lo:hi], o, qb[e * GS:(e + 1) * GS], sb[e * GS:(e + 1) * GS], y[lo:hi],
                       2.0 * (hi - lo) * N * K, nbytes, hi - lo))

    def launch(i):
        ix, o, b, sbs, ys = shares[i % len(shares)][:5]
        fp8.fp8_block_grouped_gemm_gather(qt, st, ix, o, b, sbs, accum="fp8", y=ys)

    settle_clocks(torch, lambda i, t: launch(i), args.settle)
    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize()
    ts = Timer(torch, args.steps)
    flop = nbytes = 0.0
    t0 = time.perf_counter()
    for i in range(args.steps):
        with ts:
            launch(i)
        flop += shares[i % len(shares)][5]
        nbytes += shares[i % len(shares)][6]
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    ms = ts.mean_ms()
    flop, nbytes = flop / args.steps, nbytes / args.steps
    rows = [sh[7] for sh in shares]
    return {
        "metric": "grouped FP8 GEMM TFLOP/s, one GPU's expert-parallel share", "value": flop / dt / 1e12,
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": dt * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "e4m3", "data": "synthetic",
        "config": {"workload": "one GPU's share of the MoE up-projection under 8-way expert parallelism: 32 of "
                               "the 256 experts (W [2048,7168] each) and the rows routed to them by the top-8 "
                               "routing of 8192 tokens; gathering grouped GEMM at G = 32, bf16 out; the eight "
                               "shares launched in turn",
                   "G": GS, "rows_per_share": [min(rows), max(rows)], "N": N, "K": K, "T": T},
        "kernels": {
            "fp8_block_grouped_gemm_gather (G = 32)": dict(
                {"ms": ms, "TFLOP/s": flop / (ms * 1e-3) / 1e12, "frac_fp8_peak": flop / (ms * 1e-3) / 1e12 /
                 PEAK_FP8_TFLOPS, "GB/s": nbytes / (ms * 1e-3) / 1e9,
                 "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "bytes": nbytes},
                ms_percentiles=ts.percentiles_ms()),
        },
        "roofline": {"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "traffic": _traffic("moe_ep_share_32x2048x7168_traffic.md",
                                         os.path.join(ROOT, "fp8_fine_grained_amd", "csrc", "gemm_fp8.hip")),
                     "mfma_counters": _mfma_counters("moe_ep_share_32x2048x7168_mfma_util.md")},
    }


def bench_wgrad(args, torch, fp8, workloads):
    d = workloads.wgrad()
    dy, x = d["dy"].cuda(), d["x"].cuda()
    C, T = 7168, 16384
    qa = torch.empty((C, T), dtype=torch.uint8, device="cuda")
    sa = torch.empty((C, T // 128), dtype=torch.float32, device="cuda")
    qb = torch.empty((C, T), dtype=torch.uint8, device="cuda")
    sb = torch.empty((C, T // 128), dtype=torch.float32, device="cuda")
    y = torch.empty((C, C), dtype=torch.float32, device="cuda")
    tq, tg, tf = Timer(torch, args.steps), Timer(torch, args.steps), Timer(torch, args.steps)
    for _ in range(args.warmup):
        fp8.fp8_quant_act_1x128(dy.t(), qa, sa)
        fp8.fp8_quant_act_1x128(x.t(), qb, sb)
        fp8.fp8_block_gemm(qa, sa, qb, sb, b_scale_mode="row", accum="exact", y=y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        with tq:
            fp8.fp8_quant_act_1x128(dy.t(), qa, sa)
            fp8.fp8_quant_act_1x128(x.t(), qb, sb)
        with tg:
            fp8.fp8_block_gemm(qa, sa, qb, sb, b_scale_mode="row", accum="exact", y=y)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    for _ in range(max(1, args.steps // 2)):
        with tf:
            fp8.fp8_block_gemm(qa, sa, qb, sb, b_scale_mode="row", accum="fp8", y=y)
    torch.cuda.synchronize()
    flop = 2.0 * C * C * T
    gms, fms = tg.mean_ms(), tf.mean_ms()
    qbytes = 2 * (T * C * 3 + C * (T // 128) * 4)
    return {
        "metric": "weight-gradient FP8 GEMM TFLOP/s", "value": flop / dt / 1e12, "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": dt * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "e4m3", "data": "synthetic",
        "config": {"workload": "weight gradient dW = dY^T X: dY, X bf16 [16384,7168] quantised 1x128 along "
                               "tokens (transposed read), row-scaled GEMM, fp32 out, exact accumulation",
                   "M": C, "N": C, "K": T},
        "kernels": {
            "fp8_quant_act_1x128 (transposed, x2)": _hbm_line("q", tq.mean_ms(), qbytes, {}),
            "fp8_block_gemm (row scales, exact)": {"ms": gms, "TFLOP/s": flop / (gms * 1e-3) / 1e12,
                                                   "frac_fp16_peak": flop / (gms * 1e-3) / 1e12 / PEAK_FP16_TFLOPS,
                                                   "ms_percentiles": tg.percentiles_ms()},
            "fp8_block_gemm (row scales, fp8 accum)": {"ms": fms, "TFLOP/s": flop / (fms * 1e-3) / 1e12,
                                                       "frac_fp8_peak": flop / (fms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS},
        },
        "roofline": {"bound": "mfma", "achieved": flop / (gms * 1e-3) / 1e12, "peak": PEAK_FP16_TFLOPS,
                     "unit": "TFLOP/s", "frac": flop / (gms * 1e-3) / 1e12 / PEAK_FP16_TFLOPS, "traffic": None,
                     "mfma_counters": _mfma_counters("wgrad_exact_7168x7168x16384_mfma_util.md")},
    }


def bench_dgrad(args, torch, fp8, workloads):
    # dX [M,K] = dY [M,N] W [N,K]: dY quantised 1x128 along N, W quantised 128x128
    # once for both orientations, the GEMM reads the transposed codes.
    M, N, K = 4096, 7168, 7168
    d = workloads.dgrad()
    ndy, nw = _copies(M * N * 2), _copies(N * K * 2)
    dys = [d["dy"].cuda() for _ in range(ndy)]
    ws = [d["w"].cuda() for _ in range(nw)]
    qa = torch.empty((M, N), dtype=torch.uint8, device="cuda")
    sa = torch.empty((M, N // 128), dtype=torch.float32, device="cuda")
    q = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    s = torch.empty((N // 128, K // 128), dtype=torch.float32, device="cuda")
    qt = torch.empty((K, N), dtype=torch.uint8, device="cuda")
    st = torch.empty((K // 128, N // 128), dtype=torch.float32, device="cuda")
    y = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    t_gemm = Timer(torch, args.steps)
    t_act, t_w = Timer(torch, 1), Timer(torch, 1)

    def step(i, timed):
        fp8.fp8_quant_act_1x128(dys[i % ndy], qa, sa)
        fp8.fp8_quant_weight_128x128_dual(ws[i % nw], q, s, qt, st)
        if timed:
            with t_gemm:
                fp8.fp8_block_gemm(qa, sa, qt, st, accum="fp8", y=y)
        else:
            fp8.fp8_block_gemm(qa, sa, qt, st, accum="fp8", y=y)

    settle_clocks(torch, step, args.settle)
    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, True)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    with t_act:
        for i in range(args.steps):
            fp8.fp8_quant_act_1x128(dys[i % ndy], qa, sa)
    with t_w:
        for i in range(args.steps):
            fp8.fp8_quant_weight_128x128_dual(ws[i % nw], q, s, qt, st)
    torch.cuda.synchronize()
    flop = 2.0 * M * N * K
    gms = t_gemm.mean_ms()
    act_bytes = M * N * 3 + M * (N // 128) * 4
    dual_bytes = N * K * 4 + 2 * (N // 128) * (K // 128) * 4
    return {
        "metric": "data-gradient FP8 GEMM TFLOP/s", "value": flop / dt / 1e12, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": dt * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "e4m3", "data": "synthetic",
        "config": {"workload": "data gradient dX = dY W of the dense projection: dY bf16 [4096,7168] ~ N(0,1e-3) "
                               "quantised 1x128, W bf16 [7168,7168] quantised 128x128 with the transposed codes "
                               "written in the same pass, block-scaled GEMM on W^T, bf16 out",
                   "M": M, "N": K, "K": N, "input_copies_rotated": {"dY": ndy, "W": nw}},
        "kernels": {
            "fp8_quant_act_1x128": _hbm_line("act", t_act.mean_ms() / args.steps, act_bytes, {}),
            "fp8_quant_weight_128x128_dual": _hbm_line("dual", t_w.mean_ms() / args.steps, dual_bytes, {}),
            "fp8_block_gemm": {"ms": gms, "TFLOP/s": flop / (gms * 1e-3) / 1e12,
                               "frac_fp8_peak": flop / (gms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS},
        },
        "roofline": {"bound": "mfma", "achieved": flop / (gms * 1e-3) / 1e12, "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": flop / (gms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, "traffic": None},
    }


def copy_calibration(args, torch):
    """A plain 1 GiB device-to-device copy: the reference for scaling rocprofv3 byte counters."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # The first ~100 dense GEMMs of a process run up to 25% slower while the
    # clocks ramp up; the default warm-up covers that ramp.
    ap.add_argument("--warmup", type=int, default=100)
    # Back-to-back steps before the warm-up, by wall time: the clock ramp of a
    # cold GPU is not part of a training step's steady rate.
    ap.add_argument("--settle", type=float, default=1.0, help="seconds of untimed steps before the warm-up")
    ap.add_argument("--workload", default="dense", choices=["dense", "quant", "moe", "moe_ep", "wgrad", "dgrad", "pow2", "fused", "tiny", "pertensor"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): this "
              "library has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args, torch)
        return
    import fp8_fine_grained_amd.binding as fp8
    import workloads

    fn = {"dense": bench_dense, "quant": bench_quant, "moe": bench_moe, "moe_ep": bench_moe_ep, "wgrad": bench_wgrad,
          "dgrad": bench_dgrad, "pow2": bench_pow2,
          "fused": bench_fused, "tiny": bench_tiny, "pertensor": bench_pertensor}[args.workload]
    out = fn(args, torch, fp8, workloads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
