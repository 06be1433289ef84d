#!/usr/bin/env python3
"""Benchmark of the LM-head hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input,
M=1024 tokens, K=8192 hidden, V=32768 vocabulary (x ~ N(0,1),
W ~ N(0, 0.02^2), BF16), reading the logits once in the cross-entropy:

    lmhead_logits (FP32 out) -> lmhead_xent_mean (1/n_valid from the targets)
    -> lmhead_xent_fused (forward stats + BF16 dlogits in one logits read)
    -> lmhead_xent_mean (mean loss) -> lmhead_dgrad -> lmhead_wgrad

W warmup steps, then K timed steps bracketed by torch.cuda.synchronize();
HIP events on the launch stream give each kernel's duration.  `value` is the
logits GEMM's TFLOPS (2*M*K*V per launch / mean launch time) -- the first
half of the metric.  Beside the step the same run measures:

* the same step with the cross-entropy as two passes over the logits
  (lmhead_xent_fwd -> lmhead_xent_mean -> lmhead_xent_bwd), as before the
  Transformer Engine change that removes one logits read;

* the FP32-output vs BF16-output logits GEMM, the pages' protocol
  (preallocated outputs, 10 warmup pairs, 30 alternating samples, medians;
  Megatron-LM "Add mixed-precision (FP32) LM output logits", section "GEMM
  kernel benchmark");
* the fused CE forward + FP32 backward over FP32 logits [8192 x 131072]
  (N(0, 3^2), 1% rows +30 spikes, 2% ignored) -- the second half of the
  metric, in GB/s of algorithmic bytes -- out of place, in place and with
  BF16 gradients;
* the pages' GEMM grid (M in 16/128/1024, K in 1024..16384, V = 32768),
  FP32-out vs BF16-out with the same protocol, each shape's roofline
  fraction, and the median FP32-output overhead;
* the logits GEMM cold (L2 and MALL flushed between samples) and warm at
  M=128 K=4096 and M=1024 K=8192;
* the full steps at M=4096 K=16384 V=131072, at one GPU's token shard of it
  (M=512), and at M=128 K=4096 V=32768 (per-kernel times);
* what the chip sustains: a register-only MFMA loop (all-ones and
  pseudo-random operands) and a 1 GiB copy; board power and clock (amdsmi
  sensors) while the logits GEMM and the MFMA loops run; and the vendor BLAS
  on the step's GEMM (BF16 out), for context;
* the FP64 CPU oracle on a bounded sample of every step of the same work,
  on the host threads of this process's CPU share and on one thread,
  extrapolated to the whole step (cpu_baseline).

Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LM-head GEMM TFLOPS (% MFMA peak) + fused CE fwd+bwd GB/s (% HBM peak)"
# MI355X published dense peaks: BF16 MFMA 256 CU x 4096 FLOP/clk x 2.4 GHz;
# HBM3E 8 TB/s.
PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0

# HBM bytes per launch measured with rocprofv3 (FETCH_SIZE x 2.0 and
# WRITE_SIZE x 1.0: the factors a plain 1 GiB device copy reads for these two
# counters on this GPU), valid only for the kernel sources they were taken on
# (code hash of the .hip file, see source_code_hash).  Changed code reports null.
MEASURED_TRAFFIC = {
    "logits_fp32": {"src": "gemm.hip", "sha": "5e382724501b3220",
                    "bytes": int((2 * 394628.8 + 132751.5) * 1024)},
    "xent_fwd_bwd_fp32": {"src": "xent.hip", "sha": "94784a1df1d6afbd",
                          "bytes": int((2 * 2097959.3 + 513.7 + 2 * 2056475.7 + 4195678.0) * 1024)},
    "xent_fused_bf16_1024x32768": {"src": "xent.hip", "sha": "94784a1df1d6afbd",
                                   "bytes": int((2 * 65666.2 + 65661.2) * 1024)},
}


def source_code_hash(name):
    """sha256 prefix of a kernel source with comments and whitespace removed,
    so that edits to comments do not void a measurement."""
    import hashlib
    import re

    with open(os.path.join(ROOT, "lm_head_fp32_amd", "csrc", name)) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = re.sub(r"\s+", " ", text).strip()
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def measured_traffic(key):
    t = MEASURED_TRAFFIC[key]
    return t["bytes"] if source_code_hash(t["src"]) == t["sha"] else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--samples", type=int, default=30, help="samples per side measurement")
    ap.add_argument("--ce-rows", type=int, default=8192, help="rows of the large CE workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-side", action="store_true", help="skip the side measurements")
    ap.add_argument("--grid-only", action="store_true",
                    help="run only the pages' 15-shape GEMM grid and print its JSON (profiling aid)")
    ap.add_argument("--no-grid", action="store_true",
                    help="skip the GEMM grid and the cold/warm measurement")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


class KernelTimer:
    """Start/end HIP events around the named launches on the current stream:
    every launch, or only those whose names are in `only`."""

    def __init__(self, torch, only=None):
        self.torch = torch
        self.only = only
        self.pairs = {}

    def __call__(self, name, fn):
        if self.only is not None and name not in self.only:
            return fn()
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        r = fn()
        b.record()
        self.pairs.setdefault(name, []).append((a, b))
        return r

    def ms(self, name):
        return [a.elapsed_time(b) for a, b in self.pairs.get(name, [])]


def quantiles(ts):
    """median, p10, p90 of a list of times."""
    s = sorted(ts)
    q = lambda p: s[min(len(s) - 1, max(0, int(round(p * (len(s) - 1)))))]
    return statistics.median(s), q(0.1), q(0.9)


def alternate(torch, samples, fns):
    """The pages' protocol for two variants: (10 warmup pairs done by the
    caller), then `samples` rounds in alternating order; HIP events per call."""
    tm = KernelTimer(torch)
    names = list(fns)
    for i in range(samples):
        for name in (names if i % 2 == 0 else names[::-1]):
            tm(name, fns[name])
    torch.cuda.synchronize()
    return tm


# The pages' GEMM grid: M x K at V = 32768 (Megatron-LM "Add mixed-precision
# (FP32) LM output logits", section "GEMM kernel benchmark").
GRID_M = (16, 128, 1024)
GRID_K = (1024, 2048, 4096, 8192, 16384)
GRID_V = 32768


def gemm_grid(torch, lmh, samples, seed):
    """FP32-out vs BF16-out logits GEMM over the 15 grid shapes (x ~ N(0,1),
    W ~ N(0, 0.02^2) from torch's device generator), with each shape's
    roofline fraction t_roof / t, t_roof = max(FLOP / MFMA peak, bytes / HBM
    peak) over the compulsory bytes."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    rows = []
    V = GRID_V
    for K in GRID_K:
        W = (torch.randn(V, K, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
        for M in GRID_M:
            x = torch.randn(M, K, device="cuda", generator=gen).to(torch.bfloat16)
            o32 = torch.empty((M, V), dtype=torch.float32, device="cuda")
            o16 = torch.empty((M, V), dtype=torch.bfloat16, device="cuda")
            fns = {"fp32": lambda: lmh.lmhead_logits(x, W, out=o32, out_dtype="fp32"),
                   "bf16": lambda: lmh.lmhead_logits(x, W, out=o16, out_dtype="bf16")}
            for _ in range(10):
                fns["fp32"]()
                fns["bf16"]()
            tm = alternate(torch, samples, fns)
            flop = 2.0 * M * K * V
            r = {"M": M, "K": K, "V": V}
            for name, osz in (("fp32", 4), ("bf16", 2)):
                med, p10, p90 = quantiles(tm.ms(name))
                nbytes = 2.0 * M * K + 2.0 * V * K + osz * M * V
                t_mfma = flop / (PEAK_BF16_TFLOPS * 1e12)
                t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
                r.update({f"{name}_ms": med, f"{name}_p10_ms": p10, f"{name}_p90_ms": p90,
                          f"{name}_tflops": flop / (med * 1e-3) / 1e12,
                          f"{name}_gbps": nbytes / (med * 1e-3) / 1e9,
                          f"{name}_bound": "mfma" if t_mfma >= t_hbm else "hbm",
                          f"{name}_roofline_frac": max(t_mfma, t_hbm) / (med * 1e-3)})
            r["fp32_overhead_pct"] = 100.0 * (r["fp32_ms"] / r["bf16_ms"] - 1.0)
            rows.append(r)
            log(f"[bench]   grid M={M} K={K}: fp32 {r['fp32_ms'] * 1e3:.1f} us "
                f"({r['fp32_roofline_frac'] * 100:.0f} % of {r['fp32_bound']} roofline), "
                f"bf16 {r['bf16_ms'] * 1e3:.1f} us, overhead {r['fp32_overhead_pct']:+.1f} %")
            del x, o32, o16
        del W
    ov = [r["fp32_overhead_pct"] for r in rows]
    ovk = [r["fp32_overhead_pct"] for r in rows if r["K"] >= 8192]
    return {"protocol": "10 warmup pairs, then alternating fp32/bf16 samples; medians, p10/p90",
            "shapes": rows,
            "median_fp32_overhead_pct": statistics.median(ov),
            "median_fp32_overhead_pct_k_ge_8192": statistics.median(ovk),
            "pages_context": {"hardware": "NVIDIA GB300 (another machine; context, not the target)",
                              "median_fp32_overhead_pct": 5.4,
                              "median_fp32_overhead_pct_k_ge_8192": 1.9}}


def cold_vs_warm(torch, lmh, samples, seed):
    """FP32-out logits GEMM at M=128 K=4096 and M=1024 K=8192 (V=32768), warm
    (back to back) and cold: between samples, outside the timed events, a
    512 MiB device write ("cold_write": the evicted operands are replaced by
    dirty lines that the GEMM's traffic then writes back) or a 512 MiB read
    ("cold_read": clean lines) evicts the operands from L2 and the 256 MB
    MALL."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed + 1)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    res = {}
    for M, K in ((128, 4096), (1024, 8192)):
        V = GRID_V
        W = (torch.randn(V, K, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
        x = torch.randn(M, K, device="cuda", generator=gen).to(torch.bfloat16)
        o = torch.empty((M, V), dtype=torch.float32, device="cuda")
        f = lambda: lmh.lmhead_logits(x, W, out=o, out_dtype="fp32")
        for _ in range(10):
            f()
        tm = KernelTimer(torch)
        for i in range(samples):
            tm("warm", f)
        for i in range(samples):
            flush.fill_(i & 0xFF)
            tm("cold_write", f)
        flush.fill_(1)
        for i in range(samples):
            sink = flush.view(torch.int64).sum()
            tm("cold_read", f)
        torch.cuda.synchronize()
        flop = 2.0 * M * K * V
        r = {}
        for name in ("warm", "cold_write", "cold_read"):
            med, p10, p90 = quantiles(tm.ms(name))
            r.update({f"{name}_ms": med, f"{name}_p10_ms": p10, f"{name}_p90_ms": p90,
                      f"{name}_tflops": flop / (med * 1e-3) / 1e12})
        res[f"{M}x{K}x{V}"] = r
        log(f"[bench]   {M}x{K}x{V}: warm {r['warm_ms'] * 1e3:.1f} us, cold (write flush) "
            f"{r['cold_write_ms'] * 1e3:.1f} us, cold (read flush) {r['cold_read_ms'] * 1e3:.1f} us")
        del W, x, o, sink
    del flush
    return res


def sustained_peaks(torch, lmh):
    """What the chip sustains: a register-only MFMA loop (the library's
    diagnostic kernel, two waves per SIMD) on all-ones operands (almost no
    bit switching) and on pseudo-random operands (switching like real data),
    and a 1 GiB device copy."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n_wg, iters = 2 * cus, 20000
    sink = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")
    tm = KernelTimer(torch)
    for kind in ("ones", "random"):
        for _ in range(2):
            lmh.lmhead_diag_mfma_loop(iters, n_wg, sink, operands=kind)
        for _ in range(5):
            tm(kind, lambda: lmh.lmhead_diag_mfma_loop(iters, n_wg, sink, operands=kind))
        torch.cuda.synchronize()
        want = 128.0 * iters if kind == "ones" else 0.0
        if not torch.all(sink == want).item():
            raise RuntimeError(f"MFMA loop diagnostic ({kind}) returned a wrong closed-form value")
    flop = n_wg * lmh.MFMA_LOOP_FLOP_PER_WORKGROUP_ITER * iters
    mfma_tflops = flop / (statistics.median(tm.ms("ones")) * 1e-3) / 1e12
    mfma_rand_tflops = flop / (statistics.median(tm.ms("random")) * 1e-3) / 1e12
    nb = 1 << 30
    src = torch.ones(nb // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    for _ in range(10):
        tm("copy", lambda: dst.copy_(src))
    torch.cuda.synchronize()
    t_copy = statistics.median(tm.ms("copy"))
    del src, dst, sink
    return {"mfma_bf16_loop_tflops": mfma_tflops,
            "mfma_bf16_loop_frac_of_peak": mfma_tflops / PEAK_BF16_TFLOPS,
            "mfma_bf16_loop_random_tflops": mfma_rand_tflops,
            "mfma_bf16_loop_random_frac_of_peak": mfma_rand_tflops / PEAK_BF16_TFLOPS,
            "mfma_loop": f"{n_wg} workgroups x 4 waves x 8 chains x {iters} 32x32x16 MFMAs, "
                         "register operands only; all ones, then pseudo-random BF16 "
                         "(random sign and mantissa)",
            "copy_gbps": 2.0 * nb / (t_copy * 1e-3) / 1e9,
            "copy_frac_of_peak": 2.0 * nb / (t_copy * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "copy": "1 GiB device-to-device copy, read + write bytes"}


def power_under_load(torch, fn, flop, seconds=3.0):
    """Board power (W) and graphics clock (MHz) sampled from the device's
    sensors (amdsmi, through torch.cuda) while fn runs back to back, after a
    one-second settle; with the achieved TFLOPS of that run.  None where the
    sensors cannot be read."""
    try:
        torch.cuda.power_draw()
        torch.cuda.clock_rate()
    except Exception:  # no sensor access: report nothing rather than guess
        return None
    fn()
    torch.cuda.synchronize()
    pw, ck = [], []
    t0 = time.time()
    n = 0
    while time.time() - t0 < seconds:
        for _ in range(10):
            fn()
        n += 10
        if time.time() - t0 > 1.0:
            pw.append(float(torch.cuda.power_draw()))
            ck.append(float(torch.cuda.clock_rate()))
        if n % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    dt = time.time() - t0
    if not pw:
        return None
    return {"power_w": statistics.median(pw), "clock_mhz": statistics.median(ck),
            "samples": len(pw), "tflops": flop * n / dt / 1e12}


def power_cap_w(torch):
    """The board's power cap in W (amdsmi), or None."""
    try:
        import amdsmi

        handle = torch.cuda._get_amdsmi_handler(0)
        cap = amdsmi.amdsmi_get_power_cap_info(handle)["power_cap"]
        cap = float(cap)
        return cap / 1e6 if cap > 1e5 else cap  # the library reports microwatts
    except Exception:
        return None


def vendor_context(torch, x, W, M, K, V, samples):
    """The vendor BLAS (torch.mm -> hipBLASLt) on the step's shape with a
    BF16 output, for context only: it is not part of the path."""
    y = torch.empty((M, V), dtype=torch.bfloat16, device="cuda")
    for _ in range(5):
        torch.mm(x, W.t(), out=y)
    tm = KernelTimer(torch)
    for _ in range(samples):
        tm("mm", lambda: torch.mm(x, W.t(), out=y))
    torch.cuda.synchronize()
    med, p10, p90 = quantiles(tm.ms("mm"))
    del y
    return {"what": "torch.mm (hipBLASLt), BF16 x BF16 -> BF16 out, same x and W as the step",
            "ms_median": med, "p10_ms": p10, "p90_ms": p90,
            "tflops": 2.0 * M * K * V / (med * 1e-3) / 1e12}


def step_full(torch, lmh, steps, seed, M, K, V, w_sigma, ignore_frac):
    """One whole step at (M, K, V) (x ~ N(0,1), W ~ N(0, w_sigma^2) BF16 from
    torch's device generator, targets uniform with round(ignore_frac * M) rows
    ignored): FP32 logits -> 1/n_valid -> CE fwd + bwd (BF16 dlogits; one
    logits read up to 65536 columns, forward then backward beyond) -> mean ->
    dgrad -> wgrad: the wall time per step over `steps` steps after one
    warmup, with no timing events, then per-kernel HIP-event times (medians)
    over as many steps again."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed + 5)
    x = torch.randn(M, K, device="cuda", generator=gen).to(torch.bfloat16)
    W = (torch.randn(V, K, device="cuda", generator=gen) * w_sigma).to(torch.bfloat16)
    tgt = torch.randint(0, V, (M,), device="cuda", generator=gen, dtype=torch.int32)
    n_ign = int(round(ignore_frac * M))
    if n_ign:
        tgt[torch.randperm(M, device="cuda", generator=gen)[:n_ign]] = -100
    logits = torch.empty((M, V), dtype=torch.float32, device="cuda")
    loss = torch.empty((M,), dtype=torch.float32, device="cuda")
    stats = torch.empty((M, 4), dtype=torch.float32, device="cuda")
    mean = torch.empty((1,), dtype=torch.float32, device="cuda")
    inv = torch.empty((1,), dtype=torch.float32, device="cuda")
    dlog = torch.empty((M, V), dtype=torch.bfloat16, device="cuda")
    dX = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    dW = torch.empty((V, K), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(lmh.lmhead_dgrad_workspace_bytes(M, K, V), 16), dtype=torch.uint8,
                     device="cuda")

    def one(tm):
        tm("logits", lambda: lmh.lmhead_logits(x, W, out=logits, out_dtype="fp32"))
        tm("xent_inv", lambda: lmh.lmhead_xent_mean(None, tgt, -100, inv_nvalid=inv))
        tm("xent_fused", lambda: lmh.lmhead_xent_fused(logits, tgt, inv, -100, dlogits=dlog,
                                                       grad_dtype="bf16", loss=loss, stats=stats))
        tm("xent_mean", lambda: lmh.lmhead_xent_mean(loss, tgt, -100, mean=mean, inv_nvalid=inv))
        tm("dgrad", lambda: lmh.lmhead_dgrad(dlog, W, dX=dX, dx_dtype="bf16", workspace=ws))
        tm("wgrad", lambda: lmh.lmhead_wgrad(dlog, x, dW=dW))

    one(KernelTimer(torch))
    torch.cuda.synchronize()
    quiet = KernelTimer(torch, only=())
    t0 = time.perf_counter()
    for _ in range(steps):
        one(quiet)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    tm = KernelTimer(torch)
    for _ in range(steps):
        one(tm)
    torch.cuda.synchronize()
    flop = 2.0 * M * K * V
    res = {"workload": f"M={M} K={K} V={V} full step, {n_ign} rows ignored",
           "ms_per_step": 1e3 * wall, "gemm_tflops_per_step": 3 * flop / wall / 1e12}
    for name in ("logits", "xent_inv", "xent_fused", "xent_mean", "dgrad", "wgrad"):
        med = statistics.median(tm.ms(name))
        res[f"{name}_ms"] = med
        if name in ("logits", "dgrad", "wgrad"):
            res[f"{name}_tflops"] = flop / (med * 1e-3) / 1e12
    n, nv = M * V, (M - n_ign) * V
    if V <= 65536:  # one read of the logits
        ce_bytes = 4.0 * n + 2.0 * n + 24 * M
    else:           # forward, then backward (ignored rows are not re-read)
        ce_bytes = 4.0 * n + 24 * M + 4.0 * nv + 2.0 * n + 24 * M
    res["ce_fwd_bwd_gbps"] = ce_bytes / (res["xent_fused_ms"] * 1e-3) / 1e9
    del x, W, tgt, logits, loss, stats, mean, inv, dlog, dX, dW, ws
    torch.cuda.empty_cache()
    return res


def host_cpu_share():
    """Threads the oracle may use here: the CPUs this process may run on,
    capped by OMP_NUM_THREADS when set (a host shared by several GPUs sets it
    to each GPU's CPU share)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_baseline(np, workloads, inp, M, K, V):
    """The FP64 oracle (as it is) timed on every step of the benchmark's step,
    each on a bounded sample of its work, on `threads` host threads and on
    one, and extrapolated linearly to the whole step (the work of every step
    is proportional to the rows sampled).  Inputs: the step's x, W and
    targets; for the CE steps, logits N(0, 1.8^2) of the step's shape (the
    logit spread of this workload); for dgrad and wgrad, BF16 dlogits
    N(0, (1e-3)^2).  Nothing here comes from the GPU."""
    import oracle

    thr = host_cpu_share()
    rng = np.random.default_rng(workloads.SEED + 77)
    n_ce = M
    ce = workloads.xent_logits(n_ce, V, sigma=1.8, spike_frac=0.0, ignore_frac=0.0,
                               seed=workloads.SEED + 78)
    dl = workloads.normal_bf16(rng, (M, V), 1e-3)
    flop = 2.0 * M * K * V
    ce_fwd_bytes = 4.0 * M * V + 24 * M
    ce_bwd_bytes = 4.0 * M * V + 2.0 * M * V + 24 * M

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    res = {}
    for label, nt in (("all", thr), ("one", 1)):
        g_rows = 8 * nt            # rows of M for the logits GEMM and dgrad
        w_rows = 64 * nt           # rows of V for wgrad
        c_rows = min(n_ce, 128 * nt)
        rows_m = np.linspace(0, M - 1, g_rows).astype(np.int64)
        rows_v = np.linspace(0, V - 1, w_rows).astype(np.int64)
        zc, tc = ce.logits[:c_rows], ce.target[:c_rows]
        log(f"[bench] cpu baseline ({nt} threads): logits {g_rows}/{M} rows, CE {c_rows}/{M} "
            f"rows, dgrad {g_rows}/{M} rows, wgrad {w_rows}/{V} rows")
        t_log = timed(lambda: oracle.logits(inp.x, inp.W, rows=rows_m, with_abs=False,
                                            nthreads=nt))
        st = []
        t_fwd = timed(lambda: st.append(oracle.xent_fwd(zc, tc, -100, nthreads=nt)))
        full_loss = np.resize(st[0][:, 3], M)
        t_mean = timed(lambda: oracle.xent_mean(full_loss, np.resize(tc, M), -100))
        t_bwd = timed(lambda: oracle.xent_bwd(zc, tc, -100, 1.0 / M, nthreads=nt))
        t_dg = timed(lambda: oracle.dgrad(dl, inp.W, rows=rows_m, with_abs=False, nthreads=nt))
        t_wg = timed(lambda: oracle.wgrad(dl, inp.x, rows=rows_v, with_abs=False, nthreads=nt))
        steps = {
            "logits": (t_log, M / g_rows, flop, "flop"),
            "xent_fwd": (t_fwd, M / c_rows, ce_fwd_bytes, "bytes"),
            "xent_mean": (t_mean, 1.0, None, None),
            "xent_bwd": (t_bwd, M / c_rows, ce_bwd_bytes, "bytes"),
            "dgrad": (t_dg, M / g_rows, flop, "flop"),
            "wgrad": (t_wg, V / w_rows, flop, "flop"),
        }
        per = {}
        for name, (t, scale, work, kind) in steps.items():
            full = t * scale
            e = {"sample_s": round(t, 4), "extrapolated_s": round(full, 3)}
            if kind == "flop":
                e["gflops"] = round(work / full / 1e9, 3)
            elif kind == "bytes":
                e["gbps"] = round(work / full / 1e9, 4)
            per[name] = e
        res[label] = {"threads": nt, "steps": per,
                      "step_s_extrapolated": round(sum(v["extrapolated_s"] for v in per.values()),
                                                   2),
                      "sample_s": round(sum(v["sample_s"] for v in per.values()), 2)}
        log(f"[bench]   {nt} threads: step {res[label]['step_s_extrapolated']:.1f} s "
            f"(extrapolated), logits {per['logits']['gflops']:.1f} GFLOPS, sampled in "
            f"{res[label]['sample_s']:.1f} s")
    allc = res["all"]
    return {
        "value": round(allc["steps"]["logits"]["gflops"] / 1e3, 6), "unit": "TFLOPS",
        "cores": thr, "kind": "oracle",
        "sample": f"FP64 oracle, every step of the M={M} K={K} V={V} step on a row sample, "
                  f"extrapolated: logits and dgrad {8 * thr} of {M} token rows, CE forward and "
                  f"backward {min(n_ce, 128 * thr)} of {M} rows of {V}, wgrad {64 * thr} of {V} "
                  f"vocabulary rows; value = the logits GEMM on {thr} threads",
        "host_cpus_seen": os.cpu_count(),
        "threads_note": "threads = the CPUs this process may use, capped by OMP_NUM_THREADS",
        "all_threads": allc, "one_thread": res["one"],
        "step_ms_extrapolated_all_threads": round(1e3 * allc["step_s_extrapolated"], 1),
    }


def dev_bf16(torch, np, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the multi-GPU layout is described in the design notes, not built.", flush=True)
        return 2

    import numpy as np
    import torch

    import lm_head_fp32_amd as lmh
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    lmh.lib()
    torch.cuda.set_device(0)
    dev_name = torch.cuda.get_device_name(0)
    if args.grid_only:
        log("[bench] the pages' GEMM grid only")
        print(json.dumps({"gemm_grid_fp32_vs_bf16": gemm_grid(torch, lmh, args.samples,
                                                              workloads.SEED)}), flush=True)
        return 0

    # ------------------------------------------------------------ the step
    M, K, V = 1024, 8192, 32768
    log(f"[bench] generating lmhead_1024 inputs M={M} K={K} V={V}")
    inp = workloads.lmhead_1024()
    x = dev_bf16(torch, np, inp.x)
    W = dev_bf16(torch, np, inp.W)
    tgt = torch.from_numpy(inp.target).cuda()
    logits = torch.empty((M, V), dtype=torch.float32, device="cuda")
    logits_b = torch.empty((M, V), dtype=torch.bfloat16, device="cuda")
    loss = torch.empty((M,), dtype=torch.float32, device="cuda")
    stats = torch.empty((M, 4), dtype=torch.float32, device="cuda")
    mean = torch.empty((1,), dtype=torch.float32, device="cuda")
    inv = torch.empty((1,), dtype=torch.float32, device="cuda")
    dlog = torch.empty((M, V), dtype=torch.bfloat16, device="cuda")
    dX = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    dW = torch.empty((V, K), dtype=torch.float32, device="cuda")
    # dgrad's V-split workspace (FP32 partials), allocated once
    ws_dgrad = torch.empty(max(lmh.lmhead_dgrad_workspace_bytes(M, K, V), 16), dtype=torch.uint8,
                           device="cuda")
    torch.cuda.synchronize()

    def step(tm):
        """The single-read step: 1/n_valid depends on the targets only, so the
        forward and backward share one read of the logits."""
        tm("logits", lambda: lmh.lmhead_logits(x, W, out=logits, out_dtype="fp32"))
        tm("xent_inv", lambda: lmh.lmhead_xent_mean(None, tgt, -100, inv_nvalid=inv))
        tm("xent_fused", lambda: lmh.lmhead_xent_fused(logits, tgt, inv, -100, dlogits=dlog,
                                                       grad_dtype="bf16", loss=loss, stats=stats))
        tm("xent_mean", lambda: lmh.lmhead_xent_mean(loss, tgt, -100, mean=mean, inv_nvalid=inv))
        tm("dgrad", lambda: lmh.lmhead_dgrad(dlog, W, dX=dX, dx_dtype="bf16", workspace=ws_dgrad))
        tm("wgrad", lambda: lmh.lmhead_wgrad(dlog, x, dW=dW))

    def step_two_read(tm):
        """The same step with the cross-entropy as two passes over the logits."""
        tm("logits", lambda: lmh.lmhead_logits(x, W, out=logits, out_dtype="fp32"))
        tm("xent_fwd", lambda: lmh.lmhead_xent_fwd(logits, tgt, -100, loss=loss, stats=stats))
        tm("xent_mean", lambda: lmh.lmhead_xent_mean(loss, tgt, -100, mean=mean, inv_nvalid=inv))
        tm("xent_bwd", lambda: lmh.lmhead_xent_bwd(logits, stats, tgt, inv, -100, dlogits=dlog,
                                                   grad_dtype="bf16"))
        tm("dgrad", lambda: lmh.lmhead_dgrad(dlog, W, dX=dX, dx_dtype="bf16", workspace=ws_dgrad))
        tm("wgrad", lambda: lmh.lmhead_wgrad(dlog, x, dW=dW))

    def run_steps(fn, n, only=None):
        tm = KernelTimer(torch, only)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn(tm)
        torch.cuda.synchronize()
        return tm, 1e3 * (time.perf_counter() - t0) / max(n, 1)

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(KernelTimer(torch))
    torch.cuda.synchronize()
    # The timed steps carry events around the logits GEMM only (its launches
    # give `roofline.achieved`): a pair of timing events around every launch
    # adds ~37 us to this step.  The per-kernel breakdown comes from the same
    # number of steps run right after, with events around every launch.
    log(f"[bench] timing {args.steps} steps")
    tm, ms_step = run_steps(step, args.steps, only=("logits",))
    tmk, ms_step_ev = run_steps(step, args.steps)

    flop = 2.0 * M * K * V
    n_valid_step = int((tgt != -100).sum().item())

    def kernel_table(tm, names):
        kern = {}
        for name in names:
            ts = tm.ms(name)
            kern[name] = {"ms_mean": statistics.fmean(ts), "ms_median": statistics.median(ts),
                          "ms_min": min(ts)}
        for name in ("logits", "dgrad", "wgrad"):
            if name not in kern:
                continue
            kern[name]["tflops"] = flop / (kern[name]["ms_mean"] * 1e-3) / 1e12
            kern[name]["frac_mfma_peak"] = kern[name]["tflops"] / PEAK_BF16_TFLOPS
        return kern

    kern = kernel_table(tmk, ("logits", "xent_inv", "xent_fused", "xent_mean", "dgrad", "wgrad"))
    kern["logits"] = kernel_table(tm, ("logits",))["logits"]  # from the timed steps
    kern_note = ("logits: the timed steps; the other kernels: as many steps again with events "
                 f"around every launch ({ms_step_ev:.4f} ms per step)")
    # one read of the FP32 logits, the BF16 gradient written, 24 B per row
    ce_one_bytes = 4.0 * M * V + 2.0 * M * V + 24 * M
    kern["xent_fused"]["gbps"] = ce_one_bytes / (kern["xent_fused"]["ms_mean"] * 1e-3) / 1e9
    kern["xent_fused"]["frac_hbm_peak"] = kern["xent_fused"]["gbps"] / PEAK_HBM_GBS
    kern["xent_fused"]["algorithmic_bytes"] = int(ce_one_bytes)
    kern["xent_fused"]["traffic"] = measured_traffic("xent_fused_bf16_1024x32768")
    logits_tflops = kern["logits"]["tflops"]
    log(f"[bench] step {ms_step:.3f} ms; logits {kern['logits']['ms_mean']:.3f} ms "
        f"= {logits_tflops:.1f} TFLOPS; CE (one read) {kern['xent_fused']['ms_mean'] * 1e3:.1f} us")

    out = {
        "metric": METRIC,
        "value": round(logits_tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "lm-head step M=1024 K=8192 V=32768: fp32 logits -> 1/n_valid -> CE fwd "
                        "+ bwd in one logits read (bf16 dlogits) -> mean -> dgrad -> wgrad; plus "
                        "CE fwd+bwd on fp32 logits 8192x131072",
            "M": M, "K": K, "V": V, "global_batch": M, "parallelism": "none (1 GPU)",
            "device": dev_name,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "lmhead_logits (fp32 out)",
            "achieved": round(logits_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(logits_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic("logits_fp32"),
            "algorithmic_bytes": int(2 * M * K + 2 * V * K + 4 * M * V),
        },
        "kernels": kern,
        "kernels_note": kern_note,
    }

    # The same step with the cross-entropy reading the logits twice (forward,
    # then backward), timed the same way right after.
    log(f"[bench] the two-read step, {args.steps} steps")
    for _ in range(2):
        step_two_read(KernelTimer(torch))
    _, ms_step2 = run_steps(step_two_read, args.steps, only=())
    tm2, ms_step2_ev = run_steps(step_two_read, args.steps)
    kern2 = kernel_table(tm2, ("logits", "xent_fwd", "xent_mean", "xent_bwd", "dgrad", "wgrad"))
    ce_two_bytes = (4.0 * M * V + 24 * M) + (4.0 * n_valid_step * V + 2.0 * M * V + 24 * M)
    ce_two_ms = kern2["xent_fwd"]["ms_mean"] + kern2["xent_bwd"]["ms_mean"]
    out["step_two_read"] = {
        "ms_per_step": round(ms_step2, 4), "kernels": kern2,
        "kernels_note": ("as many steps again with events around every launch "
                         f"({ms_step2_ev:.4f} ms per step)"),
        "ce_ms": ce_two_ms, "ce_gbps": ce_two_bytes / (ce_two_ms * 1e-3) / 1e9,
        "ce_one_read_ms": kern["xent_fused"]["ms_mean"],
        "ce_speedup_one_read": ce_two_ms / kern["xent_fused"]["ms_mean"],
        "step_saved_ms": ms_step2 - ms_step}
    log(f"[bench]   two-read step {ms_step2:.3f} ms (CE {ce_two_ms * 1e3:.1f} us) vs one-read "
        f"{ms_step:.3f} ms (CE {kern['xent_fused']['ms_mean'] * 1e3:.1f} us)")

    # ----------------------------------------------------- side measurements
    if not args.no_side:
        # FP32 vs BF16 epilogue, the pages' protocol
        log("[bench] fp32-out vs bf16-out logits, 10 warmup pairs + alternating samples")
        for _ in range(10):
            lmh.lmhead_logits(x, W, out=logits, out_dtype="fp32")
            lmh.lmhead_logits(x, W, out=logits_b, out_dtype="bf16")
        side = KernelTimer(torch)
        for i in range(args.samples):
            order = ("fp32", "bf16") if i % 2 == 0 else ("bf16", "fp32")
            for o in order:
                side(o, lambda o=o: lmh.lmhead_logits(x, W, out=logits if o == "fp32" else logits_b,
                                                       out_dtype=o))
        torch.cuda.synchronize()
        f32 = statistics.median(side.ms("fp32"))
        b16 = statistics.median(side.ms("bf16"))
        out["logits_fp32_vs_bf16"] = {
            "fp32_ms_median": f32, "bf16_ms_median": b16,
            "fp32_tflops": flop / (f32 * 1e-3) / 1e12, "bf16_tflops": flop / (b16 * 1e-3) / 1e12,
            "fp32_overhead_pct": 100.0 * (f32 / b16 - 1.0),
        }
        del logits_b
        # CE forward statistics from the logits GEMM's epilogue (records per
        # 256-column block, then the merge) against logits then the one-pass
        # forward (which reads the 128 MiB of logits once more).
        log("[bench] logits + CE forward: separate vs records in the GEMM epilogue")
        tgt_e = torch.from_numpy(inp.target).cuda()
        nparts = (V + 255) // 256
        part = torch.empty((nparts, M, 4), dtype=torch.float32, device="cuda")
        el = torch.empty((M,), dtype=torch.float32, device="cuda")
        es = torch.empty((M, 4), dtype=torch.float32, device="cuda")
        sep = lambda: (lmh.lmhead_logits(x, W, out=logits, out_dtype="fp32"),
                       lmh.lmhead_xent_fwd(logits, tgt_e, -100, loss=el, stats=es))
        epi = lambda: (lmh.lmhead_logits_xent(x, W, tgt_e, -100, out=logits, part=part),
                       lmh.lmhead_xent_merge(part, tgt_e, V, -100, loss=el, stats=es))
        for _ in range(5):
            sep()
            epi()
        etm = KernelTimer(torch)
        for i in range(args.samples):
            for name, fn in ((("sep", sep), ("epi", epi)) if i % 2 == 0 else (("epi", epi), ("sep", sep))):
                etm(name, fn)
            etm("gemm_stats", lambda: lmh.lmhead_logits_xent(x, W, tgt_e, -100, out=logits, part=part))
            etm("gemm", lambda: lmh.lmhead_logits(x, W, out=logits, out_dtype="fp32"))
        torch.cuda.synchronize()
        tsep, tepi = statistics.median(etm.ms("sep")), statistics.median(etm.ms("epi"))
        tgs, tg = statistics.median(etm.ms("gemm_stats")), statistics.median(etm.ms("gemm"))
        out["logits_ce_fwd_epilogue_stats"] = {
            "logits_then_xent_fwd_ms": tsep, "logits_with_records_then_merge_ms": tepi,
            "saved_pct": 100.0 * (1.0 - tepi / tsep),
            "gemm_ms": tg, "gemm_with_records_ms": tgs,
            "epilogue_overhead_pct": 100.0 * (tgs / tg - 1.0)}
        log(f"[bench]   separate {tsep:.3f} ms, epilogue records {tepi:.3f} ms "
            f"(GEMM {tg:.3f} -> {tgs:.3f} ms)")
        del part, el, es, tgt_e
        # Large-vocabulary CE
        n_ce, v_ce = args.ce_rows, 131072
        log(f"[bench] generating CE logits {n_ce}x{v_ce}")
        ce = workloads.xent_logits(n_ce, v_ce, sigma=3.0, spike_frac=0.01, spike=30.0,
                                   ignore_frac=0.02, seed=workloads.SEED)
        z = torch.from_numpy(ce.logits).cuda()
        ct = torch.from_numpy(ce.target).cuda()
        del ce
        cl = torch.empty((n_ce,), dtype=torch.float32, device="cuda")
        cs = torch.empty((n_ce, 4), dtype=torch.float32, device="cuda")
        cm = torch.empty((1,), dtype=torch.float32, device="cuda")
        ci = torch.empty((1,), dtype=torch.float32, device="cuda")
        g32 = torch.empty((n_ce, v_ce), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        log("[bench] CE fwd + bwd samples")
        for _ in range(3):
            lmh.lmhead_xent_fwd(z, ct, -100, loss=cl, stats=cs)
            lmh.lmhead_xent_mean(cl, ct, -100, mean=cm, inv_nvalid=ci)
            lmh.lmhead_xent_bwd(z, cs, ct, ci, -100, dlogits=g32)
        ctm = KernelTimer(torch)
        for _ in range(args.samples):
            ctm("fwd", lambda: lmh.lmhead_xent_fwd(z, ct, -100, loss=cl, stats=cs))
            lmh.lmhead_xent_mean(cl, ct, -100, mean=cm, inv_nvalid=ci)
            ctm("bwd", lambda: lmh.lmhead_xent_bwd(z, cs, ct, ci, -100, dlogits=g32))
        torch.cuda.synchronize()
        fwd_ms = statistics.median(ctm.ms("fwd"))
        bwd_ms = statistics.median(ctm.ms("bwd"))
        # The backward writes every row but reads only rows whose target is
        # not ignored (an ignored row's gradient is zero).
        n_valid = int((ct != -100).sum().item())
        fwd_b = 4.0 * n_ce * v_ce + 24 * n_ce
        bwd_b = 4.0 * n_valid * v_ce + 4.0 * n_ce * v_ce + 24 * n_ce
        ce_gbps = (fwd_b + bwd_b) / ((fwd_ms + bwd_ms) * 1e-3) / 1e9
        # BF16 gradients, then in place over a copy restored outside the timing
        gb = torch.empty((n_ce, v_ce), dtype=torch.bfloat16, device="cuda")
        for _ in range(2):
            lmh.lmhead_xent_bwd(z, cs, ct, ci, -100, dlogits=gb, grad_dtype="bf16")
        for _ in range(args.samples):
            ctm("bwd_bf16", lambda: lmh.lmhead_xent_bwd(z, cs, ct, ci, -100, dlogits=gb,
                                                        grad_dtype="bf16"))
        torch.cuda.synchronize()
        del gb
        bwd16_ms = statistics.median(ctm.ms("bwd_bf16"))
        n_inplace = min(args.samples, 10)
        for _ in range(n_inplace):
            g32.copy_(z)  # restore pristine logits, outside the timed events
            ctm("bwd_inplace", lambda: lmh.lmhead_xent_bwd(g32, cs, ct, ci, -100, in_place=True))
        torch.cuda.synchronize()
        bwdip_ms = statistics.median(ctm.ms("bwd_inplace"))
        out["roofline_ce"] = {
            "bound": "hbm",
            "kernel": "lmhead_xent_fwd + lmhead_xent_bwd (fp32 grads, out of place)",
            "workload": f"fp32 logits {n_ce}x{v_ce}",
            "achieved": round(ce_gbps, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(ce_gbps / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic("xent_fwd_bwd_fp32") if n_ce == 8192 else None,
            "algorithmic_bytes": int(fwd_b + bwd_b),
            "fwd_ms_median": fwd_ms, "bwd_ms_median": bwd_ms,
            "fwd_gbps": fwd_b / (fwd_ms * 1e-3) / 1e9, "bwd_gbps": bwd_b / (bwd_ms * 1e-3) / 1e9,
            "bwd_bf16_ms_median": bwd16_ms,
            "bwd_bf16_gbps": (4.0 * n_valid * v_ce + 2.0 * n_ce * v_ce + 24 * n_ce)
            / (bwd16_ms * 1e-3) / 1e9,
            "bwd_inplace_ms_median": bwdip_ms,
            "bwd_inplace_gbps": bwd_b / (bwdip_ms * 1e-3) / 1e9,
        }
        log(f"[bench] CE fwd {fwd_ms:.3f} ms bwd {bwd_ms:.3f} ms -> {ce_gbps:.0f} GB/s")
        del g32
        # Split-vocabulary forward (per-block partial statistics + merge) beside
        # the one-pass forward: the 8192 x 131072 logits above, and N(0, 3^2)
        # logits of 128 and 1024 rows x 32768 (few rows: one workgroup per row
        # leaves most of the 256 CUs idle).
        log("[bench] CE forward: one pass vs split vocabulary (4096-column blocks)")
        split = {}
        gen = torch.Generator(device="cuda")
        gen.manual_seed(workloads.SEED)
        for n_s, v_s in ((128, 32768), (1024, 32768), (n_ce, v_ce)):
            if (n_s, v_s) == (n_ce, v_ce):
                zs, ts = z, ct
            else:
                zs = torch.randn((n_s, v_s), device="cuda", generator=gen) * 3.0
                ts = torch.randint(0, v_s, (n_s,), device="cuda", generator=gen,
                                   dtype=torch.int32)
            ls = torch.empty((n_s,), dtype=torch.float32, device="cuda")
            ss = torch.empty((n_s, 4), dtype=torch.float32, device="cuda")
            nb_s = (v_s + 4095) // 4096
            ps = torch.empty((nb_s, n_s, 4), dtype=torch.float32, device="cuda")
            one = lambda: lmh.lmhead_xent_fwd(zs, ts, -100, loss=ls, stats=ss)
            two = lambda: (lmh.lmhead_xent_partial(zs, ts, -100, block_cols=4096, part=ps),
                           lmh.lmhead_xent_merge(ps, ts, v_s, -100, loss=ls, stats=ss))
            for _ in range(3):
                one()
                two()
            stm = KernelTimer(torch)
            for i in range(args.samples):
                for name, fn in ((("one", one), ("split", two)) if i % 2 == 0
                                 else (("split", two), ("one", one))):
                    stm(name, fn)
            torch.cuda.synchronize()
            by = 4.0 * n_s * v_s + 24 * n_s
            t1, t2 = statistics.median(stm.ms("one")), statistics.median(stm.ms("split"))
            split[f"{n_s}x{v_s}"] = {"one_pass_ms": t1, "split_ms": t2,
                                     "one_pass_gbps": by / (t1 * 1e-3) / 1e9,
                                     "split_gbps": by / (t2 * 1e-3) / 1e9}
            log(f"[bench]   {n_s}x{v_s}: one pass {t1 * 1e3:.1f} us, split {t2 * 1e3:.1f} us")
            del zs, ts, ls, ss, ps
        out["xent_fwd_split_vocab"] = split
        del z
        # Single-read forward + backward (upstream gradient known in advance)
        # beside forward then backward, BF16 and FP32 gradients.
        log("[bench] CE forward+backward: two reads vs one (fused)")
        fused = {}
        for n_s, v_s in ((128, 32768), (1024, 32768)):
            zs = torch.randn((n_s, v_s), device="cuda", generator=gen) * 3.0
            ts = torch.randint(0, v_s, (n_s,), device="cuda", generator=gen, dtype=torch.int32)
            ls = torch.empty((n_s,), dtype=torch.float32, device="cuda")
            ss = torch.empty((n_s, 4), dtype=torch.float32, device="cuda")
            dls = torch.full((1,), 1.0 / n_s, device="cuda")
            for gname, gdt, gsz in (("bf16", torch.bfloat16, 2), ("fp32", torch.float32, 4)):
                gs = torch.empty((n_s, v_s), dtype=gdt, device="cuda")
                two = lambda: (lmh.lmhead_xent_fwd(zs, ts, -100, loss=ls, stats=ss),
                               lmh.lmhead_xent_bwd(zs, ss, ts, dls, -100, dlogits=gs,
                                                   grad_dtype=gname))
                one = lambda: lmh.lmhead_xent_fused(zs, ts, dls, -100, dlogits=gs,
                                                    grad_dtype=gname, loss=ls, stats=ss)
                for _ in range(3):
                    two()
                    one()
                ftm = KernelTimer(torch)
                for i in range(args.samples):
                    for name, fn in ((("two", two), ("one", one)) if i % 2 == 0
                                     else (("one", one), ("two", two))):
                        ftm(name, fn)
                torch.cuda.synchronize()
                t2, t1 = statistics.median(ftm.ms("two")), statistics.median(ftm.ms("one"))
                b2 = (8.0 + gsz) * n_s * v_s + 48 * n_s
                b1 = (4.0 + gsz) * n_s * v_s + 24 * n_s
                fused[f"{n_s}x{v_s}_{gname}"] = {
                    "two_read_ms": t2, "fused_ms": t1, "speedup": t2 / t1,
                    "two_read_gbps": b2 / (t2 * 1e-3) / 1e9, "fused_gbps": b1 / (t1 * 1e-3) / 1e9}
                log(f"[bench]   {n_s}x{v_s} {gname}: fwd+bwd {t2 * 1e3:.1f} us, fused "
                    f"{t1 * 1e3:.1f} us")
                del gs
            del zs, ts, ls, ss, dls
        out["xent_fused_vs_two_read"] = fused

    # ------------------------- the pages' GEMM grid, cold/warm, sustained peaks
    if not args.no_side and not args.no_grid:
        log("[bench] the pages' GEMM grid (M x K at V=32768), fp32-out vs bf16-out")
        out["gemm_grid_fp32_vs_bf16"] = gemm_grid(torch, lmh, args.samples, workloads.SEED)
        g = out["gemm_grid_fp32_vs_bf16"]
        log(f"[bench]   median fp32-out overhead {g['median_fp32_overhead_pct']:+.2f} % "
            f"(K >= 8192: {g['median_fp32_overhead_pct_k_ge_8192']:+.2f} %)")
        log("[bench] logits GEMM cold vs warm")
        out["logits_cold_vs_warm"] = cold_vs_warm(torch, lmh, args.samples, workloads.SEED)
    if not args.no_side and not args.no_grid:
        log("[bench] the full step at M=4096 K=16384 V=131072")
        out["step_4096"] = step_full(torch, lmh, 3, workloads.SEED, 4096, 16384, 131072, 0.01,
                                     0.0)
        s4 = out["step_4096"]
        log(f"[bench]   {s4['ms_per_step']:.2f} ms per step; logits {s4['logits_tflops']:.0f}, "
            f"dgrad {s4['dgrad_tflops']:.0f}, wgrad {s4['wgrad_tflops']:.0f} TFLOPS; CE "
            f"{s4['ce_fwd_bwd_gbps']:.0f} GB/s")
        log("[bench] one GPU's token shard of that step (M=512 of 4096, eight GPUs)")
        out["step_4096_token_shard_of_8"] = step_full(torch, lmh, 3, workloads.SEED, 512, 16384,
                                                      131072, 0.01, 0.0)
        s8 = out["step_4096_token_shard_of_8"]
        log(f"[bench]   {s8['ms_per_step']:.2f} ms per step; logits {s8['logits_tflops']:.0f}, "
            f"dgrad {s8['dgrad_tflops']:.0f}, wgrad {s8['wgrad_tflops']:.0f} TFLOPS")
        log("[bench] the full step at M=128 K=4096 V=32768 (5 % rows ignored)")
        out["step_128"] = step_full(torch, lmh, 20, workloads.SEED, 128, 4096, 32768, 0.02, 0.05)
        s1 = out["step_128"]
        log(f"[bench]   {s1['ms_per_step'] * 1e3:.1f} us per step; logits "
            f"{s1['logits_ms'] * 1e3:.1f}, CE fwd + bwd {s1['xent_fused_ms'] * 1e3:.1f}, dgrad "
            f"{s1['dgrad_ms'] * 1e3:.1f}, wgrad {s1['wgrad_ms'] * 1e3:.1f} us")
    if not args.no_side:
        log("[bench] sustained peaks: MFMA loop, device copy")
        out["sustained_peaks"] = sustained_peaks(torch, lmh)
        sp = out["sustained_peaks"]
        out["roofline"]["sustained_random_operand_tflops"] = round(
            sp["mfma_bf16_loop_random_tflops"], 2)
        out["roofline"]["frac_of_sustained_random"] = round(
            logits_tflops / sp["mfma_bf16_loop_random_tflops"], 4)
        log(f"[bench]   MFMA loop {sp['mfma_bf16_loop_tflops']:.0f} TFLOPS (all-ones operands), "
            f"{sp['mfma_bf16_loop_random_tflops']:.0f} TFLOPS (random operands), copy "
            f"{sp['copy_gbps']:.0f} GB/s")
        log("[bench] board power and clock under load (logits GEMM, MFMA loops)")
        n_wg = 2 * torch.cuda.get_device_properties(0).multi_processor_count
        psink = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")
        loop_flop = n_wg * lmh.MFMA_LOOP_FLOP_PER_WORKGROUP_ITER * 2000
        out["power"] = {
            "cap_w": power_cap_w(torch),
            "logits_gemm_fp32": power_under_load(
                torch, lambda: lmh.lmhead_logits(x, W, out=logits, out_dtype="fp32"),
                2.0 * M * K * V),
            "mfma_loop_random": power_under_load(
                torch, lambda: lmh.lmhead_diag_mfma_loop(2000, n_wg, psink, operands="random"),
                loop_flop),
            "mfma_loop_ones": power_under_load(
                torch, lambda: lmh.lmhead_diag_mfma_loop(2000, n_wg, psink, operands="ones"),
                loop_flop),
        }
        del psink
        pl = out["power"]["logits_gemm_fp32"]
        if pl:
            log(f"[bench]   cap {out['power']['cap_w']} W; logits GEMM {pl['power_w']:.0f} W at "
                f"{pl['clock_mhz']:.0f} MHz, {pl['tflops']:.0f} TFLOPS")
        out["vendor_gemm_context"] = vendor_context(torch, x, W, M, K, V, args.samples)
        log(f"[bench]   vendor BLAS (bf16 out) {out['vendor_gemm_context']['tflops']:.0f} TFLOPS")

    # ------------------------------------------ counter calibration copy
    if args.calib_copy_mib > 0:
        nb = args.calib_copy_mib << 20
        src = torch.ones(nb // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = nb
        del src, dst

    # ------------------------------------------------------- CPU baseline
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(np, workloads, inp, M, K, V)

    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
