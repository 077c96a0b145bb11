"""Benchmark: exact tiled attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload (the headline configuration): B=1, 32 query heads on 8 key/value
heads, N=8192, d=128, bf16 storage, causal, scale 1/sqrt(128); Q, K, V iid
N(0,1) from seed 3 with 1% of key rows per kv head scaled x8.  Inputs are
generated on the host, copied to HBM once, and are resident before timing.

A step is one fa_fwd call over the whole batch.  First a time-based
pre-heat (--preheat-s seconds of untimed launches, reported under
"preheat": the clock needs a few hundred ms of load to reach its sustained
level), then W untimed warm-up steps, then K steps bracketed by device
synchronisation on both sides, with a HIP event recorded on the launch
stream before each step.  Prints one JSON line:
  value     causal-adjusted TFLOP/s = 4*B*H*N^2*d/2 / (wall time per step)
  roofline  the forward kernel against the dense bf16 matrix-core peak; its
            duration is the median of the per-step event times
  sclk      graphics clock sampled during the timed steps (SMU metrics), and
            pct_clock_adjusted_peak = achieved / (peak * sclk / 2400 MHz), or
            null when the samples disagree by more than 10% (stale readings)
  flushed   median step time with a 512 MiB buffer written before each step
            (L2 and Infinity Cache cold)
  cpu_baseline  the float64 oracle on a bounded sample of the same inputs
            (all 32 query heads by default, full causal rows; --cpu-heads
            bounds it), timed on the host cores.
Informational legs (skippable): short sequences, FP8, sliding window, long
context (N=32768) and the backward.  Only one GPU is used: --gpus above 1
exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix-core peak (published)
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 matrix-core peak (published)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E bandwidth (published)
PEAK_SCLK_MHZ = 2400.0        # the clock the published peaks assume
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_c3_traffic.json")
FWD_SOURCES = [os.path.join(ROOT, "exact_tiled_attention_31_amd", "csrc", f)
               for f in ("fwd_bf16.hip", "common.hpp")]


def fwd_source_hash() -> str:
    h = hashlib.sha256()
    for p in FWD_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != fwd_source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(inp, w, heads: int):
    """Time the float64 oracle on `heads` query heads of the same inputs."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()
                            if i.get("user_api") == "blas"), default=1)
    except Exception:   # threadpoolctl absent: report the affinity set
        blas_threads = len(os.sched_getaffinity(0))
    heads = max(1, min(heads, w.H))
    sel = [int(h) for h in np.linspace(0, w.H - 1, heads).round()]
    t0 = time.perf_counter()
    for h in sel:
        g = oracle.kv_head_of(h, w.H, w.Hkv)
        oracle.attention_fwd(inp.q[:, h:h + 1], inp.k[:, g:g + 1], inp.v[:, g:g + 1],
                             w.causal, w.scale)
    dt = time.perf_counter() - t0
    flops = 4.0 * w.B * len(sel) * w.N * w.N * w.d / (2.0 if w.causal else 1.0)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"float64 numpy oracle on {len(sel)} of {w.H} query heads (all "
                      f"{w.N} rows, causal prefix), same seeded inputs; "
                      f"{len(os.sched_getaffinity(0))} host cores visible, "
                      f"BLAS threads {blas_threads}"}


def tile_count_flops(w, rows: int = 32, cols: int = 64) -> float:
    """The pages' tile-count convention (flops counted per computed tile,
    4 * rows * cols * d for each (query tile, key tile) pair that is not
    skipped) for the tile the forward computes: one wave's 32 query rows
    against a 64-key tile; a key tile is skipped when its first key lies after
    the wave's last row."""
    n_q = -(-w.N // rows)
    tiles = 0
    for qt in range(n_q):
        last = min(w.N, (qt + 1) * rows) - 1
        tiles += (last // cols + 1) if w.causal else -(-w.N // cols)
    return 4.0 * rows * cols * w.d * tiles * w.B * w.H


class ClockSampler:
    """Samples the graphics clock (MHz, mean over the XCDs reported by the
    SMU metrics table) in a background thread while a region runs.  Yields
    None when the management library is unavailable."""

    def __init__(self, period_s: float = 0.002):
        self.period = period_s
        self.samples = []
        self.avg_samples = []
        self._stop = None
        self._thread = None
        self._handle = None
        self.error = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            self._handle = amdsmi.amdsmi_get_processor_handles()[0]
            self._read()
        except Exception as e:   # no library, no permission, no device
            self.error = f"{type(e).__name__}: {e}"
            self._handle = None

    def _read(self):
        """(current clock averaged over the XCDs, the SMU's own average
        clock) in MHz; either may be None."""
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._handle)
        xs = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and c > 0]
        cur = sum(xs) / len(xs) if xs else None
        if cur is None:
            c = m.get("current_gfxclk")
            cur = float(c) if isinstance(c, (int, float)) and c > 0 else None
        a = m.get("average_gfxclk_frequency")
        return cur, (float(a) if isinstance(a, (int, float)) and a > 0 else None)

    def __enter__(self):
        import threading
        if self._handle is None:
            return self
        self.samples = []
        self.avg_samples = []
        self._stop = threading.Event()

        def loop():
            while not self._stop.is_set():
                try:
                    cur, avg = self._read()
                    if cur is not None:
                        self.samples.append(cur)
                    if avg is not None:
                        self.avg_samples.append(avg)
                except Exception:
                    pass
                self._stop.wait(self.period)

        self._thread = threading.Thread(target=loop, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        return False

    def summary(self):
        if not self.samples:
            return None
        xs = sorted(self.samples)
        out = {"mean_mhz": round(sum(xs) / len(xs), 1), "min_mhz": xs[0], "max_mhz": xs[-1],
               "samples": len(xs),
               "source": "SMU metrics table (amdsmi), current_gfxclks averaged over the "
                         "XCDs; updated by firmware, so short regions give few distinct "
                         "readings"}
        if self.avg_samples:
            out["smu_average_mhz"] = round(sum(self.avg_samples) / len(self.avg_samples), 1)
        return out


def preheat(torch, call, seconds: float) -> dict:
    """Untimed load until `seconds` of wall time have passed, so the clock
    reaches its sustained level before warm-up and timing (the first tens of
    milliseconds of load run slower)."""
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            call()
        n += 8
        torch.cuda.synchronize()
    return {"seconds": round(time.perf_counter() - t0, 3), "launches": n}


def timed_steps(torch, call, stream, warmup: int, steps: int):
    """W untimed steps, then K steps between device synchronisations, with an
    event recorded on the launch stream before each step and after the last.
    Returns (wall seconds, per-step event times in ms)."""
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i].record(stream)
        call()
    evs[steps].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]


def flushed_steps(torch, call, stream, steps: int, flush_bytes: int):
    """Steps with the L2 and the MALL (Infinity Cache) flushed first: a
    buffer of `flush_bytes` is written on the launch stream before each step,
    and only the step itself is timed (events around the call)."""
    buf = torch.empty(flush_bytes // 4, dtype=torch.float32, device=stream.device)
    times = []
    for i in range(steps):
        buf.fill_(float(i))
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del buf
    return times


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def event_leg(torch, call, stream, warmup, steps, preheat_s):
    """Pre-heat, warm-up, then per-step events: (mean ms, median ms)."""
    if preheat_s > 0:
        preheat(torch, call, preheat_s)
    _, ts = timed_steps(torch, call, stream, warmup, steps)
    return sum(ts) / len(ts), median(ts)


def backward_timing(fa, W, torch, np, dev, warmup, steps, preheat_s):
    """Informational: fa_bwd on the backward workload (B=2 H=16 N=4096 d=128
    causal), timed with HIP events on the launch stream.  The rate counts the
    algorithmic work of the gradient, 2.5x the causal-adjusted forward flops
    (five N x N x d contractions instead of two)."""
    w5 = W.C5
    inp = W.gen_inputs(w5)

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = (to_dev(getattr(inp, n + "_bits")) for n in ("q", "k", "v", "do"))
    stream = torch.cuda.current_stream(dev)
    o, lse = fa.fa_fwd(q, k, v, causal=True, scale=w5.scale, stream=stream)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(16, fa.fa_bwd_workspace_bytes(w5.B, w5.H, w5.Hkv, w5.N, w5.d)),
                     dtype=torch.uint8, device=dev)

    def call():
        fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, causal=True, scale=w5.scale, stream=stream)

    mean_ms, med_ms = event_leg(torch, call, stream, warmup, steps, preheat_s)
    flops = 2.5 * w5.causal_adjusted_flops()
    return {"workload": "backward B=2 H=16 Hkv=16 N=4096 d=128 bf16 causal (seed 5)",
            "ms": round(med_ms, 4), "ms_mean": round(mean_ms, 4),
            "tflops": round(flops / (med_ms * 1e-3) / 1e12, 2),
            "flop_convention": "2.5 * 4*B*H*N^2*d/2", "steps": steps}


def local_timing(fa, w, torch, q, k, v, stream, window, warmup, steps, preheat_s):
    """Informational: fa_fwd_local (window 256, the pages' example width) on
    the headline inputs, timed with HIP events on the launch stream.  The rate
    counts 4*d flops per visible (query, key) pair: sum_i min(i+1, window)
    pairs per head."""
    n = w.N
    pairs = window * (window + 1) // 2 + (n - window) * window if n > window else n * (n + 1) // 2
    flops = 4.0 * w.d * w.B * w.H * pairs

    def call():
        fa.fa_fwd_local(q, k, v, window, scale=w.scale, stream=stream)

    mean_ms, med_ms = event_leg(torch, call, stream, warmup, steps, preheat_s)
    return {"workload": f"local causal forward, window {window}, same inputs as the headline",
            "ms": round(med_ms, 5), "ms_mean": round(mean_ms, 5),
            "tflops": round(flops / (med_ms * 1e-3) / 1e12, 2),
            "flop_convention": "4*d*B*H*sum_i min(i+1, window)", "steps": steps}


def fp8_timing(fa, W, torch, np, dev, stream, warmup, steps, preheat_s):
    """Informational: fa_fwd_fp8 on the headline draws quantized to e4m3 with
    per-tensor scales (same shape, causal), HIP events on the launch stream;
    rate against the dense fp8 matrix-core peak."""
    w = W.F3
    inp = W.gen_inputs(w)
    q, k, v = (torch.from_numpy(getattr(inp, n + "_codes")).to(dev) for n in ("q", "k", "v"))
    ds = inp.descale
    o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

    def call():
        fa.fa_fwd_fp8(q, k, v, ds["q"], ds["k"], ds["v"], o=o, lse=lse, causal=True,
                      scale=w.scale, stream=stream)

    mean_ms, med_ms = event_leg(torch, call, stream, warmup, steps, preheat_s)
    tf = w.causal_adjusted_flops() / (med_ms * 1e-3) / 1e12
    return {"workload": "fp8 e4m3 forward, headline shape and draws, per-tensor scales",
            "ms": round(med_ms, 5), "ms_mean": round(mean_ms, 5), "tflops": round(tf, 2),
            "peak_fp8": PEAK_FP8_TFLOPS, "frac": round(tf / PEAK_FP8_TFLOPS, 4),
            "flop_convention": "4*B*H*N^2*d/2", "steps": steps}


def long_context_timing(fa, W, torch, np, dev, stream, warmup, steps, preheat_s):
    """Informational: the long-context configuration (B=1, 32 query heads on 8
    kv heads, N=32768, d=128, bf16, causal, seed 4), HIP events on the launch
    stream, causal-adjusted flops against the dense bf16 peak."""
    w = W.C4
    inp = W.gen_inputs(w)
    q, k, v = (torch.from_numpy(getattr(inp, x + "_bits").view(np.int16)).view(torch.bfloat16)
               .to(dev) for x in ("q", "k", "v"))
    del inp
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

    def call():
        fa.fa_fwd(q, k, v, o=o, lse=lse, causal=True, scale=w.scale, stream=stream)

    mean_ms, med_ms = event_leg(torch, call, stream, warmup, steps, preheat_s)
    tf = w.causal_adjusted_flops() / (med_ms * 1e-3) / 1e12
    return {"workload": "long-context causal forward B=1 H=32 Hkv=8 N=32768 d=128 bf16 (seed 4)",
            "ms": round(med_ms, 4), "ms_mean": round(mean_ms, 4), "tflops": round(tf, 2),
            "frac": round(tf / PEAK_BF16_TFLOPS, 4), "flop_convention": "4*B*H*N^2*d/2",
            "steps": steps}


def short_n_sweep(fa, W, torch, np, dev, stream, warmup, steps, preheat_s):
    """Informational: the headline head layout (B=1, 32 query heads on 8 kv
    heads, d=128, bf16, causal) at decode-like short sequence lengths.  These
    launches are far too small to be compute-bound; the rate reported is the
    compulsory HBM traffic (Q, K, V read once, O and LSE written once) per
    kernel duration (median of per-step HIP events), against the 8 TB/s HBM
    peak."""
    out = []
    for n in (128, 256, 512, 1024):
        w = W.C3.with_(N=n, outlier_frac=0.0)
        inp = W.gen_inputs(w)
        q, k, v = (torch.from_numpy(getattr(inp, x + "_bits").view(np.int16)).view(torch.bfloat16)
                   .to(dev) for x in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

        def call():
            fa.fa_fwd(q, k, v, o=o, lse=lse, causal=True, scale=w.scale, stream=stream)

        _, med_ms = event_leg(torch, call, stream, warmup, steps, preheat_s)
        gbs = w.compulsory_bytes() / (med_ms * 1e-3) / 1e9
        out.append({"N": n, "us": round(med_ms * 1e3, 2), "compulsory_bytes": w.compulsory_bytes(),
                    "GB_per_s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)})
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps before timing")
    ap.add_argument("--preheat-s", type=float, default=1.0,
                    help="seconds of untimed load before the warm-up steps (the clock "
                         "needs a few hundred ms of load to reach its sustained level); "
                         "reported under 'preheat'")
    ap.add_argument("--leg-preheat-s", type=float, default=0.3,
                    help="pre-heat of each informational leg")
    ap.add_argument("--flush-steps", type=int, default=20,
                    help="steps timed with the L2 and MALL flushed before each (0: skip)")
    ap.add_argument("--flush-mib", type=int, default=512, help="flush buffer size")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=32,
                    help="query heads the oracle baseline computes (bounded sample)")
    ap.add_argument("--no-short-n", action="store_true",
                    help="skip the informational short-sequence sweep (N = 128 .. 1024)")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the informational FP8 forward timing")
    ap.add_argument("--no-local", action="store_true",
                    help="skip the informational sliding-window timing (window 256)")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the informational long-context timing (N = 32768)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the informational backward timing (B=2 H=16 N=4096 d=128 causal)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this size first (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; "
                                   "the forward shards over (batch, kv-head) groups without "
                                   "any exchange, so there is no multi-GPU path to measure"}))
        sys.exit(2)

    import numpy as np
    import torch

    import exact_tiled_attention_31_amd as fa
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    fa.lib()
    dev = torch.device("cuda:0")
    w = W.C3
    inp = W.gen_inputs(w)

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = to_dev(inp.q_bits), to_dev(inp.k_bits), to_dev(inp.v_bits)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * 2 ** 20 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def call():
        fa.fa_fwd(q, k, v, o=o, lse=lse, causal=True, scale=w.scale, stream=stream)

    clock = ClockSampler()
    heat = None
    if args.preheat_s > 0:
        with clock:
            heat = preheat(torch, call, args.preheat_s)
        heat["sclk"] = clock.summary()
    with clock:
        wall, step_ms = timed_steps(torch, call, stream, args.warmup, args.steps)

    ms_per_step = wall * 1e3 / args.steps
    kernel_ms_med = median(step_ms)
    kernel_ms_mean = sum(step_ms) / len(step_ms)
    flops = w.causal_adjusted_flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms_med * 1e-3) / 1e12
    traffic = measured_traffic()
    sclk = clock.summary()

    out = {
        "metric": "attention fwd TFLOP/s (causal-adjusted) at N=8192 d=128 bf16; % MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "GQA causal forward B=1 H=32 Hkv=8 N=8192 d=128 bf16, "
                               "1% of K rows x8 (seed 3)",
                   "B": w.B, "H": w.H, "Hkv": w.Hkv, "N": w.N, "d": w.d, "causal": True,
                   "flops_per_step": flops, "flop_convention": "4*B*H*N^2*d/2",
                   "flops_tile_count": tile_count_flops(w),
                   "tile_count_convention": "4*rows*cols*d per computed (32-row, 64-key) "
                                            "tile; key tiles past a wave's last row skipped"},
        "pct_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel_ms": round(kernel_ms_med, 5),
                     "kernel_ms_mean": round(kernel_ms_mean, 5),
                     "kernel_ms_stat": "median of per-step HIP events on the launch stream"},
        "preheat": heat,
        "sclk": sclk if sclk is not None else {"unavailable": clock.error},
    }
    if sclk is not None:
        # the nominal peak assumes 2.4 GHz; the same work at the measured clock.
        # The SMU table is refreshed by firmware and a short region can return
        # stale readings (idle clocks from before the region): the adjusted
        # figure is given only when the samples agree within 10%.
        if sclk["samples"] >= 3 and sclk["min_mhz"] >= 0.9 * sclk["max_mhz"]:
            adj_peak = PEAK_BF16_TFLOPS * sclk["mean_mhz"] / PEAK_SCLK_MHZ
            out["pct_clock_adjusted_peak"] = round(100.0 * achieved / adj_peak, 2)
        else:
            out["pct_clock_adjusted_peak"] = None
            sclk["note"] = "samples disagree by more than 10% (stale readings); not used"
    if args.flush_steps > 0:
        fl = flushed_steps(torch, call, stream, args.flush_steps, args.flush_mib * 2 ** 20)
        fm = median(fl)
        out["flushed"] = {"ms": round(fm, 5), "tflops": round(flops / (fm * 1e-3) / 1e12, 2),
                          "frac": round(flops / (fm * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "steps": args.flush_steps,
                          "flush": f"{args.flush_mib} MiB buffer written before each step"}
    if not args.no_short_n:
        out["short_n"] = short_n_sweep(fa, W, torch, np, dev, stream, args.warmup, args.steps,
                                       args.leg_preheat_s)
    if not args.no_fp8:
        out["fp8"] = fp8_timing(fa, W, torch, np, dev, stream, args.warmup, args.steps,
                                args.leg_preheat_s)
    if not args.no_local:
        out["local"] = local_timing(fa, w, torch, q, k, v, stream, 256, args.warmup, args.steps,
                                    args.leg_preheat_s)
    if not args.no_long:
        out["long_context"] = long_context_timing(fa, W, torch, np, dev, stream,
                                                  max(3, args.warmup // 10),
                                                  max(3, args.steps // 10), args.leg_preheat_s)
    if not args.no_backward:
        out["backward"] = backward_timing(fa, W, torch, np, dev, args.warmup,
                                          max(5, args.steps // 5), args.leg_preheat_s)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, w, args.cpu_heads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
