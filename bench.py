#!/usr/bin/env python3
"""Benchmark of the block-scaled FP4 W4A4 hot path on one MI355X.

Headline step (one pass of the NVFP4 W4A4 linear on the prefill-shaped
workload, X bf16 [4096 x 5120] heavy-tailed, W bf16 [10240 x 5120]):
    quantize X to NVFP4 (dynamic tensor scale: amax pass + quantize pass)
    quantize W to NVFP4 (same)
    Y = X_nvfp4 * W_nvfp4^T (fp32 out)
``value`` is the step's GEMM work 2*M*N*K divided by the step time (TFLOP/s,
whole step including both quantizations).  ``roofline`` describes the
dominant kernel (the GEMM) with its average duration measured with HIP events
on the launch stream inside the timed region.  ``cpu_baseline`` times the CPU
oracle on a bounded sample of the same workload.  ``extras`` times the other
rows of the hot path (MXFP4 with the online transform, NVFP4 decode, looped
Sigma-Delta + W4A16, the tiny NVFP4 case) with their own rooflines.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras]
                       [--no-cpu-baseline] [--only-step]
       python bench.py --extras mxfp4,decode,... [--quick]    (one row alone, for profiling)
       python bench.py --hbm-ceiling | --calibrate-copy        (reference streams)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WARM_S = 0.3          # minimum seconds of untimed warm-up before any timed region
PEAK = {"hbm_GBps": 8000.0, "fp4_TFLOPs": 10100.0, "fp8_TFLOPs": 5000.0, "fp16_TFLOPs": 2500.0,
        "bf16_TFLOPs": 2500.0, "fp64_TFLOPs": 78.6}


class ClockSampler:
    """Samples the GPU's current shader and memory clocks (the starred level
    of the driver's pp_dpm_sclk / pp_dpm_mclk files in sysfs) every few
    milliseconds on a host thread while the timed work runs.  Reports None
    fields when the files are not readable."""

    def __init__(self, torch, dev, period_s=0.005):
        import threading
        self.period = period_s
        self.samples = {"sclk": [], "mclk": []}
        self.files = {}
        self.note = None
        try:
            p = torch.cuda.get_device_properties(dev)
            base = f"/sys/bus/pci/devices/{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
            for k in ("sclk", "mclk"):
                f = os.path.join(base, f"pp_dpm_{k}")
                if self._read(f) is not None:
                    self.files[k] = f
            if not self.files:
                self.note = f"no readable pp_dpm_* under {base}"
        except Exception as e:  # pragma: no cover
            self.note = f"clock files not found: {e}"
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _read(f):
        try:
            with open(f) as fh:
                for line in fh:
                    if "*" in line:
                        tok = line.split(":", 1)[1].strip().split()[0].lower()
                        return float(tok.replace("mhz", ""))
        except Exception:
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            for k, f in self.files.items():
                v = self._read(f)
                if v is not None:
                    self.samples[k].append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.files:
            self._thread.start()
        return self

    def __exit__(self, *a):
        self._stop.set()
        if self.files:
            self._thread.join()

    def summary(self):
        out = {"source": "sysfs pp_dpm_sclk / pp_dpm_mclk, starred level, sampled every "
                         f"{self.period * 1e3:.0f} ms during warm-up and timing"}
        for k, v in self.samples.items():
            if v:
                v = sorted(v)
                out[f"{k}_MHz"] = {"min": v[0], "median": v[len(v) // 2], "max": v[-1], "samples": len(v)}
            else:
                out[f"{k}_MHz"] = None
        if self.note:
            out["note"] = self.note
        return out


# --config names (the workloads of synth.py) -> what bench.py runs for them
CONFIGS = {
    "nvfp4_tiny": "tiny",
    "nvfp4_prefill": None,                  # the headline step alone (--only-step)
    "mxfp4_transform": "mxfp4",
    "nvfp4_decode": "decode",
    "looped_sigma_delta": "sigma_delta",
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", "--iters", dest="steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-extras", action="store_true")
    p.add_argument("--no-cpu-baseline", "--no-oracle", dest="no_cpu_baseline", action="store_true")
    p.add_argument("--only-step", action="store_true", help="headline step only (for profiling)")
    p.add_argument("--config", default=None, choices=sorted(CONFIGS),
                   help="one workload alone: the headline step (nvfp4_prefill) or one of the other rows")
    p.add_argument("--extras", default=None,
                   help="comma list of extras to run alone, without the headline step (for profiling): "
                        "mxfp4, macaq, nvfp4_46, harmonize, decode, sigma_delta, tiny")
    p.add_argument("--seed", type=int, default=0,
                   help="input set: 0 is the default synthetic data; s > 0 offsets every generator seed")
    p.add_argument("--quick", action="store_true",
                   help="extras: 1 warm-up and at most 3 timed calls per operation (for profiling)")
    p.add_argument("--hbm-ceiling", action="store_true",
                   help="run only torch's copy, fill and sum on rotated buffers (practical HBM rates of this box)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run only a plain 1 GiB device-to-device copy (HBM byte-counter calibration)")
    args = p.parse_args()
    if args.config == "nvfp4_prefill":
        args.only_step = True
    elif args.config is not None:
        args.extras = CONFIGS[args.config]
    return args


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: runs on one GPU only (--gpus 1); the kernels measured here are the whole "
              "per-GPU hot path, and splitting the layer over several GPUs is not implemented.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    if args.calibrate_copy:
        # 1 GiB read + 1 GiB written per launch: the reference for FETCH_SIZE / WRITE_SIZE
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": src.numel() * 4, "bytes_written": dst.numel() * 4,
                          "launches": 3}), flush=True)
        return

    if args.hbm_ceiling:
        print(json.dumps(hbm_ceiling(torch, stream)), flush=True)
        return

    from block_scaled_fp4_mxfp4_amd import fp4q as L, synth
    global SEED
    SEED = args.seed

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.extras:
        global QUICK
        QUICK = args.quick
        only = set(args.extras.split(","))
        ex = run_extras(L, synth, np, torch, dev, stream, log, only=only)
        print(json.dumps({"extras": ex, "selected": sorted(only), "quick": args.quick}), flush=True)
        return

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    # ------------------------------------------------------------ headline
    log("generating the prefill workload (X 4096x5120, W 10240x5120 bf16)")
    wl = synth.nvfp4_prefill(seed=SEED)
    M, N, K = wl.meta["M"], wl.meta["N"], wl.meta["K"]
    x0 = bf16(wl.arrays["x_bf16"])
    w0 = bf16(wl.arrays["w_bf16"])
    stats = synth.realized_stats(synth.bf16_bits_to_f32(wl.arrays["x_bf16"][:512]))

    # Consecutive steps take different copies of X and W (and write different
    # code buffers), 4 x 188 MB = 754 MB in rotation, so a step's inputs are
    # not left in the 256 MB last-level cache by the step before.
    copies = 4
    xs = [x0] + [x0.clone() for _ in range(copies - 1)]
    ws_ = [w0] + [w0.clone() for _ in range(copies - 1)]

    def qbufs(rows):
        return (torch.empty((rows, K // 2), dtype=torch.uint8, device=dev),
                torch.empty((rows, K // 16), dtype=torch.uint8, device=dev),
                torch.empty(1, dtype=torch.float32, device=dev))

    xqs = [qbufs(M) for _ in range(copies)]
    wqs = [qbufs(N) for _ in range(copies)]
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    rot_mb = copies * (x0.numel() * 2 + w0.numel() * 2 + (M + N) * (K // 2 + K // 16)) / 1e6

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    # An event record costs the stream about 5 us of idle time on this
    # platform (a marker with a cache release), so the timed steps carry only
    # the two events that time the GEMM; the quantizer split comes from
    # separate, untimed steps with an event at every boundary.
    def step(i, record=None, gemm_only=False):
        x, w, xq, wq = xs[i % copies], ws_[i % copies], xqs[i % copies], wqs[i % copies]
        if record is not None and not gemm_only:
            record[0].record(stream)
        L.quantize_nvfp4(x, out=xq)
        if record is not None and not gemm_only:
            record[1].record(stream)
        L.quantize_nvfp4(w, out=wq)
        if record is not None:
            record[2].record(stream)
        L.gemm_w4a4(L.NVFP4, xq[0], xq[1], xq[2], wq[0], wq[1], wq[2], out=y)
        if record is not None:
            record[3].record(stream)

    def timed(nsteps, first, stride):
        recs = [[ev() for _ in range(4)] for _ in range(nsteps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(nsteps):
            step(first + i * stride, recs[i], gemm_only=True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return (t1 - t0) * 1e3 / nsteps, float(np.mean([r[2].elapsed_time(r[3]) for r in recs]))

    clocks = ClockSampler(torch, dev)
    with clocks:
        # W untimed warmup steps, continued (untimed) until the GPU has run
        # the step for WARM_S seconds: MI355X ramps its clocks over the first
        # ~10 ms of sustained matrix work, and a cold GEMM runs ~20% slower.
        log(f"warmup {args.warmup} steps (+ until {WARM_S} s of warm-up)")
        tw = time.perf_counter()
        n_warm = 0
        while n_warm < args.warmup or time.perf_counter() - tw < WARM_S:
            step(n_warm)
            n_warm += 1
            if n_warm % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        log(f"timing {args.steps} steps ({copies} input copies in rotation, {rot_mb:.0f} MB)")
        ms_step, gemm_ms = timed(args.steps, 0, 1)
        # the same steps on one copy (inputs partly cache-resident), for comparison
        warm_ms_step, warm_gemm_ms = timed(args.steps, 0, copies)
    nb = min(args.steps, 10)
    brk = [[ev() for _ in range(4)] for _ in range(nb)]
    for i in range(nb):                      # untimed: quantizer split
        step(i, brk[i])
    torch.cuda.synchronize()
    qx_ms = float(np.mean([r[0].elapsed_time(r[1]) for r in brk]))
    qw_ms = float(np.mean([r[1].elapsed_time(r[2]) for r in brk]))
    flops = 2.0 * M * N * K
    value = flops / (ms_step * 1e-3) / 1e12
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    qx_bytes = M * K * (2 + 0.5 + 1 / 16)
    qw_bytes = N * K * (2 + 0.5 + 1 / 16)
    log(f"step {ms_step:.3f} ms (one copy: {warm_ms_step:.3f} ms); quant X {qx_ms:.3f} ms, quant W {qw_ms:.3f} ms, "
        f"GEMM {gemm_ms:.3f} ms ({gemm_tflops:.1f} TFLOP/s)")

    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic_gemm_nvfp4_4096x10240x5120.json")
    if os.path.exists(tfile):
        with open(tfile) as fh:
            t = json.load(fh)
        if t.get("kernel_source_sha256") == _kernel_hash():
            traffic = t.get("bytes_per_launch")

    roofline = {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": PEAK["fp4_TFLOPs"],
                "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK["fp4_TFLOPs"], 4), "traffic": traffic,
                "kernel": "k_gemm_mx3<FMT_NV, 256, 320, 64, 1, 8, 2, M32 = 1> (8 wavefronts, 256x320 tiles, LDS-DMA tiles, exact NVFP4 dequant, 32x32x16 fp16 MFMA)",
                "algorithmic": "2*M*N*K flop per launch (M=4096, N=10240, K=5120)",
                "instruction_peak": {"dtype": "fp16 MFMA (exact NVFP4 products need 6 significant bits)",
                                     "peak": PEAK["fp16_TFLOPs"], "frac": round(gemm_tflops / PEAK["fp16_TFLOPs"], 4)}}

    out = {
        "metric": "W4A4 FP4 GEMM TFLOP/s + quantizer GB/s, fraction of MI355X roofline",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "warmup_steps_run": n_warm, "dtype": "nvfp4 (e2m1+e4m3, fp16 mfma, fp32 acc)",
        "data": f"synthetic (seeded heavy-tailed activations, N(0,0.02^2) weights; input set {SEED})",
        "config": {"workload": "nvfp4_prefill X[4096x5120] W[10240x5120] bf16 -> quantize both -> GEMM",
                   "M": M, "N": N, "K": K, "parallelism": "single GPU"},
        "roofline": roofline,
        "clocks": clocks.summary(),
        "input_rotation": {"copies": copies, "MB": round(rot_mb, 1),
                           "note": "step i uses copy i mod copies of X, W and their code buffers"},
        "single_copy_ms_per_step": round(warm_ms_step, 4),
        "single_copy_gemm_ms": round(warm_gemm_ms, 4),
        "step_breakdown_ms": {"quantize_x": round(qx_ms, 4), "quantize_w": round(qw_ms, 4),
                              "gemm": round(gemm_ms, 4),
                              "note": "gemm: events around every timed step's GEMM; quantize_x/w: "
                                      "10 further untimed steps (rotated copies) with an event at every boundary"},
        "quantizer_GBps": {"x": round(qx_bytes / (qx_ms * 1e-3) / 1e9, 1),
                           "w": round(qw_bytes / (qw_ms * 1e-3) / 1e9, 1),
                           "note": "algorithmic bytes (read bf16 once, write codes+scales) over the "
                                   "amax pass + quantize pass"},
        "input_stats_x": {k: round(v, 3) for k, v in stats.items()},
    }

    if not args.only_step and not args.no_extras:
        # context, not part of the path: the platform's dense fp16 GEMM
        # (hipBLASLt through torch.mm) on the same shape and operand layout
        log("context: library fp16 GEMM on the same shape")
        a16, w16 = x0.to(torch.float16), w0.to(torch.float16)
        y16 = torch.empty((M, N), dtype=torch.float16, device=dev)
        tl = _time_op(torch, stream, lambda i: torch.mm(a16, w16.t(), out=y16), 20)
        out["context_library_fp16_gemm"] = {
            **_fl(tl, flops, "fp16_TFLOPs"), "op": "torch.mm(fp16 X, fp16 W^T) -> fp16, hipBLASLt",
            "shape": [M, N, K], "ours_gemm_TFLOPs": round(gemm_tflops, 2)}
        del a16, w16, y16
        del xs, ws_, xqs, wqs, y, x0, w0
        torch.cuda.empty_cache()
        out["extras"] = run_extras(L, synth, np, torch, dev, stream, log)
        g = out["extras"].get("mxfp4_transform_2048x14336x4096", {}).get("gemm_mxfp4")
        if g:
            out["roofline_mxfp4_gemm"] = {"bound": "mfma", "achieved": g["TFLOPs"], "peak": PEAK["fp4_TFLOPs"],
                                          "unit": "TFLOP/s", "frac": g["frac"],
                                          "kernel": "k_gemm_mx3<FMT_MX, 256, 224, 128> (scaled FP4 MFMA 16x16x128)",
                                          "workload": "MXFP4 GEMM 2048x14336x4096, operands rotated"}

    if not args.only_step and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, M, N, K, log)
        per = cpu_baseline_configs(log)
        out["cpu_baseline"]["per_config"] = per
        _oracle_ratios(out, per, ms_step)

    print(json.dumps(out), flush=True)


def _kernel_hash():
    h = hashlib.sha256()
    for f in ("gemm_mx.hip", "codec.h"):
        with open(os.path.join(ROOT, "block_scaled_fp4_mxfp4_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def hbm_ceiling(torch, stream):
    """Streaming rates of the platform's own copy, fill and sum kernels on
    buffers rotated past the 256 MB last-level cache: what a plain
    memory-bound kernel reaches on this machine, beside the 8 TB/s spec."""
    out = {}
    for mb in (42, 105, 256):
        n = mb * (1 << 20) // 4
        c = max(3, -(-1100 // mb))
        src = [torch.ones(n, device="cuda:0") for _ in range(c)]
        dst = [torch.empty(n, device="cuda:0") for _ in range(c)]
        nbytes = n * 4
        tc = _time_op(torch, stream, lambda i: dst[i % c].copy_(src[i % c]), 30)
        tf = _time_op(torch, stream, lambda i: dst[i % c].fill_(2.0), 30)
        ts = _time_op(torch, stream, lambda i: src[i % c].sum(), 30)
        out[f"{mb}MB_x{c}"] = {"copy_GBps": round(2 * nbytes / (tc["median_ms"] * 1e-3) / 1e9, 1),
                               "fill_GBps": round(nbytes / (tf["median_ms"] * 1e-3) / 1e9, 1),
                               "sum_read_GBps": round(nbytes / (ts["median_ms"] * 1e-3) / 1e9, 1)}
        del src, dst
        torch.cuda.empty_cache()
    return {"hbm_ceiling": out, "spec_GBps": PEAK["hbm_GBps"]}


# ---------------------------------------------------------------- extras ----

QUICK = False
SEED = 0


def _time_op(torch, stream, fn, iters, warm=3):
    """GPU time per call, back to back: the calls run in batches between
    two events (no event between calls of a batch), behind a short device
    sleep that lets the host queue every call first, so host-side launch
    cost does not show as device time.  Returns the median, p10 and p90 of
    the per-call time over the batches."""
    if QUICK:
        iters, warm = min(iters, 3), 1
    else:
        iters, warm = max(iters, 100), max(warm, 10)   # at least 10 warm-up and 100 timed calls
    t0 = time.perf_counter()
    n = 0
    while n < warm or (not QUICK and time.perf_counter() - t0 < 0.05):   # >= 50 ms of warm-up per operation
        fn(n)
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    nb = min(iters, 10)
    per = max(1, iters // nb)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    torch.cuda._sleep(10_000_000)                          # ~5 ms: the host queues the batches meanwhile
    evs[0].record(stream)
    k = 0
    for j in range(nb):
        for _ in range(per):
            fn(k)
            k += 1
        evs[j + 1].record(stream)
    torch.cuda.synchronize()
    ts = sorted(evs[j].elapsed_time(evs[j + 1]) / per for j in range(nb))
    return {"median_ms": ts[len(ts) // 2], "p10_ms": ts[len(ts) // 10], "p90_ms": ts[(9 * len(ts)) // 10],
            "calls": nb * per}


def _bw(t, nbytes):
    gbps = nbytes / (t["median_ms"] * 1e-3) / 1e9
    return {**{k: round(v, 4) for k, v in t.items()}, "bytes": int(nbytes), "GBps": round(gbps, 1),
            "frac_hbm": round(gbps / PEAK["hbm_GBps"], 4)}


def _fl(t, flops, peak_key):
    tf = flops / (t["median_ms"] * 1e-3) / 1e12
    return {**{k: round(v, 4) for k, v in t.items()}, "flops": flops, "TFLOPs": round(tf, 2),
            "peak_TFLOPs": PEAK[peak_key], "frac": round(tf / PEAK[peak_key], 4)}


def run_extras(L, synth, np, torch, dev, stream, log, only=None):
    ex = {}

    def want(name):
        return only is None or name in only

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    # ---------------- MXFP4 with the online transform (2048 x 14336 x 4096)
    if want("mxfp4"):
        log("extras: MXFP4 + transform")
        wl = synth.mxfp4_transform(seed=SEED)
        M, N, K = wl.meta["M"], wl.meta["N"], wl.meta["K"]
        x, w = bf16(wl.arrays["x_bf16"]), bf16(wl.arrays["w_bf16"])
        del wl
        t, u = L.balance_scale(w, x)
        # copies in rotation, each set past 512 MB so no call finds its inputs
        # in the 256 MB last-level cache: 32 x 16.8 MB of X, 5 x 117 MB of W,
        # 16 x 35 MB of GEMM operands (X codes and W codes)
        rx, rw, rg = 32, 5, 16
        xs = [x] + [x.clone() for _ in range(rx - 1)]
        ws = [w] + [w.clone() for _ in range(rw - 1)]
        xc = [L.quantize_mxfp4(xi, t, True) for xi in xs]
        wc = [L.quantize_mxfp4(wi, u, True) for wi in ws]
        wg = [wc[i % rw] if i < rw else tuple(c.clone() for c in wc[i % rw]) for i in range(rg)]
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        mx = {"shape": [M, N, K], "copies_rotated": {"x": rx, "w": rw, "gemm_operands": rg}}
        mx["quantize_x_fused"] = _bw(_time_op(torch, stream, lambda i: L.quantize_mxfp4(xs[i % rx], t, True, out=xc[i % rx]), 64),
                                     M * K * (2 + 0.5 + 1 / 32))
        mx["quantize_w_fused"] = _bw(_time_op(torch, stream, lambda i: L.quantize_mxfp4(ws[i % rw], u, True, out=wc[i % rw]), 30),
                                     N * K * (2 + 0.5 + 1 / 32))
        yh = torch.empty((N, K), dtype=torch.float32, device=dev)
        mx["hadamard32_scale_w"] = _bw(_time_op(torch, stream, lambda i: L.hadamard32_scale(ws[i % rw], u, out=yh), 20),
                                       N * K * (2 + 4))
        del yh
        mx["gemm_mxfp4"] = _fl(_time_op(torch, stream, lambda i: L.gemm_w4a4(L.MXFP4, xc[i % rx][0], xc[i % rx][1], None,
                                                                               wg[i % rg][0], wg[i % rg][1], None, out=y), 32),
                               2.0 * M * N * K, "fp4_TFLOPs")
        st = _time_op(torch, stream, lambda i: (L.quantize_mxfp4(xs[i % rx], t, True, out=xc[i % rx]),
                                                L.gemm_w4a4(L.MXFP4, xc[i % rx][0], xc[i % rx][1], None,
                                                            wg[i % rg][0], wg[i % rg][1], None, out=y)), 32)
        mx["online_step_quantize_x_plus_gemm"] = _fl(st, 2.0 * M * N * K, "fp4_TFLOPs")
        ex["mxfp4_transform_2048x14336x4096"] = mx
        del xs, ws, xc, wc, wg, y, x, w
        torch.cuda.empty_cache()

    # ---------------- MACaQ weight-side refinement of the MXFP4 layer's weight
    if want("macaq"):
        # (14336 x 4096) on its 2048 calibration rows, both transformed
        log("extras: MACaQ Hessian + exponent screen + Flip-Refinement")
        wl = synth.mxfp4_transform(seed=SEED)
        M, N, K = wl.meta["M"], wl.meta["N"], wl.meta["K"]
        x, w = bf16(wl.arrays["x_bf16"]), bf16(wl.arrays["w_bf16"])
        del wl
        t, u = L.balance_scale(w, x)
        xp, wp = L.hadamard32_scale(x, t), L.hadamard32_scale(w, u)
        del x, w
        h = torch.zeros((K, K), dtype=torch.float64, device=dev)
        hz = _time_op(torch, stream, lambda i: L.hessian_accumulate(xp, h), 10)
        h.zero_()
        L.hessian_accumulate(xp, h)
        ws = torch.empty(L.lib.fp4q_macaq_workspace_bytes(N, K) // 8, dtype=torch.float64, device=dev)
        res = {}

        def refine(i, k):
            res[k] = L.macaq_refine(wp, h, 1.0, k, workspace=ws)

        mq = {"weight": [N, K], "calibration_rows": M, "lambda": 1.0}
        mq["hessian_accumulate"] = _fl(hz, 2.0 * K * K * M, "fp64_TFLOPs")
        mq["screen_only_K0"] = {k: round(v, 4) for k, v in _time_op(torch, stream, lambda i: refine(i, 0), 5).items()}
        mq["refine_K128"] = {k: round(v, 4) for k, v in _time_op(torch, stream, lambda i: refine(i, 128), 5).items()}
        fl = res[128][2].to(torch.int64)
        mq["flips_per_row_mean"] = round(float(fl.float().mean()), 2)
        mq["rows_at_K"] = int((fl == 128).sum())
        mq["gradient_flops"] = 2.0 * N * K * K
        ex["macaq_refine_14336x4096"] = mq
        del xp, wp, h, ws, res
        torch.cuda.empty_cache()

    # ---------------- NVFP4 4/6 block scales on the prefill weight (10240 x 5120)
    if want("nvfp4_46"):
        log("extras: NVFP4 4/6 block scales")
        wl = synth.nvfp4_prefill(seed=SEED)
        wb = bf16(wl.arrays["w_bf16"])
        del wl
        reps = 5                                       # 5 x 105 MB in rotation, past 512 MB
        ws = [wb] + [wb.clone() for _ in range(reps - 1)]
        outs = {r: [L.quantize_nvfp4(wi, rule=r) for wi in ws] for r in ("6", "4/6")}
        nbytes = wb.numel() * (2 + 0.5 + 1 / 16)
        fs = {"shape": list(wb.shape), "dynamic_tensor_scale": True}
        for r, key in (("6", "max_to_6"), ("4/6", "four_six")):
            fs[key] = _bw(_time_op(torch, stream, lambda i: L.quantize_nvfp4(ws[i % reps], rule=r, out=outs[r][i % reps]), 30),
                          nbytes)
        # a static tensor scale (given by the caller): one pass, no amax
        fs["max_to_6_static_scale"] = _bw(_time_op(torch, stream, lambda i: L.quantize_nvfp4(
            ws[i % reps], tensor_scale=outs["6"][i % reps][2], out=outs["6"][i % reps]), 30), nbytes)
        fs["note"] = ("dynamic: amax pass (reads the tensor) + finalize + quantize pass (reads it again); "
                      "GBps counts the tensor read once")
        ex["nvfp4_46_quantize_w_10240x5120"] = fs
        del ws, outs, wb
        torch.cuda.empty_cache()

    # ---------------- shared tensor scale for a fused projection (members of
    if want("harmonize"):
        # 10240 and 5120 rows, K 5120, member scales 1.82x apart): the member
        # with the smaller scale (10240 x 320 scale bytes) is rewritten in place.
        # Every call first restores the member cells (else the next call is the
        # identity and exits early); the restore alone is timed beside it.
        log("extras: fused-member scale harmonization")
        sa = torch.from_numpy(synth.uint8_bytes(430, (10240, 320), 0, 0x7F)).to(dev)
        sb = torch.from_numpy(synth.uint8_bytes(431, (5120, 320), 0, 0x7F)).to(dev)
        orig = torch.tensor([0.0021, 0.0021 * 1.82], dtype=torch.float32, device=dev)
        cells = orig.clone()
        shared = torch.empty(1, dtype=torch.float32, device=dev)

        def hz(i):
            cells.copy_(orig)
            L.harmonize_nvfp4([sa, sb], [cells[0:1], cells[1:2]], shared=shared)

        both = _time_op(torch, stream, hz, 50)
        reset = _time_op(torch, stream, lambda i: cells.copy_(orig), 50)
        net = max(both["median_ms"] - reset["median_ms"], 1e-6)
        ex["nvfp4_harmonize_fused_15360x5120"] = {
            "members": [[10240, 5120], [5120, 5120]], "scale_ratio": 1.82,
            "with_cell_restore": {k: round(v, 4) for k, v in both.items()},
            "cell_restore_only": {k: round(v, 4) for k, v in reset.items()},
            "net_ms": round(net, 4), "bytes_rewritten": 2 * sa.numel(),
            "GBps_net": round(2 * sa.numel() / (net * 1e-3) / 1e9, 1)}
        del sa, sb
        torch.cuda.empty_cache()

    # ---------------- NVFP4 decode (N 17408, K 5120, M in 1, 4, 16)
    if want("decode"):
        log("extras: NVFP4 decode")
        wl = synth.nvfp4_decode(seed=SEED)
        N, K = wl.meta["N"], wl.meta["K"]
        wd = torch.from_numpy(wl.arrays["w"]).to(dev)
        copies = 11                                    # 11 x 50 MB > 512 MB: defeats the 256 MB cache
        wq = []
        for _ in range(copies):
            wq.append(L.quantize_nvfp4(wd))
        del wd
        xall = bf16(wl.arrays["x_bf16"])
        dec = {"shape": [N, K], "weight_copies_rotated": copies}
        wbytes = N * K // 2 + N * K // 16
        for M in (1, 4, 16):
            xm = xall[:M].contiguous()
            yd = torch.empty((M, N), dtype=torch.float32, device=dev)
            ts = torch.empty(1, dtype=torch.float32, device=dev)
            tf = _time_op(torch, stream, lambda i: L.linear_w4a4(xm, wq[i % copies][0], wq[i % copies][1], wq[i % copies][2],
                                                                  out=yd, a_ts_out=ts), 50)
            nbytes = wbytes + M * K * 2 + M * N * 4
            dec[f"M{M}_fused_linear"] = _bw(tf, nbytes)
            aq = L.quantize_nvfp4(xm)
            tu = _time_op(torch, stream, lambda i: (L.quantize_nvfp4(xm, out=aq),
                                                    L.gemm_w4a4(L.NVFP4, aq[0], aq[1], aq[2], wq[i % copies][0],
                                                                wq[i % copies][1], wq[i % copies][2], out=yd)), 50)
            dec[f"M{M}_unfused_quantize_plus_gemm"] = _bw(tu, nbytes)
        ex["nvfp4_decode_17408x5120"] = dec
        del wq, xall
        torch.cuda.empty_cache()

    # ---------------- looped core: Sigma-Delta requant + W4A16 GEMMs, R = 32
    if want("sigma_delta"):
        log("extras: looped Sigma-Delta")
        wl = synth.looped_sigma_delta(seed=SEED)
        shapes = wl.meta["shapes"]
        segs, gem = [], []
        h = bf16(wl.arrays["h_bf16"])
        hd = bf16(wl.arrays["hd_bf16"])
        nw = 0
        flops = 0.0
        for i, (n, k) in enumerate(shapes):
            wm = torch.from_numpy(wl.arrays[f"w{i}"]).to(dev)
            c, s, tsc = L.quantize_nvfp4(wm)
            segs.append({"w": wm, "scales": s, "tensor_scale": tsc, "residue": torch.zeros_like(wm), "codes": c})
            a = hd if k == 3072 else h
            gem.append((a, c, s, tsc, torch.empty((a.shape[0], n), dtype=torch.float32, device=dev)))
            nw += n * k
            flops += 2.0 * a.shape[0] * n * k
        R = wl.meta["R"]
        # the per-step Sigma-Delta timing rotates 4 sets of (W, r, codes),
        # 4 x 140 MB past 512 MB; set 0 is the one the GEMMs and the forward use
        nsets = 4
        sets = [segs] + [[{**s_, "w": s_["w"].clone(), "residue": s_["residue"].clone(), "codes": s_["codes"].clone()}
                          for s_ in segs] for _ in range(nsets - 1)]

        def sd_step(i):
            L.sigma_delta_requant(sets[i % nsets], steps=1)

        def gemms(_):
            for a, c, s, tsc, yo in gem:
                L.gemm_w4a16(a, c, s, tsc, out=yo)

        sd = {"linears": len(shapes), "weights": nw, "R": R, "sigma_delta_sets_rotated": nsets}
        sd["sigma_delta_step"] = _bw(_time_op(torch, stream, sd_step, R), nw * (4 + 4 + 4 + 0.5 + 1 / 16))
        sd["w4a16_gemms_per_step"] = _fl(_time_op(torch, stream, gemms, R), flops, "bf16_TFLOPs")
        gprobs = [(a, c, s_, tsc, yo) for a, c, s_, tsc, yo in gem]

        def gemms_grouped(_):
            L.gemm_w4a16_grouped(gprobs)

        sd["w4a16_gemms_per_step_one_launch"] = _fl(_time_op(torch, stream, gemms_grouped, R), flops, "bf16_TFLOPs")

        def full_forward(_):
            for s_ in segs:
                s_["residue"].zero_()
            for _k in range(R):
                L.sigma_delta_requant(segs, steps=1)
                gemms_grouped(0)

        tfw = _time_op(torch, stream, full_forward, 3, warm=1)
        sd["forward_R32_ms"] = round(tfw["median_ms"], 3)
        sd["forward_R32_per_step_ms"] = round(tfw["median_ms"] / R, 4)

        # all R code banks in one launch: the plain multi-bank chain and the
        # reverse-order tail schedule (R/2 nearest-code banks + R/2 tail codes)
        stride = -(-max(s_["w"].numel() // 2 for s_ in segs) // 16) * 16
        banks = [torch.empty((R, stride), dtype=torch.uint8, device=dev) for _ in segs]
        # the one-launch forms read W (and r) from a rotating set, write the banks
        msets = [[{**s_, "codes": b} for s_, b in zip(st_, banks)] for st_ in sets]

        def multibank(i):
            L.sigma_delta_requant(msets[i % nsets], steps=R, bank_stride=stride)

        def schedule(i):
            L.sigma_delta_schedule(msets[i % nsets], R // 2, R - R // 2, bank_stride=stride)

        sd["multibank_R32_one_launch"] = _bw(_time_op(torch, stream, multibank, 10), nw * (4 + 4 + 4 + 0.5 * R + 1 / 16))
        sd["reverse_tail_16_plus_16_one_launch"] = _bw(_time_op(torch, stream, schedule, 10), nw * (4 + 0.5 * R + 1 / 16))

        def stochastic(i):
            L.stochastic_round_requant(msets[i % nsets], R, seed=42, bank_stride=stride)

        sd["stochastic_rounding_R32_one_launch"] = _bw(_time_op(torch, stream, stochastic, 10), nw * (4 + 0.5 * R + 1 / 16))

        def two_point(i):
            L.two_point_requant(msets[i % nsets], R, bank_stride=stride)

        sd["two_point_R32_one_launch"] = _bw(_time_op(torch, stream, two_point, 10), nw * (4 + 0.5 * R + 1 / 16))
        del banks, msets
        ex["looped_sigma_delta_13x_R32"] = sd
        del segs, sets, gem
        torch.cuda.empty_cache()

    # ---------------- tiny NVFP4 (latency only)
    if want("tiny"):
        wl = synth.nvfp4_tiny(seed=SEED)
        xt = torch.from_numpy(wl.arrays["x"]).to(dev)
        wt = torch.from_numpy(wl.arrays["w"]).to(dev)
        bq = L.quantize_nvfp4(wt)
        aq = L.quantize_nvfp4(xt)
        yt = torch.empty((64, 256), dtype=torch.float32, device=dev)
        tt = _time_op(torch, stream, lambda i: (L.quantize_nvfp4(xt, out=aq),
                                                L.gemm_w4a4(L.NVFP4, aq[0], aq[1], aq[2], bq[0], bq[1], bq[2], out=yt)), 50)
        ex["nvfp4_tiny_64x256x256"] = {k: round(v, 4) for k, v in tt.items()}
    return ex


# ---------------------------------------------------------- cpu baseline ----

def _oracle_ratios(out, per, ms_step):
    """Oracle time over GPU time per configuration, where both exist."""
    cb = out["cpu_baseline"]
    cb["gpu_speedup_over_oracle"] = {"nvfp4_prefill_4096x10240x5120": round(cb["full_step_s_est"] / (ms_step * 1e-3))}
    ex = out.get("extras")
    if not ex:
        return
    mx = ex.get("mxfp4_transform_2048x14336x4096")
    p = per.get("mxfp4_transform_2048x14336x4096")
    if mx and p:
        gpu_s = (mx["online_step_quantize_x_plus_gemm"]["median_ms"] + mx["quantize_w_fused"]["median_ms"]) * 1e-3
        cb["gpu_speedup_over_oracle"]["mxfp4_transform_2048x14336x4096"] = round(p["full_s_est"] / gpu_s)
    d = ex.get("nvfp4_decode_17408x5120")
    p = per.get("nvfp4_decode_17408x5120")
    if d and p:
        for k, v in p["per_M"].items():
            g = d.get(f"{k}_fused_linear")
            if g:
                cb["gpu_speedup_over_oracle"][f"nvfp4_decode_{k}"] = round(v["full_s_est"] / (g["median_ms"] * 1e-3))
    sd = ex.get("looped_sigma_delta_13x_R32")
    p = per.get("looped_sigma_delta_13x_R32")
    if sd and p:
        cb["gpu_speedup_over_oracle"]["looped_sigma_delta_forward_R32"] = round(
            p["forward_R32_s_est"] / (sd["forward_R32_ms"] * 1e-3))


def _cores():
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = affinity
    return min(blas_threads, affinity), affinity, blas_threads


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(wl, M, N, K, log):
    """Time the CPU oracle (as it stands) on a bounded sample of the headline
    step and extrapolate per stage to the full step."""
    import numpy as np
    from oracle import formats as OF, nvfp4 as ONV, gemm as OG

    cores, affinity, blas_threads = _cores()
    xs_rows, ws_rows, gn = 1024, 3072, 1024
    log(f"cpu baseline: oracle on {xs_rows} rows of X, {ws_rows} rows of W, GEMM {xs_rows}x{gn}x{K}")
    xf = OF.bf16_bits_to_f32(wl.arrays["x_bf16"][:xs_rows])
    wf = OF.bf16_bits_to_f32(wl.arrays["w_bf16"][:ws_rows])
    t0 = time.perf_counter()
    cx, sx, tx = ONV.quantize(xf)
    cw, sw, tw = ONV.quantize(wf)
    t1 = time.perf_counter()
    y = OG.w4a4_nvfp4(cx, sx, tx, cw[:gn], sw[:gn], tw)
    t2 = time.perf_counter()
    q_rate = (xf.size + wf.size) / (t1 - t0)                 # elements / s
    g_rate = 2.0 * xs_rows * gn * K / (t2 - t1)              # flop / s (fp64 BLAS)
    full_s = (M * K + N * K) / q_rate + 2.0 * M * N * K / g_rate
    value = 2.0 * M * N * K / full_s / 1e12
    assert np.isfinite(y).all()
    return {"value": round(value, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": (f"oracle NVFP4 quantization of {xs_rows} rows of X and {ws_rows} rows of W "
                       f"({(xf.size + wf.size) / 1e6:.2f} M elements, single-threaded NumPy, "
                       f"{t1 - t0:.1f} s) and its float64 GEMM {xs_rows}x{gn}x{K} (BLAS, {t2 - t1:.2f} s); "
                       f"full-step time extrapolated per stage: {full_s:.1f} s"),
            "full_step_s_est": round(full_s, 2),
            "host_cpu": _cpu_model(), "affinity_cores": affinity, "blas_threads": blas_threads,
            "threads_note": "quantization stages use 1 thread; the GEMM stage uses `cores` BLAS threads"}


def cpu_baseline_configs(log):
    """Oracle stage times for the other configurations, each on a bounded
    sample of the same seeded inputs the GPU timings use, extrapolated per
    stage (elements or flops) to the full configuration."""
    import numpy as np
    from oracle import formats as OF, nvfp4 as ONV, mxfp4 as OMX, balance as OB, gemm as OG
    from oracle import sigma_delta as OSD
    from block_scaled_fp4_mxfp4_amd import synth

    def clock(f, *a, **k):
        t0 = time.perf_counter()
        r = f(*a, **k)
        return r, time.perf_counter() - t0

    out = {}
    # MXFP4 with the online transform: balance statistic on the full tensors,
    # transform + quantize on 512 rows of X and 1536 rows of W, GEMM 512 x 1536
    log("cpu baseline: MXFP4 + transform stages")
    wl = synth.mxfp4_transform(seed=SEED)
    M, N, K = wl.meta["M"], wl.meta["N"], wl.meta["K"]
    xf = OF.bf16_bits_to_f32(wl.arrays["x_bf16"])
    wf = OF.bf16_bits_to_f32(wl.arrays["w_bf16"])
    (_, t32, u32), tb = clock(OB.balance_scale, wf, xf)
    xr, wr = 512, 1536
    xh, th_x = clock(OMX.hadamard32_scale, xf[:xr], t32)
    (cx, sx), tq_x = clock(OMX.quantize, xh)
    wh, th_w = clock(OMX.hadamard32_scale, wf[:wr], u32)
    (cw, sw), tq_w = clock(OMX.quantize, wh)
    _, tg = clock(OG.w4a4_mxfp4, cx, sx, cw, sw)
    st_full = {"balance_scale": tb,
               "hadamard32_scale": (th_x + th_w) / (xr + wr) * (M + N),
               "quantize_mxfp4": (tq_x + tq_w) / (xr + wr) * (M + N),
               "gemm_fp64": tg * (M * N) / (xr * wr)}
    out["mxfp4_transform_2048x14336x4096"] = {
        "sample": f"balance statistic on full X and W; transform + quantize of {xr} rows of X and {wr} of W; "
                  f"GEMM {xr}x{wr}x{K} (dequantize + fp64 BLAS)",
        "stages_s_est": {k: round(v, 3) for k, v in st_full.items()},
        "full_s_est": round(sum(st_full.values()), 2),
        "sample_s": round(tb + th_x + tq_x + th_w + tq_w + tg, 2)}
    del wl, xf, wf, xh, wh

    # NVFP4 decode: activation quantize of M rows, GEMM against 1024
    # quantized rows of W (W is quantized once, outside the step)
    log("cpu baseline: NVFP4 decode stages")
    wl = synth.nvfp4_decode(seed=SEED)
    N, K = wl.meta["N"], wl.meta["K"]
    wrows = 1024
    cw, sw, tw = ONV.quantize(wl.arrays["w"][:wrows])
    dec = {"sample": f"activation quantize of M rows; dequantize + fp64 GEMM against {wrows} of {N} weight rows",
           "per_M": {}}
    tot = 0.0
    for Mm in (1, 4, 16):
        xa = OF.bf16_bits_to_f32(wl.arrays["x_bf16"][:Mm])
        (ca, sa, ta), tqa = clock(ONV.quantize, xa)
        _, tgm = clock(OG.w4a4_nvfp4, ca, sa, ta, cw, sw, tw)
        full = tqa + tgm * N / wrows
        dec["per_M"][f"M{Mm}"] = {"quantize_x_s": round(tqa, 4), "gemm_s_est": round(tgm * N / wrows, 3),
                                  "full_s_est": round(full, 3)}
        tot += tqa + tgm
    dec["sample_s"] = round(tot, 2)
    out["nvfp4_decode_17408x5120"] = dec
    del wl

    # looped Sigma-Delta: the chain at steps {1, 2, 16, 32} on all 768 rows of
    # the first linear, and the W4A16 GEMM of one full 768 x 768 linear on
    # the [4096 x 768] hidden state
    log("cpu baseline: looped Sigma-Delta stages")
    wl = synth.looped_sigma_delta(seed=SEED)
    shapes = wl.meta["shapes"]
    nw = sum(n * k for n, k in shapes)
    w0 = wl.arrays["w0"]
    rows = 768
    sdt = {}
    tsum = 0.0
    for steps in (1, 2, 16, 32):
        _, tsd = clock(OSD.sigma_delta_nvfp4, w0[:rows], steps)
        tsum += tsd
        sdt[f"steps_{steps}_s_est"] = round(tsd * nw / (rows * w0.shape[1]), 2)
    c0, s0, st0 = ONV.quantize(w0)
    _, tg = clock(OG.w4a16, wl.arrays["h_bf16"], c0, s0, st0)
    tokens = wl.meta["tokens"]
    step_flops = sum(2.0 * tokens * n * k for n, k in shapes)
    g_step = tg * step_flops / (2.0 * tokens * w0.shape[0] * w0.shape[1])
    out["looped_sigma_delta_13x_R32"] = {
        "sample": f"oracle chain on {rows} rows of linear 0 at each step count; W4A16 GEMM "
                  f"{tokens}x{w0.shape[0]}x{w0.shape[1]} (dequantize + fp64 BLAS)",
        "sigma_delta_all_13_linears": sdt,
        "w4a16_gemms_per_step_s_est": round(g_step, 3),
        "forward_R32_s_est": round(sdt["steps_32_s_est"] + 32 * g_step, 1),
        "sample_s": round(tsum + tg, 2)}
    return out


if __name__ == "__main__":
    main()
