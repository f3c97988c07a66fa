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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-extras", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only-step", action="store_true", help="headline step only (for profiling)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run only a plain 1 GiB device-to-device copy (HBM byte-counter calibration)")
    return p.parse_args()


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

    from block_scaled_fp4_mxfp4_amd import fp4q as L, synth

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    # ------------------------------------------------------------ headline
    log("generating the prefill workload (X 4096x5120, W 10240x5120 bf16)")
    wl = synth.nvfp4_prefill()
    M, N, K = wl.meta["M"], wl.meta["N"], wl.meta["K"]
    x = bf16(wl.arrays["x_bf16"])
    w = bf16(wl.arrays["w_bf16"])
    stats = synth.realized_stats(synth.bf16_bits_to_f32(wl.arrays["x_bf16"][:512]))
    xq = (torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
          torch.empty((M, K // 16), dtype=torch.uint8, device=dev),
          torch.empty(1, dtype=torch.float32, device=dev))
    wq = (torch.empty((N, K // 2), dtype=torch.uint8, device=dev),
          torch.empty((N, K // 16), dtype=torch.uint8, device=dev),
          torch.empty(1, dtype=torch.float32, device=dev))
    y = torch.empty((M, N), dtype=torch.float32, device=dev)

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    # An event record costs the stream about 5 us of idle time on this
    # platform (a marker with a cache release), so the timed steps carry only
    # the two events that time the GEMM; the quantizer split comes from
    # separate, untimed steps with an event at every boundary.
    def step(record=None, gemm_only=False):
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

    # W untimed warmup steps, continued (untimed) until the GPU has run the
    # step for WARM_S seconds: MI355X ramps its clocks over the first ~10 ms
    # of sustained matrix work, and a cold GEMM runs ~20% slower.
    log(f"warmup {args.warmup} steps (+ until {WARM_S} s of warm-up)")
    tw = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or time.perf_counter() - tw < WARM_S:
        step()
        n_warm += 1
        if n_warm % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    recs = [[ev() for _ in range(4)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(recs[i], gemm_only=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    gemm_ms = float(np.mean([r[2].elapsed_time(r[3]) for r in recs]))
    nb = min(args.steps, 10)
    brk = [[ev() for _ in range(4)] for _ in range(nb)]
    for i in range(nb):                      # untimed: quantizer split
        step(brk[i])
    torch.cuda.synchronize()
    qx_ms = float(np.mean([r[0].elapsed_time(r[1]) for r in brk]))
    qw_ms = float(np.mean([r[1].elapsed_time(r[2]) for r in brk]))
    flops = 2.0 * M * N * K
    value = flops / (ms_step * 1e-3) / 1e12
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    qx_bytes = M * K * (2 + 0.5 + 1 / 16)
    qw_bytes = N * K * (2 + 0.5 + 1 / 16)
    log(f"step {ms_step:.3f} ms; quant X {qx_ms:.3f} ms, quant W {qw_ms:.3f} ms, GEMM {gemm_ms:.3f} ms "
        f"({gemm_tflops:.1f} TFLOP/s)")

    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic_gemm_nvfp4_4096x10240x5120.json")
    if os.path.exists(tfile):
        with open(tfile) as fh:
            t = json.load(fh)
        if t.get("kernel_source_sha256") == _kernel_hash():
            traffic = t.get("bytes_per_launch")

    roofline = {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": PEAK["fp16_TFLOPs"],
                "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK["fp16_TFLOPs"], 4), "traffic": traffic,
                "kernel": "k_gemm_mx3<FMT_NV, 256, 320, 64, 1, 8, 2, M32 = 1> (8 wavefronts, 256x320 tiles, LDS-DMA tiles, exact NVFP4 dequant, 32x32x16 fp16 MFMA)",
                "algorithmic": "2*M*N*K flop per launch (M=4096, N=10240, K=5120)",
                "frac_of_fp4_peak": round(gemm_tflops / PEAK["fp4_TFLOPs"], 4)}

    out = {
        "metric": "W4A4 FP4 GEMM TFLOP/s + quantizer GB/s, fraction of MI355X roofline",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "warmup_steps_run": n_warm, "dtype": "nvfp4 (e2m1+e4m3, fp16 mfma, fp32 acc)",
        "data": "synthetic (seeded heavy-tailed activations, N(0,0.02^2) weights)",
        "config": {"workload": "nvfp4_prefill X[4096x5120] W[10240x5120] bf16 -> quantize both -> GEMM",
                   "M": M, "N": N, "K": K, "parallelism": "single GPU"},
        "roofline": roofline,
        "step_breakdown_ms": {"quantize_x": round(qx_ms, 4), "quantize_w": round(qw_ms, 4),
                              "gemm": round(gemm_ms, 4),
                              "note": "gemm: events around every timed step's GEMM; quantize_x/w: "
                                      "10 further untimed steps with an event at every boundary"},
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
        a16, w16 = x.to(torch.float16), w.to(torch.float16)
        y16 = torch.empty((M, N), dtype=torch.float16, device=dev)
        tl = _time_op(torch, stream, lambda i: torch.mm(a16, w16.t(), out=y16), 20)
        out["context_library_fp16_gemm"] = {
            **_fl(tl, flops, "fp16_TFLOPs"), "op": "torch.mm(fp16 X, fp16 W^T) -> fp16, hipBLASLt",
            "shape": [M, N, K], "ours_gemm_TFLOPs": round(gemm_tflops, 2)}
        del a16, w16, y16
        out["extras"] = run_extras(L, synth, np, torch, dev, stream, log)

    if not args.only_step and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, M, N, K, log)

    print(json.dumps(out), flush=True)


def _kernel_hash():
    h = hashlib.sha256()
    for f in ("gemm_mx.hip", "codec.h"):
        with open(os.path.join(ROOT, "block_scaled_fp4_mxfp4_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


# ---------------------------------------------------------------- extras ----

def _time_op(torch, stream, fn, iters, warm=3):
    t0 = time.perf_counter()
    n = 0
    while n < warm or time.perf_counter() - t0 < 0.05:   # >= 50 ms of warm-up per operation
        fn(n)
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        fn(i)
        b.record(stream)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    return {"median_ms": ts[len(ts) // 2], "p10_ms": ts[len(ts) // 10], "p90_ms": ts[(9 * len(ts)) // 10]}


def _bw(t, nbytes):
    gbps = nbytes / (t["median_ms"] * 1e-3) / 1e9
    return {**{k: round(v, 4) for k, v in t.items()}, "bytes": int(nbytes), "GBps": round(gbps, 1),
            "frac_hbm": round(gbps / PEAK["hbm_GBps"], 4)}


def _fl(t, flops, peak_key):
    tf = flops / (t["median_ms"] * 1e-3) / 1e12
    return {**{k: round(v, 4) for k, v in t.items()}, "flops": flops, "TFLOPs": round(tf, 2),
            "peak_TFLOPs": PEAK[peak_key], "frac": round(tf / PEAK[peak_key], 4)}


def run_extras(L, synth, np, torch, dev, stream, log):
    ex = {}

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    # ---------------- MXFP4 with the online transform (2048 x 14336 x 4096)
    log("extras: MXFP4 + transform")
    wl = synth.mxfp4_transform()
    M, N, K = wl.meta["M"], wl.meta["N"], wl.meta["K"]
    x, w = bf16(wl.arrays["x_bf16"]), bf16(wl.arrays["w_bf16"])
    del wl
    t, u = L.balance_scale(w, x)
    reps = 3                                       # rotate copies past the 256 MB cache
    xs = [x] + [x.clone() for _ in range(reps - 1)]
    ws = [w] + [w.clone() for _ in range(reps - 1)]
    xc = [L.quantize_mxfp4(xi, t, True) for xi in xs]
    wc = [L.quantize_mxfp4(wi, u, True) for wi in ws]
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    mx = {"shape": [M, N, K]}
    mx["quantize_x_fused"] = _bw(_time_op(torch, stream, lambda i: L.quantize_mxfp4(xs[i % reps], t, True, out=xc[i % reps]), 30),
                                 M * K * (2 + 0.5 + 1 / 32))
    mx["quantize_w_fused"] = _bw(_time_op(torch, stream, lambda i: L.quantize_mxfp4(ws[i % reps], u, True, out=wc[i % reps]), 30),
                                 N * K * (2 + 0.5 + 1 / 32))
    yh = torch.empty((N, K), dtype=torch.float32, device=dev)
    mx["hadamard32_scale_w"] = _bw(_time_op(torch, stream, lambda i: L.hadamard32_scale(ws[i % reps], u, out=yh), 20),
                                   N * K * (2 + 4))
    del yh
    mx["gemm_mxfp4"] = _fl(_time_op(torch, stream, lambda i: L.gemm_w4a4(L.MXFP4, xc[i % reps][0], xc[i % reps][1], None,
                                                                           wc[i % reps][0], wc[i % reps][1], None, out=y), 30),
                           2.0 * M * N * K, "fp4_TFLOPs")
    st = _time_op(torch, stream, lambda i: (L.quantize_mxfp4(xs[i % reps], t, True, out=xc[i % reps]),
                                            L.gemm_w4a4(L.MXFP4, xc[i % reps][0], xc[i % reps][1], None,
                                                        wc[i % reps][0], wc[i % reps][1], None, out=y)), 20)
    mx["online_step_quantize_x_plus_gemm"] = _fl(st, 2.0 * M * N * K, "fp4_TFLOPs")
    ex["mxfp4_transform_2048x14336x4096"] = mx
    del xs, ws, xc, wc, y, x, w
    torch.cuda.empty_cache()

    # ---------------- MACaQ weight-side refinement of the MXFP4 layer's weight
    # (14336 x 4096) on its 2048 calibration rows, both transformed
    log("extras: MACaQ Hessian + exponent screen + Flip-Refinement")
    wl = synth.mxfp4_transform()
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
    log("extras: NVFP4 4/6 block scales")
    wl = synth.nvfp4_prefill()
    wb = bf16(wl.arrays["w_bf16"])
    del wl
    reps = 3                                       # 3 x 105 MB > 256 MB cache
    ws = [wb] + [wb.clone() for _ in range(reps - 1)]
    outs = {r: [L.quantize_nvfp4(wi, rule=r) for wi in ws] for r in ("6", "4/6")}
    nbytes = wb.numel() * (2 + 0.5 + 1 / 16)
    fs = {"shape": list(wb.shape), "dynamic_tensor_scale": True}
    for r, key in (("6", "max_to_6"), ("4/6", "four_six")):
        fs[key] = _bw(_time_op(torch, stream, lambda i: L.quantize_nvfp4(ws[i % reps], rule=r, out=outs[r][i % reps]), 30),
                      nbytes)
    ex["nvfp4_46_quantize_w_10240x5120"] = fs
    del ws, outs, wb
    torch.cuda.empty_cache()

    # ---------------- shared tensor scale for a fused projection (members of
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
    log("extras: NVFP4 decode")
    wl = synth.nvfp4_decode()
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
    log("extras: looped Sigma-Delta")
    wl = synth.looped_sigma_delta()
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

    def sd_step(_):
        L.sigma_delta_requant(segs, steps=1)

    def gemms(_):
        for a, c, s, tsc, yo in gem:
            L.gemm_w4a16(a, c, s, tsc, out=yo)

    sd = {"linears": len(shapes), "weights": nw, "R": R}
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
            sd_step(0)
            gemms_grouped(0)

    tfw = _time_op(torch, stream, full_forward, 3, warm=1)
    sd["forward_R32_ms"] = round(tfw["median_ms"], 3)
    sd["forward_R32_per_step_ms"] = round(tfw["median_ms"] / R, 4)

    # all R code banks in one launch: the plain multi-bank chain and the
    # reverse-order tail schedule (R/2 nearest-code banks + R/2 tail codes)
    stride = -(-max(s_["w"].numel() // 2 for s_ in segs) // 16) * 16
    banks = [torch.empty((R, stride), dtype=torch.uint8, device=dev) for _ in segs]
    msegs = [{**s_, "codes": b} for s_, b in zip(segs, banks)]

    def multibank(_):
        L.sigma_delta_requant(msegs, steps=R, bank_stride=stride)

    def schedule(_):
        L.sigma_delta_schedule(msegs, R // 2, R - R // 2, bank_stride=stride)

    sd["multibank_R32_one_launch"] = _bw(_time_op(torch, stream, multibank, 10), nw * (4 + 4 + 4 + 0.5 * R + 1 / 16))
    sd["reverse_tail_16_plus_16_one_launch"] = _bw(_time_op(torch, stream, schedule, 10), nw * (4 + 0.5 * R + 1 / 16))

    def stochastic(_):
        L.stochastic_round_requant(msegs, R, seed=42, bank_stride=stride)

    sd["stochastic_rounding_R32_one_launch"] = _bw(_time_op(torch, stream, stochastic, 10), nw * (4 + 0.5 * R + 1 / 16))

    def two_point(_):
        L.two_point_requant(msegs, R, bank_stride=stride)

    sd["two_point_R32_one_launch"] = _bw(_time_op(torch, stream, two_point, 10), nw * (4 + 0.5 * R + 1 / 16))
    del banks, msegs
    ex["looped_sigma_delta_13x_R32"] = sd
    del segs, gem
    torch.cuda.empty_cache()

    # ---------------- tiny NVFP4 (latency only)
    wl = synth.nvfp4_tiny()
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

def cpu_baseline(wl, M, N, K, log):
    """Time the CPU oracle (as it stands) on a bounded sample of the headline
    step and extrapolate per stage to the full step."""
    import numpy as np
    from oracle import formats as OF, nvfp4 as ONV, gemm as OG

    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = affinity
    cores = min(blas_threads, affinity)
    xs_rows, ws_rows, gn = 384, 1024, 1024
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
            "host_cpu": platform.processor() or platform.machine(), "affinity_cores": affinity,
            "threads_note": "quantization stages use 1 thread; the GEMM stage uses `cores` BLAS threads"}


if __name__ == "__main__":
    main()
