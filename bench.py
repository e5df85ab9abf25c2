"""Throughput of the weight-dequantizing linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--reps R] [--no-cpu-baseline] [--no-others]

The step is one pass of the encoder GEMM chain, the largest workload: 24 layers of four wq_gemm
calls at n = 1500 frames, d = 1024 (QKV 3072x1024 + bias; output projection 1024x1024 + bias +
residual; MLP up 4096x1024 + bias + erf-GELU; MLP down 1024x4096 + bias + residual), bf16 weights
(24 x 25 MB, distinct per layer), f32 activations. `value` is its TFLOP/s: 905,969,664,000 FLOP
per step over the step time, with every input resident in HBM. The K timed steps run back to back
in 5 equal blocks with a HIP event between blocks (and none between launches); ms_per_step is the
whole region over K, and `spread` gives the median, min and max over the blocks.

The same JSON line carries:
  roofline      the chain's dominant kernel (the GEMM that takes the most time per step, the MLP down
                projection): its FLOP per launch over its mean launch time, measured here with events
                around back-to-back launches of it alone on the same stream, against the bf16 MFMA
                peak; `traffic` is the HBM bytes per launch that FETCH_SIZE / WRITE_SIZE counted for it
                (profiles/, scaled by a copy kernel of known size), or null when the kernel sources
                changed since they were counted;
  cpu_baseline  the f64 oracle (decode + numpy product + epilogue) on two of the chain's 24 layers,
                all 1500 frames, on the host's cores;
  rooflines     every other workload at its full size: the bf16 GEMM 64x256x256 + GELU, the Q8_0
                matvec 4096x4096 at n = 1 and n = 4, the Q4_0 matvec 14336x4096, the MoE (16 tokens
                top-2 of 8 Q4_0 14336x4096 experts, gated), and the MoE at sparse routing (1 token top-2
                of 8; 16 tokens top-2 of 64). Each has the median / min / max of R repetitions of
                back-to-back calls, its GB/s (weight bytes of the experts it touches) or TFLOP/s and
                fraction of peak, the streaming-read floor for the same bytes (a plain read kernel,
                libwq_bench.so) and the fraction of it reached (frac_of_sol), counted traffic and a CPU
                baseline of its own;
                Q4_K weights (hanzo-ml matvec_q4k_gpu) add the matvec 14336x4096 at n = 1 and the
                MoE of 16 tokens top-2 of 8 experts of that shape, gated, both on Q4_K super-blocks;
                The rest of the encoder block adds LayerNorm 1500x1024, the q/k norm + rotation over
                8 heads of 128 and attention (1500 frames, 100 masked) to rooflines, each with a CPU
                baseline;
  others        the chain on the f32-accurate matrix-core path, the vendor bf16 GEMM (torch's linear)
                on the chain's four layer shapes as a same-GPU calibration, f16 weights at 4096x4096
                n = 1, the MLP-up shape with f16 / f32 / Q8_0 / Q4_0 weights, and the whole 24-block
                encoder forward (every kernel of the block; CPU baseline: one block);
  context       the shader clock measured under load, the device's maximum clock attribute, and a
                device-to-device copy rate.
Weights of the matvec and MoE workloads rotate over copies of at least 600 MB, so the 256 MB
Infinity Cache cannot serve them; the floors read the same amounts from rotating windows.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
ROTATE_BYTES = 600 * 2 ** 20
COUNTERS = os.path.join(ROOT, "profiles", "bench_hbm_counters.md")


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--reps", type=int, default=5, help="repetitions behind each median / min / max")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true")
    ap.add_argument("--legs", default="all",
                    help="comma list of workload groups to run (chain, c1, c2, c3, c4, moe1, moe64, q4k, enc, others; "
                         "default all): profiling runs select one so its kernels' counters are its own")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run an elementwise copy of 256 MiB (reads and writes that many bytes), "
                         "the reference for scaling HBM byte counters")
    return ap.parse_args()


class Timer:
    """Back-to-back calls on the current stream, timed with HIP events only around whole runs."""

    def __init__(self, torch):
        self.torch = torch
        self.stream = torch.cuda.current_stream()

    def runs(self, fn, calls, reps, warm=2, warm_ms=30.0):
        """ms per call of each of `reps` runs of `calls` back-to-back calls, after `warm` calls and
        then whole runs until the GPU has been busy for `warm_ms`: after the host-side set-up of a
        workload, memory-bound calls run up to 20% slower for their first few milliseconds (the MoE
        workload: 80-90 us for about 100 calls, then 72-75 us)."""
        torch = self.torch
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        i = warm
        while (time.perf_counter() - t0) * 1e3 < warm_ms:
            for _ in range(calls):
                fn(i)
                i += 1
            torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        i = 0
        ev[0].record(self.stream)
        for r in range(reps):
            for _ in range(calls):
                fn(i)
                i += 1
            ev[r + 1].record(self.stream)
        torch.cuda.synchronize()
        return [ev[r].elapsed_time(ev[r + 1]) / calls for r in range(reps)]


def _stats(ms_list):
    a = np.array(ms_list)
    return {"median_us": round(float(np.median(a)) * 1e3, 3), "min_us": round(float(a.min()) * 1e3, 3),
            "max_us": round(float(a.max()) * 1e3, 3), "reps": len(a)}


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 0) for i in threadpool_info()), default=0) or len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


class Floor:
    """The streaming-read floor: a plain read of `nbytes` (libwq_bench.so), from rotating windows of
    one large buffer so the reads come from HBM."""

    def __init__(self, torch, timer, dev):
        path = os.path.join(ROOT, "gemv_wq_gemm_amd", "libwq_bench.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build with `python -m gemv_wq_gemm_amd.build`")
        self.lib = ctypes.CDLL(path)
        self.lib.wq_bench_stream_read.restype = ctypes.c_int
        self.lib.wq_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                                  ctypes.c_void_p]
        self.lib.wq_bench_stream_read_lds.restype = ctypes.c_int
        self.lib.wq_bench_stream_read_lds.argtypes = self.lib.wq_bench_stream_read.argtypes
        self.lib.wq_bench_stream_read_blocks.restype = ctypes.c_int
        self.blocks = self.lib.wq_bench_stream_read_blocks(4)
        self.torch, self.timer = torch, timer
        self.buf = torch.randint(0, 2 ** 31 - 1, (1024 * 2 ** 20 // 4,), dtype=torch.int32, device=dev)
        self.out = torch.empty(self.blocks, dtype=torch.int32, device=dev)

    def us(self, nbytes, reps):
        """The faster of the two plain reads (register loads, direct-to-LDS loads) of `nbytes`."""
        nbytes = nbytes // 1024 * 1024
        windows = max(1, (self.buf.numel() * 4) // max(nbytes, 1))
        base = self.buf.data_ptr()
        stream = ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)
        out = ctypes.c_void_p(self.out.data_ptr())
        best = None
        for kind, fn_c in (("vgpr", self.lib.wq_bench_stream_read), ("lds", self.lib.wq_bench_stream_read_lds)):
            def fn(i, fn_c=fn_c):
                off = (i % windows) * nbytes
                r = fn_c(ctypes.c_void_p(base + off), nbytes, out, self.blocks, stream)
                if r != 0:
                    raise RuntimeError(f"stream read launch failed: {r}")
            calls = max(4, min(100, int(2e9 // max(nbytes, 1))))
            st = {**_stats(self.timer.runs(fn, calls, reps)), "kind": kind}
            if best is None or st["median_us"] < best["median_us"]:
                best = st
        return best


def _hbm_entry(stats, weight_bytes, floor_stats, traffic, cpu=None, extra=None):
    med = stats["median_us"] * 1e-6
    gbs = weight_bytes / med / 1e9
    floor = weight_bytes / (floor_stats["median_us"] * 1e-6) / 1e9
    e = {**stats, "GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
         "floor_GB/s": round(floor, 1), "floor_us": floor_stats["median_us"], "floor_read": floor_stats["kind"],
         "frac_of_sol": round(gbs / floor, 4),
         "weight_bytes": weight_bytes, "traffic": None if traffic is None else round(traffic)}
    if extra:
        e.update(extra)
    if cpu is not None:
        e["cpu_baseline"] = cpu
    return e


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path has no "
              f"multi-GPU mode)", file=sys.stderr)
        sys.exit(2)
    if args.steps % 5 != 0 or args.steps <= 0:
        print("--steps must be a positive multiple of 5 (the timed steps run in 5 equal blocks)", file=sys.stderr)
        sys.exit(2)

    import torch

    import gemv_wq_gemm_amd as wq
    import synth
    from gemv_wq_gemm_amd.rocprof_summary import read_traffic

    all_legs = {"chain", "c1", "c2", "c3", "c4", "moe1", "moe64", "q4k", "enc", "others"}
    legs = all_legs if args.legs == "all" else set(args.legs.split(","))
    if legs - all_legs:
        print(f"unknown legs {sorted(legs - all_legs)}; choose from {sorted(all_legs)}", file=sys.stderr)
        sys.exit(2)
    args.legs_set = legs
    wq.lib()  # fail loudly if the library is not built
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    timer = Timer(torch)

    if args.copy_calibration:
        src = torch.ones(64 * 2 ** 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    line, others = {}, {}
    if "chain" in legs:
        line, others, acts = _chain(torch, wq, synth, dev, timer, to_dev, args, props, read_traffic)
    else:
        acts = None
        line = {"metric": "GEMM TFLOP/s (encoder chain) on 1 MI355X", "value": None, "unit": "TFLOP/s",
                "note": f"profiling run of legs {sorted(legs)}; the step (the chain) was not run"}
    line["rooflines"] = _rooflines(torch, wq, synth, dev, timer, to_dev, args, read_traffic)
    if "enc" in legs:
        enc_rl, enc_other = _encoder(torch, wq, synth, dev, timer, to_dev, args, read_traffic)
        line["rooflines"].update(enc_rl)
        others.update(enc_other)
    if not args.no_others and "others" in legs:
        others.update(_others(torch, wq, synth, dev, timer, to_dev, args))
    if others:
        line["others"] = others
    if not args.no_others and "others" in legs:
        line["context"] = _context(torch, timer, dev, args)

    if not args.no_cpu_baseline:
        if acts is not None:
            line["cpu_baseline"] = _cpu_chain(synth, acts)
        for key, cpu in {**_cpu_configs(synth), **(_cpu_encoder(synth) if "enc" in legs else {})}.items():
            if key in line["rooflines"]:
                line["rooflines"][key]["cpu_baseline"] = cpu
            elif key in others:
                others[key]["cpu_baseline"] = cpu

    print(json.dumps(line), flush=True)


def _context(torch, timer, dev, args):
    """Secondary context for the figures above: the shader clock measured under load (libwq_bench.so's
    probe: shader-clock cycles over wall-counter ticks on 4 workgroups per CU), the device's maximum
    clock attribute, and a device-to-device copy rate."""
    path = os.path.join(ROOT, "gemv_wq_gemm_amd", "libwq_bench.so")
    lib = ctypes.CDLL(path)
    lib.wq_bench_clock_probe.restype = ctypes.c_int
    lib.wq_bench_clock_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    wall_khz, max_khz = ctypes.c_int(0), ctypes.c_int(0)
    lib.wq_bench_clock_rates(ctypes.byref(wall_khz), ctypes.byref(max_khz))
    blocks = 4 * torch.cuda.get_device_properties(dev).multi_processor_count
    counts = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
    sink = torch.zeros(256, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(3):  # the last run is read; the first ones bring the clock up
        r = lib.wq_bench_clock_probe(200000, ctypes.c_void_p(counts.data_ptr()), ctypes.c_void_p(sink.data_ptr()),
                                     blocks, stream)
        if r != 0:
            raise RuntimeError(f"clock probe launch failed: {r}")
    c = counts.view(blocks, 2).cpu().numpy().astype(np.float64)
    mhz = float(np.median(c[:, 0] / c[:, 1])) * wall_khz.value / 1e3 if wall_khz.value > 0 else None

    nbytes = 512 * 2 ** 20
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    ms = timer.runs(lambda i: dst.copy_(src), 4, args.reps)
    del src, dst
    return {
        "sclk_mhz_under_load": None if mhz is None else round(mhz, 1),
        "sclk_mhz_max_attribute": round(max_khz.value / 1e3, 1),
        "peaks_assume_mhz": 2400.0,
        "d2d_copy_GBps": round(2 * nbytes / (float(np.median(ms)) * 1e-3) / 1e9, 1),
        "d2d_copy_note": "torch copy_ of 512 MiB, read + written bytes over the median time",
    }


def _chain(torch, wq, synth, dev, timer, to_dev, args, props, read_traffic):
    """The step: the 24-layer encoder GEMM chain, timed; its layers one kind at a time; and (unless
    --no-others) the chain on the f32-accurate path. Returns (line, others, activations)."""
    n, d, ff = synth.ENCODER_N, synth.ENCODER_D, synth.ENCODER_FF
    acts = synth.encoder_activations()
    a1, a2, a3 = (to_dev(acts[nm]) for nm in ("a1", "a2", "a3"))
    h = to_dev(acts["h0"]).clone()
    layers = []
    for L in range(synth.ENCODER_LAYERS):
        lw = synth.encoder_layer_weights(L)
        layers.append({nm: (to_dev(v["w"]), to_dev(v["bias"])) for nm, v in lw.items()})
    qkv = torch.empty((n, 3 * d), device=dev)
    f = torch.empty((n, ff), device=dev)
    shapes = {"qkv": (a1, 3 * d, d, qkv, {}), "out": (a2, d, d, h, {"residual": True}),
              "fc1": (a3, ff, d, f, {"gelu": True}), "fc2": (f, d, ff, h, {"residual": True})}

    def bind_layer(W_, name, path):
        x, m, k, out, kw = shapes[name]
        return wq.bind_gemm(x, W_[name][0], wq.W_BF16, m=m, k=k, bias=W_[name][1], out=out, path=path, **kw)

    def bind_chain(path):
        calls = [bind_layer(W_, nm, path) for W_ in layers for nm in ("qkv", "out", "fc1", "fc2")]

        def chain(_):
            for c in calls:
                c()
        return chain

    flop_layer = 2 * n * (3 * d * d + d * d + ff * d + d * ff)
    flop_step = synth.ENCODER_LAYERS * flop_layer
    chain = bind_chain(wq.PATH_AUTO)
    for i in range(args.warmup):
        chain(i)
    torch.cuda.synchronize()
    blocks = 5
    per_block = args.steps // blocks
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(blocks + 1)]
    t0 = time.perf_counter()
    ev[0].record(timer.stream)
    for b in range(blocks):
        for _ in range(per_block):
            chain(0)
        ev[b + 1].record(timer.stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev[0].elapsed_time(ev[blocks]) / args.steps
    block_ms = [ev[b].elapsed_time(ev[b + 1]) / per_block for b in range(blocks)]
    value = flop_step / (ms_step * 1e-3) / 1e12

    # Per layer type: each layer kind alone, back to back over the 24 layers' weights.
    layer_us = {}
    for nm in ("qkv", "out", "fc1", "fc2"):
        calls = [bind_layer(W_, nm, wq.PATH_AUTO) for W_ in layers]
        layer_us[nm] = _stats(timer.runs(lambda i: calls[i % len(calls)](), len(calls), args.reps))
    dom = max(layer_us, key=lambda k_: layer_us[k_]["median_us"])
    x_, m_, k_, _, kw_ = shapes[dom]
    dom_flop = 2 * n * m_ * k_
    dom_tflops = dom_flop / (layer_us[dom]["median_us"] * 1e-6) / 1e12
    dom_kernels = {"qkv": "gemm_bf16_kernel<64, 192, 2, 2, 2, 64, false, false, false, false>",
                   "out": "gemm_bf16_kernel<64, 64, 2, 2, 3, 64, false, false, false, false>",
                   "fc1": "gemm_bf16_kernel<64, 128, 2, 4, 2, 64, false, false, false, true>",
                   "fc2": "gemm_bf16_kernel<64, 128, 2, 4, 4, 64, false, false, false, false>"}
    traffic = read_traffic(COUNTERS, f"gemm_{dom}")

    line = {
        "metric": "GEMM TFLOP/s (encoder chain, bf16 weights, X rounded to bf16) on 1 MI355X; matvec weight GB/s in rooflines",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "arithmetic": "bf16 x bf16 -> f32 on the matrix cores (f32 activations rounded to bf16, bf16 weights as stored)",
        "data": "synthetic",
        "config": {
            "workload": "encoder GEMM chain: 24 layers x {QKV 1500x3072x1024 +bias, out 1500x1024x1024 +bias+residual, "
                        "MLP up 1500x4096x1024 +bias+erf-GELU, MLP down 1500x1024x4096 +bias+residual}; "
                        "bf16 weights N(0,0.02) distinct per layer, f32 activations N(0,1)",
            "flop_per_step": flop_step,
            "weight_bytes_per_step": 24 * 2 * (3 * d * d + d * d + ff * d + d * ff),
            "parallelism": "single GPU",
        },
        "spread": {**_stats(block_ms), "unit": "per step, over 5 blocks of the timed steps"},
        "roofline": {
            "bound": "mfma",
            "kernel": f"{dom_kernels[dom]} ({dom}: {n}x{m_}x{k_})",
            "achieved": round(dom_tflops, 1),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(dom_tflops / BF16_PEAK_TFLOPS, 4),
            "traffic": None if traffic is None else round(traffic),
            "flop_per_launch": dom_flop,
            "mean_launch_us": layer_us[dom]["median_us"],
        },
        "layers": {nm: {**st, "TFLOP/s": round(2 * n * shapes[nm][1] * shapes[nm][2] / (st["median_us"] * 1e-6) / 1e12, 1),
                        "frac": round(2 * n * shapes[nm][1] * shapes[nm][2] / (st["median_us"] * 1e-6) / 1e12
                                      / BF16_PEAK_TFLOPS, 4)}
                   for nm, st in layer_us.items()},
        "device": props.name,
        "wall_s_timed_region": round(wall, 4),
    }

    others = {}
    if not args.no_others:
        med = timer.runs(bind_chain(wq.PATH_MFMA_F32), 2, args.reps, warm=1)
        st = _stats(med)
        others["encoder_chain_f32_accurate"] = {**st, "ms": round(st["median_us"] / 1e3, 4),
                                                "TFLOP/s": round(flop_step / (st["median_us"] * 1e-6) / 1e12, 1),
                                                "frac": round(flop_step / (st["median_us"] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)}
        # Calibration on the same GPU: the vendor GEMM (torch's bf16 linear, hipBLASLt) on the four
        # layer shapes over the same 24 weights, given the easier problem: X already in bf16, no
        # bias, activation or residual.
        vendor = {}
        for nm in ("qkv", "out", "fc1", "fc2"):
            x_, m_, k_, _, _ = shapes[nm]
            xv = x_.to(torch.bfloat16)
            wv = [W_[nm][0].view(torch.bfloat16).view(m_, k_) for W_ in layers]
            vendor[nm] = _stats(timer.runs(lambda i: torch.nn.functional.linear(xv, wv[i % len(wv)]), len(wv),
                                           args.reps))
            del xv, wv
        vsum = sum(v["median_us"] for v in vendor.values())
        others["vendor_gemm_bf16_same_shapes"] = {
            "layers_us": {nm: v["median_us"] for nm, v in vendor.items()},
            "layer_sum_us": round(vsum, 3),
            "TFLOP/s": round(flop_layer / (vsum * 1e-6) / 1e12, 1),
            "frac": round(flop_layer / (vsum * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "this_chain_layer_sum_us": round(sum(v["median_us"] for v in layer_us.values()), 3),
            "note": "torch.nn.functional.linear in bf16 (hipBLASLt) with X converted to bf16 beforehand and no "
                    "epilogue; this library's layers take f32 X and fuse bias, GELU and the residual",
        }
    del layers, qkv, f, h
    torch.cuda.empty_cache()

    return line, others, acts


def _rotated(torch, base, rows, copies):
    """`copies` distinct weights: the rows of `base` rolled by 7 c (no two copies share content)."""
    return torch.stack([torch.roll(base.view(rows, -1), shifts=7 * c, dims=0).reshape(-1) for c in range(copies)])


def _rooflines(torch, wq, synth, dev, timer, to_dev, args, read_traffic):
    out = {}
    legs = args.legs_set
    R = args.reps
    floor = Floor(torch, timer, dev) if legs & {"c2", "c3", "c4", "moe1", "moe64", "q4k"} else None

    # C1: bf16 GEMM 64x256x256 + bias + GELU (launch-bound by size)
    if "c1" in legs:
        _c1(torch, wq, synth, dev, timer, to_dev, R, out, read_traffic)
    if "c2" in legs:
        _c2(torch, wq, synth, dev, timer, to_dev, R, out, floor, read_traffic)
    if "c3" in legs:
        _c3(torch, wq, synth, dev, timer, to_dev, R, out, floor, read_traffic)
    if legs & {"c4", "moe1", "moe64"}:
        _moe(torch, wq, synth, dev, timer, to_dev, R, out, floor, read_traffic, legs)
    if "q4k" in legs:
        _q4k(torch, wq, synth, dev, timer, to_dev, R, out, floor, read_traffic)
    torch.cuda.empty_cache()
    return out


def _q4k(torch, wq, synth, dev, timer, to_dev, R, out, floor, read_traffic):
    """Q4_K (hanzo-ml matvec_q4k_gpu / moe_matvec_gpu) on the Q4_0 workloads' shapes: 14336 x 4096 at
    one token, and 16 tokens top-2 of 8 experts, gated."""
    m, k = 14336, 4096
    wb = wq.weight_bytes(wq.W_Q4_K, m, k)
    nc = max(2, -(-ROTATE_BYTES // wb))
    W = _rotated(torch, to_dev(synth.q4_k_weight(synth.rng(0, 6, 1), m, k).reshape(-1)), m, nc)
    x = to_dev(synth.normal_f32(synth.rng(0, 6, 2), (1, k), 1.0))
    y = torch.empty((1, m), device=dev)
    gs = [wq.bind_gemm(x, W[i], wq.W_Q4_K, m=m, k=k, out=y) for i in range(nc)]
    st = _stats(timer.runs(lambda i: gs[i % nc](), 100, R))
    out["NEXT2_q4_k_14336x4096_n1"] = _hbm_entry(st, wb, floor.us(wb, R), read_traffic(COUNTERS, "q4_k_n1"),
                                                 extra={"copies": nc})
    del W
    banks = [to_dev(np.stack([synth.q4_k_weight(synth.rng(0, 6, 3, b, e), m, k) for e in range(8)]).reshape(-1))
             for b in range(3)]
    x16 = to_dev(synth.normal_f32(synth.rng(0, 6, 4), (16, k), 1.0))
    ids, gates = synth.moe_routing(synth.rng(0, 6, 5), 16, 8, 2)
    ids_d, gates_d = to_dev(ids), to_dev(gates)
    y16 = torch.empty((16, m), device=dev)
    touched = len(np.unique(ids))
    st = _stats(timer.runs(lambda i: wq.moe_matvec(x16, banks[i % 3], wq.W_Q4_K, ids_d, gates_d, n_experts=8, m=m,
                                                   k=k, out=y16), 30, R))
    key = "NEXT2_moe_q4_k_16tok_top2_of_8"
    out[key] = _hbm_entry(st, touched * wb, floor.us(touched * wb, R), read_traffic(COUNTERS, key),
                          extra={"experts_touched": touched, "n_experts": 8, "tokens": 16, "top_k": 2})
    del banks


def _c1(torch, wq, synth, dev, timer, to_dev, R, out, read_traffic):
    c = synth.config_gemm_small()
    x, w, b = to_dev(c["x"]), to_dev(c["w"]), to_dev(c["bias"])
    y = torch.empty((64, 256), device=dev)
    g = wq.bind_gemm(x, w, wq.W_BF16, m=256, k=256, bias=b, gelu=True, out=y)
    st = _stats(timer.runs(lambda i: g(), 200, R))
    fl = 2 * 64 * 256 * 256
    tf = fl / (st["median_us"] * 1e-6) / 1e12
    out["C1_gemm_bf16_64x256x256_gelu"] = {**st, "TFLOP/s": round(tf, 3), "frac": round(tf / BF16_PEAK_TFLOPS, 5),
                                           "bound": "mfma (launch-bound by size)",
                                           "traffic": read_traffic(COUNTERS, "c1_64x256x256")}


def _c2(torch, wq, synth, dev, timer, to_dev, R, out, floor, read_traffic):
    """Q8_0 4096x4096 at n = 1 and n = 4."""
    m = k = 4096
    wb = wq.weight_bytes(wq.W_Q8_0, m, k)
    nc = max(2, -(-ROTATE_BYTES // wb))
    W = _rotated(torch, to_dev(synth.q8_0_weight(synth.rng(0, 2, 1, 0), m, k).reshape(-1)), m, nc)
    fl_st = floor.us(wb, R)
    for n_ in (1, 4):
        x = to_dev(synth.config_q8_matvec(n_)["x"])
        y = torch.empty((n_, m), device=dev)
        gs = [wq.bind_gemm(x, W[i], wq.W_Q8_0, m=m, k=k, out=y) for i in range(nc)]
        st = _stats(timer.runs(lambda i: gs[i % nc](), 200, R))
        out[f"C2_q8_0_4096x4096_n{n_}"] = _hbm_entry(st, wb, fl_st, read_traffic(COUNTERS, f"q8_0_n{n_}"),
                                                      extra={"copies": nc})
    del W


def _c3(torch, wq, synth, dev, timer, to_dev, R, out, floor, read_traffic):
    """Q4_0 14336x4096 at n = 1."""
    m, k = 14336, 4096
    wb = wq.weight_bytes(wq.W_Q4_0, m, k)
    nc = max(2, -(-ROTATE_BYTES // wb))
    cfg = synth.config_q4_matvec()
    W = _rotated(torch, to_dev(cfg["w"].reshape(-1)), m, nc)
    x = to_dev(cfg["x"])
    y = torch.empty((1, m), device=dev)
    gs = [wq.bind_gemm(x, W[i], wq.W_Q4_0, m=m, k=k, out=y) for i in range(nc)]
    st = _stats(timer.runs(lambda i: gs[i % nc](), 100, R))
    fl = floor.us(wb, R)
    out["C3_q4_0_14336x4096_n1"] = _hbm_entry(st, wb, fl, read_traffic(COUNTERS, "q4_0_n1"), extra={"copies": nc})
    # One GPU's share of the MoE workload split expert-parallel over 8 GPUs: one expert with its
    # routed tokens (32 slots over 8 experts: 4 on average), the same matvec at n = 4.
    x4 = to_dev(synth.normal_f32(synth.rng(0, 4, 7), (4, k), 1.0))
    y4 = torch.empty((4, m), device=dev)
    g4 = [wq.bind_gemm(x4, W[i], wq.W_Q4_0, m=m, k=k, out=y4) for i in range(nc)]
    st4 = _stats(timer.runs(lambda i: g4[i % nc](), 100, R))
    out["C3_q4_0_14336x4096_n4_expert_share"] = _hbm_entry(
        st4, wb, fl, None, extra={"copies": nc, "note": "one expert with the 4 tokens it receives on average: "
                                                          "the per-GPU share of the MoE workload split over 8 GPUs"})
    del W


def _moe(torch, wq, synth, dev, timer, to_dev, R, out, floor, read_traffic, legs):
    """The MoE workload (C4) and the sparse routings: Q4_0 experts 14336x4096, gated; banks rotated."""
    m, k = 14336, 4096
    wb = wq.weight_bytes(wq.W_Q4_0, m, k)
    cm = synth.config_moe()
    banks = [to_dev(synth.config_moe(bank=bank)["w"].reshape(-1)) for bank in range(3)]
    eb = wb
    x16 = to_dev(cm["x"])

    def moe_entry(key, n_exp, ids, gates, bank_list):
        n_tok, top_k = ids.shape
        x = x16[:n_tok]
        ids_d, gates_d = to_dev(ids), to_dev(gates)
        y = torch.empty((n_tok, m), device=dev)
        touched = len(np.unique(ids))
        calls = max(10, min(60, int(4e9 // (touched * eb))))
        st = _stats(timer.runs(lambda i: wq.moe_matvec(x, bank_list[i % len(bank_list)], wq.W_Q4_0, ids_d, gates_d,
                                                       n_experts=n_exp, m=m, k=k, out=y), calls, R))
        out[key] = _hbm_entry(st, touched * eb, floor.us(touched * eb, R), read_traffic(COUNTERS, key),
                              extra={"experts_touched": touched, "n_experts": n_exp, "tokens": n_tok, "top_k": top_k})

    if "c4" in legs:
        moe_entry("C4_moe_q4_0_16tok_top2_of_8", 8, cm["ids"], cm["gates"], banks)
    if "moe1" in legs:
        ids, gates = synth.moe_routing(synth.rng(0, 4, 10), 1, 8, 2)
        moe_entry("moe_q4_0_1tok_top2_of_8", 8, ids, gates, banks)
    if "moe64" not in legs:
        return
    # 64 experts per bank, two banks: expert e of bank c is expert e % 8 of the 8-expert bank
    # (c + e) % 3 with its rows rolled by 13 (e // 8) + 5 c, so no two experts share content.
    big = []
    for c in range(2):
        parts = []
        for e in range(64):
            src = banks[(c + e) % 3][(e % 8) * eb:(e % 8 + 1) * eb].view(m, -1)
            parts.append(torch.roll(src, shifts=13 * (e // 8) + 5 * c, dims=0).reshape(-1))
        big.append(torch.cat(parts))
        del parts
    del banks
    ids, gates = synth.moe_routing(synth.rng(0, 4, 11), 16, 64, 2)
    moe_entry("moe_q4_0_16tok_top2_of_64", 64, ids, gates, big)
    del big


def _encoder(torch, wq, synth, dev, timer, to_dev, args, read_traffic):
    """The rest of the encoder block at the workload's size (1500 frames, d = 1024, 8 heads of 128,
    all dims rotated, the last 100 frames masked): LayerNorm, q/k norm + rotation and attention
    each alone, and the whole 24-block forward (embedding LayerNorm, 24 blocks with bf16 weights,
    final LayerNorm). Returns (rooflines, others)."""
    R = args.reps
    n, d, heads, ff = synth.ENCODER_N, synth.ENCODER_D, synth.ENCODER_HEADS, synth.ENCODER_FF
    hd, rot = d // heads, synth.ENCODER_ROT
    g = synth.rng(60)
    rl, oth = {}, {}

    # LayerNorm [1500][1024]: reads and writes the rows once (HBM-bound).
    xs = [to_dev(synth.normal_f32(synth.rng(61, i), (n, d), 1.0)) for i in range(4)]
    wb = to_dev(synth.layer_norm_weights(g, d))
    ys = [torch.empty((n, d), device=dev) for _ in range(4)]
    # Bound calls: the kernel takes ~4 us, less than a call through the plain binding costs the host,
    # so timing that binding would time the host.
    ln = [wq.bind_layer_norm(xs[i], wb, d=d, out=ys[i]) for i in range(4)]
    st = _stats(timer.runs(lambda i: ln[i % 4](), 200, R))
    nb = 2 * n * d * 4 + 2 * d * 4
    gbs = nb / (st["median_us"] * 1e-6) / 1e9
    rl["NEXT4_layer_norm_1500x1024"] = {**st, "GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                                        "bound": "hbm", "bytes": nb,
                                        "traffic": read_traffic(COUNTERS, "enc_layer_norm")}
    del xs, ys, ln

    # q/k norm + rotation in place on [1500][3 x 1024]: q and k read and written once.
    qkvs = [to_dev(synth.normal_f32(synth.rng(62, i), (n, 3 * d), 1.0)) for i in range(4)]
    qn, kn = to_dev(synth.layer_norm_weights(g, hd)), to_dev(synth.layer_norm_weights(g, hd))
    cs = wq.rope_table(n, rot).to(dev)
    st = _stats(timer.runs(lambda i: wq.qk_norm_rope(qkvs[i % 4], cs, n=n, heads=heads, hd=hd, rot=rot, qn=qn, kn=kn),
                           200, R))
    nb = 2 * n * 2 * d * 4 + n * rot * 4
    gbs = nb / (st["median_us"] * 1e-6) / 1e9
    rl["NEXT4_qk_norm_rope_1500x8x128"] = {**st, "GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                                           "bound": "hbm", "bytes": nb,
                                           "traffic": read_traffic(COUNTERS, "enc_qk_norm_rope")}

    # Attention: the call (pack + flash kernel); 4 n^2 hd FLOP per head, masked keys included.
    valid = to_dev(synth.key_mask(n, synth.ENCODER_VALID))
    att = torch.empty((n, d), device=dev)
    ws = torch.empty(wq.attention_workspace_bytes(n, heads, hd), dtype=torch.uint8, device=dev)
    scale = float(np.float32(1.0) / np.sqrt(np.float32(hd)))
    st = _stats(timer.runs(lambda i: wq.attention(qkvs[i % 4], valid, n=n, heads=heads, hd=hd, scale=scale, out=att,
                                                  workspace=ws), 100, R))
    fl = 4 * n * n * hd * heads
    tf = fl / (st["median_us"] * 1e-6) / 1e12
    rl["NEXT4_attention_1500x8x128"] = {**st, "TFLOP/s": round(tf, 1), "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                                        "bound": "mfma", "flop": fl,
                                        "note": "pack (K, V to bf16) + flash kernel; kernel split in the trace",
                                        "traffic": {"pack": read_traffic(COUNTERS, "enc_attn_pack"),
                                                    "attention_kernel": read_traffic(COUNTERS, "enc_attention")}}
    del qkvs, att, ws

    if args.no_others:
        return rl, oth
    # The forward: 24 blocks, embedded input rows.
    model = synth.encoder_model(synth.ENCODER_LAYERS)
    layers = [{k: (None if v is None else to_dev(v)) for k, v in L.items()} for L in model["layers"]]
    descs = [wq.encoder_layer_desc(L) for L in layers]
    en, fn_ = to_dev(model["embed_norm"]), to_dev(model["final_norm"])
    x = to_dev(synth.normal_f32(synth.rng(63), (n, d), 1.0))
    h = torch.empty((n, d), device=dev)
    y = torch.empty((n, d), device=dev)
    wsl = torch.empty(wq.encoder_workspace_bytes(n, d, heads, ff), dtype=torch.uint8, device=dev)

    def forward(_):
        wq.layer_norm(x, en, d=d, out=h)
        for D in descs:
            wq.encoder_layer(h, D, wq.W_BF16, valid, cs, n=n, d=d, heads=heads, rot=rot, inter=ff, workspace=wsl)
        wq.layer_norm(h, fn_, d=d, out=y)

    st = _stats(timer.runs(forward, 2, R, warm=1))
    fl_layer = 2 * n * (3 * d * d + d * d + ff * d + d * ff) + 4 * n * n * hd * heads
    fl_fwd = synth.ENCODER_LAYERS * fl_layer
    oth["encoder_forward_24_layers"] = {
        **st, "ms": round(st["median_us"] / 1e3, 4),
        "TFLOP/s": round(fl_fwd / (st["median_us"] * 1e-6) / 1e12, 1), "flop": fl_fwd,
        "workload": "embedding LayerNorm, 24 pre-norm blocks (LayerNorm, QKV 1500x3072x1024, q/k norm + RoPE, "
                    "attention 8x128 over 1400 valid of 1500 frames, out 1500x1024x1024 + residual, LayerNorm, "
                    "MLP 4096 + GELU + residual; bf16 weights N(0,0.02)), final LayerNorm"}
    del layers, descs, wsl
    torch.cuda.empty_cache()
    return rl, oth


def _others(torch, wq, synth, dev, timer, to_dev, args):
    out = {}
    R = args.reps
    k = 4096
    # f16 weights 4096 x 4096 at n = 1 (wavo Linear type 1), rotated copies
    m16 = 4096
    wb16 = wq.weight_bytes(wq.W_F16, m16, k)
    nc16 = max(2, -(-ROTATE_BYTES // wb16))
    base = to_dev(synth.weight(synth.rng(53), wq.W_F16, m16, k).reshape(-1).view(np.uint8))
    Wc = _rotated(torch, base, m16, nc16)
    x = to_dev(synth.normal_f32(synth.rng(54), (1, k), 1.0))
    y = torch.empty((1, m16), device=dev)
    gs = [wq.bind_gemm(x, Wc[i], wq.W_F16, m=m16, k=k, out=y) for i in range(nc16)]
    st = _stats(timer.runs(lambda i: gs[i % nc16](), 100, R))
    gbs = wb16 / (st["median_us"] * 1e-6) / 1e9
    out["matvec_f16_4096x4096_n1"] = {**st, "GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
    del Wc

    # The MLP-up shape (X[1500 x 1024], W[4096 x 1024], bias + GELU) with other weight types.
    n, d, ff = synth.ENCODER_N, synth.ENCODER_D, synth.ENCODER_FF
    a3 = to_dev(synth.encoder_activations()["a3"])
    f = torch.empty((n, ff), device=dev)
    fl = 2 * n * ff * d
    for wt, name in ((wq.W_F16, "f16"), (wq.W_F32, "f32"), (wq.W_Q8_0, "q8_0"), (wq.W_Q4_0, "q4_0")):
        ws = [to_dev(synth.weight(synth.rng(40 + i, wt), wt, ff, d).reshape(-1)) for i in range(4)]
        bq = to_dev(synth.normal_f32(synth.rng(44, wt), (ff,), 0.1))
        for path, suffix in ((wq.PATH_AUTO, ""), (wq.PATH_MFMA_F32, "_f32acc")):
            if wt in (wq.W_F16, wq.W_F32) and suffix:
                continue
            gq = [wq.bind_gemm(a3, w_, wt, m=ff, k=d, bias=bq, gelu=True, out=f, path=path) for w_ in ws]
            st = _stats(timer.runs(lambda i: gq[i % 4](), 20, R))
            tf = fl / (st["median_us"] * 1e-6) / 1e12
            out[f"gemm_{name}{suffix}_{n}x{ff}x{d}_gelu"] = {**st, "TFLOP/s": round(tf, 1),
                                                              "frac": round(tf / BF16_PEAK_TFLOPS, 4)}
        del ws
    return out


def _cpu_time(fn, runs):
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def _cpu_chain(synth, acts):
    """The oracle on 2 of the chain's 24 layers, all 1500 frames: decode + f64 product + epilogue."""
    import oracle
    n, d, ff = synth.ENCODER_N, synth.ENCODER_D, synth.ENCODER_FF
    x = {nm: np.asarray(acts[nm], np.float64) for nm in ("a1", "a2", "a3")}
    h0 = np.asarray(acts["h0"], np.float64)
    layers = [synth.encoder_layer_weights(L) for L in range(2)]

    def run():
        h = h0
        for lw in layers:
            def lin(a, key, flags, y_old=None):
                w = oracle.decode(lw[key]["w"], oracle.W_BF16, lw[key]["m"], lw[key]["k"])
                return oracle.epilogue(a @ w.T, flags, lw[key]["bias"], y_old)
            lin(x["a1"], "qkv", 1)
            h = lin(x["a2"], "out", 5, h)
            fo = lin(x["a3"], "fc1", 3)
            h = lin(fo, "fc2", 5, h)
        return h

    sec = _cpu_time(run, 1)
    fl = 2 * 2 * n * (3 * d * d + d * d + ff * d + d * ff)
    return {"value": round(fl / sec / 1e9, 2), "unit": "GFLOP/s", "cores": _threads(), "kind": "oracle",
            "sample": f"2 of the 24 layers (all 1500 frames, all four GEMMs): {fl / 1e9:.1f} GFLOP in {sec:.2f} s, "
                      "f64 decode + numpy product + epilogue"}


def _cpu_encoder(synth):
    """The oracle on the encoder-block workloads: LayerNorm, q/k norm + rotation and attention at
    full size (median of 3 runs), and one of the forward's 24 blocks."""
    from oracle import encoder as enc
    n, d, heads, ff = synth.ENCODER_N, synth.ENCODER_D, synth.ENCODER_HEADS, synth.ENCODER_FF
    hd, rot = d // heads, synth.ENCODER_ROT
    cores = _threads()
    g = synth.rng(70)
    x = synth.normal_f32(g, (n, d), 1.0)
    wb = synth.layer_norm_weights(g, d)
    qkv = synth.normal_f32(g, (n, 3 * d), 1.0)
    qn, kn = synth.layer_norm_weights(g, hd), synth.layer_norm_weights(g, hd)
    cos, sin = enc.rope_table(n, rot)
    valid = synth.key_mask(n, synth.ENCODER_VALID)
    scale = float(np.float32(1.0) / np.sqrt(np.float32(hd)))
    res = {}
    sec = _cpu_time(lambda: enc.layer_norm(x, wb), 3)
    res["NEXT4_layer_norm_1500x1024"] = {"value": round((2 * n * d * 4 + 2 * d * 4) / sec / 1e9, 3), "unit": "GB/s",
                                         "cores": cores, "kind": "oracle",
                                         "sample": f"the full call, median of 3 runs: {sec:.4f} s"}
    sec = _cpu_time(lambda: enc.qk_norm_rope(qkv, heads, hd, rot, cos, sin, qn, kn), 3)
    res["NEXT4_qk_norm_rope_1500x8x128"] = {"value": round((4 * n * d * 4 + n * rot * 4) / sec / 1e9, 3),
                                            "unit": "GB/s", "cores": cores, "kind": "oracle",
                                            "sample": f"the full call, median of 3 runs: {sec:.4f} s"}
    sec = _cpu_time(lambda: enc.attention(qkv, valid, heads, hd, scale), 3)
    res["NEXT4_attention_1500x8x128"] = {"value": round(4 * n * n * hd * heads / sec / 1e9, 2), "unit": "GFLOP/s",
                                         "cores": cores, "kind": "oracle",
                                         "sample": f"the full call, median of 3 runs: {sec:.3f} s"}
    L = synth.encoder_block_weights(0)
    h = synth.normal_f32(g, (n, d), 1.0)
    sec = _cpu_time(lambda: enc.encoder_layer(h, L, 0, valid, heads, rot, cos, sin), 1)
    fl = 2 * n * (3 * d * d + d * d + ff * d + d * ff) + 4 * n * n * hd * heads
    res["encoder_forward_24_layers"] = {"value": round(fl / sec / 1e9, 2), "unit": "GFLOP/s", "cores": cores,
                                        "kind": "oracle",
                                        "sample": f"1 of the 24 blocks, all 1500 frames: {fl / 1e9:.1f} GFLOP in "
                                                  f"{sec:.2f} s"}
    return res


def _cpu_configs(synth):
    """The oracle on each matvec / MoE workload (C4: 2 of its 8 experts), median of 3 runs."""
    import oracle
    res = {}
    cores = _threads()

    def entry(sec, nbytes, sample, flop=None):
        e = {"value": round(nbytes / sec / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
             "sample": sample + f", median of 3 runs: {sec:.3f} s"}
        if flop:
            e = {"value": round(flop / sec / 1e9, 3), "unit": "GFLOP/s", "cores": cores, "kind": "oracle",
                 "sample": sample + f", median of 3 runs: {sec:.4f} s"}
        return e

    c = synth.config_gemm_small()

    def c1():
        w = oracle.decode(c["w"], oracle.W_BF16, 256, 256)
        oracle.epilogue(np.asarray(c["x"], np.float64) @ w.T, 3, c["bias"])
    res["C1_gemm_bf16_64x256x256_gelu"] = entry(_cpu_time(c1, 3), 0, "the full call", flop=2 * 64 * 256 * 256)
    for n_ in (1, 4):
        cq = synth.config_q8_matvec(n_)

        def c2():
            w = oracle.decode(cq["w"], oracle.W_Q8_0, 4096, 4096)
            np.asarray(cq["x"], np.float64) @ w.T
        res[f"C2_q8_0_4096x4096_n{n_}"] = entry(_cpu_time(c2, 3), 17825792, "the full call")
    c3c = synth.config_q4_matvec()

    def c3():
        w = oracle.decode(c3c["w"], oracle.W_Q4_0, 14336, 4096)
        np.asarray(c3c["x"], np.float64) @ w.T
    res["C3_q4_0_14336x4096_n1"] = entry(_cpu_time(c3, 3), 33030144, "the full call")
    cm = synth.config_moe()
    ids = cm["ids"]
    experts = list(np.unique(ids))[:2]

    def c4():
        x64 = np.asarray(cm["x"], np.float64)
        for e in experts:
            w = oracle.decode(cm["w"][e], oracle.W_Q4_0, 14336, 4096)
            t_idx, _ = np.nonzero(ids == e)
            x64[t_idx] @ w.T
    res["C4_moe_q4_0_16tok_top2_of_8"] = entry(_cpu_time(c4, 3), 2 * 33030144,
                                               f"experts {experts[0]} and {experts[1]} of the 8 (their routed tokens)")
    wk = synth.q4_k_weight(synth.rng(0, 6, 1), 14336, 4096)
    xk = synth.normal_f32(synth.rng(0, 6, 2), (1, 4096), 1.0)

    def q4k():
        w = oracle.decode(wk, oracle.W_Q4_K, 14336, 4096)
        np.asarray(xk, np.float64) @ w.T
    res["NEXT2_q4_k_14336x4096_n1"] = entry(_cpu_time(q4k, 3), 33030144, "the full call")
    ids_k, _ = synth.moe_routing(synth.rng(0, 6, 5), 16, 8, 2)
    xk16 = synth.normal_f32(synth.rng(0, 6, 4), (16, 4096), 1.0)
    ek = list(np.unique(ids_k))[:2]
    wks = {e: synth.q4_k_weight(synth.rng(0, 6, 3, 0, e), 14336, 4096) for e in ek}

    def q4k_moe():
        x64 = np.asarray(xk16, np.float64)
        for e in ek:
            w = oracle.decode(wks[e], oracle.W_Q4_K, 14336, 4096)
            t_idx, _ = np.nonzero(ids_k == e)
            x64[t_idx] @ w.T
    res["NEXT2_moe_q4_k_16tok_top2_of_8"] = entry(_cpu_time(q4k_moe, 3), 2 * 33030144,
                                                  f"experts {ek[0]} and {ek[1]} of the 8 (their routed tokens)")
    return res


if __name__ == "__main__":
    main()
