"""Throughput of the weight-dequantizing linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-others]

A step is one pass of the decode workload: the Q8_0 matvec with W 4096x4096
(34-byte blocks) at n = 1 and at n = 4, i.e. two wq_gemm calls. `value` is
weight GB/s: the algorithmic weight bytes of the step (2 x 17,825,792) over
the step's time, with every input resident in HBM. To keep the 256 MB
Infinity Cache from serving the weights, the calls rotate over 36 distinct
copies of W (641 MB), so every call streams its weight from HBM.

The timed region runs the K steps' calls as two back-to-back phases on one
stream (the K n=1 calls, then the K n=4 calls), with a HIP event at the start,
between the phases and at the end. No event sits between two launches, so each
phase's time over K is that kernel's mean launch duration (as a kernel trace
sees it, plus the gap between back-to-back dispatches). Calls go through
bound calls (argument conversion done once), so the host keeps ahead of the GPU.

The same JSON line carries:
  roofline      the dominant kernel's weight bytes per launch over its mean
                launch time, against the 8 TB/s HBM peak; `traffic` is the HBM
                bytes per launch that FETCH_SIZE / WRITE_SIZE counted for that
                kernel (profiles/, scaled by a copy kernel of known size), or
                null when the kernel sources changed since they were counted;
  cpu_baseline  the f64 oracle (decode + product, numpy/OpenBLAS) on a
                bounded sample of the same workload, on the host's cores;
  others        the remaining workloads (bf16 GEMM 64x256x256, Q4_0 matvec
                14336x4096, f16 matvec 4096x4096, MoE 16 tokens top-2 of 8, the
                24-layer encoder chain, also on the f32-accurate matrix-core
                path, and the MLP-up GEMM with f16 / f32 / Q8_0 / Q4_0 weights)
                with their own TFLOP/s or GB/s and roofline fractions.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
ROTATE_BYTES = 600 * 2 ** 20


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run an elementwise copy of 256 MiB (reads and writes that many bytes), "
                         "the reference for scaling HBM byte counters")
    return ap.parse_args()


def _copies(make, nbytes):
    return max(2, -(-ROTATE_BYTES // nbytes))


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path has no "
              f"multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    import torch

    import gemv_wq_gemm_amd as wq
    import synth

    wq.lib()  # fail loudly if the library is not built
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    props = torch.cuda.get_device_properties(dev)

    if args.copy_calibration:
        src = torch.ones(64 * 2 ** 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ---------------- the decode workload: Q8_0 4096x4096 at n = 1 and n = 4 ----------------
    m = k = 4096
    wbytes = wq.weight_bytes(wq.W_Q8_0, m, k)
    ncopy = _copies(None, wbytes)
    g = synth.rng(0, 2, 1, 0)
    first = synth.q8_0_weight(g, m, k)
    W = torch.empty((ncopy, first.size), dtype=torch.uint8, device=dev)
    W[0] = to_dev(first.reshape(-1))
    for c in range(1, ncopy):  # distinct bytes per copy: rows rolled, so no two copies share content
        W[c] = torch.roll(W[0].view(m, -1), shifts=c * 7, dims=0).reshape(-1)
    xs = {n: to_dev(synth.config_q8_matvec(n)["x"]) for n in (1, 4)}
    ys = {n: torch.empty((n, m), dtype=torch.float32, device=dev) for n in (1, 4)}

    binds = {n: [wq.bind_gemm(xs[n], W[c], wq.W_Q8_0, m=m, k=k, out=ys[n]) for c in range(ncopy)]
             for n in (1, 4)}

    for i in range(args.warmup):
        for n in (1, 4):
            binds[n][i % ncopy]()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        binds[1][i % ncopy]()
    ev[1].record(stream)
    for i in range(args.steps):
        binds[4][i % ncopy]()
    ev[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = ev[0].elapsed_time(ev[2])
    ms_step = ms_total / args.steps
    value = 2 * wbytes / (ms_step * 1e-3) / 1e9
    kern = {"n1": ev[0].elapsed_time(ev[1]) / args.steps, "n4": ev[1].elapsed_time(ev[2]) / args.steps}
    dom = max(kern, key=kern.get)
    achieved = wbytes / (kern[dom] * 1e-3) / 1e9
    from gemv_wq_gemm_amd.rocprof_summary import read_traffic
    traffic = read_traffic(os.path.join(ROOT, "profiles", "matvec_q8_0_4096x4096_hbm_counters.md"), dom)

    line = {
        "metric": "matvec weight GB/s (Q8_0 decode, 1 MI355X)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (Q8_0 weights)",
        "data": "synthetic",
        "config": {
            "workload": "Q8_0 matvec decode, W 4096x4096 (34-byte blocks), X f32 [n x 4096], n in {1, 4}; "
                        "one step = the n=1 and n=4 calls",
            "weight_bytes_per_call": wbytes,
            "weight_copies_rotated": ncopy,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": f"matvec {dom} (wq_gemm, Q8_0)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else round(traffic),
            "mean_launch_us": {t: round(v * 1e3, 3) for t, v in kern.items()},
        },
        "device": props.name,
        "wall_s_timed_region": round(wall, 4),
    }

    if not args.no_others:
        line["others"] = _others(torch, wq, synth, dev, stream, to_dev)

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = _cpu_baseline(synth, args.cpu_seconds)

    print(json.dumps(line), flush=True)


def _time_calls(torch, stream, fn, reps, warm=3):
    """Mean ms per call of `reps` back-to-back calls (events only around the whole run)."""
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _others(torch, wq, synth, dev, stream, to_dev):
    out = {}
    # bf16 GEMM 64x256x256 + bias + GELU (launch-bound by size)
    c = synth.config_gemm_small()
    x, w, b = to_dev(c["x"]), to_dev(c["w"]), to_dev(c["bias"])
    y = torch.empty((64, 256), device=dev)
    g = wq.bind_gemm(x, w, wq.W_BF16, m=256, k=256, bias=b, gelu=True, out=y)
    med = _time_calls(torch, stream, lambda i: g(), 200)
    fl = 2 * 64 * 256 * 256
    out["gemm_bf16_64x256x256"] = {"us": round(med * 1e3, 3), "TFLOP/s": round(fl / (med * 1e-3) / 1e12, 3),
                                   "frac_mfma": round(fl / (med * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 5)}

    # Q4_0 14336x4096, n = 1, rotated copies
    m, k = 14336, 4096
    wb = wq.weight_bytes(wq.W_Q4_0, m, k)
    nc = max(2, -(-ROTATE_BYTES // wb))
    base = to_dev(synth.config_q4_matvec()["w"].reshape(-1))
    Wc = torch.stack([torch.roll(base.view(m, -1), shifts=7 * i, dims=0).reshape(-1) for i in range(nc)])
    x = to_dev(synth.config_q4_matvec()["x"])
    y = torch.empty((1, m), device=dev)
    gs = [wq.bind_gemm(x, Wc[i], wq.W_Q4_0, m=m, k=k, out=y) for i in range(nc)]
    med = _time_calls(torch, stream, lambda i: gs[i % nc](), 100)
    out["matvec_q4_0_14336x4096_n1"] = {"us": round(med * 1e3, 3), "GB/s": round(wb / (med * 1e-3) / 1e9, 1),
                                        "frac_hbm": round(wb / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                        "copies": nc}
    del Wc

    # f16 weights 4096 x 4096 at n = 1 (wavo Linear type 1), rotated copies
    m16 = 4096
    wb16 = wq.weight_bytes(wq.W_F16, m16, k)
    nc16 = max(2, -(-ROTATE_BYTES // wb16))
    base = to_dev(synth.weight(synth.rng(53), wq.W_F16, m16, k).reshape(-1).view(np.uint8))
    Wc = torch.stack([torch.roll(base.view(m16, -1), shifts=7 * i, dims=0).reshape(-1) for i in range(nc16)])
    x = to_dev(synth.normal_f32(synth.rng(54), (1, k), 1.0))
    y = torch.empty((1, m16), device=dev)
    gs = [wq.bind_gemm(x, Wc[i], wq.W_F16, m=m16, k=k, out=y) for i in range(nc16)]
    med = _time_calls(torch, stream, lambda i: gs[i % nc16](), 100)
    out["matvec_f16_4096x4096_n1"] = {"us": round(med * 1e3, 3), "GB/s": round(wb16 / (med * 1e-3) / 1e9, 1),
                                      "frac_hbm": round(wb16 / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                      "copies": nc16}
    del Wc

    # MoE: 16 tokens, top-2 of 8 Q4_0 experts, gated; 3 banks rotated
    banks = []
    for bank in range(3):
        cm = synth.config_moe(bank=bank)
        banks.append(to_dev(cm["w"].reshape(-1)))
    cm = synth.config_moe()
    x, ids, gates = to_dev(cm["x"]), to_dev(cm["ids"]), to_dev(cm["gates"])
    y = torch.empty((16, m), device=dev)
    touched = len(np.unique(cm["ids"]))
    med = _time_calls(torch, stream, lambda i: wq.moe_matvec(x, banks[i % 3], wq.W_Q4_0, ids, gates,
                                                             n_experts=8, m=m, k=k, out=y), 60)
    mb = touched * wb
    out["moe_q4_0_16tok_top2_of_8"] = {"us": round(med * 1e3, 3), "GB/s": round(mb / (med * 1e-3) / 1e9, 1),
                                       "frac_hbm": round(mb / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                       "experts_touched": touched}
    del banks

    # Encoder chain: 24 layers x {QKV, out+res, fc1+GELU, fc2+res}, n = 1500
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

    def bind_chain(path):
        calls = []
        for W_ in layers:
            calls.append(wq.bind_gemm(a1, W_["qkv"][0], wq.W_BF16, m=3 * d, k=d, bias=W_["qkv"][1], out=qkv,
                                      path=path))
            calls.append(wq.bind_gemm(a2, W_["out"][0], wq.W_BF16, m=d, k=d, bias=W_["out"][1], residual=True,
                                      out=h, path=path))
            calls.append(wq.bind_gemm(a3, W_["fc1"][0], wq.W_BF16, m=ff, k=d, bias=W_["fc1"][1], gelu=True,
                                      out=f, path=path))
            calls.append(wq.bind_gemm(f, W_["fc2"][0], wq.W_BF16, m=d, k=ff, bias=W_["fc2"][1], residual=True,
                                      out=h, path=path))

        def chain(_):
            for c in calls:
                c()
        return chain

    fl = 24 * 2 * n * (3 * d * d + d * d + ff * d + d * ff)
    # bf16(X) on the matrix cores (the 2^-8 bound), then X as bf16 hi + lo parts (the f32 bound;
    # twice the MFMA work, FLOP counted once).
    for path, name in ((wq.PATH_AUTO, "encoder_chain_bf16_24x4_n1500"),
                       (wq.PATH_MFMA_F32, "encoder_chain_bf16_f32acc_24x4_n1500")):
        med = _time_calls(torch, stream, bind_chain(path), 10, warm=2)
        out[name] = {"ms": round(med, 4), "TFLOP/s": round(fl / (med * 1e-3) / 1e12, 1),
                     "frac_mfma": round(fl / (med * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    del layers

    # f16 / f32 weights (two / three exact bf16 parts on the matrix cores) at the same shape.
    for wt, name in ((wq.W_F16, "f16"), (wq.W_F32, "f32")):
        ws = [to_dev(synth.weight(synth.rng(50 + i, wt), wt, ff, d).reshape(-1)) for i in range(2)]
        bq = to_dev(synth.normal_f32(synth.rng(52, wt), (ff,), 0.1))
        gq = [wq.bind_gemm(a3, w_, wt, m=ff, k=d, bias=bq, gelu=True, out=f) for w_ in ws]
        med = _time_calls(torch, stream, lambda i: gq[i % 2](), 20)
        fl = 2 * n * ff * d
        out[f"gemm_{name}_{n}x{ff}x{d}_gelu"] = {"us": round(med * 1e3, 3), "TFLOP/s": round(fl / (med * 1e-3) / 1e12, 1),
                                                 "frac_mfma": round(fl / (med * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
        del ws, gq

    # Quantized weights on the matrix cores: the encoder's MLP-up shape (X[1500 x 1024], W[4096 x 1024]
    # as Q8_0 / Q4_0 blocks, bias + GELU), 4 weight copies rotated.
    for wt, name in ((wq.W_Q8_0, "q8_0"), (wq.W_Q4_0, "q4_0")):
        ws = [to_dev(synth.weight(synth.rng(40 + i, wt), wt, ff, d).reshape(-1)) for i in range(4)]
        bq = to_dev(synth.normal_f32(synth.rng(44, wt), (ff,), 0.1))
        gq = [wq.bind_gemm(a3, w_, wt, m=ff, k=d, bias=bq, gelu=True, out=f) for w_ in ws]
        med = _time_calls(torch, stream, lambda i: gq[i % 4](), 40)
        fl = 2 * n * ff * d
        out[f"gemm_{name}_{n}x{ff}x{d}_gelu"] = {"us": round(med * 1e3, 3), "TFLOP/s": round(fl / (med * 1e-3) / 1e12, 1),
                                                 "frac_mfma": round(fl / (med * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
        gq = [wq.bind_gemm(a3, w_, wt, m=ff, k=d, bias=bq, gelu=True, out=f, path=wq.PATH_MFMA_F32) for w_ in ws]
        med = _time_calls(torch, stream, lambda i: gq[i % 4](), 40)
        out[f"gemm_{name}_f32acc_{n}x{ff}x{d}_gelu"] = {
            "us": round(med * 1e3, 3), "TFLOP/s": round(fl / (med * 1e-3) / 1e12, 1),
            "frac_mfma": round(fl / (med * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
        del ws, gq
    return out


def _cpu_baseline(synth, seconds):
    """The f64 oracle on a row sample of the decode workload (decode + product per call)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 0) for i in threadpool_info()), default=0)
    except Exception:  # pragma: no cover
        threads = 0
    cores = len(os.sched_getaffinity(0))
    rows = 512
    c1, c4 = synth.config_q8_matvec(1), synth.config_q8_matvec(4)
    w = c1["w"][:rows]
    per_call = wq_bytes = 34 * rows * (4096 // 32)
    done, t0 = 0, time.perf_counter()
    while True:
        for c in (c1, c4):
            wf = oracle.decode(w, oracle.W_Q8_0, rows, 4096)
            _ = oracle.epilogue(np.asarray(c["x"], np.float64) @ wf.T, 0)
            done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {
        "value": round(done * per_call / el / 1e9, 4),
        "unit": "GB/s",
        "cores": threads or cores,
        "kind": "oracle",
        "sample": f"{rows} of 4096 weight rows of the Q8_0 4096x4096 decode workload, calls at n=1 and n=4 "
                  f"alternating, {done} calls in {el:.1f} s (f64 decode + numpy product)",
    }


if __name__ == "__main__":
    main()
