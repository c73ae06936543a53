#!/usr/bin/env python3
"""Benchmark of the block-quantized product on one MI355X.

Step = one decode pass over a 7B-shaped decoder layer with Q4_K weights
(q, k, v, o 4096-wide, gate/up 14336x4096, down 4096x14336), batch 1: four
activation quantizations and seven GEMVs. Weights are rotated over enough
distinct packed copies of the layer that the 256 MB last-level cache cannot
hold them, so every step streams its weights from HBM.

Headline value: effective packed-weight GB/s = weight bytes per step / step
time. Also reported: the GEMV kernel's roofline fraction (HIP events around
every launch), the prefill GEMM (512 x 14336 x 4096, int8 TOPS), the
decode-vs-prefill crossover at M in {1, 8, 64}, and the CPU oracle on a bounded
sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--copies R] [--no-cpu-baseline]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 matrix-core peak, TOP/s


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--copies", type=int, default=8,
                   help="distinct packed copies of the layer rotated through")
    p.add_argument("--gemm-iters", type=int, default=50)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the product "
                                   "shards by output rows, see the design notes",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    from block_quantized_qblk_amd import qblk, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    Q4_K = qblk.Q4_K
    layer = synth.LAYER_7B
    R = args.copies

    # ------------------------------------------------------------ setup (untimed)
    log(f"packing {R} copies of the 7B layer ({len(layer)} Q4_K linears)")
    t0 = time.time()
    copies = []
    for c in range(R):
        packed = {}
        for idx, (name, n, k) in enumerate(layer):
            w = synth.torch_weights("outliers", 3000 + 100 * c + idx, n, k, device=dev)
            packed[name] = qblk.qblk_pack_weights(Q4_K, w)
            del w
        copies.append(packed)
    torch.cuda.synchronize()
    log(f"packed in {time.time() - t0:.1f}s")
    weight_bytes = sum(qblk.qblk_weight_bytes(Q4_K, n, k) for _, n, k in layer)

    # activations: attention input (q,k,v), attention output (o), MLP input
    # (gate, up), MLP hidden (down)
    acts = {
        "attn": synth.torch_activations(3099, 1, 4096, device=dev),
        "o": synth.torch_activations(3098, 1, 4096, device=dev),
        "mlp": synth.torch_activations(3097, 1, 4096, device=dev),
        "down": synth.torch_activations(3096, 1, 14336, device=dev),
    }
    xq = {key: torch.empty(qblk.qblk_act_bytes(1, v.shape[1]), dtype=torch.uint8, device=dev)
          for key, v in acts.items()}
    src = {"q": "attn", "k": "attn", "v": "attn", "o": "o", "gate": "mlp", "up": "mlp",
           "down": "down"}
    ys = {name: torch.empty((1, n), dtype=torch.float32, device=dev) for name, n, _ in layer}

    def step(s, events=None):
        packed = copies[s % R]
        qblk.qblk_quantize_act(acts["attn"], out=xq["attn"])
        for name, n, k in layer:
            if name == "o":
                qblk.qblk_quantize_act(acts["o"], out=xq["o"])
            elif name == "gate":
                qblk.qblk_quantize_act(acts["mlp"], out=xq["mlp"])
            elif name == "down":
                qblk.qblk_quantize_act(acts["down"], out=xq["down"])
            if events is not None:
                events[name][0].record()
            qblk.qblk_gemv(Q4_K, packed[name], n, k, xq[src[name]], 1, y=ys[name])
            if events is not None:
                events[name][1].record()

    # ------------------------------------------------------------ timed: steps
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for s in range(args.steps):
        step(s)
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    value = weight_bytes / (ms_step * 1e-3) / 1e9
    log(f"step {ms_step * 1e3:.2f} us, {value:.1f} GB/s effective weight bandwidth")

    # ------------------------------------------------------------ timed: per-launch events
    K_EV = min(args.steps, 100)
    dur = {name: 0.0 for name, _, _ in layer}
    for s in range(K_EV):
        ev = {name: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for name, _, _ in layer}
        step(s, ev)
        torch.cuda.synchronize()
        for name in dur:
            dur[name] += ev[name][0].elapsed_time(ev[name][1])
    per_launch = {}
    alg_bytes_total = 0
    dur_total_ms = 0.0
    for name, n, k in layer:
        alg = qblk.qblk_weight_bytes(Q4_K, n, k) + qblk.qblk_act_bytes(1, k) + 4 * n
        d_ms = dur[name] / K_EV
        per_launch[name] = {"n": n, "k": k, "us": round(d_ms * 1e3, 3),
                            "GBps": round(alg / (d_ms * 1e-3) / 1e9, 1)}
        alg_bytes_total += alg
        dur_total_ms += d_ms
    achieved = alg_bytes_total / (dur_total_ms * 1e-3) / 1e9
    log(f"gemv kernel: {achieved:.1f} GB/s over {dur_total_ms * 1e3:.2f} us per layer")

    del copies
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ prefill GEMM
    gemm = gemm_bench(torch, qblk, synth, dev, args.gemm_iters)

    # ------------------------------------------------------------ CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(synth, args.cpu_seconds)

    out = {
        "metric": "Q4_K GEMV effective weight GB/s (% HBM peak); prefill GEMM int8 TOPS",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "q4_k_gemv_7b_layer",
            "linears": {name: [n, k] for name, n, k in layer},
            "batch": 1,
            "weight_bytes_per_step": weight_bytes,
            "rotating_copies": R,
            "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "gemv_kernel<Q4_K,1>",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "per_launch": per_launch,
        },
        "gemm": gemm,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def gemm_bench(torch, qblk, synth, dev, iters):
    """Q4_K prefill GEMM 512 x 14336 x 4096, and M in {1, 8, 64} against the
    GEMV on the same weights."""
    Q4_K = qblk.Q4_K
    n, k = 14336, 4096
    w = synth.torch_weights("outliers", 4000, n, k, device=dev)
    wq = qblk.qblk_pack_weights(Q4_K, w)
    del w
    res = {}
    for m in (512, 1, 8, 64):
        x = synth.torch_activations(4099, m, k, device=dev)
        xq = qblk.qblk_quantize_act(x)
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        row = {}
        fns = [("gemm", qblk.qblk_gemm)]
        if m <= 64:
            fns.append(("gemv", qblk.qblk_gemv))
        for fname, f in fns:
            for _ in range(5):
                f(Q4_K, wq, n, k, xq, m, y=y)
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(iters)]
            for a, b in ev:
                a.record()
                f(Q4_K, wq, n, k, xq, m, y=y)
                b.record()
            torch.cuda.synchronize()
            us = 1e3 * sum(a.elapsed_time(b) for a, b in ev) / iters
            ops = 2.0 * m * n * k
            row[fname] = {"us": round(us, 3), "TOPS": round(ops / (us * 1e-6) / 1e12, 2)}
        res[f"m{m}"] = row
        log(f"gemm m={m}: {row}")
    g = res["m512"]["gemm"]
    return {
        "workload": "q4_k_gemm_512x14336x4096",
        "TOPS": g["TOPS"],
        "us": g["us"],
        "roofline": {"bound": "mfma", "kernel": "gemm_kernel<Q4_K>", "achieved": g["TOPS"],
                     "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                     "frac": round(g["TOPS"] / INT8_PEAK_TOPS, 4), "traffic": None},
        "crossover": res,
    }


def cpu_baseline(synth, seconds):
    """The oracle (NumPy, int64 block sums + fp64 scaling) on the host cores,
    over a bounded sample of the same layer: the first 256 rows of each of
    the seven linears, encoded untimed, then activation quantization plus the
    product timed, repeated until `seconds` have elapsed."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from oracle import qblk_oracle as o
    rows = 256
    samples = []
    for idx, (name, n, k) in enumerate(synth.LAYER_7B):
        w = synth.weights_outliers(3900 + idx, rows, k)
        _, enc = o.encode_weights(o.TYPE_Q4_K, w)
        x = synth.activations(3999 - idx, 1, k)
        samples.append((enc, x, o.row_bytes(o.TYPE_Q4_K, k) * rows))
    done_bytes = 0
    t0 = time.perf_counter()
    reps = 0
    while True:
        for enc, x, nbytes in samples:
            act = o.quantize_act(x)
            o.product(o.TYPE_Q4_K, enc, act)
            done_bytes += nbytes
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    gbs = done_bytes / el / 1e9
    log(f"cpu oracle: {gbs:.4f} GB/s over {el:.1f}s")
    return {"value": round(gbs, 5), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {rows} rows of each of the 7 Q4_K linears of the 7B layer, "
                      f"batch 1, {reps} passes in {el:.1f}s (activation quantization + "
                      f"int64 block sums + fp64 scaling; weight encoding untimed); NumPy "
                      f"int64 einsum runs on one thread",
            "host_cores": len(os.sched_getaffinity(0))}


if __name__ == "__main__":
    main()
