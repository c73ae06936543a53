#!/usr/bin/env python3
"""Benchmark of the block-quantized product on one MI355X.

Step = one decode token of a 70B-shaped model with Q4_K weights: 80 layers,
each q/k/v (8192/1024/1024 x 8192), o (8192 x 8192), gate/up (28672 x 8192)
and down (8192 x 28672) - one full 38.5 GB weight stream per token. q/k/v
share an input and are packed as one 10240-row matrix, gate/up as one
57344-row matrix (rows are independent in the packed layout, so this changes
only the launch count). Per layer: four products, each one launch of
qblk_gemv_f32 (activation quantization fused into the GEMV), captured in a
HIP graph per token. The same token with a separate quantization launch
before each GEMV is reported beside it.

Headline value: effective packed-weight GB/s = weight bytes per token / time
per token (batch 1). Also reported: batch 4, the GEMV kernel's roofline
fraction (HIP-event-timed graphs of back-to-back GEMV launches, the same
boundary-to-boundary time a kernel trace reports), a 7B-shaped layer with rotated
weight copies, the prefill GEMM (512 x 14336 x 4096, int8 TOPS) with the
decode/prefill crossover at M in {1, 8, 64}, the Q4_0 and Q8_0 GEMVs, and the
CPU oracle on a bounded sample of the same workload (one process per host
core, and one process alone).

    python bench.py [--steps K] [--warmup W] [--layers L] [--no-cpu-baseline]
                    [--oracle-workers P]
"""

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 matrix-core peak, TOP/s


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30, help="timed decode tokens")
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--layers", type=int, default=80)
    p.add_argument("--copies", type=int, default=8,
                   help="distinct copies of the 7B-shaped layer rotated through")
    p.add_argument("--gemm-iters", type=int, default=50)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--oracle-workers", type=int, default=0,
                   help="processes for the parallel CPU oracle run (0: one per host core, "
                        "at most 16; 1: single-process run only)")
    p.add_argument("--traffic-probe", action="store_true",
                   help="only run a 1 GiB device copy and the GEMVs of 4 layers once "
                        "(for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs)")
    p.add_argument("--batch4-probe", action="store_true",
                   help="only run a 1 GiB device copy and one batch-4 decode token of 4 layers "
                        "(the matrix-core GEMV kernels; for rocprofv3 --pmc runs)")
    return p.parse_args()


# ---------------------------------------------------------------- timing helpers

def replay_percentiles(torch, graph, n):
    """p10 / p50 / p90 of `n` single replays, each between two events."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    evs[0].record()
    for i in range(n):
        graph.replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    t = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(n))
    q = lambda f: t[min(n - 1, int(round(f * (n - 1))))]
    return {"p10": round(q(0.1), 6), "p50": round(q(0.5), 6), "p90": round(q(0.9), 6), "replays": n}


def time_replays(torch, graphs, steps, warmup):
    for s in range(warmup):
        graphs[s % len(graphs)].replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for s in range(steps):
        graphs[s % len(graphs)].replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


class ClockSampler:
    """Samples the GPU engine clock (MHz) from a background thread while a
    timed region runs: the card's sysfs pp_dpm_sclk (the active level), else
    `amd-smi metric --clock --json`. summary() is None when neither source
    answers."""

    def __init__(self, dev_index=0, period=0.05):
        self.dev_index, self.period = dev_index, period
        self.samples, self.source = [], None
        self._stop = None

    def _sysfs_path(self):
        import glob
        try:
            import torch
            props = torch.cuda.get_device_properties(self.dev_index)
            bus = "%04x:%02x:%02x" % (getattr(props, "pci_domain_id", 0), props.pci_bus_id,
                                      props.pci_device_id)
            cands = glob.glob(f"/sys/bus/pci/devices/{bus}*/pp_dpm_sclk")
            if cands:
                return cands[0]
        except Exception:
            pass
        cands = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        return cands[0] if len(cands) == 1 else None

    @staticmethod
    def _read_sysfs(path):
        import re
        for line in open(path).read().splitlines():
            if line.rstrip().endswith("*"):
                m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                if m:
                    return float(m.group(1))
        return None

    def _read_amdsmi(self):
        import re
        import subprocess
        r = subprocess.run(["amd-smi", "metric", "--clock", "--json", "-g", str(self.dev_index)],
                           capture_output=True, text=True, timeout=10)
        if r.returncode != 0:
            return None
        text = r.stdout
        i = text.find("gfx")
        if i < 0:
            i = text.find("GFX")
        m = re.search(r'"clk"\s*:\s*\{?\s*"value"\s*:\s*"?(\d+)', text[i:]) if i >= 0 else None
        return float(m.group(1)) if m else None

    def _sample(self):
        path = self._sysfs_path()
        reader = None
        if path:
            try:
                if self._read_sysfs(path) is not None:
                    reader, self.source = (lambda: self._read_sysfs(path)), path
            except OSError:
                pass
        if reader is None:
            try:
                if self._read_amdsmi() is not None:
                    reader, self.source = self._read_amdsmi, "amd-smi metric --clock"
            except Exception:
                pass
        if reader is None:
            return
        while not self._stop.wait(self.period):
            try:
                v = reader()
            except Exception:
                v = None
            if v is not None:
                self.samples.append(v)

    def __enter__(self):
        import threading
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._sample, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join(timeout=15)
        return False

    def summary(self):
        if not self.samples:
            return None
        s = sorted(self.samples)
        return {"min": s[0], "median": s[len(s) // 2], "max": s[-1], "samples": len(s),
                "source": self.source}


# ---------------------------------------------------------------- decode model

class DecodeModel:
    """Packed Q4_K weights of `layers` layers and the per-layer launches of one
    decode token: (quantize input, GEMV) for qkv, o, gate_up and down."""

    def __init__(self, torch, qblk, synth, shapes, layers, seed0, dist, batch, dev):
        self.torch, self.qblk = torch, qblk
        self.batch = batch
        groups = [("qkv", ["q", "k", "v"]), ("o", ["o"]), ("gate_up", ["gate", "up"]),
                  ("down", ["down"])]
        dims = {name: (n, k) for name, n, k in shapes}
        self.groups = []
        for gname, parts in groups:
            k = dims[parts[0]][1]
            n = sum(dims[p][0] for p in parts)
            self.groups.append((gname, parts, n, k))
        Q4_K = qblk.Q4_K
        self.layers = []
        for layer in range(layers):
            packed = {}
            for gname, parts, n, k in self.groups:
                rb = qblk.qblk_weight_row_bytes(Q4_K, k)
                buf = torch.empty(n * rb, dtype=torch.uint8, device=dev)
                row = 0
                for p in parts:
                    pn = dims[p][0]
                    idx = [s[0] for s in shapes].index(p)
                    w = synth.torch_weights(dist, seed0 + 10 * layer + idx, pn, k, device=dev)
                    qblk.qblk_pack_weights(Q4_K, w, out=buf[row * rb:(row + pn) * rb])
                    del w
                    row += pn
                packed[gname] = buf
            self.layers.append(packed)
        torch.cuda.synchronize()
        self.synth = synth
        self.two_step = False
        self.set_batch(batch, seed0 + 900)
        self.weight_bytes = sum(qblk.qblk_weight_bytes(Q4_K, n, k)
                                for _, _, n, k in self.groups) * layers

    def set_batch(self, batch, seed):
        torch, qblk = self.torch, self.qblk
        dev = self.layers[0]["qkv"].device
        self.batch = batch
        self.x = {g: self.synth.torch_activations(seed + i, batch, k, device=dev)
                  for i, (g, _, _, k) in enumerate(self.groups)}
        self.xq = {g: torch.empty(qblk.qblk_act_bytes(batch, k), dtype=torch.uint8, device=dev)
                   for g, _, _, k in self.groups}
        self.work = {g: torch.zeros(qblk.qblk_gemv_f32_work_bytes(batch, k), dtype=torch.uint8,
                                    device=dev)
                     for g, _, _, k in self.groups}
        self.y = {g: torch.empty((batch, n), dtype=torch.float32, device=dev)
                  for g, _, n, _ in self.groups}

    def gemv(self, g, n, k, packed):
        """One group's product for the current activation: quantization fused
        into the GEMV (qblk_gemv_f32: one launch), or, with two_step,
        qblk_quantize_act then qblk_gemv (two launches)."""
        qblk = self.qblk
        if self.two_step:
            qblk.qblk_quantize_act(self.x[g], out=self.xq[g])
            qblk.qblk_gemv(qblk.Q4_K, packed[g], n, k, self.xq[g], self.batch, y=self.y[g])
        else:
            qblk.qblk_gemv_f32(qblk.Q4_K, packed[g], n, k, self.x[g], y=self.y[g],
                               work=self.work[g])

    def token(self, layers=None):
        """One decode token: per layer, the four group products."""
        for packed in self.layers if layers is None else layers:
            for g, _, n, k in self.groups:
                self.gemv(g, n, k, packed)

    def capture(self, layers=None):
        torch = self.torch
        self.token(layers=layers)
        torch.cuda.synchronize()
        eager = {g: y.clone() for g, y in self.y.items()}
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.token(layers=layers)
        graph.replay()
        torch.cuda.synchronize()
        for g, y in self.y.items():
            if not torch.equal(y, eager[g]):
                raise RuntimeError(f"graph replay differs from the eager run ({g})")
        return graph

    def fallbacks(self):
        """Handoff fallbacks counted in this model's workspaces (zeroed when
        they were allocated)."""
        return sum(self.qblk.handoff_fallbacks(self.work[g], self.batch, k)
                   for g, _, _, k in self.groups)

    def kernel_times(self, layers):
        """Per-launch GEMV time: for each group, one HIP graph of its product
        over `layers` layers back to back, bracketed by HIP events on the
        launch stream; time / launches is the kernel's boundary-to-boundary
        duration, as a kernel trace reports it (two-step: the GEMV alone, the
        activation quantized once before). Returns (algorithmic bytes,
        seconds, per-group table)."""
        torch, qblk = self.torch, self.qblk
        per, tot_b, tot_s = {}, 0, 0.0
        for g, _, n, k in self.groups:
            if self.two_step:
                qblk.qblk_quantize_act(self.x[g], out=self.xq[g])

            def launches():
                for packed in layers:
                    if self.two_step:
                        qblk.qblk_gemv(qblk.Q4_K, packed[g], n, k, self.xq[g], self.batch,
                                       y=self.y[g])
                    else:
                        self.gemv(g, n, k, packed)
            launches()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                launches()
            sec = time_replays(torch, [graph], 3, 1) * 1e-3
            del graph
            alg = alg_bytes(qblk, n, k, self.batch, not self.two_step) * len(layers)
            per[g] = {"n": n, "k": k, "us": round(1e6 * sec / len(layers), 3),
                      "alg_bytes": alg // len(layers),
                      "GBps": round(alg / sec / 1e9, 1)}
            tot_b += alg
            tot_s += sec
        return tot_b, tot_s, per


def alg_bytes(qblk, n, k, batch, fused):
    """Algorithmic bytes of one product launch: packed weights, the
    activation as the launch reads it (fp32 when the quantization is fused,
    else the quantized buffer) and the fp32 output."""
    act = 4 * k * batch if fused else qblk.qblk_act_bytes(batch, k)
    return qblk.qblk_weight_bytes(qblk.Q4_K, n, k) + act + 4 * n * batch


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the product "
                                   "shards by weight rows across GPUs (see the design notes)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    # the parallel oracle run starts its worker processes before anything in
    # this process touches the GPU
    cpu_par = None
    if not args.no_cpu_baseline and not args.traffic_probe:
        cpu_par = cpu_baseline_parallel(args.cpu_seconds, args.oracle_workers)
    import torch
    from block_quantized_qblk_amd import qblk, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.traffic_probe:
        traffic_probe(torch, qblk, synth, dev)
        return
    if args.batch4_probe:
        batch4_probe(torch, qblk, synth, dev)
        return

    # ------------------------------------------------------------ 70B decode, batch 1 and 4
    t0 = time.time()
    log(f"packing {args.layers} 70B-shaped Q4_K layers (Student-t weights)")
    m1 = DecodeModel(torch, qblk, synth, synth.LAYER_70B, args.layers, 5000, "student_t", 1, dev)
    log(f"packed {m1.weight_bytes / 1e9:.2f} GB in {time.time() - t0:.1f}s")
    g1 = m1.capture()
    with ClockSampler(dev_index=0) as clocks:
        ms_tok = time_replays(torch, [g1], args.steps, args.warmup)
    value = m1.weight_bytes / (ms_tok * 1e-3) / 1e9
    log(f"batch 1: {ms_tok:.3f} ms/token, {value:.1f} GB/s ({100 * value / HBM_PEAK_GBS:.1f}% "
        f"of HBM peak)")
    pct_tok = replay_percentiles(torch, g1, max(20, args.steps))
    log(f"batch 1, single tokens: {pct_tok}")
    del g1
    tot_b, tot_s, per_group = m1.kernel_times(m1.layers)
    all_gemv = tot_b / tot_s / 1e9
    # the dominant kernel streams gate_up (55% of the weight bytes)
    dom = [per_group[g] for g in DOMINANT_GROUPS]
    dom_bytes = sum(p["alg_bytes"] for p in dom)
    dom_sec = sum(p["us"] for p in dom) * 1e-6
    achieved = dom_bytes / dom_sec / 1e9
    log(f"gemv kernels (graphs of back-to-back launches): all {all_gemv:.1f} GB/s, "
        f"{DOMINANT_KERNEL} {achieved:.1f} GB/s; {per_group}")

    # the same token with the activation quantized by its own launch
    m1.two_step = True
    g2 = m1.capture()
    ms_two = time_replays(torch, [g2], max(5, args.steps // 3), 1)
    del g2
    _, _, per_two = m1.kernel_times(m1.layers)
    log(f"batch 1, quantize + GEMV launches: {ms_two:.3f} ms/token; GEMV alone {per_two}")
    m1.two_step = False

    fallbacks = m1.fallbacks()
    m1.set_batch(4, 5950)
    g4 = m1.capture()
    ms_tok4 = time_replays(torch, [g4], max(5, args.steps // 3), 1)
    fallbacks += m1.fallbacks()
    log(f"handoff fallbacks over every fused launch: {fallbacks}")
    log(f"batch 4: {ms_tok4:.3f} ms/step, {m1.weight_bytes / (ms_tok4 * 1e-3) / 1e9:.1f} GB/s")
    del g4, m1
    torch.cuda.empty_cache()

    secondary = {}
    if not args.no_secondary:
        secondary["layer_7b"] = layer_7b(torch, qblk, synth, dev, args)
        secondary["tp8_share"] = tp8_share(torch, qblk, synth, dev, args)
        secondary["gemm"] = gemm_bench(torch, qblk, synth, dev, args.gemm_iters)
        secondary["q4_0_q8_0"] = sym_bench(torch, qblk, synth, dev)
        secondary["kv_scores"] = kv_bench(torch, qblk, synth, dev)
        secondary["multi_qkv"] = multi_bench(torch, qblk, synth, dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(synth, args.cpu_seconds)
        if cpu_par is not None:
            single = dict(cpu)
            single.pop("host_cores", None)
            cpu = dict(cpu_par, single_process=single)

    out = {
        "metric": "Q4_K GEMV effective weight GB/s (% HBM peak); prefill GEMM int8 TOPS",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_tok, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "q4_k_gemv_70b_decode_80_layers",
            "layers": args.layers,
            "batch": 1,
            "weight_bytes_per_step": m_bytes(qblk, synth, args.layers),
            "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
            "tokens_per_s": round(1e3 / ms_tok, 2),
            "ms_per_token_single_replays": pct_tok,
            "batch4_ms_per_step": round(ms_tok4, 6),
            "batch4_GBps": round(m_bytes(qblk, synth, args.layers) / (ms_tok4 * 1e-3) / 1e9, 2),
            "launches_per_token": 4 * args.layers,
            "activation_quantization": "fused into each GEMV launch (qblk_gemv_f32)",
            "two_step_ms_per_step": round(ms_two, 6),
            "two_step_GBps": round(m_bytes(qblk, synth, args.layers) / (ms_two * 1e-3) / 1e9, 2),
            "two_step_gemv_per_launch": per_two,
            "handoff_fallbacks": fallbacks,
            "engine_clock_mhz": clocks.summary(),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": DOMINANT_KERNEL,
            "launches": "gate_up 57344x8192 of every layer",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_profile(GEMV_TRAFFIC, GEMV_SOURCES),
            "alg_bytes_per_launch": dom_bytes // len(dom),
            "all_gemv_GBps": round(all_gemv, 1),
            "per_launch": per_group,
        },
        "secondary": secondary,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------- HBM traffic

ROOT = os.path.dirname(os.path.abspath(__file__))
DOMINANT_KERNEL = "gemv_kernel<3, 1, 4, 1, true, true, 4>"  # <Q4_K, batch, rows/wave, chunks, in-launch quantization, activations in LDS, waves/workgroup>
DOMINANT_GROUPS = ("gate_up",)
GEMV_TRAFFIC = os.path.join(ROOT, "profiles", "gemv_q4k_70b_decode_traffic.md")
GEMV_SOURCES = ["block_quantized_qblk_amd/csrc/gemv.hip",
                "block_quantized_qblk_amd/csrc/gemv_select.cpp",
                "block_quantized_qblk_amd/csrc/qblk_device.h",
                "block_quantized_qblk_amd/csrc/qblk_internal.h"]
GEMM_TRAFFIC = os.path.join(ROOT, "profiles", "gemm_q4k_512x14336x4096.md")
GEMM_SOURCES = ["block_quantized_qblk_amd/csrc/gemm.hip",
                "block_quantized_qblk_amd/csrc/qblk_device.h",
                "block_quantized_qblk_amd/csrc/qblk_internal.h"]


def sources_sha256(sources):
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_from_profile(path, sources):
    """Measured HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated on a
    device copy) from a committed counter summary, or None when the summary is
    missing or was taken on different kernel sources."""
    try:
        text = open(path).read()
    except OSError:
        return None
    import re
    m = re.search(r"<!-- traffic (\{.*?\}) -->", text)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("sources_sha256") != sources_sha256(sources):
        return None
    return rec["hbm_bytes_per_launch"]


def traffic_probe(torch, qblk, synth, dev):
    """For rocprofv3 --pmc runs: a 1 GiB device copy (calibration), one decode
    token of four 70B-shaped layers at batch 1 (per layer: qkv, o, gate_up,
    down), then one Q4_K GEMM of 512 x 14336 x 4096 and one of 64 x 14336 x
    4096. Prints the algorithmic bytes of every GEMV launch and of the 512-row
    GEMM, in launch order."""
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).normal_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    m = DecodeModel(torch, qblk, synth, synth.LAYER_70B, 4, 5000, "student_t", 1, dev)
    m.token()
    torch.cuda.synchronize()
    gemv = [{"group": g, "n": n, "k": k, "alg_bytes": alg_bytes(qblk, n, k, 1, True)}
            for _ in range(4) for g, _, n, k in m.groups]
    del m
    n, k, mm = 14336, 4096, 512
    w = synth.torch_weights("outliers", 4000, n, k, device=dev)
    wq = qblk.qblk_pack_weights(qblk.Q4_K, w)
    xq = qblk.qblk_quantize_act(synth.torch_activations(4099, mm, k, device=dev))
    y = torch.empty((mm, n), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    qblk.qblk_gemm(qblk.Q4_K, wq, n, k, xq, mm, y=y)
    torch.cuda.synchronize()
    gemm = {"m": mm, "n": n, "k": k, "alg_bytes": qblk.qblk_weight_bytes(qblk.Q4_K, n, k)
            + qblk.qblk_act_bytes(mm, k) + 4 * mm * n}
    # the few-rows form on the same weights (m = 64)
    ms = 64
    xs = qblk.qblk_quantize_act(synth.torch_activations(4098, ms, k, device=dev))
    qblk.qblk_gemm(qblk.Q4_K, wq, n, k, xs, ms, y=y[:ms])
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": 1 << 30, "gemv_launches": gemv,
                      "gemm_launch": gemm,
                      "gemv_sources_sha256": sources_sha256(GEMV_SOURCES),
                      "gemm_sources_sha256": sources_sha256(GEMM_SOURCES)}))


def batch4_probe(torch, qblk, synth, dev):
    """For rocprofv3 --pmc runs: a 1 GiB device copy (calibration), then one
    decode token of four 70B-shaped layers at batch 4 (per layer: qkv, o,
    gate_up, down on the matrix-core kernels). Prints the algorithmic bytes
    of every GEMV launch, in launch order."""
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).normal_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    m = DecodeModel(torch, qblk, synth, synth.LAYER_70B, 4, 5000, "student_t", 4, dev)
    m.token()
    torch.cuda.synchronize()
    gemv = [{"group": g, "n": n, "k": k, "kernel": qblk.qblk_gemv_variant(qblk.Q4_K, n, k, 4, True),
             "alg_bytes": alg_bytes(qblk, n, k, 4, True)}
            for _ in range(4) for g, _, n, k in m.groups]
    print(json.dumps({"copy_bytes_each_way": 1 << 30, "gemv_launches": gemv,
                      "gemv_sources_sha256": sources_sha256(GEMV_SOURCES)}))


def gemv_launches(synth):
    """(type, n, k, batch, fused) of every GEMV product this benchmark times
    (fused: qblk_gemv_f32; else qblk_gemv on a quantized activation). The
    kernel instance each one runs must be run by a parity case too."""
    Q4_0, Q8_0, Q4_K = 1, 2, 3
    out = set()
    for shapes, batches in ((synth.LAYER_70B, (1, 4)), (synth.LAYER_7B, (1,)), (synth.LAYER_70B_TP8, (1,))):
        dims = {name: (n, k) for name, n, k in shapes}
        groups = [(dims["q"][0] + dims["k"][0] + dims["v"][0], dims["q"][1]), dims["o"],
                  (dims["gate"][0] + dims["up"][0], dims["gate"][1]), dims["down"]]
        for n, k in groups:
            for b in batches:
                out.add((Q4_K, n, k, b, True))
            if shapes is synth.LAYER_70B:
                out.add((Q4_K, n, k, 1, False))       # the two-step token
    for m in (1, 8, 64):                                # decode/prefill crossover
        out.add((Q4_K, 14336, 4096, m, False))
    out.add((Q4_0, 4096, 4096, 1, False))
    out.add((Q8_0, 14336, 4096, 1, False))
    out.add((Q4_K, 10240, 8192, 1, False))            # q/k/v concatenated, one launch
    return sorted(out)


def m_bytes(qblk, synth, layers):
    return layers * sum(qblk.qblk_weight_bytes(qblk.Q4_K, n, k) for _, n, k in synth.LAYER_70B)


def layer_7b(torch, qblk, synth, dev, args):
    """One 7B-shaped layer, batch 1, weights rotated over `copies` distinct
    packed copies (> 2 x the 256 MB last-level cache)."""
    models = [DecodeModel(torch, qblk, synth, synth.LAYER_7B, 1, 3000 + 100 * c, "outliers", 1, dev)
              for c in range(args.copies)]
    graphs = [m.capture() for m in models]
    ms = time_replays(torch, graphs, 200, 20)
    wb = models[0].weight_bytes
    tot_b, tot_s, per = models[0].kernel_times([m.layers[0] for m in models])
    res = {"workload": "q4_k_gemv_7b_layer", "us_per_layer": round(ms * 1e3, 3),
           "GBps": round(wb / (ms * 1e-3) / 1e9, 1), "weight_bytes": wb,
           "kernel_GBps": round(tot_b / tot_s / 1e9, 1), "per_launch": per,
           "rotating_copies": args.copies}
    log(f"7B layer: {res}")
    del graphs, models
    torch.cuda.empty_cache()
    return res


def tp8_share(torch, qblk, synth, dev, args):
    """One GPU's share of the 70B-shaped decode token split over 8 GPUs
    (q/k/v and gate/up by output rows, o and down along K): 80 layers of the
    shard's own shapes at batch 1, the token as one HIP graph. The
    collectives the split needs (two all-reduces of 8192 values per layer)
    are not part of it."""
    m = DecodeModel(torch, qblk, synth, synth.LAYER_70B_TP8, args.layers, 7000, "student_t", 1, dev)
    g = m.capture()
    ms = time_replays(torch, [g], max(10, args.steps // 2), 3)
    del g
    tot_b, tot_s, per = m.kernel_times(m.layers)
    res = {"workload": "q4_k_gemv_70b_decode_tp8_share", "layers": args.layers,
           "ms_per_token": round(ms, 4), "GBps": round(m.weight_bytes / (ms * 1e-3) / 1e9, 1),
           "weight_bytes_per_token": m.weight_bytes, "kernel_GBps": round(tot_b / tot_s / 1e9, 1),
           "per_launch": per, "handoff_fallbacks": m.fallbacks()}
    log(f"TP=8 share: {res}")
    del m
    torch.cuda.empty_cache()
    return res


def graph_launches(torch, fn, launches=64, reps=5, warm_s=0.0):
    """Mean per-launch time (us) of fn(0..launches-1) captured back to back
    in one HIP graph and replayed `reps` times between two events on the
    launch stream: the boundary-to-boundary duration a kernel trace reports,
    without per-launch event packets. The timed replays follow about
    `warm_s` seconds of untimed ones (at least one): on MI355X a
    compute-bound kernel runs about 20% slower during its first ~30 ms of
    sustained load, as the engine clock settles."""
    for i in range(3):
        fn(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(launches):
            fn(i)
    warm = 1
    if warm_s > 0:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        warm = max(1, int(warm_s / (a.elapsed_time(b) * 1e-3)))
    ms = time_replays(torch, [graph], reps, warm)
    del graph
    return 1e3 * ms / launches


def gemm_bench(torch, qblk, synth, dev, iters, copies=16):
    """Q4_K prefill GEMM 512 x 14336 x 4096, and M in {1, 8, 64} against the
    GEMV on the same weights; launches rotate over `copies` packed weight
    copies (16 x 33 MB, twice the 256 MB last-level cache)."""
    Q4_K = qblk.Q4_K
    n, k = 14336, 4096
    wqs = []
    for c in range(copies):
        w = synth.torch_weights("outliers", 4000 + c, n, k, device=dev)
        wqs.append(qblk.qblk_pack_weights(Q4_K, w))
        del w
    res = {}
    gemm_clock = None
    for m in (512, 1, 8, 64):
        x = synth.torch_activations(4099, m, k, device=dev)
        xq = qblk.qblk_quantize_act(x)
        y = torch.empty((m, n), dtype=torch.float32, device=dev)
        row = {}
        fns = [("gemm", qblk.qblk_gemm)]
        if m <= 64:
            fns.append(("gemv", qblk.qblk_gemv))
        for fname, f in fns:
            with ClockSampler(dev_index=0) as clk:
                us = graph_launches(torch, lambda i: f(Q4_K, wqs[i % copies], n, k, xq, m, y=y),
                                    launches=iters, warm_s=0.1)
            if m == 512:
                gemm_clock = clk.summary()
            ops = 2.0 * m * n * k
            row[fname] = {"us": round(us, 3), "TOPS": round(ops / (us * 1e-6) / 1e12, 2),
                          "weight_GBps": round(qblk.qblk_weight_bytes(Q4_K, n, k)
                                               / (us * 1e-6) / 1e9, 1)}
        res[f"m{m}"] = row
        log(f"gemm m={m}: {row}")
    del wqs
    torch.cuda.empty_cache()
    g = res["m512"]["gemm"]
    return {
        "workload": "q4_k_gemm_512x14336x4096",
        "TOPS": g["TOPS"],
        "us": g["us"],
        "engine_clock_mhz": gemm_clock,
        "roofline": {"bound": "mfma", "kernel": "gemm_kernel<3>", "achieved": g["TOPS"],
                     "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                     "frac": round(g["TOPS"] / INT8_PEAK_TOPS, 4),
                     "traffic": traffic_from_profile(GEMM_TRAFFIC, GEMM_SOURCES),
                     # the exact Q4_K scale step is two fp32 FMAs per (m, n, block):
                     # at the non-packed fp32 rate that bounds the kernel first
                     "valu_ceiling": valu_ceiling(512, 14336, 4096, g["us"])},
        "crossover": res,
    }


FP32_FMA_PER_S = 256 * 4 * 16 * 2.4e9   # non-packed fp32 FMAs per second: CUs x SIMDs x lanes per cycle x clock


def valu_ceiling(m, n, k, us):
    """The time two fp32 FMAs per (m, n, 32-block) take at the chip's
    non-packed fp32 FMA rate (the Q4_K GEMM's scale step), and the kernel's
    fraction of it."""
    t = 2 * m * n * (k // 32) / FP32_FMA_PER_S * 1e6
    return {"fma_per_block_output": 2, "us": round(t, 2), "frac": round(t / us, 4)}


def sym_bench(torch, qblk, synth, dev):
    """Q4_0 4096 x 4096 and Q8_0 14336 x 4096 GEMVs, batch 1, rotated over
    enough copies to exceed the last-level cache; beside each, the same
    weights against the fp32 activation (qblk_gemv_float, no activation
    quantization)."""
    res = {}
    for name, t, n, k in (("q4_0_gemv_4096x4096", qblk.Q4_0, 4096, 4096),
                          ("q8_0_gemv_14336x4096", qblk.Q8_0, 14336, 4096)):
        wb = qblk.qblk_weight_bytes(t, n, k)
        copies = max(2, int(600e6 // wb) + 1)
        wqs = []
        for c in range(copies):
            w = synth.torch_weights("normal", 1000 * t + c, n, k, device=dev)
            wqs.append(qblk.qblk_pack_weights(t, w))
            del w
        x = synth.torch_activations(1000 * t + 99, 1, k, device=dev)
        xq = qblk.qblk_quantize_act(x)
        y = torch.empty((1, n), dtype=torch.float32, device=dev)
        us = graph_launches(torch, lambda i: qblk.qblk_gemv(t, wqs[i % copies], n, k, xq, 1, y=y))
        res[name] = {"us": round(us, 3), "weight_bytes": wb, "GBps": round(wb / (us * 1e-6) / 1e9, 1)}
        log(f"{name}: {res[name]}")
        fname = name.replace("_gemv_", "_gemv_float_")
        us = graph_launches(torch, lambda i: qblk.qblk_gemv_float(t, wqs[i % copies], n, k, x, y=y))
        res[fname] = {"us": round(us, 3), "weight_bytes": wb, "GBps": round(wb / (us * 1e-6) / 1e9, 1)}
        log(f"{fname}: {res[fname]}")
        del wqs
        torch.cuda.empty_cache()
    return res


def multi_bench(torch, qblk, synth, dev):
    """70B-shaped q, k, v projections (8192, 1024, 1024 rows of 8192) on one
    quantized activation: three qblk_gemv launches, one qblk_gemv_multi
    launch over the three matrices, and one qblk_gemv over the same rows
    packed as one 10240-row matrix; rotated over enough layers' weights to
    exceed the last-level cache."""
    k = 8192
    ns = (8192, 1024, 1024)
    wb = sum(qblk.qblk_weight_bytes(qblk.Q4_K, n, k) for n in ns)
    copies = max(2, int(600e6 // wb) + 1)
    layers = []
    for c in range(copies):
        w = synth.torch_weights("student_t", 8100 + c, sum(ns), k, device=dev)
        cat = qblk.qblk_pack_weights(qblk.Q4_K, w)
        rb = qblk.qblk_weight_row_bytes(qblk.Q4_K, k)
        parts, r0 = [], 0
        for n in ns:
            parts.append(cat[r0 * rb:(r0 + n) * rb])
            r0 += n
        layers.append((cat, parts))
        del w
    xq = qblk.qblk_quantize_act(synth.torch_activations(8199, 1, k, device=dev))
    ys = [torch.empty((1, n), dtype=torch.float32, device=dev) for n in ns]
    ycat = torch.empty((1, sum(ns)), dtype=torch.float32, device=dev)

    def separate(i):
        for part, n, y in zip(layers[i % copies][1], ns, ys):
            qblk.qblk_gemv(qblk.Q4_K, part, n, k, xq, 1, y=y)

    def multi(i):
        qblk.qblk_gemv_multi(qblk.Q4_K, [(part, n, k, xq, y) for part, n, y in zip(layers[i % copies][1], ns, ys)],
                             1)

    def concat(i):
        qblk.qblk_gemv(qblk.Q4_K, layers[i % copies][0], sum(ns), k, xq, 1, y=ycat)

    res = {"weight_bytes": wb}
    for name, fn in (("three_launches", separate), ("multi_launch", multi), ("concatenated", concat)):
        us = graph_launches(torch, fn, launches=32)
        res[name] = {"us": round(us, 3), "GBps": round(wb / (us * 1e-6) / 1e9, 1)}
    log(f"q/k/v as three matrices: {res}")
    del layers
    torch.cuda.empty_cache()
    return res


def kv_bench(torch, qblk, synth, dev):
    """Scores of one decode step against a quantized K cache: 70B-shaped
    (64 query heads over 8 KV heads of 128, 8192 cached tokens) and the
    7B example of the KV-cache size formula (32 heads of 128, 2048 tokens),
    one launch per layer, rotated over enough layers' caches to exceed the
    last-level cache."""
    res = {}
    for name, t, n_kv, n_head, n_ctx in (("q8_0_70b_ctx8192", qblk.Q8_0, 8, 64, 8192),
                                         ("q4_0_70b_ctx8192", qblk.Q4_0, 8, 64, 8192),
                                         ("q8_0_7b_ctx2048", qblk.Q8_0, 32, 32, 2048)):
        hd = 128
        cb = qblk.qblk_kv_cache_bytes(t, n_kv, n_ctx, hd)
        copies = max(2, int(600e6 // cb) + 1)
        caches = []
        for c in range(copies):
            cache = qblk.qblk_kv_cache(t, n_kv, n_ctx, hd, device=dev)
            k = synth.torch_activations(7000 + c, n_kv * n_ctx, hd, device=dev)
            qblk.qblk_pack_weights(t, k, out=cache)  # rows (h, t) in order
            caches.append(cache)
            del k
        qq = qblk.qblk_quantize_act(synth.torch_activations(7999, n_head, hd, device=dev))
        s = torch.empty((n_head, n_ctx), dtype=torch.float32, device=dev)
        us = graph_launches(torch, lambda i: qblk.qblk_kv_scores(t, caches[i % copies], n_kv, n_ctx, n_ctx, hd,
                                                                  qq, n_head, scores=s))
        alg = cb + qblk.qblk_act_bytes(n_head, hd) + 4 * n_head * n_ctx
        res[name] = {"us": round(us, 3), "cache_bytes": cb, "alg_bytes": alg,
                     "cache_GBps": round(cb / (us * 1e-6) / 1e9, 1),
                     "GBps": round(alg / (us * 1e-6) / 1e9, 1)}
        log(f"kv scores {name}: {res[name]}")
        del caches
        torch.cuda.empty_cache()
    return res


def cpu_baseline(synth, seconds):
    """The oracle (NumPy: int64 block sums, fp64 scaling) on the host cores,
    over a bounded sample of the headline workload: the first 32 rows of each
    of the seven 70B-shaped Q4_K linears (encoded untimed), then activation
    quantization plus the product timed, repeated until `seconds` elapse."""
    o, samples, rows = _oracle_samples(synth)
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
            "sample": f"first {rows} rows of each of the 7 Q4_K linears of a 70B-shaped layer, "
                      f"batch 1, {reps} passes in {el:.1f}s (activation quantization + int64 "
                      f"block sums + fp64 scaling; weight encoding untimed); NumPy's int64 "
                      f"einsum runs on one thread",
            "host_cores": len(os.sched_getaffinity(0))}


def _oracle_samples(synth):
    """The first 32 rows of each of the seven 70B-shaped Q4_K linears, encoded
    by the oracle, with one activation row each."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from oracle import qblk_oracle as o
    rows = 32
    samples = []
    for idx, (name, n, k) in enumerate(synth.LAYER_70B):
        w = synth.weights_student_t(5900 + idx, rows, k)
        _, enc = o.encode_weights(o.TYPE_Q4_K, w)
        x = synth.activations(5999 - idx, 1, k)
        samples.append((enc, x, o.row_bytes(o.TYPE_Q4_K, k) * rows))
    return o, samples, rows


def _oracle_worker(barrier, results, seconds):
    from block_quantized_qblk_amd import synth
    o, samples, _ = _oracle_samples(synth)
    barrier.wait()
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for enc, x, nbytes in samples:
            o.product(o.TYPE_Q4_K, enc, o.quantize_act(x))
            done += nbytes
    results.put((done, time.perf_counter() - t0))


def cpu_baseline_parallel(seconds, workers):
    """The oracle on every host core at once: `workers` single-threaded
    processes, each running the cpu_baseline sample loop for `seconds` after a
    common start barrier; throughput is their total bytes over the mean
    elapsed time."""
    import multiprocessing as mp
    cores = len(os.sched_getaffinity(0))
    w = workers if workers > 0 else min(16, cores)
    # under a profiler (rocprofv3 preloads its tool into every child) the
    # workers would each carry the tool; leave the parallel run out there
    profiled = any(k.startswith("ROCPROF") for k in os.environ) or "rocprof" in os.environ.get("LD_PRELOAD", "")
    if w <= 1 or profiled:
        return None
    env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in env:
        os.environ[k] = "1"
    try:
        ctx = mp.get_context("spawn")
        barrier, results = ctx.Barrier(w), ctx.Queue()
        procs = [ctx.Process(target=_oracle_worker, args=(barrier, results, seconds)) for _ in range(w)]
        for p in procs:
            p.start()
        got = [results.get(timeout=seconds + 300) for _ in range(w)]
        for p in procs:
            p.join(timeout=60)
    finally:
        for k, v in env.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    total = sum(b for b, _ in got)
    el = sum(e for _, e in got) / len(got)
    gbs = total / el / 1e9
    log(f"cpu oracle, {w} processes: {gbs:.4f} GB/s over {el:.1f}s")
    return {"value": round(gbs, 5), "unit": "GB/s", "cores": w, "kind": "oracle",
            "sample": f"{w} single-threaded processes, each repeating the single-process sample "
                      f"(first 32 rows of each of the 7 Q4_K linears of a 70B-shaped layer, batch 1: "
                      f"activation quantization + int64 block sums + fp64 scaling) for {el:.1f}s "
                      f"after a common start",
            "host_cores": cores}


if __name__ == "__main__":
    main()
