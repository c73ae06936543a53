"""The entry points captured in a HIP graph (through torch's graph capture):
every replay, with eager work and synchronizations in between, must equal
the eager result bit for bit."""

import numpy as np
import pytest

from block_quantized_qblk_amd import qblk, synth
from oracle import qblk_oracle as o
from tests.gpu_util import check_rel, dev, expected, host, torch

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    print("graph capture: quantize + gemv + gemm", flush=True)
    t = torch()
    n, k, m = 700, 2048, 3
    w = synth.weights(3, 5, n, k)
    x = synth.act(3, m, k)
    wq = qblk.qblk_pack_weights(qblk.Q4_K, dev(w))
    xd = dev(x)
    xq = t.empty(qblk.qblk_act_bytes(m, k), dtype=t.uint8, device="cuda")
    y1 = t.empty((m, n), dtype=t.float32, device="cuda")
    y2 = t.empty((m, n), dtype=t.float32, device="cuda")

    def work():
        qblk.qblk_quantize_act(xd, out=xq)
        qblk.qblk_gemv(qblk.Q4_K, wq, n, k, xq, m, y=y1)
        qblk.qblk_gemm(qblk.Q4_K, wq, n, k, xq, m, y=y2)

    work()
    t.cuda.synchronize()
    ref1, ref2, refq = y1.clone(), y2.clone(), xq.clone()
    check_rel(host(ref1), expected(o.TYPE_Q4_K, w, x))
    check_rel(host(ref2), expected(o.TYPE_Q4_K, w, x))

    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        work()
    other = synth.act(3, m, k, index=98)
    for rep in range(4):
        # eager work in between that overwrites the same buffers
        y1.fill_(float("nan"))
        y2.zero_()
        xq.zero_()
        qblk.qblk_quantize_act(dev(other), out=xq)
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        assert t.equal(xq, refq), rep
        assert t.equal(y1, ref1), rep
        assert t.equal(y2, ref2), rep


def test_graph_replays_fused_gemv_in_launch_quantization():
    """qblk_gemv_f32 on a matrix that takes the in-launch quantization path,
    captured once: each replay reads the activation that is in x at replay
    time (new values are written between replays), and must equal quantize +
    GEMV run eagerly on those values."""
    print("graph capture: gemv_f32 with in-launch quantization", flush=True)
    t = torch()
    n, k = 17000, 4096
    w = synth.weights(3, 6, n, k)
    wq = qblk.qblk_pack_weights(qblk.Q4_K, dev(w))
    x = dev(synth.act(3, 1, k))
    y = t.empty((1, n), dtype=t.float32, device="cuda")
    work = t.zeros(qblk.qblk_gemv_f32_work_bytes(1, k), dtype=t.uint8, device="cuda")
    qblk.qblk_gemv_f32(qblk.Q4_K, wq, n, k, x, y=y, work=work)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        qblk.qblk_gemv_f32(qblk.Q4_K, wq, n, k, x, y=y, work=work)
    for rep in range(5):
        x.copy_(dev(synth.act(3, 1, k, index=90 - rep)))
        y.fill_(float("nan"))
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        ref = qblk.qblk_gemv(qblk.Q4_K, wq, n, k, qblk.qblk_quantize_act(x), 1)
        t.cuda.synchronize()
        assert t.equal(y, ref), rep


def test_graph_replays_other_entry_points():
    """The large-tile GEMM (more than 256 rows), the float-activation GEMV, the
    descriptor-list GEMV and the KV cache store + scores, captured in one
    graph: every replay, after eager work that overwrites the outputs and the
    cache, must equal the eager result bit for bit."""
    print("graph capture: gemm m>256, gemv_float, gemv_multi, kv_store + kv_scores", flush=True)
    t = torch()
    n, k, m = 300, 1024, 290
    w = synth.weights(3, 7, n, k)
    wq = qblk.qblk_pack_weights(qblk.Q4_K, dev(w))
    w8 = synth.weights(2, 8, 200, k)
    wq8 = qblk.qblk_pack_weights(qblk.Q8_0, dev(w8))
    x = synth.act(3, m, k)
    xq = qblk.qblk_quantize_act(dev(x))
    xf = dev(synth.act(3, 2, k, index=5))
    xq1 = qblk.qblk_quantize_act(xf)
    n_kv, n_head, hd, n_ctx = 2, 8, 128, 96
    kv_new = dev(synth.act(3, n_kv, hd, index=6))
    cache = qblk.qblk_kv_cache(qblk.Q8_0, n_kv, n_ctx, hd)
    for pos in range(n_ctx - 1):
        qblk.qblk_kv_store(qblk.Q8_0, dev(synth.act(3, n_kv, hd, index=100 + pos)), cache, n_ctx, pos)
    qq = qblk.qblk_quantize_act(dev(synth.act(3, n_head, hd, index=7)))
    y_gemm = t.empty((m, n), dtype=t.float32, device="cuda")
    y_float = t.empty((2, n), dtype=t.float32, device="cuda")
    y_a = t.empty((2, n), dtype=t.float32, device="cuda")
    y_b = t.empty((2, 200), dtype=t.float32, device="cuda")
    scores = t.empty((n_head, n_ctx), dtype=t.float32, device="cuda")

    def work():
        qblk.qblk_gemm(qblk.Q4_K, wq, n, k, xq, m, y=y_gemm)
        qblk.qblk_gemv_float(qblk.Q4_K, wq, n, k, xf, y=y_float)
        qblk.qblk_kv_store(qblk.Q8_0, kv_new, cache, n_ctx, n_ctx - 1)
        qblk.qblk_kv_scores(qblk.Q8_0, cache, n_kv, n_ctx, n_ctx, hd, qq, n_head, scores=scores)

    def work_multi():
        qblk.qblk_gemv_multi(qblk.Q4_K, [(wq, n, k, xq1, y_a)], 2)
        qblk.qblk_gemv_multi(qblk.Q8_0, [(wq8, 200, k, xq1, y_b)], 2)

    work()
    work_multi()
    t.cuda.synchronize()
    outs = (y_gemm, y_float, y_a, y_b, scores, cache)
    refs = [v.clone() for v in outs]
    check_rel(host(y_gemm), expected(o.TYPE_Q4_K, w, x))
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        work()
        work_multi()
    for rep in range(4):
        for v in outs[:5]:
            v.fill_(float("nan"))
        # overwrite the last cache row with another token's K
        qblk.qblk_kv_store(qblk.Q8_0, dev(synth.act(3, n_kv, hd, index=60 + rep)), cache, n_ctx, n_ctx - 1)
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        for i, (v, r) in enumerate(zip(outs, refs)):
            assert t.equal(v, r), (rep, i)
