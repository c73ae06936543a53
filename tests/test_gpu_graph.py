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
