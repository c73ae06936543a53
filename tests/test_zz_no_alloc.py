"""The allocation-free fused GEMV (qblk_gemv_f32_noalloc, the library's fixed
device array as workspace) against qblk_gemv_f32 with a caller workspace:
bitwise equal, on two calls in a row, the second with a smaller input (the
array keeps the first call's contents), and within the tolerance of the
oracle on sampled rows."""

import numpy as np
import pytest

from block_quantized_qblk_amd import qblk
from oracle import qblk_oracle as o
from tests.gpu_util import check_rel, dev, dev_pack, expected, host, torch

pytestmark = pytest.mark.gpu


def _pair(wtype, n, k, batch, seed):
    print(f"gemv_f32_noalloc type={wtype} n={n} k={k} batch={batch}", flush=True)
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    x = rng.standard_normal((batch, k)).astype(np.float32)
    wq = dev_pack(wtype, w)
    xd = dev(x)
    ref = host(qblk.qblk_gemv_f32(wtype, wq, n, k, xd))
    y = torch().full((batch, n), float("nan"), device="cuda")
    got = host(qblk.qblk_gemv_f32_noalloc(wtype, wq, n, k, xd, y))
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))
    rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(seed).choice(n, 24, replace=False)]))
    check_rel(got[:, rows], expected(wtype, w[rows], x))


@pytest.mark.parametrize("wtype", [o.TYPE_Q4_K, o.TYPE_Q8_0, o.TYPE_Q4_0])
def test_noalloc_matches_workspace_entry_point(wtype):
    # the in-launch handoff at batch 4 (8 rows per wave, activations in LDS),
    # then a smaller product (batch 1, shorter rows: other slice count and
    # flag stride over the same array)
    _pair(wtype, 16400, 8192, 4, 10 + wtype)
    _pair(wtype, 3000, 4096, 1, 20 + wtype)


def test_noalloc_small_and_largest_rows():
    # a small single-row product (activation quantized in every workgroup's
    # local memory, the array unused), then rows of the largest k accepted
    _pair(o.TYPE_Q4_K, 1000, 2048, 1, 31)
    _pair(o.TYPE_Q4_K, 40, 131072, 2, 32)
    _pair(o.TYPE_Q4_K, 700, 8192, 1, 33)


def test_noalloc_limits():
    t = torch()
    wq = t.zeros(qblk.qblk_weight_bytes(o.TYPE_Q4_K, 8, 131328), dtype=t.uint8, device="cuda")
    for k, batch in ((131328, 1), (131072, 8), (8192, 9)):
        x = t.zeros((batch, k), dtype=t.float32, device="cuda")
        y = t.zeros((batch, 8), dtype=t.float32, device="cuda")
        with pytest.raises(qblk.QblkError) as ei:
            qblk.qblk_gemv_f32_noalloc(o.TYPE_Q4_K, wq, 8, k, x, y)
        assert ei.value.status == -4


def test_noalloc_in_a_graph():
    """The callers this entry point is for include code under HIP graph
    capture: captured once, every replay reads the activation in x at replay
    time (new values are written between replays, with eager use of the same
    device array in between) and must equal qblk_gemv_f32 run eagerly on them."""
    print("gemv_f32_noalloc under graph capture", flush=True)
    t = torch()
    n, k, batch = 9000, 8192, 2
    rng = np.random.default_rng(41)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    wq = dev_pack(o.TYPE_Q4_K, w)
    x = t.empty((batch, k), dtype=t.float32, device="cuda")
    y = t.empty((batch, n), dtype=t.float32, device="cuda")
    x.copy_(dev(rng.standard_normal((batch, k)).astype(np.float32)))
    qblk.qblk_gemv_f32_noalloc(o.TYPE_Q4_K, wq, n, k, x, y)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        qblk.qblk_gemv_f32_noalloc(o.TYPE_Q4_K, wq, n, k, x, y)
    y_eager = t.empty_like(y)
    for rep in range(4):
        x.copy_(dev(rng.standard_normal((batch, k)).astype(np.float32)))
        # eager use of the same array with other shapes in between
        small = dev(rng.standard_normal((1, 4096)).astype(np.float32))
        qblk.qblk_gemv_f32_noalloc(o.TYPE_Q4_K, wq, n, 4096, small, t.empty((1, n), device="cuda"))
        ref = host(qblk.qblk_gemv_f32(o.TYPE_Q4_K, wq, n, k, x, y=y_eager))
        y.fill_(float("nan"))
        t.cuda.synchronize()
        g.replay()
        got = host(y)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), rep


def test_noalloc_rejects_non_fp32_tensors():
    print("gemv_f32_noalloc dtype checks", flush=True)
    t = torch()
    wq = t.zeros(qblk.qblk_weight_bytes(qblk.Q4_K, 64, 256), dtype=t.uint8, device="cuda")
    x = t.zeros((1, 256), dtype=t.float16, device="cuda")
    y = t.zeros((1, 64), dtype=t.float32, device="cuda")
    with pytest.raises(ValueError):
        qblk.qblk_gemv_f32_noalloc(qblk.Q4_K, wq, 64, 256, x, y)
    with pytest.raises(ValueError):
        qblk.qblk_gemv_f32_noalloc(qblk.Q4_K, wq, 64, 256, x.float(), y.half())
