"""qblk_gemv_f32 launches in flight on two streams at once, each stream with
its own workspace: the in-launch handoff's tags tell the launches apart
(they are built from the dispatch packet), so each result equals the one
computed alone, bit for bit, and no workgroup falls back from the handoff."""

import numpy as np
import pytest

from block_quantized_qblk_amd import qblk, synth
from tests.gpu_util import dev, host, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,k,batch", [(9000, 8192, 1), (16400, 4096, 4)])
def test_gemv_f32_on_two_streams(n, k, batch):
    print(f"gemv_f32 on two streams n={n} k={k} batch={batch}", flush=True)
    t = torch()
    ws, xs, works, ys, refs = [], [], [], [], []
    for i in range(2):
        w = synth.torch_weights("student_t", 6100 + i, n, k)
        ws.append(qblk.qblk_pack_weights(qblk.Q4_K, w))
        del w
        xs.append(dev(synth.act(5, batch, k, index=90 + i)))
        works.append(t.zeros(qblk.qblk_gemv_f32_work_bytes(batch, k), dtype=t.uint8, device="cuda"))
        ys.append(t.empty((batch, n), dtype=t.float32, device="cuda"))
    for i in range(2):   # each product alone, on the current stream
        qblk.qblk_gemv_f32(qblk.Q4_K, ws[i], n, k, xs[i], y=ys[i], work=works[i])
        t.cuda.synchronize()
        refs.append(host(ys[i]).copy())
    fallbacks0 = [qblk.handoff_fallbacks(works[i], batch, k) for i in range(2)]
    streams = [t.cuda.Stream(), t.cuda.Stream()]   # default priority
    t.cuda.synchronize()
    for rep in range(16):
        for i in range(2):
            with t.cuda.stream(streams[i]):
                qblk.qblk_gemv_f32(qblk.Q4_K, ws[i], n, k, xs[i], y=ys[i], work=works[i])
    t.cuda.synchronize()
    for i in range(2):
        got = host(ys[i])
        assert np.array_equal(got.view(np.uint32), refs[i].view(np.uint32)), i
        assert qblk.handoff_fallbacks(works[i], batch, k) == fallbacks0[i], i
