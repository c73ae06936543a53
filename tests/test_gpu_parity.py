"""GPU parity: every entry point, called through the C ABI, against the
oracle. Integer work (activation codes, packed bytes, block sums) must be
bit-exact; fp32 outputs within REL_TOL = 1e-5 (max-normalized)."""

import numpy as np
import pytest

from block_quantized_qblk_amd import qblk, synth
from oracle import qblk_oracle as o
from tests import gemv_cases as cases
from tests.gpu_util import (REL_TOL, check_rel, dev, dev_pack, dev_quantize, expected, host,
                            oracle_act, torch)

pytestmark = pytest.mark.gpu

TYPES = [o.TYPE_Q4_0, o.TYPE_Q8_0, o.TYPE_Q4_K, o.TYPE_Q4_0_F16]
TNAME = {1: "Q4_0", 2: "Q8_0", 3: "Q4_K", 4: "Q4_0_F16"}


def _special_rows(rng, n, k, std=0.02):
    """Seeded weights with zero, constant, single-non-zero and outlier blocks."""
    w = (rng.standard_normal((n, k)) * std).astype(np.float32)
    w[0, :32] = 0
    if k >= 64:
        w[0, 32:64] = 0.011
    if n > 1 and k >= 256:
        w[1, :256] = 0
        w[1, 7] = -0.3
    if n > 2:
        w[2] = np.abs(w[2])
    idx = rng.choice(n * k, size=max(1, n * k // 1000), replace=False)
    w.reshape(-1)[idx] = np.where(rng.random(idx.size) < 0.5, -0.2, 0.2)
    return w


# ================================================================ activation quantization

@pytest.mark.parametrize("m,k", [(1, 4096), (3, 1184), (7, 32), (512, 4096), (2, 14336)])
def test_quantize_act_bit_exact(m, k):
    print(f"quantize_act m={m} k={k}", flush=True)
    x = synth.activations(1000 + m, m, k)
    x[0, :32] = 0
    if k >= 64:
        x[-1, 32:64] = 3.0
    got = host(dev_quantize(x))
    ref = o.pack_act(*oracle_act(x))
    assert got.shape == ref.shape
    assert np.array_equal(got, ref)


def test_quantize_act_ties_and_denormals():
    print("quantize_act ties/denormals", flush=True)
    x = np.zeros((1, 128), dtype=np.float32)
    # block 0: d = 127/127 = 1, ties x.5 must round away from zero
    x[0, :8] = [127.0, 2.5, -2.5, 0.5, -0.5, 126.5, -3.5, 1.4999999]
    # block 1: tiny normal amax -> subnormal d
    x[0, 32:40] = np.float32(1e-38) * np.array([1, -0.5, 0.25, 0.75, -1, 0.1, 0, 0.3], np.float32)
    # block 2: subnormal inputs
    x[0, 64:70] = np.float32(1e-42) * np.array([1, 2, -3, 4, -5, 6], np.float32)
    # block 3: huge values
    x[0, 96:100] = [3e38, -1e38, 1e30, -3e38]
    got = host(dev_quantize(x))
    q, d, s = oracle_act(x)
    assert q[0, 1] == 3 and q[0, 2] == -3 and q[0, 3] == 1 and q[0, 4] == -1
    assert np.array_equal(got, o.pack_act(q, d, s))


def test_quantize_act_strided_rows():
    print("quantize_act strided", flush=True)
    big = synth.activations(7, 5, 640)
    xs = dev(big)[:, 64:64 + 512]
    got = host(qblk.qblk_quantize_act(xs))
    assert np.array_equal(got, o.pack_act(*oracle_act(big[:, 64:576])))


# ================================================================ weight packing

@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("n,k", [(37, 1024), (5, 256), (64, 4096), (3, 2304)])
def test_pack_weights_bit_exact(wtype, n, k):
    print(f"pack {TNAME[wtype]} n={n} k={k}", flush=True)
    rng = np.random.default_rng(50 * wtype + n)
    w = _special_rows(rng, n, k)
    got = host(dev_pack(wtype, w)).reshape(n, -1)
    ref, _ = o.encode_weights(wtype, w)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("wtype", [o.TYPE_Q4_0, o.TYPE_Q8_0, o.TYPE_Q4_0_F16])
def test_pack_weights_padded_header(wtype):
    """k = 416: 13 blocks, 52 header bytes padded to 64 (fp16 scales: 26
    padded to 32)."""
    print(f"pack padded {TNAME[wtype]}", flush=True)
    rng = np.random.default_rng(3)
    w = _special_rows(rng, 9, 416)
    buf = torch().full((qblk.qblk_weight_bytes(wtype, 9, 416),), 0xAB, dtype=torch().uint8,
                       device="cuda")
    qblk.qblk_pack_weights(wtype, dev(w), out=buf)
    ref, _ = o.encode_weights(wtype, w)
    assert np.array_equal(host(buf).reshape(9, -1), ref)


def test_pack_q4_0_f16_extreme_scales():
    """fp16 scales in the subnormal range, rounding to zero, and saturating
    at 65504, next to ordinary rows."""
    print("pack Q4_0_F16 extremes", flush=True)
    rng = np.random.default_rng(13)
    w = (rng.standard_normal((6, 256)) * 0.02).astype(np.float32)
    w[0] *= 1e-4                      # d in the fp16 subnormal range
    w[1] *= 1e-8                      # d rounds to zero: all codes 0
    w[2] *= 1e8                       # d saturates at 65504
    w[3, :32] = 0.0                   # zero block
    w[4, 5] = 7.0 * 0.25              # amax/7 exactly an fp16 value
    got = host(dev_pack(o.TYPE_Q4_0_F16, w)).reshape(6, -1)
    ref, _ = o.encode_weights(o.TYPE_Q4_0_F16, w)
    assert np.array_equal(got, ref)


def test_pack_q4_k_extreme_ranges():
    """Tiny, huge and single-signed super-blocks."""
    print("pack Q4_K extremes", flush=True)
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((6, 512)) * 0.02).astype(np.float32)
    w[0] *= 1e-6                      # d in the fp16 subnormal range
    w[1] *= 1e3                       # large scales
    w[2] = np.abs(w[2]) + 0.5         # all positive: no min term
    w[3] = -np.abs(w[3]) - 0.5        # all negative
    w[4, :256] = 0.0                  # zero super-block
    w[5, ::2] = 0.0
    got = host(dev_pack(o.TYPE_Q4_K, w)).reshape(6, -1)
    ref, enc = o.encode_weights(o.TYPE_Q4_K, w)
    assert np.array_equal(got, ref)


# ================================================================ block sums

@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("m,n,k", [(1, 1, 256), (3, 37, 512), (5, 7, 2304)])
def test_block_sums_bit_exact(wtype, m, n, k):
    print(f"block_sums {TNAME[wtype]} m={m} n={n} k={k}", flush=True)
    rng = np.random.default_rng(7 * wtype + m)
    w = _special_rows(rng, n, k)
    x = rng.standard_normal((m, k)).astype(np.float32)
    sums = qblk.qblk_block_sums(wtype, dev_pack(wtype, w), n, k, dev_quantize(x), m)
    _, enc = o.encode_weights(wtype, w)
    aq, _, _ = oracle_act(x)
    ref = o.block_sums(o.weight_codes_for_sums(wtype, enc), aq)
    assert np.array_equal(host(sums).astype(np.int64), ref)


# ================================================================ exact-arithmetic products

def _exact_case(wtype, n, k, m, seed):
    """Codes and power-of-two scales chosen so that every fp32 step of the
    product is exact: the device result must equal the oracle bit for bit,
    which pins the integer block sums inside the production kernels."""
    rng = np.random.default_rng(seed)
    nb = k // 32
    if wtype == o.TYPE_Q4_K:
        enc = dict(d_bits=np.full((n, k // 256), 0x1C00, np.uint16),       # 2^-8
                   dmin_bits=np.full((n, k // 256), 0x9800, np.uint16),    # -2^-9
                   sc=rng.integers(0, 8, (n, k // 256, 8)),
                   mn=rng.integers(0, 64, (n, k // 256, 8)),
                   q=rng.integers(0, 16, (n, k)))
        packed = o.pack_q4_k(enc)
    elif wtype == o.TYPE_Q4_0:
        enc = dict(q=rng.integers(-8, 8, (n, k)), d=np.full((n, nb), 2.0 ** -6, np.float32))
        packed = o.pack_q4_0(enc["q"], enc["d"])
    elif wtype == o.TYPE_Q4_0_F16:
        enc = dict(q=rng.integers(-8, 8, (n, k)), d=np.full((n, nb), 2.0 ** -6, np.float32))
        packed = o.pack_q4_0_f16(enc["q"], enc["d"])
    else:
        enc = dict(q=rng.integers(-12, 13, (n, k)), d=np.full((n, nb), 2.0 ** -7, np.float32))
        packed = o.pack_q8_0(enc["q"], enc["d"])
    a = rng.integers(-8, 9, (m, k))
    a[:, ::32] = 127 * np.where(rng.random((m, nb)) < 0.5, -1, 1)
    x = (a * 0.25).astype(np.float32)
    act = oracle_act(x)
    assert np.array_equal(act[0], a)
    y32, y64 = o.product(wtype, enc, act)
    assert np.array_equal(y32.astype(np.float64), y64)   # exact in fp32
    return packed, x, y32


@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("batch", cases.GEMV_EXACT_BATCH)
def test_gemv_exact_arithmetic(wtype, batch):
    print(f"gemv exact {TNAME[wtype]} batch={batch}", flush=True)
    n, k = 67, 2304 if wtype == o.TYPE_Q4_K else 2336
    packed, x, y32 = _exact_case(wtype, n, k, batch, 900 + wtype)
    y = qblk.qblk_gemv(wtype, dev(packed.reshape(-1)), n, k, dev_quantize(x), batch)
    assert np.array_equal(host(y), y32)


@pytest.mark.parametrize("n,k,batch", cases.GEMV_RING_EXACT)
def test_gemv_ring_exact_arithmetic(n, k, batch):
    """Q4_K's matrix-core GEMV (2-8 activation rows, k a multiple of 2048)
    with power-of-two scales: every partial sum is exact in fp32, so y must
    equal the oracle bit for bit whatever the summation order."""
    print(f"gemv ring exact n={n} k={k} batch={batch}", flush=True)
    assert qblk.qblk_gemv_variant(o.TYPE_Q4_K, n, k, batch, False).startswith("gemv_ring")
    packed, x, y32 = _exact_case(o.TYPE_Q4_K, n, k, batch, 950 + batch)
    y = qblk.qblk_gemv(o.TYPE_Q4_K, dev(packed.reshape(-1)), n, k, dev_quantize(x), batch)
    assert np.array_equal(host(y), y32)


@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("m", [1, 16, 37, 64, 130, 300])
def test_gemm_exact_arithmetic(wtype, m):
    print(f"gemm exact {TNAME[wtype]} m={m}", flush=True)
    n, k = 150, 1024 if wtype == o.TYPE_Q4_K else 1056
    packed, x, y32 = _exact_case(wtype, n, k, m, 700 + wtype + m)
    y = qblk.qblk_gemm(wtype, dev(packed.reshape(-1)), n, k, dev_quantize(x), m)
    assert np.array_equal(host(y), y32)


# ================================================================ random products

@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("n,k,batch", cases.GEMV_RANDOM)
def test_gemv_random(wtype, n, k, batch):
    print(f"gemv {TNAME[wtype]} n={n} k={k} batch={batch}", flush=True)
    rng = np.random.default_rng(31 * wtype + n + batch)
    w = _special_rows(rng, n, k)
    x = rng.standard_normal((batch, k)).astype(np.float32)
    y = qblk.qblk_gemv(wtype, dev_pack(wtype, w), n, k, dev_quantize(x), batch)
    check_rel(host(y), expected(wtype, w, x))


@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("m,n,k", [(1, 37, 256), (5, 300, 1024), (70, 129, 2304),
                                   (130, 257, 512), (256, 128, 4096), (16, 513, 2304),
                                   (33, 100, 256), (64, 1000, 4096), (17, 47, 7168),
                                   # one output, and rows long enough for many K steps
                                   (1, 1, 256), (70, 65, 32768),
                                   # 5-8 rows past 8192 weight rows: the few-rows kernel
                                   # for Q4_0 / Q8_0 (qblk_gemv's kernels at fewer rows)
                                   (8, 9000, 1024),
                                   # the few-rows kernel's 32- and 16-row tiles (short matrices)
                                   (40, 5000, 2304), (24, 4100, 1024),
                                   # the 128 x 128 kernel past the few-rows range, with K split over
                                   # two wave groups (at most 256 workgroups): more than 256 rows
                                   # (ragged), more than 128 rows past 8192 weight rows, and the
                                   # shortest K (two steps); then more than 256 workgroups
                                   (520, 300, 1024), (200, 8300, 512), (300, 700, 256),
                                   (300, 12000, 256)])
def test_gemm_random(wtype, m, n, k):
    print(f"gemm {TNAME[wtype]} m={m} n={n} k={k}", flush=True)
    rng = np.random.default_rng(41 * wtype + m + n)
    w = _special_rows(rng, n, k)
    x = rng.standard_normal((m, k)).astype(np.float32)
    y = qblk.qblk_gemm(wtype, dev_pack(wtype, w), n, k, dev_quantize(x), m)
    check_rel(host(y), expected(wtype, w, x))


def test_gemv_ldy_and_empty_calls():
    print("gemv ldy / empty", flush=True)
    rng = np.random.default_rng(5)
    n, k, b = 100, 512, 3
    w = _special_rows(rng, n, k)
    x = rng.standard_normal((b, k)).astype(np.float32)
    wq, xq = dev_pack(o.TYPE_Q4_K, w), dev_quantize(x)
    ybig = torch().full((b, 160), -7.0, device="cuda")
    qblk.qblk_gemv(o.TYPE_Q4_K, wq, n, k, xq, b, y=ybig[:, :n])
    yh = host(ybig)
    check_rel(yh[:, :n], expected(o.TYPE_Q4_K, w, x))
    assert np.all(yh[:, n:] == -7.0)
    # empty calls write nothing
    qblk.qblk_gemv(o.TYPE_Q4_K, wq, 0, k, xq, b, y=ybig[:, :0])
    qblk.qblk_gemm(o.TYPE_Q4_K, wq, 0, k, xq, b, y=ybig[:, :0])
    assert np.all(host(ybig)[:, n:] == -7.0)


def test_gemm_few_rows_runs_gemv_kernels():
    """qblk_gemm with at most 8 rows runs qblk_gemv's kernels where they are
    faster: its result is then qblk_gemv's bit for bit (and the few-rows
    kernel's, on the remaining shapes, within the tolerance of the oracle)."""
    print("gemm few rows", flush=True)
    rng = np.random.default_rng(91)
    for wtype, n, k, m in ((o.TYPE_Q4_K, 300, 4096, 1), (o.TYPE_Q4_K, 9000, 4096, 8),
                           (o.TYPE_Q8_0, 700, 1024, 6), (o.TYPE_Q4_0, 9000, 512, 3)):
        w = _special_rows(rng, n, k)
        x = rng.standard_normal((m, k)).astype(np.float32)
        wq, xq = dev_pack(wtype, w), dev_quantize(x)
        yg = host(qblk.qblk_gemm(wtype, wq, n, k, xq, m))
        yv = host(qblk.qblk_gemv(wtype, wq, n, k, xq, m))
        assert np.array_equal(yg.view(np.uint32), yv.view(np.uint32)), (wtype, n, k, m)
        check_rel(yg, expected(wtype, w, x))


@pytest.mark.parametrize("fn", ["gemv", "gemm"])
def test_deterministic(fn):
    print(f"determinism {fn}", flush=True)
    rng = np.random.default_rng(77)
    n, k, m = 513, 4096, 4
    w = _special_rows(rng, n, k)
    x = rng.standard_normal((m, k)).astype(np.float32)
    wq, xq = dev_pack(o.TYPE_Q4_K, w), dev_quantize(x)
    f = qblk.qblk_gemv if fn == "gemv" else qblk.qblk_gemm
    a = host(f(o.TYPE_Q4_K, wq, n, k, xq, m))
    b = host(f(o.TYPE_Q4_K, wq, n, k, xq, m))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ================================================================ full workload sizes

def _sample_rows(n, count, seed):
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(n, size=min(count, n), replace=False))
    return np.unique(np.concatenate([[0, n - 1], rows]))


def _full_size_check(wtype, w_dev, x_np, rows, use_gemm=False):
    """Device: pack all of W, quantize x, product. Oracle: the sampled rows."""
    n, k = w_dev.shape
    m = x_np.shape[0]
    wq = qblk.qblk_pack_weights(wtype, w_dev)
    xq = dev_quantize(x_np)
    f = qblk.qblk_gemm if use_gemm else qblk.qblk_gemv
    y = host(f(wtype, wq, n, k, xq, m))
    w_rows = host(w_dev[torch().from_numpy(rows).cuda()])
    # the packed rows themselves are bit-exact
    packed = host(wq).reshape(n, -1)[rows]
    ref_packed, _ = o.encode_weights(wtype, w_rows)
    assert np.array_equal(packed, ref_packed)
    return check_rel(y[:, rows], expected(wtype, w_rows, x_np))


@pytest.mark.parametrize("case", cases.GEMV_FULL_SIZE)
def test_gemv_full_size_sampled(case):
    name, wl, wtype, n, k = case
    print(f"full-size gemv {name}", flush=True)
    w = synth.weights(wl, 0, n, k)
    x = synth.act(wl, 1, k)
    _full_size_check(wtype, dev(w), x, _sample_rows(n, 96, n + k))


@pytest.mark.parametrize("m", cases.GEMV_70B_BATCH)
@pytest.mark.parametrize("name,n,k", cases.GEMV_70B)
def test_gemv_70b_layer_sampled(name, n, k, m):
    print(f"70B-shaped gemv {name} {n}x{k} batch={m}", flush=True)
    w = synth.torch_weights("student_t", 5000 + n % 97, n, k)
    x = synth.act(5, m, k)
    _full_size_check(o.TYPE_Q4_K, w, x, _sample_rows(n, 48, n))
    del w
    torch().cuda.empty_cache()


@pytest.mark.parametrize("m", cases.GEMM_PREFILL_M)
def test_gemm_prefill_full_size_sampled(m):
    print(f"full-size gemm Q4_K m={m}", flush=True)
    n, k = 14336, 4096
    w = synth.weights(4, 0, n, k)
    x = synth.act(4, m, k)
    _full_size_check(o.TYPE_Q4_K, dev(w), x, _sample_rows(n, 64, m), use_gemm=True)
    if m <= 64:   # the decode kernel on the same inputs agrees too
        _full_size_check(o.TYPE_Q4_K, dev(w), x, _sample_rows(n, 32, m + 1))


# ================================================================ fused quantize + GEMV

@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("n,k,batch", cases.GEMV_F32)
def test_gemv_f32_matches_quantize_then_gemv(wtype, n, k, batch):
    if wtype == o.TYPE_Q4_K and k % 256:
        pytest.skip("Q4_K needs k % 256 == 0")
    print(f"gemv_f32 {TNAME[wtype]} n={n} k={k} batch={batch}", flush=True)
    assert batch <= qblk.qblk_gemv_f32_max_batch(k)
    rng = np.random.default_rng(61 * wtype + n + batch)
    w = _special_rows(rng, n, k)
    x = rng.standard_normal((batch, k)).astype(np.float32)
    x[0, :32] = 0
    wq = dev_pack(wtype, w)
    xd = dev(x)
    fused = host(qblk.qblk_gemv_f32(wtype, wq, n, k, xd))
    two_step = host(qblk.qblk_gemv(wtype, wq, n, k, qblk.qblk_quantize_act(xd), batch))
    assert np.array_equal(fused.view(np.uint32), two_step.view(np.uint32))
    if n * k <= 2000 * 28672:
        rows = _sample_rows(n, 64, n + batch)
        check_rel(fused[:, rows], expected(wtype, w[rows], x))


def _in_launch(n, k, batch):
    """Whether qblk_gemv_f32 quantizes the activation once per launch into
    the workspace (else in every workgroup's local memory)."""
    return not (batch == 1 and n * k <= 32 << 20 and (k <= 2048 or (k <= 4096 and n <= 2048)))


@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("n,k,batch", cases.GEMV_F32_IN_LAUNCH)
def test_gemv_f32_in_launch_quantization_reused_workspace(wtype, n, k, batch):
    """Products that quantize the activation once per launch into the
    workspace, one slice per (activation row, 64 blocks). One
    workspace serves consecutive calls on different activations (a stale
    slice would reproduce the previous call's result), also when it starts
    out holding arbitrary bytes; (16400, 2304, 3) has a partial last slice in
    every row, and the k = 2^24 cases have fewer workgroups than slices."""
    t = torch()
    print(f"gemv_f32 in-launch {TNAME[wtype]} n={n} k={k} batch={batch}", flush=True)
    assert _in_launch(n, k, batch)
    rng = np.random.default_rng(5 * wtype + n + k)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    wq = dev_pack(wtype, w)
    work = t.randint(0, 256, (qblk.qblk_gemv_f32_work_bytes(batch, k),), dtype=t.uint8,
                     device="cuda")
    fallbacks0 = qblk.handoff_fallbacks(work, batch, k)
    for call in range(3):
        x = rng.standard_normal((batch, k)).astype(np.float32)
        if call == 1:
            x *= np.float32(1e-3)
        xd = dev(x)
        fused = host(qblk.qblk_gemv_f32(wtype, wq, n, k, xd, work=work))
        two_step = host(qblk.qblk_gemv(wtype, wq, n, k, qblk.qblk_quantize_act(xd), batch))
        assert np.array_equal(fused.view(np.uint32), two_step.view(np.uint32)), call
    # no workgroup gave up waiting for the producers
    assert qblk.handoff_fallbacks(work, batch, k) == fallbacks0
    if k <= 28672:
        rows = _sample_rows(n, 16, n)
        check_rel(fused[:, rows], expected(wtype, w[rows], x))


@pytest.mark.parametrize("n,k,batch", cases.GEMV_F32_RING_TILES)
def test_gemv_f32_ring_tiles(n, k, batch):
    """Q4_K's tile-walking matrix-core kernel with the in-launch handoff, on
    grids where some workgroups take a second tile: bitwise equal to quantize
    + qblk_gemv on two calls, no fallback, within the tolerance of the
    oracle."""
    t = torch()
    print(f"gemv_f32 ring tiles n={n} k={k} batch={batch}", flush=True)
    assert qblk.qblk_gemv_variant(o.TYPE_Q4_K, n, k, batch, True).startswith("gemv_ring_tiles_kernel")
    rng = np.random.default_rng(n + 7 * k + batch)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    x = rng.standard_normal((batch, k)).astype(np.float32)
    wq = dev_pack(o.TYPE_Q4_K, w)
    xd = dev(x)
    work = t.zeros(qblk.qblk_gemv_f32_work_bytes(batch, k), dtype=t.uint8, device="cuda")
    for call in range(2):
        fused = host(qblk.qblk_gemv_f32(o.TYPE_Q4_K, wq, n, k, xd, work=work))
        two_step = host(qblk.qblk_gemv(o.TYPE_Q4_K, wq, n, k, qblk.qblk_quantize_act(xd), batch))
        assert np.array_equal(fused.view(np.uint32), two_step.view(np.uint32)), call
    assert qblk.handoff_fallbacks(work, batch, k) == 0
    rows = _sample_rows(n, 24, n + batch)
    check_rel(fused[:, rows], expected(o.TYPE_Q4_K, w[rows], x))


@pytest.mark.parametrize("n,k,batch", cases.GEMV_F32_RING_TILES_EXACT)
def test_gemv_f32_ring_tiles_exact_arithmetic(n, k, batch):
    """The tile-walking kernel with the in-launch handoff and power-of-two
    scales: every partial sum is exact in fp32, so y equals the oracle bit
    for bit."""
    print(f"gemv_f32 ring tiles exact n={n} k={k} batch={batch}", flush=True)
    packed, x, y32 = _exact_case(o.TYPE_Q4_K, n, k, batch, 990 + batch)
    y = qblk.qblk_gemv_f32(o.TYPE_Q4_K, dev(packed.reshape(-1)), n, k, dev(x))
    assert np.array_equal(host(y), y32)


@pytest.mark.parametrize("batch", cases.GEMV_F32_70B_BATCH)
@pytest.mark.parametrize("name,n,k", cases.GEMV_F32_70B)
def test_gemv_f32_70b_decode_shapes_sampled(name, n, k, batch):
    """qblk_gemv_f32 on the matrices of the 70B-shaped decode token as the
    benchmark launches them (q/k/v and gate/up concatenated by rows):
    bitwise equal to quantize + qblk_gemv, and within the tolerance of the
    oracle on sampled rows."""
    print(f"gemv_f32 70B-shaped {name} {n}x{k} batch={batch}", flush=True)
    t = torch()
    w = synth.torch_weights("student_t", 5100 + n % 89, n, k)
    x = synth.act(5, batch, k)
    wq = qblk.qblk_pack_weights(o.TYPE_Q4_K, w)
    xd = dev(x)
    fused = host(qblk.qblk_gemv_f32(o.TYPE_Q4_K, wq, n, k, xd))
    two_step = host(qblk.qblk_gemv(o.TYPE_Q4_K, wq, n, k, qblk.qblk_quantize_act(xd), batch))
    assert np.array_equal(fused.view(np.uint32), two_step.view(np.uint32))
    rows = _sample_rows(n, 40, n + batch)
    w_rows = host(w[t.from_numpy(rows).cuda()])
    del w, wq
    t.cuda.empty_cache()
    check_rel(fused[:, rows], expected(o.TYPE_Q4_K, w_rows, x))


@pytest.mark.parametrize("wtype", [o.TYPE_Q4_K, o.TYPE_Q8_0])
@pytest.mark.parametrize("n,k,batch", [(9000, 8192, 1), (16400, 8192, 4), (16400, 2304, 3),
                                       (3, 1 << 20, 4), (8200, 4096, 2), (10000, 8192, 8)])
def test_gemv_f32_handoff_fallback_is_bit_exact(wtype, n, k, batch):
    """With the handoff's wait bound set to 0 ticks every workgroup that
    finds a slice unpublished quantizes the whole activation itself, racing
    the producers over the same workspace bytes: the result is still bitwise
    that of quantize + qblk_gemv, and the workspace counter records the
    fallbacks. (3, 2^20, 4): one workgroup, which publishes every slice itself
    before it waits. Q4_K at (16400, 8192, 4), (8200, 4096, 2) and (10000,
    8192, 8): the tile-walking matrix-core kernel."""
    if wtype == o.TYPE_Q4_K and k % 256:
        pytest.skip("Q4_K needs k % 256 == 0")
    t = torch()
    print(f"gemv_f32 forced fallback {TNAME[wtype]} n={n} k={k} batch={batch}", flush=True)
    rng = np.random.default_rng(17 * wtype + n + batch)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    wq = dev_pack(wtype, w)
    work = t.zeros(qblk.qblk_gemv_f32_work_bytes(batch, k), dtype=t.uint8, device="cuda")
    x = dev(rng.standard_normal((batch, k)).astype(np.float32))
    two_step = host(qblk.qblk_gemv(wtype, wq, n, k, qblk.qblk_quantize_act(x), batch))
    qblk.qblk_gemv_f32_set_wait_limit(0)
    try:
        for call in range(2):
            fused = host(qblk.qblk_gemv_f32(wtype, wq, n, k, x, work=work))
            assert np.array_equal(fused.view(np.uint32), two_step.view(np.uint32)), call
    finally:
        qblk.qblk_gemv_f32_set_wait_limit(-1)
    fb = qblk.handoff_fallbacks(work, batch, k)
    print(f"  fallbacks: {fb}", flush=True)
    if n >= 9000:
        assert fb > 0
    # the default bound again: no fallback
    work.zero_()
    fused = host(qblk.qblk_gemv_f32(wtype, wq, n, k, x, work=work))
    assert np.array_equal(fused.view(np.uint32), two_step.view(np.uint32))
    assert qblk.handoff_fallbacks(work, batch, k) == 0


def test_gemv_f32_strided_rows_and_limits():
    print("gemv_f32 strided x / limits", flush=True)
    rng = np.random.default_rng(8)
    n, k = 513, 2048
    w = _special_rows(rng, n, k)
    big = rng.standard_normal((3, k + 64)).astype(np.float32)
    wq = dev_pack(o.TYPE_Q4_K, w)
    xs = dev(big)[:, 32:32 + k]
    y = host(qblk.qblk_gemv_f32(o.TYPE_Q4_K, wq, n, k, xs))
    check_rel(y, expected(o.TYPE_Q4_K, w, big[:, 32:32 + k]))
    assert qblk.qblk_gemv_f32_max_batch(28672) == 8
    assert qblk.qblk_gemv_f32_max_batch(4096) == 8
    assert qblk.qblk_gemv_f32_max_batch(100) == 0
    x9 = dev(rng.standard_normal((9, 256)).astype(np.float32))
    wq9 = dev_pack(o.TYPE_Q4_K, _special_rows(rng, 8, 256))
    with pytest.raises(qblk.QblkError) as ei:
        qblk.qblk_gemv_f32(o.TYPE_Q4_K, wq9, 8, 256, x9)
    assert ei.value.status == -4


# ================================================================ float activations

def _float_expected(wtype, w, x):
    _, enc = o.encode_weights(wtype, w)
    return o.product_float(wtype, enc, x)[1]


@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("n,k,batch", [(37, 1024, 1), (300, 4096, 2), (129, 2304, 3), (70, 256, 8),
                                       (1000, 8192, 1), (65, 512, 11), (40, 28672, 1), (50, 4096, 8)])
def test_gemv_float_random(wtype, n, k, batch):
    print(f"gemv float {TNAME[wtype]} n={n} k={k} batch={batch}", flush=True)
    rng = np.random.default_rng(91 * wtype + n + batch)
    w = _special_rows(rng, n, k)
    x = rng.standard_normal((batch, k)).astype(np.float32)
    y = qblk.qblk_gemv_float(wtype, dev_pack(wtype, w), n, k, dev(x))
    check_rel(host(y), _float_expected(wtype, w, x))


@pytest.mark.parametrize("wtype", [o.TYPE_Q4_0, o.TYPE_Q8_0, o.TYPE_Q4_0_F16])
def test_gemv_float_ragged_blocks(wtype):
    """k = 1056 (33 blocks: one chunk of 64 blocks, half the lanes idle) and a
    strided activation (ldx > k) with a strided output (ldy > n)."""
    print(f"gemv float ragged {TNAME[wtype]}", flush=True)
    rng = np.random.default_rng(95 + wtype)
    n, k, b = 45, 1056, 3
    w = _special_rows(rng, n, k)
    xbig = rng.standard_normal((b, k + 36)).astype(np.float32)
    x = dev(xbig)[:, :k]
    ybig = torch().full((b, n + 7), -5.0, device="cuda")
    qblk.qblk_gemv_float(wtype, dev_pack(wtype, w), n, k, x, y=ybig[:, :n])
    yh = host(ybig)
    check_rel(yh[:, :n], _float_expected(wtype, w, xbig[:, :k]))
    assert np.all(yh[:, n:] == -5.0)


def test_gemv_float_full_size_sampled():
    """Q4_K 14336 x 4096 and Q4_0 4096 x 4096 at the workload sizes, on sampled rows."""
    for wl, wtype, n, k in ((3, o.TYPE_Q4_K, 14336, 4096), (1, o.TYPE_Q4_0, 4096, 4096)):
        print(f"full-size gemv float {TNAME[wtype]} {n}x{k}", flush=True)
        w = synth.weights(wl, 0, n, k)
        x = synth.act(wl, 1, k)
        wq = qblk.qblk_pack_weights(wtype, dev(w))
        y = host(qblk.qblk_gemv_float(wtype, wq, n, k, dev(x)))
        rows = _sample_rows(n, 64, n + 7)
        check_rel(y[:, rows], _float_expected(wtype, w[rows], x))


# ================================================================ quantized KV cache

KV_TYPES = [o.TYPE_Q4_0, o.TYPE_Q8_0, o.TYPE_Q4_0_F16]


def _kv_fill(wtype, k, n_ctx):
    """Device cache holding k [n_kv, n_tok, hd] in rows (h, t), written per
    head with the weight packer (a prefill's bulk write)."""
    n_kv, n_tok, hd = k.shape
    cache = qblk.qblk_kv_cache(wtype, n_kv, n_ctx, hd)
    rb = qblk.qblk_weight_row_bytes(wtype, hd)
    for h in range(n_kv):
        view = cache[h * n_ctx * rb:(h * n_ctx + n_tok) * rb]
        qblk.qblk_pack_weights(wtype, dev(k[h]), out=view)
    return cache


@pytest.mark.parametrize("wtype", KV_TYPES)
def test_kv_store_bit_exact(wtype):
    """Token-by-token stores land in rows (h, pos) with the packer's bytes;
    rows not written stay untouched."""
    print(f"kv store {TNAME[wtype]}", flush=True)
    rng = np.random.default_rng(120 + wtype)
    n_kv, n_ctx, n_tok, hd = 3, 40, 29, 128
    k = rng.standard_normal((n_kv, n_tok, hd)).astype(np.float32)
    k[1, 3] = 0.0
    cache = qblk.qblk_kv_cache(wtype, n_kv, n_ctx, hd)
    for t in range(n_tok):
        qblk.qblk_kv_store(wtype, dev(np.ascontiguousarray(k[:, t])), cache, n_ctx, t)
    got = host(cache).reshape(n_kv, n_ctx, -1)
    for h in range(n_kv):
        ref, _ = o.encode_weights(wtype, k[h])
        assert np.array_equal(got[h, :n_tok], ref)
        assert np.all(got[h, n_tok:] == 0)


@pytest.mark.parametrize("wtype", KV_TYPES)
@pytest.mark.parametrize("n_kv,n_head,hd,n_ctx,n_tok", [(1, 1, 128, 64, 1), (2, 8, 128, 300, 257),
                                                        (4, 8, 64, 100, 100), (2, 16, 256, 50, 33),
                                                        (3, 6, 128, 80, 45), (2, 10, 64, 700, 650),
                                                        (1, 7, 256, 40, 40), (16, 64, 64, 8300, 8200),
                                                        (32, 32, 256, 4200, 4100)])
def test_kv_scores_random(wtype, n_kv, n_head, hd, n_ctx, n_tok):
    print(f"kv scores {TNAME[wtype]} n_kv={n_kv} n_head={n_head} hd={hd} n_tok={n_tok}", flush=True)
    rng = np.random.default_rng(130 + wtype + n_tok)
    k = rng.standard_normal((n_kv, n_tok, hd)).astype(np.float32)
    k[0, 0, :32] = 0.0
    q = rng.standard_normal((n_head, hd)).astype(np.float32)
    cache = _kv_fill(wtype, k, n_ctx)
    s = torch().full((n_head, n_tok + 5), -9.0, device="cuda")
    qblk.qblk_kv_scores(wtype, cache, n_kv, n_ctx, n_tok, hd, dev_quantize(q), n_head, scores=s[:, :n_tok])
    sh = host(s)
    check_rel(sh[:, :n_tok], o.kv_scores(wtype, k, q, n_head)[1])
    assert np.all(sh[:, n_tok:] == -9.0)


def test_kv_scores_prefix_and_stores_agree():
    """Scores over a prefix of the cache, after token-by-token stores, equal
    the oracle's on that prefix; an empty prefix writes nothing."""
    print("kv scores prefix", flush=True)
    rng = np.random.default_rng(140)
    n_kv, n_head, hd, n_ctx, n_tok = 2, 4, 128, 64, 50
    k = rng.standard_normal((n_kv, n_tok, hd)).astype(np.float32)
    q = rng.standard_normal((n_head, hd)).astype(np.float32)
    cache = qblk.qblk_kv_cache(o.TYPE_Q8_0, n_kv, n_ctx, hd)
    for t in range(n_tok):
        qblk.qblk_kv_store(o.TYPE_Q8_0, dev(np.ascontiguousarray(k[:, t])), cache, n_ctx, t)
    qq = dev_quantize(q)
    for prefix in (1, 17, 50):
        s = qblk.qblk_kv_scores(o.TYPE_Q8_0, cache, n_kv, n_ctx, prefix, hd, qq, n_head)
        check_rel(host(s)[:, :prefix], o.kv_scores(o.TYPE_Q8_0, k[:, :prefix], q, n_head)[1])
    s = torch().full((n_head, 4), -1.0, device="cuda")
    qblk.qblk_kv_scores(o.TYPE_Q8_0, cache, n_kv, n_ctx, 0, hd, qq, n_head, scores=s)
    assert np.all(host(s) == -1.0)


@pytest.mark.parametrize("wtype", KV_TYPES)
@pytest.mark.parametrize("n_ctx,n_tok", [(8192, 8192), (20000, 16411)])
def test_kv_scores_70b_shape_sampled(wtype, n_ctx, n_tok):
    """70B-shaped decode step: 64 query heads over 8 KV heads of 128, 8192
    cached tokens, or 16411 of 20000 (over 2^17 cache rows, where Q8_0 takes
    two token steps per wave, with a ragged last workgroup); the oracle checks
    sampled tokens of every head."""
    print(f"kv scores 70B shape {TNAME[wtype]} n_tok={n_tok}", flush=True)
    rng = np.random.default_rng(150 + wtype)
    n_kv, n_head, hd = 8, 64, 128
    k = rng.standard_normal((n_kv, n_tok, hd)).astype(np.float32)
    q = rng.standard_normal((n_head, hd)).astype(np.float32)
    cache = _kv_fill(wtype, k, n_ctx)
    s = host(qblk.qblk_kv_scores(wtype, cache, n_kv, n_ctx, n_tok, hd, dev_quantize(q), n_head))
    assert s.shape == (n_head, n_tok)
    toks = np.unique(np.concatenate([_sample_rows(n_tok, 200, 151), np.arange(n_tok - 70, n_tok)]))
    check_rel(s[:, toks], o.kv_scores(wtype, k[:, toks], q, n_head)[1])


# ================================================================ multi-product launch

@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("batch,ks", [(1, (4096, 4096, 2304)), (3, (1024, 1024, 2048)),
                                      (1, (28672, 4096, 256)), (9, (512, 512, 768)),
                                      # every k a multiple of 2048: the matrix-core form
                                      (4, (4096, 4096, 2048)), (10, (2048, 2048, 4096))])
def test_gemv_multi_matches_single_products(wtype, batch, ks):
    """Three descriptors (q/k/v-like row counts, one with its own activation
    and k) in one launch: each output is bit-identical to its own qblk_gemv
    (within 1e-6 where qblk_gemv runs the matrix-core kernel but the list
    mixes k that it cannot take, so the list runs the dot4 kernel) and within
    the bar of the oracle."""
    print(f"gemv multi {TNAME[wtype]} batch={batch} ks={ks}", flush=True)
    rng = np.random.default_rng(160 + wtype + batch)
    ns = (300, 77, 1030)
    prods, refs = [], []
    xs = {}
    for n, k in zip(ns, ks):
        if wtype == o.TYPE_Q4_K and k % 256:
            k = 256 * max(1, k // 256)
        w = _special_rows(rng, n, k)
        if k not in xs:
            xs[k] = rng.standard_normal((batch, k)).astype(np.float32)
        wq, xq = dev_pack(wtype, w), dev_quantize(xs[k])
        y = torch().full((batch, n + 3), -4.0, device="cuda")
        prods.append((wq, n, k, xq, y[:, :n]))
        refs.append((w, xs[k], qblk.qblk_gemv(wtype, wq, n, k, xq, batch), y))
    qblk.qblk_gemv_multi(wtype, prods, batch)
    ring_list = wtype == o.TYPE_Q4_K and all(k % 2048 == 0 for (_, _, k, _, _) in prods)
    for (w, x, ysingle, ybig), (_, n, k, _, _) in zip(refs, prods):
        yh = host(ybig)
        if not ring_list and qblk.qblk_gemv_variant(wtype, n, k, batch, False).startswith("gemv_ring"):
            # qblk_gemv runs the matrix-core kernel here: the same block
            # products and scale steps, summed in another order
            ys = host(ysingle)
            assert np.max(np.abs(yh[:, :n] - ys)) <= 1e-6 * np.max(np.abs(ys))
        else:
            assert np.array_equal(yh[:, :n], host(ysingle))
        assert np.all(yh[:, n:] == -4.0)
        check_rel(yh[:, :n], expected(wtype, w, x))


def test_gemv_multi_skips_empty_descriptors():
    print("gemv multi empty descriptors", flush=True)
    rng = np.random.default_rng(170)
    k = 1024
    w = _special_rows(rng, 64, k)
    x = rng.standard_normal((1, k)).astype(np.float32)
    wq, xq = dev_pack(o.TYPE_Q8_0, w), dev_quantize(x)
    y = torch().zeros((1, 64), device="cuda")
    empty = torch().full((1, 1), -3.0, device="cuda")
    qblk.qblk_gemv_multi(o.TYPE_Q8_0, [(wq, 0, k, xq, empty), (wq, 64, k, xq, y)], 1)
    check_rel(host(y), expected(o.TYPE_Q8_0, w, x))
    assert host(empty)[0, 0] == -3.0
