"""Host-side checks of the C ABI: the library loads without a GPU, exports
exactly the functions include/qblk.h declares, its size functions match the
oracle's layouts, and invalid arguments are rejected with the documented
status before anything is launched. No compute call is made here."""

import ctypes
import os
import re
import shutil
import subprocess

import pytest

from block_quantized_qblk_amd import qblk
from oracle import qblk_oracle as o

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qblk.h")

OK, ERR_ARG, ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED = 0, -1, -2, -3, -4

# plausible 256-byte aligned device addresses that are never dereferenced
# (validation fails before any launch in every call below)
FAKE = 0x7F0000000000


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qblk_\w+)\s*\(", text)))


def test_library_loads_and_reports_abi():
    lib = qblk.lib()
    text = open(HEADER).read()
    abi = int(re.search(r"#define QBLK_ABI_VERSION (\d+)", text).group(1))
    layout = int(re.search(r"#define QBLK_LAYOUT_VERSION (\d+)", text).group(1))
    v = lib.qblk_abi_version()
    assert (v >> 8, v & 0xFF) == (abi, layout) == (2, 1)
    assert qblk.strerror(0) == "ok"
    assert "shape" in qblk.strerror(-2)


def test_exports_match_header():
    declared = _declared()
    assert len(declared) >= 10
    lib = qblk.lib()
    for name in declared:
        assert hasattr(lib, name), name
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", qblk.LIB_PATH],
                             capture_output=True, text=True, check=True).stdout
        exported = sorted(set(re.findall(r"\b[TW] (qblk_\w+)", out)))
        assert exported == declared


@pytest.mark.parametrize("k", [32, 96, 256, 416, 1024, 4096, 14336, 28672])
def test_size_functions_match_oracle(k):
    for t in (o.TYPE_Q4_0, o.TYPE_Q8_0, o.TYPE_Q4_K, o.TYPE_Q4_0_F16):
        if t == o.TYPE_Q4_K and k % 256:
            assert qblk.qblk_weight_row_bytes(t, k) == 0
            continue
        assert qblk.qblk_weight_row_bytes(t, k) == o.row_bytes(t, k)
        assert qblk.qblk_weight_bytes(t, 37, k) == 37 * o.row_bytes(t, k)
        assert qblk.qblk_weight_row_bytes(t, k) % 16 == 0
    assert qblk.qblk_act_bytes(5, k) == o.act_bytes(5, k)


def test_size_functions_reject_invalid():
    assert qblk.qblk_weight_row_bytes(0, 256) == 0
    assert qblk.qblk_weight_row_bytes(o.TYPE_Q4_0, 48) == 0
    assert qblk.qblk_weight_row_bytes(o.TYPE_Q4_0, 0) == 0
    assert qblk.qblk_weight_bytes(o.TYPE_Q8_0, -1, 256) == 0
    assert qblk.qblk_act_bytes(1, 33) == 0
    assert qblk.qblk_act_bytes(-1, 32) == 0
    assert qblk.qblk_act_bytes(0, 32) == 0


def _p(addr):
    return ctypes.c_void_p(addr)


NULL = ctypes.c_void_p(0)


def test_product_argument_validation():
    lib = qblk.lib()
    for fname in ("qblk_gemv", "qblk_gemm"):
        f = getattr(lib, fname)
        w, x, y = _p(FAKE), _p(FAKE + 0x100000), _p(FAKE + 0x200000)
        assert f(9, w, 16, 256, x, 1, y, 16, NULL) == ERR_ARG          # unknown type
        assert f(3, w, -1, 256, x, 1, y, 16, NULL) == ERR_ARG          # negative n
        assert f(3, w, 16, 256, x, -2, y, 16, NULL) == ERR_ARG         # negative m
        assert f(3, w, 16, 288, x, 1, y, 16, NULL) == ERR_SHAPE        # Q4_K k % 256
        assert f(1, w, 16, 48, x, 1, y, 16, NULL) == ERR_SHAPE         # k % 32
        assert f(2, w, 16, 0, x, 1, y, 16, NULL) == ERR_SHAPE          # k == 0
        assert f(3, NULL, 16, 256, x, 1, y, 16, NULL) == ERR_ARG       # null wq
        assert f(3, w, 16, 256, NULL, 1, y, 16, NULL) == ERR_ARG       # null xq
        assert f(3, w, 16, 256, x, 1, NULL, 16, NULL) == ERR_ARG       # null y
        assert f(3, w, 16, 256, x, 1, y, 15, NULL) == ERR_SHAPE        # ldy < n
        assert f(3, _p(FAKE + 8), 16, 256, x, 1, y, 16, NULL) == ERR_ALIGN
        assert f(3, w, 16, 256, _p(FAKE + 4), 1, y, 16, NULL) == ERR_ALIGN
        assert f(3, w, 16, 256, x, 1, _p(FAKE + 2), 16, NULL) == ERR_ALIGN
        # empty calls are valid no-ops, even with null pointers
        assert f(3, NULL, 0, 256, NULL, 1, NULL, 0, NULL) == OK
        assert f(3, NULL, 16, 256, NULL, 0, NULL, 16, NULL) == OK
    assert lib.qblk_gemv(3, _p(FAKE), 16, 256, _p(FAKE), 65, _p(FAKE), 16, NULL) == ERR_UNSUPPORTED
    assert lib.qblk_gemm(3, _p(FAKE), 16, 256, _p(FAKE), 65536 * 128, _p(FAKE), 16,
                         NULL) == ERR_UNSUPPORTED
    assert lib.qblk_gemm(3, _p(FAKE), 16, (1 << 24) + 256, _p(FAKE), 4, _p(FAKE), 16,
                         NULL) == ERR_UNSUPPORTED


def test_quantize_and_pack_argument_validation():
    lib = qblk.lib()
    x, xq = _p(FAKE), _p(FAKE + 0x100000)
    q = lib.qblk_quantize_act
    assert q(x, -1, 256, 256, xq, NULL) == ERR_ARG
    assert q(x, 2, 100, 256, xq, NULL) == ERR_SHAPE
    assert q(x, 2, 256, 255, xq, NULL) == ERR_SHAPE
    assert q(x, 2, 256, 258, xq, NULL) == ERR_ALIGN
    assert q(_p(FAKE + 4), 2, 256, 256, xq, NULL) == ERR_ALIGN
    assert q(x, 2, 256, 256, _p(FAKE + 8), NULL) == ERR_ALIGN
    assert q(NULL, 2, 256, 256, xq, NULL) == ERR_ARG
    assert q(NULL, 0, 256, 256, NULL, NULL) == OK
    p = lib.qblk_pack_weights
    assert p(5, x, 4, 256, 256, xq, NULL) == ERR_ARG
    assert p(3, x, 4, 32, 32, xq, NULL) == ERR_SHAPE
    assert p(1, x, 4, 32, 16, xq, NULL) == ERR_SHAPE
    assert p(1, x, 4, 32, 34, xq, NULL) == ERR_ALIGN
    assert p(2, x, 4, 32, 32, _p(FAKE + 4), NULL) == ERR_ALIGN
    assert p(2, x, -4, 32, 32, xq, NULL) == ERR_ARG
    assert p(2, NULL, 0, 32, 32, NULL, NULL) == OK
    b = lib.qblk_block_sums
    assert b(3, x, 4, 256, xq, 2, NULL, NULL) == ERR_ARG
    assert b(3, x, 4, 200, xq, 2, _p(FAKE), NULL) == ERR_SHAPE


def test_gemv_f32_workspace_size_and_validation():
    for k in (32, 2048, 4096, 8192, 28672, 1 << 20):
        for b in (1, 4, 8):
            wb = qblk.qblk_gemv_f32_work_bytes(b, k)
            # the activation buffer plus 8 copies of one 8-byte flag per
            # (activation row, 64-block slice)
            assert wb >= o.act_bytes(b, k) + 8 * 8 * b * (-(-k // 2048))
            assert wb % 256 == 0
    assert qblk.qblk_gemv_f32_work_bytes(9, 4096) == 0
    assert qblk.qblk_gemv_f32_work_bytes(1, 100) == 0
    assert qblk.qblk_gemv_f32_work_bytes(-1, 4096) == 0
    lib = qblk.lib()
    f = lib.qblk_gemv_f32
    w, x, y, wk = _p(FAKE), _p(FAKE + 0x100000), _p(FAKE + 0x200000), _p(FAKE + 0x300000)
    assert f(3, w, 16, 256, x, 256, 1, y, 16, NULL, NULL) == ERR_ARG            # null work
    assert f(3, w, 16, 256, x, 256, 1, y, 16, _p(FAKE + 0x300010), NULL) == ERR_ALIGN
    assert f(3, w, 16, 256, x, 255, 1, y, 16, wk, NULL) == ERR_SHAPE            # ldx < k
    assert f(3, w, 16, 256, x, 258, 1, y, 16, wk, NULL) == ERR_ALIGN            # ldx % 4
    assert f(3, w, 16, 256, _p(FAKE + 4), 256, 1, y, 16, wk, NULL) == ERR_ALIGN
    assert f(3, w, 16, 256, x, 256, 9, y, 16, wk, NULL) == ERR_UNSUPPORTED      # batch > 8
    assert f(3, w, 16, 288, x, 288, 1, y, 16, wk, NULL) == ERR_SHAPE
    assert f(3, NULL, 0, 256, NULL, 256, 1, NULL, 0, NULL, NULL) == OK          # empty


def test_gemv_float_validation():
    lib = qblk.lib()
    f = lib.qblk_gemv_float
    w, x, y = _p(FAKE), _p(FAKE + 0x100000), _p(FAKE + 0x200000)
    assert f(9, w, 16, 256, x, 256, 1, y, 16, NULL) == ERR_ARG                  # unknown type
    assert f(3, w, 16, 288, x, 288, 1, y, 16, NULL) == ERR_SHAPE                # Q4_K k % 256
    assert f(1, w, 16, 256, x, 255, 1, y, 16, NULL) == ERR_SHAPE                # ldx < k
    assert f(1, w, 16, 256, x, 258, 1, y, 16, NULL) == ERR_ALIGN                # ldx % 4
    assert f(1, w, 16, 256, _p(FAKE + 4), 256, 1, y, 16, NULL) == ERR_ALIGN     # x alignment
    assert f(1, w, 16, 256, x, 256, 1, y, 15, NULL) == ERR_SHAPE                # ldy < n
    assert f(1, NULL, 16, 256, x, 256, 1, y, 16, NULL) == ERR_ARG               # null wq
    assert f(2, w, 16, 256, x, 256, 65, y, 16, NULL) == ERR_UNSUPPORTED         # batch > 64
    assert f(3, NULL, 0, 256, NULL, 256, 1, NULL, 0, NULL) == OK                # empty
    assert f(3, NULL, 16, 256, NULL, 256, 0, NULL, 16, NULL) == OK


def test_kv_cache_validation():
    for t in (o.TYPE_Q4_0, o.TYPE_Q8_0, o.TYPE_Q4_0_F16):
        for hd in (64, 128, 256):
            assert qblk.qblk_kv_cache_bytes(t, 8, 1000, hd) == 8 * 1000 * o.row_bytes(t, hd)
    assert qblk.qblk_kv_cache_bytes(o.TYPE_Q4_K, 8, 1000, 256) == 0
    assert qblk.qblk_kv_cache_bytes(o.TYPE_Q8_0, 8, 1000, 96) == 0
    assert qblk.qblk_kv_cache_bytes(o.TYPE_Q8_0, 0, 1000, 128) == 0
    assert qblk.qblk_kv_cache_bytes(o.TYPE_Q8_0, 8, 0, 128) == 0
    lib = qblk.lib()
    x, c, q, s = _p(FAKE), _p(FAKE + 0x100000), _p(FAKE + 0x200000), _p(FAKE + 0x300000)
    st = lib.qblk_kv_store
    assert st(3, x, 8, 128, 128, c, 100, 0, NULL) == ERR_ARG                  # Q4_K
    assert st(2, x, 8, 96, 96, c, 100, 0, NULL) == ERR_SHAPE                  # head_dim
    assert st(2, x, 8, 128, 128, c, 100, 100, NULL) == ERR_SHAPE              # pos == n_ctx
    assert st(2, x, 8, 128, 128, c, 100, -1, NULL) == ERR_SHAPE
    assert st(2, x, 8, 128, 127, c, 100, 0, NULL) == ERR_SHAPE                # ldx < head_dim
    assert st(2, x, 8, 128, 130, c, 100, 0, NULL) == ERR_ALIGN                # ldx % 4
    assert st(2, x, 8, 128, 128, _p(FAKE + 8), 100, 0, NULL) == ERR_ALIGN
    assert st(2, NULL, 8, 128, 128, c, 100, 0, NULL) == ERR_ARG
    assert st(2, NULL, 0, 128, 128, NULL, 100, 0, NULL) == OK                 # no heads
    sc = lib.qblk_kv_scores
    assert sc(3, c, 8, 100, 10, 128, q, 64, s, 10, NULL) == ERR_ARG          # Q4_K
    assert sc(2, c, 8, 100, 10, 128, q, 60, s, 10, NULL) == ERR_ARG          # n_head % n_kv
    assert sc(2, c, 0, 100, 10, 128, q, 64, s, 10, NULL) == ERR_ARG
    assert sc(2, c, 8, 100, 101, 128, q, 64, s, 101, NULL) == ERR_SHAPE      # n_tok > n_ctx
    assert sc(2, c, 8, 100, 10, 128, q, 64, s, 9, NULL) == ERR_SHAPE         # lds < n_tok
    assert sc(2, c, 8, 100, 10, 128, _p(FAKE + 4), 64, s, 10, NULL) == ERR_ALIGN
    assert sc(2, c, 8, 100, 10, 128, q, 64, _p(FAKE + 2), 10, NULL) == ERR_ALIGN
    assert sc(2, c, 4, 100, 10, 128, q, 64, s, 10, NULL) == ERR_UNSUPPORTED  # group 16
    assert sc(2, NULL, 8, 100, 0, 128, NULL, 64, NULL, 0, NULL) == OK        # no tokens


def test_gemv_multi_validation():
    lib = qblk.lib()
    f = lib.qblk_gemv_multi
    D = qblk.GemvDesc
    good = D(FAKE, 16, 256, FAKE + 0x100000, FAKE + 0x200000, 16)
    arr = (D * 17)(*([good] * 17))
    p = ctypes.cast(arr, ctypes.c_void_p)
    assert f(9, p, 1, 1, NULL) == ERR_ARG                       # unknown type
    assert f(3, p, -1, 1, NULL) == ERR_ARG                      # negative count
    assert f(3, NULL, 1, 1, NULL) == ERR_ARG                    # null descriptors
    assert f(3, NULL, 0, 1, NULL) == OK                         # empty list
    assert f(3, p, 1, 0, NULL) == OK                            # no activation rows
    assert f(3, p, 17, 1, NULL) == ERR_UNSUPPORTED              # too many descriptors
    assert f(3, p, 2, 65, NULL) == ERR_UNSUPPORTED              # batch
    bad = (D * 2)(good, D(FAKE, 16, 288, FAKE, FAKE, 16))     # Q4_K k % 256 in the second
    assert f(3, ctypes.cast(bad, ctypes.c_void_p), 2, 1, NULL) == ERR_SHAPE
    bad = (D * 2)(good, D(FAKE + 8, 16, 256, FAKE, FAKE, 16))
    assert f(3, ctypes.cast(bad, ctypes.c_void_p), 2, 1, NULL) == ERR_ALIGN
    bad = (D * 2)(good, D(FAKE, 16, 256, FAKE, FAKE, 15))     # ldy < n
    assert f(3, ctypes.cast(bad, ctypes.c_void_p), 2, 1, NULL) == ERR_SHAPE


def test_gemv_variant_names():
    assert qblk.qblk_gemv_variant(o.TYPE_Q4_K, 57344, 8192, 1, True) == \
        "gemv_kernel<3, 1, 4, 1, true, true, 4>"
    # Q4_K at 2-8 activation rows with k a multiple of 2048: the matrix-core kernel
    assert qblk.qblk_gemv_variant(o.TYPE_Q4_K, 57344, 8192, 4, True) == "gemv_ring_tiles_kernel<4, true>"
    assert qblk.qblk_gemv_variant(o.TYPE_Q4_K, 8208, 4096, 3, False) == "gemv_ring_tiles_kernel<3, false>"
    assert qblk.qblk_gemv_variant(o.TYPE_Q4_K, 8208, 2048, 3, False) == "gemv_ring_kernel<3, false>"  # one chunk
    assert qblk.qblk_gemv_variant(o.TYPE_Q4_K, 8192, 4096, 3, False) == "gemv_ring_kernel<3, false>"
    assert qblk.qblk_gemv_variant(o.TYPE_Q4_K, 57344, 8192, 8, True) == "gemv_ring_tiles_kernel<8, true>"
    assert qblk.qblk_gemv_variant(o.TYPE_Q4_K, 8192, 8192, 3, False) == "gemv_ring_kernel<3, false>"
    assert qblk.qblk_gemv_variant(o.TYPE_Q4_K, 8192, 2304, 4, True) == "gemv_kernel<3, 4, 2, 1, true, true, 4>"
    assert qblk.qblk_gemv_variant(o.TYPE_Q4_K, 57344, 6400, 8, True) == "gemv_kernel<3, 8, 8, 1, true, false, 4>"
    assert qblk.qblk_gemv_variant(o.TYPE_Q8_0, 8192, 8192, 4, True) == "gemv_kernel<2, 4, 4, 1, true, true, 4>"
    assert qblk.qblk_gemv_variant(o.TYPE_Q4_K, 1024, 2048, 1, True).startswith("gemv_pipe_kernel<3, 1, 2, true")
    assert qblk.qblk_gemv_variant(o.TYPE_Q8_0, 14336, 4096, 1, False) == \
        "gemv_kernel<2, 1, 2, 2, false, true, 4>"
    assert qblk.qblk_gemv_variant(o.TYPE_Q4_K, 8192, 8192, 2, True) == "gemv_ring_kernel<2, true>"
    assert qblk.qblk_gemv_variant(o.TYPE_Q4_K, 8192, 8192, 5, True) == "gemv_ring_kernel<5, true>"
    assert qblk.qblk_gemv_variant(o.TYPE_Q4_K, 8192, 6400, 5, True) == \
        "gemv_kernel<3, 5, 4, 1, true, false, 8>"
    assert qblk.qblk_gemv_variant(o.TYPE_Q4_K, 8192, 2304, 2, True) == \
        "gemv_kernel<3, 2, 2, 1, true, true, 4>"
    lib = qblk.lib()
    buf = ctypes.create_string_buffer(8)
    assert lib.qblk_gemv_variant(3, 57344, 8192, 1, 1, buf, 8) == ERR_ARG      # too short
    assert lib.qblk_gemv_variant(3, 57344, 8100, 1, 1, buf, 8) == ERR_SHAPE
    assert lib.qblk_gemv_variant(3, 57344, 8192, 9, 1, buf, 8) == ERR_UNSUPPORTED
    assert lib.qblk_gemv_variant(9, 57344, 8192, 1, 1, buf, 8) == ERR_ARG


def test_benchmarked_gemv_instances_have_parity_cases():
    """Every GEMV kernel instance the benchmark times (the host's kernel
    selection replayed for each of its launches) is run by at least one GPU
    parity case."""
    import bench
    from block_quantized_qblk_amd import synth
    from tests import gemv_cases

    def name(case):
        t, n, k, b, fused = case
        return qblk.qblk_gemv_variant(t, n, k, min(b, 8), fused)

    covered = {name(c) for c in gemv_cases.covered()}
    missing = {}
    for c in bench.gemv_launches(synth):
        v = name(c)
        if v not in covered:
            missing[c] = v
    assert not missing, missing


def test_gemv_f32_fallback_counter_location():
    for batch, k in ((1, 4096), (4, 8192), (8, 28672), (3, 2304)):
        off = qblk.qblk_gemv_f32_fallback_offset(batch, k)
        assert off % 256 == 0
        assert off >= qblk.qblk_act_bytes(batch, k)
        assert off + 4 <= qblk.qblk_gemv_f32_work_bytes(batch, k)
    assert qblk.qblk_gemv_f32_fallback_offset(9, 4096) == 0
    assert qblk.qblk_gemv_f32_fallback_offset(1, 100) == 0
    assert qblk.lib().qblk_gemv_f32_set_wait_limit(0) == OK
    assert qblk.lib().qblk_gemv_f32_set_wait_limit(-1) == OK


def test_huge_sizes_are_rejected_without_overflow():
    """Sizes whose byte counts or grids would overflow 64-bit arithmetic are
    reported as invalid or unsupported (the sanitizer run of these tests
    halts on any signed overflow in the checks themselves)."""
    lib = qblk.lib()
    big, huge = 1 << 40, 1 << 62
    assert qblk.qblk_act_bytes(big, 1 << 20) == (1 << 60) + (1 << 58)   # still representable
    assert qblk.qblk_act_bytes(huge, 1 << 20) == 0
    assert qblk.qblk_weight_bytes(o.TYPE_Q8_0, huge, 1 << 20) == 0
    assert qblk.qblk_kv_cache_bytes(o.TYPE_Q8_0, 8, huge, 128) == 0
    w, x, y = _p(FAKE), _p(FAKE + 0x100000), _p(FAKE + 0x200000)
    for n in (big, huge):
        assert lib.qblk_pack_weights(2, x, n, 4096, 4096, w, NULL) == ERR_UNSUPPORTED
        assert lib.qblk_gemv(3, w, n, 256, x, 1, y, n, NULL) == ERR_UNSUPPORTED
        assert lib.qblk_gemv_float(3, w, n, 256, x, 256, 1, y, n, NULL) == ERR_UNSUPPORTED
        assert lib.qblk_gemm(3, w, n, 256, x, 512, y, n, NULL) == ERR_UNSUPPORTED
        assert lib.qblk_block_sums(3, w, n, 256, x, n, _p(FAKE), NULL) == ERR_UNSUPPORTED
        assert lib.qblk_quantize_act(x, n, 4096, 4096, w, NULL) == ERR_UNSUPPORTED
    work = _p(FAKE + 0x400000)
    assert lib.qblk_gemv_f32(3, w, huge, 256, x, 256, 1, y, huge, work, NULL) == ERR_UNSUPPORTED
    assert lib.qblk_kv_store(2, x, 8, 128, 128, w, huge, 0, NULL) == ERR_UNSUPPORTED
    assert lib.qblk_kv_scores(2, w, 8, huge, 16, 128, x, 64, y, 16, NULL) == ERR_UNSUPPORTED
