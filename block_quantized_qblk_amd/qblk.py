"""Python binding of libqblk.so (ctypes). Argument marshalling only: every
step of the product runs in the library's HIP kernels. torch supplies device
memory and the current stream.

Function names match the C ABI in include/qblk.h.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqblk.so")

Q4_0, Q8_0, Q4_K, Q4_0_F16 = 1, 2, 3, 4
TYPES = {"Q4_0": Q4_0, "Q8_0": Q8_0, "Q4_K": Q4_K, "Q4_0_F16": Q4_0_F16}
GEMV_MAX_BATCH = 64

_lib = None


class QblkError(RuntimeError):
    def __init__(self, status, what, hip_error=None):
        self.status = status
        self.hip_error = hip_error
        extra = f", hipError_t {hip_error}" if hip_error is not None else ""
        super().__init__(f"{what}: status {status} ({strerror(status)}{extra})")


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        # there is no fallback path: the library must have been built
        raise RuntimeError(f"{LIB_PATH} is missing; build it first with "
                           "`python -m block_quantized_qblk_amd.build_lib`")
    # torch's HIP runtime libraries are loaded before the library's own
    # (ROCm's): a process that had loaded ROCm's HIP and HSA libraries first
    # and then initialised torch's saw the library's first launch fail with
    # hipErrorNoDevice
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    sig = {
        "qblk_abi_version": (i32, []),
        "qblk_strerror": (ctypes.c_char_p, [i32]),
        "qblk_last_hip_error": (i32, []),
        "qblk_weight_row_bytes": (ctypes.c_size_t, [i32, i64]),
        "qblk_weight_bytes": (ctypes.c_size_t, [i32, i64, i64]),
        "qblk_act_bytes": (ctypes.c_size_t, [i64, i64]),
        "qblk_pack_weights": (i32, [i32, vp, i64, i64, i64, vp, vp]),
        "qblk_quantize_act": (i32, [vp, i64, i64, i64, vp, vp]),
        "qblk_gemv": (i32, [i32, vp, i64, i64, vp, i64, vp, i64, vp]),
        "qblk_gemm": (i32, [i32, vp, i64, i64, vp, i64, vp, i64, vp]),
        "qblk_gemv_f32_max_batch": (i32, [i64]),
        "qblk_gemv_f32_work_bytes": (ctypes.c_size_t, [i64, i64]),
        "qblk_gemv_f32": (i32, [i32, vp, i64, i64, vp, i64, i64, vp, i64, vp, vp]),
        "qblk_gemv_f32_fallback_offset": (ctypes.c_size_t, [i64, i64]),
        "qblk_gemv_f32_noalloc": (i32, [i32, vp, i64, i64, vp, i64, i64, vp, i64, vp]),
        "qblk_gemv_f32_set_wait_limit": (i32, [i64]),
        "qblk_gemv_float": (i32, [i32, vp, i64, i64, vp, i64, i64, vp, i64, vp]),
        "qblk_gemv_multi": (i32, [i32, vp, i32, i64, vp]),
        "qblk_gemv_variant": (i32, [i32, i64, i64, i64, i32, ctypes.c_char_p, ctypes.c_size_t]),
        "qblk_kv_cache_bytes": (ctypes.c_size_t, [i32, i64, i64, i64]),
        "qblk_kv_store": (i32, [i32, vp, i64, i64, i64, vp, i64, i64, vp]),
        "qblk_kv_scores": (i32, [i32, vp, i64, i64, i64, i64, vp, i64, vp, i64, vp]),
        "qblk_block_sums": (i32, [i32, vp, i64, i64, vp, i64, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def lib():
    return _load()


def _type(t):
    if isinstance(t, str):
        return TYPES[t]
    return int(t)


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _check(status, what):
    if status != 0:
        # a failed launch: the HIP error code the library kept for it
        hip = int(_load().qblk_last_hip_error()) if status == -5 else None  # QBLK_ERR_LAUNCH
        raise QblkError(status, what, hip)


def _require_cuda(t, name, rows=False):
    """Device tensor, contiguous (or, with rows=True, unit stride inside each
    row so that stride(0) can be passed as the leading dimension)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if rows:
        if t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{name} must be 2-D with unit stride along rows")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ---------------------------------------------------------------- sizes

def abi_version():
    return _load().qblk_abi_version()


def strerror(status):
    return _load().qblk_strerror(int(status)).decode()


def qblk_weight_row_bytes(wtype, k):
    return int(_load().qblk_weight_row_bytes(_type(wtype), int(k)))


def qblk_weight_bytes(wtype, n, k):
    return int(_load().qblk_weight_bytes(_type(wtype), int(n), int(k)))


def qblk_act_bytes(m, k):
    return int(_load().qblk_act_bytes(int(m), int(k)))


# ---------------------------------------------------------------- entry points

def qblk_pack_weights(wtype, w, out=None, stream=None):
    """Quantize fp32 weights w [n, k] (device) into a packed uint8 buffer."""
    import torch
    _require_cuda(w, "w", rows=True)
    if w.dtype != torch.float32 or w.dim() != 2:
        raise ValueError("w must be a 2-D float32 tensor")
    n, k = w.shape
    t = _type(wtype)
    nbytes = qblk_weight_bytes(t, n, k)
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=w.device)
    elif out.numel() < nbytes:
        raise ValueError("out too small")
    _check(_load().qblk_pack_weights(t, _ptr(w), n, k, w.stride(0), _ptr(out), _stream(stream)),
           "qblk_pack_weights")
    return out


def qblk_quantize_act(x, out=None, stream=None):
    """Quantize fp32 activations x [m, k] (device) into an activation buffer."""
    import torch
    _require_cuda(x, "x", rows=True)
    if x.dtype != torch.float32 or x.dim() != 2:
        raise ValueError("x must be a 2-D float32 tensor")
    m, k = x.shape
    nbytes = qblk_act_bytes(m, k)
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    elif out.numel() < nbytes:
        raise ValueError("out too small")
    _check(_load().qblk_quantize_act(_ptr(x), m, k, x.stride(0), _ptr(out), _stream(stream)),
           "qblk_quantize_act")
    return out


def _product(fname, wtype, wq, n, k, xq, m, y, stream):
    import torch
    _require_cuda(wq, "wq")
    _require_cuda(xq, "xq")
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=wq.device)
    _require_cuda(y, "y", rows=True)
    if y.dtype != torch.float32 or y.dim() != 2 or y.shape[0] < m or y.shape[1] < n:
        raise ValueError("y must be float32 [m, >= n]")
    if wq.numel() < qblk_weight_bytes(wtype, n, k) or xq.numel() < qblk_act_bytes(m, k):
        raise ValueError("wq or xq smaller than the packed sizes")
    fn = getattr(_load(), fname)
    _check(fn(_type(wtype), _ptr(wq), int(n), int(k), _ptr(xq), int(m), _ptr(y), y.stride(0),
              _stream(stream)), fname)
    return y


def qblk_gemv(wtype, wq, n, k, xq, batch=1, y=None, stream=None):
    """y[b, :n] = W x_b for b < batch (decode path, batch <= 64)."""
    return _product("qblk_gemv", wtype, wq, n, k, xq, batch, y, stream)


def qblk_gemv_f32_max_batch(k):
    return int(_load().qblk_gemv_f32_max_batch(int(k)))


def qblk_gemv_f32_work_bytes(batch, k):
    return int(_load().qblk_gemv_f32_work_bytes(int(batch), int(k)))


def qblk_gemv_f32_fallback_offset(batch, k):
    return int(_load().qblk_gemv_f32_fallback_offset(int(batch), int(k)))


def qblk_gemv_f32_set_wait_limit(ticks):
    """Test setting: the in-launch handoff's wait bound for this thread's
    later launches (100 MHz ticks; negative restores the 20 ms default)."""
    _check(_load().qblk_gemv_f32_set_wait_limit(int(ticks)), "qblk_gemv_f32_set_wait_limit")


def handoff_fallbacks(work, batch, k):
    """The fallback counter inside a qblk_gemv_f32 workspace (a device read)."""
    off = qblk_gemv_f32_fallback_offset(batch, k)
    return int(work[off:off + 4].view(__import__("torch").int32).item())


def qblk_gemv_f32(wtype, wq, n, k, x, batch=None, y=None, work=None, stream=None):
    """y[b, :n] = W quant(x_b): activation quantization fused into the GEMV.
    x: float32 [batch, >= k] device tensor with unit stride along rows.
    work: uint8 device workspace of qblk_gemv_f32_work_bytes(batch, k) bytes
    (allocated and zeroed here when None); calls that may overlap need their
    own. Its fallback counter (handoff_fallbacks) counts only if the caller
    zeroed the workspace once."""
    import torch
    _require_cuda(wq, "wq")
    _require_cuda(x, "x", rows=True)
    if x.dtype != torch.float32 or x.shape[1] < k:
        raise ValueError("x must be float32 [batch, >= k]")
    if batch is None:
        batch = x.shape[0]
    if y is None:
        y = torch.empty((batch, n), dtype=torch.float32, device=wq.device)
    _require_cuda(y, "y", rows=True)
    if y.dtype != torch.float32 or y.shape[0] < batch or y.shape[1] < n:
        raise ValueError("y must be float32 [batch, >= n]")
    if wq.numel() < qblk_weight_bytes(wtype, n, k):
        raise ValueError("wq smaller than the packed size")
    need = qblk_gemv_f32_work_bytes(batch, k)
    if work is None:
        work = torch.zeros(max(need, 1), dtype=torch.uint8, device=wq.device)
    _require_cuda(work, "work")
    if work.numel() < need:
        raise ValueError("work smaller than qblk_gemv_f32_work_bytes(batch, k)")
    _check(_load().qblk_gemv_f32(_type(wtype), _ptr(wq), int(n), int(k), _ptr(x), x.stride(0),
                                 int(batch), _ptr(y), y.stride(0), _ptr(work), _stream(stream)),
           "qblk_gemv_f32")
    return y


def qblk_gemv_f32_noalloc(wtype, wq, n, k, x, y, batch=None, stream=None):
    """qblk_gemv_f32 without a workspace (the library's fixed device array;
    allocates nothing, so y must be given). Calls that overlap on one GPU
    race on the array."""
    import torch
    _require_cuda(wq, "wq")
    _require_cuda(x, "x", rows=True)
    _require_cuda(y, "y", rows=True)
    if x.dtype != torch.float32 or y.dtype != torch.float32:
        raise ValueError("x and y must be float32")
    if batch is None:
        batch = x.shape[0]
    if x.shape[1] < k or y.shape[0] < batch or y.shape[1] < n:
        raise ValueError("x must be [batch, >= k] and y [batch, >= n]")
    if wq.numel() < qblk_weight_bytes(wtype, n, k):
        raise ValueError("wq smaller than the packed size")
    _check(_load().qblk_gemv_f32_noalloc(_type(wtype), _ptr(wq), int(n), int(k), _ptr(x), x.stride(0),
                                         int(batch), _ptr(y), y.stride(0), _stream(stream)),
           "qblk_gemv_f32_noalloc")
    return y


class GemvDesc(ctypes.Structure):
    """One product of qblk_gemv_multi (mirrors qblk_gemv_desc)."""
    _fields_ = [("wq", ctypes.c_void_p), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("xq", ctypes.c_void_p), ("y", ctypes.c_void_p), ("ldy", ctypes.c_int64)]


def qblk_gemv_variant(wtype, n, k, batch=1, fused=False):
    """Name of the kernel instance qblk_gemv (fused=False) or qblk_gemv_f32
    (fused=True) launches for this shape (host only, no GPU)."""
    buf = ctypes.create_string_buffer(128)
    _check(_load().qblk_gemv_variant(_type(wtype), int(n), int(k), int(batch), int(bool(fused)),
                                     buf, len(buf)), "qblk_gemv_variant")
    return buf.value.decode()


def qblk_gemv_multi(wtype, products, batch, stream=None):
    """Several qblk_gemv products in one launch. products: list of
    (wq, n, k, xq, y) with y a float32 [>= batch, >= n] device tensor
    (unit stride along rows). Returns the list of y."""
    import torch
    descs = (GemvDesc * max(1, len(products)))()
    for i, (wq, n, k, xq, y) in enumerate(products):
        _require_cuda(wq, "wq")
        _require_cuda(xq, "xq")
        _require_cuda(y, "y", rows=True)
        if y.dtype != torch.float32 or y.shape[0] < batch or y.shape[1] < n:
            raise ValueError("y must be float32 [batch, >= n]")
        if wq.numel() < qblk_weight_bytes(wtype, n, k):
            raise ValueError("wq smaller than the packed size")
        if xq.numel() < qblk_act_bytes(batch, k):
            raise ValueError("xq smaller than qblk_act_bytes(batch, k)")
        descs[i] = GemvDesc(_ptr(wq), int(n), int(k), _ptr(xq), _ptr(y), y.stride(0))
    _check(_load().qblk_gemv_multi(_type(wtype), ctypes.cast(descs, ctypes.c_void_p), len(products), int(batch),
                                   _stream(stream)), "qblk_gemv_multi")
    return [p[4] for p in products]


def qblk_gemv_float(wtype, wq, n, k, x, batch=None, y=None, stream=None):
    """y[b, :n] = dequant(W) x_b with fp32 activations (no activation
    quantization). x: float32 [batch, >= k] device tensor with unit stride
    along rows and a row stride that is a multiple of 4."""
    import torch
    _require_cuda(wq, "wq")
    _require_cuda(x, "x", rows=True)
    if x.dtype != torch.float32 or x.shape[1] < k:
        raise ValueError("x must be float32 [batch, >= k]")
    if batch is None:
        batch = x.shape[0]
    if y is None:
        y = torch.empty((batch, n), dtype=torch.float32, device=wq.device)
    _require_cuda(y, "y", rows=True)
    if y.dtype != torch.float32 or y.shape[0] < batch or y.shape[1] < n:
        raise ValueError("y must be float32 [batch, >= n]")
    if wq.numel() < qblk_weight_bytes(wtype, n, k):
        raise ValueError("wq smaller than the packed size")
    _check(_load().qblk_gemv_float(_type(wtype), _ptr(wq), int(n), int(k), _ptr(x), x.stride(0),
                                   int(batch), _ptr(y), y.stride(0), _stream(stream)),
           "qblk_gemv_float")
    return y


def qblk_kv_cache_bytes(wtype, n_kv, n_ctx, head_dim):
    return int(_load().qblk_kv_cache_bytes(_type(wtype), int(n_kv), int(n_ctx), int(head_dim)))


def qblk_kv_cache(wtype, n_kv, n_ctx, head_dim, device="cuda"):
    """A zeroed uint8 device buffer holding an n_kv x n_ctx quantized cache."""
    import torch
    nbytes = qblk_kv_cache_bytes(wtype, n_kv, n_ctx, head_dim)
    if nbytes == 0:
        raise ValueError("invalid KV cache shape or type")
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def qblk_kv_store(wtype, x, cache, n_ctx, pos, stream=None):
    """Quantize x (float32 [n_kv, head_dim], rows with unit stride) into rows
    (h, pos) of the cache."""
    import torch
    _require_cuda(x, "x", rows=True)
    _require_cuda(cache, "cache")
    if x.dtype != torch.float32:
        raise ValueError("x must be float32 [n_kv, head_dim]")
    n_kv, head_dim = x.shape
    if cache.numel() < qblk_kv_cache_bytes(wtype, n_kv, n_ctx, head_dim):
        raise ValueError("cache smaller than qblk_kv_cache_bytes")
    _check(_load().qblk_kv_store(_type(wtype), _ptr(x), int(n_kv), int(head_dim), x.stride(0), _ptr(cache),
                                 int(n_ctx), int(pos), _stream(stream)), "qblk_kv_store")
    return cache


def qblk_kv_scores(wtype, cache, n_kv, n_ctx, n_tok, head_dim, q, n_head, scores=None, stream=None):
    """float32 [n_head, n_tok] scores of the quantized queries q (activation
    buffer of n_head rows of head_dim) against tokens [0, n_tok) of the cache."""
    import torch
    _require_cuda(cache, "cache")
    _require_cuda(q, "q")
    if cache.numel() < qblk_kv_cache_bytes(wtype, n_kv, n_ctx, head_dim):
        raise ValueError("cache smaller than qblk_kv_cache_bytes")
    if q.numel() < qblk_act_bytes(n_head, head_dim):
        raise ValueError("q smaller than qblk_act_bytes(n_head, head_dim)")
    if scores is None:
        scores = torch.empty((n_head, max(int(n_tok), 1)), dtype=torch.float32, device=cache.device)
    _require_cuda(scores, "scores", rows=True)
    if scores.dtype != torch.float32 or scores.shape[0] < n_head or scores.shape[1] < n_tok:
        raise ValueError("scores must be float32 [n_head, >= n_tok]")
    _check(_load().qblk_kv_scores(_type(wtype), _ptr(cache), int(n_kv), int(n_ctx), int(n_tok), int(head_dim),
                                  _ptr(q), int(n_head), _ptr(scores), scores.stride(0), _stream(stream)),
           "qblk_kv_scores")
    return scores


def qblk_gemm(wtype, wq, n, k, xq, m, y=None, stream=None):
    """Y[m, :n] = X W^T (prefill path, int8 matrix cores)."""
    return _product("qblk_gemm", wtype, wq, n, k, xq, m, y, stream)


def qblk_block_sums(wtype, wq, n, k, xq, m, out=None, stream=None):
    """int32 [m, n, k/32] integer block sums (test export)."""
    import torch
    _require_cuda(wq, "wq")
    _require_cuda(xq, "xq")
    if out is None:
        out = torch.empty((m, n, k // 32), dtype=torch.int32, device=wq.device)
    _require_cuda(out, "out")
    if out.numel() < m * n * (k // 32):
        raise ValueError("out too small")
    _check(_load().qblk_block_sums(_type(wtype), _ptr(wq), int(n), int(k), _ptr(xq), int(m),
                                   _ptr(out), _stream(stream)), "qblk_block_sums")
    return out
