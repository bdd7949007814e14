"""fp8_fine_grained_quant_amd -- Python binding of libfp8q (MI355X, gfx950).

Argument marshalling only: every step runs in the HIP kernels of libfp8q.so,
reached through its C ABI (include/fp8q.h).  PyTorch supplies device memory
and the current HIP stream.  There is no CPU fallback: if the library is
missing or a call is rejected, an exception is raised.

Raw entry points (same names and argument order as the C ABI, with torch
tensors in place of pointer + leading dimension):

    fp8q_quant_act_1x128(x, q, scale)
    fp8q_quant_weight_128x128(w, q, q_t, scale)        # q_t may be None
    fp8q_quant_transpose(x, q_t, scale_t)
    fp8q_gemm_fprop(xq, xs, wq, ws, y)
    fp8q_gemm_dgrad(dyq, dys, wq_t, ws, dx)
    fp8q_gemm_wgrad(dyq_t, dys_t, xq_t, xs_t, dw, accumulate=False)
    fp8q_grouped_gemm(xq, xs, wq, ws, offsets, y)
    fp8q_quant_mx_1x32(x, q, s)                        # microscaling variant
    fp8q_quant_mx_transpose(x, q_t, s_t, q=None, s=None)
    fp8q_gemm_mx(aq, as_, bq, bs, c, accumulate=False)
    fp8q_grouped_gemm_mx(xq, xs, wq, ws, offsets, y)
    fp8q_grouped_gemm_mx_dgrad(dyq, dys, wq_t, ws_t, offsets, dx)

Each GEMM also takes exact=True, which calls the *_exact entry point (BF16
matrix instruction on exactly converted codes: the exact-accumulation variant).

Convenience wrappers that allocate the outputs: quant_act_1x128,
quant_weight_128x128, quant_transpose, gemm_fprop, gemm_dgrad, gemm_wgrad,
grouped_gemm, quant_mx, quant_mx_transpose, gemm_mx, grouped_gemm_mx, grouped_gemm_mx_dgrad (and those of the MoE
backward and the dual-output quantizer).
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8q.so")
# the same library built with FP8Q_DEBUG: its grouped entry points also read
# the device expert offsets back and reject malformed ones (synchronously)
DEBUG_LIB_PATH = os.path.join(_HERE, "libfp8q_debug.so")

FP8Q_BF16, FP8Q_F32 = 0, 1
_STATUS = ["FP8Q_OK", "FP8Q_ERR_NULL", "FP8Q_ERR_SHAPE", "FP8Q_ERR_STRIDE",
           "FP8Q_ERR_ALIGN", "FP8Q_ERR_DTYPE", "FP8Q_ERR_LAUNCH"]
EXPORTS = ["fp8q_status_string", "fp8q_set_gemm_tile", "fp8q_quant_act_1x128", "fp8q_quant_weight_128x128",
           "fp8q_quant_transpose", "fp8q_gemm_fprop", "fp8q_gemm_dgrad", "fp8q_gemm_wgrad",
           "fp8q_grouped_gemm", "fp8q_gemm_fprop_exact", "fp8q_gemm_dgrad_exact", "fp8q_gemm_wgrad_exact",
           "fp8q_grouped_gemm_exact", "fp8q_quant_transpose_grouped", "fp8q_grouped_gemm_dgrad",
           "fp8q_grouped_gemm_wgrad", "fp8q_quant_act_transpose", "fp8q_quant_mx_1x32",
           "fp8q_quant_mx_transpose", "fp8q_gemm_mx", "fp8q_grouped_gemm_mx",
           "fp8q_grouped_gemm_mx_dgrad", "fp8q_gemm_fprop_quant", "fp8q_gemm_dgrad_quant",
           "fp8q_gemm_fprop_interval", "fp8q_quant_batch"]


MAX_QUANT_JOBS = 8
QUANT_KINDS = {"act": 0, "weight": 1, "transpose": 2, "act_transpose": 3}


class QuantJob(ctypes.Structure):
    """fp8q_quant_job of include/fp8q.h."""
    _fields_ = [("kind", ctypes.c_int32), ("xt", ctypes.c_int32), ("x", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("ld_x", ctypes.c_int64),
                ("q", ctypes.c_void_p), ("ld_q", ctypes.c_int64), ("scale", ctypes.c_void_p),
                ("ld_s", ctypes.c_int64), ("q_t", ctypes.c_void_p), ("ld_qt", ctypes.c_int64),
                ("scale_t", ctypes.c_void_p), ("ld_st", ctypes.c_int64)]


class Fp8qError(RuntimeError):
    def __init__(self, status, name):
        self.status = status
        super().__init__(f"{name}: {status_string(status)}")


_lib = None


def load_library(path=LIB_PATH):
    """Load libfp8q.so (once) and declare its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = _open(path)
    return _lib


_debug_lib = None


def load_debug_library():
    """libfp8q_debug.so (once), with the same C signatures; the wrappers of
    this module keep calling libfp8q.so."""
    global _debug_lib
    if _debug_lib is None:
        _debug_lib = _open(DEBUG_LIB_PATH)
    return _debug_lib


def _open(path):
    if not os.path.exists(path):
        raise RuntimeError(f"{os.path.basename(path)} not built ({path}); run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sig = {
        "fp8q_status_string": ([I32], ctypes.c_char_p),
        "fp8q_set_gemm_tile": ([I32], I32),
        "fp8q_quant_act_1x128": ([P, I32, I64, I64, I64, P, I64, P, I64, P], I32),
        "fp8q_quant_weight_128x128": ([P, I32, I64, I64, I64, P, I64, P, I64, P, I64, P], I32),
        "fp8q_quant_transpose": ([P, I32, I64, I64, I64, P, I64, P, I64, P], I32),
        "fp8q_gemm_fprop": ([P, P, P, P, I64, I64, I64, P, I32, I64, P], I32),
        "fp8q_gemm_dgrad": ([P, P, P, P, I64, I64, I64, P, I32, I64, P], I32),
        "fp8q_gemm_wgrad": ([P, P, P, P, I64, I64, I64, P, I64, I32, P], I32),
        "fp8q_grouped_gemm": ([P, P, P, P, P, I64, I64, I64, I64, P, I32, I64, P], I32),
        "fp8q_quant_transpose_grouped": ([P, I32, I64, I64, I64, P, I64, P, I64, P, I64, P], I32),
        "fp8q_quant_act_transpose": ([P, I32, I64, I64, I64, P, I64, P, I64, P, I64, P, I64, P], I32),
        "fp8q_grouped_gemm_dgrad": ([P, P, P, P, P, I64, I64, I64, I64, P, I32, I64, P], I32),
        "fp8q_grouped_gemm_wgrad": ([P, P, P, P, P, I64, I64, I64, I64, I64, P, I32, P], I32),
        "fp8q_quant_mx_1x32": ([P, I32, I64, I64, I64, P, I64, P, I64, P], I32),
        "fp8q_quant_mx_transpose": ([P, I32, I64, I64, I64, P, I64, P, I64, P, I64, P, I64, P], I32),
        "fp8q_gemm_mx": ([P, P, I64, I64, P, P, I64, I64, I64, I64, I64, P, I32, I64, I32, P], I32),
        "fp8q_grouped_gemm_mx": ([P, P, P, P, P, I64, I64, I64, I64, P, I32, I64, P], I32),
        "fp8q_grouped_gemm_mx_dgrad": ([P, P, P, P, P, I64, I64, I64, I64, P, I32, I64, P], I32),
        "fp8q_gemm_fprop_quant": ([P, P, P, P, I64, I64, I64, P, I64, P, I64, P, I64, I32, P], I32),
        "fp8q_gemm_dgrad_quant": ([P, P, P, P, I64, I64, I64, P, I64, P, I64, P, I64, I32, P], I32),
        "fp8q_gemm_fprop_interval": ([P, P, P, P, I64, I64, I64, P, I64, I64, P], I32),
        "fp8q_quant_batch": ([P, I32, P], I32),
    }
    for name in ["fp8q_gemm_fprop", "fp8q_gemm_dgrad", "fp8q_gemm_wgrad", "fp8q_grouped_gemm"]:
        sig[name + "_exact"] = sig[name]
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


def status_string(status):
    return load_library().fp8q_status_string(int(status)).decode()


_TILES = {"auto": 0, "256x128": 1, "256x256": 2}


def set_gemm_tile(tile):
    """Force the GEMMs' workgroup tile ("256x128", "256x256") or give the
    choice back to the library ("auto"); results are bit-identical."""
    _check(load_library().fp8q_set_gemm_tile(_TILES[tile]), "fp8q_set_gemm_tile")


# ----------------------------------------------------------------- marshalling
def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _ld(t):
    """Row stride (elements) of a 2-D tensor whose rows are contiguous."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("expected a 2-D tensor with contiguous rows")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0))


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return FP8Q_BF16
    if t.dtype == torch.float32:
        return FP8Q_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _expect(t, shape, dtype, what):
    """Shape and dtype of an operand the library will read or write through a
    raw pointer: a mismatch would make a kernel run past the allocation, so it
    is refused here (shape entries: an int, None for any, or ("min", n) for at
    least n)."""
    if t is None:
        raise ValueError(f"{what} is required")
    if t.dtype != dtype:
        raise TypeError(f"{what}: dtype {t.dtype}, expected {dtype}")
    if t.dim() != len(shape):
        raise ValueError(f"{what}: {t.dim()}-D, expected {len(shape)}-D {shape}")
    for got, want in zip(t.shape, shape):
        ok = want is None or (got >= want[1] if isinstance(want, tuple) else got == want)
        if not ok:
            raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {shape}")


_U8, _F32 = torch.uint8, torch.float32


def _check(status, name):
    if status != 0:
        raise Fp8qError(status, name)


def _on_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("fp8q works on GPU tensors only")


def fp8q_quant_act_1x128(x, q, scale, stream=None):
    rows, cols = x.shape
    _expect(q, (rows, cols), _U8, "q")
    _expect(scale, (rows, _cdiv(cols, 128)), _F32, "scale")
    _on_gpu(x, q, scale)
    _check(load_library().fp8q_quant_act_1x128(_ptr(x), _dtype_code(x), rows, cols, _ld(x), _ptr(q), _ld(q),
                                                _ptr(scale), _ld(scale), _stream(stream)),
           "fp8q_quant_act_1x128")


def fp8q_quant_weight_128x128(w, q, q_t, scale, stream=None):
    rows, cols = w.shape
    _expect(q, (rows, cols), _U8, "q")
    if q_t is not None:
        _expect(q_t, (cols, rows), _U8, "q_t")
    _expect(scale, (_cdiv(rows, 128), _cdiv(cols, 128)), _F32, "scale")
    _on_gpu(w, q, q_t, scale)
    ld_qt = _ld(q_t) if q_t is not None else 0
    _check(load_library().fp8q_quant_weight_128x128(_ptr(w), _dtype_code(w), rows, cols, _ld(w), _ptr(q),
                                                     _ld(q), _ptr(q_t), ld_qt, _ptr(scale), _ld(scale),
                                                     _stream(stream)),
           "fp8q_quant_weight_128x128")


def fp8q_quant_transpose(x, q_t, scale_t, stream=None):
    rows, cols = x.shape
    _expect(q_t, (cols, rows), _U8, "q_t")
    _expect(scale_t, (cols, _cdiv(rows, 128)), _F32, "scale_t")
    _on_gpu(x, q_t, scale_t)
    _check(load_library().fp8q_quant_transpose(_ptr(x), _dtype_code(x), rows, cols, _ld(x), _ptr(q_t),
                                                _ld(q_t), _ptr(scale_t), _ld(scale_t), _stream(stream)),
           "fp8q_quant_transpose")


def _fn(name, exact):
    return getattr(load_library(), name + ("_exact" if exact else ""))


def _contig(*ts):
    for t in ts:
        if not t.is_contiguous():
            raise ValueError("GEMM operands and scales must be contiguous")


def fp8q_gemm_fprop(xq, xs, wq, ws, y, stream=None, exact=False):
    m, k = xq.shape
    n = wq.shape[0]
    _expect(xq, (m, k), _U8, "xq")
    _expect(xs, (m, _cdiv(k, 128)), _F32, "xs")
    _expect(wq, (n, k), _U8, "wq")
    _expect(ws, (_cdiv(n, 128), _cdiv(k, 128)), _F32, "ws")
    _expect(y, (m, n), y.dtype, "y")
    _on_gpu(xq, xs, wq, ws, y)
    _contig(xq, xs, wq, ws)
    _check(_fn("fp8q_gemm_fprop", exact)(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), m, n, k, _ptr(y),
                                           _dtype_code(y), _ld(y), _stream(stream)),
           "fp8q_gemm_fprop")


def fp8q_gemm_dgrad(dyq, dys, wq_t, ws, dx, stream=None, exact=False):
    m, n = dyq.shape
    k = wq_t.shape[0]
    _expect(dyq, (m, n), _U8, "dyq")
    _expect(dys, (m, _cdiv(n, 128)), _F32, "dys")
    _expect(wq_t, (k, n), _U8, "wq_t")
    _expect(ws, (_cdiv(n, 128), _cdiv(k, 128)), _F32, "ws")
    _expect(dx, (m, k), dx.dtype, "dx")
    _on_gpu(dyq, dys, wq_t, ws, dx)
    _contig(dyq, dys, wq_t, ws)
    _check(_fn("fp8q_gemm_dgrad", exact)(_ptr(dyq), _ptr(dys), _ptr(wq_t), _ptr(ws), m, n, k, _ptr(dx),
                                           _dtype_code(dx), _ld(dx), _stream(stream)),
           "fp8q_gemm_dgrad")


def fp8q_gemm_wgrad(dyq_t, dys_t, xq_t, xs_t, dw, accumulate=False, stream=None, exact=False):
    n, t = dyq_t.shape
    k = xq_t.shape[0]
    _expect(dyq_t, (n, t), _U8, "dyq_t")
    _expect(dys_t, (n, _cdiv(t, 128)), _F32, "dys_t")
    _expect(xq_t, (k, t), _U8, "xq_t")
    _expect(xs_t, (k, _cdiv(t, 128)), _F32, "xs_t")
    _expect(dw, (n, k), _F32, "dw")
    _on_gpu(dyq_t, dys_t, xq_t, xs_t, dw)
    _contig(dyq_t, dys_t, xq_t, xs_t)
    _check(_fn("fp8q_gemm_wgrad", exact)(_ptr(dyq_t), _ptr(dys_t), _ptr(xq_t), _ptr(xs_t), t, n, k, _ptr(dw),
                                           _ld(dw), int(bool(accumulate)), _stream(stream)),
           "fp8q_gemm_wgrad")


def fp8q_gemm_fprop_quant(xq, xs, wq, ws, y, yq, ys, stream=None, exact=False):
    """Fprop with the output's 1x128 quantization in the epilogue: y [M, N]
    BF16 (or None: codes only), yq [M, N] uint8, ys [M, N/128] FP32."""
    m, k = xq.shape
    n = wq.shape[0]
    _expect(xq, (m, k), _U8, "xq")
    _expect(xs, (m, _cdiv(k, 128)), _F32, "xs")
    _expect(wq, (n, k), _U8, "wq")
    _expect(ws, (_cdiv(n, 128), _cdiv(k, 128)), _F32, "ws")
    if y is not None:
        _expect(y, (m, n), torch.bfloat16, "y")
    _expect(yq, (m, n), _U8, "yq")
    _expect(ys, (m, _cdiv(n, 128)), _F32, "ys")
    _on_gpu(xq, xs, wq, ws, y, yq, ys)
    _contig(xq, xs, wq, ws)
    _check(load_library().fp8q_gemm_fprop_quant(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), m, n, k, _ptr(y),
                                                 _ld(y) if y is not None else 0, _ptr(yq), _ld(yq), _ptr(ys),
                                                 _ld(ys), int(bool(exact)), _stream(stream)),
           "fp8q_gemm_fprop_quant")


def fp8q_quant_batch(jobs, stream=None):
    """Several quantizations in one launch.  jobs: a list of
        ("act", x, q, scale)
        ("weight", w, q, q_t, scale)          # q_t may be None
        ("transpose", x, q_t, scale_t)
        ("act_transpose", x, q, scale, q_t, scale_t)
    with the tensors of the single entry points (same shape rules)."""
    if len(jobs) > MAX_QUANT_JOBS:
        raise ValueError(f"at most {MAX_QUANT_JOBS} jobs per batch")
    arr = (QuantJob * max(1, len(jobs)))()
    for i, job in enumerate(jobs):
        kind, x = job[0], job[1]
        rows, cols = x.shape
        q = scale = q_t = scale_t = None
        if kind == "act":
            q, scale = job[2:]
        elif kind == "weight":
            q, q_t, scale = job[2:]
        elif kind == "transpose":
            q_t, scale_t = job[2:]
        elif kind == "act_transpose":
            q, scale, q_t, scale_t = job[2:]
        else:
            raise ValueError(f"unknown quantization kind {kind!r}")
        if q is not None:
            _expect(q, (rows, cols), _U8, f"job {i} q")
        if scale is not None:
            gr = (_cdiv(rows, 128), _cdiv(cols, 128)) if kind == "weight" else (rows, _cdiv(cols, 128))
            _expect(scale, gr, _F32, f"job {i} scale")
        if q_t is not None:
            _expect(q_t, (cols, rows), _U8, f"job {i} q_t")
        if scale_t is not None:
            _expect(scale_t, (cols, _cdiv(rows, 128)), _F32, f"job {i} scale_t")
        _on_gpu(x, q, scale, q_t, scale_t)
        j = arr[i]
        j.kind, j.xt, j.x, j.rows, j.cols, j.ld_x = QUANT_KINDS[kind], _dtype_code(x), _ptr(x), rows, cols, _ld(x)
        if q is not None:
            j.q, j.ld_q, j.scale, j.ld_s = _ptr(q), _ld(q), _ptr(scale), _ld(scale)
        if q_t is not None:
            j.q_t, j.ld_qt = _ptr(q_t), _ld(q_t)
        if scale_t is not None:
            j.scale_t, j.ld_st = _ptr(scale_t), _ld(scale_t)
    _check(load_library().fp8q_quant_batch(ctypes.cast(arr, ctypes.c_void_p), len(jobs), _stream(stream)),
           "fp8q_quant_batch")


def fp8q_gemm_fprop_interval(xq, xs, wq, ws, y, interval, stream=None):
    """The promotion-interval study: Fprop into FP32 y [M, N] with partials
    chained through the matrix instruction over `interval` K (128, 256, 512,
    1024; 0 = all of K); scales must be constant over each interval."""
    m, k = xq.shape
    n = wq.shape[0]
    _expect(xq, (m, k), _U8, "xq")
    _expect(xs, (m, _cdiv(k, 128)), _F32, "xs")
    _expect(wq, (n, k), _U8, "wq")
    _expect(ws, (_cdiv(n, 128), _cdiv(k, 128)), _F32, "ws")
    _expect(y, (m, n), _F32, "y")
    _on_gpu(xq, xs, wq, ws, y)
    _contig(xq, xs, wq, ws)
    _check(load_library().fp8q_gemm_fprop_interval(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), m, n, k, _ptr(y),
                                                    _ld(y), int(interval), _stream(stream)),
           "fp8q_gemm_fprop_interval")


def fp8q_gemm_dgrad_quant(dyq, dys, wq_t, ws, dx, dxq, dxs, stream=None, exact=False):
    """Dgrad with the output's 1x128 quantization in the epilogue: dx [M, K]
    BF16 (or None: codes only), dxq [M, K] uint8, dxs [M, K/128] FP32."""
    m, n = dyq.shape
    k = wq_t.shape[0]
    _expect(dyq, (m, n), _U8, "dyq")
    _expect(dys, (m, _cdiv(n, 128)), _F32, "dys")
    _expect(wq_t, (k, n), _U8, "wq_t")
    _expect(ws, (_cdiv(n, 128), _cdiv(k, 128)), _F32, "ws")
    if dx is not None:
        _expect(dx, (m, k), torch.bfloat16, "dx")
    _expect(dxq, (m, k), _U8, "dxq")
    _expect(dxs, (m, _cdiv(k, 128)), _F32, "dxs")
    _on_gpu(dyq, dys, wq_t, ws, dx, dxq, dxs)
    _contig(dyq, dys, wq_t, ws)
    _check(load_library().fp8q_gemm_dgrad_quant(_ptr(dyq), _ptr(dys), _ptr(wq_t), _ptr(ws), m, n, k, _ptr(dx),
                                                 _ld(dx) if dx is not None else 0, _ptr(dxq), _ld(dxq), _ptr(dxs),
                                                 _ld(dxs), int(bool(exact)), _stream(stream)),
           "fp8q_gemm_dgrad_quant")


def fp8q_grouped_gemm(xq, xs, wq, ws, offsets, y, stream=None, exact=False):
    m_total, k = xq.shape
    e, n, _ = wq.shape
    _expect(xq, (m_total, k), _U8, "xq")
    _expect(xs, (m_total, _cdiv(k, 128)), _F32, "xs")
    _expect(wq, (e, n, k), _U8, "wq")
    _expect(ws, (e, _cdiv(n, 128), _cdiv(k, 128)), _F32, "ws")
    _expect(offsets, (e + 1,), torch.int32, "offsets")
    _expect(y, (m_total, n), y.dtype, "y")
    _on_gpu(xq, xs, wq, ws, offsets, y)
    _contig(xq, xs, wq, ws, offsets)
    _check(_fn("fp8q_grouped_gemm", exact)(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(offsets), e, m_total,
                                             n, k, _ptr(y), _dtype_code(y), _ld(y), _stream(stream)),
           "fp8q_grouped_gemm")


def fp8q_quant_act_transpose(x, q, scale, q_t, scale_t, stream=None):
    rows, cols = x.shape
    _expect(q, (rows, cols), _U8, "q")
    _expect(scale, (rows, _cdiv(cols, 128)), _F32, "scale")
    _expect(q_t, (cols, rows), _U8, "q_t")
    _expect(scale_t, (cols, _cdiv(rows, 128)), _F32, "scale_t")
    _on_gpu(x, q, scale, q_t, scale_t)
    _check(load_library().fp8q_quant_act_transpose(_ptr(x), _dtype_code(x), rows, cols, _ld(x), _ptr(q), _ld(q),
                                                    _ptr(scale), _ld(scale), _ptr(q_t), _ld(q_t), _ptr(scale_t),
                                                    _ld(scale_t), _stream(stream)),
           "fp8q_quant_act_transpose")


def fp8q_quant_transpose_grouped(x, offsets, q_t, scale_t, stream=None):
    rows, cols = x.shape
    e = offsets.shape[0] - 1
    cap = token_capacity(rows, e)
    _expect(offsets, (e + 1,), torch.int32, "offsets")
    _expect(q_t, (cols, ("min", cap)), _U8, "q_t")
    _expect(scale_t, (cols, ("min", cap // 128)), _F32, "scale_t")
    _on_gpu(x, offsets, q_t, scale_t)
    _contig(offsets)
    _check(load_library().fp8q_quant_transpose_grouped(_ptr(x), _dtype_code(x), rows, cols, _ld(x),
                                                        _ptr(offsets), e, _ptr(q_t), _ld(q_t), _ptr(scale_t),
                                                        _ld(scale_t), _stream(stream)),
           "fp8q_quant_transpose_grouped")


def fp8q_grouped_gemm_dgrad(dyq, dys, wq_t, ws, offsets, dx, stream=None):
    """wq_t [K, E*N], ws [E*N/128, K/128] (quant_weight_128x128 of the stacked
    weights [E*N, K])."""
    m_total, n = dyq.shape
    k = wq_t.shape[0]
    e = offsets.shape[0] - 1
    _expect(offsets, (e + 1,), torch.int32, "offsets")
    _expect(dyq, (m_total, n), _U8, "dyq")
    _expect(dys, (m_total, _cdiv(n, 128)), _F32, "dys")
    _expect(wq_t, (k, e * n), _U8, "wq_t")
    _expect(ws, (_cdiv(e * n, 128), _cdiv(k, 128)), _F32, "ws")
    _expect(dx, (m_total, k), dx.dtype, "dx")
    _on_gpu(dyq, dys, wq_t, ws, offsets, dx)
    _contig(dyq, dys, wq_t, ws, offsets)
    _check(load_library().fp8q_grouped_gemm_dgrad(_ptr(dyq), _ptr(dys), _ptr(wq_t), _ptr(ws), _ptr(offsets), e,
                                                   m_total, n, k, _ptr(dx), _dtype_code(dx), _ld(dx),
                                                   _stream(stream)),
           "fp8q_grouped_gemm_dgrad")


def fp8q_grouped_gemm_wgrad(dyq_t, dys_t, xq_t, xs_t, offsets, m_total, dw, accumulate=False, stream=None):
    """Token-padded operands [N, ld_t] / [K, ld_t] (quant_transpose_grouped);
    dw [E, N, K] FP32 contiguous."""
    n, ld_t = dyq_t.shape
    k = xq_t.shape[0]
    e = offsets.shape[0] - 1
    _expect(offsets, (e + 1,), torch.int32, "offsets")
    _expect(dyq_t, (n, ld_t), _U8, "dyq_t")
    _expect(dys_t, (n, ld_t // 128), _F32, "dys_t")
    _expect(xq_t, (k, ld_t), _U8, "xq_t")
    _expect(xs_t, (k, ld_t // 128), _F32, "xs_t")
    _expect(dw, (e, n, k), _F32, "dw")
    if ld_t % 128 != 0:
        raise ValueError("the padded token stride is a multiple of 128")
    _on_gpu(dyq_t, dys_t, xq_t, xs_t, offsets, dw)
    _contig(dyq_t, dys_t, xq_t, xs_t, offsets, dw)
    _check(load_library().fp8q_grouped_gemm_wgrad(_ptr(dyq_t), _ptr(dys_t), _ptr(xq_t), _ptr(xs_t), _ptr(offsets),
                                                   e, m_total, n, k, ld_t, _ptr(dw), int(bool(accumulate)),
                                                   _stream(stream)),
           "fp8q_grouped_gemm_wgrad")


def fp8q_quant_mx_1x32(x, q, s, stream=None):
    rows, cols = x.shape
    _expect(q, (rows, cols), _U8, "q")
    _expect(s, (rows, _cdiv(cols, 32)), _U8, "s")
    _on_gpu(x, q, s)
    _check(load_library().fp8q_quant_mx_1x32(_ptr(x), _dtype_code(x), rows, cols, _ld(x), _ptr(q), _ld(q),
                                              _ptr(s), _ld(s), _stream(stream)),
           "fp8q_quant_mx_1x32")


def fp8q_quant_mx_transpose(x, q_t, s_t, q=None, s=None, stream=None):
    rows, cols = x.shape
    _expect(q_t, (cols, rows), _U8, "q_t")
    _expect(s_t, (cols, _cdiv(rows, 32)), _U8, "s_t")
    if q is not None or s is not None:
        _expect(q, (rows, cols), _U8, "q")
        _expect(s, (rows, _cdiv(cols, 32)), _U8, "s")
    _on_gpu(x, q_t, s_t, q, s)
    ldq = _ld(q) if q is not None else 0
    lds = _ld(s) if s is not None else 0
    _check(load_library().fp8q_quant_mx_transpose(_ptr(x), _dtype_code(x), rows, cols, _ld(x), _ptr(q_t),
                                                   _ld(q_t), _ptr(s_t), _ld(s_t), _ptr(q), ldq, _ptr(s), lds,
                                                   _stream(stream)),
           "fp8q_quant_mx_transpose")


def fp8q_gemm_mx(aq, as_, bq, bs, c, accumulate=False, stream=None):
    """C [M, N] (= or +=) A . B^T; aq [M, K], as_ [M, >= K/32], bq [N, K],
    bs [N, >= K/32] (uint8 codes and E8M0 bytes, rows may be padded)."""
    m, k = aq.shape
    n = bq.shape[0]
    _expect(aq, (m, k), _U8, "aq")
    _expect(as_, (m, ("min", _cdiv(k, 32))), _U8, "as_")
    _expect(bq, (n, k), _U8, "bq")
    _expect(bs, (n, ("min", _cdiv(k, 32))), _U8, "bs")
    _expect(c, (m, n), c.dtype, "c")
    _on_gpu(aq, as_, bq, bs, c)
    _check(load_library().fp8q_gemm_mx(_ptr(aq), _ptr(as_), _ld(aq), _ld(as_), _ptr(bq), _ptr(bs), _ld(bq),
                                        _ld(bs), m, n, k, _ptr(c), _dtype_code(c), _ld(c), int(bool(accumulate)),
                                        _stream(stream)),
           "fp8q_gemm_mx")


def fp8q_grouped_gemm_mx(xq, xs, wq, ws, offsets, y, stream=None):
    """Y [M_total, N] = per expert X rows . W_e^T; xq [M_total, K], xs [M_total, K/32],
    wq [E, N, K], ws [E, N, K/32] (uint8 codes and E8M0 bytes, contiguous)."""
    m_total, k = xq.shape
    e, n, _ = wq.shape
    _expect(xq, (m_total, k), _U8, "xq")
    _expect(xs, (m_total, _cdiv(k, 32)), _U8, "xs")
    _expect(wq, (e, n, k), _U8, "wq")
    _expect(ws, (e, n, _cdiv(k, 32)), _U8, "ws")
    _expect(offsets, (e + 1,), torch.int32, "offsets")
    _expect(y, (m_total, n), y.dtype, "y")
    _on_gpu(xq, xs, wq, ws, offsets, y)
    _contig(xq, xs, wq, ws, offsets)
    _check(load_library().fp8q_grouped_gemm_mx(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(offsets), e, m_total,
                                                n, k, _ptr(y), _dtype_code(y), _ld(y), _stream(stream)),
           "fp8q_grouped_gemm_mx")


def fp8q_grouped_gemm_mx_dgrad(dyq, dys, wq_t, ws_t, offsets, dx, stream=None):
    """dX [M_total, K] = per expert dY rows . W_e; dyq [M_total, N], dys [M_total, N/32],
    wq_t [K, E*N], ws_t [K, E*N/32] (quant_mx_transpose of the stacked weights [E*N, K])."""
    m_total, n = dyq.shape
    k = wq_t.shape[0]
    e = offsets.shape[0] - 1
    _expect(offsets, (e + 1,), torch.int32, "offsets")
    _expect(dyq, (m_total, n), _U8, "dyq")
    _expect(dys, (m_total, _cdiv(n, 32)), _U8, "dys")
    _expect(wq_t, (k, e * n), _U8, "wq_t")
    _expect(ws_t, (k, _cdiv(e * n, 32)), _U8, "ws_t")
    _expect(dx, (m_total, k), dx.dtype, "dx")
    _on_gpu(dyq, dys, wq_t, ws_t, offsets, dx)
    _contig(dyq, dys, wq_t, ws_t, offsets)
    _check(load_library().fp8q_grouped_gemm_mx_dgrad(_ptr(dyq), _ptr(dys), _ptr(wq_t), _ptr(ws_t), _ptr(offsets), e,
                                                      m_total, n, k, _ptr(dx), _dtype_code(dx), _ld(dx),
                                                      _stream(stream)),
           "fp8q_grouped_gemm_mx_dgrad")


# ---------------------------------------------------------------- convenience
def _cdiv(a, b):
    return (a + b - 1) // b


def quant_act_1x128(x, stream=None):
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    s = torch.empty((rows, _cdiv(cols, 128)), dtype=torch.float32, device=x.device)
    fp8q_quant_act_1x128(x, q, s, stream)
    return q, s


def quant_weight_128x128(w, transpose=True, stream=None):
    rows, cols = w.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=w.device)
    q_t = torch.empty((cols, rows), dtype=torch.uint8, device=w.device) if transpose else None
    s = torch.empty((_cdiv(rows, 128), _cdiv(cols, 128)), dtype=torch.float32, device=w.device)
    fp8q_quant_weight_128x128(w, q, q_t, s, stream)
    return q, s, q_t


def quant_transpose(x, stream=None):
    rows, cols = x.shape
    q_t = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    s_t = torch.empty((cols, _cdiv(rows, 128)), dtype=torch.float32, device=x.device)
    fp8q_quant_transpose(x, q_t, s_t, stream)
    return q_t, s_t


def gemm_fprop(xq, xs, wq, ws, out_dtype=torch.bfloat16, stream=None, exact=False):
    y = torch.empty((xq.shape[0], wq.shape[0]), dtype=out_dtype, device=xq.device)
    fp8q_gemm_fprop(xq, xs, wq, ws, y, stream, exact)
    return y


def gemm_fprop_quant(xq, xs, wq, ws, with_output=True, stream=None, exact=False):
    """Fprop with fused output quantization: (y BF16 or None, yq, ys)."""
    m, n = xq.shape[0], wq.shape[0]
    y = torch.empty((m, n), dtype=torch.bfloat16, device=xq.device) if with_output else None
    yq = torch.empty((m, n), dtype=torch.uint8, device=xq.device)
    ys = torch.empty((m, _cdiv(n, 128)), dtype=torch.float32, device=xq.device)
    fp8q_gemm_fprop_quant(xq, xs, wq, ws, y, yq, ys, stream, exact)
    return y, yq, ys


def gemm_dgrad_quant(dyq, dys, wq_t, ws, with_output=True, stream=None, exact=False):
    """Dgrad with fused output quantization: (dx BF16 or None, dxq, dxs)."""
    m, k = dyq.shape[0], wq_t.shape[0]
    dx = torch.empty((m, k), dtype=torch.bfloat16, device=dyq.device) if with_output else None
    dxq = torch.empty((m, k), dtype=torch.uint8, device=dyq.device)
    dxs = torch.empty((m, _cdiv(k, 128)), dtype=torch.float32, device=dyq.device)
    fp8q_gemm_dgrad_quant(dyq, dys, wq_t, ws, dx, dxq, dxs, stream, exact)
    return dx, dxq, dxs


def gemm_dgrad(dyq, dys, wq_t, ws, out_dtype=torch.bfloat16, stream=None, exact=False):
    dx = torch.empty((dyq.shape[0], wq_t.shape[0]), dtype=out_dtype, device=dyq.device)
    fp8q_gemm_dgrad(dyq, dys, wq_t, ws, dx, stream, exact)
    return dx


def gemm_wgrad(dyq_t, dys_t, xq_t, xs_t, dw=None, stream=None, exact=False):
    accumulate = dw is not None
    if dw is None:
        dw = torch.empty((dyq_t.shape[0], xq_t.shape[0]), dtype=torch.float32, device=dyq_t.device)
    fp8q_gemm_wgrad(dyq_t, dys_t, xq_t, xs_t, dw, accumulate, stream, exact)
    return dw


def grouped_gemm(xq, xs, wq, ws, offsets, out_dtype=torch.bfloat16, stream=None, exact=False):
    y = torch.empty((xq.shape[0], wq.shape[1]), dtype=out_dtype, device=xq.device)
    fp8q_grouped_gemm(xq, xs, wq, ws, offsets, y, stream, exact)
    return y


def token_capacity(m_total, experts):
    """Padded token capacity of the grouped weight-gradient operands."""
    return 128 * (m_total // 128 + experts)


def quant_transpose_grouped(x, offsets, stream=None):
    rows, cols = x.shape
    cap = token_capacity(rows, offsets.shape[0] - 1)
    q_t = torch.zeros((cols, cap), dtype=torch.uint8, device=x.device)
    s_t = torch.zeros((cols, cap // 128), dtype=torch.float32, device=x.device)
    fp8q_quant_transpose_grouped(x, offsets, q_t, s_t, stream)
    return q_t, s_t


def grouped_gemm_dgrad(dyq, dys, wq_t, ws, offsets, out_dtype=torch.bfloat16, stream=None):
    dx = torch.empty((dyq.shape[0], wq_t.shape[0]), dtype=out_dtype, device=dyq.device)
    fp8q_grouped_gemm_dgrad(dyq, dys, wq_t, ws, offsets, dx, stream)
    return dx


def grouped_gemm_wgrad(dyq_t, dys_t, xq_t, xs_t, offsets, m_total, dw=None, stream=None):
    accumulate = dw is not None
    if dw is None:
        dw = torch.empty((offsets.shape[0] - 1, dyq_t.shape[0], xq_t.shape[0]), dtype=torch.float32,
                         device=dyq_t.device)
    fp8q_grouped_gemm_wgrad(dyq_t, dys_t, xq_t, xs_t, offsets, m_total, dw, accumulate, stream)
    return dw


def quant_act_transpose(x, stream=None):
    """Both quantizations of x from one read: (q, s, q_t, s_t)."""
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    s = torch.empty((rows, _cdiv(cols, 128)), dtype=torch.float32, device=x.device)
    q_t = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    s_t = torch.empty((cols, _cdiv(rows, 128)), dtype=torch.float32, device=x.device)
    fp8q_quant_act_transpose(x, q, s, q_t, s_t, stream)
    return q, s, q_t, s_t


def quant_mx(x, stream=None):
    """MXFP8 along rows: (q [rows, cols], s [rows, ceil(cols/32)] E8M0 bytes)."""
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    s = torch.empty((rows, _cdiv(cols, 32)), dtype=torch.uint8, device=x.device)
    fp8q_quant_mx_1x32(x, q, s, stream)
    return q, s


def quant_mx_transpose(x, dual=False, stream=None):
    """MXFP8 along columns, transposed: (q_t, s_t), or with dual=True
    (q, s, q_t, s_t) from one read of x."""
    rows, cols = x.shape
    q_t = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    s_t = torch.empty((cols, _cdiv(rows, 32)), dtype=torch.uint8, device=x.device)
    if not dual:
        fp8q_quant_mx_transpose(x, q_t, s_t, stream=stream)
        return q_t, s_t
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    s = torch.empty((rows, _cdiv(cols, 32)), dtype=torch.uint8, device=x.device)
    fp8q_quant_mx_transpose(x, q_t, s_t, q, s, stream=stream)
    return q, s, q_t, s_t


def gemm_mx(aq, as_, bq, bs, out_dtype=torch.bfloat16, c=None, stream=None):
    """A . B^T of MX operands; with c given (FP32), adds into it."""
    accumulate = c is not None
    if c is None:
        c = torch.empty((aq.shape[0], bq.shape[0]), dtype=out_dtype, device=aq.device)
    fp8q_gemm_mx(aq, as_, bq, bs, c, accumulate, stream)
    return c


def grouped_gemm_mx(xq, xs, wq, ws, offsets, out_dtype=torch.bfloat16, stream=None):
    """Grouped (MoE) MX Fprop: rows [o_e, o_{e+1}) of the output are X[o_e:o_{e+1}] . W_e^T."""
    y = torch.empty((xq.shape[0], wq.shape[1]), dtype=out_dtype, device=xq.device)
    fp8q_grouped_gemm_mx(xq, xs, wq, ws, offsets, y, stream)
    return y


def grouped_gemm_mx_dgrad(dyq, dys, wq_t, ws_t, offsets, out_dtype=torch.bfloat16, stream=None):
    """Grouped (MoE) MX Dgrad: rows [o_e, o_{e+1}) of dX are dY[o_e:o_{e+1}] . W_e."""
    dx = torch.empty((dyq.shape[0], wq_t.shape[0]), dtype=out_dtype, device=dyq.device)
    fp8q_grouped_gemm_mx_dgrad(dyq, dys, wq_t, ws_t, offsets, dx, stream)
    return dx
