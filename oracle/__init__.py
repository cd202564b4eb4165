"""CPU oracle for the block-scale quantiser: numpy wrappers over liboracle.so.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the GPU library (``block_scaled_precision_hdiag_amd``) and never imports it.

Arrays are numpy: float32 tensors as ``np.float32``; bfloat16 tensors as their
raw bits in ``np.uint16``.  What each function computes, and the passages it
follows, is documented in ``oracle.c``.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")

NAIVE, SSE_OPT, H_OPT, NAIVE_OCP = 0, 1, 2, 3
INT8_E4M3, NVFP4, MXFP4, MXFP8, FP8_E4M3S = 0, 1, 2, 3, 4
NVFP4_UE4M4, NVFP4_UE5M3, NVINT4 = 5, 6, 7
FP4_F16, INT4_F16 = 8, 9
FOUR_BIT = (NVFP4, MXFP4, NVFP4_UE4M4, NVFP4_UE5M3, NVINT4, FP4_F16, INT4_F16)
F16_SCALES = (FP4_F16, INT4_F16)
F32, BF16 = 0, 1

FORMAT_NAMES = {INT8_E4M3: "INT8_E4M3", NVFP4: "NVFP4", MXFP4: "MXFP4",
                MXFP8: "MXFP8", FP8_E4M3S: "FP8_E4M3S", NVFP4_UE4M4: "NVFP4_UE4M4",
                NVFP4_UE5M3: "NVFP4_UE5M3", NVINT4: "NVINT4", FP4_F16: "FP4_F16",
                INT4_F16: "INT4_F16"}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from oracle import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.orc_fp_table.argtypes = [i32, i32, i32, i32, P, i32]
        L.orc_e8m0_table.argtypes = [P, i32]
        L.orc_rne_index.argtypes = [P, i32, dbl]
        L.orc_rne_index_batch.argtypes = [P, i32, P, i64, P]
        L.orc_rne_index_batch.restype = None
        L.orc_candidates.argtypes = [i32, P, P]
        L.orc_scale_value.argtypes = [i32, i32]
        L.orc_scale_value.restype = ctypes.c_float
        L.orc_naive_scale_code.argtypes = [i32, ctypes.c_float]
        L.orc_naive_ocp_code.argtypes = [i32, ctypes.c_float]
        L.orc_f16_code.argtypes = [dbl]
        L.orc_block_all_objectives.argtypes = [i32, i32, P, P, P, P]
        L.orc_quantize.argtypes = [i32, i32, i32, P, i32, i64, i64, P, P, P, P, P, i32]
        L.orc_dequantize.argtypes = [i32, i32, P, P, i64, i64, P, i32]
        L.orc_objectives_at.argtypes = [i32, i32, P, i32, i64, i64, P, P, P, i32]
        L.orc_hdiag.argtypes = [P, i32, i64, i64, P, i32]
        L.orc_weight_error.argtypes = [P, i32, P, i32, i64, i64, P, P, i32]
        L.orc_weight_error.restype = dbl
        L.orc_output_error.argtypes = [P, i32, i64, P, i32, P, i32, i64, i64, P, P, i32]
        L.orc_output_error.restype = dbl
        L.orc_matmul_nt.argtypes = [P, i32, i64, P, i32, i64, i64, P, i32]
        L.orc_matmul_nt.restype = None
        L.orc_xtx.argtypes = [P, i32, i64, i64, P, i32]
        L.orc_tensor_scale.argtypes = [i32, P, i32, i64]
        L.orc_tensor_scale.restype = ctypes.c_float
        L.orc_quantize_tensor_scaled.argtypes = [i32, i32, i32, P, i32, i64, i64, P, P, P, P, P, i32]
        L.orc_dequantize_tensor_scaled.argtypes = [i32, i32, P, P, ctypes.c_float, i64, i64, P, i32]
        L.orc_gptq.argtypes = [i32, i32, i32, P, i32, i64, i64, P, dbl, i32, P, P, P, i32]
        L.orc_gptq_emulated.argtypes = [i32, i32, i32, P, i32, i64, i64, P, dbl, i32, P, P, P, i32, i32]
        L.orc_max_threads.argtypes = []
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dt(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("oracle inputs are float32 or bfloat16 bits (uint16), got %s" % a.dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s failed with status %d" % (what, rc))


def max_threads():
    return int(lib().orc_max_threads())


def fp_table(ebits, mbits, bias, reserve):
    """Non-negative values of an EeMm format in code order (see oracle.c)."""
    out = np.zeros(1 << (ebits + mbits), np.float64)
    n = lib().orc_fp_table(ebits, mbits, bias, reserve, _ptr(out), out.size)
    _check(0 if n > 0 else n, "fp_table")
    return out[:n].copy()


def e8m0_table():
    out = np.zeros(255, np.float64)
    lib().orc_e8m0_table(_ptr(out), 255)
    return out


def rne_index(table, x):
    """Index of the table entry x rounds to (x >= 0; array or scalar)."""
    T = np.ascontiguousarray(table, np.float64)
    xs = np.ascontiguousarray(np.atleast_1d(x), np.float32)
    out = np.zeros(xs.size, np.int32)
    lib().orc_rne_index_batch(_ptr(T), T.size, _ptr(xs), xs.size, _ptr(out))
    return out if np.ndim(x) else int(out[0])


def candidates(fmt):
    a, b = ctypes.c_int(), ctypes.c_int()
    _check(0 if lib().orc_candidates(fmt, ctypes.byref(a), ctypes.byref(b)) > 0 else -1, "candidates")
    return np.arange(a.value, b.value + 1)


def scale_value(fmt, code):
    return np.float32(lib().orc_scale_value(fmt, int(code)))


def naive_scale_code(fmt, amax):
    return int(lib().orc_naive_scale_code(fmt, float(np.float32(amax))))


def naive_ocp_code(fmt, amax):
    """OCP MX rule 2^(floor(log2 amax) - emax) as an E8M0 code (-1: not an E8M0 format)."""
    return int(lib().orc_naive_ocp_code(fmt, float(np.float32(amax))))


def f16_code(v):
    """Binary16 bit pattern of v >= 0 by the oracle's table rounding (RNE,
    saturating at 65504)."""
    return int(lib().orc_f16_code(float(v)))


def scale_dtype(fmt):
    """Scale codes are one byte, or binary16 bits (uint16) for FP16 scales."""
    return np.uint16 if fmt in F16_SCALES else np.uint8


def block_all_objectives(fmt, w, h=None):
    """(codes, objectives) of one block over every candidate scale."""
    w = np.ascontiguousarray(w, np.float32)
    hh = None if h is None else np.ascontiguousarray(h, np.float32)
    n = candidates(fmt).size
    obj = np.zeros(n, np.float64)
    codes = np.zeros(n, np.int32)
    rc = lib().orc_block_all_objectives(fmt, w.size, _ptr(w), _ptr(hh), _ptr(obj), _ptr(codes))
    _check(0 if rc > 0 else rc, "block_all_objectives")
    return codes, obj


def codes_shape(fmt, N, K):
    return (N, K // 2) if fmt in FOUR_BIT else (N, K)


def quantize(method, fmt, B, W, h=None, scales_in=None, nthreads=0):
    """Returns (codes uint8, scales [N, K/B] (uint8, or uint16 for FP16 scales),
    block objective float64 [N, K/B])."""
    W = np.ascontiguousarray(W)
    N, K = W.shape
    codes = np.zeros(codes_shape(fmt, N, K), np.uint8)
    scales = np.zeros((N, K // B), scale_dtype(fmt))
    obj = np.zeros((N, K // B), np.float64)
    hh = None if h is None else np.ascontiguousarray(h, np.float32)
    si = None if scales_in is None else np.ascontiguousarray(scales_in, scale_dtype(fmt))
    rc = lib().orc_quantize(method, fmt, B, _ptr(W), _dt(W), N, K, _ptr(hh), _ptr(si),
                            _ptr(codes), _ptr(scales), _ptr(obj), nthreads)
    _check(rc, "quantize")
    return codes, scales, obj


def objectives_at(fmt, B, W, scales_in, h=None, nthreads=0):
    """Per-block objective of W encoded at the given scale codes."""
    W = np.ascontiguousarray(W)
    N, K = W.shape
    obj = np.zeros((N, K // B), np.float64)
    hh = None if h is None else np.ascontiguousarray(h, np.float32)
    si = np.ascontiguousarray(scales_in, scale_dtype(fmt))
    rc = lib().orc_objectives_at(fmt, B, _ptr(W), _dt(W), N, K, _ptr(hh), _ptr(si), _ptr(obj), nthreads)
    _check(rc, "objectives_at")
    return obj


def dequantize(fmt, B, codes, scales, N, K, nthreads=0):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, scale_dtype(fmt))
    out = np.zeros((N, K), np.float32)
    rc = lib().orc_dequantize(fmt, B, _ptr(codes), _ptr(scales), N, K, _ptr(out), nthreads)
    _check(rc, "dequantize")
    return out


def hdiag(X, nthreads=0):
    X = np.ascontiguousarray(X)
    M, K = X.shape
    h = np.zeros(K, np.float32)
    _check(lib().orc_hdiag(_ptr(X), _dt(X), M, K, _ptr(h), nthreads), "hdiag")
    return h


def weight_error(W, Wq, nthreads=0, sums=False):
    W = np.ascontiguousarray(W)
    Wq = np.ascontiguousarray(Wq)
    N, K = W.shape
    a, b = ctypes.c_double(), ctypes.c_double()
    r = lib().orc_weight_error(_ptr(W), _dt(W), _ptr(Wq), _dt(Wq), N, K,
                               ctypes.byref(a), ctypes.byref(b), nthreads)
    return (r, a.value, b.value) if sums else r


def matmul_nt(X, W, nthreads=0):
    """Y = X W^T in float64 ([M, N]), each entry summed in k order."""
    X = np.ascontiguousarray(X)
    W = np.ascontiguousarray(W)
    M, K = X.shape
    N = W.shape[0]
    Y = np.empty((M, N), dtype=np.float64)
    lib().orc_matmul_nt(_ptr(X), _dt(X), M, _ptr(W), _dt(W), N, K, _ptr(Y), nthreads)
    return Y


def output_error(X, W, Wq, nthreads=0, sums=False):
    X = np.ascontiguousarray(X)
    W = np.ascontiguousarray(W)
    Wq = np.ascontiguousarray(Wq)
    M, K = X.shape
    N = W.shape[0]
    d, y = ctypes.c_double(), ctypes.c_double()
    r = lib().orc_output_error(_ptr(X), _dt(X), M, _ptr(W), _dt(W), _ptr(Wq), _dt(Wq), N, K,
                               ctypes.byref(d), ctypes.byref(y), nthreads)
    return (r, d.value, y.value) if sums else r


def xtx(X, nthreads=0):
    """H = X^T X in float64 ([K, K])."""
    X = np.ascontiguousarray(X)
    M, K = X.shape
    H = np.empty((K, K), dtype=np.float64)
    _check(lib().orc_xtx(_ptr(X), _dt(X), M, K, _ptr(H), nthreads), "xtx")
    return H


def gptq(method, fmt, B, W, H, damp=0.01, ordered=False, nthreads=0):
    """GPTQ-Seq (ordered=False) or GPTQ-Ord on top of `method`'s scale choice,
    given H = X^T X.  Returns (codes, scales, block_order) like quantize."""
    W = np.ascontiguousarray(W)
    N, K = W.shape
    H = np.ascontiguousarray(H, np.float64)
    codes = np.zeros(codes_shape(fmt, N, K), np.uint8)
    scales = np.zeros((N, K // B), scale_dtype(fmt))
    order = np.zeros(K // B, np.int32)
    rc = lib().orc_gptq(method, fmt, B, _ptr(W), _dt(W), N, K, _ptr(H), float(damp), int(bool(ordered)),
                        _ptr(codes), _ptr(scales), _ptr(order), nthreads)
    _check(rc, "gptq")
    return codes, scales, order


# precision experiment flags of gptq_emulated (see oracle.c)
GPTQ_EMUL_H32, GPTQ_EMUL_U32, GPTQ_EMUL_W32, GPTQ_EMUL_HULP = 1, 2, 4, 8


def gptq_emulated(method, fmt, B, W, H, emul, damp=0.01, ordered=False, nthreads=0):
    """gptq() with selected quantities rounded to float32 or perturbed by one
    float64 ulp (flags above): a precision experiment, not a reference."""
    W = np.ascontiguousarray(W)
    N, K = W.shape
    H = np.ascontiguousarray(H, np.float64)
    codes = np.zeros(codes_shape(fmt, N, K), np.uint8)
    scales = np.zeros((N, K // B), scale_dtype(fmt))
    order = np.zeros(K // B, np.int32)
    rc = lib().orc_gptq_emulated(method, fmt, B, _ptr(W), _dt(W), N, K, _ptr(H), float(damp), int(bool(ordered)),
                                 _ptr(codes), _ptr(scales), _ptr(order), nthreads, int(emul))
    _check(rc, "gptq_emulated")
    return codes, scales, order


def quantize_tensor_scaled(method, fmt, B, W, h=None, nthreads=0):
    """Per-tensor scale + E4M3 block scales (see oracle.c).  Returns (codes,
    scales, tensor_scale float32, block objective of W / tensor_scale)."""
    W = np.ascontiguousarray(W)
    N, K = W.shape
    codes = np.zeros(codes_shape(fmt, N, K), np.uint8)
    scales = np.zeros((N, K // B), np.uint8)
    obj = np.zeros((N, K // B), np.float64)
    st = ctypes.c_float()
    hh = None if h is None else np.ascontiguousarray(h, np.float32)
    rc = lib().orc_quantize_tensor_scaled(method, fmt, B, _ptr(W), _dt(W), N, K, _ptr(hh), _ptr(codes), _ptr(scales),
                                          ctypes.byref(st), _ptr(obj), nthreads)
    _check(rc, "quantize_tensor_scaled")
    return codes, scales, np.float32(st.value), obj


def dequantize_tensor_scaled(fmt, B, codes, scales, tensor_scale, N, K, nthreads=0):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    out = np.zeros((N, K), np.float32)
    rc = lib().orc_dequantize_tensor_scaled(fmt, B, _ptr(codes), _ptr(scales), float(np.float32(tensor_scale)), N, K,
                                            _ptr(out), nthreads)
    _check(rc, "dequantize_tensor_scaled")
    return out

