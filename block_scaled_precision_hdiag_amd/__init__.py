"""MI355X (gfx950) block-scale quantiser: a thin Python binding of libhdiag.so.

Every function here only marshals arguments (device pointers of torch tensors,
sizes, the current HIP stream) to the C ABI declared in ``include/hdiag.h``;
all arithmetic runs in the library's HIP kernels.  torch supplies device memory
and streams.  If the library has not been built the binding raises instead of
computing anything some other way: build it with
``python block_scaled_precision_hdiag_amd/build.py`` (or ``__graft_entry__.build()``).

Names follow the C ABI: ``hdiag``, ``quantize_blocks``, ``encode_blocks``,
``dequantize``, ``weight_error``, ``output_error``, ``output_error_given_ref``,
``output_reference``, ``output_error_codes``, ``output_gram``, ``output_reference_gram``,
``output_error_gram``, ``gptq_hessian``, ``gptq_quantize``,
``hdiag_format_info``.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhdiag.so")

# enums of include/hdiag.h
HD_OK, HD_ERR_INVALID_ARG, HD_ERR_UNSUPPORTED, HD_ERR_HIP = 0, -1, -2, -3
HD_F32, HD_BF16 = 0, 1
SCHED_GRAM_GANGS, SCHED_GPTQ_TILE, SCHED_GRAM_BANDS = 0, 1, 2
PROBE_READ, PROBE_ENCODE, PROBE_WRITE, PROBE_DEQUANT = 0, 1, 2, 3
NAIVE, SSE_OPT, H_OPT, NAIVE_OCP = 0, 1, 2, 3
INT8_E4M3, NVFP4, MXFP4, MXFP8, FP8_E4M3S = 0, 1, 2, 3, 4
NVFP4_UE4M4, NVFP4_UE5M3, NVINT4 = 5, 6, 7
FP4_F16, INT4_F16 = 8, 9
FORMATS = {"INT8_E4M3": INT8_E4M3, "NVFP4": NVFP4, "MXFP4": MXFP4, "MXFP8": MXFP8, "FP8_E4M3S": FP8_E4M3S,
           "NVFP4_UE4M4": NVFP4_UE4M4, "NVFP4_UE5M3": NVFP4_UE5M3, "NVINT4": NVINT4, "FP4_F16": FP4_F16,
           "INT4_F16": INT4_F16}
METHODS = {"naive": NAIVE, "sse": SSE_OPT, "h": H_OPT, "naive_ocp": NAIVE_OCP}
FOUR_BIT = (NVFP4, MXFP4, NVFP4_UE4M4, NVFP4_UE5M3, NVINT4, FP4_F16, INT4_F16)
# formats whose block scales are binary16 values (stored as torch.float16)
F16_SCALES = (FP4_F16, INT4_F16)

EXPORTS = ["hdiag_set_schedule", "hdiag", "hdiag_workspace_size", "hdiag_noalloc", "quantize_blocks", "quantize_blocks_instrumented", "encode_blocks", "dequantize",
           "weight_error", "weight_error_workspace_size", "dequantize_weight_error", "output_error", "output_error_workspace_size",
           "output_error_given_ref", "output_reference", "output_reference_size", "output_error_codes",
           "output_error_codes_workspace_size", "output_gram", "output_gram_size", "output_gram_workspace_size",
           "output_reference_gram", "output_error_gram", "output_error_gram_workspace_size",
           "output_error_gram_batch", "output_error_gram_batch_workspace_size",
           "quantize_blocks_tensor_scaled",
           "quantize_blocks_tensor_scaled_workspace_size", "dequantize_tensor_scaled", "gptq_hessian", "gptq_hessian_workspace_size", "gptq_quantize",
           "gptq_workspace_size", "gptq_factor", "gptq_factor_size", "gptq_factor_workspace_size",
           "gptq_quantize_factored",
           "hdiag_strerror", "hdiag_last_error", "hdiag_format_info", "hdiag_version", "hdiag_stream_probe"]


class HdiagError(RuntimeError):
    def __init__(self, status, what, detail):
        super().__init__("%s failed: %s (%d): %s" % (what, _strerror(status), status, detail))
        self.status = status


_lib = None


def lib():
    """The loaded libhdiag.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libhdiag.so is not built (%s); run block_scaled_precision_hdiag_amd/build.py"
                               % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        L.hdiag.argtypes = [P, i32, i64, i64, P, P, sz, P]
        L.hdiag_workspace_size.argtypes = [i64, i64]
        L.hdiag_noalloc.argtypes = [P, i32, i64, i64, P, P]
        L.hdiag_set_schedule.argtypes = [i32, i32]
        L.hdiag_stream_probe.argtypes = [i32, i64, P, P, P, P, P]
        L.hdiag_workspace_size.restype = sz
        L.quantize_blocks.argtypes = [i32, i32, i32, P, i32, i64, i64, P, P, P, P, P]
        L.quantize_blocks_instrumented.argtypes = [i32, i32, i32, P, i32, i64, i64, P, P, P, P, P, P]
        L.encode_blocks.argtypes = [i32, i32, P, i32, i64, i64, P, P, P, P, P]
        L.dequantize.argtypes = [i32, i32, P, P, i64, i64, P, i32, P]
        L.weight_error_workspace_size.argtypes = [i64, i64]
        L.weight_error_workspace_size.restype = sz
        L.weight_error.argtypes = [P, i32, P, i32, i64, i64, P, P, P, sz, P]
        L.dequantize_weight_error.argtypes = [i32, i32, P, P, i64, i64, P, i32, P, i32, P, P, P, sz, P]
        L.output_error_workspace_size.argtypes = [i64, i64, i64]
        L.output_error_workspace_size.restype = sz
        L.output_error.argtypes = [P, i32, i64, P, i32, P, i32, i64, i64, P, P, P, sz, P]
        L.output_error_given_ref.argtypes = [P, i32, i64, P, i32, P, i32, i64, i64, P, P, P, P, sz, P]
        L.output_reference_size.argtypes = [i64, i64, i64]
        L.output_reference_size.restype = sz
        L.output_reference.argtypes = [P, i32, i64, P, i32, i64, i64, P, sz, P]
        L.output_error_codes_workspace_size.argtypes = [i64, i64, i64]
        L.output_error_codes_workspace_size.restype = sz
        L.output_error_codes.argtypes = [i32, i32, P, i32, i64, P, P, i64, i64, P, sz, P, P, P, sz, P]
        L.output_gram_size.argtypes = [i64]
        L.output_gram_size.restype = sz
        L.output_gram_workspace_size.argtypes = [i64, i64]
        L.output_gram_workspace_size.restype = sz
        L.output_gram.argtypes = [P, i32, i64, i64, P, P, sz, P, sz, P]
        L.output_error_gram_workspace_size.argtypes = [i64, i64]
        L.output_error_gram_workspace_size.restype = sz
        L.output_reference_gram.argtypes = [P, i32, i64, i64, P, sz, P, P, sz, P]
        L.output_error_gram.argtypes = [i32, i32, P, P, P, i32, i64, i64, P, sz, P, P, P, P, sz, P]
        L.output_error_gram_batch_workspace_size.argtypes = [i32, i64, i64]
        L.output_error_gram_batch_workspace_size.restype = sz
        L.output_error_gram_batch.argtypes = [i32, P, P, P, P, P, i32, i64, i64, P, sz, P, P, P, P, sz, P]
        L.hdiag_strerror.argtypes = [i32]
        L.hdiag_strerror.restype = ctypes.c_char_p
        L.hdiag_last_error.argtypes = []
        L.hdiag_last_error.restype = ctypes.c_char_p
        L.hdiag_format_info.argtypes = [i32, i32, P, P, P, P]
        L.hdiag_version.argtypes = []
        L.hdiag_version.restype = ctypes.c_char_p
        L.quantize_blocks_tensor_scaled_workspace_size.argtypes = [i64, i64]
        L.quantize_blocks_tensor_scaled_workspace_size.restype = sz
        L.quantize_blocks_tensor_scaled.argtypes = [i32, i32, i32, P, i32, i64, i64, P, P, P, P, P, P, sz, P]
        L.dequantize_tensor_scaled.argtypes = [i32, i32, P, P, P, i64, i64, P, i32, P]
        L.gptq_hessian_workspace_size.argtypes = [i64, i64]
        L.gptq_hessian_workspace_size.restype = sz
        L.gptq_hessian.argtypes = [P, i32, i64, i64, P, P, sz, P]
        L.gptq_workspace_size.argtypes = [i32, i64, i64]
        L.gptq_workspace_size.restype = sz
        L.gptq_quantize.argtypes = [i32, i32, i32, P, i32, i64, i64, P, ctypes.c_double, i32, P, P, P, P, P, sz, P]
        L.gptq_factor_size.argtypes = [i64]
        L.gptq_factor_size.restype = sz
        L.gptq_factor_workspace_size.argtypes = [i64]
        L.gptq_factor_workspace_size.restype = sz
        L.gptq_factor.argtypes = [P, i64, ctypes.c_double, P, sz, P, P, sz, P]
        L.gptq_quantize_factored.argtypes = [i32, i32, i32, P, i32, i64, i64, P, P, sz, P, P, P, P, P, sz, P]
        for name in ("hdiag_set_schedule", "hdiag", "hdiag_noalloc", "quantize_blocks", "quantize_blocks_instrumented", "encode_blocks", "dequantize", "weight_error",
                     "dequantize_weight_error", "output_error", "output_error_given_ref", "output_reference", "output_error_codes",
                     "output_gram", "output_reference_gram", "output_error_gram", "output_error_gram_batch",
                     "hdiag_format_info", "gptq_hessian", "gptq_quantize", "gptq_factor", "gptq_quantize_factored", "quantize_blocks_tensor_scaled",
                     "dequantize_tensor_scaled"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def _strerror(status):
    return lib().hdiag_strerror(status).decode()


def hdiag_strerror(status):
    """Static description of a status code; host-only."""
    return _strerror(status)


def hdiag_last_error():
    """Description of the calling thread's last failure ("" if none); host-only."""
    return lib().hdiag_last_error().decode()


def hdiag_version():
    """Library version string; host-only."""
    return lib().hdiag_version().decode()


def _check(status, what):
    if status != HD_OK:
        raise HdiagError(status, what, lib().hdiag_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dt(t):
    if t.dtype == torch.bfloat16:
        return HD_BF16
    if t.dtype == torch.float32:
        return HD_F32
    raise TypeError("expected a float32 or bfloat16 tensor, got %s" % t.dtype)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t):
    if not t.is_cuda:
        raise ValueError("tensors must be on a GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.device


def codes_shape(fmt, N, K):
    return (N, K // 2) if fmt in FOUR_BIT else (N, K)


def scale_dtype(fmt):
    """torch dtype of a scale tensor: float16 (the binary16 scale itself) for
    the FP16-scale formats, uint8 codes otherwise."""
    return torch.float16 if fmt in F16_SCALES else torch.uint8


def hdiag_set_schedule(knob, value):
    """Set a process-wide schedule setting (SCHED_GRAM_GANGS, SCHED_GPTQ_TILE,
    SCHED_GRAM_BANDS; 0 = automatic); host-only."""
    _check(lib().hdiag_set_schedule(knob, value), "hdiag_set_schedule")


def hdiag_stream_probe(kind, n, in0=None, in1=None, out0=None, out1=None, device=None):
    """One streaming probe of n 16-bit elements (PROBE_READ, PROBE_ENCODE,
    PROBE_WRITE, PROBE_DEQUANT; buffers as include/hdiag.h gives them)."""
    t = next(x for x in (in0, out0) if x is not None)
    _check(lib().hdiag_stream_probe(kind, n, _ptr(in0), _ptr(in1), _ptr(out0), _ptr(out1), _stream(_dev(t))),
           "hdiag_stream_probe")


def hdiag_workspace_size(M, K):
    return int(lib().hdiag_workspace_size(M, K))


def hdiag(X, out=None, workspace=None):
    """h[j] = sum_t X[t, j]^2 (float32 [K]) for X [M, K] float32 / bfloat16."""
    d = _dev(X)
    M, K = X.shape
    h = out if out is not None else torch.empty(K, dtype=torch.float32, device=d)
    need = hdiag_workspace_size(M, K)
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=d)
    _check(lib().hdiag(_ptr(X), _dt(X), M, K, _ptr(h), _ptr(ws), ws.numel(), _stream(d)), "hdiag")
    return h


# bytes of the static device scratch behind hdiag_noalloc (HD_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 16 << 20


def hdiag_noalloc(X, out):
    """hdiag() into a caller-given float32 [K] tensor `out`, with the library's
    static per-GPU scratch instead of a workspace: the call allocates nothing.
    Calls that overlap on one GPU race (they share the scratch)."""
    d = _dev(X)
    M, K = X.shape
    _check(lib().hdiag_noalloc(_ptr(X), _dt(X), M, K, _ptr(out), _stream(d)), "hdiag_noalloc")
    return out


def quantize_blocks(method, fmt, B, W, h=None, block_obj=False, codes=None, scales=None):
    """Scale choice + encode.  Returns (codes uint8, scales [N, K/B] (uint8 codes,
    or float16 for FP16 scales), block_obj or None)."""
    d = _dev(W)
    N, K = W.shape
    codes = codes if codes is not None else torch.empty(codes_shape(fmt, N, K), dtype=torch.uint8, device=d)
    scales = scales if scales is not None else torch.empty((N, K // B if B else 0), dtype=scale_dtype(fmt), device=d)
    obj = torch.empty((N, K // B if B else 0), dtype=torch.float32, device=d) if block_obj else None
    _check(lib().quantize_blocks(method, fmt, B, _ptr(W), _dt(W), N, K, _ptr(h), _ptr(codes), _ptr(scales),
                                 _ptr(obj), _stream(d)), "quantize_blocks")
    return codes, scales, obj


def quantize_blocks_instrumented(method, fmt, B, W, evaluated, h=None, block_obj=False, codes=None, scales=None):
    """quantize_blocks, adding to `evaluated` (a device int64 tensor of one
    element, cleared by the caller) the (weight, candidate) pairs the search
    evaluated.  Returns what quantize_blocks returns."""
    d = _dev(W)
    N, K = W.shape
    if evaluated.dtype != torch.int64 or evaluated.numel() != 1:
        raise ValueError("evaluated must be a device int64 tensor of one element")
    codes = codes if codes is not None else torch.empty(codes_shape(fmt, N, K), dtype=torch.uint8, device=d)
    scales = scales if scales is not None else torch.empty((N, K // B), dtype=scale_dtype(fmt), device=d)
    obj = torch.empty((N, K // B), dtype=torch.float32, device=d) if block_obj else None
    _check(lib().quantize_blocks_instrumented(method, fmt, B, _ptr(W), _dt(W), N, K, _ptr(h), _ptr(codes),
                                              _ptr(scales), _ptr(obj), _ptr(evaluated), _stream(d)),
           "quantize_blocks_instrumented")
    return codes, scales, obj


def encode_blocks(fmt, B, W, scales, h=None, block_obj=False):
    """Encode W with given scale codes.  Returns (codes, block_obj or None)."""
    d = _dev(W)
    N, K = W.shape
    codes = torch.empty(codes_shape(fmt, N, K), dtype=torch.uint8, device=d)
    obj = torch.empty((N, K // B), dtype=torch.float32, device=d) if block_obj else None
    _check(lib().encode_blocks(fmt, B, _ptr(W), _dt(W), N, K, _ptr(scales), _ptr(h), _ptr(codes), _ptr(obj),
                               _stream(d)), "encode_blocks")
    return codes, obj


def dequantize(fmt, B, codes, scales, N, K, dtype=torch.float32, out=None):
    d = _dev(codes)
    out = out if out is not None else torch.empty((N, K), dtype=dtype, device=d)
    _check(lib().dequantize(fmt, B, _ptr(codes), _ptr(scales), N, K, _ptr(out), _dt(out), _stream(d)),
           "dequantize")
    return out


def weight_error_workspace_size(N, K):
    return int(lib().weight_error_workspace_size(N, K))


def weight_error(W, Wq, sums=False, workspace=None, out=None):
    """||Wq - W||_F / ||W||_F as a float64 device tensor of shape [1] (and [2] sums)."""
    d = _dev(W)
    N, K = W.shape
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device=d)
    s = torch.empty(2, dtype=torch.float64, device=d) if sums else None
    need = int(lib().weight_error_workspace_size(N, K))
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=d)
    _check(lib().weight_error(_ptr(W), _dt(W), _ptr(Wq), _dt(Wq), N, K, _ptr(out), _ptr(s), _ptr(ws),
                              ws.numel(), _stream(d)), "weight_error")
    return (out, s) if sums else out


def dequantize_weight_error(fmt, B, codes, scales, W, dtype=torch.float32, out=None, err=None, sums=False,
                            workspace=None):
    """dequantize() and weight_error() in one pass: (Wq, err[, sums]) with Wq
    as dequantize writes it and err (float64 [1]) as weight_error(W, Wq) gives it."""
    d = _dev(W)
    N, K = W.shape
    out = out if out is not None else torch.empty((N, K), dtype=dtype, device=d)
    err = err if err is not None else torch.empty(1, dtype=torch.float64, device=d)
    s = torch.empty(2, dtype=torch.float64, device=d) if sums else None
    need = int(lib().weight_error_workspace_size(N, K))
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=d)
    _check(lib().dequantize_weight_error(fmt, B, _ptr(codes), _ptr(scales), N, K, _ptr(out), _dt(out), _ptr(W),
                                         _dt(W), _ptr(err), _ptr(s), _ptr(ws), ws.numel(), _stream(d)),
           "dequantize_weight_error")
    return (out, err, s) if sums else (out, err)


def output_error_workspace_size(M, N, K):
    return int(lib().output_error_workspace_size(M, N, K))


def output_error(X, W, Wq, sums=False, workspace=None):
    """||X Wq^T - X W^T||_F / ||X W^T||_F as a float64 device tensor [1] (and [2] sums)."""
    d = _dev(X)
    M, K = X.shape
    N = W.shape[0]
    out = torch.empty(1, dtype=torch.float64, device=d)
    s = torch.empty(2, dtype=torch.float64, device=d) if sums else None
    need = output_error_workspace_size(M, N, K)
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=d)
    _check(lib().output_error(_ptr(X), _dt(X), M, _ptr(W), _dt(W), _ptr(Wq), _dt(Wq), N, K, _ptr(out), _ptr(s),
                              _ptr(ws), ws.numel(), _stream(d)), "output_error")
    return (out, s) if sums else out


def output_error_given_ref(X, W, Wq, ysq, sums=False, workspace=None):
    """output_error with ||X W^T||^2 given as the float64 device scalar ysq
    (e.g. sums[1] of an earlier output_error on the same X and W)."""
    d = _dev(X)
    M, K = X.shape
    N = W.shape[0]
    out = torch.empty(1, dtype=torch.float64, device=d)
    s = torch.empty(2, dtype=torch.float64, device=d) if sums else None
    need = output_error_workspace_size(M, N, K)
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=d)
    _check(lib().output_error_given_ref(_ptr(X), _dt(X), M, _ptr(W), _dt(W), _ptr(Wq), _dt(Wq), N, K, _ptr(ysq),
                                        _ptr(out), _ptr(s), _ptr(ws), ws.numel(), _stream(d)),
           "output_error_given_ref")
    return (out, s) if sums else out


REF_Y_OFFSET = 256  # HD_REF_Y_OFFSET


def output_reference_size(M, N, K):
    return int(lib().output_reference_size(M, N, K))


def output_reference(X, W, ref=None):
    """Fill (or allocate) the reference buffer of (X, W) for output_error_codes:
    ||X W^T||^2 and Y = X W^T (see reference_ysq / reference_y).  Returns it
    as a uint8 device tensor."""
    d = _dev(X)
    M, K = X.shape
    N = W.shape[0]
    need = output_reference_size(M, N, K)
    if ref is None:
        ref = torch.empty(need, dtype=torch.uint8, device=d)
    _check(lib().output_reference(_ptr(X), _dt(X), M, _ptr(W), _dt(W), N, K, _ptr(ref), ref.numel(), _stream(d)),
           "output_reference")
    return ref


def reference_ysq(ref):
    """||X W^T||^2 of a reference buffer, as a float64 device tensor [1] (a view)."""
    return ref[:8].view(torch.float64)


def reference_y(ref, M, N):
    """Y = X W^T of a reference buffer, as a float32 device tensor [M, N] (a view)."""
    return ref[REF_Y_OFFSET:REF_Y_OFFSET + M * N * 4].view(torch.float32).view(M, N)


def output_error_codes_workspace_size(M, N, K):
    return int(lib().output_error_codes_workspace_size(M, N, K))


def output_error_codes(fmt, B, X, codes, scales, ref, N, K, sums=False, workspace=None, out=None):
    """||X Wq^T - X W^T||_F / ||X W^T||_F for Wq = dequantize(fmt, B, codes,
    scales), against the reference buffer of (X, W)."""
    d = _dev(X)
    M = X.shape[0]
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device=d)
    s = torch.empty(2, dtype=torch.float64, device=d) if sums else None
    need = output_error_codes_workspace_size(M, N, K)
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=d)
    _check(lib().output_error_codes(fmt, B, _ptr(X), _dt(X), M, _ptr(codes), _ptr(scales), N, K, _ptr(ref),
                                    ref.numel(), _ptr(out), _ptr(s), _ptr(ws), ws.numel(), _stream(d)),
           "output_error_codes")
    return (out, s) if sums else out


def output_gram_size(K):
    return int(lib().output_gram_size(K))


def output_gram_workspace_size(M, K):
    return int(lib().output_gram_workspace_size(M, K))


def output_gram(X, h=None, gram=None, workspace=None):
    """Fill (or allocate) the Gram buffer of X (bfloat16 [M, K]) for
    output_reference_gram / output_error_gram.  h: hdiag(X) if already
    computed.  Returns it as a uint8 device tensor."""
    d = _dev(X)
    M, K = X.shape
    if gram is None:
        gram = torch.empty(max(output_gram_size(K), 16), dtype=torch.uint8, device=d)
    need = output_gram_workspace_size(M, K)
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=d)
    _check(lib().output_gram(_ptr(X), _dt(X), M, K, _ptr(h), _ptr(gram), gram.numel(), _ptr(ws), ws.numel(),
                             _stream(d)), "output_gram")
    return gram


def output_error_gram_workspace_size(N, K):
    return int(lib().output_error_gram_workspace_size(N, K))


def output_reference_gram(W, gram, workspace=None, out=None):
    """||X W^T||_F^2 from the Gram buffer of X, as a float64 device tensor [1]."""
    d = _dev(W)
    N, K = W.shape
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device=d)
    need = output_error_gram_workspace_size(N, K)
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=d)
    _check(lib().output_reference_gram(_ptr(W), _dt(W), N, K, _ptr(gram), gram.numel(), _ptr(out), _ptr(ws),
                                       ws.numel(), _stream(d)), "output_reference_gram")
    return out


def output_error_gram(fmt, B, codes, scales, W, gram, ysq, sums=False, workspace=None, out=None):
    """||X Wq^T - X W^T||_F / sqrt(ysq) for Wq = dequantize(fmt, B, codes,
    scales), from the Gram buffer of X; ysq from output_reference_gram."""
    d = _dev(W)
    N, K = W.shape
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device=d)
    s = torch.empty(3, dtype=torch.float64, device=d) if sums else None
    need = output_error_gram_workspace_size(N, K)
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=d)
    _check(lib().output_error_gram(fmt, B, _ptr(codes), _ptr(scales), _ptr(W), _dt(W), N, K, _ptr(gram),
                                   gram.numel(), _ptr(ysq), _ptr(out), _ptr(s), _ptr(ws), ws.numel(), _stream(d)),
           "output_error_gram")
    return (out, s) if sums else out


def output_error_gram_batch_workspace_size(count, N, K):
    return int(lib().output_error_gram_batch_workspace_size(count, N, K))


def output_error_gram_batch(items, W, gram, ysq, sums=False, workspace=None, out=None):
    """output_error_gram for several quantisations of W in one call: items is a
    sequence of (fmt, B, codes, scales).  Returns a float64 device tensor
    [len(items)] (and [len(items), 3] sums: ||X D^T||^2, ||X W^T||^2 and the
    diagonal sum of each; `sums` may be such a float64 tensor to fill)."""
    d = _dev(W)
    N, K = W.shape
    n = len(items)
    if out is None:
        out = torch.empty(n, dtype=torch.float64, device=d)
    if isinstance(sums, torch.Tensor):
        if sums.dtype != torch.float64 or sums.numel() < 3 * n or not sums.is_contiguous():
            raise ValueError("sums must be a contiguous float64 tensor of 3 x %d values" % n)
        s = sums
    else:
        s = torch.empty((n, 3), dtype=torch.float64, device=d) if sums else None
    fm = (ctypes.c_int * n)(*[int(it[0]) for it in items])
    bs = (ctypes.c_int32 * n)(*[int(it[1]) for it in items])
    cs = (ctypes.c_void_p * n)(*[it[2].data_ptr() for it in items])
    ss = (ctypes.c_void_p * n)(*[it[3].data_ptr() for it in items])
    need = output_error_gram_batch_workspace_size(n, N, K)
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=d)
    _check(lib().output_error_gram_batch(n, fm, bs, cs, ss, _ptr(W), _dt(W), N, K, _ptr(gram), gram.numel(),
                                         _ptr(ysq), _ptr(out), _ptr(s), _ptr(ws), ws.numel(), _stream(d)),
           "output_error_gram_batch")
    return (out, s) if s is not None else out


def quantize_blocks_tensor_scaled_workspace_size(N, K):
    return int(lib().quantize_blocks_tensor_scaled_workspace_size(N, K))


def quantize_blocks_tensor_scaled(method, fmt, B, W, h=None, block_obj=False, workspace=None):
    """Per-tensor scale + E4M3 block scales.  Returns (codes, scales, tensor_scale
    float32 [1], block_obj of W / tensor_scale or None)."""
    d = _dev(W)
    N, K = W.shape
    codes = torch.empty(codes_shape(fmt, N, K), dtype=torch.uint8, device=d)
    scales = torch.empty((N, K // B), dtype=torch.uint8, device=d)
    ts = torch.empty(1, dtype=torch.float32, device=d)
    obj = torch.empty((N, K // B), dtype=torch.float32, device=d) if block_obj else None
    need = quantize_blocks_tensor_scaled_workspace_size(N, K)
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=d)
    _check(lib().quantize_blocks_tensor_scaled(method, fmt, B, _ptr(W), _dt(W), N, K, _ptr(h), _ptr(codes),
                                               _ptr(scales), _ptr(ts), _ptr(obj), _ptr(ws), ws.numel(), _stream(d)),
           "quantize_blocks_tensor_scaled")
    return codes, scales, ts, obj


def dequantize_tensor_scaled(fmt, B, codes, scales, tensor_scale, N, K, dtype=torch.float32, out=None):
    d = _dev(codes)
    out = out if out is not None else torch.empty((N, K), dtype=dtype, device=d)
    _check(lib().dequantize_tensor_scaled(fmt, B, _ptr(codes), _ptr(scales), _ptr(tensor_scale), N, K, _ptr(out),
                                          _dt(out), _stream(d)), "dequantize_tensor_scaled")
    return out


def gptq_hessian_workspace_size(M, K):
    return int(lib().gptq_hessian_workspace_size(M, K))


def gptq_hessian(X, H=None, workspace=None):
    """H = X^T X (float32 [K, K]) for bfloat16 X [M, K], on the MFMA units."""
    d = _dev(X)
    M, K = X.shape
    H = H if H is not None else torch.empty((K, K), dtype=torch.float32, device=d)
    need = gptq_hessian_workspace_size(M, K)
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=d)
    _check(lib().gptq_hessian(_ptr(X), _dt(X), M, K, _ptr(H), _ptr(ws), ws.numel(), _stream(d)), "gptq_hessian")
    return H


def gptq_workspace_size(B, N, K):
    return int(lib().gptq_workspace_size(B, N, K))


def gptq_quantize(method, fmt, B, W, H, damp=0.01, ordered=False, codes=None, scales=None, workspace=None):
    """GPTQ-Seq (ordered=False) or GPTQ-Ord on top of `method`'s scale choice,
    given H = X^T X (float32 [K, K]).  Returns (codes, scales, block_order
    int32 [K/B], info int32 [1]: 0, or 1 + the first non-positive pivot)."""
    d = _dev(W)
    N, K = W.shape
    codes = codes if codes is not None else torch.empty(codes_shape(fmt, N, K), dtype=torch.uint8, device=d)
    scales = scales if scales is not None else torch.empty((N, K // B), dtype=scale_dtype(fmt), device=d)
    order = torch.empty(K // B, dtype=torch.int32, device=d)
    info = torch.zeros(1, dtype=torch.int32, device=d)
    need = gptq_workspace_size(B, N, K)
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=d)
    _check(lib().gptq_quantize(method, fmt, B, _ptr(W), _dt(W), N, K, _ptr(H), float(damp), int(bool(ordered)),
                               _ptr(codes), _ptr(scales), _ptr(order), _ptr(info), _ptr(ws), ws.numel(), _stream(d)),
           "gptq_quantize")
    return codes, scales, order, info


def gptq_factor_size(K):
    return int(lib().gptq_factor_size(K))


def gptq_factor_workspace_size(K):
    return int(lib().gptq_factor_workspace_size(K))


def gptq_factor(H, damp=0.01, factor=None, workspace=None):
    """The sequential-order GPTQ factor of H (float32 [K, K]) and damp, as a
    uint8 device tensor, and its status (int32 [1])."""
    d = _dev(H)
    K = H.shape[0]
    if factor is None:
        factor = torch.empty(max(gptq_factor_size(K), 16), dtype=torch.uint8, device=d)
    info = torch.zeros(1, dtype=torch.int32, device=d)
    need = gptq_factor_workspace_size(K)
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=d)
    _check(lib().gptq_factor(_ptr(H), K, float(damp), _ptr(factor), factor.numel(), _ptr(info), _ptr(ws), ws.numel(),
                             _stream(d)), "gptq_factor")
    return factor, info


def gptq_quantize_factored(method, fmt, B, W, H, factor, codes=None, scales=None, workspace=None):
    """GPTQ-Seq from a factor made by gptq_factor(H, damp): the results of
    gptq_quantize(method, fmt, B, W, H, damp, ordered=False)."""
    d = _dev(W)
    N, K = W.shape
    codes = codes if codes is not None else torch.empty(codes_shape(fmt, N, K), dtype=torch.uint8, device=d)
    scales = scales if scales is not None else torch.empty((N, K // B), dtype=scale_dtype(fmt), device=d)
    order = torch.empty(K // B, dtype=torch.int32, device=d)
    info = torch.zeros(1, dtype=torch.int32, device=d)
    need = gptq_workspace_size(B, N, K)
    ws = workspace if workspace is not None else torch.empty(max(need, 16), dtype=torch.uint8, device=d)
    _check(lib().gptq_quantize_factored(method, fmt, B, _ptr(W), _dt(W), N, K, _ptr(H), _ptr(factor), factor.numel(),
                                        _ptr(codes), _ptr(scales), _ptr(order), _ptr(info), _ptr(ws), ws.numel(),
                                        _stream(d)), "gptq_quantize_factored")
    return codes, scales, order, info


def hdiag_format_info(fmt, B):
    """(elem_bits, scale_bits, n_candidates, bits_per_weight); host-only."""
    e, s, n = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    bpw = ctypes.c_double()
    _check(lib().hdiag_format_info(fmt, B, ctypes.byref(e), ctypes.byref(s), ctypes.byref(n),
                                   ctypes.byref(bpw)), "hdiag_format_info")
    return e.value, s.value, n.value, bpw.value


def version():
    return lib().hdiag_version().decode()
