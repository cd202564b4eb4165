"""Host-side checks of libhdiag.so (no GPU needed, no kernel is launched).

- the library loads and exports every function include/hdiag.h declares;
- hdiag_format_info reports the bits/weight the pages print;
- argument validation rejects bad calls before touching any memory.
"""
import ctypes
import os
import re

import pytest

import block_scaled_precision_hdiag_amd as hd
from conftest import ROOT, golden_rows

HEADER = os.path.join(ROOT, "include", "hdiag.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_header_declares_the_binding_exports():
    assert sorted(declared_functions()) == sorted(hd.EXPORTS)


def test_binding_has_every_declared_call():
    """The Python binding offers each C entry point under the same name."""
    missing = [n for n in hd.EXPORTS if not callable(getattr(hd, n, None))]
    assert not missing
    assert hd.hdiag_version().startswith("hdiag ")
    assert hd.hdiag_strerror(hd.HD_OK)
    assert hd.weight_error_workspace_size(64, 256) > 0


def test_library_exports_every_declared_symbol():
    L = hd.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert "gfx950" in hd.version()


def test_format_info_bits_per_weight():
    # qwantize "Results", "Larger blocks" layout table (FP4 + 8-bit scale)
    for B, scale_bpw, total in golden_rows("bits_per_weight.txt"):
        e, s, n, bpw = hd.hdiag_format_info(hd.NVFP4, int(B))
        assert (e, s, n) == (4, 8, 126)
        assert bpw == float(total) and s / int(B) == float(scale_bpw)
    assert hd.hdiag_format_info(hd.MXFP4, 32)[2] == 255
    assert hd.hdiag_format_info(hd.MXFP8, 32)[:3] == (8, 8, 255)
    assert hd.hdiag_format_info(hd.INT8_E4M3, 32)[3] == 8.25
    # the unsigned scale grids have 255 candidates (qwantize "Exotic Scales"),
    # NVINT4 keeps E4M3's 126; all three are 4-bit elements with 8-bit scales
    assert hd.hdiag_format_info(hd.NVFP4_UE4M4, 16) == (4, 8, 255, 4.5)
    assert hd.hdiag_format_info(hd.NVFP4_UE5M3, 16) == (4, 8, 255, 4.5)
    assert hd.hdiag_format_info(hd.NVINT4, 16) == (4, 8, 126, 4.5)


def test_format_info_fp16_scales():
    # qwantize "Results", "Larger blocks" layout table: FP16 E5M10 scales at
    # B = 128 cost 0.125 bits per weight, 4.125 in total with 4-bit elements
    for B, scale_bpw, total in golden_rows("bits_per_weight_f16.txt"):
        for f in hd.F16_SCALES:
            e, s, n, bpw = hd.hdiag_format_info(f, int(B))
            assert (e, s, n) == (4, 16, 0x7BFF)
            assert bpw == float(total) and s / int(B) == float(scale_bpw)


def test_strerror():
    assert hd._strerror(hd.HD_ERR_INVALID_ARG) == "invalid argument"
    assert hd._strerror(hd.HD_OK) == "success"


# fake, never-dereferenced device addresses (validation must fail first)
A = ctypes.c_void_p(1 << 20)
MIS = ctypes.c_void_p((1 << 20) + 4)


@pytest.mark.parametrize("args,needle", [
    ((hd.SSE_OPT, hd.NVFP4, 12, A, hd.HD_BF16, 4, 48, None, A, A, None, None), "block size"),
    ((hd.SSE_OPT, hd.NVFP4, 16, A, hd.HD_BF16, 4, 40, None, A, A, None, None), "multiple of B"),
    ((7, hd.NVFP4, 16, A, hd.HD_BF16, 4, 32, None, A, A, None, None), "unknown method"),
    ((hd.SSE_OPT, 10, 16, A, hd.HD_BF16, 4, 32, None, A, A, None, None), "unknown format"),
    ((hd.SSE_OPT, hd.NVFP4, 16, A, 5, 4, 32, None, A, A, None, None), "unknown dtype"),
    ((hd.H_OPT, hd.NVFP4, 16, A, hd.HD_BF16, 4, 32, None, A, A, None, None), "needs h"),
    ((hd.SSE_OPT, hd.NVFP4, 16, None, hd.HD_BF16, 4, 32, None, A, A, None, None), "W is NULL"),
    ((hd.SSE_OPT, hd.NVFP4, 16, MIS, hd.HD_BF16, 4, 32, None, A, A, None, None), "aligned"),
    ((hd.SSE_OPT, hd.NVFP4, 16, A, hd.HD_BF16, -1, 32, None, A, A, None, None), "negative"),
])
def test_quantize_blocks_rejects(args, needle):
    rc = hd.lib().quantize_blocks(*args, None)
    assert rc == hd.HD_ERR_INVALID_ARG
    assert needle in hd.lib().hdiag_last_error().decode()


def test_ocp_rule_needs_e8m0():
    rc = hd.lib().quantize_blocks(hd.NAIVE_OCP, hd.NVFP4, 16, A, hd.HD_BF16, 4, 32, None, A, A, None, None)
    assert rc == hd.HD_ERR_INVALID_ARG and "E8M0" in hd.lib().hdiag_last_error().decode()
    rc = hd.lib().quantize_blocks(4, hd.MXFP4, 32, A, hd.HD_BF16, 4, 32, None, A, A, None, None)
    assert rc == hd.HD_ERR_INVALID_ARG and "unknown method" in hd.lib().hdiag_last_error().decode()
    rc = hd.lib().quantize_blocks(hd.SSE_OPT, 10, 32, A, hd.HD_BF16, 4, 32, None, A, A, None, None)
    assert rc == hd.HD_ERR_INVALID_ARG and "unknown format" in hd.lib().hdiag_last_error().decode()
    for f in hd.F16_SCALES:
        rc = hd.lib().quantize_blocks(hd.NAIVE_OCP, f, 128, A, hd.HD_BF16, 4, 128, None, A, A, None, None)
        assert rc == hd.HD_ERR_INVALID_ARG and "E8M0" in hd.lib().hdiag_last_error().decode()


def test_empty_inputs_are_noops():
    L = hd.lib()
    assert L.quantize_blocks(hd.SSE_OPT, hd.NVFP4, 16, None, hd.HD_BF16, 0, 32, None, None, None, None, None) == 0
    assert L.quantize_blocks(hd.NAIVE, hd.MXFP4, 32, None, hd.HD_F32, 5, 0, None, None, None, None, None) == 0
    assert L.dequantize(hd.NVFP4, 16, None, None, 0, 16, None, hd.HD_F32, None) == 0
    assert L.hdiag(None, hd.HD_BF16, 10, 0, None, None, 0, None) == 0


def test_workspace_queries():
    assert hd.hdiag_workspace_size(244449, 9728) >= 9728 * 8
    assert hd.lib().hdiag_workspace_size(-1, 5) == 0
    ws = hd.output_error_workspace_size(16384, 2560, 9728)
    assert ws >= 2560 * 9728 * 2  # holds bf16(Wq - W)
    L = hd.lib()
    rc = L.hdiag(A, hd.HD_BF16, 1000, 64, A, A, 8, None)
    assert rc == hd.HD_ERR_INVALID_ARG and "workspace" in L.hdiag_last_error().decode()


def test_hdiag_noalloc_validation():
    """hdiag_noalloc refuses shapes whose partials exceed its static scratch,
    and bad arguments, before any HIP call."""
    L = hd.lib()
    assert hd.hdiag_workspace_size(1, 4 << 20) > hd.NOALLOC_SCRATCH_BYTES
    assert hd.hdiag_workspace_size(244449, 9728) <= hd.NOALLOC_SCRATCH_BYTES
    assert hd.hdiag_workspace_size(65536, 28672) <= hd.NOALLOC_SCRATCH_BYTES
    rc = L.hdiag_noalloc(A, hd.HD_BF16, 1, 4 << 20, A, None)
    assert rc == hd.HD_ERR_UNSUPPORTED and "static scratch" in L.hdiag_last_error().decode()
    assert L.hdiag_noalloc(A, 7, 10, 64, A, None) == hd.HD_ERR_INVALID_ARG
    assert L.hdiag_noalloc(A, hd.HD_BF16, 10, 64, None, None) == hd.HD_ERR_INVALID_ARG
    assert L.hdiag_noalloc(MIS, hd.HD_BF16, 10, 64, A, None) == hd.HD_ERR_INVALID_ARG
    assert L.hdiag_noalloc(None, hd.HD_BF16, 10, 0, None, None) == hd.HD_OK


def test_block4_only_on_the_naive_path():
    """B = 4 is accepted by Naive / encode / dequantize (K % 8 == 0) and
    refused as unsupported by the search and the codes-to-operand routes."""
    L = hd.lib()
    for m in (hd.SSE_OPT, hd.H_OPT):
        rc = L.quantize_blocks(m, hd.NVFP4, 4, A, hd.HD_BF16, 4, 32, A, A, A, None, None)
        assert rc == hd.HD_ERR_UNSUPPORTED and "block size 4" in L.hdiag_last_error().decode()
    rc = L.quantize_blocks(hd.NAIVE, hd.NVFP4, 4, A, hd.HD_BF16, 4, 12, None, A, A, None, None)
    assert rc == hd.HD_ERR_INVALID_ARG and "K % 8" in L.hdiag_last_error().decode()
    assert L.quantize_blocks(hd.NAIVE, hd.NVFP4, 4, A, hd.HD_BF16, 0, 32, None, A, A, None, None) == hd.HD_OK
    assert L.dequantize(hd.NVFP4, 4, A, A, 0, 32, A, hd.HD_F32, None) == hd.HD_OK
    M, N, K = 300, 200, 512
    rb = hd.output_reference_size(M, N, K)
    ws = hd.output_error_codes_workspace_size(M, N, K)
    rc = L.output_error_codes(hd.NVFP4, 4, A, hd.HD_BF16, M, A, A, N, K, A, rb, A, None, A, ws, None)
    assert rc == hd.HD_ERR_UNSUPPORTED
    assert L.gptq_workspace_size(4, 8, 64) == 0


def test_dequantize_weight_error_validation():
    """The fused dequantize + weight error checks its arguments on the host."""
    L = hd.lib()
    ws = hd.weight_error_workspace_size(4, 32)
    f = L.dequantize_weight_error
    cases = [
        ((hd.INT8_E4M3, 16, A, A, 4, 32, A, 7, A, hd.HD_BF16, A, None, A, ws, None), "dtype"),
        ((hd.INT8_E4M3, 16, A, A, 4, 32, A, hd.HD_F32, A, hd.HD_BF16, None, None, A, ws, None), "out is NULL"),
        ((hd.INT8_E4M3, 16, A, A, 4, 32, A, hd.HD_F32, A, hd.HD_BF16, A, None, A, 8, None), "workspace"),
        ((hd.INT8_E4M3, 16, A, A, 4, 32, A, hd.HD_F32, None, hd.HD_BF16, A, None, A, ws, None), "W is NULL"),
        ((hd.INT8_E4M3, 16, A, None, 4, 32, A, hd.HD_F32, A, hd.HD_BF16, A, None, A, ws, None), "scales"),
        ((hd.INT8_E4M3, 12, A, A, 4, 48, A, hd.HD_F32, A, hd.HD_BF16, A, None, A, ws, None), "block size"),
        ((hd.NVFP4, 4, A, A, 4, 12, A, hd.HD_F32, A, hd.HD_BF16, A, None, A, ws, None), "K % 8"),
        ((hd.FP4_F16, 128, A, ctypes.c_void_p((1 << 20) + 1), 4, 128, A, hd.HD_F32, A, hd.HD_BF16, A, None, A,
          ws, None), "2-byte aligned"),
    ]
    for args, needle in cases:
        rc = f(*args)
        assert rc == hd.HD_ERR_INVALID_ARG, needle
        assert needle in L.hdiag_last_error().decode(), (needle, L.hdiag_last_error())


def test_schedule_settings():
    """hdiag_set_schedule validates the setting and value on the host."""
    L = hd.lib()
    assert L.hdiag_set_schedule(hd.SCHED_GRAM_GANGS, 0) == hd.HD_OK
    assert L.hdiag_set_schedule(hd.SCHED_GPTQ_TILE, 0) == hd.HD_OK
    assert L.hdiag_set_schedule(hd.SCHED_GRAM_BANDS, 0) == hd.HD_OK
    assert L.hdiag_set_schedule(3, 0) == hd.HD_ERR_INVALID_ARG
    assert "unknown schedule" in L.hdiag_last_error().decode()
    assert L.hdiag_set_schedule(hd.SCHED_GRAM_GANGS, -1) == hd.HD_ERR_INVALID_ARG
    assert L.hdiag_set_schedule(hd.SCHED_GPTQ_TILE, 96) == hd.HD_ERR_INVALID_ARG
    assert L.hdiag_set_schedule(hd.SCHED_GRAM_BANDS, -2) == hd.HD_ERR_INVALID_ARG
    for v in (64, 128, 0):
        hd.hdiag_set_schedule(hd.SCHED_GPTQ_TILE, v)


def test_output_reference_validation():
    L = hd.lib()
    M, N, K = 300, 200, 512
    need = hd.output_reference_size(M, N, K)
    # Y (float32 M x N) and the float16 copy of X fit, after the 256-byte header
    assert need >= hd.REF_Y_OFFSET + M * N * 4 + M * K * 2
    assert L.output_reference_size(-1, 2, 3) == 0
    rc = L.output_reference(A, hd.HD_F32, M, A, hd.HD_BF16, N, K, A, need, None)
    assert rc == hd.HD_ERR_UNSUPPORTED and "bfloat16" in L.hdiag_last_error().decode()
    rc = L.output_reference(A, hd.HD_BF16, M, A, hd.HD_BF16, N, 12, A, need, None)
    assert rc == hd.HD_ERR_INVALID_ARG and "multiple of 8" in L.hdiag_last_error().decode()
    rc = L.output_reference(A, hd.HD_BF16, M, A, hd.HD_BF16, N, K, A, need - 1, None)
    assert rc == hd.HD_ERR_INVALID_ARG and "too small" in L.hdiag_last_error().decode()
    rc = L.output_reference(A, hd.HD_BF16, M, A, hd.HD_BF16, N, K, MIS, need, None)
    assert rc == hd.HD_ERR_INVALID_ARG and "aligned" in L.hdiag_last_error().decode()


def test_output_error_codes_validation():
    L = hd.lib()
    M, N, K = 300, 200, 512
    rb = hd.output_reference_size(M, N, K)
    ws = hd.output_error_codes_workspace_size(M, N, K)
    assert ws >= N * K * 2  # the 16-bit weight operand
    args = [hd.INT8_E4M3, 32, A, hd.HD_BF16, M, A, A, N, K, A, rb, A, None, A, ws, None]
    bad = list(args); bad[1] = 12
    assert L.output_error_codes(*bad) == hd.HD_ERR_INVALID_ARG
    assert "block size" in L.hdiag_last_error().decode()
    bad = list(args); bad[3] = hd.HD_F32
    assert L.output_error_codes(*bad) == hd.HD_ERR_UNSUPPORTED
    bad = list(args); bad[10] = rb - 8
    assert L.output_error_codes(*bad) == hd.HD_ERR_INVALID_ARG
    bad = list(args); bad[14] = ws - 8
    assert L.output_error_codes(*bad) == hd.HD_ERR_INVALID_ARG
    assert "workspace" in L.hdiag_last_error().decode()
    bad = list(args); bad[11] = None
    assert L.output_error_codes(*bad) == hd.HD_ERR_INVALID_ARG
    assert "out is NULL" in L.hdiag_last_error().decode()
    for f in hd.F16_SCALES:  # s val(q) is not an exact 16-bit operand with FP16 scales
        bad = list(args); bad[0] = f; bad[1] = 128
        assert L.output_error_codes(*bad) == hd.HD_ERR_UNSUPPORTED
        assert "FP16" in L.hdiag_last_error().decode()


def test_gram_validation():
    """Argument checks of the Gram-route calls, all taken before any GPU work."""
    L = hd.lib()
    K = 256
    gb = L.output_gram_size(K)
    assert gb >= 2 * K * K and L.output_gram_size(-1) == 0
    assert L.output_gram_workspace_size(-1, K) == 0
    ws1 = L.output_error_gram_workspace_size(300, K)
    assert ws1 == L.output_error_gram_batch_workspace_size(1, 300, K) > 0
    assert L.output_error_gram_batch_workspace_size(3, 300, K) >= 3 * 512 * K * 2  # 300 rows pad to 512
    assert L.output_error_gram_batch_workspace_size(0, 300, K) == 0
    # output_gram: float32 X is unsupported; K % 8; short buffer; misaligned pointers
    rc = L.output_gram(A, hd.HD_F32, 8, K, None, A, gb, A, 1 << 30, None)
    assert rc == hd.HD_ERR_UNSUPPORTED
    rc = L.output_gram(A, hd.HD_BF16, 8, 12, None, A, gb, A, 1 << 30, None)
    assert rc == hd.HD_ERR_INVALID_ARG and "multiple of 8" in L.hdiag_last_error().decode()
    rc = L.output_gram(A, hd.HD_BF16, 8, K, None, A, gb - 1, A, 1 << 30, None)
    assert rc == hd.HD_ERR_INVALID_ARG and "too small" in L.hdiag_last_error().decode()
    rc = L.output_gram(A, hd.HD_BF16, 8, K, None, MIS, gb, A, 1 << 30, None)
    assert rc == hd.HD_ERR_INVALID_ARG and "aligned" in L.hdiag_last_error().decode()
    # output_reference_gram: NULL ysq, short workspace
    rc = L.output_reference_gram(A, hd.HD_BF16, 4, K, A, gb, None, A, 1 << 30, None)
    assert rc == hd.HD_ERR_INVALID_ARG and "ysq" in L.hdiag_last_error().decode()
    rc = L.output_reference_gram(A, hd.HD_BF16, 4, K, A, gb, A, A, 16, None)
    assert rc == hd.HD_ERR_INVALID_ARG and "workspace" in L.hdiag_last_error().decode()
    # output_error_gram(_batch): count, block size, NULL arrays / pointers
    n = 2
    fm = (ctypes.c_int * n)(hd.INT8_E4M3, hd.NVFP4)
    bs = (ctypes.c_int32 * n)(32, 24)
    cs = (ctypes.c_void_p * n)(A.value, A.value)
    ss = (ctypes.c_void_p * n)(A.value, A.value)
    rc = L.output_error_gram_batch(n, fm, bs, cs, ss, A, hd.HD_BF16, 4, K, A, gb, A, A, None, A, 1 << 30, None)
    assert rc == hd.HD_ERR_INVALID_ARG and "block size 24" in L.hdiag_last_error().decode()
    rc = L.output_error_gram_batch(0, fm, bs, cs, ss, A, hd.HD_BF16, 4, K, A, gb, A, A, None, A, 1 << 30, None)
    assert rc == hd.HD_ERR_INVALID_ARG and "count" in L.hdiag_last_error().decode()
    rc = L.output_error_gram_batch(n, None, bs, cs, ss, A, hd.HD_BF16, 4, K, A, gb, A, A, None, A, 1 << 30, None)
    assert rc == hd.HD_ERR_INVALID_ARG and "host arrays" in L.hdiag_last_error().decode()
    rc = L.output_error_gram(hd.INT8_E4M3, 32, None, A, A, hd.HD_BF16, 4, K, A, gb, A, A, None, A, 1 << 30, None)
    assert rc == hd.HD_ERR_INVALID_ARG and "codes" in L.hdiag_last_error().decode()
    rc = L.output_error_gram(hd.INT8_E4M3, 32, A, A, A, hd.HD_BF16, 4, K, A, gb, A, None, None, A, 1 << 30, None)
    assert rc == hd.HD_ERR_INVALID_ARG and "out" in L.hdiag_last_error().decode()


def test_stream_probe_validation():
    """hdiag_stream_probe rejects unknown kinds, sizes that are not whole
    8192-element groups and missing buffers before launching anything."""
    L = hd.lib()
    buf = ctypes.c_void_p(4096)  # never dereferenced: every call below fails or is empty
    assert L.hdiag_stream_probe(7, 8192, buf, None, buf, None, None) == hd.HD_ERR_INVALID_ARG
    assert "unknown probe" in L.hdiag_last_error().decode()
    assert L.hdiag_stream_probe(hd.PROBE_READ, 4096, buf, None, buf, None, None) == hd.HD_ERR_INVALID_ARG
    assert L.hdiag_stream_probe(hd.PROBE_READ, -8192, buf, None, buf, None, None) == hd.HD_ERR_INVALID_ARG
    assert L.hdiag_stream_probe(hd.PROBE_READ, 8192, None, None, buf, None, None) == hd.HD_ERR_INVALID_ARG
    assert L.hdiag_stream_probe(hd.PROBE_ENCODE, 8192, buf, None, buf, None, None) == hd.HD_ERR_INVALID_ARG
    assert L.hdiag_stream_probe(hd.PROBE_DEQUANT, 8192, buf, None, buf, None, None) == hd.HD_ERR_INVALID_ARG
    assert L.hdiag_stream_probe(hd.PROBE_WRITE, 8192, None, None, None, None, None) == hd.HD_ERR_INVALID_ARG
    assert L.hdiag_stream_probe(hd.PROBE_WRITE, 0, None, None, None, None, None) == hd.HD_OK
