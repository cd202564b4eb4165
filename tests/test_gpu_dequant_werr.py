"""dequantize_weight_error: dequantize() and weight_error() in one pass.

Bars: the written Wq bit-identical to dequantize()'s (float32 and bfloat16),
the ratio and its two sums bit-identical to weight_error(W, Wq) on that Wq
(the fused kernel takes the same chunks in the same order), and both against
the oracle: Wq exactly its dequantised values, the ratio within 1e-9
relative (float64 sums in another order).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import block_scaled_precision_hdiag_amd as hd

pytestmark = pytest.mark.gpu

ALL_FMTS = [hd.INT8_E4M3, hd.NVFP4, hd.MXFP4, hd.MXFP8, hd.FP8_E4M3S, hd.NVFP4_UE4M4, hd.NVFP4_UE5M3, hd.NVINT4,
            hd.FP4_F16, hd.INT4_F16]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hd.lib()


def weights(fmt, N, K, seed, dtype):
    std = {hd.FP8_E4M3S: 4.0, hd.MXFP8: 0.05}.get(fmt, 0.02)
    return synth.weights("t4", N, K, std=std, seed=seed, gain_seed=seed + 1, dtype=dtype)


def sc_np(s):
    """Scales for the oracle: uint8 codes, or the binary16 bits of float16 scales."""
    if s.dtype == torch.float16:
        return s.view(torch.int16).cpu().numpy().view(np.uint16)
    return s.cpu().numpy()


def bits_equal(a, b):
    """Bitwise equality (signed zeros told apart)."""
    iv = torch.int32 if a.dtype == torch.float32 else torch.int16
    return torch.equal(a.contiguous().view(iv), b.contiguous().view(iv))


def fused_vs_two_calls(fmt, B, W, method, out_dtype):
    Wd = W.contiguous().cuda()
    N, K = W.shape
    c, s, _ = hd.quantize_blocks(method, fmt, B, Wd)
    Wq_ref = hd.dequantize(fmt, B, c, s, N, K, dtype=out_dtype)
    e_ref, s_ref = hd.weight_error(Wd, Wq_ref, sums=True)
    Wq, e, sm = hd.dequantize_weight_error(fmt, B, c, s, Wd, dtype=out_dtype, sums=True)
    torch.cuda.synchronize()
    assert bits_equal(Wq, Wq_ref)
    assert torch.equal(e, e_ref) and torch.equal(sm, s_ref)
    return c, s, Wq, e


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_fused_equals_dequantize_then_weight_error(fmt, out_dtype):
    B = 128 if fmt in hd.F16_SCALES else 16
    N, K = 77, 2048  # N ragged against the 256-thread workgroups
    W = weights(fmt, N, K, 6100 + fmt, torch.bfloat16)
    c, s, Wq, e = fused_vs_two_calls(fmt, B, W, hd.NAIVE if fmt in hd.F16_SCALES else hd.SSE_OPT, out_dtype)
    deq_o = oracle.dequantize(fmt, B, c.cpu().numpy(), sc_np(s), N, K)
    if out_dtype == torch.float32:
        np.testing.assert_array_equal(Wq.cpu().numpy(), deq_o)
        we_o = oracle.weight_error(synth.bits(W), deq_o)
        assert e.item() == pytest.approx(we_o, rel=1e-9)
    else:
        assert torch.equal(Wq.cpu(), torch.from_numpy(deq_o).to(torch.bfloat16))


@pytest.mark.parametrize("fmt,B", [(hd.NVFP4, 4), (hd.INT8_E4M3, 4), (hd.MXFP8, 32), (hd.INT8_E4M3, 256)])
def test_fused_block_sizes_and_float32_weights(fmt, B):
    W = weights(fmt, 40, 512, 6200 + B, torch.float32)
    fused_vs_two_calls(fmt, B, W, hd.NAIVE, torch.float32)
    fused_vs_two_calls(fmt, B, W, hd.NAIVE, torch.bfloat16)


def test_fused_at_the_step_shape():
    """2560 x 9728 INT8 (the grid-stride loop takes several chunk pairs per
    thread, with a ragged last round), each block size of the step."""
    W, _ = synth.config_inputs(2)
    for B in (32, 64, 128, 256):
        fused_vs_two_calls(hd.INT8_E4M3, B, W, hd.SSE_OPT, torch.float32)


def test_fused_empty():
    W = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((0, 64), dtype=torch.uint8, device="cuda")
    s = torch.empty((0, 4), dtype=torch.uint8, device="cuda")
    Wq, e = hd.dequantize_weight_error(hd.INT8_E4M3, 16, c, s, W)
    torch.cuda.synchronize()
    assert Wq.shape == (0, 64) and np.isnan(e.item())
