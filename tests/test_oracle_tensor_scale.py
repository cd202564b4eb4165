"""Pins of the oracle's per-tensor scaling over E4M3 block scales ("Is Finer
Better?" §5.1, UE4M3-S), read as s_T = amax_T / (C * 448), W' = fl32(W / s_T)
quantised by the format, x^ = fl32(s_T * fl32(s q)).

What fixes it other than the oracle: exact power-of-two relations (scaling W
by 2^k scales s_T by 2^k and leaves every code; when s_T is itself a power of
two, the result is the plain quantiser on W / s_T), the closed form of the
largest block (its scale lands on the top E4M3 code), the zero tensor, and the
page's claim that per-tensor scaling removes the narrow-tensor error growth
(the sigma study of the same paper: the plain grid collapses, the scaled one
keeps the MSE / sigma^2 of wide tensors).
"""
import numpy as np
import pytest

import oracle

FMTS = [oracle.NVFP4, oracle.NVINT4, oracle.FP8_E4M3S, oracle.INT8_E4M3]
C = {oracle.NVFP4: 6.0, oracle.NVINT4: 7.0, oracle.FP8_E4M3S: 448.0, oracle.INT8_E4M3: 1.0}


def weights(seed, N=24, K=512, std=0.02):
    return (np.random.default_rng(seed).standard_t(4, (N, K)) * std).astype(np.float32)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("method", [oracle.NAIVE, oracle.SSE_OPT])
def test_power_of_two_scaling(fmt, method):
    W = weights(1)
    c0, s0, t0, o0 = oracle.quantize_tensor_scaled(method, fmt, 16, W)
    for k in (5, -7):
        c1, s1, t1, o1 = oracle.quantize_tensor_scaled(method, fmt, 16, W * np.float32(2.0 ** k))
        assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
        assert t1 == t0 * np.float32(2.0 ** k)
        np.testing.assert_array_equal(o1, o0)


@pytest.mark.parametrize("fmt", FMTS)
def test_power_of_two_tensor_scale_is_the_plain_quantiser(fmt):
    """amax_T = C * 448 * 2^-9: s_T = 2^-9 exactly, so W' = W * 2^9 exactly and
    the codes are the plain quantiser's on W * 2^9; x^ = 2^-9 times its x^."""
    W = weights(2)
    top = np.float32(C[fmt] * 448.0 * 2.0 ** -9)
    W = (W * (0.999 * top / np.abs(W).max())).astype(np.float32)
    W[0, 0] = top
    c, s, t, _ = oracle.quantize_tensor_scaled(oracle.SSE_OPT, fmt, 32, W)
    assert t == np.float32(2.0 ** -9)
    c0, s0, _ = oracle.quantize(oracle.SSE_OPT, fmt, 32, W * np.float32(2.0 ** 9))
    assert np.array_equal(c, c0) and np.array_equal(s, s0)
    N, K = W.shape
    Wq = oracle.dequantize_tensor_scaled(fmt, 32, c, s, t, N, K)
    np.testing.assert_array_equal(Wq, oracle.dequantize(fmt, 32, c0, s0, N, K) * np.float32(2.0 ** -9))


@pytest.mark.parametrize("fmt", [oracle.NVFP4, oracle.NVINT4, oracle.FP8_E4M3S])
def test_largest_block_takes_the_top_scale(fmt):
    W = weights(3)
    _, s, t, _ = oracle.quantize_tensor_scaled(oracle.NAIVE, fmt, 16, W)
    r, b = np.unravel_index(np.argmax(np.abs(W)), W.shape)
    assert s[r, b // 16] == 126 and s.max() == 126  # E4M3 code 0x7E = 448
    assert t == np.float32(np.abs(W).max() / np.float32(C[fmt] * 448.0))


def test_zero_tensor_and_formats():
    W = np.zeros((4, 64), np.float32)
    c, s, t, _ = oracle.quantize_tensor_scaled(oracle.NAIVE, oracle.NVFP4, 16, W)
    assert t == 1.0 and not c.any() and not s.any()
    for fmt in (oracle.MXFP4, oracle.NVFP4_UE5M3, oracle.FP4_F16):
        with pytest.raises(ValueError):
            oracle.quantize_tensor_scaled(oracle.NAIVE, fmt, 16, W)


def test_narrow_tensors_keep_their_relative_error():
    Z = np.random.default_rng(0).standard_normal((64, 4096))
    rel = {}
    for sigma in (3e-4, 1e-2, 1e-1):
        W = (Z * sigma).astype(np.float32)
        c, s, t, _ = oracle.quantize_tensor_scaled(oracle.NAIVE, oracle.NVFP4, 16, W)
        Wq = oracle.dequantize_tensor_scaled(oracle.NVFP4, 16, c, s, t, *W.shape)
        rel[sigma] = np.mean((Wq - W.astype(np.float64)) ** 2) / sigma ** 2
        c0, s0, _ = oracle.quantize(oracle.NAIVE, oracle.NVFP4, 16, W)
        Wq0 = oracle.dequantize(oracle.NVFP4, 16, c0, s0, *W.shape)
        rel0 = np.mean((Wq0 - W.astype(np.float64)) ** 2) / sigma ** 2
        if sigma == 3e-4:
            assert rel0 > 0.99 and rel[sigma] < 0.012  # plain UE4M3 collapses, UE4M3-S does not
    assert max(rel.values()) < 1.05 * min(rel.values())
