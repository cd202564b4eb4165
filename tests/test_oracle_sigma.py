"""Pins of the block-size / sigma study ("Is Finer Better?", §3.2 and Fig. 2,
§4.3 and App. F.3-F.4, §5.2) on the oracle: Normal tensors of standard
deviation sigma quantised with E2M1 elements and Naive scales.

What the page states and these check, on seeded N(0, sigma^2) tensors:
  - with quantised UE4M3 (= positive E4M3) scales, block size 8 has a larger
    MSE than block size 16 below a crossover near sigma = 2e-2 and a smaller
    one above it;
  - with (nearly) unquantised scales - binary16 here - the finer block is
    better at every sigma;
  - when the block maximum / 6 falls in the zero bin of the scale grid (below
    half of UE4M3's smallest value 2^-9), every element rounds to zero: the
    MSE is exactly the mean square of the tensor;
  - UE5M3 (smallest value 2^-17) keeps such narrow tensors representable and
    shows no crossover.
"""
import numpy as np
import pytest

import oracle

Z = np.random.default_rng(0).standard_normal((128, 4096))


def mse(fmt, B, W):
    c, s, _ = oracle.quantize(oracle.NAIVE, fmt, B, W)
    Wq = oracle.dequantize(fmt, B, c, s, *W.shape)
    return float(np.mean((Wq.astype(np.float64) - W.astype(np.float64)) ** 2))


def tensor(sigma):
    return (Z * sigma).astype(np.float32)


def test_crossover_with_ue4m3_scales():
    below, above = tensor(1e-2), tensor(5e-2)
    assert mse(oracle.NVFP4, 8, below) > 1.1 * mse(oracle.NVFP4, 16, below)
    assert mse(oracle.NVFP4, 8, above) < 0.9 * mse(oracle.NVFP4, 16, above)
    # the sign change sits between 1e-2 and 3e-2
    sig = np.geomspace(1e-2, 3e-2, 7)
    d = [mse(oracle.NVFP4, 8, tensor(s)) - mse(oracle.NVFP4, 16, tensor(s)) for s in sig]
    assert d[0] > 0 and d[-1] < 0


@pytest.mark.parametrize("fmt", [oracle.NVFP4_UE5M3, oracle.FP4_F16])
def test_no_crossover_with_wide_or_fine_scales(fmt):
    for sigma in (3e-4, 3e-3, 1e-2, 3e-2, 1e-1):
        W = tensor(sigma)
        assert mse(fmt, 8, W) < mse(fmt, 16, W) < mse(fmt, 32, W)


@pytest.mark.parametrize("B", [8, 16, 32])
def test_zero_scale_collapse(B):
    W = tensor(3e-4)
    assert np.abs(W).max() / 6 <= 2.0 ** -10  # every block's amax / 6 is in the zero bin
    m = mse(oracle.NVFP4, B, W)
    assert m == float(np.mean(W.astype(np.float64) ** 2))
    assert mse(oracle.NVFP4_UE5M3, B, W) < 0.02 * m
