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


# ---- per-block comparison (Fig. 2(a)) and the parts of App. F, on the oracle
import torch  # noqa: E402

import bench  # noqa: E402
import synth  # noqa: E402


def objectives(fmt, B, W):
    return torch.from_numpy(oracle.quantize(oracle.NAIVE, fmt, B, W)[2])


def test_block_pairs_sharing_an_amax_are_on_the_diagonal():
    """When both 8-weight halves of every 16-weight block hold the block's
    largest magnitude, B = 8 and B = 16 pick the same scale and the same
    codes: every block is on the diagonal, none above."""
    W = tensor(1e-2).copy()
    blk = W.reshape(W.shape[0], -1, 16)
    m = np.abs(blk).max(axis=2) * 1.5
    blk[:, :, 0] = m
    blk[:, :, 8] = -m
    W = blk.reshape(W.shape).astype(np.float32)
    for fmt in (oracle.NVFP4, oracle.NVFP4_UE5M3, oracle.FP4_F16):
        r = bench.block_pair_comparison(objectives(fmt, 8, W), objectives(fmt, 16, W))
        assert r["above"] == 0.0 and r["below"] == 0.0 and r["equal"] == 1.0


def test_about_a_quarter_of_blocks_above_the_diagonal():
    """"Is Finer Better?" §3.2: with UE4M3 scales about 25% of 16-weight
    blocks have a larger error at B = 8 than at B = 16 (a real tensor there;
    the config-4 stand-in weights here)."""
    W = synth.bits(synth.config_inputs(4, rows=256)[0])
    r = bench.block_pair_comparison(objectives(oracle.NVFP4, 8, W), objectives(oracle.NVFP4, 16, W))
    assert 0.15 < r["above"] < 0.4
    assert abs(r["above"] + r["equal"] + r["below"] - 1.0) < 1e-12


def _decomp(fmt, B, W):
    c, s, _ = oracle.quantize(oracle.NAIVE, fmt, B, W)
    Wq = oracle.dequantize(fmt, B, c, s, *W.shape)
    parts = bench.mse_decomposition(torch.from_numpy(W), torch.from_numpy(Wq), torch.from_numpy(s == 0), B)
    return parts, float(np.mean((Wq.astype(np.float64) - W.astype(np.float64)) ** 2))


@pytest.mark.parametrize("B", [4, 8, 16, 32])
def test_mse_parts_add_up(B):
    for sigma in (1e-3, 1e-2, 1e-1):
        parts, total = _decomp(oracle.NVFP4, B, tensor(sigma))
        assert sum(parts.values()) == pytest.approx(total, rel=1e-12)


def test_mse_parts_at_the_ends():
    """A tensor whose every block falls into the zero bin is all zero-scale
    error; binary16 scales never zero a block; a block whose maximum is
    exactly 6 s for a UE4M3 value s has no error at the maximum."""
    parts, total = _decomp(oracle.NVFP4, 8, tensor(3e-4))
    assert parts["s_zero"] == pytest.approx(total, rel=1e-12) and parts["x_max"] == 0.0 == parts["x_other"]
    parts, _ = _decomp(oracle.FP4_F16, 8, tensor(1e-2))
    assert parts["s_zero"] == 0.0 and parts["x_max"] > 0.0
    W = tensor(1e-2).copy()
    blk = W.reshape(W.shape[0], -1, 8)
    blk[:] = np.clip(blk, -0.3, 0.3)
    blk[:, :, 3] = 0.375  # 6 x 2^-4: the Naive UE4M3 scale is exactly 2^-4
    W = blk.reshape(W.shape).astype(np.float32)
    parts, _ = _decomp(oracle.NVFP4, 8, W)
    assert parts["x_max"] == 0.0 and parts["x_other"] > 0.0 and parts["s_zero"] == 0.0
