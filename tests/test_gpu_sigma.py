"""GPU parity of the block-size / sigma study ("Is Finer Better?", §3.2,
§4.3, §5.2): N(0, sigma^2) tensors quantised with E2M1 elements and Naive
scales on the UE4M3 (E4M3), UE5M3 and binary16 grids.  Codes and scales are
bit-exact with the oracle, and the per-tensor MSE (from weight_error's float64
sums) matches the oracle's to 1e-12 relative; the crossover and the
zero-scale collapse are checked on the GPU's own numbers."""
import numpy as np
import pytest
import torch

import oracle
import synth
import block_scaled_precision_hdiag_amd as hd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hd.lib()


Z = None


def tensor(sigma):
    global Z
    if Z is None:
        Z = synth.weights("normal", 128, 4096, std=1.0, seed=61, dtype=torch.float32)
    return (Z * sigma).contiguous()


def gpu_mse(fmt, B, W):
    Wd = W.cuda()
    c, s, _ = hd.quantize_blocks(hd.NAIVE, fmt, B, Wd)
    Wq = hd.dequantize(fmt, B, c, s, *W.shape)
    _, sums = hd.weight_error(Wd, Wq, sums=True)
    torch.cuda.synchronize()
    return c, s, sums[0].item() / W.numel()


@pytest.mark.parametrize("sigma", [3e-4, 1e-2, 5e-2])
@pytest.mark.parametrize("fmt", [hd.NVFP4, hd.NVFP4_UE5M3, hd.FP4_F16])
@pytest.mark.parametrize("B", [4, 8, 16])
def test_sigma_mse_parity(sigma, fmt, B):
    W = tensor(sigma)
    c, s, m = gpu_mse(fmt, B, W)
    Wn = W.numpy()
    c_o, s_o, _ = oracle.quantize(oracle.NAIVE, fmt, B, Wn)
    np.testing.assert_array_equal(c.cpu().numpy(), c_o)
    s_g = s.cpu().view(torch.int16).numpy().view(np.uint16) if s.dtype == torch.float16 else s.cpu().numpy()
    np.testing.assert_array_equal(s_g, s_o)
    Wq_o = oracle.dequantize(fmt, B, c_o, s_o, *Wn.shape)
    _, d2, _ = oracle.weight_error(Wn, Wq_o, sums=True)
    assert m == pytest.approx(d2 / Wn.size, rel=1e-12)


def test_crossover_and_collapse_on_the_gpu():
    lo, hi, tiny = tensor(1e-2), tensor(5e-2), tensor(3e-4)
    assert gpu_mse(hd.NVFP4, 8, lo)[2] > gpu_mse(hd.NVFP4, 16, lo)[2]
    assert gpu_mse(hd.NVFP4, 8, hi)[2] < gpu_mse(hd.NVFP4, 16, hi)[2]
    for fmt in (hd.NVFP4_UE5M3, hd.FP4_F16):
        assert gpu_mse(fmt, 8, lo)[2] < gpu_mse(fmt, 16, lo)[2]
    m = gpu_mse(hd.NVFP4, 16, tiny)[2]
    assert m == pytest.approx(float((tiny.double() ** 2).mean()), rel=1e-12)


@pytest.mark.parametrize("sigma", [3e-3, 1e-2, 5e-2])
@pytest.mark.parametrize("fmt", [hd.NVFP4, hd.NVFP4_UE5M3, hd.FP4_F16])
def test_block_pair_comparison_parity(sigma, fmt):
    """Fig. 2(a) of "Is Finer Better?": the per-block objectives at B = 8 and
    B = 16 from the kernels match the oracle's (float32 of the float64 sum,
    2e-6), and the fractions of 16-weight blocks above / on / below the
    diagonal come out the same from both."""
    import bench

    W = tensor(sigma)
    Wd = W.cuda()
    r = {}
    for src in ("gpu", "oracle"):
        o = {}
        for B in (8, 16):
            if src == "gpu":
                o[B] = hd.quantize_blocks(hd.NAIVE, fmt, B, Wd, block_obj=True)[2].cpu()
            else:
                o[B] = torch.from_numpy(oracle.quantize(oracle.NAIVE, fmt, B, W.numpy())[2])
        r[src] = (bench.block_pair_comparison(o[8], o[16]), o)
    for B in (8, 16):
        np.testing.assert_allclose(r["gpu"][1][B].numpy(), r["oracle"][1][B].numpy().astype(np.float32), rtol=2e-6)
    assert r["gpu"][0] == r["oracle"][0]
