"""GPU parity of the reference-based output error (output_reference +
output_error_codes) against the oracle.

Y = X W^T is compared entry by entry with the oracle's float64 product, within
the float32-accumulation bound 1e-5 * sum_k |x_k w_k|; the output error of each
format's codes is compared with the oracle's output error of the dequantised
weights (the definition), within 1e-4 relative.  Shapes span several
256 x 256 tiles with ragged edges and K tails that are not multiples of 64.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import block_scaled_precision_hdiag_amd as hd

pytestmark = pytest.mark.gpu

FMTS = [hd.INT8_E4M3, hd.NVFP4, hd.MXFP4, hd.MXFP8, hd.FP8_E4M3S, hd.NVFP4_UE4M4, hd.NVFP4_UE5M3, hd.NVINT4]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hd.lib()


def dev(t):
    return t.contiguous().cuda()


def npy(t):
    return t.detach().cpu().numpy()


def weights_for(fmt, N, K, seed):
    std = {hd.FP8_E4M3S: 4.0, hd.MXFP8: 0.05}.get(fmt, 0.02)
    return synth.weights("t4", N, K, std=std, seed=seed, gain_seed=seed + 1, dtype=torch.bfloat16)


def acts(M, K, seed):
    return synth.activations(M, K, seed, n_out=3, out_gain=50.0, idx_seed=seed + 1, dtype=torch.bfloat16)


def check_y(X, W, ref):
    M, N = X.shape[0], W.shape[0]
    Y = npy(hd.reference_y(ref, M, N))
    ysq = hd.reference_ysq(ref).item()
    Xb, Wb = synth.bits(X), synth.bits(W)
    Yo = oracle.matmul_nt(Xb, Wb)
    bound = oracle.matmul_nt(np.abs(X.float().numpy()), np.abs(W.float().numpy()))
    err = np.abs(Y.astype(np.float64) - Yo)
    assert np.all(err <= 1e-5 * bound + 1e-30), float((err / np.maximum(bound, 1e-30)).max())
    assert ysq == pytest.approx(float((Yo ** 2).sum()), rel=1e-5)


@pytest.mark.parametrize("M,N,K", [(300, 200, 512), (257, 300, 520), (64, 64, 16), (513, 257, 1024), (1, 1, 8)])
def test_output_reference_y(M, N, K):
    X, W = acts(M, K, 31 + M), weights_for(hd.NVFP4, N, K, 900 + N)
    ref = hd.output_reference(dev(X), dev(W))
    torch.cuda.synchronize()
    check_y(X, W, ref)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B,M,N,K", [(16, 300, 200, 512), (256, 257, 300, 1024), (8, 70, 40, 520)])
def test_output_error_codes_parity(fmt, B, M, N, K):
    X, W = acts(M, K, 40 + B), weights_for(fmt, N, K, 950 + B)
    Xd, Wd = dev(X), dev(W)
    c, s, _ = hd.quantize_blocks(hd.SSE_OPT, fmt, B, Wd)
    ref = hd.output_reference(Xd, Wd)
    out, sums = hd.output_error_codes(fmt, B, Xd, c, s, ref, N, K, sums=True)
    Wq = hd.dequantize(fmt, B, c, s, N, K)
    generic = hd.output_error(Xd, Wd, Wq).item()
    torch.cuda.synchronize()
    oe_o, d_o, y_o = oracle.output_error(synth.bits(X), synth.bits(W), oracle.dequantize(fmt, B, npy(c), npy(s), N, K),
                                         sums=True)
    assert out.item() == pytest.approx(oe_o, rel=1e-4)
    np.testing.assert_allclose(npy(sums), [d_o, y_o], rtol=2e-4)
    assert out.item() == pytest.approx(generic, rel=1e-4)
    assert sums[1].item() == hd.reference_ysq(ref).item()


def test_output_error_codes_x_dynamic_range():
    """Rows of X spread over 2^-60 .. 2^60, a zero row and a 1e4 outlier
    channel: the per-row power-of-two carried with the fp16 copy of X (INT8)
    keeps every row exact."""
    M, N, K = 96, 80, 256
    X = acts(M, K, 5).float()
    X *= torch.from_numpy(np.exp2(np.linspace(-60, 60, M)).astype(np.float32))[:, None]
    X[7] = 0.0
    X[:, 11] *= 1e4
    X = X.to(torch.bfloat16)
    for fmt, B in ((hd.INT8_E4M3, 32), (hd.NVFP4, 16), (hd.MXFP8, 32)):
        W = weights_for(fmt, N, K, 77)
        Xd, Wd = dev(X), dev(W)
        c, s, _ = hd.quantize_blocks(hd.NAIVE, fmt, B, Wd)
        ref = hd.output_reference(Xd, Wd)
        out = hd.output_error_codes(fmt, B, Xd, c, s, ref, N, K).item()
        Wq = oracle.dequantize(fmt, B, npy(c), npy(s), N, K)
        assert out == pytest.approx(oracle.output_error(synth.bits(X), synth.bits(W), Wq), rel=1e-4)


def test_output_error_codes_on_grid_is_zero():
    """W built on the NVFP4 grid: the bf16 operand is W itself, the product is
    the reference's to the bit, and D = 0 exactly."""
    M, N, K, B = 300, 260, 512, 16
    W0 = weights_for(hd.NVFP4, N, K, 3)
    c, s, _ = hd.quantize_blocks(hd.NAIVE, hd.NVFP4, B, dev(W0))
    Wg = hd.dequantize(hd.NVFP4, B, c, s, N, K, dtype=torch.bfloat16)  # exact in bf16
    c2, _ = hd.encode_blocks(hd.NVFP4, B, Wg, s)  # re-encoding at the same scales is exact
    s2 = s
    assert torch.equal(hd.dequantize(hd.NVFP4, B, c2, s2, N, K, dtype=torch.bfloat16), Wg)
    X = dev(acts(M, K, 9))
    ref = hd.output_reference(X, Wg)
    out, sums = hd.output_error_codes(hd.NVFP4, B, X, c2, s2, ref, N, K, sums=True)
    torch.cuda.synchronize()
    assert out.item() == 0.0 and sums[0].item() == 0.0


def test_output_error_codes_reuse_and_streams():
    """One reference serves several quantisations; results do not depend on
    call order and repeat bit for bit."""
    M, N, K = 300, 200, 512
    X, W = dev(acts(M, K, 12)), dev(weights_for(hd.INT8_E4M3, N, K, 13))
    ref = hd.output_reference(X, W)
    res = []
    for B in (32, 64, 128):
        c, s, _ = hd.quantize_blocks(hd.SSE_OPT, hd.INT8_E4M3, B, W)
        res.append((c, s, B, hd.output_error_codes(hd.INT8_E4M3, B, X, c, s, ref, N, K).item()))
    for c, s, B, v in reversed(res):
        assert hd.output_error_codes(hd.INT8_E4M3, B, X, c, s, ref, N, K).item() == v


def test_output_reference_unsupported():
    X = torch.randn(8, 16, device="cuda")
    W = torch.randn(4, 16, device="cuda")
    with pytest.raises(hd.HdiagError) as e:
        hd.output_reference(X, W, ref=torch.empty(hd.output_reference_size(8, 4, 16), dtype=torch.uint8,
                                                  device="cuda"))
    assert e.value.status == hd.HD_ERR_UNSUPPORTED
