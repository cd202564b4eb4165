"""GPU parity of per-tensor scaling over E4M3 block scales ("Is Finer
Better?" §5.1, UE4M3-S) with the oracle: the tensor scale, the block scales
and the codes bit-exact (the blocks see the same W / s_T, an IEEE division on
both sides), block objectives within 2e-6 (float32 of a float64 sum),
dequantised values bit-exact in float32 and RNE-exact in bfloat16."""
import numpy as np
import pytest
import torch

import oracle
import synth
import block_scaled_precision_hdiag_amd as hd

pytestmark = pytest.mark.gpu

FMTS = [hd.NVFP4, hd.NVINT4, hd.FP8_E4M3S, hd.INT8_E4M3]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hd.lib()


def npy(t):
    return t.detach().cpu().numpy()


def h_for(K, seed):
    X = synth.activations(256, K, seed, n_out=4, out_gain=50.0, idx_seed=seed + 1, dtype=torch.float32)
    return oracle.hdiag(synth.bits(X))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B", [16, 128])
@pytest.mark.parametrize("method", [hd.NAIVE, hd.SSE_OPT, hd.H_OPT])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("std", [3e-4, 0.02])
def test_tensor_scaled_parity(fmt, B, method, dtype, std):
    N, K = 37, 1024
    W = synth.weights("t4", N, K, std=std, seed=70 + B, gain_seed=71, dtype=dtype)
    h = h_for(K, 9)
    hh = h if method == hd.H_OPT else None
    c, s, ts, obj = hd.quantize_blocks_tensor_scaled(method, fmt, B, W.cuda(),
                                                     h=torch.from_numpy(h).cuda() if hh is not None else None,
                                                     block_obj=True)
    torch.cuda.synchronize()
    c_o, s_o, t_o, obj_o = oracle.quantize_tensor_scaled(method, fmt, B, synth.bits(W), h=hh)
    assert npy(ts)[0] == t_o
    np.testing.assert_array_equal(npy(s), s_o)
    np.testing.assert_array_equal(npy(c), c_o)
    np.testing.assert_allclose(npy(obj), obj_o.astype(np.float32), rtol=2e-6)
    Wq = npy(hd.dequantize_tensor_scaled(fmt, B, c, s, ts, N, K))
    Wq_o = oracle.dequantize_tensor_scaled(fmt, B, c_o, s_o, t_o, N, K)
    np.testing.assert_array_equal(Wq, Wq_o)
    Wq16 = hd.dequantize_tensor_scaled(fmt, B, c, s, ts, N, K, dtype=torch.bfloat16)
    np.testing.assert_array_equal(npy(Wq16.float()), torch.from_numpy(Wq_o).to(torch.bfloat16).float().numpy())


def test_zero_tensor_and_invalid_formats():
    W = torch.zeros(8, 256, device="cuda")
    c, s, ts, _ = hd.quantize_blocks_tensor_scaled(hd.NAIVE, hd.NVFP4, 16, W)
    torch.cuda.synchronize()
    assert ts.item() == 1.0 and not c.any() and not s.any()
    for fmt in (hd.MXFP4, hd.NVFP4_UE5M3, hd.FP4_F16):
        with pytest.raises(hd.HdiagError):
            hd.quantize_blocks_tensor_scaled(hd.NAIVE, fmt, 16, W)
    with pytest.raises(hd.HdiagError):
        hd.quantize_blocks_tensor_scaled(hd.NAIVE_OCP, hd.NVFP4, 16, W)
