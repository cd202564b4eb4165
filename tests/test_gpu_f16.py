"""GPU parity (through the C ABI) of the FP16-scale formats FP4_F16 and
INT4_F16 with the oracle: binary16 block scales, Naive and the SSE / H
alternation of qwantize "Results", "Larger blocks: bs=64 (E4M3 scales) and
bs=128 (FP16 scales)".

Bars: Naive scales and codes bit-exact; encode at given scales bit-exact for
every finite bf16 value at a sample of binary16 scales spanning subnormals to
65504; alternation scales identical on >= 99.99% of blocks (the sums of s* are
exact float64 products added in a different order, so a differing block can
only come from a float64 rounding tie; any such block's oracle objective at the
GPU's scale must be within 1e-6 relative of the oracle's), element codes
bit-exact at the GPU's scales, block objectives within 2e-6 (float32 of a
float64 sum); dequantize bit-exact (fp32) and RNE-exact (bf16).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import block_scaled_precision_hdiag_amd as hd

pytestmark = pytest.mark.gpu

F16 = [hd.FP4_F16, hd.INT4_F16]
BLOCKS = [8, 16, 32, 64, 128, 256]
C = {hd.FP4_F16: 6.0, hd.INT4_F16: 7.0}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hd.lib()


def dev(t):
    return t.contiguous().cuda()


def npy(t):
    return t.detach().cpu().numpy()


def s_bits(t):
    """binary16 bits (uint16) of a float16 scale tensor"""
    return npy(t.view(torch.int16)).view(np.uint16)


def s_tensor(bits):
    return dev(torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.float16))


def weights(N, K, seed, dtype=torch.bfloat16):
    return synth.weights("t4", N, K, std=0.02, seed=seed, gain_seed=seed + 1, dtype=dtype)


def h_for(K, seed):
    X = synth.activations(512, K, seed, n_out=4, out_gain=50.0, idx_seed=seed + 1, dtype=torch.float32)
    return oracle.hdiag(synth.bits(X))


def with_edge_rows(W, B):
    """rows 0-3: an all-zero block, a single negative non-zero, a block below
    the binary16 range (zero scale) and one beyond it (saturated scale)"""
    W = W.float().clone()
    W[0, :B] = 0.0
    W[1, :B] = 0.0
    W[1, 3] = -0.3
    W[2, :B] = 2.0 ** -30
    W[3, :B] = 1e6
    return W


@pytest.mark.parametrize("fmt", F16)
@pytest.mark.parametrize("B", BLOCKS)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_naive_bit_exact(fmt, B, dtype):
    N, K = 37, 1024
    W = with_edge_rows(weights(N, K, 2000 + fmt * 10 + B, dtype), B).to(dtype)
    h = h_for(K, 7)
    c_o, s_o, obj_o = oracle.quantize(hd.NAIVE, fmt, B, synth.bits(W), h=h)
    c_g, s_g, obj_g = hd.quantize_blocks(hd.NAIVE, fmt, B, dev(W), h=dev(torch.from_numpy(h)), block_obj=True)
    torch.cuda.synchronize()
    assert s_g.dtype == torch.float16
    np.testing.assert_array_equal(s_bits(s_g), s_o)
    np.testing.assert_array_equal(npy(c_g), c_o)
    np.testing.assert_allclose(npy(obj_g), obj_o.astype(np.float32), rtol=2e-6)
    # the scale tensor holds the scale values themselves
    np.testing.assert_array_equal(npy(s_g.float()), s_o.view(np.float16).astype(np.float32))


SAMPLE_SCALES = [1, 2, 3, 0x3FF, 0x400, 0x401, 0x1000, 0x2E66, 0x3165, 0x3C00, 0x3C01, 0x4000, 0x5000,
                 0x7000, 0x7BFE, 0x7BFF]


@pytest.mark.parametrize("fmt", F16)
def test_encode_every_bf16_at_sampled_scales(fmt):
    """Every finite bf16 value (both signs) encoded at 40 binary16 scales
    (subnormal, normal and the largest, plus random ones): bit-exact codes."""
    pos = np.arange(0, 0x7F80, dtype=np.uint32)
    x = np.concatenate([pos, pos | 0x8000]).astype(np.uint16)  # 65280 values
    B = 128
    rng = np.random.default_rng(3)
    sc = np.array(SAMPLE_SCALES + list(rng.integers(1, 0x7BFF, 40 - len(SAMPLE_SCALES))), np.uint16)
    W = np.tile(x, (sc.size, 1))
    scales = np.repeat(sc[:, None], x.size // B, axis=1)
    c_o, _, _ = oracle.quantize(hd.NAIVE, fmt, B, W, scales_in=scales)
    Wg = dev(torch.from_numpy(W.view(np.int16)).view(torch.bfloat16))
    c_g, _ = hd.encode_blocks(fmt, B, Wg, s_tensor(scales))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(npy(c_g), c_o)


@pytest.mark.parametrize("fmt", F16)
def test_encode_fp32_random_at_sampled_scales(fmt):
    rng = np.random.default_rng(4)
    sc = np.array(SAMPLE_SCALES, np.uint16)
    K, B = 4096, 64
    s_val = sc.view(np.float16).astype(np.float64)
    # quotients spread over 0 .. 16 around each scale, plus far outliers
    W = (rng.uniform(-16, 16, (sc.size, K)) * s_val[:, None]).astype(np.float32)
    W[:, :64] *= np.float32(1e6)
    scales = np.repeat(sc[:, None], K // B, axis=1)
    c_o, _, obj_o = oracle.quantize(hd.NAIVE, fmt, B, W, scales_in=scales)
    c_g, obj_g = hd.encode_blocks(fmt, B, dev(torch.from_numpy(W)), s_tensor(scales), block_obj=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(npy(c_g), c_o)
    np.testing.assert_allclose(npy(obj_g), obj_o.astype(np.float32), rtol=2e-6)


def check_alternation(fmt, B, W, h, method, frac=0.9999):
    Wo = synth.bits(W)
    hh = h if method == hd.H_OPT else None
    c_o, s_o, obj_o = oracle.quantize(method, fmt, B, Wo, h=hh)
    hdev = dev(torch.from_numpy(h)) if hh is not None else None
    c_g, s_g, obj_g = hd.quantize_blocks(method, fmt, B, dev(W), h=hdev, block_obj=True)
    torch.cuda.synchronize()
    sg, c_g, obj_g = s_bits(s_g), npy(c_g), npy(obj_g)
    same = sg == s_o
    assert same.mean() >= frac, "scale agreement %.6f" % same.mean()
    at = oracle.objectives_at(fmt, B, Wo, sg, h=hh)
    if not same.all():
        rel = (at - obj_o) / np.maximum(obj_o, 1e-300)
        assert np.all(rel[~same] <= 1e-6), rel[~same].max()
    c_ref, _, _ = oracle.quantize(hd.NAIVE, fmt, B, Wo, scales_in=sg)
    np.testing.assert_array_equal(c_g, c_ref)
    np.testing.assert_allclose(obj_g, at.astype(np.float32), rtol=2e-6, atol=0)
    return same.mean()


@pytest.mark.parametrize("fmt", F16)
@pytest.mark.parametrize("B", BLOCKS)
@pytest.mark.parametrize("method", [hd.SSE_OPT, hd.H_OPT])
def test_alternation_parity(fmt, B, method):
    N, K = 301, 2048  # ragged row count: the last workgroup is partly empty
    W = with_edge_rows(weights(N, K, 3000 + fmt * 10 + B), B).to(torch.bfloat16)
    check_alternation(fmt, B, W, h_for(K, 11), method)


@pytest.mark.parametrize("fmt", F16)
@pytest.mark.parametrize("method", [hd.SSE_OPT, hd.H_OPT])
def test_alternation_parity_fp32_inputs(fmt, method):
    N, K = 129, 1024
    W = weights(N, K, 4000 + fmt, torch.float32)
    W[5] *= 2.0 ** -20  # scales in the binary16 subnormal range
    W[6] *= 2.0 ** 12   # and near its top
    check_alternation(fmt, 128, W, h_for(K, 12), method)
    check_alternation(fmt, 16, W, h_for(K, 12), method)


@pytest.mark.parametrize("fmt", F16)
def test_alternation_never_worse_than_naive(fmt):
    """The result is the best visited scale, Naive included: per block its
    objective is <= Naive's (GPU objectives, each method's own weighting)."""
    N, K, B = 256, 4096, 128
    W = dev(weights(N, K, 51))
    h = dev(torch.from_numpy(h_for(K, 13)))
    for m in (hd.SSE_OPT, hd.H_OPT):
        hh = h if m == hd.H_OPT else None
        _, _, on = hd.quantize_blocks(hd.NAIVE, fmt, B, W, h=hh, block_obj=True)
        _, _, om = hd.quantize_blocks(m, fmt, B, W, h=hh, block_obj=True)
        torch.cuda.synchronize()
        assert bool((om <= on).all())
        assert float(om.double().sum()) < float(on.double().sum())


@pytest.mark.parametrize("fmt", F16)
@pytest.mark.parametrize("B", [16, 128])
def test_dequantize_and_weight_error(fmt, B):
    N, K = 65, 1024
    W = weights(N, K, 5000 + B)
    c, s, _ = hd.quantize_blocks(hd.SSE_OPT, fmt, B, dev(W))
    Wq = hd.dequantize(fmt, B, c, s, N, K)
    Wq16 = hd.dequantize(fmt, B, c, s, N, K, dtype=torch.bfloat16)
    we = hd.weight_error(dev(W), Wq).item()
    torch.cuda.synchronize()
    Wq_o = oracle.dequantize(fmt, B, npy(c), s_bits(s), N, K)
    np.testing.assert_array_equal(npy(Wq), Wq_o)
    np.testing.assert_array_equal(npy(Wq16.float()), torch.from_numpy(Wq_o).to(torch.bfloat16).float().numpy())
    assert we == pytest.approx(oracle.weight_error(synth.bits(W), Wq_o), rel=1e-9)


def test_invalid_scale_codes_decode_to_zero():
    """binary16 patterns above 0x7BFF (Inf, NaN, negative) are not scales:
    encode uses the zero scale for them and dequantize gives 0."""
    N, K, B = 4, 256, 128
    W = weights(N, K, 6)
    bits = np.full((N, K // B), 0x3C00, np.uint16)
    bits[1, 0], bits[2, 1], bits[3, 0] = 0x7C00, 0x7E00, 0xBC00
    c, _ = hd.encode_blocks(hd.FP4_F16, B, dev(W), s_tensor(bits))
    Wq = npy(hd.dequantize(hd.FP4_F16, B, c, s_tensor(bits), N, K))
    c_o, _, _ = oracle.quantize(hd.NAIVE, hd.FP4_F16, B, synth.bits(W), scales_in=np.where(bits > 0x7BFF, 0, bits))
    np.testing.assert_array_equal(npy(c), c_o)
    assert not Wq[1, :B].any() and not Wq[2, B:].any() and not Wq[3, :B].any()


def test_output_error_codes_unsupported():
    X = dev(synth.activations(64, 256, 1, dtype=torch.bfloat16))
    W = dev(weights(32, 256, 2))
    ref = hd.output_reference(X, W)
    c, s, _ = hd.quantize_blocks(hd.NAIVE, hd.FP4_F16, 128, W)
    with pytest.raises(hd.HdiagError) as e:
        hd.output_error_codes(hd.FP4_F16, 128, X, c, s, ref, 32, 256)
    assert e.value.status == hd.HD_ERR_UNSUPPORTED


@pytest.mark.parametrize("fmt", F16)
def test_fullsize_down_proj_sampled_rows(fmt):
    """The down_proj stand-in at full size (W 2560 x 9728 bf16, B = 128, the
    pages' FP16-scale block size) in the benchmark's launch configuration; the
    oracle checks 50 sampled rows (blocks are independent).  h comes from the
    first 2048 rows of X."""
    W, X = synth.config_inputs(2, x_rows=2048)
    N, K = W.shape
    B = 128
    h = oracle.hdiag(synth.bits(X))
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(8).choice(N, 48, replace=False)]))
    Wd, hd_dev = dev(W), dev(torch.from_numpy(h))
    Ws = np.ascontiguousarray(synth.bits(W)[rows])
    for m in (hd.NAIVE, hd.SSE_OPT, hd.H_OPT):
        hh = h if m == hd.H_OPT else None
        c_g, s_g, o_g = hd.quantize_blocks(m, fmt, B, Wd, h=hd_dev if hh is not None else None, block_obj=True)
        torch.cuda.synchronize()
        c_o, s_o, o_o = oracle.quantize(m, fmt, B, Ws, h=hh)
        np.testing.assert_array_equal(s_bits(s_g)[rows], s_o)
        np.testing.assert_array_equal(npy(c_g)[rows], c_o)
        np.testing.assert_allclose(npy(o_g)[rows], o_o.astype(np.float32), rtol=2e-6)
