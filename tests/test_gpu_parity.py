"""Parity of the HIP path (through the C ABI) with the CPU oracle on the GPU.

Bars (stated per test): bit-exact codes and scales for Naive and for encode
with given scales; for the searches, identical scale codes on >= 99.99% of
blocks and, on any block that differs, the oracle's objective at the GPU's
scale within 1e-6 relative of the oracle's minimum (several scales can be
correct at a tie); element codes bit-exact at the scale the GPU chose;
hdiag within 1e-6 relative (both sum exact squares in float64); the error
metrics within 1e-4 relative (the output error runs on bf16 MFMA).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import block_scaled_precision_hdiag_amd as hd

pytestmark = pytest.mark.gpu

FMTS = [hd.INT8_E4M3, hd.NVFP4, hd.MXFP4, hd.MXFP8, hd.FP8_E4M3S, hd.NVFP4_UE4M4, hd.NVFP4_UE5M3, hd.NVINT4]
BLOCKS = [8, 16, 32, 64, 128, 256]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hd.lib()


def dev(t):
    return t.contiguous().cuda()


def npy(t):
    return t.detach().cpu().numpy()


def weights_for(fmt, N, K, seed, dtype=torch.bfloat16):
    # magnitudes that keep every format's competitive scales away from the grid ends
    std = {hd.FP8_E4M3S: 4.0, hd.MXFP8: 0.05}.get(fmt, 0.02)
    return synth.weights("t4", N, K, std=std, seed=seed, gain_seed=seed + 1, dtype=dtype)


def h_for(K, seed):
    X = synth.activations(512, K, seed, n_out=4, out_gain=50.0, idx_seed=seed + 1, dtype=torch.float32)
    return oracle.hdiag(synth.bits(X))


def check_search(fmt, B, W, h, method, frac=0.9999):
    Wo = synth.bits(W)
    hh = h if method == hd.H_OPT else None
    c_o, s_o, obj_o = oracle.quantize(method, fmt, B, Wo, h=hh)
    hdev = dev(torch.from_numpy(h)) if hh is not None else None
    c_g, s_g, obj_g = hd.quantize_blocks(method, fmt, B, dev(W), h=hdev, block_obj=True)
    torch.cuda.synchronize()
    s_g, c_g, obj_g = npy(s_g), npy(c_g), npy(obj_g)
    same = s_g == s_o
    assert same.mean() >= frac, "scale agreement %.6f" % same.mean()
    if not same.all():
        at = oracle.objectives_at(fmt, B, Wo, s_g, h=hh)
        rel = (at - obj_o) / np.maximum(obj_o, 1e-300)
        assert np.all(rel[~same] <= 1e-6), rel[~same].max()
    # element codes: bit-exact at the scales the GPU chose
    c_ref, _, _ = oracle.quantize(hd.NAIVE, fmt, B, Wo, scales_in=s_g)
    np.testing.assert_array_equal(c_g, c_ref)
    np.testing.assert_allclose(obj_g, obj_o.astype(np.float32), rtol=2e-6, atol=0)
    return same.mean()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B", BLOCKS)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_naive_bit_exact(fmt, B, dtype):
    N, K = 37, 3 * 256 + B * (1 if B < 256 else 0)  # ragged row count, several column tiles
    K = (K // B) * B
    W = weights_for(fmt, N, K, 1000 + fmt * 10 + B, dtype)
    h = h_for(K, 7)
    c_o, s_o, obj_o = oracle.quantize(hd.NAIVE, fmt, B, synth.bits(W), h=h)
    c_g, s_g, obj_g = hd.quantize_blocks(hd.NAIVE, fmt, B, dev(W), h=dev(torch.from_numpy(h)), block_obj=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(npy(s_g), s_o)
    np.testing.assert_array_equal(npy(c_g), c_o)
    np.testing.assert_allclose(npy(obj_g), obj_o.astype(np.float32), rtol=2e-6)


ALL_FMTS = FMTS + [hd.FP4_F16, hd.INT4_F16]


def scales_np(s):
    return npy(s.view(torch.int16)).view(np.uint16) if s.dtype == torch.float16 else npy(s)


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_block4_naive_encode_dequantize_bit_exact(fmt, dtype):
    """B = 4 ("Is Finer Better?" App. F's smallest block): two blocks per
    8-weight lane chunk.  Naive scales, codes and (h-weighted) objectives,
    encode with given scales, and dequantize to float32 and bfloat16, all
    bit-exact with the oracle; all-zero and single-nonzero blocks included."""
    N, K, B = 37, 1032, 4  # ragged rows, K % 512 != 0
    W = weights_for(fmt, N, K, 7000 + fmt, dtype).float()
    W[2, :4] = 0.0
    W[3, 4:8] = 0.0
    W[3, 5] = 1.0
    W = W.to(dtype)
    h = h_for(K, 17)
    hd_h = dev(torch.from_numpy(h))
    c_o, s_o, obj_o = oracle.quantize(hd.NAIVE, fmt, B, synth.bits(W), h=h)
    c_g, s_g, obj_g = hd.quantize_blocks(hd.NAIVE, fmt, B, dev(W), h=hd_h, block_obj=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(scales_np(s_g), s_o)
    np.testing.assert_array_equal(npy(c_g), c_o)
    np.testing.assert_allclose(npy(obj_g), obj_o.astype(np.float32), rtol=2e-6)
    # encode at given scales (every block at a scale shifted from its Naive one)
    s_in = s_g.clone()
    if s_in.dtype == torch.uint8:
        s_in = torch.clamp(s_in.to(torch.int16) - 3, 1, 126).to(torch.uint8)
    c_e, _ = hd.encode_blocks(fmt, B, dev(W), s_in)
    c_eo, _, _ = oracle.quantize(hd.NAIVE, fmt, B, synth.bits(W), scales_in=scales_np(s_in))
    np.testing.assert_array_equal(npy(c_e), c_eo)
    deq_o = oracle.dequantize(fmt, B, c_o, s_o, N, K)
    np.testing.assert_array_equal(npy(hd.dequantize(fmt, B, c_g, s_g, N, K)), deq_o)
    deq_b = hd.dequantize(fmt, B, c_g, s_g, N, K, dtype=torch.bfloat16)
    assert torch.equal(deq_b.cpu(), torch.from_numpy(deq_o).to(torch.bfloat16))


@pytest.mark.parametrize("fmt", [hd.MXFP4, hd.MXFP8])
def test_block4_ocp_and_tensor_scaled(fmt):
    N, K, B = 20, 512, 4
    W = weights_for(fmt, N, K, 7100 + fmt)
    c_o, s_o, _ = oracle.quantize(oracle.NAIVE_OCP, fmt, B, synth.bits(W))
    c_g, s_g, _ = hd.quantize_blocks(hd.NAIVE_OCP, fmt, B, dev(W))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(npy(s_g), s_o)
    np.testing.assert_array_equal(npy(c_g), c_o)
    Wn = weights_for(hd.NVFP4, N, K, 7200)
    c_t, s_t, ts, _ = hd.quantize_blocks_tensor_scaled(hd.NAIVE, hd.NVFP4, B, dev(Wn))
    c_to, s_to, ts_o, _ = oracle.quantize_tensor_scaled(hd.NAIVE, hd.NVFP4, B, synth.bits(Wn))
    np.testing.assert_array_equal(npy(s_t), s_to)
    np.testing.assert_array_equal(npy(c_t), c_to)
    assert ts.item() == ts_o
    np.testing.assert_array_equal(npy(hd.dequantize_tensor_scaled(hd.NVFP4, B, c_t, s_t, ts, N, K)),
                                  oracle.dequantize_tensor_scaled(hd.NVFP4, B, c_to, s_to, ts_o, N, K))


@pytest.mark.parametrize("fmt", [hd.MXFP4, hd.MXFP8])
@pytest.mark.parametrize("B", [8, 32, 256])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_naive_ocp_bit_exact(fmt, B, dtype):
    """The OCP MX floor rule for power-of-two scales, bit-exact with the oracle
    (scales, codes, objectives), including all-zero and tiny blocks."""
    N, K = 41, 1024
    W = weights_for(fmt, N, K, 1500 + fmt * 10 + B, dtype).float()
    W[3, :B] = 0.0
    W[5, :B] *= 1e-30
    W = W.to(dtype)
    c_o, s_o, obj_o = oracle.quantize(oracle.NAIVE_OCP, fmt, B, synth.bits(W))
    c_g, s_g, obj_g = hd.quantize_blocks(hd.NAIVE_OCP, fmt, B, dev(W), block_obj=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(npy(s_g), s_o)
    np.testing.assert_array_equal(npy(c_g), c_o)
    np.testing.assert_allclose(npy(obj_g), obj_o.astype(np.float32), rtol=2e-6)
    with pytest.raises(hd.HdiagError):
        hd.quantize_blocks(hd.NAIVE_OCP, hd.NVFP4, 16, dev(W))


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_every_bf16_at_every_scale(fmt):
    """Every finite bf16 value (both signs) encoded at every candidate scale:
    bit-exact codes.  This runs the quotient / rounding helpers of the search."""
    pos = np.arange(0, 0x7F80, dtype=np.uint32)
    allbits = np.concatenate([pos, pos | 0x8000]).astype(np.uint16)
    B = 8
    K = (allbits.size // B) * B
    x = allbits[:K]
    cands = oracle.candidates(fmt)
    W = np.tile(x, (cands.size, 1))
    scales = np.repeat(cands.astype(np.uint8)[:, None], K // B, axis=1)
    c_o, _, _ = oracle.quantize(hd.NAIVE, fmt, B, W, scales_in=scales)
    Wt = torch.from_numpy(W.view(np.int16)).view(torch.bfloat16)
    c_g, _ = hd.encode_blocks(fmt, B, dev(Wt), dev(torch.from_numpy(scales)))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(npy(c_g), c_o)


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_fp32_random_at_every_scale(fmt):
    rng = np.random.default_rng(3 + fmt)
    cands = oracle.candidates(fmt)
    K = 4096
    # log-uniform magnitudes over the range where the element codes change
    W = (np.exp(rng.uniform(-25, 12, (cands.size, K))) * rng.choice([-1, 1], (cands.size, K))).astype(np.float32)
    scales = np.repeat(cands.astype(np.uint8)[:, None], K // 8, axis=1)
    c_o, _, _ = oracle.quantize(hd.NAIVE, fmt, 8, W, scales_in=scales)
    c_g, _ = hd.encode_blocks(fmt, 8, dev(torch.from_numpy(W)), dev(torch.from_numpy(scales)))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(npy(c_g), c_o)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B", BLOCKS)
@pytest.mark.parametrize("method", [hd.SSE_OPT, hd.H_OPT])
def test_search_parity(fmt, B, method):
    N, K = 300, 1024  # 2 row tiles (ragged), 4..128 block columns
    W = weights_for(fmt, N, K, 2000 + fmt * 10 + B)
    check_search(fmt, B, W, h_for(K, 11), method)


@pytest.mark.parametrize("fmt", [hd.FP8_E4M3S, hd.MXFP8])
@pytest.mark.parametrize("B", BLOCKS)
@pytest.mark.parametrize("method", [hd.SSE_OPT, hd.H_OPT])
def test_search_parity_configs_width(fmt, B, method):
    """E4M3 elements at the configs' weight width (std 0.02, Student-t with a
    per-row gain), where the Naive E4M3 scale of most blocks falls into the
    zero bin and the search walks down to the grid's small-scale end."""
    N, K = 300, 1024
    W = synth.weights("t4", N, K, std=0.02, seed=2500 + fmt * 10 + B, gain_seed=2501 + B)
    if fmt == hd.FP8_E4M3S:
        _, s_n, _ = oracle.quantize(hd.NAIVE, fmt, B, synth.bits(W))
        assert (s_n == 0).mean() > 0.5  # the Naive collapse the pages describe
    check_search(fmt, B, W, h_for(K, 13), method)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("method", [hd.SSE_OPT, hd.H_OPT])
def test_search_parity_near_saturation(fmt, method):
    """Blocks with one outlier 6-40x the rest, so the optimum clips it: the
    chosen scale saturates an element in many blocks, where the kernel's
    float32 residual of the clipped element is rounded (at most 2^-24
    relative; the oracle subtracts exactly)."""
    N, K, B = 256, 1024, 32
    rng = np.random.default_rng(6000 + fmt)
    W = rng.standard_normal((N, K)) * 0.02
    col = rng.integers(0, B, (N, K // B)) + np.arange(K // B) * B
    W[np.arange(N)[:, None], col] *= rng.uniform(6.0, 40.0, (N, K // B))
    Wt = torch.from_numpy(W.astype(np.float32)).to(torch.bfloat16)
    frac = check_search(fmt, B, Wt, h_for(K, 14), method)
    assert frac >= 0.9999
    # the case is exercised: in some blocks the chosen scale clips the
    # outlier (|w| / s beyond the largest element)
    _, s_g, _ = hd.quantize_blocks(method, fmt, B, dev(Wt), h=dev(torch.from_numpy(h_for(K, 14))))
    sv = np.array([oracle.scale_value(fmt, int(c)) for c in range(256)])[npy(s_g).astype(np.int64)]
    qmax = {hd.INT8_E4M3: 127.0, hd.NVINT4: 7.0, hd.MXFP8: 448.0, hd.FP8_E4M3S: 448.0}.get(fmt, 6.0)
    amax = np.abs(Wt.float().numpy()).reshape(N, K // B, B).max(axis=2)
    if fmt != hd.FP8_E4M3S:  # E4M3 elements on E4M3 scales almost never clip
        assert (amax > qmax * sv).mean() > 0.01


@pytest.mark.parametrize("fmt", [hd.INT8_E4M3, hd.NVFP4])
def test_search_parity_fp32_inputs(fmt):
    W = weights_for(fmt, 100, 512, 31, dtype=torch.float32)
    for m in (hd.SSE_OPT, hd.H_OPT):
        check_search(fmt, 32, W, h_for(512, 12), m)


def test_config1_tiny_end_to_end():
    W, X = synth.config_inputs(1)
    h_o = oracle.hdiag(synth.bits(X))
    h_g = hd.hdiag(dev(X))
    torch.cuda.synchronize()
    np.testing.assert_allclose(npy(h_g), h_o, rtol=1e-6)
    for m in (hd.NAIVE, hd.SSE_OPT, hd.H_OPT):
        if m == hd.NAIVE:
            c_o, s_o, _ = oracle.quantize(m, hd.INT8_E4M3, 32, synth.bits(W))
            c_g, s_g, _ = hd.quantize_blocks(m, hd.INT8_E4M3, 32, dev(W))
            np.testing.assert_array_equal(npy(s_g), s_o)
        else:
            check_search(hd.INT8_E4M3, 32, W, h_o, m, frac=1.0)
            c_g, s_g, _ = hd.quantize_blocks(m, hd.INT8_E4M3, 32, dev(W), h=dev(torch.from_numpy(h_o)))
        Wq_g = hd.dequantize(hd.INT8_E4M3, 32, c_g, s_g, 64, 256)
        Wq_o = oracle.dequantize(hd.INT8_E4M3, 32, npy(c_g), npy(s_g), 64, 256)
        np.testing.assert_array_equal(npy(Wq_g), Wq_o)
        we_g = hd.weight_error(dev(W), Wq_g).item()
        we_o = oracle.weight_error(synth.bits(W), Wq_o)
        assert we_g == pytest.approx(we_o, rel=1e-9)
        oe_g = hd.output_error(dev(X), dev(W), Wq_g).item()
        oe_o = oracle.output_error(synth.bits(X), synth.bits(W), Wq_o)
        assert oe_g == pytest.approx(oe_o, rel=1e-4)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("M,K", [(1, 8), (257, 1000), (3001, 1536), (700, 37), (64, 4096)])
def test_hdiag_parity(dtype, M, K):
    X = synth.activations(M, K, 5 + M, n_out=2 if K > 2 else 0, out_gain=30.0, idx_seed=9, dtype=dtype)
    h_o = oracle.hdiag(synth.bits(X))
    h_g = hd.hdiag(dev(X))
    torch.cuda.synchronize()
    np.testing.assert_allclose(npy(h_g), h_o, rtol=1e-6)


def test_hdiag_exact_cases():
    X = torch.ones(5000, 520, dtype=torch.bfloat16)
    assert torch.equal(hd.hdiag(dev(X)).cpu(), torch.full((520,), 5000.0))
    Xi = torch.randint(-3, 4, (2049, 64), generator=torch.Generator().manual_seed(1)).float()
    want = (Xi.double() ** 2).sum(0).float()
    assert torch.equal(hd.hdiag(dev(Xi)).cpu(), want)
    # bf16 values whose squares lie below float32's normal range (2^-136 here)
    # or near its top: the squares are summed in float64, as in the oracle
    g = torch.Generator().manual_seed(2)
    mant = 1.0 + torch.randint(0, 128, (4096, 24), generator=g).double() / 128.0
    ex = torch.tensor([-68.0] * 8 + [-75.0] * 8 + [56.0] * 8, dtype=torch.float64)
    Xs = (mant * torch.pow(2.0, ex)).to(torch.bfloat16)
    want = oracle.hdiag(synth.bits(Xs))
    assert np.isfinite(want).all() and (want[:16] > 0).all()
    np.testing.assert_allclose(npy(hd.hdiag(dev(Xs))), want, rtol=1e-6)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B", [16, 128])
def test_dequantize_and_weight_error(fmt, B):
    N, K = 77, 2048
    W = weights_for(fmt, N, K, 4000 + fmt)
    c_g, s_g, _ = hd.quantize_blocks(hd.SSE_OPT, fmt, B, dev(W))
    deq_o = oracle.dequantize(fmt, B, npy(c_g), npy(s_g), N, K)
    deq_g = hd.dequantize(fmt, B, c_g, s_g, N, K)
    deq_b = hd.dequantize(fmt, B, c_g, s_g, N, K, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(npy(deq_g), deq_o)
    assert torch.equal(deq_b.cpu(), torch.from_numpy(deq_o).to(torch.bfloat16))
    we_o, num_o, den_o = oracle.weight_error(synth.bits(W), deq_o, sums=True)
    we_g, sums = hd.weight_error(dev(W), deq_g, sums=True)
    assert we_g.item() == pytest.approx(we_o, rel=1e-9)
    np.testing.assert_allclose(npy(sums), [num_o, den_o], rtol=1e-9)


@pytest.mark.parametrize("M,N,K", [(300, 200, 512), (129, 131, 96), (1000, 256, 1024), (64, 64, 8)])
def test_output_error_parity(M, N, K):
    W = weights_for(hd.NVFP4, N, K, 5000 + M)
    X = synth.activations(M, K, 77 + N, n_out=2, out_gain=50.0, idx_seed=3, dtype=torch.bfloat16)
    c_g, s_g, _ = hd.quantize_blocks(hd.SSE_OPT, hd.INT8_E4M3, 8, dev(W))
    Wq = hd.dequantize(hd.INT8_E4M3, 8, c_g, s_g, N, K)
    oe_o, d_o, y_o = oracle.output_error(synth.bits(X), synth.bits(W), npy(Wq), sums=True)
    oe_g, sums = hd.output_error(dev(X), dev(W), Wq, sums=True)
    torch.cuda.synchronize()
    assert oe_g.item() == pytest.approx(oe_o, rel=1e-4)
    np.testing.assert_allclose(npy(sums), [d_o, y_o], rtol=1e-4)


@pytest.mark.parametrize("M,N,K", [(300, 200, 512), (64, 64, 16)])
def test_output_error_given_ref(M, N, K):
    """Given ||X W^T||^2 from a first call, the D-only path returns the same
    sums: its D products are the same MFMAs in the same order."""
    W = weights_for(hd.NVFP4, N, K, 5100 + M)
    X = synth.activations(M, K, 78 + N, n_out=2, out_gain=50.0, idx_seed=3, dtype=torch.bfloat16)
    c_g, s_g, _ = hd.quantize_blocks(hd.H_OPT, hd.NVFP4, 16, dev(W), h=hd.hdiag(dev(X)))
    Wq = hd.dequantize(hd.NVFP4, 16, c_g, s_g, N, K)
    oe, sums = hd.output_error(dev(X), dev(W), Wq, sums=True)
    oe2, sums2 = hd.output_error_given_ref(dev(X), dev(W), Wq, sums[1:2].clone(), sums=True)
    torch.cuda.synchronize()
    assert torch.equal(sums, sums2) and torch.equal(oe, oe2)
    oe_o = oracle.output_error(synth.bits(X), synth.bits(W), npy(Wq))
    assert oe2.item() == pytest.approx(oe_o, rel=1e-4)


def test_output_error_identity_equals_weight_error():
    K, N = 256, 96
    W = weights_for(hd.NVFP4, N, K, 6000)
    X = torch.eye(K, dtype=torch.bfloat16)
    c_g, s_g, _ = hd.quantize_blocks(hd.SSE_OPT, hd.NVFP4, 16, dev(W))
    Wq = hd.dequantize(hd.NVFP4, 16, c_g, s_g, N, K, dtype=torch.bfloat16)
    oe = hd.output_error(dev(X), dev(W), Wq).item()
    we = hd.weight_error(dev(W), Wq).item()
    assert oe == pytest.approx(we, rel=1e-5)


def test_determinism():
    W = weights_for(hd.NVFP4, 300, 1024, 7000)
    h = dev(torch.from_numpy(h_for(1024, 13)))
    a = hd.quantize_blocks(hd.H_OPT, hd.NVFP4, 16, dev(W), h=h, block_obj=True)
    b = hd.quantize_blocks(hd.H_OPT, hd.NVFP4, 16, dev(W), h=h, block_obj=True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    X = synth.activations(3000, 1024, 1, dtype=torch.bfloat16)
    assert torch.equal(hd.hdiag(dev(X)), hd.hdiag(dev(X)))


def test_edge_blocks():
    # all-zero block, a single non-zero, negative zeros, values far above the
    # largest scale, subnormal bf16 values, and a block on a grid point
    rows = [
        [0.0] * 32,
        [0.0] * 31 + [0.013],
        [-0.0] * 16 + [0.0] * 16,
        [3e30, -2e30] + [1.0] * 30,
        [1e-40, -3e-39, 2e-38] + [0.0] * 29,
        [0.0078125 * q for q in ([0, 0.5, 1, 1.5, 2, 3, 4, 6] * 4)],
    ]
    W = torch.tensor(rows, dtype=torch.float32).to(torch.bfloat16)
    h = np.ones(32, np.float32)
    for fmt in FMTS:
        for m in (hd.NAIVE, hd.SSE_OPT, hd.H_OPT):
            c_o, s_o, _ = oracle.quantize(m, fmt, 32, synth.bits(W), h=h)
            c_g, s_g, _ = hd.quantize_blocks(m, fmt, 32, dev(W), h=dev(torch.from_numpy(h)))
            torch.cuda.synchronize()
            np.testing.assert_array_equal(npy(s_g), s_o, err_msg="fmt %d method %d" % (fmt, m))
            np.testing.assert_array_equal(npy(c_g), c_o, err_msg="fmt %d method %d" % (fmt, m))


def test_invalid_call_raises():
    W = dev(torch.zeros(4, 40, dtype=torch.bfloat16))
    with pytest.raises(hd.HdiagError):
        hd.quantize_blocks(hd.SSE_OPT, hd.NVFP4, 16, W)


@pytest.mark.parametrize("fmt", [hd.INT8_E4M3, hd.NVFP4, hd.MXFP4, hd.FP8_E4M3S])
@pytest.mark.parametrize("method", [hd.SSE_OPT, hd.H_OPT])
def test_instrumented_search_counts(fmt, method):
    """quantize_blocks_instrumented gives quantize_blocks' results bit for bit
    and counts the (weight, candidate) pairs the search walked: the same on
    every run, at least the first window per weight and at most the grid
    plus one widening step per weight; Naive adds nothing."""
    N, K, B = 300, 1024, 32
    W = dev(weights_for(fmt, N, K, 8000 + fmt))
    h = dev(torch.from_numpy(h_for(K, 21)))
    hh = h if method == hd.H_OPT else None
    c0, s0, o0 = hd.quantize_blocks(method, fmt, B, W, h=hh, block_obj=True)
    counts = []
    for _ in range(2):
        ev = torch.zeros(1, dtype=torch.int64, device="cuda")
        c1, s1, o1 = hd.quantize_blocks_instrumented(method, fmt, B, W, ev, h=hh, block_obj=True)
        torch.cuda.synchronize()
        assert torch.equal(c0, c1) and torch.equal(s0, s1) and torch.equal(o0, o1)
        counts.append(ev.item())
    assert counts[0] == counts[1]
    ncand = hd.hdiag_format_info(fmt, B)[2]
    first = 10 if fmt == hd.INT8_E4M3 else 13 if fmt != hd.MXFP4 else 2
    assert N * K * first <= counts[0] <= N * K * (ncand + 24)
    ev = torch.zeros(1, dtype=torch.int64, device="cuda")
    hd.quantize_blocks_instrumented(hd.NAIVE, fmt, B, W, ev)
    torch.cuda.synchronize()
    assert ev.item() == 0
