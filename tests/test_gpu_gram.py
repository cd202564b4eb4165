"""GPU parity of the output error through G = X^T X (output_gram,
output_reference_gram, output_error_gram) against the oracle.

The output error of every format's codes is compared with the oracle's output
error of the dequantised weights (the definition, ||X Wq^T - X W^T||_F /
||X W^T||_F in float64), within 1e-4 relative; ||X W^T||^2 likewise.  The
library's Gram buffer is also checked entry by entry: h bit for bit against
hdiag(), and the stored correlations C = G / sqrt(h_j h_k) (upper block
triangle, off-diagonal 256 x 256 blocks doubled, zero diagonal) against the
oracle's float64 X^T X within the float16 rounding plus the float32
accumulation bound.  Shapes span several 256 x 256 tiles with ragged edges and
K tails that are not multiples of 256.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import block_scaled_precision_hdiag_amd as hd

pytestmark = pytest.mark.gpu

FMTS = [hd.INT8_E4M3, hd.NVFP4, hd.MXFP4, hd.MXFP8, hd.FP8_E4M3S, hd.NVFP4_UE4M4, hd.NVFP4_UE5M3, hd.NVINT4,
        hd.FP4_F16, hd.INT4_F16]


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
    std = {hd.FP8_E4M3S: 4.0, hd.MXFP8: 0.05}.get(fmt, 0.02)
    return synth.weights("t4", N, K, std=std, seed=seed, gain_seed=seed + 1, dtype=dtype)


def acts(M, K, seed):
    return synth.activations(M, K, seed, n_out=3, out_gain=50.0, idx_seed=seed + 1, dtype=torch.bfloat16)


def method_for(fmt):
    return hd.SSE_OPT


def sc_np(s):
    """Scales for the oracle: uint8 codes, or the binary16 bits of float16 scales."""
    if s.dtype == torch.float16:
        return npy(s.view(torch.int16)).view(np.uint16)
    return npy(s)


def al256(x):
    return (x + 255) // 256 * 256


def gram_parts(gram, K):
    """h, C (float16 [K, K]) of a Gram buffer, at the library's offsets."""
    g = gram.cpu()
    h = g[:4 * K].view(torch.float32).numpy()
    c0 = 3 * al256(4 * K)
    C = g[c0:c0 + 2 * K * K].view(torch.float16).float().numpy().reshape(K, K)
    return h, C


@pytest.mark.parametrize("M,K", [(700, 600), (300, 512), (1, 8), (513, 1032)])
def test_gram_buffer(M, K):
    X = acts(M, K, 60 + K)
    Xf = X.float()
    Xf[:, 3] = 0.0  # a zero column: its h is 0 and its row and column of C are 0
    X = Xf.to(torch.bfloat16)
    Xd = dev(X)
    gram = hd.output_gram(Xd)
    h_dev = hd.hdiag(Xd)
    gram2 = hd.output_gram(Xd, h=h_dev)
    torch.cuda.synchronize()
    h, C = gram_parts(gram, K)
    h2, C2 = gram_parts(gram2, K)
    blk = np.arange(K) // 256
    upper = blk[:, None] <= blk[None, :]  # the part of C the library writes and reads
    np.testing.assert_array_equal(h, h2)
    np.testing.assert_array_equal(C[upper], C2[upper])
    np.testing.assert_array_equal(h, oracle.hdiag(synth.bits(X)))
    Xt = np.ascontiguousarray(synth.bits(X).T)
    G = oracle.matmul_nt(Xt, Xt)
    hg = np.diag(G).copy()
    r = np.where(hg > 0, 1.0 / np.sqrt(np.where(hg > 0, hg, 1.0)), 0.0)
    Ct = G * r[:, None] * r[None, :]
    fold = np.where(blk[:, None] < blk[None, :], 2.0, 1.0)
    np.fill_diagonal(Ct, 0.0)
    exp = (fold * Ct)[upper]
    got = C[upper].astype(np.float64)
    tol = fold[upper] * (2.0 ** -11 * np.abs(Ct[upper]) + 1e-4) + 2.0 ** -24
    assert np.all(np.abs(got - exp) <= tol), float(np.max(np.abs(got - exp) - tol))
    assert np.all(np.diag(C) == 0.0)
    assert np.all(C[:3, 3] == 0.0) and np.all(C[3, 4:][blk[4:] >= blk[3]] == 0.0)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B,M,N,K", [(16, 300, 200, 512), (256, 257, 300, 1024), (8, 700, 40, 520)])
def test_output_error_gram_parity(fmt, B, M, N, K):
    X, W = acts(M, K, 40 + B), weights_for(fmt, N, K, 950 + B)
    Xd, Wd = dev(X), dev(W)
    c, s, _ = hd.quantize_blocks(method_for(fmt), fmt, B, Wd)
    gram = hd.output_gram(Xd)
    ysq = hd.output_reference_gram(Wd, gram)
    out, sums = hd.output_error_gram(fmt, B, c, s, Wd, gram, ysq, sums=True)
    torch.cuda.synchronize()
    oe_o, d_o, y_o = oracle.output_error(synth.bits(X), synth.bits(W), oracle.dequantize(fmt, B, npy(c), sc_np(s), N, K),
                                         sums=True)
    assert out.item() == pytest.approx(oe_o, rel=1e-4)
    np.testing.assert_allclose(npy(sums)[:2], [d_o, y_o], rtol=1e-4)
    assert ysq.item() == pytest.approx(y_o, rel=1e-4)
    # the third value is the exact diagonal part sum_j d_j^2 h_j
    Wq = oracle.dequantize(fmt, B, npy(c), sc_np(s), N, K).astype(np.float64)
    Dd = Wq - W.float().numpy().astype(np.float64)
    b_o = float((Dd ** 2 @ oracle.hdiag(synth.bits(X)).astype(np.float64)).sum())
    assert sums[2].item() == pytest.approx(b_o, rel=1e-6)


@pytest.mark.parametrize("fmt", [hd.FP8_E4M3S, hd.MXFP8])
@pytest.mark.parametrize("method", [hd.NAIVE, hd.SSE_OPT, hd.H_OPT])
def test_output_error_gram_configs_width(fmt, method):
    """E4M3 elements on weights of the configs' width (std 0.02), where the
    E4M3-scale Naive collapses most blocks to the zero scale: all three scale
    choices, Gram route against the oracle's direct fp64 product."""
    M, N, K, B = 300, 200, 512, 32
    X = acts(M, K, 61)
    W = synth.weights("t4", N, K, std=0.02, seed=62, gain_seed=63)
    Xd, Wd = dev(X), dev(W)
    h = hd.hdiag(Xd)
    c, s, _ = hd.quantize_blocks(method, fmt, B, Wd, h=h if method == hd.H_OPT else None)
    gram = hd.output_gram(Xd, h=h)
    ysq = hd.output_reference_gram(Wd, gram)
    out = hd.output_error_gram(fmt, B, c, s, Wd, gram, ysq).item()
    Wq = oracle.dequantize(fmt, B, npy(c), sc_np(s), N, K)
    assert out == pytest.approx(oracle.output_error(synth.bits(X), synth.bits(W), Wq), rel=1e-4)


@pytest.mark.parametrize("fmt,B", [(hd.INT8_E4M3, 32), (hd.NVFP4, 16)])
def test_output_error_gram_float32_weights(fmt, B):
    M, N, K = 400, 260, 768
    X, W = acts(M, K, 3), weights_for(fmt, N, K, 4, dtype=torch.float32)
    Xd, Wd = dev(X), dev(W)
    c, s, _ = hd.quantize_blocks(hd.H_OPT, fmt, B, Wd, h=hd.hdiag(Xd))
    gram = hd.output_gram(Xd)
    ysq = hd.output_reference_gram(Wd, gram)
    out = hd.output_error_gram(fmt, B, c, s, Wd, gram, ysq).item()
    Wq = oracle.dequantize(fmt, B, npy(c), sc_np(s), N, K)
    assert out == pytest.approx(oracle.output_error(synth.bits(X), synth.bits(W), Wq), rel=1e-4)


def test_output_error_gram_x_dynamic_range():
    """A 1e4 outlier channel, a zero channel and rows over 2^-30 .. 2^30: the
    diagonal term is exact and C is scale-free."""
    M, N, K = 384, 80, 512
    X = acts(M, K, 5).float()
    X *= torch.from_numpy(np.exp2(np.linspace(-30, 30, M)).astype(np.float32))[:, None]
    X[:, 11] *= 1e4
    X[:, 12] = 0.0
    X = X.to(torch.bfloat16)
    for fmt, B in ((hd.INT8_E4M3, 32), (hd.NVFP4, 16), (hd.MXFP8, 32)):
        W = weights_for(fmt, N, K, 77)
        Xd, Wd = dev(X), dev(W)
        c, s, _ = hd.quantize_blocks(hd.NAIVE, fmt, B, Wd)
        gram = hd.output_gram(Xd)
        ysq = hd.output_reference_gram(Wd, gram)
        out = hd.output_error_gram(fmt, B, c, s, Wd, gram, ysq).item()
        Wq = oracle.dequantize(fmt, B, npy(c), sc_np(s), N, K)
        assert out == pytest.approx(oracle.output_error(synth.bits(X), synth.bits(W), Wq), rel=1e-4)


def test_output_error_gram_on_grid_is_zero():
    """W on the NVFP4 grid: D = 0, so the error is exactly 0."""
    M, N, K, B = 300, 260, 512, 16
    W0 = weights_for(hd.NVFP4, N, K, 3)
    c, s, _ = hd.quantize_blocks(hd.NAIVE, hd.NVFP4, B, dev(W0))
    Wg = hd.dequantize(hd.NVFP4, B, c, s, N, K, dtype=torch.bfloat16)
    X = dev(acts(M, K, 9))
    gram = hd.output_gram(X)
    ysq = hd.output_reference_gram(Wg, gram)
    out, sums = hd.output_error_gram(hd.NVFP4, B, c, s, Wg, gram, ysq, sums=True)
    torch.cuda.synchronize()
    assert out.item() == 0.0 and sums[0].item() == 0.0 and ysq.item() > 0.0


def test_output_error_gram_no_rows():
    """M = 0: G = 0, so both norms are 0 and the quotient is NaN, as the
    definition gives."""
    N, K, B = 64, 256, 32
    W = dev(weights_for(hd.INT8_E4M3, N, K, 1))
    X = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
    gram = hd.output_gram(X)
    ysq = hd.output_reference_gram(W, gram)
    c, s, _ = hd.quantize_blocks(hd.NAIVE, hd.INT8_E4M3, B, W)
    out, sums = hd.output_error_gram(hd.INT8_E4M3, B, c, s, W, gram, ysq, sums=True)
    torch.cuda.synchronize()
    assert ysq.item() == 0.0 and sums[0].item() == 0.0 and np.isnan(out.item())


def test_output_error_gram_partition_and_repeat():
    """How the K-block pairs are split between workgroups (the schedule
    settings SCHED_GRAM_GANGS and SCHED_GRAM_BANDS) changes only the
    summation order; repeated calls agree bit for bit."""
    M, N, K, B = 600, 300, 1536, 32
    X, W = dev(acts(M, K, 21)), dev(weights_for(hd.INT8_E4M3, N, K, 22))
    c, s, _ = hd.quantize_blocks(hd.SSE_OPT, hd.INT8_E4M3, B, W)
    gram = hd.output_gram(X)
    ysq = hd.output_reference_gram(W, gram)
    vals = []
    try:
        for nq in (1, 2, 5, 21, 1000, 0):
            hd.hdiag_set_schedule(hd.SCHED_GRAM_GANGS, nq)
            a = hd.output_error_gram(hd.INT8_E4M3, B, c, s, W, gram, ysq).item()
            b = hd.output_error_gram(hd.INT8_E4M3, B, c, s, W, gram, ysq).item()
            assert a == b
            vals.append(a)
        for qa in (1, 2, 3, 5, 6, 8, 64):
            hd.hdiag_set_schedule(hd.SCHED_GRAM_BANDS, qa)
            a = hd.output_error_gram(hd.INT8_E4M3, B, c, s, W, gram, ysq).item()
            b = hd.output_error_gram(hd.INT8_E4M3, B, c, s, W, gram, ysq).item()
            assert a == b
            vals.append(a)
    finally:
        hd.hdiag_set_schedule(hd.SCHED_GRAM_GANGS, 0)
        hd.hdiag_set_schedule(hd.SCHED_GRAM_BANDS, 0)
    assert max(vals) == pytest.approx(min(vals), rel=1e-9)
    generic = hd.output_error(X, W, hd.dequantize(hd.INT8_E4M3, B, c, s, N, K)).item()
    assert vals[0] == pytest.approx(generic, rel=1e-4)


def test_output_gram_errors():
    X = torch.randn(8, 16, device="cuda")
    with pytest.raises(hd.HdiagError) as e:
        hd.output_gram(X)
    assert e.value.status == hd.HD_ERR_UNSUPPORTED
    Xb = torch.randn(8, 12, device="cuda").bfloat16()
    with pytest.raises(hd.HdiagError) as e:
        hd.output_gram(Xb, gram=torch.empty(hd.output_gram_size(12), dtype=torch.uint8, device="cuda"))
    assert e.value.status == hd.HD_ERR_INVALID_ARG
    Xb = torch.randn(8, 16, device="cuda").bfloat16()
    with pytest.raises(hd.HdiagError) as e:
        hd.output_gram(Xb, gram=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert e.value.status == hd.HD_ERR_INVALID_ARG


def test_output_error_gram_wide_rows():
    """K = 16640 > 16384: the operand kernel's two-pass path (the row does not
    stay in registers)."""
    M, N, K, B = 96, 24, 16640, 32
    X, W = acts(M, K, 31), weights_for(hd.INT8_E4M3, N, K, 32)
    Xd, Wd = dev(X), dev(W)
    c, s, _ = hd.quantize_blocks(hd.SSE_OPT, hd.INT8_E4M3, B, Wd)
    gram = hd.output_gram(Xd)
    ysq = hd.output_reference_gram(Wd, gram)
    out, sums = hd.output_error_gram(hd.INT8_E4M3, B, c, s, Wd, gram, ysq, sums=True)
    torch.cuda.synchronize()
    oe_o, d_o, y_o = oracle.output_error(synth.bits(X), synth.bits(W),
                                         oracle.dequantize(hd.INT8_E4M3, B, npy(c), sc_np(s), N, K), sums=True)
    assert out.item() == pytest.approx(oe_o, rel=1e-4)
    np.testing.assert_allclose(npy(sums)[:2], [d_o, y_o], rtol=1e-4)


@pytest.mark.parametrize("N,K", [(300, 512), (2560, 1536), (40, 520)])
def test_output_error_gram_batch(N, K):
    """A batch of mixed formats and block sizes (N padded to whole 256-row
    tiles inside) gives each quantisation's output error as the single call
    does (up to summation order) and as the oracle does."""
    M = 600
    X = acts(M, K, 70 + N)
    W = weights_for(hd.NVFP4, N, K, 71 + N)
    Xd, Wd = dev(X), dev(W)
    h = hd.hdiag(Xd)
    gram = hd.output_gram(Xd, h=h)
    ysq = hd.output_reference_gram(Wd, gram)
    items = []
    for fmt, B, m in ((hd.INT8_E4M3, 32, hd.SSE_OPT), (hd.NVFP4, 16, hd.H_OPT), (hd.MXFP4, 32, hd.NAIVE),
                      (hd.INT8_E4M3, 8, hd.H_OPT), (hd.FP4_F16, 16, hd.SSE_OPT)):
        if K % B:
            continue
        c, s, _ = hd.quantize_blocks(m, fmt, B, Wd, h=h)
        items.append((fmt, B, c, s))
    out, sums = hd.output_error_gram_batch(items, Wd, gram, ysq, sums=True)
    torch.cuda.synchronize()
    for q, (fmt, B, c, s) in enumerate(items):
        single = hd.output_error_gram(fmt, B, c, s, Wd, gram, ysq).item()
        # the two schedules cut the K blocks into different runs, each summed
        # in float32 accumulators before the float64 partials
        assert out[q].item() == pytest.approx(single, rel=1e-6)
        oe_o = oracle.output_error(synth.bits(X), synth.bits(W), oracle.dequantize(fmt, B, npy(c), sc_np(s), N, K))
        assert out[q].item() == pytest.approx(oe_o, rel=1e-4)
        assert sums[q, 1].item() == ysq.item()


def test_output_error_gram_batch_errors():
    W = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    X = torch.zeros((32, 256), dtype=torch.bfloat16, device="cuda")
    gram = hd.output_gram(X)
    ysq = hd.output_reference_gram(W, gram)
    c, s, _ = hd.quantize_blocks(hd.NAIVE, hd.INT8_E4M3, 32, W)
    with pytest.raises(hd.HdiagError) as e:
        hd.output_error_gram_batch([(hd.INT8_E4M3, 32, c, s), (hd.INT8_E4M3, 24, c, s)], W, gram, ysq)
    assert e.value.status == hd.HD_ERR_INVALID_ARG
    with pytest.raises(hd.HdiagError) as e:
        hd.output_error_gram_batch([], W, gram, ysq)
    assert e.value.status == hd.HD_ERR_INVALID_ARG


def test_output_error_gram_batch_same_format_over_16():
    """18 quantisations of one format: the fused operand pass runs as two
    launches (16 + 2); each result equals its single call."""
    M, N, K = 400, 300, 768
    X, W = dev(acts(M, K, 81)), dev(weights_for(hd.NVFP4, N, K, 82))
    h = hd.hdiag(X)
    gram = hd.output_gram(X, h=h)
    ysq = hd.output_reference_gram(W, gram)
    items = []
    for k in range(18):
        B = (16, 32, 64)[k % 3]
        m = (hd.NAIVE, hd.SSE_OPT, hd.H_OPT)[(k // 3) % 3]
        c, s, _ = hd.quantize_blocks(m, hd.NVFP4, B, W, h=h)
        items.append((hd.NVFP4, B, c, s))
    out = hd.output_error_gram_batch(items, W, gram, ysq)
    torch.cuda.synchronize()
    for q, (fmt, B, c, s) in enumerate(items):
        assert out[q].item() == pytest.approx(hd.output_error_gram(fmt, B, c, s, W, gram, ysq).item(), rel=1e-6)


def test_output_error_gram_correlated_x():
    """Strongly correlated activations (rank-8 structure plus 30% noise and
    two outlier channels): the off-diagonal part of d^T G d is large here,
    and the float16 route still meets the 1e-4 bar against the oracle."""
    M, N, K = 1024, 256, 1024
    rng = np.random.default_rng(91)
    Xf = rng.standard_normal((M, 8)) @ rng.standard_normal((8, K)) * 3.0 + 0.3 * rng.standard_normal((M, K))
    Xf[:, [5, 700]] *= 100.0
    X = torch.from_numpy(Xf.astype(np.float32)).to(torch.bfloat16)
    Xd = dev(X)
    h = hd.hdiag(Xd)
    gram = hd.output_gram(Xd, h=h)
    for fmt, B, m in ((hd.INT8_E4M3, 32, hd.H_OPT), (hd.NVFP4, 16, hd.H_OPT), (hd.MXFP8, 32, hd.SSE_OPT)):
        W = weights_for(fmt, N, K, 92)
        Wd = dev(W)
        ysq = hd.output_reference_gram(Wd, gram)
        c, s, _ = hd.quantize_blocks(m, fmt, B, Wd, h=h)
        out = hd.output_error_gram(fmt, B, c, s, Wd, gram, ysq).item()
        Wq = oracle.dequantize(fmt, B, npy(c), sc_np(s), N, K)
        assert out == pytest.approx(oracle.output_error(synth.bits(X), synth.bits(W), Wq), rel=1e-4)


def _paired_x(M, K, rho, seed):
    rng = np.random.default_rng(seed)
    Z = rng.standard_normal((M, K))
    X = Z.copy()
    X[:, 1::2] = rho * Z[:, 0::2] + np.sqrt(1.0 - rho * rho) * Z[:, 1::2]
    return torch.from_numpy(X.astype(np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("rho", [0.5, 0.875, 0.99])
def test_output_error_gram_cancellation(rho):
    """Quantisation errors of opposite sign on channel pairs of correlation
    rho, so t = ||X D^T||^2 falls to about b (1 - rho), b the diagonal sum:
    the route's float16 error scales with b / t, which sums[2] / sums[0]
    reports.  W is built as W' - D with W' on the INT8 grid of fixed scales
    and |D| under half a step, so the codes give Wq = W' and D exactly."""
    M, N, K, B, fmt = 2048, 64, 256, 32, hd.INT8_E4M3
    X = _paired_x(M, K, rho, 11)
    rng = np.random.default_rng(12)
    sc = np.full((N, K // B), 0x38, dtype=np.uint8)  # E4M3 1.0: s = fl32(1 / 127)
    s = np.float32(oracle.scale_value(fmt, 0x38))
    Wp = (s * rng.integers(-100, 101, (N, K)).astype(np.float32)).astype(np.float32)
    Dp = np.zeros((N, K), dtype=np.float32)
    Dp[:, 0::2] = rng.uniform(-0.3, 0.3, (N, K // 2)).astype(np.float32) * s
    Dp[:, 1::2] = -Dp[:, 0::2]
    W = (Wp - Dp).astype(np.float32)
    Wd, Xd = dev(torch.from_numpy(W)), dev(X)
    c, _ = hd.encode_blocks(fmt, B, Wd, dev(torch.from_numpy(sc)))
    Wq = oracle.dequantize(fmt, B, npy(c), sc, N, K)
    np.testing.assert_array_equal(Wq, Wp)
    gram = hd.output_gram(Xd)
    ysq = hd.output_reference_gram(Wd, gram)
    out, sums = hd.output_error_gram(fmt, B, c, dev(torch.from_numpy(sc)), Wd, gram, ysq, sums=True)
    torch.cuda.synchronize()
    oe_o, t_o, _ = oracle.output_error(synth.bits(X), W, Wq, sums=True)
    ratio = sums[2].item() / sums[0].item()
    assert ratio == pytest.approx(1.0 / (1.0 - rho), rel=0.15)
    err = abs(out.item() - oe_o) / oe_o
    assert err <= 5e-5 * ratio + 1e-6, (err, ratio)
    if ratio <= 2.0:
        assert err <= 1e-4
    # the direct product has no such dependence
    direct = hd.output_error(Xd, Wd, dev(torch.from_numpy(Wq))).item()
    assert direct == pytest.approx(oe_o, rel=1e-4)


def test_output_error_gram_after_gptq_on_correlated_x():
    """GPTQ-quantised W on correlated activations: GPTQ pushes each error
    against the channels correlated with it, which lowers t below b.  The
    Gram route stays within its stated bound (4e-5 per unit of the b / t it
    reports) and within 1e-4 whenever b / t <= 2; the direct route within 1e-4."""
    M, N, K, B = 2048, 128, 512, 16
    rng = np.random.default_rng(93)
    Xf = rng.standard_normal((M, 16)) @ rng.standard_normal((16, K)) + 0.3 * rng.standard_normal((M, K))
    X = torch.from_numpy(Xf.astype(np.float32)).to(torch.bfloat16)
    W = weights_for(hd.NVFP4, N, K, 94)
    Xd, Wd = dev(X), dev(W)
    H = hd.gptq_hessian(Xd)
    gram = hd.output_gram(Xd)
    ysq = hd.output_reference_gram(Wd, gram)
    for fmt, m in ((hd.NVFP4, hd.H_OPT), (hd.INT8_E4M3, hd.SSE_OPT)):
        c, s, _, info = hd.gptq_quantize(m, fmt, B, Wd, H)
        out, sums = hd.output_error_gram(fmt, B, c, s, Wd, gram, ysq, sums=True)
        Wq = hd.dequantize(fmt, B, c, s, N, K)
        direct = hd.output_error(Xd, Wd, Wq).item()
        torch.cuda.synchronize()
        assert info.item() == 0
        oe_o = oracle.output_error(synth.bits(X), synth.bits(W), npy(Wq))
        ratio = sums[2].item() / sums[0].item()
        assert ratio > 1.0  # GPTQ's errors cancel across correlated channels
        err = abs(out.item() - oe_o) / oe_o
        assert err <= 5e-5 * ratio + 1e-6, (fmt, err, ratio)
        if ratio <= 2.0:
            assert err <= 1e-4
        assert direct == pytest.approx(oe_o, rel=1e-4)
