"""GPU parity (through the C ABI) of GPTQ (qwantize "Results", "GPTQ
Quantization") with the oracle.

- gptq_hessian: H = X^T X against the oracle's float64 product, entry by entry
  within the float32-accumulation bound 2e-6 * sum_t |x_ti x_tj|.
- gptq_quantize: the oracle runs on the GPU's own H (widened to float64), so
  the comparison isolates the column loop.  Both carry the working weights,
  the errors and the factor of (H + lambda I)^-1 in float64 (the GPU by a
  recursive Cholesky-with-inverse and panel-blocked updates, the oracle
  column by column), so they differ only by float64 rounding order.  GPTQ's
  decisions cascade along a row, but a float64-order perturbation moves no
  decision on the oracle's own precision experiment
  (tests/test_oracle_gptq_precision.py: with float32 working weights about
  0.3% of INT8 elements move).  Bars, as the search's: block order identical
  (GPTQ-Ord), scales identical on >= 99.99% of blocks, dequantised weights
  identical on >= 99.99% of elements, weight and output error within 1e-4
  relative.  With a diagonal H there is nothing to compensate and the result
  must equal quantize_blocks bit for bit.
"""
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


def dev(t):
    return t.contiguous().cuda()


def npy(t):
    return t.detach().cpu().numpy()


def scales_np(s):
    return npy(s.view(torch.int16)).view(np.uint16) if s.dtype == torch.float16 else npy(s)


@pytest.mark.parametrize("M,K", [(1000, 200), (4096, 512), (77, 64), (1, 8), (513, 130), (700, 776)])
def test_hessian(M, K):
    X = synth.activations(M, K, 3 + M, n_out=3, out_gain=50.0, idx_seed=4, dtype=torch.bfloat16)
    H = npy(hd.gptq_hessian(dev(X)))
    Xb = synth.bits(X)
    Ho = oracle.xtx(Xb)
    Xa = np.abs(X.float().numpy())
    bound = oracle.xtx(Xa)
    assert np.all(np.abs(H - Ho) <= 2e-6 * bound + 1e-30)
    if K % 8 == 0:  # the lower triangle, mirrored
        assert np.array_equal(H, H.T)


def gptq_inputs(N, K, M, seed):
    W = synth.weights("t4", N, K, std=0.02, seed=seed, gain_seed=seed + 1, dtype=torch.bfloat16)
    X = synth.activations(M, K, seed + 2, n_out=6, out_gain=30.0, idx_seed=seed + 3, dtype=torch.bfloat16)
    return W, X


def compare(fmt, B, method, ordered, W, X, Hd):
    N, K = W.shape
    c, s, order, info = hd.gptq_quantize(method, fmt, B, dev(W), Hd, ordered=ordered)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    H64 = npy(Hd).astype(np.float64)
    Wb = synth.bits(W)
    c_o, s_o, order_o = oracle.gptq(method, fmt, B, Wb, H64, ordered=ordered)
    if ordered:
        np.testing.assert_array_equal(npy(order), order_o)
    else:
        np.testing.assert_array_equal(npy(order), np.arange(K // B))
    sg = scales_np(s)
    Wq = npy(hd.dequantize(fmt, B, c, s, N, K))
    Wq_o = oracle.dequantize(fmt, B, c_o, s_o, N, K)
    fs, fe = (sg == s_o).mean(), (Wq == Wq_o).mean()
    print("gptq agreement fmt %d B %d method %d ordered %d: scales %.6f elements %.6f"
          % (fmt, B, method, int(ordered), fs, fe), flush=True)
    assert fs >= 0.9999, fs
    assert fe >= 0.9999, fe
    Xb = synth.bits(X)
    assert oracle.weight_error(Wb, Wq) == pytest.approx(oracle.weight_error(Wb, Wq_o), rel=1e-4)
    oe, oe_o = oracle.output_error(Xb, Wb, Wq), oracle.output_error(Xb, Wb, Wq_o)
    assert oe == pytest.approx(oe_o, rel=1e-4)
    return oe


CASES = [(hd.NVFP4, 16), (hd.INT8_E4M3, 32), (hd.MXFP4, 32), (hd.NVINT4, 16), (hd.FP4_F16, 128),
         (hd.NVFP4_UE4M4, 16), (hd.MXFP8, 64), (hd.INT8_E4M3, 256)]


@pytest.mark.parametrize("fmt,B", CASES)
@pytest.mark.parametrize("method", [hd.NAIVE, hd.SSE_OPT, hd.H_OPT])
@pytest.mark.parametrize("ordered", [False, True])
def test_gptq_parity(fmt, B, method, ordered):
    N, K, M = 67, 512, 1024  # ragged row count: the last row slab is partly empty
    W, X = gptq_inputs(N, K, M, 100 + fmt)
    Hd = hd.gptq_hessian(dev(X))
    compare(fmt, B, method, ordered, W, X, Hd)


@pytest.mark.parametrize("tile", [64, 128])
def test_gptq_parity_each_fp64_gemm_tile(tile):
    """K = 1024: the recursion's top products are 512 x 512, small enough that
    the automatic choice takes 64-wide tiles; the schedule setting
    SCHED_GPTQ_TILE forces each width of the float64 matrix-core kernel, and
    both must meet the parity bar (ragged N, GPTQ-Ord, H-Optimal)."""
    hd.hdiag_set_schedule(hd.SCHED_GPTQ_TILE, tile)
    try:
        N, K, M = 45, 1024, 2048
        W, X = gptq_inputs(N, K, M, 31)
        Hd = hd.gptq_hessian(dev(X))
        compare(hd.NVFP4, 16, hd.H_OPT, True, W, X, Hd)
    finally:
        hd.hdiag_set_schedule(hd.SCHED_GPTQ_TILE, 0)


@pytest.mark.parametrize("N,K,B,fmt", [(1, 8, 8, hd.NVFP4), (3, 24, 8, hd.INT8_E4M3), (5, 40, 8, hd.MXFP4),
                                       (2, 16, 16, hd.NVINT4), (7, 200, 8, hd.NVFP4)])
def test_gptq_tiny(N, K, B, fmt):
    """Leaves smaller than one 16-column panel, a single row, K below one
    64-wide leaf and a ragged leaf (K = 200: leaves of 64 and 8 columns)."""
    W, X = gptq_inputs(N, K, 64, 41 + K)
    Hd = hd.gptq_hessian(dev(X))
    for ordered in (False, True):
        c, s, order, info = hd.gptq_quantize(hd.SSE_OPT, fmt, B, dev(W), Hd, ordered=ordered)
        torch.cuda.synchronize()
        assert int(info.item()) == 0
        c_o, s_o, order_o = oracle.gptq(hd.SSE_OPT, fmt, B, synth.bits(W), npy(Hd).astype(np.float64),
                                        ordered=ordered)
        np.testing.assert_array_equal(npy(order), order_o)
        np.testing.assert_array_equal(scales_np(s), s_o)
        np.testing.assert_array_equal(npy(hd.dequantize(fmt, B, c, s, N, K)),
                                      oracle.dequantize(fmt, B, c_o, s_o, N, K))


def test_gptq_parity_two_panels_and_fp32_weights():
    """K spans several 128-column panels with a short last one (K % 128 != 0),
    float32 weights, the OCP rule as the scale choice."""
    N, K, M = 40, 448, 900
    W, X = gptq_inputs(N, K, M, 7)
    Hd = hd.gptq_hessian(dev(X))
    for fmt, B, m in ((hd.MXFP4, 32, hd.NAIVE_OCP), (hd.NVFP4, 16, hd.H_OPT)):
        c, s, _, info = hd.gptq_quantize(m, fmt, B, dev(W.float()), Hd)
        c_o, s_o, _ = oracle.gptq(m, fmt, B, synth.bits(W.float()), npy(Hd).astype(np.float64))
        assert (scales_np(s) == s_o).mean() >= 0.9999
        Wq = npy(hd.dequantize(fmt, B, c, s, N, K))
        assert (Wq == oracle.dequantize(fmt, B, c_o, s_o, N, K)).mean() >= 0.9999


@pytest.mark.parametrize("fmt,B,method", [(hd.INT8_E4M3, 32, hd.SSE_OPT), (hd.NVFP4, 16, hd.H_OPT)])
def test_gptq_parity_many_panels(fmt, B, method):
    """K = 2048: sixteen 128-column panels, so each row's decisions cascade
    through fifteen trailing updates on the float64 matrix cores."""
    N, K, M = 256, 2048, 4096
    W, X = gptq_inputs(N, K, M, 17)
    Hd = hd.gptq_hessian(dev(X))
    compare(fmt, B, method, False, W, X, Hd)


@pytest.mark.parametrize("fmt,B", [(hd.NVFP4, 16), (hd.INT8_E4M3, 128), (hd.FP4_F16, 128), (hd.MXFP4, 32)])
@pytest.mark.parametrize("method", [hd.NAIVE, hd.SSE_OPT, hd.H_OPT])
def test_diagonal_h_is_quantize_blocks(fmt, B, method):
    """No coupling between columns: GPTQ (Seq and Ord) returns exactly the
    method's own codes and scales."""
    N, K = 50, 1024
    W, _ = gptq_inputs(N, K, 8, 11)
    h = torch.from_numpy(np.random.default_rng(2).lognormal(0, 1, K).astype(np.float32))
    Hd = dev(torch.diag(h))
    c0, s0, _ = hd.quantize_blocks(method, fmt, B, dev(W), h=dev(h))
    for ordered in (False, True):
        c, s, _, _ = hd.gptq_quantize(method, fmt, B, dev(W), Hd, ordered=ordered)
        torch.cuda.synchronize()
        assert torch.equal(c, c0) and torch.equal(s, s0)


def test_gptq_lowers_output_error():
    """The page's GPTQ rows: lower output error, higher weight error than the
    same method without GPTQ; GPTQ-Ord at or below GPTQ-Seq here."""
    N, K, M = 256, 1024, 4096
    W, X = gptq_inputs(N, K, M, 21)
    Wd, Xd = dev(W), dev(X)
    Hd = hd.gptq_hessian(Xd)
    h = hd.hdiag(Xd)
    for fmt, B in ((hd.NVFP4, 16), (hd.NVINT4, 16)):
        c0, s0, _ = hd.quantize_blocks(hd.H_OPT, fmt, B, Wd, h=h)
        W0 = hd.dequantize(fmt, B, c0, s0, N, K)
        res = []
        for ordered in (False, True):
            c, s, _, _ = hd.gptq_quantize(hd.H_OPT, fmt, B, Wd, Hd, ordered=ordered)
            res.append(hd.dequantize(fmt, B, c, s, N, K))
        oe0 = hd.output_error(Xd, Wd, W0).item()
        oes = [hd.output_error(Xd, Wd, r).item() for r in res]
        assert oes[0] < 0.95 * oe0 and oes[1] < 0.95 * oe0
        assert hd.weight_error(Wd, res[0]).item() > hd.weight_error(Wd, W0).item()


def test_info_reports_an_indefinite_hessian():
    """A Hessian with a negative diagonal entry (not a Gram matrix) is not
    positive definite after damping: info is set, the call still completes."""
    K, N = 128, 8
    h = torch.ones(K)
    h[40] = -50.0
    W, _ = gptq_inputs(N, K, 8, 5)
    _, _, _, info = hd.gptq_quantize(hd.NAIVE, hd.NVFP4, 16, dev(W), dev(torch.diag(h)))
    torch.cuda.synchronize()
    assert int(info.item()) > 0


def test_invalid_calls():
    W = dev(torch.zeros(4, 64, dtype=torch.bfloat16))
    H = dev(torch.eye(64))
    with pytest.raises(hd.HdiagError):
        hd.gptq_quantize(hd.NAIVE_OCP, hd.NVFP4, 16, W, H)
    with pytest.raises(hd.HdiagError):
        hd.gptq_quantize(hd.NAIVE, hd.NVFP4, 12, W, H)
    with pytest.raises(hd.HdiagError):
        hd.gptq_quantize(hd.NAIVE, hd.NVFP4, 16, W, H, damp=-1.0)
    with pytest.raises(hd.HdiagError) as e:
        hd.gptq_hessian(dev(torch.zeros(8, 64)))
    assert e.value.status == hd.HD_ERR_UNSUPPORTED


@pytest.mark.parametrize("fmt,B,method", [(hd.INT8_E4M3, 32, hd.H_OPT), (hd.NVFP4, 16, hd.SSE_OPT),
                                          (hd.MXFP4, 32, hd.NAIVE), (hd.FP4_F16, 64, hd.H_OPT)])
def test_gptq_factored_matches_gptq_seq(fmt, B, method):
    """One factor of (H, damp) serves every sequential-order call: the same
    codes, scales, block order and status as gptq_quantize, bit for bit."""
    N, K, M = 96, 512, 1024
    X = synth.activations(M, K, 61, n_out=3, out_gain=20.0, idx_seed=62, dtype=torch.bfloat16)
    W = synth.weights("t4", N, K, std=0.02, seed=63, gain_seed=64, dtype=torch.bfloat16)
    Hd = hd.gptq_hessian(dev(X))
    factor, finfo = hd.gptq_factor(Hd, damp=0.01)
    c0, s0, o0, i0 = hd.gptq_quantize(method, fmt, B, dev(W), Hd, damp=0.01, ordered=False)
    c1, s1, o1, i1 = hd.gptq_quantize_factored(method, fmt, B, dev(W), Hd, factor)
    torch.cuda.synchronize()
    assert torch.equal(c0, c1) and torch.equal(s0, s1) and torch.equal(o0, o1)
    assert int(i0.item()) == int(i1.item()) == int(finfo.item()) == 0


def test_gptq_factor_reports_an_indefinite_hessian():
    K = 256
    h = torch.ones(K)
    h[7] = -1.0
    Hd = dev(torch.diag(h))
    factor, finfo = hd.gptq_factor(Hd, damp=0.0)
    W = dev(synth.weights("t4", 32, K, std=0.02, seed=1, gain_seed=2, dtype=torch.bfloat16))
    _, _, _, info = hd.gptq_quantize_factored(hd.NAIVE, hd.NVFP4, 16, W, Hd, factor)
    _, _, _, info0 = hd.gptq_quantize(hd.NAIVE, hd.NVFP4, 16, W, Hd, damp=0.0)
    torch.cuda.synchronize()
    assert int(finfo.item()) > 0 and int(info.item()) == int(finfo.item()) == int(info0.item())
