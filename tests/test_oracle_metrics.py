"""Pins of the oracle's hdiag and error metrics (CPU only).

Closed forms: X = ones gives h = M; integer X gives exact integer sums; the
output error equals the weight error for X = I, and for X with orthogonal
columns it equals sqrt(sum_j h_j dW_j^2 / sum_j h_j W_j^2) with h = diag(X^T X)
(which also ties the output error to the H-weighted objective).  The last test
checks the qualitative ordering the qwantize "Results" tables report
(Naive > SSE-Optimal > H-Optimal in output error) on synthetic stand-in data.
"""
import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
import synth
from oracle import NAIVE, SSE_OPT, H_OPT, INT8_E4M3, NVFP4, MXFP4


def test_hdiag_ones():
    X = np.ones((777, 40), np.float32)
    np.testing.assert_array_equal(oracle.hdiag(X), np.full(40, 777, np.float32))


def test_hdiag_integer_exact():
    rng = np.random.default_rng(1)
    Xi = rng.integers(-3, 4, (3001, 130))
    want = (Xi.astype(np.int64) ** 2).sum(0).astype(np.float32)
    np.testing.assert_array_equal(oracle.hdiag(Xi.astype(np.float32)), want)


def test_hdiag_bf16_and_float():
    import torch
    rng = np.random.default_rng(2)
    X = rng.normal(0, 1, (500, 96)).astype(np.float32)
    Xb = torch.from_numpy(X).to(torch.bfloat16)
    bits = Xb.view(torch.int16).numpy().view(np.uint16)
    ref = (Xb.double().numpy() ** 2).sum(0)
    np.testing.assert_allclose(oracle.hdiag(bits), ref.astype(np.float32), rtol=1e-7)


def test_hdiag_empty_rows():
    np.testing.assert_array_equal(oracle.hdiag(np.zeros((0, 8), np.float32)), np.zeros(8, np.float32))


def test_weight_error_closed_forms():
    rng = np.random.default_rng(3)
    W = rng.normal(0, 1, (13, 48)).astype(np.float32)
    assert oracle.weight_error(W, W) == 0.0
    assert oracle.weight_error(W, 2 * W) == pytest.approx(1.0, abs=1e-15)
    assert oracle.weight_error(W, np.zeros_like(W)) == pytest.approx(1.0, abs=1e-15)
    Wq = W.copy()
    Wq[5, 7] += np.float32(0.5)
    d = float(Wq[5, 7]) - float(W[5, 7])
    want = abs(d) / np.sqrt((W.astype(np.float64) ** 2).sum())
    assert oracle.weight_error(W, Wq) == pytest.approx(want, rel=1e-14)


def _quantized(W, fmt=NVFP4, B=16):
    codes, sc, _ = oracle.quantize(SSE_OPT, fmt, B, W)
    return oracle.dequantize(fmt, B, codes, sc, *W.shape)


def test_output_error_identity_x_equals_weight_error():
    rng = np.random.default_rng(4)
    W = rng.normal(0, 0.02, (24, 64)).astype(np.float32)   # N != K: a transposed operand fails
    Wq = _quantized(W)
    X = np.eye(64, dtype=np.float32)
    assert oracle.output_error(X, W, Wq) == pytest.approx(oracle.weight_error(W, Wq), rel=1e-13)


def test_output_error_orthogonal_columns():
    rng = np.random.default_rng(5)
    K = 128
    c = rng.uniform(0.25, 4.0, K).astype(np.float32)
    X = (scipy.linalg.hadamard(K).astype(np.float32) * c[None, :]).astype(np.float32)
    h = oracle.hdiag(X)                                      # = K c^2, exactly
    np.testing.assert_allclose(h, K * c.astype(np.float64) ** 2, rtol=1e-7)
    W = rng.normal(0, 0.02, (40, K)).astype(np.float32)
    Wq = _quantized(W)
    dW = Wq.astype(np.float64) - W.astype(np.float64)
    hd = h.astype(np.float64)
    want = np.sqrt((hd * dW ** 2).sum() / (hd * W.astype(np.float64) ** 2).sum())
    assert oracle.output_error(X, W, Wq) == pytest.approx(want, rel=1e-6)


def test_output_error_zero_and_scaling():
    rng = np.random.default_rng(6)
    X = rng.normal(0, 1, (30, 32)).astype(np.float32)
    W = rng.normal(0, 1, (9, 32)).astype(np.float32)
    assert oracle.output_error(X, W, W) == 0.0
    assert oracle.output_error(X, W, 4 * W) == pytest.approx(3.0, rel=1e-14)
    r, dsq, ysq = oracle.output_error(X, W, np.zeros_like(W), sums=True)
    assert r == pytest.approx(1.0, rel=1e-14) and dsq == pytest.approx(ysq, rel=1e-14)


def test_published_ordering_on_stand_in_data():
    """qwantize "Results" (INT8, NVFP4 and MXFP4 tables): output error falls
    from Naive to SSE-Optimal to H-Optimal, H-Optimal has the larger weight
    error, and the H gain is smaller with power-of-two (E8M0) scales."""
    rng = np.random.default_rng(7)
    N, K, M = 96, 1024, 2048
    W = (rng.standard_t(4, (N, K)) * 0.02 * rng.lognormal(0, 0.5, N)[:, None]).astype(np.float32)
    X = rng.normal(0, 1, (M, K)).astype(np.float32)
    X[:, rng.choice(K, 8, replace=False)] *= 50
    h = oracle.hdiag(X)
    gain = {}
    for fmt, B in ((INT8_E4M3, 32), (NVFP4, 16), (MXFP4, 16)):
        oe, we = {}, {}
        for m in (NAIVE, SSE_OPT, H_OPT):
            codes, sc, _ = oracle.quantize(m, fmt, B, W, h=h)
            Wq = oracle.dequantize(fmt, B, codes, sc, N, K)
            oe[m] = oracle.output_error(X[:256], W, Wq)
            we[m] = oracle.weight_error(W, Wq)
        assert oe[NAIVE] > oe[SSE_OPT] > oe[H_OPT], (fmt, oe)
        assert we[SSE_OPT] <= we[H_OPT], (fmt, we)
        gain[fmt] = 1 - oe[H_OPT] / oe[SSE_OPT]
    assert gain[MXFP4] < gain[NVFP4]


def test_matmul_nt_identity_and_integers():
    """Y = X W^T: X = I gives W^T exactly; small integers give the exact
    integer product (brute force in Python integers); bf16 inputs are widened
    exactly; sum Y^2 is the ||X W^T||^2 the output error divides by."""
    rng = np.random.default_rng(7)
    W = rng.standard_normal((5, 12)).astype(np.float32)
    Y = oracle.matmul_nt(np.eye(12, dtype=np.float32), W)
    np.testing.assert_array_equal(Y, W.T.astype(np.float64))
    Xi = rng.integers(-50, 51, (7, 9))
    Wi = rng.integers(-50, 51, (4, 9))
    Y = oracle.matmul_nt(Xi.astype(np.float32), Wi.astype(np.float32))
    exact = [[sum(int(Xi[t, k]) * int(Wi[n, k]) for k in range(9)) for n in range(4)] for t in range(7)]
    np.testing.assert_array_equal(Y, np.array(exact, dtype=np.float64))
    Xb = torch.from_numpy(Xi.astype(np.float32)).to(torch.bfloat16)
    Wb = torch.from_numpy(Wi.astype(np.float32)).to(torch.bfloat16)
    np.testing.assert_array_equal(oracle.matmul_nt(synth.bits(Xb), synth.bits(Wb)), Y)
    X = rng.standard_normal((6, 12)).astype(np.float32)
    _, _, ysq = oracle.output_error(X, W, W, sums=True)
    assert (oracle.matmul_nt(X, W) ** 2).sum() == pytest.approx(ysq, rel=1e-14)
    assert oracle.matmul_nt(np.zeros((0, 12), np.float32), W).shape == (0, 5)
