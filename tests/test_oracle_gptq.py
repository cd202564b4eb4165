"""Pins of the oracle's GPTQ (qwantize "Results", "GPTQ Quantization"; the
quantisation-algorithms note, §1: H = X^T X + lambda I, columns quantised in
sequence with each residual propagated through H^-1).

What fixes it, other than the oracle: numpy's matmul (X^T X); exact special
cases (a diagonal H leaves nothing to compensate, so GPTQ is the plain
quantiser; two coupled columns get the closed-form optimal-brain-surgeon
correction); an independent formulation with numpy solves (after each column
is fixed, the free columns sit at the minimiser of (w - w0)^T H (w - w0) given
the fixed ones - what GPTQ's recurrence maintains); the GPTQ-Ord / GPTQ-Seq
relation through the block permutation; and the qualitative effects the
page's tables show (GPTQ lowers the output error and raises the weight error).
"""
import numpy as np
import pytest

import oracle

FMTS = [oracle.NVFP4, oracle.INT8_E4M3, oracle.MXFP4, oracle.NVINT4, oracle.FP4_F16]
METHODS = [oracle.NAIVE, oracle.SSE_OPT, oracle.H_OPT]


def test_xtx_is_the_gram_matrix():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((300, 40)).astype(np.float32)
    X[:, 3] *= 50
    H = oracle.xtx(X)
    ref = X.astype(np.float64).T @ X.astype(np.float64)
    np.testing.assert_allclose(H, ref, rtol=1e-12, atol=1e-9)
    assert np.array_equal(H, H.T)
    Xb = (X.view(np.uint32) >> 16).astype(np.uint16)  # bf16 bits
    Hb = oracle.xtx(Xb)
    xb = (Xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_allclose(Hb, xb.T @ xb, rtol=1e-12, atol=1e-9)


def plain(method, fmt, B, W, H):
    return oracle.quantize(method, fmt, B, W, h=np.diag(H).astype(np.float32))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("ordered", [False, True])
def test_diagonal_h_is_the_plain_quantiser(fmt, method, ordered):
    """No off-diagonal H: every propagated error has zero weight, so GPTQ-Seq
    and GPTQ-Ord both give exactly the method's own codes and scales (the Ord
    case checks that the block permutation is undone)."""
    rng = np.random.default_rng(2)
    N, K, B = 9, 128, 16
    W = (rng.standard_t(4, (N, K)) * 0.02).astype(np.float32)
    H = np.diag(rng.lognormal(0, 1, K))
    c, s, order = oracle.gptq(method, fmt, B, W, H, ordered=ordered)
    c0, s0, _ = plain(method, fmt, B, W, H)
    assert np.array_equal(c, c0) and np.array_equal(s, s0)
    assert sorted(order) == list(range(K // B))


@pytest.mark.parametrize("method", METHODS)
def test_two_coupled_columns_closed_form(method):
    """H couples column a (block 0) with column b (block 1) only: after a is
    quantised to q_a, b moves by the optimal-brain-surgeon correction
    -(H_ba / H_bb) (q_a - w_a) (no damping), and block 1 is then quantised
    from the corrected values."""
    fmt, B, N, K = oracle.NVFP4, 8, 5, 16
    a, b, rho = 3, 11, 0.45
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    H = np.eye(K)
    H[b, b] = 1.5
    H[a, b] = H[b, a] = rho
    c, s, _ = oracle.gptq(method, fmt, B, W, H, damp=0.0)
    # the plain quantiser on block 0, then on the corrected block 1
    c0, s0, _ = plain(method, fmt, B, W, H)
    qa = oracle.dequantize(fmt, B, c0, s0, N, K)[:, a].astype(np.float64)
    W1 = W.astype(np.float64)
    W1[:, b] -= (H[b, a] / H[b, b]) * (qa - W[:, a])
    W1 = W1.astype(np.float32)
    c1, s1, _ = plain(method, fmt, B, W1, H)
    assert np.array_equal(s[:, 0], s0[:, 0]) and np.array_equal(s[:, 1], s1[:, 1])
    assert np.array_equal(c, c1)


def obs_reference(method, fmt, B, W, H, damp=0.01):
    """GPTQ-Seq written as a sequence of constrained least-squares problems
    (numpy solves; no Cholesky factor of H^-1): columns are fixed to their
    quantised values one at a time, and after each the free columns are reset
    to argmin (w - w0)^T Hd (w - w0) with the fixed ones held, i.e.
    w_F = w0_F - Hd_FF^-1 Hd_FQ (q_Q - w0_Q).  Block scales are chosen from the
    block's values when its first column is reached."""
    N, K = W.shape
    Hd = H + damp * np.mean(np.diag(H)) * np.eye(K)
    h = np.diag(H).astype(np.float32)
    w0 = W.astype(np.float64)
    codes = np.zeros(oracle.codes_shape(fmt, N, K), np.uint8)
    scales = np.zeros((N, K // B), oracle.scale_dtype(fmt))
    for n in range(N):
        w = w0[n].copy()
        q = np.zeros(K)
        for cs in range(0, K, B):
            blk = w[cs:cs + B].astype(np.float32)[None, :]
            _, sc, _ = oracle.quantize(method, fmt, B, blk, h=h[cs:cs + B])
            scales[n, cs // B] = sc[0, 0]
            for j in range(cs, cs + B):
                # encode column j (its code depends only on its value and the scale)
                blk = w[cs:cs + B].astype(np.float32)[None, :]
                cj, _, _ = oracle.quantize(oracle.NAIVE, fmt, B, blk, scales_in=sc)
                qj = oracle.dequantize(fmt, B, cj, sc, 1, B)[0, j - cs]
                if fmt in oracle.FOUR_BIT:
                    nib = (cj[0, (j - cs) // 2] >> (4 * ((j - cs) % 2))) & 15
                    codes[n, j // 2] |= np.uint8(nib << (4 * (j % 2)))
                else:
                    codes[n, j] = cj[0, j - cs]
                q[j] = qj
                Q, F = np.arange(j + 1), np.arange(j + 1, K)
                if F.size:
                    d = q[Q] - w0[n, Q]
                    w[F] = w0[n, F] - np.linalg.solve(Hd[np.ix_(F, F)], Hd[np.ix_(F, Q)] @ d)
    return codes, scales


@pytest.mark.parametrize("fmt", [oracle.NVFP4, oracle.INT8_E4M3, oracle.NVINT4])
@pytest.mark.parametrize("method", METHODS)
def test_matches_the_least_squares_formulation(fmt, method):
    rng = np.random.default_rng(4)
    N, K, B, M = 4, 48, 8, 200
    X = rng.standard_normal((M, K)) @ (np.eye(K) + 0.3 * rng.standard_normal((K, K)))  # correlated columns
    X = X.astype(np.float32)
    H = oracle.xtx(X)
    W = (rng.standard_t(4, (N, K)) * 0.02).astype(np.float32)
    c, s, _ = oracle.gptq(method, fmt, B, W, H)
    c_ref, s_ref = obs_reference(method, fmt, B, W, H)
    assert np.array_equal(s, s_ref)
    assert np.array_equal(c, c_ref)


@pytest.mark.parametrize("method", METHODS)
def test_ordered_is_seq_on_the_permuted_problem(method):
    """GPTQ-Ord = GPTQ-Seq on W and H with their block columns permuted into
    the processing order, un-permuted afterwards; that order sorts the blocks
    by descending h-weighted loss of the method's plain quantisation."""
    fmt, B, N, K, M = oracle.NVFP4, 16, 12, 256, 400
    rng = np.random.default_rng(5)
    X = (rng.standard_normal((M, K)) @ (np.eye(K) + 0.2 * rng.standard_normal((K, K)))).astype(np.float32)
    X[:, 40:56] *= 8.0  # one block column of inputs dominates the loss
    H = oracle.xtx(X)
    W = (rng.standard_t(4, (N, K)) * 0.02).astype(np.float32)
    c, s, order = oracle.gptq(method, fmt, B, W, H, ordered=True)
    h = np.diag(H).astype(np.float32)
    _, sp, _ = oracle.quantize(method, fmt, B, W, h=h)
    loss = oracle.objectives_at(fmt, B, W, sp, h=h).sum(axis=0)
    assert list(order) == list(np.argsort(-loss, kind="stable"))
    assert order[0] == 40 // B
    cols = (order[:, None] * B + np.arange(B)[None, :]).ravel()
    cp, sp2, _ = oracle.gptq(method, fmt, B, np.ascontiguousarray(W[:, cols]), H[np.ix_(cols, cols)])
    # un-permute: block i of the permuted problem is original block order[i]
    assert np.array_equal(s[:, order], sp2)
    Wq = oracle.dequantize(fmt, B, c, s, N, K)
    Wqp = oracle.dequantize(fmt, B, cp, sp2, N, K)
    assert np.array_equal(Wq[:, cols], Wqp)


@pytest.mark.parametrize("fmt", [oracle.NVFP4, oracle.MXFP4, oracle.NVINT4])
def test_gptq_trades_weight_error_for_output_error(fmt):
    """The direction of every GPTQ row of the page's tables: lower output
    error than the same method without GPTQ, higher weight error."""
    rng = np.random.default_rng(6)
    N, K, B, M = 48, 512, 16, 1024
    X = (rng.standard_normal((M, K)) @ (np.eye(K) + 0.1 * rng.standard_normal((K, K)))).astype(np.float32)
    X[:, rng.choice(K, 6, replace=False)] *= 30.0
    H = oracle.xtx(X)
    W = (rng.standard_t(4, (N, K)) * 0.02).astype(np.float32)
    for m in METHODS:
        c0, s0, _ = plain(m, fmt, B, W, H)
        c1, s1, _ = oracle.gptq(m, fmt, B, W, H)
        W0 = oracle.dequantize(fmt, B, c0, s0, N, K)
        W1 = oracle.dequantize(fmt, B, c1, s1, N, K)
        assert oracle.output_error(X, W, W1) < 0.95 * oracle.output_error(X, W, W0)
        assert oracle.weight_error(W, W1) > oracle.weight_error(W, W0)


def test_degenerate_inputs():
    W = np.zeros((3, 32), np.float32)
    H = np.zeros((32, 32))  # no activations: the damping term alone
    c, s, _ = oracle.gptq(oracle.SSE_OPT, oracle.NVFP4, 16, W, H)
    assert not c.any()
    c2, s2, _ = oracle.gptq(oracle.NAIVE, oracle.INT8_E4M3, 16, W, H)
    assert not c2.any() and not s2.any()
    with pytest.raises(ValueError):
        oracle.gptq(oracle.NAIVE_OCP, oracle.NVFP4, 16, W, H)
