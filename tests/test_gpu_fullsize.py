"""Parity at the configurations' full sizes, in the launch configurations the
benchmark uses (the GPU always processes the whole tensors).

The oracle checks what it can compute one by one: every column of h (its own
fp64 hdiag over the full X), and the scales / codes / objectives of a sample
of rows of W (blocks are independent, so a row's result does not depend on
the others).  The output-error GEMM is checked at full size by properties that
hold at any size (Wq = W gives 0, Wq = 2W gives exactly 1: dW = W then takes
the same MFMAs as Y) and against the oracle on a row subset of X.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import block_scaled_precision_hdiag_amd as hd

pytestmark = pytest.mark.gpu

FMT = {"INT8_E4M3": hd.INT8_E4M3, "NVFP4": hd.NVFP4, "MXFP4": hd.MXFP4, "MXFP8": hd.MXFP8,
       "FP8_E4M3S": hd.FP8_E4M3S}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hd.lib()


def sample_rows(N, n, seed):
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(N, n, replace=False))
    return np.unique(np.concatenate([[0, N - 1], rows]))


def check_rows(method, fmt, B, W, h_np, h_dev, rows):
    """GPU on all of W; oracle on the sampled rows."""
    Wd = W.cuda()
    c_g, s_g, o_g = hd.quantize_blocks(method, fmt, B, Wd, h=h_dev if method != hd.SSE_OPT else None,
                                       block_obj=True)
    torch.cuda.synchronize()
    Ws = synth.bits(W)[rows]
    hh = h_np if method != hd.SSE_OPT else None
    c_o, s_o, o_o = oracle.quantize(method, fmt, B, np.ascontiguousarray(Ws), h=hh)
    s_gr = s_g.cpu().numpy()[rows]
    same = s_gr == s_o
    assert same.mean() >= 0.9999, same.mean()
    if not same.all():
        at = oracle.objectives_at(fmt, B, np.ascontiguousarray(Ws), s_gr, h=hh)
        assert np.all(((at - o_o) / np.maximum(o_o, 1e-300))[~same] <= 1e-6)
    c_ref, _, _ = oracle.quantize(hd.NAIVE, fmt, B, np.ascontiguousarray(Ws), scales_in=s_gr)
    np.testing.assert_array_equal(c_g.cpu().numpy()[rows], c_ref)
    if method == hd.NAIVE:
        np.testing.assert_array_equal(s_gr, s_o)
    np.testing.assert_allclose(o_g.cpu().numpy()[rows], o_o.astype(np.float32), rtol=2e-6)
    return c_g, s_g


def full_x_checks(X, W, Wq_dev, R=192):
    """Output error at full size (properties) and on the first R rows (oracle)."""
    Xd, Wd = X.cuda(), W.cuda()
    zero = hd.output_error(Xd, Wd, Wd.float()).item()
    assert zero == 0.0
    two = hd.output_error(Xd, Wd, (2 * Wd).contiguous()).item()
    assert two == 1.0
    full = hd.output_error(Xd, Wd, Wq_dev).item()
    assert 0.0 < full < 1.0
    sub = hd.output_error(Xd[:R].contiguous(), Wd, Wq_dev).item()
    sub_o = oracle.output_error(synth.bits(X[:R]), synth.bits(W), Wq_dev.cpu().numpy())
    assert sub == pytest.approx(sub_o, rel=1e-4)
    return full


def test_config2_int8_full():
    W, X = synth.config_inputs(2)
    h_o = oracle.hdiag(synth.bits(X))
    h = hd.hdiag(X.cuda())
    torch.cuda.synchronize()
    np.testing.assert_allclose(h.cpu().numpy(), h_o, rtol=1e-6)
    rows = sample_rows(W.shape[0], 24, 2)
    for B in (32, 64, 128, 256):
        for m in (hd.NAIVE, hd.SSE_OPT, hd.H_OPT):
            c, s = check_rows(m, hd.INT8_E4M3, B, W, h_o, h, rows)
    Wq = hd.dequantize(hd.INT8_E4M3, 256, c, s, *W.shape)
    full_x_checks(X, W, Wq)


def test_config2_gram_route_full():
    """The bench step's output error (through G = X^T X) at config 2's full
    size: against the direct route (X Wq^T - Y, an independent product) over
    the whole X for every quantisation of the step, and against the oracle on
    the first R rows of X (G of that row subset).  W = Wq gives exactly 0."""
    W, X = synth.config_inputs(2)
    Xd, Wd = X.cuda(), W.cuda()
    N, K = W.shape
    h = hd.hdiag(Xd)
    gram = hd.output_gram(Xd, h=h)
    ysq = hd.output_reference_gram(Wd, gram)
    ref = hd.output_reference(Xd, Wd)
    assert ysq.item() == pytest.approx(hd.reference_ysq(ref).item(), rel=1e-4)
    items, singles = [], []
    for B in (32, 64, 128, 256):
        for m in (hd.NAIVE, hd.SSE_OPT, hd.H_OPT):
            c, s, _ = hd.quantize_blocks(m, hd.INT8_E4M3, B, Wd, h=h)
            g = hd.output_error_gram(hd.INT8_E4M3, B, c, s, Wd, gram, ysq).item()
            d = hd.output_error_codes(hd.INT8_E4M3, B, Xd, c, s, ref, N, K).item()
            assert g == pytest.approx(d, rel=1e-4), (B, m)
            items.append((hd.INT8_E4M3, B, c, s))
            singles.append(g)
    # the step's batch (walks of two quantisations at this size) and a batch of
    # three (walks of two and one, with different walk schedules): each result
    # as its single call gives it, up to summation order
    for batch in (items, items[:3]):
        out = hd.output_error_gram_batch(batch, Wd, gram, ysq)
        torch.cuda.synchronize()
        for q in range(len(batch)):
            assert out[q].item() == pytest.approx(singles[q], rel=1e-6), q
    R = 192
    Xs = Xd[:R].contiguous()
    gram_s = hd.output_gram(Xs)
    ysq_s = hd.output_reference_gram(Wd, gram_s)
    sub = hd.output_error_gram(hd.INT8_E4M3, 256, c, s, Wd, gram_s, ysq_s).item()
    Wq = hd.dequantize(hd.INT8_E4M3, 256, c, s, N, K)
    sub_o = oracle.output_error(synth.bits(X[:R]), synth.bits(W), Wq.cpu().numpy())
    assert sub == pytest.approx(sub_o, rel=1e-4)
    # W = the codes' own float32 dequantisation: D = 0 exactly
    ysq_q = hd.output_reference_gram(Wq, gram)
    assert hd.output_error_gram(hd.INT8_E4M3, 256, c, s, Wq, gram, ysq_q).item() == 0.0


def test_config3_nvfp4_full_x():
    W, _ = synth.config_inputs(3, x_rows=0)
    cfg = synth.CONFIGS[3]["X"]
    # the full 244449 x 9728 bf16 X (4.76 GB), streamed to the GPU in chunks
    Xd = torch.empty((cfg["M"], cfg["K"]), dtype=torch.bfloat16, device="cuda")
    Xh = torch.empty((cfg["M"], cfg["K"]), dtype=torch.bfloat16)
    r = 0
    for ch in synth.activation_chunks(cfg["M"], cfg["K"], cfg["seed"], cfg["n_out"], cfg["out_gain"],
                                      cfg["idx_seed"]):
        Xh[r:r + ch.shape[0]] = ch
        Xd[r:r + ch.shape[0]] = ch.cuda()
        r += ch.shape[0]
    h = hd.hdiag(Xd)
    h_o = oracle.hdiag(synth.bits(Xh))
    torch.cuda.synchronize()
    np.testing.assert_allclose(h.cpu().numpy(), h_o, rtol=1e-6)
    rows = sample_rows(W.shape[0], 24, 3)
    for B in (16, 32):
        for m in (hd.NAIVE, hd.SSE_OPT, hd.H_OPT):
            c, s = check_rows(m, hd.NVFP4, B, W, h_o, h, rows)
    Wq = hd.dequantize(hd.NVFP4, 32, c, s, *W.shape)
    Wd = W.cuda()
    assert hd.output_error(Xd, Wd, (2 * Wd).contiguous()).item() == 1.0
    full = hd.output_error(Xd, Wd, Wq).item()
    sub = hd.output_error(Xd[:192].contiguous(), Wd, Wq).item()
    sub_o = oracle.output_error(synth.bits(Xh[:192]), synth.bits(W), Wq.cpu().numpy())
    assert sub == pytest.approx(sub_o, rel=1e-4)
    # iid rows: the full-X error is close to the error on a row subset
    assert full == pytest.approx(sub, rel=0.1)


@pytest.mark.parametrize("fmt", ["MXFP4", "NVFP4", "MXFP8", "FP8_E4M3S"])
def test_config4_block_sweep(fmt):
    W, _ = synth.config_inputs(4)
    rows = sample_rows(W.shape[0], 16, 4)
    Wd = W.cuda()
    werr = {}
    for B in (8, 16, 32, 64, 128, 256):
        for m in (hd.NAIVE, hd.SSE_OPT):
            c, s = check_rows(m, FMT[fmt], B, W, None, None, rows)
        Wq = hd.dequantize(FMT[fmt], B, c, s, *W.shape)
        werr[B] = hd.weight_error(Wd, Wq).item()
    # weight error of SSE-Optimal falls (weakly) as blocks shrink, for every grid here
    assert werr[8] <= werr[256]


def test_config5_large_layer():
    W, _ = synth.config_inputs(5, x_rows=0)
    cfg = synth.CONFIGS[5]["X"]
    Xd = torch.empty((cfg["M"], cfg["K"]), dtype=torch.bfloat16, device="cuda")
    Xh = torch.empty((cfg["M"], cfg["K"]), dtype=torch.bfloat16)
    r = 0
    for ch in synth.activation_chunks(cfg["M"], cfg["K"], cfg["seed"], cfg["n_out"], cfg["out_gain"],
                                      cfg["idx_seed"], rows_per_chunk=4096):
        Xh[r:r + ch.shape[0]] = ch
        Xd[r:r + ch.shape[0]] = ch.cuda()
        r += ch.shape[0]
    h = hd.hdiag(Xd)
    h_o = oracle.hdiag(synth.bits(Xh))
    torch.cuda.synchronize()
    np.testing.assert_allclose(h.cpu().numpy(), h_o, rtol=1e-6)
    rows = sample_rows(W.shape[0], 12, 5)
    Wd = W.cuda()
    # the output error through G = X^T X at this size too (K = 28672: the
    # operand's two-pass path, 112 bands of C)
    gram = hd.output_gram(Xd, h=h)
    ysq = hd.output_reference_gram(Wd, gram)
    for fmt, B in ((hd.NVFP4, 16), (hd.INT8_E4M3, 128)):
        c, s = check_rows(hd.H_OPT, fmt, B, W, h_o, h, rows)
        Wq = hd.dequantize(fmt, B, c, s, *W.shape)
        # the fused dequantize and weight error at this size (many chunk pairs per thread)
        Wq_f, we_f = hd.dequantize_weight_error(fmt, B, c, s, Wd)
        assert torch.equal(Wq_f.view(torch.int32), Wq.view(torch.int32))
        assert we_f.item() == hd.weight_error(Wd, Wq).item()
        del Wq_f
        full = hd.output_error(Xd, Wd, Wq).item()
        assert hd.output_error_gram(fmt, B, c, s, Wd, gram, ysq).item() == pytest.approx(full, rel=1e-4)
        sub = hd.output_error(Xd[:64].contiguous(), Wd, Wq).item()
        sub_o = oracle.output_error(synth.bits(Xh[:64]), synth.bits(W), Wq.cpu().numpy())
        assert sub == pytest.approx(sub_o, rel=1e-4)
        assert 0.0 < full < 1.0
