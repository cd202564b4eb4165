"""hdiag_noalloc: hdiag with the library's static per-GPU scratch in place of a
caller workspace, for callers that cannot allocate device memory.

Its output must equal hdiag()'s (the same kernels on the same partial layout,
so bit for bit) and meet hdiag's parity bar against the oracle (1e-6
relative), on two calls in a row with the second on a smaller X, since the
scratch keeps the previous call's contents.
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


def _case(M, K, dtype, seed):
    X = synth.activations(M, K, seed, n_out=3, out_gain=50.0, idx_seed=seed + 1, dtype=dtype)
    Xd = X.contiguous().cuda()
    want = hd.hdiag(Xd)
    got = torch.full((K,), float("nan"), dtype=torch.float32, device=Xd.device)
    out = hd.hdiag_noalloc(Xd, got)
    assert out is got
    torch.cuda.synchronize()
    assert torch.equal(got.cpu(), want.cpu()), (M, K, dtype)
    np.testing.assert_allclose(got.cpu().numpy(), oracle.hdiag(synth.bits(X)), rtol=1e-6)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_hdiag_two_calls(dtype):
    # several 512-column strips and row chunks, then a smaller X on the same
    # scratch (fewer chunks and columns than the first call left behind)
    _case(20000, 4104, dtype, 301)
    _case(3000, 1032, dtype, 303)


def test_noalloc_ragged_columns_and_empty_rows():
    # K % 8 != 0 takes the one-column-per-lane kernel; then M = 0 gives zeros
    _case(777, 1001, torch.bfloat16, 305)
    _case(515, 37, torch.float32, 307)
    Xe = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    h = torch.full((64,), 1.0, dtype=torch.float32, device="cuda")
    hd.hdiag_noalloc(Xe, h)
    torch.cuda.synchronize()
    assert torch.equal(h.cpu(), torch.zeros(64))


def test_noalloc_on_a_side_stream():
    X = synth.activations(4096, 2048, 309, dtype=torch.bfloat16).cuda()
    want = hd.hdiag(X)
    s = torch.cuda.Stream()
    got = torch.empty(2048, dtype=torch.float32, device="cuda")
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        hd.hdiag_noalloc(X, got)
    s.synchronize()
    assert torch.equal(got.cpu(), want.cpu())


def test_noalloc_rejects_shapes_beyond_the_scratch():
    X = torch.zeros((1, 8), dtype=torch.bfloat16, device="cuda")
    h = torch.zeros(8, dtype=torch.float32, device="cuda")
    L = hd.lib()
    # a 4M-column X needs 32 MiB of partials: refused before any launch
    rc = L.hdiag_noalloc(hd._ptr(X), hd.HD_BF16, 1, 4 << 20, hd._ptr(h), None)
    assert rc == hd.HD_ERR_UNSUPPORTED
    assert "static scratch" in L.hdiag_last_error().decode()
