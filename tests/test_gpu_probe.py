"""The streaming probes (hdiag_stream_probe) read and write exactly the bytes
their header describes: every output is compared with the same function of
the input computed on the host with numpy."""
import numpy as np
import pytest
import torch

import block_scaled_precision_hdiag_amd as hd

pytestmark = pytest.mark.gpu

N = 8192 * 5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hd.lib()


def words(n_bytes, seed):
    return np.random.default_rng(seed).integers(0, 2**32, n_bytes // 4, dtype=np.uint64).astype(np.uint32)


def test_probe_read():
    w = words(2 * N, 1)
    src = torch.from_numpy(w.view(np.int32)).cuda()
    out = torch.zeros(N // 8192, dtype=torch.int32, device="cuda")
    hd.hdiag_stream_probe(hd.PROBE_READ, N, in0=src, out0=out)
    want = np.bitwise_xor.reduce(w.reshape(-1, 4096), axis=1)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want)


def test_probe_encode():
    w = words(2 * N, 2)
    src = torch.from_numpy(w.view(np.int32)).cuda()
    codes = torch.zeros(N // 2, dtype=torch.uint8, device="cuda")
    sc = torch.zeros(N // 16, dtype=torch.uint8, device="cuda")
    hd.hdiag_stream_probe(hd.PROBE_ENCODE, N, in0=src, out0=codes, out1=sc)
    x = np.bitwise_xor.reduce(w.reshape(-1, 4), axis=1)  # one word per 8 elements
    assert np.array_equal(codes.cpu().numpy().view(np.uint32), x)
    assert np.array_equal(sc.cpu().numpy(), (x[0::2] & 255).astype(np.uint8))


def test_probe_write():
    out = torch.zeros(N, dtype=torch.int16, device="cuda")
    hd.hdiag_stream_probe(hd.PROBE_WRITE, N, out0=out)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), np.arange(N // 2, dtype=np.uint32))


def test_probe_dequant():
    c = words(N // 2, 3)
    s = np.random.default_rng(4).integers(0, 256, N // 16, dtype=np.uint8)
    out = torch.zeros(N, dtype=torch.int16, device="cuda")
    hd.hdiag_stream_probe(hd.PROBE_DEQUANT, N, in0=torch.from_numpy(c.view(np.int32)).cuda(),
                          in1=torch.from_numpy(s).cuda(), out0=out)
    sv = np.repeat(s.astype(np.uint32), 2)
    want = np.stack([c ^ sv, c + sv, np.uint32(3) * c, c >> np.uint32(3)], axis=1).reshape(-1)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want)
