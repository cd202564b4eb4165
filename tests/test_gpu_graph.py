"""A captured HIP graph of one step of the path (hdiag, output_gram,
output_reference_gram, quantize_blocks, dequantize, weight_error,
output_error_gram_batch) replayed several times, with eager work and
synchronisations between the replays: every replay reproduces the eager
results bit for bit (the library issues no memset or allocation inside the
step, so nothing in the graph depends on state left by an earlier replay)."""
import pytest
import torch

import synth
import block_scaled_precision_hdiag_amd as hd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hd.lib()


def test_step_graph_replays_match_eager():
    M, N, K = 700, 300, 1024
    dev = torch.device("cuda:0")
    W = synth.weights("t4", N, K, std=0.02, seed=5, gain_seed=6, dtype=torch.bfloat16).to(dev)
    X = synth.activations(M, K, 7, n_out=3, out_gain=50.0, idx_seed=8, dtype=torch.bfloat16).to(dev)
    h = torch.empty(K, dtype=torch.float32, device=dev)
    ws_h = torch.empty(max(hd.hdiag_workspace_size(M, K), 16), dtype=torch.uint8, device=dev)
    gram = torch.empty(hd.output_gram_size(K), dtype=torch.uint8, device=dev)
    ws_g = torch.empty(hd.output_gram_workspace_size(M, K), dtype=torch.uint8, device=dev)
    ws_o = torch.empty(hd.output_error_gram_batch_workspace_size(3, N, K), dtype=torch.uint8, device=dev)
    ws_w = torch.empty(hd.weight_error_workspace_size(N, K), dtype=torch.uint8, device=dev)
    ysq = torch.empty(1, dtype=torch.float64, device=dev)
    plan = [(hd.NAIVE, 32), (hd.SSE_OPT, 64), (hd.H_OPT, 128)]
    codes = [torch.empty((N, K), dtype=torch.uint8, device=dev) for _ in plan]
    scales = [torch.empty((N, K // B), dtype=torch.uint8, device=dev) for _, B in plan]
    Wq = torch.empty((N, K), dtype=torch.float32, device=dev)
    werr = torch.empty(len(plan), dtype=torch.float64, device=dev)
    oerr = torch.empty(len(plan), dtype=torch.float64, device=dev)

    def step():
        hd.hdiag(X, out=h, workspace=ws_h)
        hd.output_gram(X, h=h, gram=gram, workspace=ws_g)
        hd.output_reference_gram(W, gram, workspace=ws_o, out=ysq)
        for i, (m, B) in enumerate(plan):
            hd.quantize_blocks(m, hd.INT8_E4M3, B, W, h=h, codes=codes[i], scales=scales[i])
            hd.dequantize(hd.INT8_E4M3, B, codes[i], scales[i], N, K, out=Wq)
            hd.weight_error(W, Wq, workspace=ws_w, out=werr[i:i + 1])
        hd.output_error_gram_batch([(hd.INT8_E4M3, B, codes[i], scales[i]) for i, (_, B) in enumerate(plan)], W,
                                   gram, ysq, workspace=ws_o, out=oerr)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (h, ysq, werr, oerr, *codes, *scales)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        for t in (h, ysq, werr, oerr, *codes, *scales):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (h, ysq, werr, oerr, *codes, *scales)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), r
        # eager work between replays
        step()
        torch.cuda.synchronize()


def test_two_stream_step_graph_replays_match_eager():
    """The step as the benchmark replays it: after hdiag, output_gram and
    output_reference_gram on a second stream beside the quantisation chains
    (quantize_blocks, dequantize_weight_error) on the first, which waits for
    the second before output_error_gram_batch.  Every replay reproduces the
    one-stream eager results bit for bit."""
    M, N, K = 700, 300, 1024
    dev = torch.device("cuda:0")
    W = synth.weights("t4", N, K, std=0.02, seed=15, gain_seed=16, dtype=torch.bfloat16).to(dev)
    X = synth.activations(M, K, 17, n_out=3, out_gain=50.0, idx_seed=18, dtype=torch.bfloat16).to(dev)
    h = torch.empty(K, dtype=torch.float32, device=dev)
    ws_h = torch.empty(max(hd.hdiag_workspace_size(M, K), 16), dtype=torch.uint8, device=dev)
    gram = torch.empty(hd.output_gram_size(K), dtype=torch.uint8, device=dev)
    ws_g = torch.empty(hd.output_gram_workspace_size(M, K), dtype=torch.uint8, device=dev)
    ws_o = torch.empty(hd.output_error_gram_batch_workspace_size(3, N, K), dtype=torch.uint8, device=dev)
    ws_w = torch.empty(hd.weight_error_workspace_size(N, K), dtype=torch.uint8, device=dev)
    ysq = torch.empty(1, dtype=torch.float64, device=dev)
    plan = [(hd.NAIVE, 32), (hd.SSE_OPT, 64), (hd.H_OPT, 128)]
    codes = [torch.empty((N, K), dtype=torch.uint8, device=dev) for _ in plan]
    scales = [torch.empty((N, K // B), dtype=torch.uint8, device=dev) for _, B in plan]
    Wq = torch.empty((N, K), dtype=torch.float32, device=dev)
    werr = torch.empty(len(plan), dtype=torch.float64, device=dev)
    oerr = torch.empty(len(plan), dtype=torch.float64, device=dev)
    side = torch.cuda.Stream(device=dev)

    def step(two):
        hd.hdiag(X, out=h, workspace=ws_h)
        if two:
            side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side) if two else torch.cuda.stream(torch.cuda.current_stream()):
            hd.output_gram(X, h=h, gram=gram, workspace=ws_g)
            hd.output_reference_gram(W, gram, workspace=ws_o, out=ysq)
        for i, (m, B) in enumerate(plan):
            hd.quantize_blocks(m, hd.INT8_E4M3, B, W, h=h, codes=codes[i], scales=scales[i])
            hd.dequantize_weight_error(hd.INT8_E4M3, B, codes[i], scales[i], W, out=Wq, err=werr[i:i + 1],
                                       workspace=ws_w)
        if two:
            torch.cuda.current_stream().wait_stream(side)
        hd.output_error_gram_batch([(hd.INT8_E4M3, B, codes[i], scales[i]) for i, (_, B) in enumerate(plan)], W,
                                   gram, ysq, workspace=ws_o, out=oerr)

    step(False)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (h, ysq, werr, oerr, Wq, *codes, *scales)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(True)
    for r in range(3):
        for t in (h, ysq, werr, oerr, Wq, *codes, *scales):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (h, ysq, werr, oerr, Wq, *codes, *scales)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), r
        step(False)
        torch.cuda.synchronize()
