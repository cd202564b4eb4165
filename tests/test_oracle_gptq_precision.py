"""How far GPTQ's decisions move under rounding alone (oracle only, host).

GPTQ quantises a row's columns in sequence and propagates each error to the
later columns, so one flipped element changes the compensation of the rest
of its row.  This runs the oracle's float64 GPTQ against its precision
experiment (oracle.gptq_emulated), which changes one thing at a time:
  - HULP: H moved by one float64 ulp on half of its entries, what a float64
    computation in another order does;
  - W32: working weights stored in float32 after every update (errors and
    products in float32), the precision a float32 implementation keeps.
A float64-order perturbation moves no decision, so an implementation that
keeps the loop in float64 can be held to the search's 99.99% bar; float32
working weights move a few tenths of a percent of INT8 elements (the finest
grid), which is why the GPU loop is float64.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

INT8_E4M3, NVFP4, MXFP4 = 0, 1, 2
NAIVE, SSE_OPT, H_OPT = 0, 1, 2


@pytest.fixture(scope="module")
def inputs():
    N, K, M = 128, 1024, 2048
    W = synth.weights("t4", N, K, std=0.02, seed=5, gain_seed=6, dtype=torch.bfloat16)
    X = synth.activations(M, K, 7, n_out=6, out_gain=30.0, idx_seed=8, dtype=torch.bfloat16)
    Wb = synth.bits(W)
    return Wb, oracle.xtx(synth.bits(X)), N, K


def agreement(inputs, fmt, B, method, emul):
    Wb, H, N, K = inputs
    c0, s0, _ = oracle.gptq(method, fmt, B, Wb, H)
    c1, s1, _ = oracle.gptq_emulated(method, fmt, B, Wb, H, emul)
    q0 = oracle.dequantize(fmt, B, c0, s0, N, K)
    q1 = oracle.dequantize(fmt, B, c1, s1, N, K)
    return (s0 == s1).mean(), (q0 == q1).mean()


@pytest.mark.parametrize("fmt,B,method", [(NVFP4, 16, H_OPT), (INT8_E4M3, 32, SSE_OPT), (MXFP4, 32, NAIVE)])
def test_float64_order_moves_no_decision(inputs, fmt, B, method):
    fs, fe = agreement(inputs, fmt, B, method, oracle.GPTQ_EMUL_HULP)
    assert fs == 1.0 and fe == 1.0


def test_float32_working_weights_move_int8_decisions(inputs):
    fs, fe = agreement(inputs, INT8_E4M3, 32, SSE_OPT, oracle.GPTQ_EMUL_W32)
    assert 0.99 < fe < 0.9995 and fs < 0.9995


def test_emulation_off_is_the_oracle(inputs):
    fs, fe = agreement(inputs, NVFP4, 16, H_OPT, 0)
    assert fs == 1.0 and fe == 1.0
