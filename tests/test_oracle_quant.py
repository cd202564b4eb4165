"""Pins of the oracle's scale choice, encode and dequantize (CPU only).

- Exact brute force: every candidate scale of small blocks is evaluated here in
  exact rational arithmetic with the independent step-size rounding of fpref.py;
  the oracle must pick an exact minimiser (the lowest code when it is unique).
- Encode of every bfloat16 value at every candidate scale against fpref.py.
- Closed-form Naive cases: zero-scale bin, saturation, INT8 amax/127, E8M0 snap.
- Invariants that hold because Naive's scale is one of the candidates, and exact
  special cases (sign flip, power-of-two shifts, weights on a grid point, h = 2^k).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import fpref
from oracle import (NAIVE, SSE_OPT, H_OPT, NAIVE_OCP, INT8_E4M3, NVFP4, MXFP4, MXFP8, FP8_E4M3S,
                    NVFP4_UE4M4, NVFP4_UE5M3, NVINT4)

ALL_FMTS = [INT8_E4M3, NVFP4, MXFP4, MXFP8, FP8_E4M3S, NVFP4_UE4M4, NVFP4_UE5M3, NVINT4]
E2M1_FMTS = (NVFP4, MXFP4, NVFP4_UE4M4, NVFP4_UE5M3)
E4M3_GRID = fpref.grid(4, 3, 7, True)
UE4M4_GRID = fpref.grid(4, 4, 7, False)
UE5M3_GRID = fpref.grid(5, 3, 15, False)


def ref_scales(fmt):
    """(code, fp32 scale) of every candidate, derived here independently."""
    if fmt == INT8_E4M3:
        return [(c, np.float32(E4M3_GRID[c]) / np.float32(127)) for c in range(1, 127)]
    if fmt in (NVFP4, FP8_E4M3S, NVINT4):
        return [(c, np.float32(E4M3_GRID[c])) for c in range(1, 127)]
    if fmt == NVFP4_UE4M4:
        return [(c, np.float32(UE4M4_GRID[c])) for c in range(1, 256)]
    if fmt == NVFP4_UE5M3:
        return [(c, np.float32(UE5M3_GRID[c])) for c in range(1, 256)]
    return [(c, np.float32(np.ldexp(1.0, c - 127))) for c in range(255)]


def ref_elem_round(fmt, x):
    if fmt == INT8_E4M3:
        return fpref.int_round(x, 127)
    if fmt == NVINT4:
        return fpref.int_round(x, 7)
    if fmt in E2M1_FMTS:
        return fpref.p4_round(x, fpref.E2M1)
    return fpref.p4_round(x, fpref.E4M3)


def ref_dequant_block(fmt, s, w):
    """fp32 sign * fl32(s * Q(fl32(|w| / s))) for a float32 block."""
    with np.errstate(over="ignore", divide="ignore"):
        x = np.abs(w).astype(np.float32) / np.float32(s)
    q = ref_elem_round(fmt, x).astype(np.float32)
    with np.errstate(over="ignore"):
        mag = np.float32(s) * q
    return np.where(np.signbit(w), -mag, mag).astype(np.float32)


def exact_objective(fmt, s, w, h):
    wq = ref_dequant_block(fmt, s, w)
    tot = Fraction(0)
    for j in range(w.size):
        d = Fraction(float(w[j])) - Fraction(float(wq[j]))
        tot += (Fraction(float(h[j])) if h is not None else 1) * d * d
    return tot


def tiny_blocks(seed, B, count):
    rng = np.random.default_rng(seed)
    blocks = []
    for i in range(count):
        kind = i % 4
        if kind == 0:
            w = rng.normal(0, 0.02, B)
        elif kind == 1:
            w = rng.standard_t(3, B) * 0.05
        elif kind == 2:
            w = rng.normal(0, 1.0, B)
            w[rng.integers(B)] *= 20  # an outlier
        else:
            w = rng.laplace(0, 3e-3, B)
        blocks.append(w.astype(np.float32))
    return blocks


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("method", [SSE_OPT, H_OPT])
def test_search_is_exact_argmin(fmt, method):
    B = 8
    blocks = tiny_blocks(100 + fmt, B, 16)
    rng = np.random.default_rng(7 + fmt)
    h = (rng.normal(0, 1, (64, B)) ** 2).sum(0).astype(np.float32)
    h[rng.integers(B)] *= 1e4  # an outlier channel
    W = np.stack(blocks)
    hh = h if method == H_OPT else None
    _, scales, obj = oracle.quantize(method, fmt, B, W, h=hh)
    cands = ref_scales(fmt)
    for i, w in enumerate(blocks):
        objs = [(exact_objective(fmt, s, w, hh), c) for c, s in cands]
        best = min(objs)
        chosen = scales[i, 0]
        ex = dict((c, o) for o, c in objs)[chosen]
        assert ex == best[0], "block %d: oracle code %d is not a minimiser" % (i, chosen)
        if sum(1 for o, _ in objs if o == best[0]) == 1:
            assert chosen == best[1]
        assert abs(float(ex) - obj[i, 0]) <= 1e-12 * max(float(ex), 1e-300)


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_block_all_objectives_exact(fmt):
    w = tiny_blocks(300 + fmt, 16, 1)[0]
    codes, obj = oracle.block_all_objectives(fmt, w)
    cands = ref_scales(fmt)
    assert [c for c, _ in cands] == list(codes)
    for (c, s), o in zip(cands, obj):
        ex = exact_objective(fmt, s, w, None)
        assert abs(float(ex) - o) <= 1e-12 * float(ex) + 1e-300


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_encode_every_bf16_at_every_scale(fmt):
    x = fpref.all_positive_bf16()
    x = np.concatenate([x, -x[1::7]])  # and a spread of negative values
    B = 8
    K = (x.size // B) * B
    x = x[:K]
    cands = ref_scales(fmt)
    step = 1 if fmt in (INT8_E4M3, NVFP4, FP8_E4M3S, NVINT4) else 3
    cands = cands[::step]
    W = np.tile(x, (len(cands), 1))
    scales_in = np.array([[c] * (K // B) for c, _ in cands], np.uint8)
    codes, _, _ = oracle.quantize(NAIVE, fmt, B, W, scales_in=scales_in)
    deq = oracle.dequantize(fmt, B, codes, scales_in, W.shape[0], K)
    for r, (c, s) in enumerate(cands):
        ref = ref_dequant_block(fmt, s, x)
        np.testing.assert_array_equal(deq[r], ref)
        assert np.array_equal(np.signbit(deq[r]), np.signbit(x)) or fmt in (INT8_E4M3, NVINT4)


def _naive_code_ref(fmt, amax):
    amax = np.float32(amax)
    if fmt == INT8_E4M3:
        v = fpref.p4_round(np.array([amax]), fpref.E4M3)[0]
        return int(np.nonzero(E4M3_GRID == v)[0][0])
    C = np.float32(6) if fmt in E2M1_FMTS else (np.float32(7) if fmt == NVINT4 else np.float32(448))
    v = amax / C
    if fmt in (NVFP4, FP8_E4M3S, NVINT4):
        r = fpref.p4_round(np.array([v]), fpref.E4M3)[0]
        return int(np.nonzero(E4M3_GRID == r)[0][0])
    if fmt in (NVFP4_UE4M4, NVFP4_UE5M3):
        spec, grid = (fpref.UE4M4, UE4M4_GRID) if fmt == NVFP4_UE4M4 else (fpref.UE5M3, UE5M3_GRID)
        r = fpref.p4_round(np.array([v]), spec)[0]
        return int(np.nonzero(grid == r)[0][0])
    if v == 0:
        return 0
    fv = Fraction(float(v))
    E = 0
    while Fraction(2) ** E > fv:
        E -= 1
    while Fraction(2) ** (E + 1) <= fv:
        E += 1
    if fv >= Fraction(3, 2) * Fraction(2) ** E:  # nearer power of two, ties upward
        E += 1
    return min(max(E, -127), 127) + 127


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_naive_code_closed_form(fmt):
    rng = np.random.default_rng(11 + fmt)
    amaxes = np.concatenate([rng.lognormal(-3, 3, 400), [0.0, 1.0, 6.0, 9.0, 448.0, 2688.0, 1e6, 1e-30]])
    for a in amaxes.astype(np.float32):
        assert oracle.naive_scale_code(fmt, a) == _naive_code_ref(fmt, a), (fmt, a)


def test_naive_special_cases():
    # zero-scale bin ("Is Finer Better?", App. F.3): amax/C <= s_min/2 = 2^-10
    # rounds the E4M3 scale to 0; the exact tie goes to the even code 0
    t = np.float32(2.0 ** -10)
    assert oracle.naive_scale_code(NVFP4, 6 * t) == 0
    assert oracle.naive_scale_code(NVFP4, np.nextafter(6 * t, np.float32(1))) == 1
    assert oracle.naive_scale_code(INT8_E4M3, t) == 0
    assert oracle.naive_scale_code(INT8_E4M3, np.nextafter(t, np.float32(1))) == 1
    assert oracle.naive_scale_code(FP8_E4M3S, 448 * t) == 0
    # saturation of the scale at 448
    assert oracle.naive_scale_code(NVFP4, 448 * 6 * 4) == 126
    assert oracle.naive_scale_code(INT8_E4M3, 1000.0) == 126
    # INT8: amax = 1.0 -> E4M3 code 0x38, effective scale fl32(1/127)
    assert oracle.naive_scale_code(INT8_E4M3, 1.0) == 0x38
    assert oracle.scale_value(INT8_E4M3, 0x38) == np.float32(1) / np.float32(127)
    # E8M0: v = amax/6; 1.0 -> 2^0; 1.5 is a tie and goes up
    assert oracle.naive_scale_code(MXFP4, 6.0) == 127
    assert oracle.naive_scale_code(MXFP4, 9.0) == 128
    assert oracle.naive_scale_code(MXFP4, np.nextafter(np.float32(9.0), np.float32(0))) == 127
    assert oracle.naive_scale_code(MXFP4, 0.0) == 0
    assert oracle.naive_scale_code(MXFP4, np.float32(2.0 ** 127)) == 251  # 2^127/6 = (4/3) 2^124
    assert oracle.naive_scale_code(MXFP4, np.float32(1e-40)) == 0      # clamped at 2^-127


def test_zero_scale_block_encodes_to_signed_zeros():
    w = np.array([[3e-4, -2e-4, 0.0, -0.0, 1e-4, -5e-4, 5.8e-3, 0.0]], np.float32)
    codes, scales, obj = oracle.quantize(NAIVE, NVFP4, 8, w)
    assert scales[0, 0] == 0
    # E2M1 codes: sign bit 3; element 2i in the low nibble
    assert list(codes[0]) == [0x80, 0x80, 0x80, 0x00]
    assert obj[0, 0] == pytest.approx(float((w.astype(np.float64) ** 2).sum()), rel=1e-15)


def test_e2m1_packing_order():
    s_code = 0x38  # 1.0
    w = np.array([[6.0, 0.5, -1.5, 3.0, 0, 0, 0, 0]], np.float32)
    codes, _, _ = oracle.quantize(NAIVE, NVFP4, 8, w, scales_in=np.array([[s_code]], np.uint8))
    assert codes[0, 0] == 0x17  # element 0 -> low nibble (6.0 = 0b111), element 1 -> high (0.5 = 0b001)
    assert codes[0, 1] == 0x5B  # -1.5 = 0b1011, 3.0 = 0b0101


def mid_weights(seed, N=48, K=512, dtype=np.float32):
    rng = np.random.default_rng(seed)
    g = rng.lognormal(0, 0.5, N)[:, None]
    return (rng.standard_t(4, (N, K)) * 0.02 * g).astype(dtype)


def mid_h(seed, K=512):
    rng = np.random.default_rng(seed)
    X = rng.normal(0, 1, (256, K))
    X[:, rng.choice(K, 4, replace=False)] *= 50
    return (X ** 2).sum(0).astype(np.float32)


@pytest.mark.parametrize("fmt,B", [(INT8_E4M3, 32), (INT8_E4M3, 128), (NVFP4, 16), (MXFP4, 32),
                                   (MXFP8, 32), (FP8_E4M3S, 16), (NVFP4_UE4M4, 16), (NVFP4_UE5M3, 16),
                                   (NVINT4, 16)])
def test_per_block_invariants(fmt, B):
    W = mid_weights(21)
    h = mid_h(22)
    _, sn, _ = oracle.quantize(NAIVE, fmt, B, W)
    _, ss, _ = oracle.quantize(SSE_OPT, fmt, B, W)
    _, sh, _ = oracle.quantize(H_OPT, fmt, B, W, h=h)
    sse = lambda sc: oracle.objectives_at(fmt, B, W, sc)
    hw = lambda sc: oracle.objectives_at(fmt, B, W, sc, h=h)
    assert np.all(sse(ss) <= sse(sn))
    assert np.all(hw(sh) <= hw(ss))
    assert np.all(hw(sh) <= hw(sn))
    assert np.all(sse(ss) <= sse(sh))


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_h_power_of_two_equals_sse(fmt):
    W = mid_weights(31, N=16, K=256)
    _, ss, os_ = oracle.quantize(SSE_OPT, fmt, 32, W)
    for k in (0, 2, -3):
        h = np.full(256, 2.0 ** k, np.float32)
        _, sh, oh = oracle.quantize(H_OPT, fmt, 32, W, h=h)
        assert np.array_equal(ss, sh)
        assert np.array_equal(oh, os_ * 2.0 ** k)


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_sign_flip(fmt):
    W = mid_weights(41, N=16, K=256)
    h = mid_h(42, 256)
    for m in (NAIVE, SSE_OPT, H_OPT):
        c1, s1, o1 = oracle.quantize(m, fmt, 32, W, h=h)
        c2, s2, o2 = oracle.quantize(m, fmt, 32, -W, h=h)
        assert np.array_equal(s1, s2) and np.array_equal(o1, o2)
        if fmt == INT8_E4M3:
            assert np.array_equal(c1.view(np.int8), -c2.view(np.int8))
        elif fmt == NVINT4:  # two's complement nibbles: negate each
            neg = lambda c: ((-(c & 15)) & 15) | (((-(c >> 4)) & 15) << 4)
            assert np.array_equal(neg(c1.astype(int)), c2.astype(int))
        elif fmt in E2M1_FMTS:
            assert np.array_equal(c1 ^ 0x88, c2)
        else:
            assert np.array_equal(c1 ^ 0x80, c2)


@pytest.mark.parametrize("fmt", [MXFP4, MXFP8])
def test_e8m0_power_of_two_shift(fmt):
    W = mid_weights(51, N=16, K=256)
    h = mid_h(52, 256)
    for m in (NAIVE, SSE_OPT, H_OPT):
        c1, s1, _ = oracle.quantize(m, fmt, 32, W, h=h)
        for k in (-5, 3, 17):
            c2, s2, _ = oracle.quantize(m, fmt, 32, (W * np.float32(2.0 ** k)).astype(np.float32), h=h)
            assert np.array_equal(s2.astype(int), s1.astype(int) + k)
            assert np.array_equal(c1, c2)


@pytest.mark.parametrize("fmt,step", [(INT8_E4M3, 8), (NVFP4, 8), (FP8_E4M3S, 8), (NVINT4, 8),
                                      (NVFP4_UE4M4, 16), (NVFP4_UE5M3, 8)])
def test_e4m3_scale_binade_shift(fmt, step):
    # magnitudes ~1 keep every competitive candidate in the normal range of
    # the scale grid, so doubling W moves the chosen scale up by one binade
    # (8 codes; 16 on the UE4M4 grid)
    rng = np.random.default_rng(61)
    W = (rng.standard_t(4, (16, 256)) * (0.3 if fmt != FP8_E4M3S else 40.0)).astype(np.float32)
    h = mid_h(62, 256)
    for m in (NAIVE, SSE_OPT, H_OPT):
        c1, s1, o1 = oracle.quantize(m, fmt, 32, W, h=h)
        c2, s2, o2 = oracle.quantize(m, fmt, 32, (2 * W).astype(np.float32), h=h)
        assert np.array_equal(s2.astype(int), s1.astype(int) + step)
        assert np.array_equal(c1, c2)
        np.testing.assert_allclose(o2, 4 * o1, rtol=1e-15)


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_weights_on_a_grid_point(fmt):
    rng = np.random.default_rng(71 + fmt)
    B, nb = 16, 12
    cands = ref_scales(fmt)
    rows = []
    for i in range(nb):
        c, s = cands[rng.integers(len(cands) // 4, 3 * len(cands) // 4)]
        if fmt == INT8_E4M3:
            q = rng.integers(-127, 128, B).astype(np.float32)
        elif fmt == NVINT4:
            q = rng.integers(-7, 8, B).astype(np.float32)
        elif fmt in E2M1_FMTS:
            q = rng.choice([0, .5, 1, 1.5, 2, 3, 4, 6], B) * rng.choice([-1, 1], B)
        else:
            q = rng.choice(E4M3_GRID[1:], B) * rng.choice([-1, 1], B)
        rows.append((np.float32(s) * q.astype(np.float32)).astype(np.float32))
    W = np.concatenate(rows)[None, :]
    codes, sc, obj = oracle.quantize(SSE_OPT, fmt, B, W)
    assert np.all(obj == 0)
    deq = oracle.dequantize(fmt, B, codes, sc, 1, W.size)
    np.testing.assert_array_equal(deq, W)


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_dequantize_matches_block_objective(fmt):
    W = mid_weights(81, N=8, K=256)
    B = 32
    codes, sc, obj = oracle.quantize(SSE_OPT, fmt, B, W)
    deq = oracle.dequantize(fmt, B, codes, sc, 8, 256)
    d = (W.astype(np.float64) - deq.astype(np.float64)).reshape(8, 256 // B, B)
    np.testing.assert_allclose((d * d).sum(-1), obj, rtol=1e-12)


def test_bf16_input_equals_widened_fp32():
    W = mid_weights(91, N=8, K=256)
    import torch
    Wb = torch.from_numpy(W).to(torch.bfloat16)
    bits = Wb.view(torch.int16).numpy().view(np.uint16)
    W32 = Wb.float().numpy()
    h = mid_h(92, 256)
    for m in (NAIVE, SSE_OPT, H_OPT):
        a = oracle.quantize(m, NVFP4, 16, bits, h=h)
        b = oracle.quantize(m, NVFP4, 16, W32, h=h)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


def test_invalid_arguments():
    W = np.zeros((2, 30), np.float32)
    with pytest.raises(ValueError):
        oracle.quantize(SSE_OPT, NVFP4, 16, W)  # K % B != 0
    with pytest.raises(ValueError):
        oracle.quantize(H_OPT, NVFP4, 2, np.zeros((2, 32), np.float32))  # H-Optimal needs h


def test_nvint4_codes_and_packing():
    # scale 1.0 (E4M3 code 0x38): integers encode as themselves, halves tie to
    # even, |x| > 7 saturates; two's complement nibbles, element 2i low
    w = np.array([[7.0, -7.0, 1.0, -1.0, 0.0, 3.4, -3.5, 2.5, 9.0, -0.4, 4.5, -6.5, 0, 0, 0, 0]], np.float32)
    codes, _, obj = oracle.quantize(NAIVE, NVINT4, 16, w, scales_in=np.array([[0x38]], np.uint8))
    assert list(codes[0]) == [0x97, 0xF1, 0x30, 0x2C, 0x07, 0xA4, 0x00, 0x00]
    deq = oracle.dequantize(NVINT4, 16, codes, np.array([[0x38]], np.uint8), 1, 16)
    np.testing.assert_array_equal(deq[0], [7, -7, 1, -1, 0, 3, -4, 2, 7, -0.0, 4, -6, 0, 0, 0, 0])
    # Naive: E4M3(amax / 7); amax = 7 -> scale 1.0
    assert oracle.naive_scale_code(NVINT4, 7.0) == 0x38
    # the INT4 code -8 (0x8 nibble) is not a symmetric INT4 value
    with pytest.raises(ValueError):
        oracle.dequantize(NVINT4, 8, np.array([[0x08, 0, 0, 0]], np.uint8), np.array([[0x38]], np.uint8), 1, 8)


def test_unsigned_scale_grids():
    # 255 positive candidates each; UE4M4 halves the E4M3 step (16 codes per
    # binade), UE5M3 keeps 8 per binade and reaches 2^-17 .. 122880
    for fmt, grid in ((NVFP4_UE4M4, UE4M4_GRID), (NVFP4_UE5M3, UE5M3_GRID)):
        assert oracle.candidates(fmt).tolist() == list(range(1, 256))
        assert [oracle.scale_value(fmt, c) for c in range(256)] == [np.float32(v) for v in grid]
    assert oracle.scale_value(NVFP4_UE4M4, 255) == 496.0
    assert oracle.scale_value(NVFP4_UE5M3, 1) == np.float32(2.0 ** -17)
    assert oracle.scale_value(NVFP4_UE5M3, 255) == 122880.0
    # one E4M3 binade [1, 2) holds 8 codes, UE4M4's holds 16
    assert sum(1 <= v < 2 for v in UE4M4_GRID) == 16 and sum(1 <= v < 2 for v in E4M3_GRID) == 8
    # Naive zero bin: amax / 6 at or below half the smallest positive scale
    assert oracle.naive_scale_code(NVFP4_UE5M3, np.float32(6 * 2.0 ** -18)) == 0
    assert oracle.naive_scale_code(NVFP4_UE5M3, np.nextafter(np.float32(6 * 2.0 ** -18), np.float32(1))) == 1
    assert oracle.naive_scale_code(NVFP4_UE4M4, np.float32(6 * 496.0 * 2)) == 255  # saturates


def test_ocp_floor_naive():
    # OCP MX: 2^(floor(log2 amax) - emax), emax = 2 (E2M1), 8 (E4M3)
    assert oracle.naive_ocp_code(MXFP4, 6.0) == 127          # floor(log2 6) = 2
    assert oracle.naive_ocp_code(MXFP4, np.float32(7.99)) == 127
    assert oracle.naive_ocp_code(MXFP4, 8.0) == 128
    assert oracle.naive_ocp_code(MXFP4, np.nextafter(np.float32(4.0), np.float32(0))) == 126
    assert oracle.naive_ocp_code(MXFP8, 448.0) == 127        # floor(log2 448) = 8
    assert oracle.naive_ocp_code(MXFP8, 1.0) == 119
    assert oracle.naive_ocp_code(MXFP4, 0.0) == 0
    assert oracle.naive_ocp_code(MXFP4, np.float32(2.0 ** -140)) == 0   # clamped at 2^-127
    assert oracle.naive_ocp_code(NVFP4, 1.0) == -1                      # not an E8M0 format
    # unlike the nearest-power-of-two snap, the floor rule never rounds up:
    # amax = 9 (v = 1.5) snaps to 2^1 but floors to 2^1 as well; amax = 7 (v =
    # 1.17) snaps to 2^0 and floors to 2^0; amax = 11.9 snaps to 2^1, floors to 2^1
    W = mid_weights(101, N=8, K=256)
    for fmt in (MXFP4, MXFP8):
        c, s, o = oracle.quantize(NAIVE_OCP, fmt, 32, W)
        amax = np.abs(W).reshape(8, 8, 32).max(-1)
        assert np.array_equal(s, np.vectorize(lambda a: oracle.naive_ocp_code(fmt, a))(amax))
        # no element of a floor-rule block saturates: amax / s < 2^(emax + 1)
        emax = 2 if fmt == MXFP4 else 8
        sv = np.vectorize(lambda cc: float(oracle.scale_value(fmt, cc)))(s)
        assert np.all(amax / sv < 2.0 ** (emax + 1))
    with pytest.raises(ValueError):
        oracle.quantize(NAIVE_OCP, NVFP4, 16, W)
