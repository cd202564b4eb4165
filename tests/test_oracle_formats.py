"""Pins of the oracle's number formats and element rounding (CPU only).

The tables are checked against the facts the pages print (tests/golden/formats.txt)
and against a direct enumeration of the LLM-FP4 value formula; the sorted-table
rounding is checked against the independent step-size quantiser in fpref.py,
exhaustively over every bfloat16 value and over whole float32 binades.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from conftest import golden_kv, golden_rows
import fpref



def tbl_e2m1():
    return oracle.fp_table(2, 1, 1, 0)


def tbl_e4m3():
    return oracle.fp_table(4, 3, 7, 1)


def test_formats_against_printed_facts():
    g = golden_kv("formats.txt")
    e2 = tbl_e2m1()
    assert [Fraction(v) for v in e2] == g["e2m1_values"]
    assert Fraction(e2.max()) == g["e2m1_max"]
    assert Fraction(fpref.p4_qmax(2, 1, 1)) == g["e2m1_qmax_formula"]
    e4 = tbl_e4m3()
    assert e4[0] == 0 and np.all(np.diff(e4) > 0)
    assert (e4 > 0).sum() == g["e4m3_positive_count"]
    assert Fraction(e4.max()) == g["e4m3_max"]
    assert Fraction(e4[1]) == g["e4m3_min_positive"]
    # the P4 Q_max formula gives 480 for E4M3: exactly one top step (32) above
    # 448, the all-ones code OCP reserves for NaN
    assert fpref.p4_qmax(4, 3, 7) == e4.max() + 32
    assert oracle.fp_table(4, 3, 7, 0).max() == fpref.p4_qmax(4, 3, 7)
    ue44 = oracle.fp_table(4, 4, 7, 0)
    assert (ue44 > 0).sum() == g["ue4m4_positive_count"]
    assert Fraction(ue44.max()) == g["ue4m4_max"]
    ue53 = oracle.fp_table(5, 3, 15, 0)
    assert (ue53 > 0).sum() == g["ue5m3_positive_count"]
    assert Fraction(ue53.max()) == g["ue5m3_max"]
    assert Fraction(ue53[1]) == g["ue5m3_min_positive"]
    e52 = oracle.fp_table(5, 2, 15, 2)
    assert Fraction(e52.max()) == g["e5m2_max"]
    e8 = oracle.e8m0_table()
    assert e8.size == 255 and Fraction(e8[0]) == g["e8m0_min"]
    assert np.all(e8[1:] == 2 * e8[:-1]) and e8[-1] == 2.0 ** 127


@pytest.mark.parametrize("e,m,b,res", [(2, 1, 1, 0), (4, 3, 7, 1), (4, 4, 7, 0), (5, 3, 15, 0)])
def test_table_matches_value_formula(e, m, b, res):
    assert np.array_equal(oracle.fp_table(e, m, b, res), fpref.grid(e, m, b, res))


def test_e2m1_boundary_ties():
    T = tbl_e2m1()
    for q, val, idx in golden_rows("e2m1_ties.txt"):
        assert oracle.rne_index(T, float(q)) == idx
        assert T[int(idx)] == float(val)


def _check_rounding(T, x, fmt):
    idx = oracle.rne_index(T, x)
    ref = fpref.p4_round(x, fmt)
    got = T[idx]
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, "first mismatch x=%r oracle=%r ref=%r" % (x[bad[0]], got[bad[0]], ref[bad[0]])


@pytest.mark.parametrize("name", ["e2m1", "e4m3"])
def test_rounding_every_bf16(name):
    T, fmt = (tbl_e2m1(), fpref.E2M1) if name == "e2m1" else (tbl_e4m3(), fpref.E4M3)
    x = fpref.all_positive_bf16()
    _check_rounding(T, np.concatenate([x, np.array([np.inf], np.float32)]), fmt)


def test_rounding_e2m1_whole_binades():
    # every float32 in [2^-4, 2^4): all seven decision boundaries and saturation
    T = tbl_e2m1()
    for e in range(-4, 4):
        _check_rounding(T, fpref.binade_f32(e, e + 1), fpref.E2M1)


def test_rounding_e4m3_whole_binades():
    # subnormal range and the zero bin, one normal binade, the top and saturation
    T = tbl_e4m3()
    for e in list(range(-12, -5)) + [0, 7, 8, 9]:
        _check_rounding(T, fpref.binade_f32(e, e + 1), fpref.E4M3)


def test_rounding_int8():
    T = np.arange(128, dtype=np.float64)
    x = fpref.all_positive_bf16()
    ties = np.arange(0, 130, dtype=np.float32) + np.float32(0.5)
    near = np.concatenate([np.nextafter(ties, np.float32(0)), ties, np.nextafter(ties, np.float32(1e9))])
    rng = np.random.default_rng(5)
    rand = rng.uniform(0, 140, 1 << 20).astype(np.float32)
    for xs in (x, near, rand):
        idx = oracle.rne_index(T, xs)
        assert np.array_equal(T[idx], fpref.int_round(xs, 127))
