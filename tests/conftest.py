import os
import sys
from fractions import Fraction

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _num(tok):
    if tok.startswith("2^"):
        return Fraction(2) ** int(tok[2:])
    return Fraction(tok) if "e" not in tok else Fraction(float(tok))


def golden_kv(name):
    """key = value(s) lines of tests/golden/<name>; values as Fractions."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = line.split("=", 1)
            vals = [_num(t) for t in v.split()]
            out[k.strip()] = vals if len(vals) > 1 else vals[0]
    return out


def golden_rows(name):
    """Whitespace-separated numeric rows of tests/golden/<name>."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append([_num(t) for t in line.split()])
    return rows
