"""Pins of the oracle's Lloyd-Max codebooks (CPU only).

What fixes them: the printed 3-bit table (TurboQuant pages, "Algorithm",
values bullet), the 1-bit closed form (+-sqrt(2/pi), distortion 1 - 2/pi),
the Lloyd-Max optimality conditions themselves, the pages' distortion
anchors (about 0.36 / 0.117 / 0.03 at 1 / 2 / 3 bits, TurboQuant page
"Oracle chain") and the Panter-Dite high-resolution law.
"""
import math
import os

import numpy as np
import pytest
from scipy.special import ndtr

from oracle import lloyd_max, tables, write_tables

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "printed_3bit_table.txt")


def _printed():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    return [float(x) for x in rows[0]], [float(x) for x in rows[1]]


def test_printed_3bit_table_is_the_lloyd_max_fixed_point():
    cent, bnd = _printed()
    c, b, _ = lloyd_max.lloyd_max_normal(3)
    assert np.allclose(np.round(c, 5), cent, atol=0, rtol=0)
    assert np.allclose(np.round(b, 5), bnd, atol=0, rtol=0)


def test_printed_boundaries_are_midpoints_of_printed_centroids():
    cent, bnd = _printed()
    mids = [round((cent[i] + cent[i + 1]) / 2, 5) for i in range(7)]
    assert mids == pytest.approx(bnd, abs=1e-12)


def test_frozen_3bit_table_is_the_printed_one():
    cent, bnd = _printed()
    c32, b32 = tables.codebook(3)
    assert np.array_equal(c32, np.array(cent, np.float32))
    assert np.array_equal(b32, np.array(bnd, np.float32))


def test_frozen_tables_regenerate_identically():
    with open(tables.TABLE_FILE) as f:
        assert f.read() == write_tables.build()


def test_one_bit_closed_form():
    c, b, _ = lloyd_max.lloyd_max_normal(1)
    assert c[1] == pytest.approx(math.sqrt(2 / math.pi), rel=1e-12)
    assert lloyd_max.distortion(c, b) == pytest.approx(1 - 2 / math.pi, rel=1e-12)


@pytest.mark.parametrize("bits", [2, 4, 5, 8])
def test_lloyd_max_conditions(bits):
    c, b, _ = lloyd_max.lloyd_max_normal(bits)
    # nearest-neighbour condition
    assert np.allclose(b, 0.5 * (c[:-1] + c[1:]), atol=1e-15)
    # centroid condition: c_k = E[X | cell k], computed with the lower tail
    edges = np.concatenate(([-np.inf], b, [np.inf]))
    phi = lambda x: np.where(np.isinf(x), 0.0, np.exp(-0.5 * np.where(np.isinf(x), 0, x) ** 2)) / math.sqrt(2 * math.pi)
    mass = ndtr(edges[1:]) - ndtr(edges[:-1])
    mean = (phi(edges[:-1]) - phi(edges[1:])) / mass
    # the far tails carry tiny mass; the lower-tail CDF loses digits there
    big = mass > 1e-6
    assert np.allclose(mean[big], c[big], rtol=1e-9, atol=1e-11)
    assert np.allclose(c, -c[::-1], atol=1e-15)


def test_distortion_anchors_from_the_pages():
    d = {b: lloyd_max.distortion(*lloyd_max.lloyd_max_normal(b)[:2]) for b in (1, 2, 3)}
    assert d[1] == pytest.approx(0.36, abs=0.005)
    assert d[2] == pytest.approx(0.117, abs=0.001)
    assert d[3] == pytest.approx(0.0345, abs=0.0005)


def test_high_resolution_law():
    # Panter-Dite: D ~ (pi*sqrt(3)/2) * 4^-b for a unit normal, as b grows
    c, b, _ = lloyd_max.lloyd_max_normal(8)
    pd = math.pi * math.sqrt(3) / 2 * 4.0 ** -8
    assert lloyd_max.distortion(c, b) == pytest.approx(pd, rel=0.02)


@pytest.mark.parametrize("bits", lloyd_max.TABLE_BITS)
def test_frozen_table_shape(bits):
    c, b = tables.codebook(bits)
    n = 1 << bits
    assert c.dtype == np.float32 and c.shape == (n,) and b.shape == (n - 1,)
    assert np.all(np.diff(c) > 0) and np.all(np.diff(b) > 0)
    assert np.all(c[:-1] < b) and np.all(b < c[1:])
    assert np.array_equal(c, -c[::-1]) and b[n // 2 - 1] == 0


MAX1960 = os.path.join(os.path.dirname(__file__), "golden", "max1960_gaussian_quantizers.txt")


def _max_table():
    out, cur = {}, None
    for line in open(MAX1960):
        if not line.strip() or line.startswith("#"):
            continue
        key, *vals = line.split()
        if key == "N":
            cur = out.setdefault(int(vals[0]), {})
        else:
            cur[key] = vals
    return out


def _unit(s):
    # one unit in the last printed decimal place of a table entry
    return 10.0 ** -(len(s.split(".")[1]) if "." in s else 0)


@pytest.mark.parametrize("levels", [4, 8, 16])
def test_tables_match_max_1960(levels):
    """The oracle's iteration against the classical published Gaussian quantizers:
    an external anchor for the 2- and 4-bit tables (and the 3-bit one) that the
    pages do not print."""
    row = _max_table()[levels]
    bits = levels.bit_length() - 1
    c, b, _ = lloyd_max.lloyd_max_normal(bits)
    n = len(c)
    for s, v in zip(row["y"], c[n // 2:]):
        assert abs(float(s) - v) <= _unit(s) * 1.0001, (levels, "y", s, v)
    for s, v in zip(row["x"], b[n // 2 - 1:]):
        assert abs(float(s) - v) <= _unit(s) * 1.0001, (levels, "x", s, v)
    if "mse" in row:
        s = row["mse"][0]
        assert abs(float(s) - lloyd_max.distortion(c, b)) <= _unit(s) * 1.0001
