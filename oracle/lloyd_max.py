"""Lloyd-Max scalar quantizer for the unit normal density (oracle, test infrastructure).

TurboQuant KV design page, "Algorithm", values bullet: the value code is a
Lloyd-Max quantizer designed for a unit normal, generated once and then
frozen as constants.  The pages obtain theirs by a sampled iteration whose
random stream is not available here; this module instead runs the classical
Lloyd-Max fixed-point iteration on the exact N(0, 1) density in float64:

* boundaries are midpoints of neighbouring centroids (nearest-centroid rule);
* each centroid is the conditional mean of N(0, 1) over its cell,
  ``c = (phi(a) - phi(b)) / (Q(a) - Q(b))`` for the cell (a, b), with
  ``phi`` the density and ``Q(x) = P(X > x)`` the upper tail.

The quantizer is symmetric, so only the positive half is iterated (the
middle boundary is 0 for an even number of levels).  Tail masses use the
upper tail ``Q`` so that cells far out keep their precision.

The fp32 tables are the round-to-nearest float32 of the float64 fixed
point.  The 3-bit table is the one the pages print, taken verbatim.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import ndtr, ndtri

_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _phi(x):
    return _INV_SQRT_2PI * np.exp(-0.5 * x * x)


def _upper_tail(x):
    return ndtr(-x)


def lloyd_max_normal(bits: int, tol: float = 1e-12, max_iter: int = 2_000_000):
    """Converged float64 (centroids, boundaries, iterations) for 2**bits levels."""
    levels = 1 << bits
    half = levels // 2
    # quantile initialisation of the positive centroids
    k = np.arange(half, levels, dtype=np.float64)
    c = ndtri((k + 0.5) / levels)
    for it in range(1, max_iter + 1):
        inner = 0.5 * (c[:-1] + c[1:])
        lo = np.concatenate(([0.0], inner))
        hi = np.concatenate((inner, [np.inf]))
        mass = _upper_tail(lo) - _upper_tail(hi)
        new = (_phi(lo) - _phi(hi)) / mass
        delta = np.max(np.abs(new - c))
        c = new
        if delta < tol:
            break
    else:
        raise RuntimeError(f"Lloyd-Max {bits}-bit did not converge")
    cent = np.concatenate((-c[::-1], c))
    bnd = 0.5 * (cent[:-1] + cent[1:])
    bnd[half - 1] = 0.0
    return cent, bnd, it


def distortion(centroids, boundaries) -> float:
    """Mean squared error of the quantizer on N(0, 1), exact by cell integrals.

    For a cell (a, b) with centroid c:  E[(X - c)^2; a < X < b]
      = [x phi]  terms + (1 + c^2) mass - 2 c (phi(a) - phi(b)).
    """
    edges = np.concatenate(([-np.inf], np.asarray(boundaries, np.float64), [np.inf]))
    c = np.asarray(centroids, np.float64)
    a, b = edges[:-1], edges[1:]
    mass = ndtr(b) - ndtr(a)
    dphi = _phi(a) - _phi(b)
    # E[X^2; a<X<b] = mass + a phi(a) - b phi(b)   (with x phi(x) -> 0 at +-inf)
    fa = np.where(np.isinf(a), 0.0, a)
    fb = np.where(np.isinf(b), 0.0, b)
    aphi = fa * _phi(fa) * np.isfinite(a)
    bphi = fb * _phi(fb) * np.isfinite(b)
    ex2 = mass + aphi - bphi
    return float(np.sum(ex2 - 2.0 * c * dphi + c * c * mass))


# 3-bit table as printed on the TurboQuant KV design pages ("Algorithm",
# values bullet): centroids +-{0.24509, 0.75601, 1.34391, 2.15195},
# boundaries +-{0.50055, 1.04996, 1.74793} and 0.
PRINTED_3BIT_CENTROIDS = ("-2.15195", "-1.34391", "-0.75601", "-0.24509",
                          "0.24509", "0.75601", "1.34391", "2.15195")
PRINTED_3BIT_BOUNDARIES = ("-1.74793", "-1.04996", "-0.50055", "0",
                           "0.50055", "1.04996", "1.74793")

# Widths the tables are built for: the served value widths {2,3,4,5,8}
# plus 1 bit, used only by the distortion-anchor tests.
TABLE_BITS = (1, 2, 3, 4, 5, 8)


def fp32_table(bits: int):
    """(centroids, boundaries) as float32 arrays for ``bits``."""
    if bits == 3:
        cent = np.array([float(s) for s in PRINTED_3BIT_CENTROIDS], dtype=np.float32)
        bnd = np.array([float(s) for s in PRINTED_3BIT_BOUNDARIES], dtype=np.float32)
        return cent, bnd
    cent, bnd, _ = lloyd_max_normal(bits)
    return cent.astype(np.float32), bnd.astype(np.float32)
