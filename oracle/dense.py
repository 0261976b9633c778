"""Plain CPU oracle of the paper variant of the codec (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
module; the library never imports or calls it.

Source: the "Oracle chain" section of the TurboQuant KV design pages (on both
the TurboQuant page and the TurboQuant KV design page).  It sets the paper's
own codec apart from the served one: a dense random rotation obtained from
the QR decomposition of a Gaussian matrix, no groups (one norm per vector),
the same codec for keys and values, and an optional QJL stage on the
residual.  The rotation makes every coordinate of a unit vector close to
Gaussian, which is why a Lloyd-Max scalar code is the right one, and the
distortion shrinks about fourfold per bit.  The same section describes a
third design with whole-vector norms and "MSE" and "Prod" codecs, whose
unit-vector MSE anchors are about 0.36, 0.117 and 0.03 at 1, 2 and 3 bits;
the pins in tests/test_oracle_dense.py hold this oracle to them.

The pages give the design, not its arithmetic.  Readings taken (each the
plainest one the rest supports; the QJL estimator is the published one of
the TurboQuant paper the pages cite):

* The rotation P and the Gaussian projection S are d x d inputs, drawn once
  and handed over in bf16 like the cache rows; this oracle takes their bf16
  values exactly.
* norm = ||x||_2 of the bf16 row, stored as float32.
* MSE code: u = sqrt(d) * (P x) / norm, so that each u_i is close to N(0, 1),
  and idx_i = #{boundaries < u_i} with the N(0, 1) Lloyd-Max table of the
  served codec (searchsorted, left side).  A zero row has u = 0.
  Reconstruction: x_hat = P^T (norm32 * centroid[idx] / sqrt(d)).
* QJL stage (b MSE bits plus one sign bit per coordinate): the residual is
  taken in the rotated domain, rho = P x - norm32 * centroid[idx] / sqrt(d);
  gamma = ||rho||_2 is stored as float32 and the sign bits are
  q_i = [(S rho)_i >= 0].  Reconstruction adds
  sqrt(pi/2) / d * gamma32 * S^T (2q - 1) to the rotated-domain vector before
  P^T.  Projecting rho rather than P^T rho is the same estimator in law: for
  orthogonal P, S P^T has the same iid Gaussian law as S.
* Arithmetic is float64; the matrix products are numpy matmuls.
"""
from __future__ import annotations

import math

import numpy as np

from .codec import bf16_to_f32, pack_bits, unpack_bits
from .tables import codebook

HEAD_DIMS = (64, 128, 256)
MSE_BITS = (1, 2, 3, 4)


def _f64_bf16(bits) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


def check(d: int, bits: int, qjl: bool) -> None:
    if d not in HEAD_DIMS:
        raise ValueError(f"head_dim {d} not in {HEAD_DIMS}")
    if bits not in MSE_BITS:
        raise ValueError(f"bits {bits} not in {MSE_BITS}")
    if qjl and d > 128:
        raise ValueError("the QJL stage is served for head_dim <= 128")


def plane_row_bytes(d: int, bits: int, qjl: bool) -> dict:
    out = {"idx": d * bits // 8, "norm": 4}
    if qjl:
        out.update({"qjl": d // 8, "gamma": 4})
    return out


def quantize(x_bf16, rot_bf16, bits: int, proj_bf16=None) -> dict:
    """Paper-variant quantization of bf16 rows [R, d].

    Returns the stored planes (idx packed, norm float32, and with a projection
    qjl packed and gamma float32) plus the float64 intermediates the parity
    tests use to recognise near-ties: y = P x, u, rho and s = S rho.
    """
    x = _f64_bf16(x_bf16)
    r, d = x.shape
    P = _f64_bf16(rot_bf16)
    cent, bnd = codebook(bits)
    cent = cent.astype(np.float64)
    bnd = bnd.astype(np.float64)
    norm = np.sqrt(np.sum(x * x, axis=1))
    y = x @ P.T
    safe = np.where(norm > 0, norm, 1.0)
    u = np.where(norm[:, None] > 0, math.sqrt(d) * y / safe[:, None], 0.0)
    idx = np.searchsorted(bnd, u, side="left").astype(np.int64)
    norm32 = norm.astype(np.float32)
    out = {"idx": idx, "idx_packed": pack_bits(idx, bits), "norm": norm32, "y": y, "u": u}
    if proj_bf16 is not None:
        S = _f64_bf16(proj_bf16)
        y_hat = norm32.astype(np.float64)[:, None] * cent[idx] / math.sqrt(d)
        rho = y - y_hat
        gamma = np.sqrt(np.sum(rho * rho, axis=1))
        s = rho @ S.T
        q = (s >= 0).astype(np.int64)
        out.update({"qjl": q, "qjl_packed": pack_bits(q, 1), "gamma": gamma.astype(np.float32),
                    "rho": rho, "s": s, "y_hat": y_hat})
    return out


def rotated_reconstruction(idx, norm32, bits: int, d: int, qjl=None, gamma32=None, proj_bf16=None):
    """The rotated-domain vector the decoder rebuilds before P^T."""
    cent, _ = codebook(bits)
    idx = np.asarray(idx)
    y_hat = np.asarray(norm32, np.float32).astype(np.float64)[:, None] * cent.astype(np.float64)[idx] / math.sqrt(d)
    if qjl is not None:
        S = _f64_bf16(proj_bf16)
        signs = 2.0 * np.asarray(qjl, np.float64) - 1.0
        coef = math.sqrt(math.pi / 2.0) / d
        y_hat = y_hat + coef * np.asarray(gamma32, np.float32).astype(np.float64)[:, None] * (signs @ S)
    return y_hat


def dequantize(idx, norm32, rot_bf16, bits: int, qjl=None, gamma32=None, proj_bf16=None) -> np.ndarray:
    """x_hat = P^T y_hat in float64, [R, d]."""
    idx = np.asarray(idx)
    d = idx.shape[1]
    y_hat = rotated_reconstruction(idx, norm32, bits, d, qjl, gamma32, proj_bf16)
    return y_hat @ _f64_bf16(rot_bf16)


def unpack_planes(planes: dict, d: int, bits: int) -> dict:
    """Packed planes -> index arrays (idx, and qjl when present)."""
    out = {"idx": unpack_bits(planes["idx_packed"], bits, d).astype(np.int64)}
    if "qjl_packed" in planes:
        out["qjl"] = unpack_bits(planes["qjl_packed"], 1, d).astype(np.int64)
    return out
