"""Comparators between the HIP library's outputs and the oracle's (test helpers).

Acceptance (readings of the stated bar):
* fp16 scale / zero planes: bit-exact.
* Indices and packed bytes: bit-exact, except an index may differ by one
  where the oracle's normalised value lies within 1e-6 of a decision point
  (a value boundary, or a key half-integer evaluated in float64); such
  differences are counted and returned, not failed.
* bf16 dequant outputs: bit-exact expected; any element that is not must
  satisfy |gpu - ref32| <= 1e-3 * max(1, |ref32|) + ulp_bf16(ref32).
"""
from __future__ import annotations

import numpy as np

from oracle import codec
from oracle.tables import codebook

TIE = 1e-6


def _u16(t):
    return np.ascontiguousarray(t).view(np.uint16)


def compare_planes(gpu: dict, ref: dict, d: int, kb: int, vb: int) -> dict:
    """gpu: numpy planes [R, bytes] (uint8 / float16); ref: codec.quantize_kv output."""
    out = {}
    for name in ("k_scale", "k_zero", "v_scale"):
        g, r = _u16(gpu[name]).reshape(-1), _u16(ref[name]).reshape(-1)
        bad = np.nonzero(g != r)[0]
        assert bad.size == 0, f"{name}: {bad.size} fp16 mismatches, first at {bad[:5]} gpu={g[bad[:5]]} ref={r[bad[:5]]}"
    # keys
    gk = codec.key_indices(np.asarray(gpu["k_q"]).reshape(-1, codec.plane_row_bytes(d, kb, vb)["k_q"]), kb, d)
    rk = ref["k_idx"]
    diff = gk != rk
    if diff.any():
        t = ref["k_t64"][diff]
        near = np.abs(t - (np.floor(t) + 0.5)) < TIE
        one = np.abs(gk[diff] - rk[diff]) == 1
        assert np.all(near & one), (f"key index mismatches not at ties: {np.sum(~(near & one))} "
                                    f"of {diff.sum()}; t={t[~(near & one)][:5]}")
    out["key_ties"] = int(diff.sum())
    # values
    gv = codec.unpack_bits(np.asarray(gpu["v_q"]).reshape(-1, d * vb // 8), vb, d).astype(np.int32)
    rv = ref["v_idx"]
    diff = gv != rv
    if diff.any():
        _, bnd = codebook(vb)
        yn = ref["v_yn"][diff].astype(np.float64)
        near = np.min(np.abs(yn[:, None] - bnd[None, :].astype(np.float64)), axis=1) < TIE
        one = np.abs(gv[diff] - rv[diff]) == 1
        assert np.all(near & one), (f"value index mismatches not at ties: {np.sum(~(near & one))} "
                                    f"of {diff.sum()}; yn={yn[~(near & one)][:5]}")
    out["value_ties"] = int(diff.sum())
    # where the indices agree, the packed bytes must agree too
    if out["key_ties"] == 0:
        assert np.array_equal(np.asarray(gpu["k_q"]).reshape(-1), np.asarray(ref["k_q"]).reshape(-1))
    if out["value_ties"] == 0:
        assert np.array_equal(np.asarray(gpu["v_q"]).reshape(-1), np.asarray(ref["v_q"]).reshape(-1))
    return out


def bf16_ulp(x):
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -133)))
    return 2.0 ** (np.maximum(e, -133) - 7)


def compare_bf16(gpu_bits: np.ndarray, ref32: np.ndarray, what: str) -> int:
    """Returns the number of non-bit-exact elements (asserting the tolerance)."""
    g = _u16(gpu_bits).reshape(-1)
    r = codec.f32_to_bf16(np.asarray(ref32, np.float32)).reshape(-1)
    bad = np.nonzero(g != r)[0]
    if bad.size:
        gv = codec.bf16_to_f32(g[bad]).astype(np.float64)
        rv = np.asarray(ref32, np.float32).reshape(-1)[bad].astype(np.float64)
        both_nan = np.isnan(gv) & np.isnan(rv)
        tol = 1e-3 * np.maximum(1.0, np.abs(rv)) + bf16_ulp(rv)
        ok = both_nan | (np.abs(gv - rv) <= tol)
        assert np.all(ok), f"{what}: {np.sum(~ok)} elements beyond tolerance, first gpu={gv[~ok][:4]} ref={rv[~ok][:4]}"
    return int(bad.size)


def attention_close(gpu_bits: np.ndarray, ref64: np.ndarray) -> dict:
    """Per element |o - ref| <= 2e-3 * max_j |ref_row| + ulp_bf16(ref)."""
    g = codec.bf16_to_f32(_u16(gpu_bits)).astype(np.float64).reshape(ref64.shape)
    rowmax = np.max(np.abs(ref64), axis=-1, keepdims=True)
    tol = 2e-3 * rowmax + bf16_ulp(ref64)
    err = np.abs(g - ref64)
    assert np.all(err <= tol), f"attention: {np.sum(err > tol)} elements beyond tolerance; worst {np.max(err - tol)}"
    num = np.linalg.norm(g - ref64, axis=-1)
    den = np.maximum(np.linalg.norm(ref64, axis=-1), 1e-30)
    return {"max_rel_l2": float(np.max(num / den)), "max_abs_err": float(np.max(err))}
