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

# Parity record kept for the run's summary: per configuration, the counted
# boundary-tie index differences (keys, values), the dequantized elements that
# were not bit-exact, and the rows checked.  tests/conftest.py prints it.
RECORD: dict = {}


def record(config: str, **counts) -> None:
    r = RECORD.setdefault(config, {})
    for k, v in counts.items():
        if isinstance(v, float):
            r[k] = max(r.get(k, 0.0), v)
        else:
            r[k] = r.get(k, 0) + int(v)


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


def compare_bf16(gpu_bits: np.ndarray, ref32: np.ndarray, what: str, kinds: dict | None = None) -> int:
    """Returns the number of elements that are not bit-exact (asserting the
    tolerance).  With `kinds`, adds to kinds["zero_sign"] the elements that
    differ only in the sign of an exact zero, and to kinds["value"] the
    others."""
    g = _u16(gpu_bits).reshape(-1)
    r = codec.f32_to_bf16(np.asarray(ref32, np.float32)).reshape(-1)
    bad = np.nonzero(g != r)[0]
    if kinds is not None:
        zs = int(np.sum(((g[bad] & 0x7FFF) == 0) & ((r[bad] & 0x7FFF) == 0)))
        kinds["zero_sign"] = kinds.get("zero_sign", 0) + zs
        kinds["value"] = kinds.get("value", 0) + int(bad.size) - zs
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
    den = np.maximum(np.linalg.norm(ref64, axis=-1), 1e-30)
    # the output is bf16: rounding the exact result to bf16 alone leaves a
    # relative L2 error, the floor any bf16 output has
    rb = codec.bf16_to_f32(codec.f32_to_bf16(ref64.astype(np.float32))).astype(np.float64).reshape(ref64.shape)
    return {"max_rel_l2": float(np.max(np.linalg.norm(g - ref64, axis=-1) / den)),
            "max_rel_l2_bf16_floor": float(np.max(np.linalg.norm(rb - ref64, axis=-1) / den)),
            "max_abs_err": float(np.max(err))}


# ------------------------------------------------------------ paper variant
# The paper variant's products are float32 sums of exact bf16 products, so the
# GPU and the float64 oracle may take a different side of a decision point
# only within the sum's rounding bound.  Per element the bound is built from
# the oracle's own float64 terms: gamma_n * sum |terms| for an n-term float32
# sum (gamma_n = n * 2^-23, the rounding of an MFMA accumulation step taken as
# a full ulp), plus 2^-17 of every operand split into bf16 hi + lo.
U = 2.0 ** -24


def _gamma(n):
    return n * 2.0 ** -23


def compare_dense_planes(gpu: dict, ref: dict, x_bits, rot_bits, proj_bits, d: int, bits: int) -> dict:
    """gpu: numpy planes {idx [R, d*bits/8] u8, norm [R] f32, qjl, gamma}; ref: dense.quantize output."""
    from oracle import dense
    x = codec.bf16_to_f32(x_bits).astype(np.float64)
    P = codec.bf16_to_f32(rot_bits).astype(np.float64)
    n_ref = np.sqrt(np.sum(x * x, axis=1))
    n_gpu = np.asarray(gpu["norm"], np.float64).reshape(-1)
    tol_n = (d + 8) * U * n_ref
    assert np.all(np.abs(n_gpu - n_ref) <= tol_n), f"norm: max err {np.max(np.abs(n_gpu - n_ref) - tol_n)} over bound"
    # index decisions: u = sqrt(d) y / norm against the boundaries
    ey = _gamma(d) * (np.abs(x) @ np.abs(P).T)                       # |y_gpu - y| bound
    safe = np.where(n_ref > 0, n_ref, 1.0)[:, None]
    eps_u = np.sqrt(d) * ey / safe + np.abs(ref["u"]) * (d + 16) * U
    gi = codec.unpack_bits(np.asarray(gpu["idx"]).reshape(len(x), -1), bits, d).astype(np.int64)
    ri = ref["idx"]
    diff = gi != ri
    out = {"index_ties": int(diff.sum())}
    if diff.any():
        _, bnd = codebook(bits)
        k = np.minimum(gi[diff], ri[diff])
        one = np.abs(gi[diff] - ri[diff]) == 1
        near = np.abs(ref["u"][diff] - bnd.astype(np.float64)[np.clip(k, 0, len(bnd) - 1)]) <= eps_u[diff]
        assert np.all(one & near), (f"index mismatches outside the rounding band: {np.sum(~(one & near))} of "
                                    f"{diff.sum()}; u={ref['u'][diff][~(one & near)][:5]}")
    if "qjl" not in ref:
        if not diff.any():
            assert np.array_equal(np.asarray(gpu["idx"]).reshape(len(x), -1), ref["idx_packed"])
        return out
    S = codec.bf16_to_f32(proj_bits).astype(np.float64)
    rows_ok = ~diff.any(axis=1)
    # residual: y error, the norm's error through y_hat, one rounding of the fma
    cent, _ = codebook(bits)
    c = cent.astype(np.float64)[ri]
    drho = ey + np.abs(c) / np.sqrt(d) * (tol_n[:, None] + (d + 16) * U * n_ref[:, None]) + U * np.abs(ref["rho"])
    eps_s = (np.abs(drho) @ np.abs(S).T + (2.0 ** -17 + _gamma(2 * d)) * (np.abs(ref["rho"]) @ np.abs(S).T))
    gq = codec.unpack_bits(np.asarray(gpu["qjl"]).reshape(len(x), -1), 1, d).astype(np.int64)
    qd = (gq != ref["qjl"]) & rows_ok[:, None]
    if qd.any():
        near = np.abs(ref["s"][qd]) <= eps_s[qd]
        assert np.all(near), (f"QJL sign mismatches outside the rounding band: {np.sum(~near)} of {qd.sum()}; "
                              f"s={ref['s'][qd][~near][:5]} eps={eps_s[qd][~near][:5]}")
    out["sign_ties"] = int(qd.sum())
    out["rows_with_index_ties"] = int((~rows_ok).sum())
    g_gpu = np.asarray(gpu["gamma"], np.float64).reshape(-1)
    g_ref = np.sqrt(np.sum(ref["rho"] ** 2, axis=1))
    tol_g = np.sqrt(np.sum(drho ** 2, axis=1)) + (d + 8) * U * g_ref
    okg = np.abs(g_gpu - g_ref) <= tol_g
    assert np.all(okg[rows_ok]), f"gamma outside bound: {np.sum(~okg[rows_ok])} rows"
    # a tie moves the residual by at most one centroid gap: gamma stays finite and close
    if (~rows_ok).any():
        gap = np.max(np.diff(cent.astype(np.float64))) * n_ref[~rows_ok] / np.sqrt(d)
        assert np.all(np.abs(g_gpu[~rows_ok] - g_ref[~rows_ok]) <= gap * np.sqrt(d) + tol_g[~rows_ok])
    return out


def compare_dense_dequant(gpu_bits, planes: dict, rot_bits, proj_bits, d: int, bits: int) -> dict:
    """GPU bf16 reconstruction of the oracle's planes against the float64 oracle, element-wise:
    |gpu - ref| <= eps + ulp_bf16(|ref| + eps) / 2, eps the float32 bound of the two products."""
    from oracle import dense
    qjl = planes.get("qjl")
    gamma = planes.get("gamma")
    y_hat = dense.rotated_reconstruction(planes["idx"], planes["norm"], bits, d, qjl, gamma, proj_bits)
    P = codec.bf16_to_f32(rot_bits).astype(np.float64)
    ref = y_hat @ P
    # float32 errors of the rotated-domain vector the kernel builds: the scale
    # norm / sqrt(d) and its product (4 ulp), and with QJL the float32 sum
    # S^T q (exact +-S terms) scaled by sqrt(pi/2)/d * gamma (3 ulp)
    mse = dense.rotated_reconstruction(planes["idx"], planes["norm"], bits, d)
    dy = 4 * U * (np.abs(mse) + np.abs(y_hat))
    if qjl is not None:
        S = codec.bf16_to_f32(proj_bits).astype(np.float64)
        coef = np.sqrt(np.pi / 2) / d * np.asarray(gamma, np.float64)[:, None]
        dy = dy + coef * (_gamma(d) + 3 * U) * np.sum(np.abs(S), axis=0)[None, :]
    eps = (dy + (2.0 ** -17 + _gamma(2 * d) + 2 * U) * np.abs(y_hat)) @ np.abs(P)
    g = codec.bf16_to_f32(_u16(gpu_bits).reshape(ref.shape)).astype(np.float64)
    tol = eps + 0.5 * bf16_ulp(np.abs(ref) + eps)
    bad = np.abs(g - ref) > tol
    assert not bad.any(), (f"dequant outside bound: {bad.sum()} elements; gpu={g[bad][:5]} ref={ref[bad][:5]} "
                           f"tol={tol[bad][:5]}")
    exact = codec.f32_to_bf16(ref.astype(np.float32)) == _u16(gpu_bits).reshape(ref.shape)
    return {"not_bit_exact": int((~exact).sum()), "max_err_over_tol": float(np.max(np.abs(g - ref) / tol))}
