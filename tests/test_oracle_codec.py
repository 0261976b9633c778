"""Pins of the oracle codec against what the pages and the mathematics fix (CPU only).

Sources: the mlx-bun TurboQuant pages, "Algorithm (vllm-metal reference
semantics, exact)" (keys, values, pack, dequant, bytes) and "Gates" item 2
(transform involution/orthogonality, 3-bit round-trip distortion band).
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import codec
from oracle.attention import hadamard_matrix
from oracle.tables import codebook

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def bf16(x):
    return codec.f32_to_bf16(np.asarray(x, np.float32))


# ------------------------------------------------------------ number formats
_F16_FINITE = [Fraction(float(np.uint16(b).view(np.float16))) for b in range(0x7C00)]


def _rne_f16_exact(v: float) -> int:
    """binary16 pattern of a finite double by exact rational nearest-even
    rounding over the list of all finite non-negative halves."""
    sign = 0x8000 if math.copysign(1.0, v) < 0 else 0
    a = Fraction(abs(v))
    # one ulp above 65504 the rounding goes to infinity (halfway at 65520)
    if a >= Fraction(65520):
        return sign | 0x7C00
    import bisect
    i = bisect.bisect_left(_F16_FINITE, a)
    if i < len(_F16_FINITE) and _F16_FINITE[i] == a:
        return sign | i
    if i == len(_F16_FINITE):            # between 65504 and the halfway 65520
        return sign | 0x7BFF
    lo, hi = i - 1, i
    dl, dh = a - _F16_FINITE[lo], _F16_FINITE[hi] - a
    if dl < dh or (dl == dh and lo % 2 == 0):
        return sign | lo
    return sign | hi


@pytest.mark.parametrize("v", [1.0, 65504.0, 65519.996, 65520.0, 1e5, 2.0 ** -24,
                               2.0 ** -25, 3 * 2.0 ** -26, 1.0 + 2.0 ** -11,
                               1.0 + 3 * 2.0 ** -11, 6.1e-5, -0.3333333, 2.0 ** -14 - 2.0 ** -25])
def test_f16_rounding_matches_exact_rationals(v):
    v32 = float(np.float32(v))
    assert int(codec.f32_to_f16(np.float32(v32))) == _rne_f16_exact(v32)


def test_f16_special_values():
    x = np.array([np.inf, -np.inf, np.nan, -np.nan, -0.0], np.float32)
    assert list(codec.f32_to_f16(x)) == [0x7C00, 0xFC00, 0x7E00, 0x7E00, 0x8000]


def test_bf16_round_to_nearest_even():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> up
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, np.nan, -0.0], np.float32)
    assert list(codec.f32_to_bf16(x)) == [0x3F80, 0x3F82, 0x3F81, 0x7FC0, 0x8000]


def test_inverse_sqrt_constants():
    got = {d: int(np.float32(codec.inv_sqrt_d(d)).view(np.uint32)) for d in (64, 128, 256, 512)}
    assert got == {64: 0x3E000000, 128: 0x3DB504F3, 256: 0x3D800000, 512: 0x3D3504F3}


# ----------------------------------------------------------------- bitstream
def test_pack_examples_from_golden():
    n = 0
    for line in open(os.path.join(GOLD, "pack_examples.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        bits, idx, hexes = [p.strip() for p in line.split("|")]
        idx = np.array([[int(x) for x in idx.split()]])
        want = bytes(int(h, 16) for h in hexes.split())
        got = codec.pack_bits(idx, int(bits))
        assert got.tobytes() == want
        assert np.array_equal(codec.unpack_bits(got, int(bits), idx.shape[1]), idx)
        n += 1
    assert n == 6


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 8])
@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_pack_is_the_little_endian_integer(bits, d):
    rng = np.random.default_rng(bits * 1000 + d)
    idx = rng.integers(0, 1 << bits, size=(3, d))
    packed = codec.pack_bits(idx, bits)
    assert packed.shape == (3, d * bits // 8)
    for r in range(3):
        big = sum(int(v) << (bits * j) for j, v in enumerate(idx[r]))
        assert packed[r].tobytes() == big.to_bytes(d * bits // 8, "little")
    assert np.array_equal(codec.unpack_bits(packed, bits, d), idx)


def test_byte_accounting_golden():
    rows = [l for l in open(os.path.join(GOLD, "byte_accounting.txt")) if l.strip() and not l.startswith("#")]
    for line in rows:
        head, planes, tot = [p.split() for p in line.split("|")]
        d, kb, vb = map(int, head)
        got = codec.plane_row_bytes(d, kb, vb)
        assert [got[k] for k in ("k_q", "k_scale", "k_zero", "v_q", "v_scale")] == list(map(int, planes))
        assert codec.bytes_per_row(d, kb, vb) == int(tot[0])
        assert 4 * d == int(tot[1])
        assert 4 * d / codec.bytes_per_row(d, kb, vb) == pytest.approx(2.56)


def test_other_configs_row_bytes():
    assert codec.bytes_per_row(256, 4, 4) == 304
    assert codec.bytes_per_row(512, 5, 2) == 544


def test_scheme_validation():
    codec.check_scheme(128, 8, 3)
    for bad in [(96, 8, 3), (128, 3, 3), (128, 8, 1), (128, 8, 6), (128, 8, 7)]:
        with pytest.raises(ValueError):
            codec.check_scheme(*bad)


# ---------------------------------------------------------------------- keys
def _grid_group(bits, rng, s_exp, z):
    lo, hi = codec.key_range(bits)
    idx = rng.integers(lo, hi + 1, size=32)
    idx[0], idx[1] = lo, hi          # both clip ends present
    return idx, (idx + z) * 2.0 ** s_exp


@pytest.mark.parametrize("bits", [8, 2, 4, 5])
def test_keys_exact_grid_round_trip(bits):
    rng = np.random.default_rng(7 + bits)
    rows, idx_all = [], []
    for r in range(16):
        groups = []
        for g in range(4):
            z = int(rng.integers(-100, 100)) if bits == 8 else int(rng.integers(-200, 40))
            idx, x = _grid_group(bits, rng, int(rng.integers(-12, 4)), z)
            groups.append(x)
            idx_all.append(idx)
        rows.append(np.concatenate(groups))
    x = np.array(rows, np.float64)
    assert np.array_equal(bf16(x).astype(np.uint32) << 16, np.float32(x).view(np.uint32))  # exact in bf16
    q = codec.quantize_keys(bf16(x), bits)
    assert np.array_equal(q["idx"], np.array(idx_all).reshape(16, 128))
    k = codec.dequantize_keys_f32(q["idx"], q["scale16"], q["zero16"])
    assert np.array_equal(k, x.astype(np.float32))


@pytest.mark.parametrize("bits", [8, 2, 4, 5])
def test_keys_nearest_grid_point_and_range(bits):
    rng = np.random.default_rng(bits)
    x = rng.standard_normal((64, 128)).astype(np.float32) * rng.uniform(0.1, 10, (64, 1)).astype(np.float32)
    xb = bf16(x)
    q = codec.quantize_keys(xb, bits)
    lo, hi = codec.key_range(bits)
    assert q["idx"].min() >= lo and q["idx"].max() <= hi
    xf = codec.bf16_to_f32(xb).astype(np.float64).reshape(64, 4, 32)
    s = codec.f16_to_f32(q["scale16"]).astype(np.float64)[..., None]
    z = codec.f16_to_f32(q["zero16"]).astype(np.float64)[..., None]
    recon = (q["idx"].reshape(64, 4, 32) + z) * s
    # every element is within half a step (plus fp16 scale rounding) of its code
    err = np.abs(recon - xf) / s
    assert err.max() <= 0.5 + 2e-3 * (abs(lo) + hi + np.abs(z).max())
    # both extremes of each group reach the clip ends (asymmetric affine)
    g = q["idx"].reshape(64, 4, 32)
    assert np.all(g.max(-1) - g.min(-1) >= hi - lo - 1)


def test_constant_block_zero_point_overflows():
    x = np.zeros((1, 64), np.float32)
    x[0, :32] = 1.5
    x[0, 32:] = 0.0
    q = codec.quantize_keys(bf16(x), 8)
    assert list(q["scale16"][0]) == [0, 0]
    assert q["zero16"][0, 0] == 0x7C00          # +Inf
    assert q["zero16"][0, 1] == 0x7E00          # 0/0 -> NaN
    assert np.all(q["idx"] == -127)
    k = codec.dequantize_keys_f32(q["idx"], q["scale16"], q["zero16"])
    assert np.all(np.isnan(k))
    qn = codec.quantize_keys(bf16(-x), 4)        # unsigned: zero = round(min / 0)
    assert qn["zero16"][0, 0] == 0xFC00 and qn["zero16"][0, 1] == 0x7E00
    assert np.all(qn["idx"] == 0)


def test_signed_zero_and_nan_groups():
    x = np.zeros((1, 64), np.float32)
    x[0, 1] = -0.0
    x[0, 40] = np.nan
    q = codec.quantize_keys(bf16(x), 8)
    assert q["scale16"][0, 0] == 0x0000         # +0 - (-0) = +0
    assert q["scale16"][0, 1] == 0x7E00 and q["zero16"][0, 1] == 0x7E00
    assert np.all(q["idx"][0, 32:] == -127)


# -------------------------------------------------------------------- values
@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_fwht_is_the_hadamard_matrix(d):
    rng = np.random.default_rng(d)
    u = rng.standard_normal((8, d)).astype(np.float32)
    got = codec.fwht(u).astype(np.float64)
    want = u.astype(np.float64) @ hadamard_matrix(d).T
    bound = np.abs(u).astype(np.float64) @ np.ones((d, 1)) * math.log2(d) * 2.0 ** -23
    assert np.all(np.abs(got - want) <= bound)


@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_rotation_involution_and_orthogonality(d):
    rng = np.random.default_rng(d + 1)
    s = np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)
    x = rng.standard_normal((32, d)).astype(np.float32)
    y = codec.rotate(x, s)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-5)
    back = codec.unrotate(y, s)
    assert np.max(np.abs(back - x)) <= 2e-6 * math.log2(d) * np.max(np.abs(x))


def test_rotation_of_a_signed_basis_vector_is_flat():
    d = 128
    s = np.where(np.arange(d) % 3 == 0, -1, 1).astype(np.int8)
    x = np.zeros((1, d), np.float32)
    x[0, 0] = 2.0 * s[0]
    y = codec.rotate(x, s)
    assert np.all(y == np.float32(2.0) * codec.inv_sqrt_d(d))
    q = codec.quantize_values(bf16(x), s, 3)
    rms = np.float32(2.0) * codec.inv_sqrt_d(d)
    assert np.all(q["scale16"] == codec.f32_to_f16(rms))
    # y_n ~ 1 lies between boundaries 0.50055 and 1.04996 -> index 5 of 0..7
    assert np.all(q["idx"] == 5)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 8])
def test_value_index_is_nearest_centroid(bits):
    rng = np.random.default_rng(bits + 50)
    s = np.where(rng.random(128) < 0.5, -1, 1).astype(np.int8)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    q = codec.quantize_values(bf16(x), s, bits)
    cent, bnd = codebook(bits)
    yn = q["yn"].astype(np.float64)
    brute = np.argmin(np.abs(yn[..., None] - cent.astype(np.float64)), axis=-1)
    tie = np.min(np.abs(yn[..., None] - bnd.astype(np.float64)), axis=-1) < 1e-6
    assert np.array_equal(q["idx"][~tie], brute[~tie])
    counted = (bnd[None, None, :] < q["yn"][..., None]).sum(-1)
    assert np.array_equal(q["idx"], counted)


def test_value_scale_is_group_rms():
    rng = np.random.default_rng(3)
    s = np.ones(128, np.int8)
    x = rng.standard_normal((16, 128)).astype(np.float32)
    q = codec.quantize_values(bf16(x), s, 3)
    y = codec.rotate(codec.bf16_to_f32(bf16(x)), s).astype(np.float64).reshape(16, 4, 32)
    rms = np.sqrt(np.mean(y * y, axis=-1))
    assert np.allclose(codec.f16_to_f32(q["scale16"]), rms, rtol=1e-3)


def _round_trip_rel_mse(bits, rows=4000, d=128, seed=11):
    rng = np.random.default_rng(seed)
    s = np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)
    x = rng.standard_normal((rows, d)).astype(np.float32)
    xb = bf16(x)
    xf = codec.bf16_to_f32(xb).astype(np.float64)
    q = codec.quantize_values(xb, s, bits)
    v = codec.dequantize_values_f32(q["idx"], q["scale16"], s, bits).astype(np.float64)
    return np.sum((v - xf) ** 2) / np.sum(xf ** 2)


@pytest.mark.parametrize("bits,band", [(1, (0.33, 0.39)), (2, (0.10, 0.13)), (3, (0.028, 0.038))])
def test_round_trip_distortion_anchors(bits, band):
    mse = _round_trip_rel_mse(bits)
    assert band[0] <= mse <= band[1]


def test_high_width_round_trip_is_near_lossless():
    # 8-bit Lloyd-Max distortion is ~4.1e-5; a wrong inverse (signs before
    # the transform, a missing normalisation) is O(1)
    assert _round_trip_rel_mse(8, rows=500) < 1e-4


def test_nan_value_row():
    s = np.ones(64, np.int8)
    x = np.ones((1, 64), np.float32)
    x[0, 5] = np.nan
    q = codec.quantize_values(bf16(x), s, 3)
    assert np.all(q["idx"] == 0) and np.all(q["scale16"] == 0x7E00)


# ------------------------------------------------------------------ whole row
def test_quantize_kv_planes_and_round_trip():
    rng = np.random.default_rng(5)
    s = np.where(rng.random(128) < 0.5, -1, 1).astype(np.int8)
    k = bf16(rng.standard_normal((10, 128)))
    v = bf16(rng.standard_normal((10, 128)))
    p = codec.quantize_kv(k, v, s, 8, 3)
    assert p["k_q"].shape == (10, 128) and p["v_q"].shape == (10, 48)
    assert p["k_scale"].shape == (10, 4) and p["v_scale"].shape == (10, 4)
    kb, vb = codec.dequantize_kv(p, s, 128, 8, 3)
    kf, vf = codec.bf16_to_f32(k), codec.bf16_to_f32(v)
    assert np.max(np.abs(codec.bf16_to_f32(kb) - kf)) < 0.05
    rel = np.sum((codec.bf16_to_f32(vb) - vf) ** 2) / np.sum(vf ** 2)
    assert rel < 0.04
