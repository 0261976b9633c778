"""Plain CPU oracle of the TurboQuant-style KV-cache codec (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
module; the library never imports or calls it.

Sources (the mlx-bun TurboQuant design pages):

* "Algorithm (vllm-metal reference semantics, exact)" on the TurboQuant page,
  and "Algorithm" on the TurboQuant KV design page: per token and kv-head,
  groups of 32 along head_dim; asymmetric affine keys; sign-flipped,
  1/sqrt(d)-normalised Walsh-Hadamard-rotated values with a per-group RMS
  scale and a Lloyd-Max index; a little-endian bitstream; fp16 scales.
* The same sections' byte accounting: k8v3 at d=128 is 200 bytes per
  token-head.

The pages fix fp32 for the key affine arithmetic with only scale and zero
cast to fp16 at the end; this oracle uses the same policy for values.  Every
operation below is one IEEE float32 operation, round-to-nearest-even, on
numpy float32 arrays (vectorised over rows only; the per-element order of
operations is the one written here).  Readings where the pages are silent:

* round = half-to-even;  clip maps NaN to the low end of the range;
* key min/max are IEEE 754-2019 minimum/maximum: NaN propagates and
  -0 < +0;
* the transform runs the Sylvester butterfly with h = 1, 2, 4, ..., d/2 and
  one final multiply by float32(1/sqrt(d));
* the group mean square sums adjacent pairs, then adjacent pair sums, and so
  on (a fixed binary tree), then multiplies by 1/32;
* the value index is the count of boundaries strictly below the normalised
  value (searchsorted, left side); NaN gives index 0;
* the inverse applies the transform first and the signs last;
* fp16 conversion is round-to-nearest-even with subnormals, overflow gives
  +-Inf and every NaN is stored as 0x7E00; bf16 outputs round to nearest
  even and every NaN is stored as 0x7FC0.
"""
from __future__ import annotations

import numpy as np

from .tables import codebook as fp32_table

GROUP = 32
HEAD_DIMS = (64, 128, 256, 512)
KEY_BITS = (2, 4, 5, 8)
VALUE_BITS = (2, 3, 4, 5, 8)

F32 = np.float32


# ----------------------------------------------------------------- formats
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 patterns, round to nearest even; NaN -> 0x7FC0."""
    x = np.asarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) & 0xFFFF
    r = r.astype(np.uint16)
    r[np.isnan(x)] = 0x7FC0
    return r


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    """float32 -> binary16 patterns, round to nearest even; NaN -> 0x7E00."""
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        h = x.astype(np.float16).view(np.uint16).copy()
    h[np.isnan(x)] = 0x7E00
    return h


def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    """binary16 patterns -> float32 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def inv_sqrt_d(d: int) -> np.float32:
    """float32(1/sqrt(d)), the transform's normalisation."""
    return F32(1.0 / np.sqrt(np.float64(d)))


# ------------------------------------------------------------- row layout
def plane_row_bytes(d: int, k_bits: int, v_bits: int) -> dict:
    """Bytes per (token, kv-head) row in each of the five planes."""
    g = d // GROUP
    return {"k_q": d * k_bits // 8, "k_scale": 2 * g, "k_zero": 2 * g,
            "v_q": d * v_bits // 8, "v_scale": 2 * g}


def bytes_per_row(d: int, k_bits: int, v_bits: int) -> int:
    return sum(plane_row_bytes(d, k_bits, v_bits).values())


def check_scheme(d: int, k_bits: int, v_bits: int) -> None:
    if d not in HEAD_DIMS:
        raise ValueError(f"head_dim {d} not in {HEAD_DIMS}")
    if k_bits not in KEY_BITS:
        raise ValueError(f"k_bits {k_bits} not in {KEY_BITS}")
    if v_bits not in VALUE_BITS:
        raise ValueError(f"v_bits {v_bits} not in {VALUE_BITS}")


# --------------------------------------------------------------- bitstream
def pack_bits(idx: np.ndarray, bits: int) -> np.ndarray:
    """Little-endian bitstream per row: element j occupies stream bits
    [j*bits, j*bits + bits), index LSB first; stream bit n is bit n%8 of
    byte n//8.  idx: [R, d] non-negative ints < 2**bits -> uint8 [R, d*bits/8]."""
    idx = np.asarray(idx, dtype=np.uint32)
    r, d = idx.shape
    planes = (idx[:, :, None] >> np.arange(bits, dtype=np.uint32)) & 1
    stream = planes.reshape(r, d * bits).astype(np.uint8)
    return np.packbits(stream, axis=1, bitorder="little")


def unpack_bits(packed: np.ndarray, bits: int, d: int) -> np.ndarray:
    """Inverse of pack_bits: uint8 [R, d*bits/8] -> uint32 [R, d]."""
    packed = np.asarray(packed, dtype=np.uint8)
    r = packed.shape[0]
    stream = np.unpackbits(packed, axis=1, bitorder="little")[:, : d * bits]
    planes = stream.reshape(r, d, bits).astype(np.uint32)
    return (planes << np.arange(bits, dtype=np.uint32)).sum(axis=2, dtype=np.uint32)


# -------------------------------------------------------------------- keys
def _group_minimum(g: np.ndarray) -> np.ndarray:
    """IEEE minimum over the last axis: NaN propagates, -0 < +0."""
    with np.errstate(invalid="ignore"):
        m = np.min(g, axis=-1)
    zero = m == 0
    neg_zero_present = np.any((g == 0) & np.signbit(g), axis=-1)
    m = np.where(zero, np.where(neg_zero_present, F32(-0.0), F32(0.0)), m)
    return m.astype(np.float32)


def _group_maximum(g: np.ndarray) -> np.ndarray:
    """IEEE maximum over the last axis: NaN propagates, -0 < +0."""
    with np.errstate(invalid="ignore"):
        m = np.max(g, axis=-1)
    zero = m == 0
    pos_zero_present = np.any((g == 0) & ~np.signbit(g), axis=-1)
    m = np.where(zero, np.where(pos_zero_present, F32(0.0), F32(-0.0)), m)
    return m.astype(np.float32)


def key_range(bits: int):
    """Clip range of the key index: signed -127..127 at 8 bits, else 0..2^b-1."""
    return (-127, 127) if bits == 8 else (0, (1 << bits) - 1)


def quantize_keys(k_bf16: np.ndarray, bits: int) -> dict:
    """Per-32-group asymmetric affine key quantizer.

    signed (bits = 8):   scale = (max - min) / 254
                         zero  = round((max + min) / (2 * scale))
    unsigned (2, 4, 5):  scale = (max - min) / (2^bits - 1)
                         zero  = round(min / scale)
    both:                idx   = clip(round(x / scale - zero), lo, hi)
    Returns idx [R, d] (int32), scale16 / zero16 [R, d/32] (fp16 patterns),
    and the float64 normalised value t = x/scale - zero (for tie detection).
    """
    x = bf16_to_f32(k_bf16)
    r, d = x.shape
    g = x.reshape(r, d // GROUP, GROUP)
    mn = _group_minimum(g)
    mx = _group_maximum(g)
    lo, hi = key_range(bits)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        if bits == 8:
            scale = (mx - mn) / F32(254.0)
            zero = np.rint((mx + mn) / (F32(2.0) * scale))
        else:
            scale = (mx - mn) / F32((1 << bits) - 1)
            zero = np.rint(mn / scale)
        t = (g / scale[..., None]) - zero[..., None]
        q = np.rint(t)
        q = np.where(np.isnan(q), F32(lo), np.clip(q, F32(lo), F32(hi)))
        t64 = g.astype(np.float64) / scale[..., None].astype(np.float64) \
            - zero[..., None].astype(np.float64)
    return {"idx": q.reshape(r, d).astype(np.int32),
            "scale16": f32_to_f16(scale),
            "zero16": f32_to_f16(zero),
            "t64": t64.reshape(r, d)}


def dequantize_keys_f32(idx: np.ndarray, scale16: np.ndarray, zero16: np.ndarray) -> np.ndarray:
    """k_hat = (float(idx) + float(zero16)) * float(scale16), in float32."""
    idx = np.asarray(idx)
    r, d = idx.shape
    q = idx.astype(np.float32).reshape(r, d // GROUP, GROUP)
    z = f16_to_f32(zero16)[..., None]
    s = f16_to_f32(scale16)[..., None]
    with np.errstate(invalid="ignore", over="ignore"):
        out = (q + z) * s
    return out.reshape(r, d)


# ------------------------------------------------------------------ values
def fwht(u: np.ndarray) -> np.ndarray:
    """Unnormalised Sylvester Walsh-Hadamard butterfly on float32 rows.

    Stage h (h = 1, 2, 4, ..., d/2): for every i with (i & h) == 0,
    (u_i, u_{i+h}) <- (u_i + u_{i+h}, u_i - u_{i+h}).
    """
    u = np.asarray(u, dtype=np.float32)
    r, d = u.shape
    h = 1
    with np.errstate(invalid="ignore", over="ignore"):
        while h < d:
            v = u.reshape(r, d // (2 * h), 2, h)
            a = v[:, :, 0, :]
            b = v[:, :, 1, :]
            u = np.stack((a + b, a - b), axis=2).reshape(r, d)
            h *= 2
    return u


def rotate(v: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """y = FWHT(v * signs) * float32(1/sqrt(d))."""
    v = np.asarray(v, dtype=np.float32)
    s = np.asarray(signs).astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        return fwht(v * s[None, :]) * inv_sqrt_d(v.shape[1])


def unrotate(z: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """Inverse rotation: FWHT first, then * float32(1/sqrt(d)), then * signs."""
    z = np.asarray(z, dtype=np.float32)
    s = np.asarray(signs).astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        return (fwht(z) * inv_sqrt_d(z.shape[1])) * s[None, :]


def group_rms(y: np.ndarray) -> np.ndarray:
    """sqrt(mean(y^2)) per 32-group with the fixed adjacent-pair tree."""
    r, d = y.shape
    with np.errstate(invalid="ignore", over="ignore"):
        e = (y * y).reshape(r, d // GROUP, GROUP)
        while e.shape[-1] > 1:
            e = e[..., 0::2] + e[..., 1::2]
        mean = e[..., 0] * F32(1.0 / GROUP)
        return np.sqrt(mean)


def quantize_values(v_bf16: np.ndarray, signs: np.ndarray, bits: int) -> dict:
    """Sign flip + normalised FWHT + per-group RMS + Lloyd-Max index.

    y = FWHT(v * signs) / sqrt(d);  scale = sqrt(mean(y^2)) per group;
    y_n = y / (scale + 1e-8);  idx = #{boundaries < y_n}.
    Returns idx [R, d] (int32), scale16 [R, d/32], and y_n (float32, for
    tie detection).
    """
    _, bnd = fp32_table(bits)
    x = bf16_to_f32(v_bf16)
    r, d = x.shape
    y = rotate(x, signs)
    scale = group_rms(y)
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        den = scale + F32(1e-8)
        yn = (y.reshape(r, d // GROUP, GROUP) / den[..., None]).reshape(r, d)
    idx = np.searchsorted(bnd, yn, side="left").astype(np.int32)
    idx[np.isnan(yn)] = 0
    return {"idx": idx, "scale16": f32_to_f16(scale), "yn": yn}


def dequantize_values_rotated_f32(idx: np.ndarray, scale16: np.ndarray, bits: int) -> np.ndarray:
    """Rotated-domain value reconstruction z = centroid[idx] * float(scale16)."""
    cent, _ = fp32_table(bits)
    idx = np.asarray(idx)
    r, d = idx.shape
    c = cent[idx].reshape(r, d // GROUP, GROUP)
    with np.errstate(invalid="ignore", over="ignore"):
        z = c * f16_to_f32(scale16)[..., None]
    return z.reshape(r, d)


def dequantize_values_f32(idx, scale16, signs, bits) -> np.ndarray:
    """Eager value dequant: signs * FWHT(centroid[idx] * scale) / sqrt(d)."""
    return unrotate(dequantize_values_rotated_f32(idx, scale16, bits), signs)


# --------------------------------------------------------- whole-row codec
def quantize_kv(k_bf16: np.ndarray, v_bf16: np.ndarray, signs: np.ndarray,
                k_bits: int, v_bits: int) -> dict:
    """Quantize [R, d] bf16 K and V rows into the five byte planes.

    k_q: int8 bytes at 8 bits, else the packed unsigned bitstream;
    k_scale, k_zero, v_scale: fp16 patterns [R, d/32]; v_q: packed stream.
    Also returns the unpacked indices and the tie-detection values.
    """
    k_bf16 = np.asarray(k_bf16, dtype=np.uint16)
    v_bf16 = np.asarray(v_bf16, dtype=np.uint16)
    d = k_bf16.shape[1]
    check_scheme(d, k_bits, v_bits)
    kq = quantize_keys(k_bf16, k_bits)
    vq = quantize_values(v_bf16, signs, v_bits)
    if k_bits == 8:
        k_plane = kq["idx"].astype(np.int8).view(np.uint8)
    else:
        k_plane = pack_bits(kq["idx"], k_bits)
    return {"k_q": k_plane, "k_scale": kq["scale16"], "k_zero": kq["zero16"],
            "v_q": pack_bits(vq["idx"], v_bits), "v_scale": vq["scale16"],
            "k_idx": kq["idx"], "v_idx": vq["idx"], "k_t64": kq["t64"], "v_yn": vq["yn"]}


def key_indices(k_plane: np.ndarray, k_bits: int, d: int) -> np.ndarray:
    """Key indices from a key plane (int8 bytes or packed stream)."""
    k_plane = np.asarray(k_plane, dtype=np.uint8)
    if k_bits == 8:
        return k_plane.view(np.int8).astype(np.int32).reshape(-1, d)
    return unpack_bits(k_plane, k_bits, d).astype(np.int32)


def dequantize_kv_f32(planes: dict, signs: np.ndarray, d: int, k_bits: int, v_bits: int):
    """float32 (K_hat, V_hat) rows from the five planes (before bf16 rounding)."""
    kidx = key_indices(planes["k_q"], k_bits, d)
    vidx = unpack_bits(planes["v_q"], v_bits, d).astype(np.int32)
    k = dequantize_keys_f32(kidx, planes["k_scale"], planes["k_zero"])
    v = dequantize_values_f32(vidx, planes["v_scale"], signs, v_bits)
    return k, v


def dequantize_kv(planes: dict, signs: np.ndarray, d: int, k_bits: int, v_bits: int):
    """bf16 (K_hat, V_hat) patterns from the five planes."""
    k, v = dequantize_kv_f32(planes, signs, d, k_bits, v_bits)
    return f32_to_bf16(k), f32_to_bf16(v)
