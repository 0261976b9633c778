"""Appending to and fetching from a quantized KV cache (oracle, test infrastructure).

Only the tests use this module.  Sources:

* TurboQuant page, "Architecture in mlx-bun": the cache's update quantizes
  only the newly appended tokens into packed storage and hands back the
  active window dequantized to bf16;
* TurboQuant page, "Deferred inverse FWHT": the deferred variant hands back
  the value window still in the rotated domain (rounded to bf16 there), and
  attention un-rotates its output instead;
* campaign execution-log page, the KV append dispatch probe: a cache's
  storage grows in 256-token steps, by allocating zero padding and
  concatenating the old storage in front of it.

Caches here are dicts of numpy planes shaped [B, H, capacity, row_bytes]
(uint8 for k_q / v_q, uint16 fp16 patterns for the scale and zero planes),
the layout the library addresses with row(b, g, t) = b*H*cap + g*cap + t.
"""
from __future__ import annotations

import numpy as np

from . import codec

PLANES = ("k_q", "k_scale", "k_zero", "v_q", "v_scale")
CAPACITY_STEP = 256


def grown_capacity(tokens: int) -> int:
    """The capacity a cache that must hold `tokens` tokens grows to: the
    smallest whole number of 256-token steps that covers them (0 for 0)."""
    if tokens < 0:
        raise ValueError("negative token count")
    return -(-tokens // CAPACITY_STEP) * CAPACITY_STEP


def grow_kv(cache: dict, new_capacity: int) -> dict:
    """The cache re-laid at `new_capacity` tokens per (sequence, kv head): the
    old storage concatenated in front of zero padding.  Rows t below both
    capacities keep their bytes; rows past the old capacity are zero bytes;
    with a smaller new capacity the rows past it are dropped (a trim)."""
    out = {}
    for name in PLANES:
        old = np.asarray(cache[name])
        B, H, cap, w = old.shape
        keep = min(cap, new_capacity)
        pad = np.zeros((B, H, new_capacity - keep, w), old.dtype)
        out[name] = np.concatenate([old[:, :, :keep], pad], axis=2)
    return out


def append_kv(cache: dict, k_new: np.ndarray, v_new: np.ndarray, positions, signs: np.ndarray,
              k_bits: int, v_bits: int) -> dict:
    """A copy of `cache` with the bf16 tokens k_new / v_new [B, n, H, d] quantized
    into token positions[b] + j; tokens outside [0, capacity) are dropped and
    every other cache row is left as it was."""
    B, n, H, d = k_new.shape
    cap = cache["k_q"].shape[2]
    kr = np.ascontiguousarray(np.asarray(k_new, np.uint16).transpose(0, 2, 1, 3)).reshape(-1, d)
    vr = np.ascontiguousarray(np.asarray(v_new, np.uint16).transpose(0, 2, 1, 3)).reshape(-1, d)
    q = codec.quantize_kv(kr, vr, signs, k_bits, v_bits)
    out = {name: np.array(cache[name], copy=True) for name in PLANES}
    for name in PLANES:
        rows = np.asarray(q[name]).reshape(B, H, n, -1)
        for b in range(B):
            for j in range(n):
                t = int(positions[b]) + j
                if 0 <= t < cap:
                    out[name][b, :, t] = rows[b, :, j]
    return out


def fetch_kv(cache: dict, lens, window: int, signs: np.ndarray, d: int, k_bits: int, v_bits: int,
             values_rotated: bool = False):
    """bf16 patterns (K, V) shaped [B, H, window, d]: token t of each (sequence,
    kv head) for t < lens[b], +0 rows after it.  Keys are dequantized;
    values are dequantized and un-rotated, or with values_rotated left as
    centroid * scale16 rounded to bf16."""
    B, H, cap = cache["k_q"].shape[:3]
    k_out = np.zeros((B, H, window, d), np.uint16)
    v_out = np.zeros((B, H, window, d), np.uint16)
    for b in range(B):
        n = min(int(lens[b]), window, cap)
        if n <= 0:
            continue
        rows = {name: np.ascontiguousarray(cache[name][b, :, :n]).reshape(H * n, -1) for name in PLANES}
        kidx = codec.key_indices(rows["k_q"], k_bits, d)
        k = codec.dequantize_keys_f32(kidx, rows["k_scale"], rows["k_zero"])
        vidx = codec.unpack_bits(rows["v_q"], v_bits, d).astype(np.int32)
        if values_rotated:
            v = codec.dequantize_values_rotated_f32(vidx, rows["v_scale"], v_bits)
        else:
            v = codec.dequantize_values_f32(vidx, rows["v_scale"], signs, v_bits)
        k_out[b, :, :n] = codec.f32_to_bf16(k).reshape(H, n, d)
        v_out[b, :, :n] = codec.f32_to_bf16(v).reshape(H, n, d)
    return k_out, v_out
