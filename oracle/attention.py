"""Decode attention over a quantized KV cache, plain definition in float64
(oracle, test infrastructure).

TurboQuant page, "Deferred inverse FWHT": attention is linear in V, so the
inverse rotation can be applied once to the attention output instead of to
every cached value row.  The fused decode computes, for batch b and query
head h (kv head g = h // (Hq / Hkv), consecutive query heads share a kv
head):

    s_t = softmax_scale * sum_j q_j * k_hat_{t,j}        for t < ctx_b
    p_t = exp(s_t - max_t s_t),   l = sum_t p_t
    a_j = sum_t p_t * z_{t,j} / l                          (rotated domain)
    o   = signs * (H a) / sqrt(d)                          (one inverse rotation)

with k_hat the float32 key reconstruction (idx + zero16) * scale16 and
z = centroid[idx] * scale16 the rotated-domain value.  H is the Sylvester
Hadamard matrix, H_ij = (-1)^popcount(i & j), built entry by entry here (not
the butterfly).  ``eager_decode_attention`` un-rotates every value row first;
the two agree to float64 rounding, which is the deferred identity.

A sequence with ctx_b <= 0 yields a zero output row; ctx_b is clamped to the
cache capacity.
"""
from __future__ import annotations

import numpy as np


def hadamard_matrix(d: int) -> np.ndarray:
    i = np.arange(d)
    bits = np.bitwise_and(i[:, None], i[None, :])
    pop = np.zeros_like(bits)
    while np.any(bits):
        pop += bits & 1
        bits >>= 1
    return np.where(pop % 2 == 0, 1.0, -1.0)


def _softmax_weights(q64, k64, scale):
    s = (k64 @ q64) * scale
    p = np.exp(s - np.max(s))
    return p, np.sum(p)


def decode_attention(q: np.ndarray, k_hat: np.ndarray, z_rot: np.ndarray,
                     signs: np.ndarray, ctx_lens, softmax_scale: float) -> np.ndarray:
    """q [B, Hq, d] (float values), k_hat / z_rot [B, Hkv, N, d] float32,
    signs [d], ctx_lens [B] -> o [B, Hq, d] float64 (deferred form)."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hkv, N = k_hat.shape[1], k_hat.shape[2]
    rep = Hq // Hkv
    H = hadamard_matrix(d)
    s = np.asarray(signs, np.float64)
    out = np.zeros((B, Hq, d), np.float64)
    for b in range(B):
        n = min(int(ctx_lens[b]), N)
        if n <= 0:
            continue
        for h in range(Hq):
            g = h // rep
            k64 = k_hat[b, g, :n].astype(np.float64)
            z64 = z_rot[b, g, :n].astype(np.float64)
            p, l = _softmax_weights(q[b, h], k64, float(softmax_scale))
            a = (p @ z64) / l
            out[b, h] = s * (H @ a) / np.sqrt(d)
    return out


def eager_decode_attention(q, k_hat, z_rot, signs, ctx_lens, softmax_scale):
    """Same output with every value row un-rotated before the weighted sum."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hkv, N = k_hat.shape[1], k_hat.shape[2]
    rep = Hq // Hkv
    H = hadamard_matrix(d)
    s = np.asarray(signs, np.float64)
    out = np.zeros((B, Hq, d), np.float64)
    for b in range(B):
        n = min(int(ctx_lens[b]), N)
        if n <= 0:
            continue
        for h in range(Hq):
            g = h // rep
            k64 = k_hat[b, g, :n].astype(np.float64)
            v64 = (z_rot[b, g, :n].astype(np.float64) @ H.T) / np.sqrt(d) * s[None, :]
            p, l = _softmax_weights(q[b, h], k64, float(softmax_scale))
            out[b, h] = (p @ v64) / l
    return out


def multi_query_attention(q: np.ndarray, k_hat: np.ndarray, z_rot: np.ndarray,
                          signs: np.ndarray, ctx_lens, softmax_scale: float) -> np.ndarray:
    """Causal multi-query form: q [B, M, Hq, d]; query m of sequence b is the
    cached token at ctx_b - M + m and attends to tokens t < ctx_b - M + 1 + m
    (ctx_b clamped to the cache).  Each query is the single-query case with
    that context, so this is the plain definition written by reuse of it;
    a query with no visible token gives a zero row."""
    q = np.asarray(q, np.float64)
    B, M, Hq, d = q.shape
    N = k_hat.shape[2]
    out = np.zeros((B, M, Hq, d), np.float64)
    for m in range(M):
        lens = [min(int(ctx_lens[b]), N) - M + 1 + m for b in range(B)]
        out[:, m] = decode_attention(q[:, m], k_hat, z_rot, signs, lens, softmax_scale)
    return out
