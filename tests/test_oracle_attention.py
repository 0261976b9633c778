"""Pins of the float64 decode-attention oracle (CPU only).

TurboQuant page, "Deferred inverse FWHT": un-rotating the attention output
once equals un-rotating every value row first (linearity in V).  Special
cases fix the rest: one cached token returns that token's value, equal keys
return the mean value, a dominant score returns its value, and with the
dequantized K/V materialised the result is ordinary scaled-dot-product
attention (checked against torch's implementation on the CPU in float64).
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention, codec


def _cache(B, Hkv, N, d, kb, vb, seed):
    rng = np.random.default_rng(seed)
    s = np.where(rng.random(d) < 0.5, -1, 1).astype(np.int8)
    k = codec.f32_to_bf16(rng.standard_normal((B * Hkv * N, d)).astype(np.float32))
    v = codec.f32_to_bf16(rng.standard_normal((B * Hkv * N, d)).astype(np.float32))
    p = codec.quantize_kv(k, v, s, kb, vb)
    kidx = codec.key_indices(p["k_q"], kb, d)
    khat = codec.dequantize_keys_f32(kidx, p["k_scale"], p["k_zero"]).reshape(B, Hkv, N, d)
    vidx = codec.unpack_bits(p["v_q"], vb, d)
    z = codec.dequantize_values_rotated_f32(vidx, p["v_scale"], vb).reshape(B, Hkv, N, d)
    return s, khat, z


def _q(B, Hq, d, seed):
    rng = np.random.default_rng(seed)
    return codec.bf16_to_f32(codec.f32_to_bf16(rng.standard_normal((B, Hq, d)).astype(np.float32)))


def test_deferred_equals_eager():
    s, khat, z = _cache(2, 2, 50, 128, 8, 3, 1)
    q = _q(2, 8, 128, 2)
    ctx = [50, 33]
    a = attention.decode_attention(q, khat, z, s, ctx, 1 / math.sqrt(128))
    b = attention.eager_decode_attention(q, khat, z, s, ctx, 1 / math.sqrt(128))
    assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(b))


def test_matches_torch_sdpa_on_dequantized_cache():
    B, Hq, Hkv, N, d = 2, 8, 2, 40, 64
    s, khat, z = _cache(B, Hkv, N, d, 4, 4, 3)
    q = _q(B, Hq, d, 4)
    o = attention.decode_attention(q, khat, z, s, [N, N], 1 / math.sqrt(d))
    vhat = (z.reshape(-1, d).astype(np.float64) @ attention.hadamard_matrix(d).T / math.sqrt(d)) * s
    vhat = vhat.reshape(B, Hkv, N, d)
    rep = Hq // Hkv
    kt = torch.from_numpy(khat.astype(np.float64)).repeat_interleave(rep, dim=1)
    vt = torch.from_numpy(vhat).repeat_interleave(rep, dim=1)
    qt = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, :, 0, :].numpy()
    assert np.max(np.abs(o - ref)) <= 1e-12


def test_single_token_returns_its_value():
    s, khat, z = _cache(1, 1, 5, 128, 8, 3, 5)
    q = _q(1, 4, 128, 6)
    o = attention.decode_attention(q, khat, z, s, [1], 0.1)
    v0 = (attention.hadamard_matrix(128) @ z[0, 0, 0].astype(np.float64)) / math.sqrt(128) * s
    for h in range(4):
        assert np.allclose(o[0, h], v0, rtol=0, atol=1e-12)


def test_equal_keys_average_values():
    s, khat, z = _cache(1, 1, 7, 64, 8, 4, 7)
    khat[:] = khat[0, 0, 0]
    q = _q(1, 2, 64, 8)
    o = attention.decode_attention(q, khat, z, s, [7], 1.0)
    mean = (attention.hadamard_matrix(64) @ z[0, 0].astype(np.float64).mean(0)) / 8.0 * s
    assert np.allclose(o[0, 0], mean, atol=1e-12)


def test_dominant_score_selects_its_value():
    s, khat, z = _cache(1, 1, 9, 64, 8, 3, 9)
    q = _q(1, 1, 64, 10)
    khat[0, 0, 4] = 50.0 * np.sign(q[0, 0])
    o = attention.decode_attention(q, khat, z, s, [9], 1.0)
    v4 = (attention.hadamard_matrix(64) @ z[0, 0, 4].astype(np.float64)) / 8.0 * s
    assert np.allclose(o[0, 0], v4, atol=1e-9)


def test_gqa_head_mapping_is_consecutive():
    s, khat, z = _cache(1, 2, 6, 64, 8, 3, 11)
    q = np.repeat(_q(1, 1, 64, 12), 4, axis=1)
    o = attention.decode_attention(q, khat, z, s, [6], 0.125)
    assert np.allclose(o[0, 0], o[0, 1]) and np.allclose(o[0, 2], o[0, 3])
    assert not np.allclose(o[0, 1], o[0, 2])


def test_empty_context_gives_zero_row_and_clamps_long_context():
    s, khat, z = _cache(2, 1, 4, 64, 8, 3, 13)
    q = _q(2, 1, 64, 14)
    o = attention.decode_attention(q, khat, z, s, [0, 99], 0.125)
    assert np.all(o[0] == 0)
    full = attention.decode_attention(q, khat, z, s, [0, 4], 0.125)
    assert np.array_equal(o, full)


def test_hadamard_matrix_closed_form():
    H = attention.hadamard_matrix(8)
    assert np.array_equal(H @ H.T, 8 * np.eye(8))
    assert list(H[3]) == [1, -1, -1, 1, 1, -1, -1, 1]


def test_multi_query_is_causal_and_reduces_to_decode():
    # one query equals the decode form; query m of a chunk ignores the later
    # tokens of the chunk (changing them leaves it unchanged) and equals the
    # decode form over the prefix ending at itself
    rng = np.random.default_rng(3)
    B, M, Hq, Hkv, N, d = 2, 3, 4, 2, 9, 64
    q = rng.standard_normal((B, M, Hq, d))
    k = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    z = rng.standard_normal((B, Hkv, N, d)).astype(np.float32)
    signs = np.where(rng.integers(0, 2, d) == 1, 1, -1).astype(np.int8)
    ctx = [9, 5]
    o = attention.multi_query_attention(q, k, z, signs, ctx, 0.125)
    one = attention.multi_query_attention(q[:, 2:], k, z, signs, ctx, 0.125)
    assert np.array_equal(one[:, 0], attention.decode_attention(q[:, 2], k, z, signs, ctx, 0.125))
    assert np.array_equal(o[:, 2], one[:, 0])
    k2, z2 = k.copy(), z.copy()
    k2[:, :, 4:] += 10.0
    z2[:, :, 4:] -= 7.0                     # tokens 4.. of sequence 1 are after its query 0 (position 2)
    o2 = attention.multi_query_attention(q, k2, z2, signs, ctx, 0.125)
    assert np.array_equal(o2[1, 0], o[1, 0])
    assert not np.allclose(o2[1, 2], o[1, 2])
    # a query with nothing visible is a zero row
    o3 = attention.multi_query_attention(q, k, z, signs, [2, 9], 0.125)
    assert not o3[0, 0].any()
