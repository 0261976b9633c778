"""Pins of the cache append / fetch oracle (oracle/cache.py) against the
codec oracle it places: placement, untouched rows, dropped tokens, the +0
tail of a window, and the deferred identity between the rotated and the
eager value windows."""
import numpy as np

from kv_cache_quantization_02_amd import synth
from oracle import cache as oc
from oracle import codec


def _empty(B, H, cap, d, kb, vb, fill=0):
    rb = codec.plane_row_bytes(d, kb, vb)
    rng = np.random.default_rng(5)
    c = {}
    for name in oc.PLANES:
        if name in ("k_q", "v_q"):
            c[name] = rng.integers(0, 256, (B, H, cap, rb[name]), dtype=np.uint8) if fill else \
                np.zeros((B, H, cap, rb[name]), np.uint8)
        else:
            c[name] = rng.integers(0, 0x3C00, (B, H, cap, rb[name] // 2), dtype=np.uint16) if fill else \
                np.zeros((B, H, cap, rb[name] // 2), np.uint16)
    return c


def test_append_places_quantized_rows_and_leaves_the_rest():
    B, n, H, d, kb, vb, cap = 3, 5, 2, 64, 8, 3, 12
    k, v = synth.kv_inputs("normal", B, n, H, d, 21)
    kb16, vb16 = synth.bf16_bits(k), synth.bf16_bits(v)
    signs = synth.sign_vector(d)
    before = _empty(B, H, cap, d, kb, vb, fill=1)
    pos = [0, 9, -2]          # second sequence runs past the capacity, third starts before 0
    after = oc.append_kv(before, kb16, vb16, pos, signs, kb, vb)
    for b in range(B):
        for j in range(n):
            t = pos[b] + j
            single = codec.quantize_kv(kb16[b, j], vb16[b, j], signs, kb, vb)   # rows [H, d]
            if 0 <= t < cap:
                for name in oc.PLANES:
                    assert np.array_equal(after[name][b, :, t], np.asarray(single[name]).reshape(H, -1))
    written = {(b, p + j) for b, p in enumerate(pos) for j in range(n) if 0 <= p + j < cap}
    for b in range(B):
        for t in range(cap):
            if (b, t) not in written:
                for name in oc.PLANES:
                    assert np.array_equal(after[name][b, :, t], before[name][b, :, t])
    assert len(written) == 5 + 3 + 3


def test_fetch_window_matches_dequantize_and_zero_tail():
    B, n, H, d, kb, vb = 2, 7, 2, 128, 4, 4
    k, v = synth.kv_inputs("normal", B, n, H, d, 22)
    signs = synth.sign_vector(d)
    c = oc.append_kv(_empty(B, H, 10, d, kb, vb), synth.bf16_bits(k), synth.bf16_bits(v), [0, 0], signs, kb, vb)
    lens, window = [7, 3], 8
    K, V = oc.fetch_kv(c, lens, window, signs, d, kb, vb)
    kr = synth.bf16_bits(k.permute(0, 2, 1, 3).contiguous()).reshape(-1, d)
    vr = synth.bf16_bits(v.permute(0, 2, 1, 3).contiguous()).reshape(-1, d)
    kd, vd = codec.dequantize_kv(codec.quantize_kv(kr, vr, signs, kb, vb), signs, d, kb, vb)
    kd, vd = kd.reshape(B, H, n, d), vd.reshape(B, H, n, d)
    for b in range(B):
        assert np.array_equal(K[b, :, :lens[b]], kd[b, :, :lens[b]])
        assert np.array_equal(V[b, :, :lens[b]], vd[b, :, :lens[b]])
        assert not K[b, :, lens[b]:].any() and not V[b, :, lens[b]:].any()


def test_rotated_window_unrotates_to_the_eager_one():
    # deferred identity on the fetched rows: signs * FWHT(z) / sqrt(d) of the
    # float32 rotated values is the eager float32 value (bf16 rounding of the
    # rotated window aside, which is the documented difference)
    B, n, H, d, kb, vb = 1, 6, 2, 256, 8, 3
    k, v = synth.kv_inputs("normal", B, n, H, d, 23)
    signs = synth.sign_vector(d)
    c = oc.append_kv(_empty(B, H, n, d, kb, vb), synth.bf16_bits(k), synth.bf16_bits(v), [0], signs, kb, vb)
    _, Vr = oc.fetch_kv(c, [n], n, signs, d, kb, vb, values_rotated=True)
    _, Ve = oc.fetch_kv(c, [n], n, signs, d, kb, vb)
    z = codec.bf16_to_f32(Vr).reshape(-1, d).astype(np.float64)
    h = codec.fwht(z.astype(np.float32)).astype(np.float64) * (1 / np.sqrt(d)) * signs
    e = codec.bf16_to_f32(Ve).reshape(-1, d).astype(np.float64)
    scale = np.max(np.abs(e), axis=1, keepdims=True)
    assert np.max(np.abs(h - e) / scale) < 2 ** -6
    # and without the bf16 step it is exact up to float32 rounding of the transform
    vidx = codec.unpack_bits(np.ascontiguousarray(c["v_q"][0]).reshape(H * n, -1), vb, d).astype(np.int32)
    zf = codec.dequantize_values_rotated_f32(vidx, np.ascontiguousarray(c["v_scale"][0]).reshape(H * n, -1), vb)
    assert np.array_equal(codec.unrotate(zf, signs),
                          codec.dequantize_values_f32(vidx, np.ascontiguousarray(c["v_scale"][0]).reshape(H * n, -1),
                                                      signs, vb))


def test_grown_capacity_takes_whole_256_token_steps():
    # the cache grows in 256-token steps (campaign execution-log page, KV
    # append dispatch probe); the depths are the ones that probe ran
    assert oc.grown_capacity(0) == 0
    for t, want in [(1, 256), (65, 256), (255, 256), (256, 256), (257, 512), (2048, 2048), (2049, 2304),
                     (8192, 8192), (8193, 8448)]:
        assert oc.grown_capacity(t) == want
    for t in range(0, 2000, 7):
        c = oc.grown_capacity(t)
        assert c % 256 == 0 and t <= c < t + 256


def test_grow_keeps_rows_and_zero_pads():
    B, H, cap, d, kb, vb = 3, 2, 7, 64, 4, 3
    before = _empty(B, H, cap, d, kb, vb, fill=1)
    after = oc.grow_kv(before, 11)
    for name in oc.PLANES:
        assert after[name].shape[:3] == (B, H, 11) and after[name].dtype == before[name].dtype
        assert np.array_equal(after[name][:, :, :cap], before[name])
        assert not after[name][:, :, cap:].any()
    signs = synth.sign_vector(d)
    lens = [7, 4, 0]
    for rotated in (False, True):
        K0, V0 = oc.fetch_kv(before, lens, 9, signs, d, kb, vb, values_rotated=rotated)
        K1, V1 = oc.fetch_kv(after, lens, 9, signs, d, kb, vb, values_rotated=rotated)
        assert np.array_equal(K0, K1) and np.array_equal(V0, V1)


def test_trim_drops_rows_past_the_new_capacity():
    B, H, cap, d, kb, vb = 2, 3, 9, 64, 8, 2
    before = _empty(B, H, cap, d, kb, vb, fill=1)
    trimmed = oc.grow_kv(before, 5)
    regrown = oc.grow_kv(trimmed, 9)
    for name in oc.PLANES:
        assert np.array_equal(trimmed[name], before[name][:, :, :5])
        assert np.array_equal(regrown[name][:, :, :5], before[name][:, :, :5])
        assert not regrown[name][:, :, 5:].any()


def test_appends_across_a_growth_boundary_match_one_large_cache():
    # a stream of tokens appended in chunks into a small cache that grows when
    # the next chunk would not fit gives the same planes, byte for byte, as
    # the whole stream appended into a cache created at the final capacity
    # (both start as zero bytes); B != H so that a transposed (b, g) shows
    B, H, d, kb, vb = 2, 3, 64, 5, 4
    chunks = [3, 4, 1, 6, 2]
    total = sum(chunks)
    k, v = synth.kv_inputs("normal", B, total, H, d, 24)
    kb16, vb16 = synth.bf16_bits(k), synth.bf16_bits(v)
    signs = synth.sign_vector(d)
    step = 5                                   # a small growth step keeps the oracle fast
    small = _empty(B, H, step, d, kb, vb)
    pos = 0
    grows = 0
    for n in chunks:
        cap = small["k_q"].shape[2]
        if pos + n > cap:
            small = oc.grow_kv(small, -(-(pos + n) // step) * step)
            grows += 1
        small = oc.append_kv(small, kb16[:, pos:pos + n], vb16[:, pos:pos + n], [pos] * B, signs, kb, vb)
        pos += n
    assert grows >= 2
    cap = small["k_q"].shape[2]
    big = oc.append_kv(_empty(B, H, cap, d, kb, vb), kb16, vb16, [0] * B, signs, kb, vb)
    for name in oc.PLANES:
        assert np.array_equal(small[name], big[name])
    K, V = oc.fetch_kv(small, [total, total - 3], cap, signs, d, kb, vb)
    Kb, Vb = oc.fetch_kv(big, [total, total - 3], cap, signs, d, kb, vb)
    assert np.array_equal(K, Kb) and np.array_equal(V, Vb)
