"""GPU parity of tq_decode_attn_quant against the float64 oracle.

The oracle quantizes the same bf16 cache rows itself, reconstructs the
float32 keys and rotated-domain values, and evaluates the plain definition
of the attention (oracle/attention.py).  Bar: per element
|o - ref| <= 2e-3 * max_j |ref_row| + ulp_bf16(ref).
"""
import math

import numpy as np
import pytest
import torch

from kv_cache_quantization_02_amd import binding as tq
from kv_cache_quantization_02_amd import synth
from oracle import attention, codec
from parity import attention_close, compare_planes, record

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print(*a, flush=True)


def _oracle_cache(k_bits_rows, v_bits_rows, signs, kb, vb, d):
    ref = codec.quantize_kv(k_bits_rows, v_bits_rows, signs, kb, vb)
    khat = codec.dequantize_keys_f32(ref["k_idx"], ref["k_scale"], ref["k_zero"])
    z = codec.dequantize_values_rotated_f32(ref["v_idx"], ref["v_scale"], vb)
    return khat, z


def _scaled(t, f):
    return t if f == 1.0 else (t.float() * f).to(torch.bfloat16)


def _misaligned(cache):
    """Copies of the planes at base addresses that break the 16-byte (key
    bytes) and 4-byte (fp16 planes) alignment of fresh allocations."""
    out = {}
    for name, t in cache.items():
        shift = 8 if t.dtype == torch.uint8 else 1
        buf = torch.empty(t.numel() + shift, dtype=t.dtype, device=t.device)
        view = buf[shift:].view(t.shape)
        view.copy_(t)
        out[name] = view
    return out


def run_case(B, Hq, Hkv, N, d, kb, vb, ctx, seed, tag, k_mul=1.0, v_mul=1.0, q_mul=1.0, misalign=False):
    _say(f"[gpu attn] {tag}: B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} k{kb}v{vb} ctx={list(ctx)[:8]}")
    k, v = synth.kv_inputs("normal", B, N, Hkv, d, seed)         # [B, N, Hkv, d]
    q = synth.queries(B, Hq, d, seed + 7)
    k, v, q = _scaled(k, k_mul), _scaled(v, v_mul), _scaled(q, q_mul)
    signs = synth.sign_vector(d)
    sig = torch.from_numpy(signs).to(DEV)
    cache = tq.quantize_into_cache(k.to(DEV), v.to(DEV), sig, kb, vb)
    if misalign:
        cache = _misaligned(cache)
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    out = tq.decode_attn(q.to(DEV), cache, ctx_t, sig, kb, vb, Hkv)
    torch.cuda.synchronize()
    kr = synth.bf16_bits(k.permute(0, 2, 1, 3).contiguous()).reshape(-1, d)
    vr = synth.bf16_bits(v.permute(0, 2, 1, 3).contiguous()).reshape(-1, d)
    khat, z = _oracle_cache(kr, vr, signs, kb, vb, d)
    qf = codec.bf16_to_f32(synth.bf16_bits(q))
    ref = attention.decode_attention(qf, khat.reshape(B, Hkv, N, d), z.reshape(B, Hkv, N, d),
                                     signs, ctx, np.float32(1 / math.sqrt(d)))
    st = attention_close(synth.bf16_bits(out).reshape(B, Hq, d), ref)
    _say(f"[gpu attn] {tag}: {st}")
    return out, ref


def test_small_gqa_ragged_contexts():
    run_case(3, 8, 2, 700, 128, 8, 3, [700, 513, 1], 11, "small gqa4")


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (16, 2), (12, 2)])
def test_head_groupings(Hq, Hkv):
    run_case(2, Hq, Hkv, 300, 128, 8, 3, [300, 171], 12, f"rep{Hq // Hkv}")


@pytest.mark.parametrize("d,kb,vb", [(64, 8, 3), (256, 4, 4), (512, 5, 2), (128, 2, 5), (128, 8, 8),
                                     (64, 4, 2), (256, 8, 3)])
def test_schemes(d, kb, vb):
    run_case(2, 8, 2, 257, d, kb, vb, [257, 100], 13, f"d{d} k{kb}v{vb}")


@pytest.mark.parametrize("k_mul,v_mul,q_mul", [(1.0, 1e-4, 1.0), (1.0, 1e-6, 1.0), (1e-3, 1.0, 1e3),
                                               (1e-5, 1.0, 2e5), (1.0, 1.0, 1e-3), (1.0, 300.0, 1.0)])
def test_magnitudes(k_mul, v_mul, q_mul):
    # tiny values, keys and queries of opposite extreme scales, near-uniform
    # attention, large values: the fp16 operands must stay in range
    run_case(2, 8, 2, 400, 128, 8, 3, [400, 233], 15, f"k*{k_mul} v*{v_mul} q*{q_mul}", k_mul, v_mul, q_mul)


@pytest.mark.parametrize("d,vb", [(128, 3), (64, 2)])
def test_misaligned_planes(d, vb):
    # planes off the 16/4-byte alignment the DMA copies need: the other kernel serves them
    run_case(2, 8, 2, 300, d, 8, vb, [300, 129], 16, f"misaligned d{d} v{vb}", misalign=True)


def test_many_steps_ragged_tails():
    # 1024 (sequence, kv-head) units fill the grid without splitting the
    # context: one split of 1024 tokens per unit, eight 32-token steps per
    # wave; the contexts end inside the first step, mid-way and one token
    # short of the cache
    ctx = [1000, 999, 517, 33]
    run_case(4, 256, 256, 1000, 128, 8, 3, ctx, 17, "many steps ragged")


def test_empty_context_gives_zero_rows():
    out, ref = run_case(2, 4, 1, 64, 128, 8, 3, [0, 64], 14, "empty context")
    o = synth.bf16_bits(out).reshape(2, 4, 128)
    assert np.all(o[0] == 0)


def test_full_size_decode_pairs():
    # 32 of the 128 (sequence, kv head) pairs, every query head of each: all kv
    # heads of the first and last sequence and 16 more drawn at random
    cfg = synth.DECODE_ATTN
    B, Hq, Hkv, d, N = cfg["batch"], cfg["q_heads"], cfg["kv_heads"], cfg["head_dim"], cfg["context"]
    kb, vb, seed = cfg["k_bits"], cfg["v_bits"], cfg["seed"]
    _say(f"[gpu attn] full size decode: B={B} Hq={Hq} Hkv={Hkv} N={N}")
    k, v = synth.kv_inputs("normal", B, N, Hkv, d, seed, device=DEV)
    q = synth.queries(B, Hq, d, seed + 7, device=DEV)
    signs = synth.sign_vector(d)
    sig = torch.from_numpy(signs).to(DEV)
    cache = tq.quantize_into_cache(k, v, sig, kb, vb)
    ctx_t = torch.full((B,), N, dtype=torch.int32, device=DEV)
    out = tq.decode_attn(q, cache, ctx_t, sig, kb, vb, Hkv)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    pairs = [(0, g) for g in range(Hkv)] + [(B - 1, g) for g in range(Hkv)]
    rest = [(b, g) for b in range(1, B - 1) for g in range(Hkv)]
    pairs += [rest[i] for i in rng.choice(len(rest), size=16, replace=False)]
    rep = Hq // Hkv
    worst = {"max_rel_l2": 0.0, "max_rel_l2_bf16_floor": 0.0, "max_abs_err": 0.0}
    kt = vt = 0
    for i, (b, g) in enumerate(pairs):
        kr = synth.bf16_bits(k[b, :, g]).reshape(-1, d)
        vr = synth.bf16_bits(v[b, :, g]).reshape(-1, d)
        ref_p = codec.quantize_kv(kr, vr, signs, kb, vb)
        # the GPU cache rows of this pair against the oracle's planes (ties counted)
        st_p = compare_planes({n: cache[n][b, g].cpu().numpy() for n in tq.PLANES}, ref_p, d, kb, vb)
        kt += st_p["key_ties"]
        vt += st_p["value_ties"]
        khat = codec.dequantize_keys_f32(ref_p["k_idx"], ref_p["k_scale"], ref_p["k_zero"])
        z = codec.dequantize_values_rotated_f32(ref_p["v_idx"], ref_p["v_scale"], vb)
        qb = codec.bf16_to_f32(synth.bf16_bits(q[b:b + 1, g * rep:(g + 1) * rep]))
        ref = attention.decode_attention(qb, khat.reshape(1, 1, N, d), z.reshape(1, 1, N, d),
                                         signs, [N], np.float32(1 / math.sqrt(d)))
        got = synth.bf16_bits(out[b:b + 1, g * rep:(g + 1) * rep])
        st = attention_close(got.reshape(1, rep, d), ref)
        worst = {key: max(worst[key], st[key]) for key in worst}
        if i % 8 == 0:
            _say(f"[gpu attn] full size pair {i + 1}/{len(pairs)} (b={b}, kv head {g}): {st}")
    record(f"decode attention k8v3 d128 (B{B} Hq{Hq} Hkv{Hkv} ctx{N}, {len(pairs)} of {B * Hkv} pairs)",
           rows=len(pairs) * N, key_ties=kt, value_ties=vt, max_rel_l2=worst["max_rel_l2"],
           max_rel_l2_bf16_floor=worst["max_rel_l2_bf16_floor"], max_abs_err=worst["max_abs_err"])
    _say(f"[gpu attn] full size decode: {len(pairs)} pairs, ties k={kt} v={vt}, worst {worst}")


def run_mq_case(B, M, Hq, Hkv, N, d, kb, vb, ctx, seed, tag, k_mul=1.0, v_mul=1.0, q_mul=1.0):
    _say(f"[gpu attn] multi-query {tag}: B={B} M={M} Hq={Hq} Hkv={Hkv} N={N} d={d} k{kb}v{vb} ctx={ctx}")
    k, v = synth.kv_inputs("normal", B, N, Hkv, d, seed)
    q = synth.queries(B * M, Hq, d, seed + 7).reshape(B, M, Hq, d)
    k, v, q = _scaled(k, k_mul), _scaled(v, v_mul), _scaled(q, q_mul)
    signs = synth.sign_vector(d)
    sig = torch.from_numpy(signs).to(DEV)
    cache = tq.quantize_into_cache(k.to(DEV), v.to(DEV), sig, kb, vb)
    out = tq.attn_quant(q.to(DEV), cache, torch.tensor(ctx, dtype=torch.int32, device=DEV), sig, kb, vb, Hkv)
    torch.cuda.synchronize()
    kr = synth.bf16_bits(k.permute(0, 2, 1, 3).contiguous()).reshape(-1, d)
    vr = synth.bf16_bits(v.permute(0, 2, 1, 3).contiguous()).reshape(-1, d)
    khat, z = _oracle_cache(kr, vr, signs, kb, vb, d)
    qf = codec.bf16_to_f32(synth.bf16_bits(q))
    ref = attention.multi_query_attention(qf, khat.reshape(B, Hkv, N, d), z.reshape(B, Hkv, N, d),
                                          signs, ctx, np.float32(1 / math.sqrt(d)))
    got = synth.bf16_bits(out)
    st = attention_close(got.reshape(B * M, Hq, d), ref.reshape(B * M, Hq, d))
    _say(f"[gpu attn] multi-query {tag}: {st}")
    return got, ref


@pytest.mark.parametrize("M", [1, 4])
def test_multi_query_causal(M):
    # the last sequence is shorter than the query chunk: its first queries see nothing
    got, ref = run_mq_case(3, M, 8, 2, 300, 128, 8, 3, [300, 133, 2], 18, f"M{M}")
    if M == 4:
        assert not got[2, 0].any() and not got[2, 1].any()


@pytest.mark.parametrize("M", [1, 2])
def test_gqa6_d256(M):
    # the pages' research attention shape: GQA 6 at head_dim 256
    run_mq_case(2, M, 12, 2, 400, 256, 8, 3, [400, 257], 19, f"gqa6 d256 M{M}")


# More than four (query, head) rows per kv head run 16 rows per block, so a
# cached token is scored once for all of them.  Row counts below, at and above
# one tile, idle rows, a sequence shorter than the query chunk, many splits.
@pytest.mark.parametrize("B,M,Hq,Hkv,N,d,vb,ctx", [
    (2, 1, 16, 2, 300, 128, 3, [300, 171]),      # rep 8, one query: 8 rows
    (2, 1, 10, 2, 300, 128, 3, [300, 45]),       # rep 5: 5 rows
    (2, 4, 16, 4, 520, 128, 5, [520, 250]),      # 16 rows, 5-bit values
    (2, 8, 8, 4, 400, 128, 3, [400, 5]),         # 16 rows; the second sequence's first queries see nothing
    (1, 9, 8, 4, 700, 64, 2, [700]),             # 18 rows: two tiles, the second ragged
    (2, 3, 24, 4, 260, 256, 4, [260, 255]),      # rep 6 x 3 queries = 18 rows at d256
    (1, 4, 32, 8, 9000, 128, 3, [9000]),         # many splits
])
def test_sixteen_row_tiles(B, M, Hq, Hkv, N, d, vb, ctx):
    got, ref = run_mq_case(B, M, Hq, Hkv, N, d, 8, vb, ctx, 24, f"16-row tiles M{M} rep{Hq // Hkv} d{d} v{vb}")
    for b, c in enumerate(ctx):
        for m in range(M):
            if c - M + m + 1 <= 0:
                assert not got[b, m].any()


# Packed 5-, 4- and 2-bit keys run on the matrix cores too: their indices
# are spread into bytes and the query operand follows their order.  One
# query (four rows), 16-row tiles (4-bit keys), and 2- and 5-bit keys over
# several rows (four-row tiles).  8-bit values take single-entry centroid
# lookups; value rows that fill whole 16-byte copies (v8, v4, v2 at d >= 128)
# are copied 16 bytes per lane.
@pytest.mark.parametrize("B,M,Hq,Hkv,N,d,kb,vb,ctx", [
    (2, 1, 8, 2, 300, 128, 4, 3, [300, 171]),
    (2, 1, 8, 2, 300, 128, 2, 2, [300, 33]),
    (2, 4, 16, 4, 520, 128, 4, 5, [520, 250]),
    (2, 3, 24, 4, 260, 256, 4, 4, [260, 255]),
    (1, 9, 8, 4, 700, 64, 4, 2, [700]),
    (2, 4, 16, 4, 400, 128, 2, 3, [400, 3]),
    (1, 1, 32, 8, 9000, 256, 2, 4, [9000]),
    (2, 1, 8, 2, 300, 128, 5, 3, [300, 171]),
    (2, 4, 16, 4, 400, 256, 5, 2, [400, 97]),
    (1, 1, 32, 8, 9000, 128, 5, 5, [9000]),
    (2, 1, 8, 2, 300, 128, 8, 8, [300, 171]),
    (2, 4, 16, 4, 520, 128, 8, 8, [520, 250]),
    (2, 1, 12, 2, 400, 256, 8, 8, [400, 257]),
    (2, 2, 8, 2, 300, 64, 4, 8, [300, 77]),
    (1, 1, 32, 8, 9000, 128, 8, 4, [9000]),
    (2, 3, 8, 2, 300, 256, 8, 2, [300, 200]),
    # 2-bit keys at d64: 16-byte key rows, one DMA instruction whose upper lanes re-read the last chunk
    (2, 1, 8, 2, 300, 64, 2, 3, [300, 45]),
    (1, 3, 16, 4, 333, 64, 2, 5, [333]),
    (2, 1, 4, 1, 260, 64, 2, 8, [260, 31]),
    (1, 1, 8, 2, 5000, 64, 2, 2, [4999]),
])
def test_packed_keys_on_matrix_cores(B, M, Hq, Hkv, N, d, kb, vb, ctx):
    got, ref = run_mq_case(B, M, Hq, Hkv, N, d, kb, vb, ctx, 26, f"packed keys k{kb}v{vb} d{d} M{M} rep{Hq // Hkv}")
    for b, c in enumerate(ctx):
        for m in range(M):
            if c - M + m + 1 <= 0:
                assert not got[b, m].any()


@pytest.mark.parametrize("kb", [5, 4, 2])
@pytest.mark.parametrize("k_mul,v_mul,q_mul", [(1e-5, 1.0, 2e5), (1.0, 1.0, 1e-3), (1e3, 300.0, 1e-3)])
def test_packed_key_magnitudes(kb, k_mul, v_mul, q_mul):
    run_mq_case(2, 4, 16, 4, 400, 128, kb, 3, [400, 233], 27, f"packed k{kb} k*{k_mul} v*{v_mul} q*{q_mul}",
                k_mul, v_mul, q_mul)


@pytest.mark.parametrize("k_mul,v_mul,q_mul", [(1.0, 1e-6, 1.0), (1e-5, 1.0, 2e5), (1.0, 1.0, 1e-3),
                                               (1.0, 300.0, 1.0)])
def test_sixteen_row_magnitudes(k_mul, v_mul, q_mul):
    run_mq_case(2, 4, 8, 2, 400, 128, 8, 3, [400, 233], 25, f"16-row k*{k_mul} v*{v_mul} q*{q_mul}",
                k_mul, v_mul, q_mul)


def test_multi_query_valu_schemes():
    run_mq_case(2, 3, 8, 2, 200, 128, 4, 4, [200, 77], 20, "k4v4")
    run_mq_case(2, 3, 8, 4, 200, 512, 5, 2, [150, 200], 21, "d512 k5v2")


def test_multi_query_matches_decode_at_m1():
    # tq_attn_quant with one query is tq_decode_attn_quant
    B, Hq, Hkv, N, d = 2, 8, 2, 256, 128
    k, v = synth.kv_inputs("normal", B, N, Hkv, d, 22)
    q = synth.queries(B, Hq, d, 29)
    sig = torch.from_numpy(synth.sign_vector(d)).to(DEV)
    cache = tq.quantize_into_cache(k.to(DEV), v.to(DEV), sig, 8, 3)
    ctx = torch.tensor([256, 100], dtype=torch.int32, device=DEV)
    a = tq.decode_attn(q.to(DEV), cache, ctx, sig, 8, 3, Hkv)
    b = tq.attn_quant(q.to(DEV).reshape(B, 1, Hq, d), cache, ctx, sig, 8, 3, Hkv)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.reshape(B, Hq, d).view(torch.int16))


def _splits(sch, B, Hq, Hkv, N, d):
    return tq.tq_decode_attn_workspace_bytes(sch, B, Hq, Hkv, N) // (B * Hq * (d + 4) * 4)


# The merge reads each row's splits in batches sized to how many one lane
# merges: one, two, four or eight at a time (the block-per-row merge spreads
# 16 splits of d = 128 over a block), and eight at a time with a second
# batch in the row-per-lanes merge of 9 to 15 splits.
@pytest.mark.parametrize("Hq,Hkv,N,ctx,splits", [(32, 8, 2048, [2048], 16), (32, 8, 8192, [8192], 32),
                                                 (16, 4, 8192, [8192], 64),
                                                 (32, 8, 8192, [8192, 8000, 100, 4097, 1], 13)])
def test_merge_batch_sizes(Hq, Hkv, N, ctx, splits):
    d, kb, vb, B = 128, 8, 3, len(ctx)
    assert _splits(tq.scheme(d, kb, vb), B, Hq, Hkv, N, d) == splits
    run_case(B, Hq, Hkv, N, d, kb, vb, ctx, 29, f"merge of {splits} splits")


@pytest.mark.parametrize("Hq,Hkv,N,d,kb,vb,ctx", [(4, 1, 9000, 128, 8, 3, [8999]), (12, 2, 9000, 256, 8, 3, [9000]),
                                                  (8, 2, 2600, 512, 5, 2, [2600]),
                                                  (4, 1, 9000, 128, 8, 3, [9000, 700]),
                                                  (8, 2, 2600, 512, 5, 2, [1, 2600])])
def test_many_splits_block_merge(Hq, Hkv, N, d, kb, vb, ctx):
    # one or two sequences and few kv heads: the context is cut into 16+
    # splits, merged by the block-per-row combine; a short second context
    # leaves most of its splits empty (m = -inf, l = 0) for the merge
    B = len(ctx)
    sch = tq.scheme(d, kb, vb)
    from kv_cache_quantization_02_amd.binding import lib  # noqa: F401  (library loaded)
    run_case(B, Hq, Hkv, N, d, kb, vb, ctx, 23, f"many splits d{d} k{kb}v{vb}")
    ws = tq.tq_decode_attn_workspace_bytes(sch, B, Hq, Hkv, N)
    assert ws >= 16 * B * Hq * (d + 4) * 4


# Every GQA grouping from 1 to 16 query heads per kv head, one to five query
# tokens per sequence: rows per kv head from 1 to 80, so tiles of four and of
# 16 rows with every count of idle rows in the last tile; contexts that end on
# a step boundary, one past it, and inside the first step.
@pytest.mark.parametrize("rep", [1, 2, 3, 5, 7, 16])
@pytest.mark.parametrize("M", [1, 2, 5])
def test_gqa_groupings_and_query_counts(rep, M):
    Hkv = 2
    ctx = [257, 128, 33]
    run_mq_case(3, M, rep * Hkv, Hkv, 257, 128, 8, 3, ctx, 31 + rep + 7 * M, f"rep{rep} M{M}")


@pytest.mark.parametrize("kb,vb", [(4, 3), (2, 4), (5, 2), (8, 8)])
@pytest.mark.parametrize("rep", [3, 6])
def test_gqa_groupings_packed_schemes(kb, vb, rep):
    run_mq_case(2, 2, rep * 2, 2, 300, 128, kb, vb, [300, 129], 41 + kb + rep, f"k{kb}v{vb} rep{rep}")
