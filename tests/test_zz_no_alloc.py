"""tq_attn_quant_noalloc (the entry point that allocates nothing) against
tq_attn_quant with a caller workspace: the same kernels, so the outputs must
be identical, on two calls in a row (the second smaller, reusing the
library's scratch) and after other work; a problem too large for the scratch
is refused before anything is launched."""
import numpy as np
import pytest
import torch

from kv_cache_quantization_02_amd import binding as tq
from kv_cache_quantization_02_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print(*a, flush=True)


def _case(B, M, Hq, Hkv, N, d, kb, vb, ctx, seed):
    k, v = synth.kv_inputs("normal", B, N, Hkv, d, seed, device=DEV)
    q = synth.queries(B * M, Hq, d, seed + 1, device=DEV).reshape(B, M, Hq, d)
    sig = torch.from_numpy(synth.sign_vector(d)).to(DEV)
    cache = tq.quantize_into_cache(k, v, sig, kb, vb)
    return q, cache, torch.tensor(ctx, dtype=torch.int32, device=DEV), sig


def _both(q, cache, ctx, sig, kb, vb, Hkv):
    B, M, Hq, d = q.shape
    N = cache["k_q"].shape[2]
    sch = tq.scheme(d, kb, vb)
    assert tq.tq_attn_quant_workspace_bytes(sch, B, M, Hq, Hkv, N) <= tq.NOALLOC_SCRATCH_BYTES
    want = tq.attn_quant(q, cache, ctx, sig, kb, vb, Hkv)
    got = torch.full_like(want, float("nan"))
    st = tq.tq_attn_quant_noalloc(sch, q, B, M, Hq, Hkv, tq.planes_struct(cache), Hkv * N, N, ctx, N,
                                  float(d ** -0.5), sig, got)
    assert st == 0, tq.status_string(st)
    torch.cuda.synchronize()
    return got, want


@pytest.mark.parametrize("d,kb,vb", [(128, 8, 3), (256, 4, 4)])
def test_noalloc_matches_workspace_call_twice(d, kb, vb):
    # first call: 4 sequences x 2 queries over 2000 tokens (many split partials);
    # second: a smaller problem that reuses only part of the scratch
    _say(f"[gpu noalloc] d={d} k{kb}v{vb} call 1: B=4 M=2 Hq=16 Hkv=4 N=2000")
    got, want = _both(*_case(4, 2, 16, 4, 2000, d, kb, vb, [2000, 1999, 700, 3], 41), kb, vb, 4)
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    _say(f"[gpu noalloc] d={d} k{kb}v{vb} call 2: B=2 M=1 Hq=8 Hkv=2 N=300")
    got, want = _both(*_case(2, 1, 8, 2, 300, d, kb, vb, [300, 51], 42), kb, vb, 2)
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    assert not torch.isnan(got.float()).any()


def test_noalloc_refuses_problems_beyond_its_scratch():
    d, kb, vb = 128, 8, 3
    sch = tq.scheme(d, kb, vb)
    B, M, Hq, Hkv, N = 64, 8, 64, 8, 32768
    need = tq.tq_attn_quant_workspace_bytes(sch, B, M, Hq, Hkv, N)
    assert need > tq.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((16,), dtype=torch.bfloat16, device=DEV)
    planes = tq.Planes(*([q.data_ptr()] * 5))
    ctx = torch.zeros((B,), dtype=torch.int32, device=DEV)
    st = tq.tq_attn_quant_noalloc(sch, q, B, M, Hq, Hkv, planes, Hkv * N, N, ctx, N, 0.088, q, q)
    assert st == -6
