"""Kernels replayed from a captured HIP graph (GPU).

bench.py times the decode-append step as 64 per-layer quantize launches
replayed from a captured graph.  Each replay here must write exactly the
planes of the eager launches; the planes are cleared between replays by
the program's own eager work (torch's fill kernel, not a memset node), with
synchronizations in between, and the graph is replayed several times.
"""
import pytest
import torch

from kv_cache_quantization_02_amd import binding as tq
from kv_cache_quantization_02_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("d,kb,vb", [(128, 8, 3), (64, 4, 5)])
def test_per_layer_quantize_graph_replays_match_eager(d, kb, vb):
    L, T, H = 8, 32, 4
    _say(f"[gpu graph] per-layer quantize d={d} k{kb}v{vb} {L}x{T}x{H}")
    k, v = synth.kv_inputs("normal", L, T, H, d, 61, device=DEV)
    sig = torch.from_numpy(synth.sign_vector(d)).to(DEV)
    sch = tq.scheme(d, kb, vb)
    eager = tq.quantize_kv(k, v, sig, kb, vb)
    planes = tq.alloc_planes(sch, (L, T, H), DEV)
    per_layer = [(k[l:l + 1], v[l:l + 1], {n: t[l:l + 1] for n, t in planes.items()}) for l in range(L)]

    def layers():
        for kl, vl, pl in per_layer:
            tq.quantize_kv(kl, vl, sig, kb, vb, out=pl)

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layers()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        layers()
    for rep in range(4):
        for t in planes.values():
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in tq.PLANES:
            assert torch.equal(planes[n].view(torch.uint8), eager[n].view(torch.uint8)), f"replay {rep}: {n} differs"
    del graph
