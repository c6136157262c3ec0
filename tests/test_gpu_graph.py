"""The decode path under HIP graph capture.

qsa_decode enqueues only kernel launches on the caller's stream (no
allocation, no memset, no synchronisation), so a whole step can be captured
once and replayed.  Each replay must reproduce the eager step bit for bit,
also with eager work on the same buffers between the replays.
"""
import pytest
import torch

from tests import harness, inputs

pytestmark = pytest.mark.gpu


def same(a, b):
    return torch.equal(a.view(torch.int32), b.view(torch.int32)) if a.dtype == torch.float32 \
        else torch.equal(a, b)


def clobber(case):
    case.token_ids.fill_(-7)
    case.width.fill_(-7)
    case.out.fill_(float("nan"))
    case.lse.fill_(float("nan"))


@pytest.mark.parametrize("rows", ["compact", "fused", "dedup"])
def test_graph_replays_match_eager(rows):
    lens = [9000, 2055, 70001, 300, 0, 4096]
    spec = inputs.custom("graph", lens, h_i=4, d_i=64, h_q=4, h_kv=2, d=128, budget=512,
                         keys="normal", slots="perm")
    data = inputs.make(spec, seed=41, device="cpu")
    case = harness.GpuCase(data)
    case.decode(rows=rows)
    torch.cuda.synchronize()
    ref = case.results()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        case.decode(rows=rows)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        case.decode(rows=rows)
    torch.cuda.synchronize()
    for rep in range(3):
        clobber(case)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = case.results()
        for a, b in zip(got, ref):
            assert same(a, b), f"replay {rep} differs from the eager step"
    # eager again after the replays: the graph left nothing behind
    clobber(case)
    case.decode(rows=rows)
    torch.cuda.synchronize()
    for a, b in zip(case.results(), ref):
        assert same(a, b)
    del graph
