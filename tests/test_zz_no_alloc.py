"""qsa_decode_noalloc, the entry point for callers that cannot allocate
device memory: called through the C ABI, its results equal qsa_decode's with
a caller workspace bit for bit, on calls in a row over the library's one
static buffer -- the full decode batch (32 x 262,144 tokens) in passes of 4
rows, then smaller inputs whose runs start from whatever the previous call
left in the buffer -- and a shape that needs more than the buffer is refused
before anything is enqueued, outputs untouched."""
import pytest
import torch

import top_sparse_attention_qsa_amd as qsa
from tests import harness, inputs

pytestmark = pytest.mark.gpu


def with_rows_in_flight(shape, r):
    return qsa.make_shape(shape.batch, shape.queries, shape.index_heads, shape.index_dim,
                          shape.q_heads, shape.kv_heads, shape.head_dim, shape.budget_groups,
                          shape.max_groups, shape.kv_slots, r)


def sentinel_outputs(case):
    rows, stride = case.shape.rows, case.shape.token_stride
    s = case.spec
    dev = case.index_q.device
    return (torch.full((rows, stride), -7, dtype=torch.int32, device=dev),
            torch.full((rows,), -7, dtype=torch.int32, device=dev),
            torch.full((rows, s.h_q, s.d), 1234.5, device=dev),
            torch.full((rows, s.h_q), 1234.5, device=dev))


def noalloc(case, shape, outs):
    ids, width, out, lse = outs
    qsa.qsa_decode_noalloc(shape, case.index_q, case.pooled, case.pooled_off, case.seq_len,
                           case.slot_map, case.slot_off, case.k_cache, case.v_cache, case.q,
                           case.scale, ids, width, out, lse)
    torch.cuda.synchronize()
    return outs


def reference(case):
    case.decode()
    torch.cuda.synchronize()
    return case.results()


def assert_bitwise(got, ref, what):
    for name, a, b in zip(("token_ids", "width", "out", "lse"), got, ref):
        assert torch.equal(a, b), f"{what}: {name} differs from qsa_decode"


def test_noalloc_equals_decode_on_calls_in_a_row():
    # 1. the full decode batch, 4 rows per pass (the buffer holds 7)
    print("noalloc: decode_32x262144, rows_in_flight 4", flush=True)
    big = harness.GpuCase(inputs.make(inputs.spec("decode_32x262144"), seed=3, device="cuda"))
    ref = reference(big)
    got = noalloc(big, with_rows_in_flight(big.shape, 4), sentinel_outputs(big))
    assert_bitwise(got, ref, "decode_32x262144")
    assert int(got[1].min()) == 2048
    # too large for the static buffer: refused, nothing written
    outs = sentinel_outputs(big)
    with pytest.raises(qsa.QSAError) as e:
        noalloc(big, with_rows_in_flight(big.shape, 0), outs)
    assert e.value.status == qsa.QSA_ERR_STATIC_WORKSPACE
    assert qsa.qsa_workspace_bytes(big.shape) > qsa.NOALLOC_WORKSPACE_BYTES
    torch.cuda.synchronize()
    assert bool((outs[0] == -7).all()) and bool((outs[1] == -7).all())
    assert bool((outs[2] == 1234.5).all()) and bool((outs[3] == 1234.5).all())
    del big
    torch.cuda.empty_cache()
    # 2. smaller inputs in the same buffer: one 65,537-token row on a ring slot
    #    map, then the 2,055-token row and its dense-parity neighbours
    for name in ("ring_65537", "dup_100000"):
        print(f"noalloc: {name}", flush=True)
        case = harness.GpuCase(inputs.make(inputs.spec(name), seed=3, device="cpu"))
        assert_bitwise(noalloc(case, case.shape, sentinel_outputs(case)), reference(case), name)
    print("noalloc: ragged small rows", flush=True)
    spec = inputs.custom("small", [2055, 2051, 5, 0, 9000], h_i=4, d_i=32, h_q=2, h_kv=1, d=64,
                         keys="grid")
    case = harness.GpuCase(inputs.make(spec, seed=3, device="cpu"))
    assert_bitwise(noalloc(case, case.shape, sentinel_outputs(case)), reference(case), "small")


def test_noalloc_causal_chunk_rows():
    """Chunk rows (MFMA scoring, certified selection) through the static buffer."""
    print("noalloc: causal chunk rows", flush=True)
    spec = inputs.custom("chunk", [3000, 40000], queries=16, h_i=16, d_i=128, h_q=8, h_kv=2,
                         d=128, keys="normal", slots="perm")
    case = harness.GpuCase(inputs.make(spec, seed=4, device="cpu"), rows_in_flight=8)
    assert qsa.qsa_workspace_bytes(case.shape) <= qsa.NOALLOC_WORKSPACE_BYTES
    ref = reference(case)
    got = noalloc(case, case.shape, sentinel_outputs(case))
    assert_bitwise(got, ref, "chunk")
