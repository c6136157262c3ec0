"""Chunk dedup: one union gather per pass of rows (qsa_union_gather,
qsa_online_attend_indexed, qsa_decode_dedup).

The union must hold exactly the groups the oracle's rows touch (selected
groups and raw-tail groups), ordered by (sequence, position), each token's
K/V row a bitwise copy of its cache row; every row's position list must point
at its own tokens; and the attention read through the positions must give the
per-row compact path's bits (AFN-016 "A sparse mask is not sparse attention",
§Why compact gather comes before fusion: one bounded copy of only selected
rows; AFN-017 capsule evidence: chunk/decode equality).
"""
import numpy as np
import pytest
import torch

import top_sparse_attention_qsa_amd as qsa
from tests import harness, inputs

pytestmark = pytest.mark.gpu


def same(a, b):
    """Bitwise equality that also matches NaN payload positions."""
    return torch.equal(a.view(torch.int32), b.view(torch.int32)) if a.dtype == torch.float32 \
        else torch.equal(a, b)


def assert_same_results(x, y):
    for a, b in zip(x, y):
        assert same(a, b)


def chunk_case(lens, queries, seed, rows_in_flight=0, **kw):
    base = dict(h_i=16, d_i=64, h_q=8, h_kv=2, d=128, budget=512, keys="normal", slots="perm")
    base.update(kw)
    spec = inputs.custom("union", lens, queries=queries, **base)
    data = inputs.make(spec, seed=seed, device="cpu")
    return data, harness.GpuCase(data, rows_in_flight=rows_in_flight)


def oracle_union(data):
    """Sorted (sequence, group) pairs the oracle's rows touch, and per-row IDs."""
    s = data["spec"]
    rows_ids = []
    members = set()
    for r in range(s.rows):
        exp = harness.oracle_row(data, r, exact=False)
        ids = np.asarray(exp["ids"], np.int64)
        rows_ids.append(ids)
        b = r // s.queries
        members.update((b, int(g)) for g in np.unique(ids // 4))
    return sorted(members), rows_ids


def test_union_membership_positions_and_rows():
    data, case = chunk_case([2100, 5000, 9001], queries=8, seed=21)
    case.decode()
    torch.cuda.synchronize()
    s, sh = case.spec, case.shape
    members, rows_ids = oracle_union(data)
    rank = {m: i for i, m in enumerate(members)}

    cap = sh.rows * sh.token_stride
    ku = torch.full((cap, s.h_kv, s.d), float("nan"), device="cuda")
    vu = torch.full_like(ku, float("nan"))
    pos = torch.empty((sh.rows, sh.token_stride), dtype=torch.int32, device="cuda")
    count = torch.zeros(1, dtype=torch.int32, device="cuda")
    qsa.qsa_union_gather(sh, case.token_ids, case.width, case.seq_len, case.slot_map,
                         case.slot_off, case.k_cache, case.v_cache, ku, vu, pos, count,
                         case.workspace)
    torch.cuda.synchronize()
    assert int(count) == len(members)
    assert len(members) < sum(len(i) for i in rows_ids) // 4  # the rows really share groups

    pos_h = pos.cpu().numpy()
    smap = data["slot_map"].numpy()
    off = data["raw_off"].numpy()
    kc, vc = data["k_cache"], data["v_cache"]
    ku_h, vu_h = ku.cpu(), vu.cpu()
    for r, ids in enumerate(rows_ids):
        b = r // s.queries
        w = len(ids)
        expect = np.array([4 * rank[(b, int(t) // 4)] + int(t) % 4 for t in ids], np.int64)
        assert np.array_equal(pos_h[r, :w], expect), r
        assert np.all(pos_h[r, w:] == -1)
        slots = smap[off[b] + ids]
        assert torch.equal(ku_h[torch.as_tensor(expect)], kc[torch.as_tensor(slots)]), r
        assert torch.equal(vu_h[torch.as_tensor(expect)], vc[torch.as_tensor(slots)]), r

    # the attention read through the positions gives the compact path's bits
    out = torch.empty_like(case.out)
    lse = torch.empty_like(case.lse)
    qsa.qsa_online_attend_indexed(sh, case.q, ku, vu, pos, case.width, case.scale, out, lse,
                                  case.workspace)
    torch.cuda.synchronize()
    assert same(out, case.out) and same(lse, case.lse)


@pytest.mark.parametrize("rows_in_flight", [0, 8, 20, 3])
def test_dedup_equals_compact_across_pass_splits(rows_in_flight):
    """Passes that hold whole sequences, split sequences, or straddle two."""
    data, case = chunk_case([2100, 5000, 9001, 4101], queries=8, seed=22,
                            rows_in_flight=rows_in_flight)
    case.decode()
    ref = case.results()
    case.decode(rows="dedup")
    assert_same_results(case.results(), ref)


@pytest.mark.parametrize("h_i,d_i,h_q,h_kv,d,q", [(4, 32, 2, 2, 64, 16), (8, 128, 16, 1, 64, 8),
                                                  (16, 32, 16, 16, 128, 4)])
def test_dedup_shapes(h_i, d_i, h_q, h_kv, d, q):
    data, case = chunk_case([2055, 2300, 30000], queries=q, seed=h_i + d, h_i=h_i, d_i=d_i,
                            h_q=h_q, h_kv=h_kv, d=d)
    case.decode()
    ref = case.results()
    case.decode(rows="dedup")
    assert_same_results(case.results(), ref)


@pytest.mark.parametrize("name", ["tail_2055", "ring_65537", "dup_100000"])
def test_dedup_decode_rows_equal_compact(name):
    """queries = 1: each row's union is its own rows."""
    data = inputs.make(inputs.spec(name), seed=1, device="cpu")
    case = harness.GpuCase(data)
    case.decode()
    ref = case.results()
    case.decode(rows="dedup")
    assert_same_results(case.results(), ref)


def test_dedup_ragged_small_budget_and_empty_rows():
    lens = [0, 3, 63, 64, 65, 257, 1000, 4097]
    spec = inputs.custom("ragged_u", lens, queries=1, h_i=4, d_i=32, h_q=4, h_kv=2, d=64,
                         budget=16, keys="grid", slots="perm")
    data = inputs.make(spec, seed=23, device="cpu")
    case = harness.GpuCase(data)
    case.decode()
    ref = case.results()
    case.decode(rows="dedup")
    assert_same_results(case.results(), ref)


def test_dedup_tie_heavy_and_tied_rows():
    data, case = chunk_case([40000, 12000], queries=8, seed=24, h_i=16, d_i=64, h_q=4, h_kv=1,
                            d=64, keys="grid_dup")
    case.decode()
    ref = case.results()
    case.decode(rows="dedup")
    assert_same_results(case.results(), ref)
    data, case = chunk_case([20001, 4100], queries=4, seed=25, h_i=16, d_i=32, h_q=1, h_kv=1,
                            d=64, keys="zero_query")
    case.decode()
    ref = case.results()
    case.decode(rows="dedup")
    assert_same_results(case.results(), ref)


def test_dedup_out_of_range_slot_and_invalid_row():
    spec = inputs.custom("bad_u", [9000, 700, 300], queries=4, h_i=4, d_i=32, h_q=2, h_kv=1,
                         d=64)
    data = inputs.make(spec, seed=26, device="cpu")
    case = harness.GpuCase(data)
    case.slot_map[int(case.slot_off[2]) + 5] = case.shape.kv_slots + 3
    case.seq_len[0] = 4 * case.shape.max_groups + 8  # rows of sequence 0 become invalid
    case.decode()
    ref = case.results()
    case.decode(rows="dedup")
    assert_same_results(case.results(), ref)
    s = case.spec
    assert torch.all(case.width[:s.queries] == -1)
    assert torch.isnan(case.out[2 * s.queries]).all()        # token 5 is in every row of seq 2
    assert torch.isfinite(case.out[s.queries:2 * s.queries]).all()


def test_dedup_long_rows_global_bitmaps():
    """Rows of more than 262,144 groups: the per-row group bitmaps no longer fit
    in LDS and are built in global memory; the result is still the compact
    path's, and the oracle's on the longest rows."""
    data, case = chunk_case([1_100_003, 3000], queries=4, seed=23, h_i=4, d_i=32, h_q=2,
                            h_kv=1, d=64, budget=64)
    assert case.shape.max_groups // 32 > 8192
    case.decode()
    ref = case.results()
    case.decode(rows="dedup")
    assert_same_results(case.results(), ref)
    ids = ref[0].cpu().numpy()
    for r in (0, 3):
        exp = harness.oracle_row(data, r, exact=False)
        w = len(exp["ids"])
        assert np.array_equal(ids[r, :w], exp["ids"])
