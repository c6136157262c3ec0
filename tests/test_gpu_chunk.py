"""Causal chunks (prefill rows) against single-query decodes and the oracle.

Each of Q query rows of a sequence sees seq_len - Q + 1 + j tokens and has its
own top-k selection; the chunk path scores them on MFMA with certified bounds
and rescores the candidates exactly, so its results must equal, bit for bit,
one decode per row (AFN-017 "Top-k chooses the set; time chooses the order",
capsule evidence: chunk/decode equality).
"""
import numpy as np
import pytest
import torch

import oracle
import top_sparse_attention_qsa_amd as qsa
from tests import harness, inputs

pytestmark = pytest.mark.gpu


def decode_per_row(case, rows_in_flight=0):
    """The same rows as independent decodes: row r becomes a sequence of its own
    whose history is its visible prefix (same pooled keys, slot map, queries)."""
    s = case.spec
    rows = s.rows
    dev = case.index_q.device
    n_rows = torch.tensor([inputs.row_tokens(s, r) for r in range(rows)], dtype=torch.int32,
                          device=dev)
    seq_of_row = torch.arange(rows, device=dev) // s.queries
    sh = qsa.make_shape(rows, 1, s.h_i, s.d_i, s.h_q, s.h_kv, s.d, s.budget,
                        case.shape.max_groups, case.shape.kv_slots, rows_in_flight)
    ws = torch.empty(qsa.qsa_workspace_bytes(sh), dtype=torch.uint8, device=dev)
    ids = torch.empty((rows, sh.token_stride), dtype=torch.int32, device=dev)
    width = torch.empty(rows, dtype=torch.int32, device=dev)
    out = torch.empty((rows, s.h_q, s.d), device=dev)
    lse = torch.empty((rows, s.h_q), device=dev)
    qsa.qsa_decode(sh, case.index_q, case.pooled, case.pooled_off[seq_of_row].contiguous(),
                   n_rows, case.slot_map, case.slot_off[seq_of_row].contiguous(), case.k_cache,
                   case.v_cache, case.q, case.scale, ids, width, out, lse, ws)
    torch.cuda.synchronize()
    return ids, width, out, lse


def assert_same(case, ref):
    ids, width, out, lse = ref
    torch.cuda.synchronize()
    assert torch.equal(case.width, width)
    assert torch.equal(case.token_ids, ids)
    assert torch.equal(case.out, out)
    assert torch.equal(case.lse, lse)


@pytest.mark.parametrize("h_i,d_i,keys", [(16, 128, "normal"), (8, 64, "grid"), (4, 32, "normal")])
def test_chunk_bounds_hold(h_i, d_i, keys):
    """|approx - chain score| <= bound for every row and group, and the bound
    is far below the scores' own spread."""
    q = 64 // h_i * 4
    spec = inputs.custom("bounds", [3000, 9000], queries=q, h_i=h_i, d_i=d_i, h_q=2, h_kv=1,
                         d=64, budget=64, keys=keys)
    data = inputs.make(spec, seed=h_i, device="cpu")
    case = harness.GpuCase(data)
    sh = case.shape
    approx = torch.full((spec.rows, sh.max_groups), float("nan"), device="cuda")
    bound = torch.full_like(approx, float("nan"))
    qsa.qsa_score_groups_chunk(sh, case.index_q, case.pooled, case.pooled_off, case.seq_len,
                               approx, bound)
    approx, bound = approx.cpu().numpy(), bound.cpu().numpy()
    worst = 0.0
    for r in range(spec.rows):
        n = inputs.row_tokens(spec, r)
        off = int(data["raw_off"][r // q])
        exact = oracle.score(data["index_q"][r].numpy(),
                             oracle.pool_full(data["raw_keys"][off:off + n].numpy()))
        g = len(exact)
        err = np.abs(approx[r, :g].astype(np.float64) - exact)
        assert np.all(err <= bound[r, :g]), r
        worst = max(worst, float(np.max(err / np.maximum(bound[r, :g], 1e-30))))
        assert np.all(np.isnan(approx[r, g:]))  # untouched past G
        assert np.median(bound[r, :g]) < 1e-2 * max(float(np.median(exact)), 1e-3)
    print(f"max error / bound = {worst:.3g}")


@pytest.mark.parametrize("h_i,d_i,q", [(16, 128, 8), (8, 64, 16), (4, 32, 32)])
def test_chunk_equals_decode_per_row_small(h_i, d_i, q):
    spec = inputs.custom("chunk", [2055, 2100, 7000, 30000], queries=q, h_i=h_i, d_i=d_i,
                         h_q=8, h_kv=2, d=128, budget=512, keys="normal", slots="perm")
    data = inputs.make(spec, seed=q, device="cpu")
    case = harness.GpuCase(data)
    case.decode()
    assert_same(case, decode_per_row(case))
    # and the oracle on a few rows
    ids = case.token_ids.cpu().numpy()
    out = case.out.cpu().numpy()
    for r in (0, q - 1, 2 * q + 3, spec.rows - 1):
        exp = harness.oracle_row(data, r)
        w = len(exp["ids"])
        assert np.array_equal(ids[r, :w], exp["ids"])
        assert harness.normwise_rel_err(out[r], exp["out_exact"]) <= 2e-6


def test_chunk_tie_heavy_grid_duplicates():
    spec = inputs.custom("chunk_ties", [40000, 12000], queries=8, h_i=16, d_i=64, h_q=4, h_kv=1,
                         d=64, budget=512, keys="grid_dup", slots="perm")
    data = inputs.make(spec, seed=4, device="cpu")
    case = harness.GpuCase(data)
    case.decode()
    assert_same(case, decode_per_row(case))


def test_chunk_bounds_hold_for_tiny_keys():
    """Keys scaled by 2^-56 and queries by 2^56 (exact scalings: the products,
    and so the chain scores, are those of the unscaled inputs): the keys' sums
    of squares fall below 2^-96, where the kernel raises them before the
    hardware square root; the bound must still hold for every group."""
    h_i, d_i, q = 16, 128, 16
    spec = inputs.custom("bounds_tiny", [3000, 9000], queries=q, h_i=h_i, d_i=d_i, h_q=2,
                         h_kv=1, d=64, budget=64)
    data = inputs.make(spec, seed=11, device="cpu")
    data["raw_keys"] = data["raw_keys"] * 2.0 ** -56
    data["index_q"] = data["index_q"] * 2.0 ** 56
    case = harness.GpuCase(data)
    sh = case.shape
    approx = torch.full((spec.rows, sh.max_groups), float("nan"), device="cuda")
    bound = torch.full_like(approx, float("nan"))
    qsa.qsa_score_groups_chunk(sh, case.index_q, case.pooled, case.pooled_off, case.seq_len,
                               approx, bound)
    approx, bound = approx.cpu().numpy(), bound.cpu().numpy()
    for r in range(spec.rows):
        n = inputs.row_tokens(spec, r)
        off = int(data["raw_off"][r // q])
        pooled = oracle.pool_full(data["raw_keys"][off:off + n].numpy())
        assert float(np.max(np.sum(pooled.astype(np.float64) ** 2, axis=1))) < 2.0 ** -96
        exact = oracle.score(data["index_q"][r].numpy(), pooled)
        g = len(exact)
        err = np.abs(approx[r, :g].astype(np.float64) - exact)
        assert np.all(err <= bound[r, :g]), r


def test_chunk_all_tied_streaming_path():
    """Zero index queries: every bound is 0 and every score +0, so the candidate
    buffer overflows and exact keys are streamed; groups 0..k-1 must win."""
    spec = inputs.custom("chunk_zero", [20001, 4100], queries=4, h_i=16, d_i=32, h_q=1, h_kv=1,
                         d=64, budget=512, keys="zero_query")
    data = inputs.make(spec, seed=5, device="cpu")
    case = harness.GpuCase(data)
    case.decode()
    assert_same(case, decode_per_row(case))
    assert np.array_equal(case.token_ids[0, :2048].cpu().numpy(), np.arange(2048))


def test_full_chunk_equals_256_single_query_decodes():
    """8 sequences of lengths drawn from [2,051, 262,144] (plus the 2,051
    boundary), 256 causal queries each, indexer 16 x 128, attention 32 q /
    4 KV x 128: chunk results, with per-row compact gathers and with one
    union gather per sequence, equal 256 sequential decodes per sequence."""
    spec = inputs.spec("chunk_8x256", seed=1)
    spec.seq_lens[0] = 2051 + 255          # first row sees exactly 2,051 tokens
    data = inputs.make(spec, seed=1, device="cuda")
    case = harness.GpuCase(data, rows_in_flight=256)
    case.decode()
    ref = decode_per_row(case, rows_in_flight=256)
    assert_same(case, ref)
    # one union gather per pass of 256 rows gives the same bits
    case.decode(rows="dedup")
    assert_same(case, ref)
    assert int(case.width[0]) == 2051     # boundary row: dense, 512 groups + 3 tail
    # the oracle on 512 rows spread over all eight sequences: each sequence's
    # first and last 16 rows and 32 rows evenly between (the 2,051-token
    # boundary row is row 0)
    rows = []
    for b in range(spec.batch):
        inner = np.linspace(16, 239, 32).round().astype(int).tolist()
        rows += [b * 256 + j for j in list(range(16)) + inner + list(range(240, 256))]
    assert len(rows) == 512 and 0 in rows
    fetch = harness.device_kv_fetch(case.k_cache, case.v_cache)
    expected = harness.oracle_rows(data, rows, kv_fetch=fetch)
    ids = case.token_ids.cpu().numpy()
    width = case.width.cpu().numpy()
    out = case.out.cpu().numpy()
    worst_norm = worst_elem = 0.0
    for r, exp in zip(rows, expected):
        w = len(exp["ids"])
        assert width[r] == w, r
        assert np.array_equal(ids[r, :w], exp["ids"]), r
        err = harness.normwise_rel_err(out[r], exp["out_exact"])
        assert err <= 2e-6, (r, err)
        worst_norm = max(worst_norm, err)
        worst_elem = max(worst_elem, harness.elementwise_rel_err(out[r], exp["out_exact"]))
    print(f"512 chunk rows: max normwise error {worst_norm:.3g}, max elementwise error "
          f"(floor 1e-6 max|o|) {worst_elem:.3g}")
