"""GPU parity: every step of the HIP path against the CPU oracle on the same
seeded inputs.  Integer results (selected IDs, widths, slots, compact copies,
pooled keys, scores) must be bit-exact; attention outputs must be within
2e-6 normwise relative error of the exact (float64) attention over the
oracle's own selected rows.

Sources: AFN-017 "Top-k chooses the set; time chooses the order" and AFN-016
"A sparse mask is not sparse attention".
"""
import numpy as np
import pytest
import torch

import oracle
import top_sparse_attention_qsa_amd as qsa
from tests import harness, inputs

pytestmark = pytest.mark.gpu

ATTN_TOL = 2e-6  # normwise relative, against the exact attention


def untile(pooled_flat, off, g, d_i):
    """Tiled pooled-key buffer of one sequence -> plain [G][D_I] (host)."""
    tiles = (g + 63) // 64
    t = pooled_flat[off:off + tiles * 64 * d_i].view(tiles, d_i // 4, 64, 4)
    return t.permute(0, 2, 1, 3).reshape(tiles * 64, d_i)[:g].cpu().numpy()


def bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def check_rows(case, rows=None, tol=ATTN_TOL, kv_fetch=None):
    s = case.spec
    torch.cuda.synchronize()
    ids = case.token_ids.cpu().numpy()
    width = case.width.cpu().numpy()
    out = case.out.cpu().numpy()
    lse = case.lse.cpu().numpy()
    rows = range(s.rows) if rows is None else rows
    for r in rows:
        exp = harness.oracle_row(case.data, r, kv_fetch=kv_fetch)
        w = len(exp["ids"])
        assert width[r] == w, (s.name, r)
        assert np.array_equal(ids[r, :w], exp["ids"]), (s.name, r)
        assert np.all(ids[r, w:] == -1)
        if w == 0:
            assert np.all(out[r] == 0) and np.all(np.isneginf(lse[r]))
            continue
        err = harness.normwise_rel_err(out[r], exp["out_exact"])
        assert err <= tol, (s.name, r, err)
        assert np.allclose(lse[r], exp["lse_exact"], rtol=0, atol=1e-5), (s.name, r)


@pytest.fixture(scope="module", params=["tail_2055", "ring_65537", "dup_100000"])
def named(request):
    data = inputs.make(inputs.spec(request.param), seed=1, device="cpu")
    case = harness.GpuCase(data)
    case.decode()
    torch.cuda.synchronize()
    return case


def test_pooled_keys_bitexact(named):
    s = named.spec
    for b in range(s.batch):
        g = s.seq_lens[b] // 4
        got = untile(named.pooled, int(named.pooled_off[b]), g, s.d_i)
        off = int(named.data["raw_off"][b])
        want = oracle.pool_full(named.data["raw_keys"][off:off + s.seq_lens[b]].numpy())
        assert np.array_equal(bits(got), bits(want))


def test_incremental_pooling_equals_full(named):
    """Pooling only the groups completed since the previous call, in several
    steps, gives the same bits as pooling the whole history."""
    s = named.spec
    sh = named.shape
    pooled = torch.full_like(named.pooled, float("nan"))
    raw = named.data["raw_keys"].cuda()
    n_full = s.seq_lens[0]
    steps = sorted({0, 5, n_full // 3, n_full // 3 + 1, n_full // 2, n_full - 1, n_full})
    prev_g = 0
    for n in steps[1:]:
        seq = torch.tensor([n] + s.seq_lens[1:], dtype=torch.int32, device="cuda")
        first = torch.tensor([prev_g] + [0] * (s.batch - 1), dtype=torch.int32, device="cuda")
        qsa.qsa_pool_groups(sh, raw, named.raw_off, seq, first, pooled, named.pooled_off)
        prev_g = n // 4
    g = n_full // 4
    a = untile(pooled, 0, g, s.d_i)
    b = untile(named.pooled, 0, g, s.d_i)
    assert np.array_equal(bits(a), bits(b))


def test_scores_bitexact(named):
    s = named.spec
    scores = torch.full((s.rows, named.shape.max_groups), -1.0, device="cuda")
    qsa.qsa_score_groups(named.shape, named.index_q, named.pooled, named.pooled_off,
                         named.seq_len, scores)
    got = scores.cpu().numpy()
    for r in range(s.rows):
        n = inputs.row_tokens(s, r)
        off = int(named.data["raw_off"][r // s.queries])
        pooled = oracle.pool_full(named.data["raw_keys"][off:off + n].numpy())
        want = oracle.score(named.data["index_q"][r].numpy(), pooled)
        assert np.array_equal(bits(got[r, :len(want)]), bits(want))
        assert np.all(got[r, len(want):] == -1.0)  # untouched past G


def test_decode_matches_oracle(named):
    check_rows(named)


def test_select_then_emit_equals_fused(named):
    s, sh = named.spec, named.shape
    scores = torch.empty((s.rows, sh.max_groups), device="cuda")
    qsa.qsa_score_groups(sh, named.index_q, named.pooled, named.pooled_off, named.seq_len, scores)
    bitmap = torch.full((s.rows, sh.max_groups // 32), -1, dtype=torch.int32, device="cuda")
    qsa.qsa_select_topk(sh, scores, named.seq_len, bitmap, named.workspace)
    ids = torch.empty_like(named.token_ids)
    width = torch.empty_like(named.width)
    qsa.qsa_emit_chronological(sh, bitmap, named.seq_len, ids, width)
    assert torch.equal(ids, named.token_ids)
    assert torch.equal(width, named.width)
    bm = bitmap.cpu().numpy().view(np.uint32)
    for r in range(s.rows):
        exp = harness.oracle_row(named.data, r, exact=False)
        g = exp["n"] // 4
        flags = (bm[r][np.arange(g) // 32] >> (np.arange(g) % 32)) & 1
        assert np.array_equal(np.nonzero(flags)[0], np.sort(exp["chosen"]))
        assert np.all(bm[r][(g + 31) // 32:] == 0)


def test_gather_bitexact(named):
    s, sh = named.spec, named.shape
    # compact layout [row][KV head][position][dim]
    kc = torch.full((s.rows, s.h_kv, sh.token_stride, s.d), 7.0, device="cuda")
    vc = torch.full_like(kc, 7.0)
    phys = torch.full((s.rows, sh.token_stride), -7, dtype=torch.int32, device="cuda")
    qsa.qsa_resolve_gather(sh, named.token_ids, named.width, named.seq_len, named.slot_map,
                           named.slot_off, named.k_cache, named.v_cache, kc, vc, phys)
    kc, vc, phys = kc.cpu().numpy(), vc.cpu().numpy(), phys.cpu().numpy()
    for r in range(s.rows):
        exp = harness.oracle_row(named.data, r, exact=False)
        w = len(exp["ids"])
        assert np.array_equal(phys[r, :w], exp["slots"])
        assert np.all(phys[r, w:] == -7)
        kx = np.ascontiguousarray(kc[r, :, :w].transpose(1, 0, 2))
        vx = np.ascontiguousarray(vc[r, :, :w].transpose(1, 0, 2))
        assert kx.tobytes() == exp["kx"].tobytes()
        assert vx.tobytes() == exp["vx"].tobytes()
        assert np.all(kc[r, :, w:] == 7.0)


def test_standalone_attend_equals_decode(named):
    s, sh = named.spec, named.shape
    kc = torch.empty((s.rows, s.h_kv, sh.token_stride, s.d), device="cuda")
    vc = torch.empty_like(kc)
    qsa.qsa_resolve_gather(sh, named.token_ids, named.width, named.seq_len, named.slot_map,
                           named.slot_off, named.k_cache, named.v_cache, kc, vc)
    out = torch.empty_like(named.out)
    lse = torch.empty_like(named.lse)
    qsa.qsa_online_attend(sh, named.q, kc, vc, named.width, named.scale, out, lse,
                          named.workspace)
    assert torch.equal(out, named.out) and torch.equal(lse, named.lse)


def test_decode_is_deterministic(named):
    ref = (named.token_ids.clone(), named.width.clone(), named.out.clone(), named.lse.clone())
    for _ in range(3):
        named.decode()
        torch.cuda.synchronize()
        assert torch.equal(ref[0], named.token_ids) and torch.equal(ref[1], named.width)
        assert torch.equal(ref[2], named.out) and torch.equal(ref[3], named.lse)


def test_unselected_rows_never_enter_the_arithmetic(named):
    """Physical sparsity: NaN in every K/V row outside the selected slots
    changes nothing (AFN-016 §Decision: only selected rows are gathered)."""
    s = named.spec
    keep = torch.zeros(named.k_cache.shape[0], dtype=torch.bool)
    for r in range(s.rows):
        keep[torch.as_tensor(harness.oracle_row(named.data, r, exact=False)["slots"],
                             dtype=torch.int64)] = True
    keep = keep.cuda()
    case = harness.GpuCase(named.data)
    case.k_cache[~keep] = float("nan")
    case.v_cache[~keep] = float("nan")
    case.decode()
    torch.cuda.synchronize()
    assert torch.equal(case.token_ids, named.token_ids)
    assert torch.equal(case.out, named.out) and torch.isfinite(case.out).all()


# ------------------------------------------------------------- edge cases

def run_and_check(spec, seed=1, rows_in_flight=0, tol=ATTN_TOL):
    data = inputs.make(spec, seed=seed, device="cpu")
    case = harness.GpuCase(data, rows_in_flight=rows_in_flight)
    case.decode()
    check_rows(case, tol=tol)
    return case


def test_dense_parity_sweep():
    """0-5 and 2,047-2,052 visible tokens: at or below the budget the row is
    0..N-1 exactly; at 2,052 one group is dropped (AFN-017 capsule evidence)."""
    lens = inputs.sweep_prefixes()
    spec = inputs.custom("sweep", lens, h_i=4, d_i=32, h_q=1, h_kv=1, d=64, keys="grid")
    case = run_and_check(spec)
    ids = case.token_ids.cpu().numpy()
    for r, n in enumerate(lens):
        if n <= 2051:
            assert np.array_equal(ids[r, :n], np.arange(n))
        else:
            assert int(case.width[r]) == 2048


@pytest.mark.parametrize("h_i,d_i,h_q,h_kv,d", [
    (1, 32, 2, 2, 64), (2, 64, 4, 1, 128), (4, 128, 16, 1, 64), (16, 32, 16, 16, 128),
    (8, 128, 8, 2, 64), (4, 64, 16, 1, 128), (4, 32, 8, 1, 64), (2, 32, 2, 1, 128)])
def test_shapes_ragged_batch_small_budget(h_i, d_i, h_q, h_kv, d):
    lens = [0, 3, 63, 64, 65, 257, 1000, 4097]
    spec = inputs.custom("ragged", lens, h_i=h_i, d_i=d_i, h_q=h_q, h_kv=h_kv, d=d, budget=16,
                         keys="grid", slots="perm")
    run_and_check(spec, seed=h_i * 7 + d)


@pytest.mark.parametrize("k", [1, 2, 63, 64, 65, 512, 1024])
def test_budgets(k):
    lens = [4 * k - 1, 4 * k, 4 * k + 3, 4 * k + 4, 4 * k + 5, 9000]
    spec = inputs.custom("budget", lens, h_i=4, d_i=32, h_q=2, h_kv=1, d=64, budget=k,
                         keys="grid", slots="perm")
    run_and_check(spec, seed=k)


def test_all_scores_tied_streaming_path():
    """A zero index query makes every score +0: more candidates than LDS holds,
    so the streaming path runs and must keep groups 0..k-1 (reached through
    each candidate pass: 1,024 segments all at the threshold, 5,000 segments
    -- too many to list -- and the full scan)."""
    spec = inputs.custom("ties", [20000, 70001, 513, 65536, 80000], h_i=4, d_i=32, h_q=1,
                         h_kv=1, d=64, keys="zero_query")
    case = run_and_check(spec)
    ids = case.token_ids.cpu().numpy()
    assert np.array_equal(ids[0, :2048], np.arange(2048))


def test_rows_longer_than_the_staged_maxima():
    """More than 4,096 segment maxima (G > 65,536 groups): the selection
    folds the maxima up to 8:1 and scans the whole row; a zero query on a
    long row streams every key (all tied)."""
    spec = inputs.custom("long", [600001, 300000], h_i=4, d_i=32, h_q=2, h_kv=1, d=64,
                         keys="normal", slots="perm")
    run_and_check(spec, seed=31)
    spec = inputs.custom("long_ties", [400003], h_i=4, d_i=32, h_q=1, h_kv=1, d=64,
                         keys="zero_query")
    case = run_and_check(spec, seed=32)
    assert np.array_equal(case.token_ids[0, :2048].cpu().numpy(), np.arange(2048))


def test_tie_heavy_grid_duplicates():
    spec = inputs.custom("dups", [30000, 12345], h_i=8, d_i=64, h_q=8, h_kv=1, d=128,
                         keys="grid_dup", slots="perm")
    run_and_check(spec, seed=5)


def test_rows_in_flight_passes_are_identical():
    spec = inputs.custom("passes", [5000, 9000, 2055, 7, 12000], h_i=4, d_i=64, h_q=4, h_kv=2,
                         d=128, keys="normal", slots="perm")
    data = inputs.make(spec, seed=9, device="cpu")
    a = harness.GpuCase(data)
    a.decode()
    b = harness.GpuCase(data, rows_in_flight=2)
    b.decode()
    torch.cuda.synchronize()
    assert torch.equal(a.token_ids, b.token_ids) and torch.equal(a.out, b.out)
    assert b.workspace.numel() < a.workspace.numel()
    check_rows(b)


def test_chunk_rows_match_oracle():
    """Several causal query rows per sequence: row j sees seq_len - Q + 1 + j
    tokens and has its own selection."""
    spec = inputs.custom("chunk", [2100, 5000], queries=8, h_i=4, d_i=64, h_q=4, h_kv=1, d=64,
                         budget=64, keys="grid", slots="perm")
    run_and_check(spec, seed=11)


def test_invalid_rows_are_flagged_not_faulted():
    spec = inputs.custom("bad", [9000, 100], h_i=4, d_i=32, h_q=1, h_kv=1, d=64)
    data = inputs.make(spec, seed=2, device="cpu")
    case = harness.GpuCase(data)
    case.seq_len[0] = 4 * case.shape.max_groups + 4  # more groups than max_groups
    case.decode()
    torch.cuda.synchronize()
    assert int(case.width[0]) == -1
    assert torch.all(case.token_ids[0] == -1)
    assert torch.isnan(case.out[0]).all()
    check_rows(case, rows=[1])


def test_out_of_range_slots_give_nan_rows():
    spec = inputs.custom("slots", [300], h_i=4, d_i=32, h_q=1, h_kv=1, d=64)
    data = inputs.make(spec, seed=3, device="cpu")
    case = harness.GpuCase(data)
    case.slot_map[5] = case.shape.kv_slots + 3
    case.decode()
    torch.cuda.synchronize()
    sh = case.shape
    kc = torch.zeros((1, 1, sh.token_stride, 64), device="cuda")
    vc = torch.zeros_like(kc)
    phys = torch.zeros((1, sh.token_stride), dtype=torch.int32, device="cuda")
    qsa.qsa_resolve_gather(sh, case.token_ids, case.width, case.seq_len, case.slot_map,
                           case.slot_off, case.k_cache, case.v_cache, kc, vc, phys)
    assert int(phys[0, 5]) == -1 and torch.isnan(kc[0, 0, 5]).all()
    assert torch.isnan(case.out[0]).all()


# ---------------------------------------------------------- fused gather

def _fused_copy(case):
    fused = harness.GpuCase(case.data, rows_in_flight=case.shape.rows_in_flight)
    fused.decode(fused=True)
    torch.cuda.synchronize()
    return fused


def test_fused_equals_compact(named):
    """Fusing the gather into the attention reads the same rows in the same
    order: identical bits (AFN-016 §Why compact gather comes before fusion)."""
    fused = _fused_copy(named)
    assert torch.equal(fused.token_ids, named.token_ids)
    assert torch.equal(fused.width, named.width)
    assert torch.equal(fused.out, named.out) and torch.equal(fused.lse, named.lse)


@pytest.mark.parametrize("h_i,d_i,h_q,h_kv,d", [(1, 32, 2, 2, 64), (4, 128, 16, 1, 64),
                                                (16, 32, 16, 16, 128), (2, 64, 8, 1, 64),
                                                (8, 32, 4, 2, 128)])
def test_fused_ragged_shapes(h_i, d_i, h_q, h_kv, d):
    lens = [0, 3, 63, 64, 65, 257, 1000, 4097]
    spec = inputs.custom("ragged_f", lens, h_i=h_i, d_i=d_i, h_q=h_q, h_kv=h_kv, d=d, budget=16,
                         keys="grid", slots="perm")
    data = inputs.make(spec, seed=h_i * 5 + d, device="cpu")
    case = harness.GpuCase(data)
    case.decode()
    fused = _fused_copy(case)
    assert torch.equal(fused.token_ids, case.token_ids)
    assert torch.equal(fused.out, case.out) and torch.equal(fused.lse, case.lse)


def test_fused_out_of_range_slot_gives_nan():
    spec = inputs.custom("slots_f", [300, 700], h_i=4, d_i=32, h_q=2, h_kv=1, d=64)
    data = inputs.make(spec, seed=3, device="cpu")
    case = harness.GpuCase(data)
    case.slot_map[5] = case.shape.kv_slots + 3
    case.decode(fused=True)
    torch.cuda.synchronize()
    assert torch.isnan(case.out[0]).all()
    check_rows(case, rows=[1])


def test_fused_chunk_rows_equal_compact():
    spec = inputs.custom("chunk_f", [2100, 9000], queries=16, h_i=16, d_i=64, h_q=8, h_kv=2,
                         d=128, budget=512, keys="normal", slots="perm")
    data = inputs.make(spec, seed=12, device="cpu")
    case = harness.GpuCase(data)
    case.decode()
    fused = _fused_copy(case)
    assert torch.equal(fused.token_ids, case.token_ids)
    assert torch.equal(fused.out, case.out) and torch.equal(fused.lse, case.lse)


# ------------------------------------------------------------ dense GPU row

def test_dense_gpu_row_equals_sparse_below_budget():
    """At or below the budget the sparse GPU row and the bounded dense GPU row
    are the same row in the same order, so their outputs are equal bit for
    bit; one group past the cut the dense row is refused (width -1)."""
    lens = inputs.sweep_prefixes()
    spec = inputs.custom("dense", lens, h_i=4, d_i=32, h_q=4, h_kv=2, d=128, keys="grid",
                         slots="perm")
    data = inputs.make(spec, seed=8, device="cpu")
    case = harness.GpuCase(data)
    case.decode()
    ids = torch.empty_like(case.token_ids)
    width = torch.empty_like(case.width)
    out = torch.empty_like(case.out)
    lse = torch.empty_like(case.lse)
    qsa.qsa_dense_attend(case.shape, case.seq_len, case.slot_map, case.slot_off, case.k_cache,
                         case.v_cache, case.q, case.scale, ids, width, out, lse, case.workspace)
    torch.cuda.synchronize()
    for r, n in enumerate(lens):
        if n <= 2051:
            assert int(width[r]) == n
            assert torch.equal(ids[r], case.token_ids[r])
            assert torch.equal(out[r], case.out[r]) and torch.equal(lse[r], case.lse[r])
        else:
            assert int(width[r]) == -1 and torch.isnan(out[r]).all()
    # and the dense rows against the oracle's dense row
    for r, n in enumerate(lens):
        if 0 < n <= 2051:
            dense = oracle.dense_row(n, data["slot_map"].numpy()[int(data["raw_off"][r]):],
                                     data["kv_slots"], data["k_cache"].numpy(),
                                     data["v_cache"].numpy(), data["q"][r].numpy(), case.scale)
            kx, vx = oracle.gather(oracle.resolve(dense["ids"],
                                                  data["slot_map"].numpy()[int(data["raw_off"][r]):],
                                                  data["kv_slots"]),
                                   data["k_cache"].numpy(), data["v_cache"].numpy())
            ex, _ = oracle.attend_exact(data["q"][r].numpy(), kx, vx, case.scale)
            assert harness.normwise_rel_err(out[r].cpu().numpy(), ex) <= 2e-6
