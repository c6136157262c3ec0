"""Seeded random shapes: each case draws its own indexer and attention shapes,
budget, key distribution, slot map, batch of sequence lengths (edge lengths
around 0-5 and the budget, and random lengths up to 80,000 tokens) and, for
index shapes the chunk scoring covers, causal chunk rows.  Every row must
match the oracle (selected IDs, widths bit-exact; attention within 2e-6 of
the exact attention over the oracle's rows), the fused and union variants
must equal the compact one bit for bit, and the bounded dense row must equal
the sparse one wherever the row fits the budget; causal-chunk rows must
equal one decode per row bit for bit.

Sources: AFN-017 "Top-k chooses the set; time chooses the order" and AFN-016
"A sparse mask is not sparse attention".
"""
import numpy as np
import pytest
import torch

import top_sparse_attention_qsa_amd as qsa
from tests import harness, inputs
from tests.test_gpu_chunk import assert_same, decode_per_row
from tests.test_gpu_parity import check_rows

pytestmark = pytest.mark.gpu

CASES = 80


def random_spec(i):
    rng = np.random.default_rng(9000 + i)
    h_i = int(rng.choice([1, 2, 4, 8, 16]))
    d_i = int(rng.choice([32, 64, 128]))
    d = int(rng.choice([64, 128]))
    h_kv = int(rng.choice([1, 2, 4]))
    h_q = h_kv * int(rng.choice([1, 2, 4, 8, 16]))
    budget = int(rng.choice([1, 7, 64, 128, 333, 512, 700]))
    keys = str(rng.choice(["normal", "grid", "grid_dup"]))
    queries = 1
    if h_i in (4, 8, 16) and rng.random() < 0.35:
        queries = 4 * (16 // h_i) * int(rng.choice([1, 2]))  # whole chunk-scoring blocks
    batch = int(rng.integers(1, 6))
    edge = [0, 1, 2, 3, 4, 5, 4 * budget - 1, 4 * budget, 4 * budget + 3, 4 * budget + 4,
            4 * budget + 5]
    lens = []
    for _ in range(batch):
        n = int(rng.choice(edge)) if rng.random() < 0.3 else int(rng.integers(1, 80000))
        lens.append(max(n, queries - 1))  # every row sees at least 0 tokens
    kw = dict(queries=queries, h_i=h_i, d_i=d_i, h_q=h_q, h_kv=h_kv, d=d, budget=budget,
              keys=keys)
    if batch == 1 and rng.random() < 0.5:
        kw.update(slots="ring", capacity=lens[0] + int(rng.integers(1, 5000)))
    else:
        kw.update(slots="perm")
    return inputs.custom(f"random_{i}", lens, **kw)


@pytest.mark.parametrize("i", range(CASES))
def test_random_shape_matches_oracle_and_variants_agree(i):
    spec = random_spec(i)
    print(f"case {i}: {spec}", flush=True)
    data = inputs.make(spec, seed=100 + i, device="cpu")
    case = harness.GpuCase(data)
    case.decode()
    check_rows(case)
    ref = case.results()
    # the bounded dense row: the same row as the sparse one at or below the
    # budget (N <= 4k+3), refused above it
    ids = torch.empty_like(case.token_ids)
    width = torch.empty_like(case.width)
    out = torch.empty_like(case.out)
    lse = torch.empty_like(case.lse)
    qsa.qsa_dense_attend(case.shape, case.seq_len, case.slot_map, case.slot_off, case.k_cache,
                         case.v_cache, case.q, case.scale, ids, width, out, lse, case.workspace)
    torch.cuda.synchronize()
    for r in range(spec.rows):
        n = inputs.row_tokens(spec, r)
        if n <= 4 * spec.budget + 3:
            assert int(width[r]) == n and torch.equal(ids[r], ref[0][r]), (spec.name, r)
            assert torch.equal(out[r].view(torch.int32), ref[2][r].view(torch.int32))
            assert torch.equal(lse[r].view(torch.int32), ref[3][r].view(torch.int32))
        else:
            assert int(width[r]) == -1 and torch.isnan(out[r]).all(), (spec.name, r)
    if spec.queries > 1:
        # causal-chunk rows equal one decode per row, bit for bit
        assert_same(case, decode_per_row(case))
    for rows in ("fused", "dedup"):
        case.decode(rows=rows)
        torch.cuda.synchronize()
        for a, b in zip(case.results(), ref):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                               b.view(torch.int32) if b.dtype == torch.float32 else b), \
                (spec.name, rows)


def bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


@pytest.mark.parametrize("i", range(0, CASES, 2))
def test_random_shape_step_by_step(i):
    """The per-step entry points on the same random shapes: scores bit-exact
    against the oracle; select + emit give the decode's IDs and widths (for
    causal-chunk rows that is the exact selection against the certified one);
    the gather copies the oracle's rows bit for bit; the standalone attention
    equals the decode's output; NaN in every unselected cache row changes
    nothing."""
    import oracle
    spec = random_spec(i)
    print(f"case {i}: {spec}", flush=True)
    data = inputs.make(spec, seed=100 + i, device="cpu")
    case = harness.GpuCase(data)
    case.decode()
    torch.cuda.synchronize()
    sh = case.shape
    s = spec

    scores = torch.full((s.rows, sh.max_groups), -1.0, device="cuda")
    qsa.qsa_score_groups(sh, case.index_q, case.pooled, case.pooled_off, case.seq_len, scores)
    bitmap = torch.full((s.rows, sh.max_groups // 32), -1, dtype=torch.int32, device="cuda")
    qsa.qsa_select_topk(sh, scores, case.seq_len, bitmap, case.workspace)
    ids = torch.empty_like(case.token_ids)
    width = torch.empty_like(case.width)
    qsa.qsa_emit_chronological(sh, bitmap, case.seq_len, ids, width)
    assert torch.equal(ids, case.token_ids) and torch.equal(width, case.width)

    kc = torch.full((s.rows, s.h_kv, sh.token_stride, s.d), 7.0, device="cuda")
    vc = torch.full_like(kc, 7.0)
    qsa.qsa_resolve_gather(sh, case.token_ids, case.width, case.seq_len, case.slot_map,
                           case.slot_off, case.k_cache, case.v_cache, kc, vc)
    out = torch.empty_like(case.out)
    lse = torch.empty_like(case.lse)
    qsa.qsa_online_attend(sh, case.q, kc, vc, case.width, case.scale, out, lse, case.workspace)
    assert torch.equal(out, case.out) and torch.equal(lse, case.lse)

    got_scores = scores.cpu().numpy()
    kc, vc = kc.cpu().numpy(), vc.cpu().numpy()
    keep = torch.zeros(data["kv_slots"], dtype=torch.bool)
    for r in range(s.rows):
        exp = harness.oracle_row(data, r, exact=False)
        n = exp["n"]
        b = r // s.queries
        off = int(data["raw_off"][b])
        want = oracle.score(data["index_q"][r].numpy(),
                            oracle.pool_full(data["raw_keys"][off:off + n].numpy()))
        assert np.array_equal(bits(got_scores[r, :len(want)]), bits(want)), (s.name, r)
        w = len(exp["ids"])
        kx = np.ascontiguousarray(kc[r, :, :w].transpose(1, 0, 2))
        vx = np.ascontiguousarray(vc[r, :, :w].transpose(1, 0, 2))
        assert kx.tobytes() == exp["kx"].tobytes() and vx.tobytes() == exp["vx"].tobytes()
        keep[torch.as_tensor(exp["slots"], dtype=torch.int64)] = True

    poisoned = harness.GpuCase(data)
    keep = keep.cuda()
    poisoned.k_cache[~keep] = float("nan")
    poisoned.v_cache[~keep] = float("nan")
    poisoned.decode()
    torch.cuda.synchronize()
    assert torch.equal(poisoned.token_ids, case.token_ids)
    assert torch.equal(poisoned.out.view(torch.int32), case.out.view(torch.int32))


def untile(pooled_flat, off, g, d_i):
    """Tiled pooled-key buffer of one sequence -> plain [G][D_I] (host)."""
    tiles = (g + 63) // 64
    t = pooled_flat[off:off + tiles * 64 * d_i].view(tiles, d_i // 4, 64, 4)
    return t.permute(0, 2, 1, 3).reshape(tiles * 64, d_i)[:g].cpu().numpy()


@pytest.mark.parametrize("i", range(1, CASES, 2))
def test_random_shape_pooling(i):
    """Group pooling on the random shapes: every sequence's pooled keys are the
    oracle's bit for bit, and pooling in random increments (each call pools
    only the groups completed since the previous one, every sequence on its
    own schedule) gives the same bits as pooling the whole history."""
    import oracle
    spec = random_spec(i)
    print(f"case {i}: {spec}", flush=True)
    data = inputs.make(spec, seed=100 + i, device="cpu")
    case = harness.GpuCase(data)
    torch.cuda.synchronize()
    s = spec
    for b in range(s.batch):
        g = s.seq_lens[b] // 4
        off = int(data["raw_off"][b])
        want = oracle.pool_full(data["raw_keys"][off:off + s.seq_lens[b]].numpy())
        got = untile(case.pooled, int(case.pooled_off[b]), g, s.d_i)
        assert np.array_equal(bits(got), bits(want)), (s.name, b)

    rng = np.random.default_rng(700 + i)
    raw = data["raw_keys"].cuda()
    pooled = torch.full_like(case.pooled, float("nan"))
    done = [0] * s.batch   # tokens pooled so far per sequence
    while any(d < n for d, n in zip(done, s.seq_lens)):
        nxt = [min(n, d + int(rng.integers(0, 9000))) for d, n in zip(done, s.seq_lens)]
        if rng.random() < 0.3:
            nxt = [d + 1 if d < n else d for d, n in zip(done, s.seq_lens)]  # one token
        seq = torch.tensor(nxt, dtype=torch.int32, device="cuda")
        first = torch.tensor([d // 4 for d in done], dtype=torch.int32, device="cuda")
        qsa.qsa_pool_groups(case.shape, raw, case.raw_off, seq, first, pooled, case.pooled_off)
        done = nxt
    torch.cuda.synchronize()
    for b in range(s.batch):
        g = s.seq_lens[b] // 4
        a = untile(pooled, int(case.pooled_off[b]), g, s.d_i)
        c = untile(case.pooled, int(case.pooled_off[b]), g, s.d_i)
        assert np.array_equal(bits(a), bits(c)), (s.name, b)
