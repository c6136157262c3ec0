"""Pins for the CPU oracle: closed forms, brute force, special cases and the
double-precision definition -- never the oracle's own formula retyped.

Sources: AFN-017 "Top-k chooses the set; time chooses the order" and AFN-016
"A sparse mask is not sparse attention" (Hebrus notes).
"""
import numpy as np
import pytest
import torch

import oracle
from tests import inputs
from tests.golden_io import load

U = 2.0 ** -24  # unit roundoff of IEEE single


def gamma(n):
    return n * U / (1 - n * U)


def grid(rng, shape):
    return rng.integers(-2, 3, size=shape).astype(np.float32) / 8.0


# ------------------------------------------------------------------ pooling

def test_pool_grid_is_exact_integer_mean():
    rng = np.random.default_rng(11)
    for n in (0, 3, 4, 7, 8, 2055):
        raw = grid(rng, (n, 32))
        pooled = oracle.pool_full(raw)
        ints = (raw * 8).astype(np.int64)
        g = n // 4
        want = ints[:4 * g].reshape(g, 4, 32).sum(axis=1)  # 32 * mean, exactly
        assert pooled.shape == (g, 32)
        assert np.array_equal((pooled.astype(np.float64) * 32).astype(np.int64), want)
        assert np.all(pooled.astype(np.float64) * 32 == want)


def test_pool_full_equals_incremental_bitwise():
    rng = np.random.default_rng(12)
    for n in (0, 1, 4, 5, 9, 2055, 4099):
        raw = rng.standard_normal((n, 64)).astype(np.float32)
        a = oracle.pool_full(raw)
        b = oracle.pool_incremental(raw)
        assert a.tobytes() == b.tobytes()


def test_pool_normal_matches_float64_mean_within_rounding():
    rng = np.random.default_rng(13)
    raw = rng.standard_normal((4 * 500, 16)).astype(np.float32)
    pooled = oracle.pool_full(raw).astype(np.float64)
    r = raw.astype(np.float64).reshape(500, 4, 16)
    exact = r.mean(axis=1)
    bound = gamma(3) * np.abs(r).sum(axis=1) * 0.25
    assert np.all(np.abs(pooled - exact) <= bound + 1e-300)


def test_pool_golden():
    f = load("score_worked.txt")
    d = int(f["d_i"])
    raw = np.array(f["raw"], np.float32).reshape(-1, d)
    pooled = oracle.pool_full(raw)
    assert np.array_equal(pooled, np.array(f["pooled"], np.float32).reshape(-1, d))


# ------------------------------------------------------------------ scoring

def test_score_golden():
    f = load("score_worked.txt")
    d, h = int(f["d_i"]), int(f["h_i"])
    pooled = np.array(f["pooled"], np.float32).reshape(-1, d)
    qi = np.array(f["qi"], np.float32).reshape(h, d)
    assert np.array_equal(oracle.score(qi, pooled), np.array(f["scores"], np.float32))


@pytest.mark.parametrize("h_i,d_i", [(4, 32), (8, 64), (16, 128)])
def test_score_grid_is_exact(h_i, d_i):
    """Grid keys/queries: 256*score is an integer recomputed exactly in int64."""
    rng = np.random.default_rng(21 + h_i)
    raw = grid(rng, (4 * 700, d_i))
    pooled = oracle.pool_full(raw)
    qi = grid(rng, (h_i, d_i))
    s = oracle.score(qi, pooled)
    q8 = (qi * 8).astype(np.int64)                    # integers in [-2, 2]
    k32 = (pooled.astype(np.float64) * 32).astype(np.int64)  # integers in [-8, 8]
    dots = k32 @ q8.T                                 # [G][H] = 256 * dot
    want = np.maximum(dots, 0).sum(axis=1)            # 256 * score
    assert np.array_equal((s.astype(np.float64) * 256), want.astype(np.float64))


@pytest.mark.parametrize("h_i,d_i", [(8, 64), (16, 128)])
def test_score_normal_within_closed_form_bound(h_i, d_i):
    rng = np.random.default_rng(31 + h_i)
    pooled = rng.standard_normal((3000, d_i)).astype(np.float32)
    qi = rng.standard_normal((h_i, d_i)).astype(np.float32)
    s = oracle.score(qi, pooled).astype(np.float64)
    q64, k64 = qi.astype(np.float64), pooled.astype(np.float64)
    dots = k64 @ q64.T
    exact = np.maximum(dots, 0).sum(axis=1)
    a_abs = np.abs(k64) @ np.abs(q64).T               # sum_d |q k| per head
    bound = gamma(d_i) * a_abs.sum(axis=1) + gamma(h_i) * (exact + gamma(d_i) * a_abs.sum(axis=1))
    err = np.abs(s - exact)
    assert np.all(err <= bound)
    # the bound is not vacuous: a dropped head or term would break it by far
    assert np.median(bound / np.maximum(exact, 1e-30)) < 1e-3


def test_score_has_no_negative_zero_or_nan():
    rng = np.random.default_rng(41)
    pooled = rng.standard_normal((500, 32)).astype(np.float32)
    qi = -np.abs(rng.standard_normal((4, 32)).astype(np.float32))
    pooled = np.abs(pooled)                           # every dot negative
    s = oracle.score(qi, pooled)
    assert np.all(s.view(np.uint32) == 0)             # +0.0 exactly


# ---------------------------------------------------------------- selection

def rank_count_select(scores, k):
    """Independent definition: g is chosen iff fewer than k groups precede it
    in (score desc, position asc) order -- counted pairwise, O(G^2)."""
    s = np.asarray(scores, np.float64)
    g = s.shape[0]
    better = (s[None, :] > s[:, None]) | ((s[None, :] == s[:, None]) &
                                          (np.arange(g)[None, :] < np.arange(g)[:, None]))
    rank = better.sum(axis=1)
    chosen = np.nonzero(rank < k)[0]
    return chosen[np.argsort(rank[chosen])]


def test_select_matches_rank_count_bruteforce():
    rng = np.random.default_rng(51)
    for trial in range(10000):
        g = int(rng.integers(0, 65))
        k = int(rng.integers(1, 17))
        levels = int(rng.integers(1, 6))
        scores = (rng.integers(0, levels, size=g) / 4.0).astype(np.float32)
        got = oracle.select(scores, k)
        want = rank_count_select(scores, k)
        assert np.array_equal(got, want), (trial, g, k, scores)


def test_select_special_cases():
    # all equal: the first k positions
    assert np.array_equal(np.sort(oracle.select(np.ones(100, np.float32), 7)), np.arange(7))
    # at or below budget: everything
    s = np.random.default_rng(1).random(40).astype(np.float32)
    assert np.array_equal(np.sort(oracle.select(s, 40)), np.arange(40))
    assert np.array_equal(np.sort(oracle.select(s, 512)), np.arange(40))
    # k distinct high scores plus a tied block at the threshold
    s = np.zeros(50, np.float32)
    s[[3, 30, 44]] = 9.0
    s[[5, 10, 20, 40]] = 4.0                           # tied block, 2 places left
    assert np.array_equal(np.sort(oracle.select(s, 5)), [3, 5, 10, 30, 44])
    # -0 and +0 are equal scores: position decides
    s = np.array([0.0, -0.0, 0.0], np.float32)
    s[0] = -0.0
    assert np.array_equal(oracle.select(s, 2), [0, 1])
    assert oracle.select(np.zeros(0, np.float32), 4).shape == (0,)


def _mutant_select_tie_after_sort(scores, k):
    # planted mistake: ties broken by LARGER position (recovered later)
    order = sorted(range(len(scores)), key=lambda g: (-scores[g], -g))
    return np.array(order[:k])


def _mutant_emit_rank_order(chosen, n_tokens):
    # planted mistake: rank order used as emission order
    ids = [4 * g + j for g in chosen for j in range(4)]
    ids += list(range(4 * (n_tokens // 4), n_tokens))
    return np.array(ids, np.int32)


def test_selection_and_emission_golden_and_mutants():
    f = load("tie_membership.txt")
    scores = np.array(f["scores"], np.float32)
    k, n = int(f["k"]), int(f["n_tokens"])
    chosen = oracle.select(scores, k)
    assert np.array_equal(chosen, np.array(f["rank_order"], np.int64))
    ids = oracle.emit(chosen, n)
    assert np.array_equal(ids, np.array(f["ids"], np.int32))
    assert ids.shape[0] == int(f["width"])
    # the same checks catch both mistakes the notes warn about
    assert not np.array_equal(np.sort(_mutant_select_tie_after_sort(scores, k)),
                              np.array(f["chosen_chronological"]))
    assert not np.array_equal(_mutant_emit_rank_order(chosen, n), ids)


# ----------------------------------------------------------------- emission

def check_row_shape(ids, chosen, n_tokens):
    g = n_tokens // 4
    tail = n_tokens % 4
    m = len(chosen)
    assert ids.shape[0] == 4 * m + tail
    assert np.all(np.diff(ids) > 0)                    # strictly chronological
    body = ids[:4 * m].reshape(m, 4)
    assert np.all(body[:, 0] % 4 == 0)                 # group-aligned runs of four
    assert np.all(body - body[:, :1] == np.arange(4))  # contiguous
    assert np.array_equal(body[:, 0] // 4, np.sort(chosen))
    assert np.array_equal(ids[4 * m:], np.arange(4 * g, n_tokens))  # raw tail last


def test_emit_closed_form_random():
    rng = np.random.default_rng(61)
    for _ in range(500):
        n = int(rng.integers(0, 400))
        g = n // 4
        k = int(rng.integers(1, 40))
        scores = rng.standard_normal(g).astype(np.float32)
        chosen = oracle.select(scores, k)
        ids = oracle.emit(chosen, n)
        check_row_shape(ids, chosen, n)


@pytest.mark.parametrize("n", inputs.sweep_prefixes())
def test_dense_parity_sweep_ids(n):
    """Below the cut every group is kept and the row is the dense causal row."""
    rng = np.random.default_rng(71)
    scores = rng.standard_normal(n // 4).astype(np.float32)
    ids = oracle.emit(oracle.select(scores, 512), n)
    if n <= 4 * 512 + 3:
        assert np.array_equal(ids, np.arange(n, dtype=np.int32))
    else:
        assert ids.shape[0] == 2048 and not np.array_equal(ids, np.arange(2048))


# --------------------------------------------------------- resolve / gather

def test_resolve_closed_forms():
    n = 1000
    ids = np.arange(0, n, 3, dtype=np.int32)
    assert np.array_equal(oracle.resolve(ids, np.arange(n, dtype=np.int32), n), ids)
    cap, off = 1200, 777
    ring = ((np.arange(n) + off) % cap).astype(np.int32)
    assert np.array_equal(oracle.resolve(ids, ring, cap), (ids + off) % cap)
    perm = np.random.default_rng(3).permutation(n).astype(np.int32)
    slots = oracle.resolve(ids, perm, n)
    inv = np.empty(n, np.int32)
    inv[perm] = np.arange(n)
    assert np.array_equal(inv[slots], ids)
    with pytest.raises(IndexError):
        oracle.resolve(np.array([n], np.int32), perm, n)
    with pytest.raises(IndexError):
        oracle.resolve(np.array([0], np.int32), np.array([cap], np.int32), cap)


def test_gather_is_direct_indexing():
    rng = np.random.default_rng(81)
    kc = rng.standard_normal((300, 2, 8)).astype(np.float32)
    vc = rng.standard_normal((300, 2, 8)).astype(np.float32)
    slots = rng.integers(0, 300, 57).astype(np.int32)
    kx, vx = oracle.gather(slots, kc, vc)
    assert kx.tobytes() == kc[slots].tobytes() and vx.tobytes() == vc[slots].tobytes()


# ---------------------------------------------------------------- attention

def softmax_ref(q, kx, vx, scale):
    """Library-routine reference: numpy float64 softmax-weighted sum."""
    h_q, d = q.shape
    h_kv = kx.shape[1]
    grp = h_q // h_kv
    out = np.empty((h_q, d))
    lse = np.empty(h_q)
    for hq in range(h_q):
        s = kx[:, hq // grp, :].astype(np.float64) @ q[hq].astype(np.float64) * scale
        m = s.max()
        e = np.exp(s - m)
        out[hq] = e @ vx[:, hq // grp, :].astype(np.float64) / e.sum()
        lse[hq] = m + np.log(e.sum())
    return out, lse


def test_attend_golden():
    f = load("attend_worked.txt")
    q = np.array(f["q"], np.float32).reshape(1, 2)
    kx = np.array(f["k"], np.float32).reshape(-1, 1, 2)
    vx = np.array(f["v"], np.float32).reshape(-1, 1, 2)
    out, lse = oracle.attend_online(q, kx, vx, f["scale"])
    assert np.array_equal(out[0], np.array(f["out"], np.float32))
    assert abs(np.exp(np.float64(lse[0])) - f["lse_exp"]) < 1e-6
    oe, le = oracle.attend_exact(q, kx, vx, f["scale"])
    assert np.allclose(oe[0], f["out"], rtol=0, atol=1e-15)


def test_attend_exact_matches_numpy_definition():
    rng = np.random.default_rng(91)
    for w, h_q, h_kv, d in [(1, 1, 1, 8), (37, 4, 2, 16), (700, 8, 1, 64), (2051, 2, 2, 128)]:
        q = rng.standard_normal((h_q, d)).astype(np.float32)
        kx = rng.standard_normal((w, h_kv, d)).astype(np.float32)
        vx = rng.standard_normal((w, h_kv, d)).astype(np.float32)
        scale = float(np.float32(1 / np.sqrt(d)))
        out, lse = oracle.attend_exact(q, kx, vx, scale)
        ro, rl = softmax_ref(q, kx, vx, scale)
        assert np.allclose(out, ro, rtol=1e-12, atol=1e-13)
        assert np.allclose(lse, rl, rtol=1e-12, atol=1e-12)


def test_attend_online_special_cases():
    rng = np.random.default_rng(92)
    # one row: the output is that V row, bit for bit
    q = rng.standard_normal((3, 16)).astype(np.float32)
    kx = rng.standard_normal((1, 3, 16)).astype(np.float32)
    vx = rng.standard_normal((1, 3, 16)).astype(np.float32)
    out, _ = oracle.attend_online(q, kx, vx, 0.25)
    assert np.array_equal(out, vx[0])
    # identical keys: the mean of the V rows (up to summation rounding)
    w = 333
    kx = np.repeat(rng.standard_normal((1, 1, 16)).astype(np.float32), w, axis=0)
    vx = rng.standard_normal((w, 1, 16)).astype(np.float32)
    out, lse = oracle.attend_online(q[:1], kx, vx, 0.25)
    mean = vx[:, 0, :].astype(np.float64).mean(axis=0)
    bound = gamma(w + 2) * np.abs(vx[:, 0, :]).astype(np.float64).mean(axis=0)
    assert np.all(np.abs(out[0] - mean) <= bound)
    # empty row
    out, lse = oracle.attend_online(q, np.zeros((0, 3, 16), np.float32),
                                    np.zeros((0, 3, 16), np.float32), 0.25)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("w,h_q,h_kv,d", [(5, 1, 1, 64), (2051, 1, 1, 64),
                                          (2048, 8, 1, 128), (2048, 8, 4, 128)])
def test_attend_online_within_bound_of_exact(w, h_q, h_kv, d):
    """Elementwise |o - o_exact| <= gamma_(W+D+8) * sum p|v| / sum p."""
    rng = np.random.default_rng(93 + w)
    q = rng.standard_normal((h_q, d)).astype(np.float32)
    kx = rng.standard_normal((w, h_kv, d)).astype(np.float32)
    vx = rng.standard_normal((w, h_kv, d)).astype(np.float32)
    scale = float(np.float32(1 / np.sqrt(d)))
    out, lse = oracle.attend_online(q, kx, vx, scale)
    ex, lex = oracle.attend_exact(q, kx, vx, scale)
    grp = h_q // h_kv
    for hq in range(h_q):
        s = kx[:, hq // grp, :].astype(np.float64) @ q[hq].astype(np.float64) * scale
        p = np.exp(s - s.max())
        mag = p @ np.abs(vx[:, hq // grp, :]).astype(np.float64) / p.sum()
        assert np.all(np.abs(out[hq] - ex[hq]) <= gamma(w + d + 8) * 8 * mag)
    assert np.allclose(lse, lex, rtol=0, atol=gamma(w + d + 8) * 8 * (np.abs(lex) + 1))


# ------------------------------------------------------ full row invariants

def _tail_row(n_tokens, data):
    raw = data["raw_keys"].numpy()
    pooled = oracle.pool_full(raw[:n_tokens])
    scale = float(np.float32(1 / np.sqrt(64)))
    return oracle.decode_row(data["index_q"][0].numpy(), pooled, n_tokens, 512,
                             data["slot_map"].numpy(), data["kv_slots"],
                             data["k_cache"].numpy(), data["v_cache"].numpy(),
                             data["q"][0].numpy(), scale)


@pytest.mark.parametrize("n", inputs.sweep_prefixes())
def test_dense_parity_sweep_attention(n):
    """At or below budget the sparse row equals the dense causal row, bit for
    bit, attention output included; just past the cut it does not."""
    data = inputs.make(inputs.spec("tail_2055"), seed=1)
    sparse = _tail_row(n, data)
    scale = float(np.float32(1 / np.sqrt(64)))
    dense = oracle.dense_row(n, data["slot_map"].numpy(), data["kv_slots"],
                             data["k_cache"].numpy(), data["v_cache"].numpy(),
                             data["q"][0].numpy(), scale)
    if n <= 2051:
        assert np.array_equal(sparse["ids"], dense["ids"])
        assert sparse["out"].tobytes() == dense["out"].tobytes()
    else:
        assert sparse["width"] == 2048 and dense["width"] == 2052
        # the dropped group is the minimum under (score desc, position asc)
        s = sparse["scores"]
        dropped = sorted(range(len(s)), key=lambda g: (-s[g], g))[-1]
        kept = set(sparse["ids"][::4] // 4)
        assert dropped not in kept and len(kept) == 512


def test_tail_2055_full_row_invariants():
    data = inputs.make(inputs.spec("tail_2055"), seed=2)
    r = _tail_row(2055, data)
    assert r["width"] == 2051                          # 512 groups * 4 + 3 tail
    chosen = r["ids"][:2048:4] // 4
    check_row_shape(r["ids"], chosen, 2055)
    want = rank_count_select(r["scores"], 512)
    assert np.array_equal(np.sort(want), chosen)


def test_chunk_rows_equal_independent_decode_rows():
    """Scoring a causal chunk's queries against the longest history and
    restricting each query to its own complete groups equals scoring each
    query alone (chunk/decode identity, AFN-017 capsule evidence)."""
    s = inputs.custom("chunk", [700], queries=16, h_i=4, d_i=32, h_q=2, h_kv=1, d=64,
                      budget=16, keys="grid")
    data = inputs.make(s, seed=3)
    pooled_all = oracle.pool_full(data["raw_keys"].numpy())
    scale = 0.125
    for j in range(16):
        n = inputs.row_tokens(s, j)
        qi = data["index_q"][j].numpy()
        full_scores = oracle.score(qi, pooled_all)     # one matrix row, all groups
        chunk_sel = oracle.select(full_scores[: n // 4], 16)
        alone = oracle.decode_row(qi, oracle.pool_full(data["raw_keys"].numpy()[:n]), n, 16,
                                  data["slot_map"].numpy(), data["kv_slots"],
                                  data["k_cache"].numpy(), data["v_cache"].numpy(),
                                  data["q"][j].numpy(), scale)
        assert np.array_equal(oracle.emit(chunk_sel, n), alone["ids"])


def test_inputs_are_seeded_and_device_independent_in_shape():
    a = inputs.make(inputs.spec("tail_2055"), seed=5)
    b = inputs.make(inputs.spec("tail_2055"), seed=5)
    for key in ("index_q", "raw_keys", "q", "k_cache", "v_cache", "slot_map"):
        assert torch.equal(a[key], b[key])
    c = inputs.make(inputs.spec("tail_2055"), seed=6)
    assert not torch.equal(a["raw_keys"], c["raw_keys"])
