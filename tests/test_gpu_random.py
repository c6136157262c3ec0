"""Seeded random shapes: each case draws its own indexer and attention shapes,
budget, key distribution, slot map, batch of sequence lengths (edge lengths
around 0-5 and the budget, and random lengths up to 80,000 tokens) and, for
index shapes the chunk scoring covers, causal chunk rows.  Every row must
match the oracle (selected IDs, widths bit-exact; attention within 2e-6 of
the exact attention over the oracle's rows), and the fused and union
variants must equal the compact one bit for bit.

Sources: AFN-017 "Top-k chooses the set; time chooses the order" and AFN-016
"A sparse mask is not sparse attention".
"""
import numpy as np
import pytest
import torch

from tests import harness, inputs
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
    for rows in ("fused", "dedup"):
        case.decode(rows=rows)
        torch.cuda.synchronize()
        for a, b in zip(case.results(), ref):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                               b.view(torch.int32) if b.dtype == torch.float32 else b), \
                (spec.name, rows)
