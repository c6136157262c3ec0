"""The threaded multi-row oracle helper (harness.oracle_rows, used by the
full-size GPU parity tests) gives, row for row, exactly what the per-row
oracle gives (harness.oracle_row): it pools each sequence once and uses the
first N//4 pooled groups of a row with N visible tokens."""
import numpy as np

from tests import harness, inputs


def test_oracle_rows_equals_oracle_row():
    spec = inputs.custom("rows", [2055, 0, 5, 4100, 9001], queries=4, h_i=4, d_i=32, h_q=4,
                         h_kv=2, d=64, budget=64, keys="normal", slots="perm")
    data = inputs.make(spec, seed=7, device="cpu")
    rows = [r for r in range(spec.rows) if inputs.row_tokens(spec, r) >= 0]
    many = harness.oracle_rows(data, rows, threads=3)
    for r, got in zip(rows, many):
        one = harness.oracle_row(data, r)
        assert got["n"] == one["n"]
        assert np.array_equal(got["scores"].view(np.uint32), one["scores"].view(np.uint32))
        assert np.array_equal(got["ids"], one["ids"]) and np.array_equal(got["slots"],
                                                                           one["slots"])
        assert np.array_equal(got["out_exact"], one["out_exact"])
        assert np.array_equal(got["lse_exact"], one["lse_exact"])


def test_elementwise_error_floor():
    ref = np.array([[1.0, 1e-9, -2.0]])
    got = ref + np.array([[1e-7, 1e-9, 0.0]])
    # the near-zero element is measured against 1e-6 * max|ref| = 2e-6
    assert np.isclose(harness.elementwise_rel_err(got, ref), 1e-9 / 2e-6)
    assert np.isclose(harness.normwise_rel_err(got, ref), 1e-7 / 2.0)
