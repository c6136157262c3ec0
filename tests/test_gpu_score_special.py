"""Group scores on special values, bit for bit against the oracle's chain.

Step 1 fixes each head's dot product as a chain of fused multiply-adds over
the dimensions in ascending order, then ReLU, then the head sum (AFN-016 "A
sparse mask is not sparse attention", §Decision and §Why a sparse mask can
still be dense).  The scoring kernels must reproduce that chain exactly:
with 4, 8 or 16 index heads on the matrix cores, with 1 or 2 on the VALU.
These cases push the arithmetic where roundings differ first:
  denormal keys, denormal products and denormal partial sums;
  products and sums that overflow to infinity (and infinities that cancel
  into NaN, which ReLU maps to 0);
  signed zeros (a chain of -0 products from +0 stays +0);
  exact cancellation of large terms, leaving sums of small ones;
  wide exponent ranges mixed in one dot product.
Every index-head count and index dimension is covered.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import top_sparse_attention_qsa_amd as qsa
from tests import harness, inputs

pytestmark = pytest.mark.gpu

LENS = [2055, 700]  # 513 and 175 complete groups: full tiles and a ragged tail


def _special(kind, rng, shape):
    """float32 array of `shape` for one value family."""
    if kind == "denormal_keys":
        return (rng.standard_normal(shape) * 1e-39).astype(np.float32)
    if kind == "denormal_products":
        return (rng.standard_normal(shape) * 1e-21).astype(np.float32)
    if kind == "overflow":
        # products near 1e37, a few single products past the float range:
        # some dot products and head sums stay finite, some overflow to
        # +-inf, some add +inf to -inf (NaN, which ReLU maps to 0)
        a = rng.standard_normal(shape) * 3e18
        a[rng.random(shape) < 0.03] *= 10.0
        return a.astype(np.float32)
    if kind == "signed_zero":
        a = rng.standard_normal(shape).astype(np.float32)
        a[rng.random(shape) < 0.7] = np.float32(-0.0)
        return a
    if kind == "cancel":
        # pairs of equal large values of opposite sign plus small terms
        a = (rng.standard_normal(shape) * 1e-3).astype(np.float32)
        big = np.float32(2.0 ** 20)
        a[..., 0::4] += big
        a[..., 1::4] -= big
        return a
    if kind == "wide_exponent":
        return (rng.standard_normal(shape) * 2.0 ** rng.integers(-60, 60, shape)).astype(np.float32)
    raise ValueError(kind)


KINDS = ["denormal_keys", "denormal_products", "overflow", "signed_zero", "cancel",
         "wide_exponent"]


@pytest.mark.parametrize("d_i", [32, 64, 128])
@pytest.mark.parametrize("h_i", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("kind", KINDS)
def test_scores_on_special_values_bitexact(kind, h_i, d_i):
    spec = inputs.custom(f"special_{kind}_{h_i}x{d_i}", LENS, h_i=h_i, d_i=d_i, h_q=1, h_kv=1,
                         d=64, keys="normal")
    data = inputs.make(spec, seed=3, device="cpu")
    rng = np.random.default_rng(zlib.crc32(f"{kind} {h_i} {d_i}".encode()))
    raw = _special(kind, rng, tuple(data["raw_keys"].shape))
    # the queries of the product families are tiny or large too, so their
    # products (not only the keys) reach the edges
    if kind in ("denormal_products", "overflow"):
        iq = _special(kind, rng, tuple(data["index_q"].shape))
    else:
        iq = rng.standard_normal(tuple(data["index_q"].shape)).astype(np.float32)
    data["raw_keys"] = torch.from_numpy(raw)
    data["index_q"] = torch.from_numpy(iq)
    case = harness.GpuCase(data)
    scores = torch.full((spec.rows, case.shape.max_groups), -1.0, device="cuda")
    qsa.qsa_score_groups(case.shape, case.index_q, case.pooled, case.pooled_off, case.seq_len,
                         scores)
    got = scores.cpu().numpy()
    for r in range(spec.rows):
        n = inputs.row_tokens(spec, r)
        off = int(data["raw_off"][r // spec.queries])
        pooled = oracle.pool_full(raw[off:off + n])
        want = oracle.score(iq[r], pooled)
        assert np.array_equal(got[r, :len(want)].view(np.uint32), want.view(np.uint32)), (
            kind, h_i, d_i, r,
            int(np.sum(got[r, :len(want)].view(np.uint32) != want.view(np.uint32))))
        assert np.all(got[r, len(want):] == -1.0)  # untouched past G
