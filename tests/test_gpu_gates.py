"""Non-completion and clean-completion gates on the GPU (AFN-016 "A sparse
mask is not sparse attention", capsule evidence: private allocation,
non-completion and clean-completion gates).

Non-completion: with every output filled with sentinels, a call that host
validation rejects (workspace one byte short, a misaligned output, budget 0,
an unsupported GQA ratio, a static workspace too small) returns its status
code and, after the device is synchronized, every sentinel is still there:
nothing was enqueued.  Clean completion: a call that succeeds overwrites
every entry of every output row -- token IDs up to the padding, widths,
attention outputs and log-sum-exps -- including the empty row (width 0) and
a dense row below the budget.
"""
import ctypes

import numpy as np
import pytest
import torch

import top_sparse_attention_qsa_amd as qsa
from tests import harness, inputs

pytestmark = pytest.mark.gpu

ID_SENTINEL = -7
F_SENTINEL = 1234.5


@pytest.fixture(scope="module")
def case():
    spec = inputs.custom("gates", [2055, 0, 5, 9000, 65537], h_i=8, d_i=64, h_q=8, h_kv=2, d=128,
                         keys="normal", slots="perm")
    return harness.GpuCase(inputs.make(spec, seed=11, device="cpu"))


def fresh_outputs(case):
    rows, stride = case.shape.rows, case.shape.token_stride
    s = case.spec
    return dict(
        ids=torch.full((rows, stride), ID_SENTINEL, dtype=torch.int32, device="cuda"),
        width=torch.full((rows,), ID_SENTINEL, dtype=torch.int32, device="cuda"),
        out=torch.full((rows * s.h_q * s.d + 4,), F_SENTINEL, device="cuda"),
        lse=torch.full((rows, s.h_q), F_SENTINEL, device="cuda"),
        scores=torch.full((rows, case.shape.max_groups), F_SENTINEL, device="cuda"),
        bitmap=torch.full((rows, case.shape.max_groups // 32), ID_SENTINEL, dtype=torch.int32,
                          device="cuda"))


def out_view(o, case, offset=0):
    s = case.spec
    n = case.shape.rows * s.h_q * s.d
    return o["out"][offset:offset + n].view(case.shape.rows, s.h_q, s.d)


def untouched(o):
    torch.cuda.synchronize()
    return (bool((o["ids"] == ID_SENTINEL).all()) and bool((o["width"] == ID_SENTINEL).all())
            and bool((o["out"] == F_SENTINEL).all()) and bool((o["lse"] == F_SENTINEL).all())
            and bool((o["scores"] == F_SENTINEL).all())
            and bool((o["bitmap"] == ID_SENTINEL).all()))


def shape_with(case, **kw):
    s = case.shape
    d = dict(batch=s.batch, queries=s.queries, index_heads=s.index_heads,
             index_dim=s.index_dim, q_heads=s.q_heads, kv_heads=s.kv_heads,
             head_dim=s.head_dim, budget_groups=s.budget_groups, max_groups=s.max_groups,
             kv_slots=s.kv_slots, rows_in_flight=s.rows_in_flight)
    d.update(kw)
    return qsa.make_shape(**d)


def decode_call(case, o, shape=None, ws=None, offset=0, variant="compact"):
    shape = shape or case.shape
    args = (shape, case.index_q, case.pooled, case.pooled_off, case.seq_len, case.slot_map,
            case.slot_off, case.k_cache, case.v_cache, case.q, case.scale, o["ids"],
            o["width"], out_view(o, case, offset), o["lse"])
    if variant == "noalloc":
        return qsa.qsa_decode_noalloc(*args)
    ws = case.workspace if ws is None else ws
    return qsa.qsa_decode(*args, ws, fused=variant == "fused", rows=variant
                          if variant != "fused" else "compact")


def rejected(fn, status):
    with pytest.raises(qsa.QSAError) as e:
        fn()
    assert e.value.status == status, (e.value.status, status)


@pytest.mark.parametrize("variant", ["compact", "fused", "dedup"])
def test_rejected_decode_leaves_outputs_untouched(case, variant):
    o = fresh_outputs(case)
    need = qsa.qsa_workspace_bytes(case.shape)
    short = case.workspace[:need - 1]
    rejected(lambda: decode_call(case, o, ws=short, variant=variant), qsa.QSA_ERR_WORKSPACE)
    assert untouched(o)
    rejected(lambda: decode_call(case, o, offset=1, variant=variant), qsa.QSA_ERR_SHAPE)
    assert untouched(o)
    rejected(lambda: decode_call(case, o, shape=shape_with(case, budget_groups=0),
                                 variant=variant), qsa.QSA_ERR_BUDGET)
    assert untouched(o)
    rejected(lambda: decode_call(case, o, shape=shape_with(case, q_heads=6),
                                 variant=variant), qsa.QSA_ERR_UNSUPPORTED)  # GQA 3
    assert untouched(o)
    rejected(lambda: decode_call(case, o, shape=shape_with(case, index_dim=48),
                                 variant=variant), qsa.QSA_ERR_UNSUPPORTED)
    assert untouched(o)


def test_rejected_noalloc_leaves_outputs_untouched(case):
    o = fresh_outputs(case)
    big = shape_with(case, rows_in_flight=0, max_groups=1 << 24)  # 5 rows x 64 MiB of scores
    assert qsa.qsa_workspace_bytes(big) > qsa.NOALLOC_WORKSPACE_BYTES
    rejected(lambda: decode_call(case, o, shape=big, variant="noalloc"),
             qsa.QSA_ERR_STATIC_WORKSPACE)
    assert untouched(o)
    rejected(lambda: decode_call(case, o, shape=shape_with(case, budget_groups=2000),
                                 variant="noalloc"), qsa.QSA_ERR_BUDGET)
    assert untouched(o)


def test_rejected_step_calls_leave_outputs_untouched(case):
    o = fresh_outputs(case)
    ws = case.workspace
    need = qsa.qsa_workspace_bytes(case.shape)
    rejected(lambda: qsa.qsa_score_groups(shape_with(case, index_heads=3), case.index_q,
                                          case.pooled, case.pooled_off, case.seq_len,
                                          o["scores"]), qsa.QSA_ERR_UNSUPPORTED)
    rejected(lambda: qsa.qsa_select_topk(case.shape, o["scores"], case.seq_len, o["bitmap"],
                                         ws[:need - 1]), qsa.QSA_ERR_WORKSPACE)
    rejected(lambda: qsa.qsa_emit_chronological(shape_with(case, budget_groups=0), o["bitmap"],
                                                case.seq_len, o["ids"], o["width"]),
             qsa.QSA_ERR_BUDGET)
    rejected(lambda: qsa.qsa_online_attend(case.shape, case.q, case.k_cache, case.v_cache,
                                           o["width"], case.scale, out_view(o, case, 1),
                                           o["lse"], ws), qsa.QSA_ERR_SHAPE)
    rejected(lambda: qsa.qsa_dense_attend(shape_with(case, q_heads=6), case.seq_len,
                                          case.slot_map, case.slot_off, case.k_cache,
                                          case.v_cache, case.q, case.scale, o["ids"],
                                          o["width"], out_view(o, case), o["lse"], ws),
             qsa.QSA_ERR_UNSUPPORTED)
    assert untouched(o)
    # a NULL workspace through the C ABI directly
    L = qsa.lib()
    rc = L.qsa_decode(ctypes.byref(case.shape), *[ctypes.c_void_p(t.data_ptr()) for t in (
        case.index_q, case.pooled, case.pooled_off, case.seq_len, case.slot_map, case.slot_off,
        case.k_cache, case.v_cache, case.q)], ctypes.c_float(case.scale),
        ctypes.c_void_p(o["ids"].data_ptr()), ctypes.c_void_p(o["width"].data_ptr()),
        ctypes.c_void_p(o["out"].data_ptr()), ctypes.c_void_p(o["lse"].data_ptr()), None,
        ctypes.c_size_t(need), None, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == qsa.QSA_ERR_NULL
    assert untouched(o)


@pytest.mark.parametrize("variant", ["compact", "fused", "dedup", "noalloc"])
def test_successful_decode_writes_every_row(case, variant):
    o = fresh_outputs(case)
    decode_call(case, o, variant=variant)
    torch.cuda.synchronize()
    width = o["width"].cpu().numpy()
    ids = o["ids"].cpu().numpy()
    out = out_view(o, case).cpu().numpy()
    lse = o["lse"].cpu().numpy()
    assert not (width == ID_SENTINEL).any()
    assert not (ids == ID_SENTINEL).any()        # body and -1 padding both written
    assert not (out == F_SENTINEL).any() and not (lse == F_SENTINEL).any()
    for r in range(case.spec.rows):
        exp = harness.oracle_row(case.data, r)
        w = len(exp["ids"])
        assert width[r] == w
        assert np.array_equal(ids[r, :w], exp["ids"]) and (ids[r, w:] == -1).all()
        if w == 0:   # empty row: +0 output, -inf log-sum-exp
            assert (out[r] == 0).all() and np.isneginf(lse[r]).all()
        else:
            assert harness.normwise_rel_err(out[r], exp["out_exact"]) <= 2e-6
    assert int(o["out"][-4:].eq(F_SENTINEL).sum()) == 4  # nothing past the output


def test_successful_step_calls_write_every_row(case):
    o = fresh_outputs(case)
    qsa.qsa_score_groups(case.shape, case.index_q, case.pooled, case.pooled_off, case.seq_len,
                         o["scores"])
    qsa.qsa_select_topk(case.shape, o["scores"], case.seq_len, o["bitmap"], case.workspace)
    qsa.qsa_emit_chronological(case.shape, o["bitmap"], case.seq_len, o["ids"], o["width"])
    torch.cuda.synchronize()
    scores = o["scores"].cpu().numpy()
    for r in range(case.spec.rows):
        g = inputs.row_tokens(case.spec, r) // 4
        assert not (scores[r, :g] == F_SENTINEL).any()     # every group scored
        assert (scores[r, g:] == F_SENTINEL).all()         # nothing past G
    assert not (o["bitmap"] == ID_SENTINEL).any()          # every bitmap word written
    assert not (o["ids"] == ID_SENTINEL).any() and not (o["width"] == ID_SENTINEL).any()
