"""CPU tests of the C-ABI boundary: libqsa.so loads, exports every symbol
include/qsa.h declares, and rejects bad arguments on the host before anything
is enqueued (no GPU is touched by these tests).

The cases that pass fake device addresses rely on host validation refusing
the call; they run only where no GPU is visible, so that a validation
regression can never launch a kernel on a fake address.  The full validation
matrix runs against stub launchers in tests/test_host_sanitized.py."""
import ctypes
import os
import re

import pytest

import top_sparse_attention_qsa_amd as qsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")

# fake device addresses are passed only where no GPU could run a kernel on them
no_gpu = pytest.mark.skipif(
    __import__("torch").cuda.is_available(),
    reason="fake device addresses: only without a visible GPU")

C4 = dict(batch=32, queries=1, index_heads=16, index_dim=128, q_heads=32, kv_heads=4,
          head_dim=128, budget_groups=512, max_groups=65536, kv_slots=8388608)


def shape(**kw):
    d = dict(C4)
    d.update(kw)
    return qsa.make_shape(**d)


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"QSA_API\s+[\w\s\*]*?\b(qsa_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) == 22, names
    L = qsa.lib()
    for n in names:
        assert hasattr(L, n), n
    assert qsa.version().endswith("gfx950")


def test_status_strings():
    for code in range(8):
        assert qsa.status_string(code)
    assert qsa.status_string(99) == "unknown status"


def test_workspace_scales_with_groups_and_width_never_tokens():
    """The workspace is sized by candidate groups, the budget and the selected
    width per row in flight; no buffer has a tokens-by-queries extent
    (AFN-016 "A sparse mask is not sparse attention", §What the checkpoint
    measures)."""
    base = qsa.qsa_workspace_bytes(shape())
    assert base > 0
    # per row: scores (4 B/group) + maxima (4 B / 16 groups) + tile widths
    # (4 B / 64 groups) + compact K/V + partials
    per_row_compact = 2 * (4 * 512 + 4) * 4 * 128 * 4
    per_row_groups = 65536 * 4 + 65536 // 16 * 4 + 65536 // 64 * 4
    per_row_part = 32 * 5 * (128 + 2) * 4  # 33 chunks of 64 rows, one partial per 8
    # union gather: row bitmap, union bitmap and word prefixes (at most one
    # sequence per row), union list, position list
    per_row_union = 3 * (65536 // 32 + 1) * 4 + 513 * 8 + (4 * 512 + 4) * 4
    assert base <= 32 * (per_row_compact + per_row_groups + per_row_part + per_row_union) + \
        16 * 256
    # bounding rows in flight bounds the workspace
    small = qsa.qsa_workspace_bytes(shape(rows_in_flight=4))
    assert small * 7 < base
    # doubling the budget grows it, a larger KV cache does not
    assert qsa.qsa_workspace_bytes(shape(budget_groups=1024)) > base
    assert qsa.qsa_workspace_bytes(shape(kv_slots=2 * 8388608)) == base


def test_accounting_ledger():
    s = shape()
    b = qsa.qsa_accounting(s, 32 * 262144)
    assert b["dense_mask"] == 0
    assert b["raw_key"] == 32 * 262144 * 128 * 4
    assert b["pooled_key"] == 32 * 65536 * 128 * 4
    assert b["kv"] == 2 * 8388608 * 4 * 128 * 4
    assert b["workspace"] == qsa.qsa_workspace_bytes(s)
    assert b["total"] == sum(b[k] for k in ("raw_key", "pooled_key", "kv", "workspace"))


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(budget_groups=0), qsa.QSA_ERR_BUDGET),
    (dict(budget_groups=1025), qsa.QSA_ERR_BUDGET),
    (dict(max_groups=100), qsa.QSA_ERR_SHAPE),
    (dict(batch=0), qsa.QSA_ERR_SHAPE),
    (dict(q_heads=30), qsa.QSA_ERR_SHAPE),
    (dict(q_heads=96, kv_heads=3), qsa.QSA_ERR_UNSUPPORTED),
    (dict(head_dim=96), qsa.QSA_ERR_UNSUPPORTED),
    (dict(index_dim=48), qsa.QSA_ERR_UNSUPPORTED),
    (dict(index_heads=3), qsa.QSA_ERR_UNSUPPORTED),
    (dict(batch=70000), qsa.QSA_ERR_UNSUPPORTED),
])
def test_invalid_shapes_are_rejected_before_enqueue(kw, code):
    s = shape(**kw)
    L = qsa.lib()
    dummy = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    rc = L.qsa_decode(ctypes.byref(s), *([dummy] * 9), ctypes.c_float(0.1), dummy, dummy,
                      dummy, None, dummy, ctypes.c_size_t(1 << 40), None, None)
    assert rc == code


@no_gpu
def test_null_pointers_and_small_workspace_rejected():
    s = shape()
    L = qsa.lib()
    p = ctypes.c_void_p(256)
    assert L.qsa_score_groups(ctypes.byref(s), None, p, p, p, p, None) == qsa.QSA_ERR_NULL
    assert L.qsa_select_topk(ctypes.byref(s), p, p, p, p, ctypes.c_size_t(10), None) == \
        qsa.QSA_ERR_WORKSPACE
    assert L.qsa_emit_chronological(ctypes.byref(s), p, p, None, p, None) == qsa.QSA_ERR_NULL
    assert L.qsa_resolve_gather(ctypes.byref(s), p, p, p, p, p, p, None, p, p, None, None) == \
        qsa.QSA_ERR_NULL
    assert L.qsa_online_attend(ctypes.byref(s), p, p, p, p, ctypes.c_float(1.0), p, None, p,
                               ctypes.c_size_t(10), None) == qsa.QSA_ERR_WORKSPACE
    assert L.qsa_decode(ctypes.byref(s), *([p] * 9), ctypes.c_float(0.1), p, p, p, None, p,
                        ctypes.c_size_t(10), None, None) == qsa.QSA_ERR_WORKSPACE
    assert L.qsa_decode(None, *([p] * 9), ctypes.c_float(0.1), p, p, p, None, p,
                        ctypes.c_size_t(1 << 40), None, None) == qsa.QSA_ERR_NULL
    assert L.qsa_decode_dedup(ctypes.byref(s), *([p] * 9), ctypes.c_float(0.1), p, p, p, None,
                              p, ctypes.c_size_t(10), None, None) == qsa.QSA_ERR_WORKSPACE
    big = ctypes.c_size_t(1 << 40)
    assert L.qsa_union_gather(ctypes.byref(s), p, p, p, p, p, p, p, p, p, None, None, p, big,
                              None) == qsa.QSA_ERR_NULL
    split = shape(rows_in_flight=4)  # one union needs every row in one pass
    assert L.qsa_union_gather(ctypes.byref(split), p, p, p, p, p, p, p, p, p, p, None, p, big,
                              None) == qsa.QSA_ERR_UNSUPPORTED
    assert L.qsa_online_attend_indexed(ctypes.byref(s), p, p, p, 0, p, p, ctypes.c_float(1.0),
                                       p, None, p, big, None) == qsa.QSA_ERR_SHAPE
    # misaligned device pointers are refused, not dereferenced
    odd = ctypes.c_void_p(258)
    assert L.qsa_score_groups(ctypes.byref(s), p, odd, p, p, p, None) == qsa.QSA_ERR_SHAPE
    chunk = shape(queries=16)
    assert L.qsa_score_groups_chunk(ctypes.byref(chunk), odd, p, p, p, p, p, None) == \
        qsa.QSA_ERR_SHAPE
    assert L.qsa_decode(ctypes.byref(s), odd, *([p] * 8), ctypes.c_float(0.1), p, p, p, None, p,
                        ctypes.c_size_t(1 << 40), None, None) == qsa.QSA_ERR_SHAPE
    assert L.qsa_accounting(ctypes.byref(s), 10, None) == qsa.QSA_ERR_NULL
    assert L.qsa_timer_create(0, 1, None) == qsa.QSA_ERR_NULL
    h = ctypes.c_void_p()
    assert L.qsa_timer_create(4, 0, ctypes.byref(h)) == qsa.QSA_ERR_SHAPE  # no stage
    assert L.qsa_timer_create(4, 1 << qsa.DECODE_STAGES, ctypes.byref(h)) == qsa.QSA_ERR_SHAPE


def test_binding_refuses_host_tensors():
    import torch
    s = shape(batch=1, max_groups=64, kv_slots=10)
    with pytest.raises(ValueError):
        qsa.qsa_score_groups(s, torch.zeros(16, 128), torch.zeros(64 * 128),
                             torch.zeros(1, dtype=torch.int64), torch.zeros(1, dtype=torch.int32),
                             torch.zeros(64))
