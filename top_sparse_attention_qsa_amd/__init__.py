"""Physically sparse QSA attention for decode on AMD Instinct MI355X (gfx950).

A thin ctypes binding over libqsa.so (include/qsa.h): every function takes
torch tensors (device memory), checks dtype, device and contiguity, and passes
raw pointers and the current HIP stream to the C entry point of the same
name.  All arithmetic runs in the HIP kernels; there is no fallback.  If the
library is missing, calls raise instead of computing anything elsewhere.

Sources: AFN-017 "Top-k chooses the set; time chooses the order" and AFN-016
"A sparse mask is not sparse attention" (Hebrus Phase 6 notes).
"""
import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqsa.so")

GROUP = 4
MAX_BUDGET = 1024
KEY_TILE = 64
DECODE_STAGES = 5
STAGE_NAMES = ("score", "select_emit", "resolve_gather", "attend_chunks", "attend_merge")

QSA_OK, QSA_ERR_NULL, QSA_ERR_SHAPE, QSA_ERR_BUDGET = 0, 1, 2, 3
QSA_ERR_WORKSPACE, QSA_ERR_HIP, QSA_ERR_UNSUPPORTED = 4, 5, 6
QSA_ERR_STATIC_WORKSPACE = 7
NOALLOC_WORKSPACE_BYTES = 64 << 20


class QSAError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class Shape(ctypes.Structure):
    """Mirror of qsa_shape."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("queries", ctypes.c_int32),
        ("index_heads", ctypes.c_int32), ("index_dim", ctypes.c_int32),
        ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("budget_groups", ctypes.c_int32),
        ("max_groups", ctypes.c_int64), ("kv_slots", ctypes.c_int64),
        ("rows_in_flight", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]

    @property
    def rows(self):
        return self.batch * self.queries

    @property
    def token_stride(self):
        return GROUP * self.budget_groups + GROUP


class Bytes(ctypes.Structure):
    """Mirror of qsa_bytes."""
    _fields_ = [(n, ctypes.c_int64) for n in
                ("raw_key", "pooled_key", "kv", "workspace", "total", "dense_mask")]


def make_shape(batch, queries, index_heads, index_dim, q_heads, kv_heads, head_dim,
               budget_groups, max_groups, kv_slots, rows_in_flight=0):
    return Shape(batch, queries, index_heads, index_dim, q_heads, kv_heads, head_dim,
                 budget_groups, max_groups, kv_slots, rows_in_flight, 0)


def round_groups(g):
    """max_groups must be a multiple of 64."""
    return (int(g) + 63) // 64 * 64


_lib = None


def lib():
    """Load libqsa.so.  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, S = ctypes.c_void_p, ctypes.POINTER(Shape)
        i32, i64, f32, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        sig = {
            "qsa_workspace_bytes": ([S], sz),
            "qsa_pool_groups": ([S, P, P, P, P, P, P, P], ctypes.c_int),
            "qsa_score_groups": ([S, P, P, P, P, P, P], ctypes.c_int),
            "qsa_score_groups_chunk": ([S, P, P, P, P, P, P, P], ctypes.c_int),
            "qsa_select_topk": ([S, P, P, P, P, sz, P], ctypes.c_int),
            "qsa_emit_chronological": ([S, P, P, P, P, P], ctypes.c_int),
            "qsa_resolve_gather": ([S, P, P, P, P, P, P, P, P, P, P, P], ctypes.c_int),
            "qsa_online_attend": ([S, P, P, P, P, f32, P, P, P, sz, P], ctypes.c_int),
            "qsa_timer_create": ([i32, ctypes.c_uint32, ctypes.POINTER(P)], ctypes.c_int),
            "qsa_timer_read": ([P, P, ctypes.POINTER(i32)], ctypes.c_int),
            "qsa_timer_reset": ([P], None),
            "qsa_timer_destroy": ([P], None),
            "qsa_decode": ([S, P, P, P, P, P, P, P, P, P, f32, P, P, P, P, P, sz, P, P],
                           ctypes.c_int),
            "qsa_decode_fused": ([S, P, P, P, P, P, P, P, P, P, f32, P, P, P, P, P, sz, P, P],
                                 ctypes.c_int),
            "qsa_dense_attend": ([S, P, P, P, P, P, P, f32, P, P, P, P, P, sz, P], ctypes.c_int),
            "qsa_union_gather": ([S, P, P, P, P, P, P, P, P, P, P, P, P, sz, P], ctypes.c_int),
            "qsa_online_attend_indexed": ([S, P, P, P, i64, P, P, f32, P, P, P, sz, P],
                                          ctypes.c_int),
            "qsa_decode_dedup": ([S, P, P, P, P, P, P, P, P, P, f32, P, P, P, P, P, sz, P, P],
                                 ctypes.c_int),
            "qsa_decode_noalloc": ([S, P, P, P, P, P, P, P, P, P, f32, P, P, P, P, P, P],
                                   ctypes.c_int),
            "qsa_accounting": ([S, i64, ctypes.POINTER(Bytes)], ctypes.c_int),
            "qsa_status_string": ([ctypes.c_int], ctypes.c_char_p),
            "qsa_version": ([], ctypes.c_char_p),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def status_string(status):
    return lib().qsa_status_string(int(status)).decode()


def version():
    return lib().qsa_version().decode()


def _ptr(t, dtype, name, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc, where):
    if rc != QSA_OK:
        raise QSAError(rc, where)


def qsa_workspace_bytes(shape):
    return int(lib().qsa_workspace_bytes(ctypes.byref(shape)))


def qsa_pool_groups(shape, raw_keys, raw_off, seq_len, first_group, pooled, pooled_off,
                    stream=None):
    _check(lib().qsa_pool_groups(
        ctypes.byref(shape), _ptr(raw_keys, torch.float32, "raw_keys"),
        _ptr(raw_off, torch.int64, "raw_off"), _ptr(seq_len, torch.int32, "seq_len"),
        _ptr(first_group, torch.int32, "first_group", True), _ptr(pooled, torch.float32, "pooled"),
        _ptr(pooled_off, torch.int64, "pooled_off"), _stream(stream)), "qsa_pool_groups")


def qsa_score_groups(shape, index_q, pooled, pooled_off, seq_len, scores, stream=None):
    _check(lib().qsa_score_groups(
        ctypes.byref(shape), _ptr(index_q, torch.float32, "index_q"),
        _ptr(pooled, torch.float32, "pooled"), _ptr(pooled_off, torch.int64, "pooled_off"),
        _ptr(seq_len, torch.int32, "seq_len"), _ptr(scores, torch.float32, "scores"),
        _stream(stream)), "qsa_score_groups")


def qsa_score_groups_chunk(shape, index_q, pooled, pooled_off, seq_len, approx, bound,
                           stream=None):
    _check(lib().qsa_score_groups_chunk(
        ctypes.byref(shape), _ptr(index_q, torch.float32, "index_q"),
        _ptr(pooled, torch.float32, "pooled"), _ptr(pooled_off, torch.int64, "pooled_off"),
        _ptr(seq_len, torch.int32, "seq_len"), _ptr(approx, torch.float32, "approx"),
        _ptr(bound, torch.float32, "bound"), _stream(stream)), "qsa_score_groups_chunk")


def qsa_select_topk(shape, scores, seq_len, sel_bitmap, workspace, stream=None):
    _check(lib().qsa_select_topk(
        ctypes.byref(shape), _ptr(scores, torch.float32, "scores"),
        _ptr(seq_len, torch.int32, "seq_len"), _ptr(sel_bitmap, torch.int32, "sel_bitmap"),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)),
        "qsa_select_topk")


def qsa_emit_chronological(shape, sel_bitmap, seq_len, token_ids, width, stream=None):
    _check(lib().qsa_emit_chronological(
        ctypes.byref(shape), _ptr(sel_bitmap, torch.int32, "sel_bitmap"),
        _ptr(seq_len, torch.int32, "seq_len"), _ptr(token_ids, torch.int32, "token_ids"),
        _ptr(width, torch.int32, "width"), _stream(stream)), "qsa_emit_chronological")


def qsa_resolve_gather(shape, token_ids, width, seq_len, slot_map, slot_off, k_cache, v_cache,
                       k_compact, v_compact, phys_slots=None, stream=None):
    _check(lib().qsa_resolve_gather(
        ctypes.byref(shape), _ptr(token_ids, torch.int32, "token_ids"),
        _ptr(width, torch.int32, "width"), _ptr(seq_len, torch.int32, "seq_len"),
        _ptr(slot_map, torch.int32, "slot_map"), _ptr(slot_off, torch.int64, "slot_off"),
        _ptr(k_cache, torch.float32, "k_cache"), _ptr(v_cache, torch.float32, "v_cache"),
        _ptr(k_compact, torch.float32, "k_compact"), _ptr(v_compact, torch.float32, "v_compact"),
        _ptr(phys_slots, torch.int32, "phys_slots", True), _stream(stream)),
        "qsa_resolve_gather")


def qsa_online_attend(shape, q, k_compact, v_compact, width, softmax_scale, out, lse,
                      workspace, stream=None):
    _check(lib().qsa_online_attend(
        ctypes.byref(shape), _ptr(q, torch.float32, "q"),
        _ptr(k_compact, torch.float32, "k_compact"), _ptr(v_compact, torch.float32, "v_compact"),
        _ptr(width, torch.int32, "width"), ctypes.c_float(softmax_scale),
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse", True),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)),
        "qsa_online_attend")


_DECODE_VARIANTS = {"compact": "qsa_decode", "fused": "qsa_decode_fused",
                    "dedup": "qsa_decode_dedup"}


def qsa_decode(shape, index_q, pooled, pooled_off, seq_len, slot_map, slot_off, k_cache,
               v_cache, q, softmax_scale, token_ids, width, out, lse, workspace, timer=None,
               stream=None, fused=False, rows="compact"):
    """Steps 1-8.  rows selects how steps 6-8 read K/V: "compact" (per-row
    gather), "fused" (slot-map loads inside the attention; also fused=True)
    or "dedup" (one union gather per pass)."""
    name = _DECODE_VARIANTS["fused" if fused else rows]
    fn = getattr(lib(), name)
    _check(fn(
        ctypes.byref(shape), _ptr(index_q, torch.float32, "index_q"),
        _ptr(pooled, torch.float32, "pooled"), _ptr(pooled_off, torch.int64, "pooled_off"),
        _ptr(seq_len, torch.int32, "seq_len"), _ptr(slot_map, torch.int32, "slot_map"),
        _ptr(slot_off, torch.int64, "slot_off"), _ptr(k_cache, torch.float32, "k_cache"),
        _ptr(v_cache, torch.float32, "v_cache"), _ptr(q, torch.float32, "q"),
        ctypes.c_float(softmax_scale), _ptr(token_ids, torch.int32, "token_ids"),
        _ptr(width, torch.int32, "width"), _ptr(out, torch.float32, "out"),
        _ptr(lse, torch.float32, "lse", True), _ptr(workspace, torch.uint8, "workspace"),
        workspace.numel(), timer.handle if timer is not None else None, _stream(stream)),
        name)


def qsa_decode_noalloc(shape, index_q, pooled, pooled_off, seq_len, slot_map, slot_off,
                       k_cache, v_cache, q, softmax_scale, token_ids, width, out, lse, timer=None,
                       stream=None):
    """qsa_decode over the library's static device workspace (no workspace
    argument, nothing allocated)."""
    _check(lib().qsa_decode_noalloc(
        ctypes.byref(shape), _ptr(index_q, torch.float32, "index_q"),
        _ptr(pooled, torch.float32, "pooled"), _ptr(pooled_off, torch.int64, "pooled_off"),
        _ptr(seq_len, torch.int32, "seq_len"), _ptr(slot_map, torch.int32, "slot_map"),
        _ptr(slot_off, torch.int64, "slot_off"), _ptr(k_cache, torch.float32, "k_cache"),
        _ptr(v_cache, torch.float32, "v_cache"), _ptr(q, torch.float32, "q"),
        ctypes.c_float(softmax_scale), _ptr(token_ids, torch.int32, "token_ids"),
        _ptr(width, torch.int32, "width"), _ptr(out, torch.float32, "out"),
        _ptr(lse, torch.float32, "lse", True), timer.handle if timer is not None else None,
        _stream(stream)), "qsa_decode_noalloc")


def qsa_decode_fused(*args, **kw):
    """qsa_decode with the gather fused into the attention (no compact scratch)."""
    return qsa_decode(*args, fused=True, **kw)


def qsa_decode_dedup(*args, **kw):
    """qsa_decode with one union gather per pass of rows."""
    return qsa_decode(*args, rows="dedup", **kw)


def qsa_union_gather(shape, token_ids, width, seq_len, slot_map, slot_off, k_cache, v_cache,
                     k_union, v_union, union_pos, union_groups, workspace, stream=None):
    _check(lib().qsa_union_gather(
        ctypes.byref(shape), _ptr(token_ids, torch.int32, "token_ids"),
        _ptr(width, torch.int32, "width"), _ptr(seq_len, torch.int32, "seq_len"),
        _ptr(slot_map, torch.int32, "slot_map"), _ptr(slot_off, torch.int64, "slot_off"),
        _ptr(k_cache, torch.float32, "k_cache"), _ptr(v_cache, torch.float32, "v_cache"),
        _ptr(k_union, torch.float32, "k_union"), _ptr(v_union, torch.float32, "v_union"),
        _ptr(union_pos, torch.int32, "union_pos"),
        _ptr(union_groups, torch.int32, "union_groups", True),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)),
        "qsa_union_gather")


def qsa_online_attend_indexed(shape, q, k_rows, v_rows, row_pos, width, softmax_scale, out, lse,
                              workspace, stream=None):
    n_rows = k_rows.shape[0]
    if v_rows.shape[0] != n_rows:
        raise ValueError("k_rows and v_rows differ in row count")
    _check(lib().qsa_online_attend_indexed(
        ctypes.byref(shape), _ptr(q, torch.float32, "q"), _ptr(k_rows, torch.float32, "k_rows"),
        _ptr(v_rows, torch.float32, "v_rows"), int(n_rows),
        _ptr(row_pos, torch.int32, "row_pos"), _ptr(width, torch.int32, "width"),
        ctypes.c_float(softmax_scale), _ptr(out, torch.float32, "out"),
        _ptr(lse, torch.float32, "lse", True), _ptr(workspace, torch.uint8, "workspace"),
        workspace.numel(), _stream(stream)),
        "qsa_online_attend_indexed")


def qsa_dense_attend(shape, seq_len, slot_map, slot_off, k_cache, v_cache, q, softmax_scale,
                     token_ids, width, out, lse, workspace, stream=None):
    _check(lib().qsa_dense_attend(
        ctypes.byref(shape), _ptr(seq_len, torch.int32, "seq_len"),
        _ptr(slot_map, torch.int32, "slot_map"), _ptr(slot_off, torch.int64, "slot_off"),
        _ptr(k_cache, torch.float32, "k_cache"), _ptr(v_cache, torch.float32, "v_cache"),
        _ptr(q, torch.float32, "q"), ctypes.c_float(softmax_scale),
        _ptr(token_ids, torch.int32, "token_ids"), _ptr(width, torch.int32, "width"),
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse", True),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)),
        "qsa_dense_attend")


def qsa_accounting(shape, total_tokens):
    b = Bytes()
    _check(lib().qsa_accounting(ctypes.byref(shape), int(total_tokens), ctypes.byref(b)),
           "qsa_accounting")
    return {n: getattr(b, n) for n, _ in Bytes._fields_}


class Timer:
    """qsa_timer: HIP events around each qsa_decode stage."""

    def __init__(self, max_calls, stages=None):
        """stages: names from STAGE_NAMES to time (default: all)."""
        mask = (1 << DECODE_STAGES) - 1 if stages is None else \
            sum(1 << STAGE_NAMES.index(n) for n in stages)
        h = ctypes.c_void_p()
        _check(lib().qsa_timer_create(int(max_calls), mask, ctypes.byref(h)), "qsa_timer_create")
        self.handle = h
        self.max_calls = int(max_calls)

    def read(self):
        """Per-call stage times in ms, shape [calls][DECODE_STAGES]."""
        buf = (ctypes.c_float * (self.max_calls * DECODE_STAGES))()
        n = ctypes.c_int32()
        _check(lib().qsa_timer_read(self.handle, buf, ctypes.byref(n)), "qsa_timer_read")
        vals = list(buf)[: n.value * DECODE_STAGES]
        return [vals[i * DECODE_STAGES:(i + 1) * DECODE_STAGES] for i in range(n.value)]

    def reset(self):
        lib().qsa_timer_reset(self.handle)

    def close(self):
        if self.handle is not None:
            lib().qsa_timer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def pooled_elems_per_seq(max_groups, index_dim):
    """Elements of one sequence's tiled pooled-key buffer (whole 64-group tiles)."""
    return (int(max_groups) + KEY_TILE - 1) // KEY_TILE * KEY_TILE * int(index_dim)
