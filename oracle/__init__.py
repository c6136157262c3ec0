"""ctypes wrapper around the sequential CPU oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module; the HIP product path never does.
Every function takes and returns numpy arrays; see qsa_oracle.h for the
definition each one follows.

Sources:
  [SET]  AFN-017 "Top-k chooses the set; time chooses the order"
  [MASK] AFN-016 "A sparse mask is not sparse attention"
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
GROUP = 4  # four-token groups ([SET] §Decision)

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.path.join(HERE, "liboracle.so")
        if not os.path.exists(path):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, f32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
        L.oracle_pool_full.argtypes = [P, i64, i32, P]
        L.oracle_pool_incremental.argtypes = [P, i64, i32, P, P]
        L.oracle_score.argtypes = [P, P, i64, i32, i32, P]
        L.oracle_select.argtypes = [P, i64, i32, P]
        L.oracle_select.restype = i64
        L.oracle_emit.argtypes = [P, i64, i64, P]
        L.oracle_emit.restype = i32
        L.oracle_resolve.argtypes = [P, i32, P, i64, i64, P]
        L.oracle_resolve.restype = i32
        L.oracle_gather.argtypes = [P, i32, P, P, i64, P, P]
        L.oracle_attend_online.argtypes = [P, P, P, i32, i32, i32, i32, f32, P, P]
        L.oracle_attend_exact.argtypes = [P, P, P, i32, i32, i32, i32, f64, P, P]
        L.oracle_decode_row.argtypes = [P, P, i64, i32, i32, i32, P, i64, i64, P, P, i32,
                                        i32, P, i32, f32, P, P, P, P, P, P, P, P]
        L.oracle_decode_row.restype = i32
        L.oracle_dense_row.argtypes = [i64, P, i64, i64, P, P, i32, i32, P, i32, f32,
                                       P, P, P, P, P, P]
        L.oracle_dense_row.restype = i32
        _lib = L
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def pool_full(raw):
    """O1: raw [N][D_I] f32 -> pooled [N//4][D_I] f32 (group mean)."""
    raw = _f32(raw)
    n, d = raw.shape
    out = np.empty((n // GROUP, d), np.float32)
    lib().oracle_pool_full(_p(raw), n, d, _p(out))
    return out


def pool_incremental(raw):
    """O1': token-by-token pooling with a carried partial sum."""
    raw = _f32(raw)
    n, d = raw.shape
    out = np.empty((n // GROUP, d), np.float32)
    partial = np.zeros(d, np.float32)
    lib().oracle_pool_incremental(_p(raw), n, d, _p(out), _p(partial))
    return out


def score(qi, pooled):
    """O2: qi [H_I][D_I], pooled [G][D_I] -> scores [G] f32."""
    qi, pooled = _f32(qi), _f32(pooled)
    h, d = qi.shape
    g = pooled.shape[0]
    assert g == 0 or pooled.shape[1] == d
    out = np.empty(g, np.float32)
    lib().oracle_score(_p(qi), _p(pooled), g, h, d, _p(out))
    return out


def select(scores, k):
    """O3: the chosen groups, in rank order (score desc, position asc)."""
    scores = _f32(scores)
    g = scores.shape[0]
    out = np.empty(max(min(g, k), 1), np.int64)
    m = lib().oracle_select(_p(scores), g, k, _p(out))
    if m < 0:
        raise MemoryError("oracle_select")
    return out[:m]


def emit(chosen, n_tokens):
    """O4-O6: chronological token-ID row and its width."""
    chosen = np.ascontiguousarray(chosen, dtype=np.int64)
    m = chosen.shape[0]
    ids = np.empty(GROUP * m + GROUP, np.int32)
    w = lib().oracle_emit(_p(chosen), m, n_tokens, _p(ids))
    if w < 0:
        raise MemoryError("oracle_emit")
    return ids[:w].copy()


def resolve(ids, slot_map, kv_slots):
    """O7: logical IDs -> physical slots (raises on an out-of-range entry)."""
    ids, slot_map = _i32(ids), _i32(slot_map)
    slots = np.empty(max(ids.shape[0], 1), np.int32)
    rc = lib().oracle_resolve(_p(ids), ids.shape[0], _p(slot_map), slot_map.shape[0],
                              kv_slots, _p(slots))
    if rc != 0:
        raise IndexError("oracle_resolve: ID or slot out of range")
    return slots[:ids.shape[0]].copy()


def gather(slots, k_cache, v_cache):
    """O8: compact copies of the K/V cache rows at the given slots."""
    slots = _i32(slots)
    k_cache, v_cache = _f32(k_cache), _f32(v_cache)
    row_shape = k_cache.shape[1:]
    row = int(np.prod(row_shape))
    w = slots.shape[0]
    kx = np.empty((w,) + row_shape, np.float32)
    vx = np.empty((w,) + row_shape, np.float32)
    lib().oracle_gather(_p(slots), w, _p(k_cache), _p(v_cache), row, _p(kx), _p(vx))
    return kx, vx


def attend_online(q, kx, vx, scale):
    """O9: F32 online softmax in row order.  q [H_q][D], kx/vx [W][H_kv][D]."""
    q, kx, vx = _f32(q), _f32(kx), _f32(vx)
    h_q, d = q.shape
    w, h_kv = kx.shape[0], (kx.shape[1] if kx.ndim == 3 else 1)
    out = np.empty((h_q, d), np.float32)
    lse = np.empty(h_q, np.float32)
    lib().oracle_attend_online(_p(q), _p(kx), _p(vx), w, h_q, h_kv, d,
                               ctypes.c_float(scale), _p(out), _p(lse))
    return out, lse


def attend_exact(q, kx, vx, scale):
    """O9-exact: the double-precision definition of the same attention."""
    q, kx, vx = _f32(q), _f32(kx), _f32(vx)
    h_q, d = q.shape
    w, h_kv = kx.shape[0], (kx.shape[1] if kx.ndim == 3 else 1)
    out = np.empty((h_q, d), np.float64)
    lse = np.empty(h_q, np.float64)
    lib().oracle_attend_exact(_p(q), _p(kx), _p(vx), w, h_q, h_kv, d, float(scale),
                              _p(out), _p(lse))
    return out, lse


def decode_row(qi, pooled, n_tokens, k, slot_map, kv_slots, k_cache, v_cache, q, scale):
    """O2-O9 for one row, all in C.  pooled is the plain [G][D_I] buffer."""
    qi, pooled, q = _f32(qi), _f32(pooled), _f32(q)
    slot_map = _i32(slot_map)
    k_cache, v_cache = _f32(k_cache), _f32(v_cache)
    h_i, d_i = qi.shape
    h_q, d = q.shape
    h_kv = k_cache.shape[1]
    g = n_tokens // GROUP
    wmax = GROUP * k + GROUP
    scores = np.empty(max(g, 1), np.float32)
    chosen = np.empty(max(min(g, k), 1), np.int64)
    ids = np.empty(wmax, np.int32)
    slots = np.empty(wmax, np.int32)
    kx = np.empty((wmax, h_kv, d), np.float32)
    vx = np.empty((wmax, h_kv, d), np.float32)
    out = np.empty((h_q, d), np.float32)
    lse = np.empty(h_q, np.float32)
    w = lib().oracle_decode_row(_p(qi), _p(pooled), n_tokens, h_i, d_i, k, _p(slot_map),
                                slot_map.shape[0], kv_slots, _p(k_cache), _p(v_cache),
                                h_kv, d, _p(q), h_q, ctypes.c_float(scale), _p(scores),
                                _p(chosen), _p(ids), _p(slots), _p(kx), _p(vx),
                                _p(out), _p(lse))
    if w < 0:
        raise IndexError("oracle_decode_row: resolution error")
    return dict(scores=scores[:g], ids=ids[:w].copy(), width=w, slots=slots[:w].copy(),
                kx=kx[:w], vx=vx[:w], out=out, lse=lse)


def dense_row(n_tokens, slot_map, kv_slots, k_cache, v_cache, q, scale):
    """O10: the dense causal row over tokens 0..N-1."""
    slot_map, q = _i32(slot_map), _f32(q)
    k_cache, v_cache = _f32(k_cache), _f32(v_cache)
    h_q, d = q.shape
    h_kv = k_cache.shape[1]
    n = max(int(n_tokens), 1)
    ids = np.empty(n, np.int32)
    slots = np.empty(n, np.int32)
    kx = np.empty((n, h_kv, d), np.float32)
    vx = np.empty((n, h_kv, d), np.float32)
    out = np.empty((h_q, d), np.float32)
    lse = np.empty(h_q, np.float32)
    w = lib().oracle_dense_row(n_tokens, _p(slot_map), slot_map.shape[0], kv_slots,
                               _p(k_cache), _p(v_cache), h_kv, d, _p(q), h_q,
                               ctypes.c_float(scale), _p(ids), _p(slots), _p(kx), _p(vx),
                               _p(out), _p(lse))
    if w < 0:
        raise IndexError("oracle_dense_row: resolution error")
    return dict(ids=ids[:w].copy(), width=w, out=out, lse=lse)
