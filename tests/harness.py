"""Test/benchmark harness: puts a generated workload on the GPU through the
product binding, and computes the oracle's expectation for chosen rows from
host copies of the same generated inputs.

The GPU side uses only top_sparse_attention_qsa_amd (HIP kernels); the
expectation side uses only the CPU oracle.  Neither sees the other's results.
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import top_sparse_attention_qsa_amd as qsa
from tests import inputs


def softmax_scale(d):
    return float(np.float32(1.0 / math.sqrt(d)))


class GpuCase:
    """A workload resident in HBM, ready for qsa_decode."""

    def __init__(self, data, rows_in_flight=0, device="cuda"):
        s = data["spec"]
        self.spec = s
        self.data = data
        dev = torch.device(device)
        to = (lambda t: t.to(dev)) if data["index_q"].device != dev else (lambda t: t)
        self.index_q = to(data["index_q"])
        self.q = to(data["q"])
        self.k_cache = to(data["k_cache"])
        self.v_cache = to(data["v_cache"])
        self.slot_map = to(data["slot_map"])
        self.seq_len = to(data["seq_len"])
        self.raw_off = to(data["raw_off"])
        self.slot_off = self.raw_off          # one slot-map entry per logical token
        g_max = qsa.round_groups(max(max(s.seq_lens) // 4, 1))
        self.shape = qsa.make_shape(s.batch, s.queries, s.h_i, s.d_i, s.h_q, s.h_kv, s.d,
                                    s.budget, g_max, data["kv_slots"], rows_in_flight)
        per_seq = qsa.pooled_elems_per_seq(g_max, s.d_i)
        self.pooled = torch.zeros(s.batch * per_seq, dtype=torch.float32, device=dev)
        self.pooled_off = torch.arange(s.batch, dtype=torch.int64, device=dev) * per_seq
        raw = to(data["raw_keys"])
        qsa.qsa_pool_groups(self.shape, raw, self.raw_off, self.seq_len, None, self.pooled,
                            self.pooled_off)
        del raw
        self.scale = softmax_scale(s.d)
        rows, stride = self.shape.rows, self.shape.token_stride
        self.workspace = torch.empty(qsa.qsa_workspace_bytes(self.shape), dtype=torch.uint8,
                                     device=dev)
        self.token_ids = torch.empty((rows, stride), dtype=torch.int32, device=dev)
        self.width = torch.empty(rows, dtype=torch.int32, device=dev)
        self.out = torch.empty((rows, s.h_q, s.d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((rows, s.h_q), dtype=torch.float32, device=dev)

    def decode(self, timer=None, fused=False, rows="compact"):
        """Steps 1-8; rows = "compact", "fused" or "dedup" (how K/V are read)."""
        qsa.qsa_decode(self.shape, self.index_q, self.pooled, self.pooled_off, self.seq_len,
                       self.slot_map, self.slot_off, self.k_cache, self.v_cache, self.q,
                       self.scale, self.token_ids, self.width, self.out, self.lse,
                       self.workspace, timer, fused=fused, rows=rows)

    def results(self):
        """Clones of (token_ids, width, out, lse)."""
        return (self.token_ids.clone(), self.width.clone(), self.out.clone(), self.lse.clone())


def host(t):
    return t.detach().cpu().numpy() if isinstance(t, torch.Tensor) else t


def oracle_row(data, row, kv_fetch=None, exact=True):
    """The oracle's result for one row from host copies of the generated
    inputs.  kv_fetch(slots) -> (kx, vx) supplies K/V rows at the oracle's own
    resolved slots when the cache is too large to copy to the host."""
    import oracle
    s = data["spec"]
    b, j = divmod(row, s.queries)
    n = inputs.row_tokens(s, row)
    off = int(data["raw_off"][b])
    raw = host(data["raw_keys"][off:off + max(n, 0)])
    pooled = oracle.pool_full(raw)
    qi = host(data["index_q"][row])
    scores = oracle.score(qi, pooled)
    chosen = oracle.select(scores, s.budget)
    ids = oracle.emit(chosen, n)
    smap = host(data["slot_map"][off:off + s.seq_lens[b]])
    slots = oracle.resolve(ids, smap, data["kv_slots"])
    if kv_fetch is None:
        kx, vx = oracle.gather(slots, host(data["k_cache"]), host(data["v_cache"]))
    else:
        kx, vx = kv_fetch(slots)
    q = host(data["q"][row])
    scale = softmax_scale(s.d)
    out, lse = oracle.attend_online(q, kx, vx, scale)
    res = dict(n=n, scores=scores, chosen=chosen, ids=ids, slots=slots, kx=kx, vx=vx,
               out=out, lse=lse)
    if exact:
        res["out_exact"], res["lse_exact"] = oracle.attend_exact(q, kx, vx, scale)
    return res


def device_kv_fetch(k_cache, v_cache):
    """K/V rows at given slots, copied from a device cache to the host."""
    def fetch(slots):
        idx = torch.as_tensor(np.asarray(slots, np.int64), device=k_cache.device)
        return (k_cache.index_select(0, idx).cpu().numpy(),
                v_cache.index_select(0, idx).cpu().numpy())
    return fetch


def oracle_threads():
    """Host threads for the oracle: the cores this process may run on, at most
    16 (the host share of one GPU on the test machines)."""
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def oracle_rows(data, rows, kv_fetch=None, threads=None):
    """The oracle's result for many rows, on host threads (the oracle is
    sequential per row; its C calls release the interpreter lock).

    Each sequence's raw index keys are copied to the host and pooled once; a
    row with N visible tokens uses the first N//4 pooled groups, which is what
    pooling its own prefix gives (a pooled group depends only on its own four
    tokens).  K/V rows are fetched at the oracle's own resolved slots by
    kv_fetch(slots) (default: host copies of the whole cache).  Returns one
    dict per row, in order: n, scores, ids, slots, out_exact, lse_exact."""
    import oracle
    s = data["spec"]
    threads = threads or oracle_threads()
    raw_off = host(data["raw_off"])
    seqs = sorted({r // s.queries for r in rows})
    raw = {b: host(data["raw_keys"][int(raw_off[b]):int(raw_off[b]) + s.seq_lens[b]])
           for b in seqs}
    smap = {b: host(data["slot_map"][int(raw_off[b]):int(raw_off[b]) + s.seq_lens[b]])
            for b in seqs}
    qi = host(data["index_q"])
    q = host(data["q"])
    if kv_fetch is None:
        kc, vc = host(data["k_cache"]), host(data["v_cache"])
        kv_fetch = lambda slots: oracle.gather(slots, kc, vc)  # noqa: E731
    scale = softmax_scale(s.d)
    with ThreadPoolExecutor(max_workers=threads) as ex:
        pooled = dict(zip(seqs, ex.map(lambda b: oracle.pool_full(raw[b]), seqs)))

        def select_row(r):
            b = r // s.queries
            n = inputs.row_tokens(s, r)
            sc = oracle.score(qi[r], pooled[b][:max(n, 0) // 4])
            ids = oracle.emit(oracle.select(sc, s.budget), n)
            return dict(n=n, scores=sc, ids=ids,
                        slots=oracle.resolve(ids, smap[b], data["kv_slots"]))
        res = list(ex.map(select_row, rows))
        kv = [kv_fetch(x["slots"]) for x in res]

        def attend_row(i):
            out, lse = oracle.attend_exact(q[rows[i]], kv[i][0], kv[i][1], scale)
            res[i]["out_exact"], res[i]["lse_exact"] = out, lse
        list(ex.map(attend_row, range(len(rows))))
    return res


def elementwise_rel_err(got, ref, floor=1e-6):
    """max over elements of |got - ref| / max(|ref|, floor * max|ref| of the
    element's output vector), in float64: the elementwise companion of
    normwise_rel_err, with a floor so that near-zero elements do not divide
    by ~0."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.maximum(np.abs(ref), floor * np.abs(ref).max(axis=-1, keepdims=True))
    return float(np.max(np.abs(got - ref) / np.maximum(scale, 1e-300)))


def normwise_rel_err(got, ref):
    """max over output vectors of max_d |got - ref| / max_d |ref| (float64)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return float(np.max(num / np.maximum(den, 1e-300)))
