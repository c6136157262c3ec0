"""Benchmark: QSA decode queries/s at 262,144 visible tokens on one MI355X.

Workload (synthetic, seeded): a decode batch of 32 independent sequences, each
with 262,144 visible tokens (65,536 complete groups, no tail), budget 512
groups, indexer 16 heads x 128, attention 32 query heads / 4 KV heads x 128,
F32, per-sequence slot maps = disjoint chunks of one random permutation of a
shared 8,388,608-slot K/V pool.  One step = one qsa_decode call covering all
eight steps of the path for the 32 rows, inputs resident in HBM.

Prints one JSON line.  The roofline object describes the dominant kernel (the
group-scoring sweep): its algorithmic bytes per launch over its mean launch
time, measured with HIP events recorded on the launch stream inside the timed
region.  cpu_baseline times the sequential CPU oracle on host cores over the
same 32 rows.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QSA decode queries/sec at 262,144 visible tokens; achieved HBM GB/s vs peak"
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published
SETTLE_MS = 150  # untimed steps before the warmup (see main)
MFMA_FP32_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix, published
COUNTERS = os.path.join(ROOT, "profiles", "score_32x262144_counters.json")


def algorithmic_bytes(B=32, G=65536, h_i=16, d_i=128, h_q=32, h_kv=4, d=128, k=512):
    """What the method moves in one decode step, item by item (the byte table
    of the hot-path scope: pooled keys read, scores written and read once,
    selected K/V rows read, the compact copy written and read back, and the
    small per-row vectors).  Implementation traffic the method does not need
    is in implementation_overhead_bytes."""
    W = 4 * k  # no tail at 262,144 tokens
    kv_row = h_kv * d * 4
    return dict(
        pooled_keys=B * G * d_i * 4,
        scores=2 * B * G * 4,
        kv_rows_read=2 * B * W * kv_row,
        compact_write_read=2 * 2 * B * W * kv_row,
        small=(B * h_i * d_i * 4 + B * h_q * d * 4 + B * h_q * d * 4 + 2 * B * G // 8
               + 2 * B * W * 4 + B * W * 4),
    )


def implementation_overhead_bytes(B=32, G=65536, h_q=32, d=128, k=512):
    """Traffic of this implementation beyond the method's bytes: the per-16-
    group score maxima (written by the scoring kernel, read by the selection)
    and the attention's range partials (one per 8 consecutive 64-row chunks,
    written by the attention, read by the merge).  The decode path writes no
    selection bitmap (the selection writes token IDs directly), so the bitmap
    entries of the method's table are not moved either."""
    parts = math.ceil(math.ceil((4 * k + 3) / 64) / 8)
    return dict(maxima=2 * B * (G // 16) * 4, attention_partials=2 * B * h_q * parts * (d + 2) * 4,
                bitmap_not_moved=-2 * B * G // 8)


def stage_bytes(B=32, G=65536, h_i=16, d_i=128, h_q=32, h_kv=4, d=128, k=512):
    """Bytes each kernel of the compact step moves (method bytes plus its share
    of the implementation overhead), for comparison with its counters."""
    W = 4 * k
    kv_row = h_kv * d * 4
    seg = G // 16
    parts = math.ceil(math.ceil((4 * k + 3) / 64) / 8)  # range partials per (row, head)
    part = B * h_q * parts * (d + 2) * 4
    return dict(
        score=B * G * d_i * 4 + B * h_i * d_i * 4 + B * G * 4 + B * seg * 4,
        select_emit=B * G * 4 + B * seg * 4 + B * (W + 4) * 4 + B * 4,
        resolve_gather=B * W * 4 * 2 + B * W * 4 + 2 * B * W * kv_row + 2 * B * W * kv_row,
        attend_chunks=2 * B * W * kv_row + B * h_q * d * 4 + part,
        attend_merge=part + B * h_q * (d + 1) * 4)


def score_roofline_bytes(B=32, G=65536, h_i=16, d_i=128):
    """The scoring kernel's method bytes: per group its pooled key (D_I floats)
    read and its score written, plus each row's index query."""
    return B * G * (d_i * 4 + 4) + B * h_i * d_i * 4


def fused_algorithmic_bytes(B=32, G=65536, h_i=16, d_i=128, h_q=32, h_kv=4, d=128, k=512):
    """The same step with resolve+gather inside the attention: the compact copy
    is neither written nor read back."""
    a = algorithmic_bytes(B, G, h_i, d_i, h_q, h_kv, d, k)
    return sum(a.values()) - a["compact_write_read"]


def source_digest():
    h = hashlib.sha256()
    for f in ("score.hip", "qsa_device.h"):
        with open(os.path.join(ROOT, "top_sparse_attention_qsa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def library_digest():
    """Digest of every source of the library (kernels and host side)."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "top_sparse_attention_qsa_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode())
                h.update(fh.read())
    return h.hexdigest()


def _counters():
    try:
        with open(COUNTERS) as f:
            return json.load(f)
    except (OSError, ValueError):
        return None


def measured_traffic():
    """HBM bytes per score launch from the committed rocprofv3 counter
    summary, or None when absent or taken on a different kernel source."""
    c = _counters()
    if c is None or c.get("source_sha256") != source_digest():
        return None
    return c.get("traffic_bytes_per_launch")


def measured_step_traffic():
    """HBM bytes per decode step by stage (FETCH_SIZE + WRITE_SIZE of each
    kernel, scaled by the copy calibration), or None when the counters were
    taken on a different library source."""
    c = _counters()
    if c is None or c.get("library_sha256") != library_digest():
        return None
    return c.get("stage_traffic_bytes")


PROBE_SRC = os.path.join(ROOT, "bench_stream_read.hip")
PROBE_LIB = os.path.join(ROOT, "bench_stream_read.so")


def build_probe():
    """Compile the streaming-read probe of the context line (not part of
    libqsa) next to this file."""
    import subprocess
    from top_sparse_attention_qsa_amd import build as qsa_build
    tmp = PROBE_LIB + ".tmp"
    cmd = [qsa_build.hipcc(), *qsa_build.HIPFLAGS, "-shared", "-o", tmp, PROBE_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PROBE_SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def context_bandwidth(reps=10):
    """Achievable-bandwidth context, not a denominator of anything reported:
    reads of 1 GiB (bench_stream_read.hip: grid-stride float4 loads, and the
    scoring kernel's tiled shape) and torch's device copy of 1 GiB."""
    import ctypes
    import torch
    n = (1 << 30) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    res = {}
    fns = [("copy", lambda: y.copy_(x), 8 * n)]
    if not os.path.exists(PROBE_LIB):
        build_probe()
    bw = ctypes.CDLL(PROBE_LIB)
    for f in (bw.bw_stream_read, bw.bw_tiled_read):
        f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]

    def reader(f):
        def read():
            s = torch.cuda.current_stream().cuda_stream
            if f(x.data_ptr(), 4 * n, sink.data_ptr(), s) != 0:
                raise RuntimeError("bandwidth probe failed")
        return read
    fns.insert(0, ("tiled_read", reader(bw.bw_tiled_read), 4 * n))
    fns.insert(0, ("stream_read", reader(bw.bw_stream_read), 4 * n))
    for name, fn, nbytes in fns:
        for _ in range(3):
            fn()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        res[f"{name}_gbps"] = nbytes / (ms * 1e-3) / 1e9
    del x, y
    torch.cuda.empty_cache()
    res["note"] = ("1 GiB of f32: a grid-stride streaming read kernel, a read in the scoring "
                   "kernel's tiled shape (32 KiB per wavefront, four 1 KiB loads in flight, five "
                   "workgroups per compute unit), and torch's device copy (bytes read + written); "
                   "context only")
    return res


def cpu_baseline(data, rows, threads, passes=2):
    """Oracle over the given rows, `passes` times (about 10 s of CPU work for
    the decode batch): score, select, emit and resolve on host copies of the
    pooled keys and slot maps (timed), K/V rows fetched at the oracle's own
    slots (not timed), then the F32 online attention (timed)."""
    import numpy as np
    import torch
    import oracle
    from tests import harness
    s = data["spec"]
    n = s.seq_lens[0]
    raw = data["raw_keys"]
    prep = []
    for r in rows:
        off = int(data["raw_off"][r])
        pooled = oracle.pool_full(raw[off:off + n].cpu().numpy())
        prep.append(dict(row=r, pooled=pooled, qi=data["index_q"][r].cpu().numpy(),
                         smap=data["slot_map"][off:off + n].cpu().numpy(),
                         q=data["q"][r].cpu().numpy()))
    scale = harness.softmax_scale(s.d)
    kv_slots = data["kv_slots"]

    def phase1(p):
        sc = oracle.score(p["qi"], p["pooled"])
        p["ids"] = oracle.emit(oracle.select(sc, s.budget), n)
        p["slots"] = oracle.resolve(p["ids"], p["smap"], kv_slots)
        return p

    def phase2(p):
        p["out"], p["lse"] = oracle.attend_online(p["q"], p["kx"], p["vx"], scale)
        return p

    timed = 0.0
    fetch = harness.device_kv_fetch(data["k_cache"], data["v_cache"])
    used = min(threads, len(prep))
    with ThreadPoolExecutor(max_workers=used) as ex:
        for _ in range(passes):
            t0 = time.perf_counter()
            list(ex.map(phase1, prep))
            t1 = time.perf_counter()
            for p in prep:
                p["kx"], p["vx"] = fetch(p["slots"])
            t2 = time.perf_counter()
            list(ex.map(phase2, prep))
            t3 = time.perf_counter()
            timed += (t1 - t0) + (t3 - t2)
        # untimed: the exact (float64) attention over the oracle's rows, the bar
        # the GPU output is held to
        for p in prep:
            p["out_exact"], _ = oracle.attend_exact(p["q"], p["kx"], p["vx"], scale)
    # one row, one thread, for reference
    p = prep[0]
    t4 = time.perf_counter()
    phase1(p)
    phase2(p)
    one_row = time.perf_counter() - t4
    res = dict(value=passes * len(rows) / timed, unit="queries/s", cores=used, kind="oracle",
               sample=f"all {len(rows)} rows of one decode step of the same workload, "
                      f"{passes} times (score+select+emit+resolve, then F32 online attention "
                      f"over the oracle's own gathered rows; pooling and the K/V row copy "
                      f"untimed); one sequential row per thread",
               affinity_cores=threads, host_cpus=os.cpu_count(),
               single_thread_row_s=one_row, cpu=cpu_description(), seconds=timed)
    return res, prep


def parity_report(case, prep):
    """The GPU step's rows against the oracle's (reported, not gated here; the
    GPU tests gate it): selected IDs bit for bit, attention error normwise
    (the 2e-6 bar) and elementwise (floor 1e-6 max|o|) against the exact
    attention over the oracle's own rows."""
    import numpy as np
    from tests import harness
    ids = case.token_ids.cpu().numpy()
    width = case.width.cpu().numpy()
    out = case.out.cpu().numpy()
    same, norm, elem = 0, 0.0, 0.0
    for p in prep:
        r = p["row"]
        e = p["ids"]
        same += int(width[r] == len(e) and np.array_equal(ids[r, :len(e)], e))
        norm = max(norm, harness.normwise_rel_err(out[r], p["out_exact"]))
        elem = max(elem, harness.elementwise_rel_err(out[r], p["out_exact"]))
    return {"rows": len(prep), "ids_bitexact_rows": same, "max_normwise_err": norm,
            "max_elementwise_err": elem, "bar_normwise": 2e-6,
            "reference": "oracle IDs; float64 attention over the oracle's rows"}


def chunk_leg(seed, steps):
    """Causal chunks: 8 sequences of lengths drawn from [2,051, 262,144], 256
    queries each (2,048 rows, rows_in_flight 256), indexer 16 x 128, attention
    32 q / 4 KV x 128.  Times one qsa_decode call over all rows with the
    per-row compact gather, the union gather and the fused attention, checks
    the three give identical bits, and counts the K/V rows each one copies."""
    import numpy as np
    import torch
    from tests import harness, inputs
    spec = inputs.spec("chunk_8x256", seed=seed)
    data = inputs.make(spec, seed=seed, device="cuda")
    case = harness.GpuCase(data, rows_in_flight=256)
    rows = spec.rows
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    res, ref = {}, None
    for mode in ("compact", "dedup", "fused"):
        case.decode(rows=mode)
        torch.cuda.synchronize()
        start.record()
        for _ in range(steps):
            case.decode(rows=mode)
        stop.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop) / steps
        got = case.results()
        if ref is None:
            ref = got
        else:
            assert all(torch.equal(a, b) for a, b in zip(got, ref)), f"{mode} differs"
        res[mode] = {"ms_per_step": ms, "rows_per_s": rows / (ms * 1e-3)}
    ids = ref[0].cpu().numpy()
    width = ref[1].cpu().numpy()
    union_groups = 0
    for b in range(spec.batch):
        blk = ids[b * spec.queries:(b + 1) * spec.queries]
        union_groups += len(np.unique(blk[blk >= 0] // 4))
    kv_row = spec.h_kv * spec.d * 4
    res["compact"]["kv_rows_copied"] = int(width.sum())
    res["dedup"]["kv_rows_copied"] = 4 * union_groups
    res["fused"]["kv_rows_copied"] = 0
    for m in ("compact", "dedup"):
        res[m]["kv_copy_bytes"] = 2 * 2 * kv_row * res[m]["kv_rows_copied"]  # K+V, read+write
    res["score_mfma"] = chunk_score_roofline(case, steps)
    return {"workload": "causal chunks: 8 sequences, lengths U[2,051, 262,144] (seeded), 256 "
                        "queries each, budget 512, indexer 16 x 128, attention 32 q / 4 KV x "
                        "128, identity slot maps, 256 rows in flight",
            "rows": rows, "steps": steps, **res}


def chunk_score_roofline(case, reps):
    """The chunk scoring kernel alone (fp32 MFMA, every row of the chunk
    workload): algorithmic flops = sum over rows of 2 x H_I x D_I x G_row,
    against MI355X's dense fp32 matrix peak."""
    import torch
    import top_sparse_attention_qsa_amd as qsa
    from tests import inputs
    s = case.spec
    sh = case.shape
    approx = torch.empty((s.rows, sh.max_groups), device="cuda")
    bound = torch.empty_like(approx)
    ms = time_calls(lambda: qsa.qsa_score_groups_chunk(sh, case.index_q, case.pooled,
                                                       case.pooled_off, case.seq_len, approx,
                                                       bound), reps)
    groups = sum(inputs.row_tokens(s, r) // 4 for r in range(s.rows))
    flop = 2.0 * s.h_i * s.d_i * groups
    achieved = flop / (ms * 1e-3) / 1e12
    del approx, bound
    return {"kernel": f"chunk_score_kernel<{s.h_i},{s.d_i}>", "bound": "mfma", "ms": ms,
            "algorithmic_flop": flop, "achieved": achieved, "peak": MFMA_FP32_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved / MFMA_FP32_PEAK_TFLOPS,
            "note": "qsa_score_groups_chunk over every row, v_mfma_f32_16x16x4_f32"}


def time_calls(fn, reps):
    """Mean milliseconds of fn() over reps calls, bracketed by synchronizations."""
    import torch
    fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def pool_leg(case, raw_keys, reps=5):
    """Group pooling of the decode batch on the GPU: 32 x 262,144 raw index
    keys of 128 floats (4 GiB) into the tiled pooled keys (1 GiB); the result
    must equal the pooled keys the inputs were built with."""
    import torch
    import top_sparse_attention_qsa_amd as qsa
    out = torch.empty_like(case.pooled)
    ms = time_calls(lambda: qsa.qsa_pool_groups(case.shape, raw_keys, case.raw_off, case.seq_len,
                                                None, out, case.pooled_off), reps)
    assert torch.equal(out, case.pooled), "pooling differs from the input build"
    s = case.spec
    groups = sum(n // 4 for n in s.seq_lens)
    nbytes = groups * s.d_i * 4 * 5  # four raw rows read, one pooled row written
    del out
    return {"ms": ms, "algorithmic_bytes": nbytes, "gbps": nbytes / (ms * 1e-3) / 1e9,
            "note": "qsa_pool_groups over every complete group of the decode batch"}


def dense_leg(case, reps=20):
    """The bounded dense row on the GPU (every visible token, no selection)
    at its largest width: the decode batch's 32 rows cut to 2,051 visible
    tokens, through the same gather, attention and merge."""
    import torch
    import top_sparse_attention_qsa_amd as qsa
    s = case.spec
    seq = torch.full_like(case.seq_len, 4 * s.budget + 3)
    ids = torch.empty_like(case.token_ids)
    width = torch.empty_like(case.width)
    out = torch.empty_like(case.out)
    lse = torch.empty_like(case.lse)
    ms = time_calls(lambda: qsa.qsa_dense_attend(case.shape, seq, case.slot_map, case.slot_off,
                                                 case.k_cache, case.v_cache, case.q, case.scale,
                                                 ids, width, out, lse, case.workspace), reps)
    assert int(width.min()) == 4 * s.budget + 3 and int(width.max()) == 4 * s.budget + 3
    return {"ms": ms, "rows_per_s": s.rows / (ms * 1e-3), "width": 4 * s.budget + 3,
            "note": "qsa_dense_attend, 32 rows of 2,051 visible tokens each"}


def cpu_description():
    """What /proc/cpuinfo says about the host CPU (model name, family, model,
    stepping, logical CPUs listed)."""
    info, n = {}, 0
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" not in line:
                    continue
                k, v = (x.strip() for x in line.split(":", 1))
                if k == "processor":
                    n += 1
                elif k in ("model name", "vendor_id", "cpu family", "model", "stepping",
                           "cpu MHz", "cache size") and k not in info:
                    info[k] = v
    except OSError:
        pass
    info["logical_cpus_listed"] = n
    return info


def copy_calibration(gib=1.0, reps=5):
    """A plain device copy of known size, for scaling FETCH_SIZE/WRITE_SIZE."""
    import torch
    n = int(gib * (1 << 30)) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "reps": reps}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-chunk", action="store_true",
                    help="skip the causal-chunk leg (compact vs union gather vs fused)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter scale factor)")
    ap.add_argument("--chunk-only", action="store_true",
                    help="only run the causal-chunk leg and print its JSON (for profiling)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this path runs on a single MI355X and has no "
              f"multi-GPU leg (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import top_sparse_attention_qsa_amd as qsa
    from tests import harness, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    qsa.lib()  # fails loudly if the HIP library is missing
    if args.copy_calibration:
        copy_calibration()
        return
    if args.chunk_only:
        print(json.dumps({"chunk": chunk_leg(args.seed, steps=5)}))
        return

    spec = inputs.spec("decode_32x262144")
    print(f"[bench] generating {spec.name} on cuda:0 (seed {args.seed})", file=sys.stderr,
          flush=True)
    data = inputs.make(spec, seed=args.seed, device="cuda")
    case = harness.GpuCase(data)
    rows = spec.rows
    print("[bench] pooling leg", file=sys.stderr, flush=True)
    pool = pool_leg(case, data["raw_keys"])
    keep_raw = not args.no_cpu_baseline
    if not keep_raw:
        data["raw_keys"] = None
    torch.cuda.synchronize()

    # Settle: after an idle gap the GPU runs about 9% slower for its first
    # ~25 steps (clock and power management; measured on this part), so the
    # timed steps are preceded by a fixed duration of untimed steps, then the
    # W warmup steps.  Both are reported.
    print(f"[bench] settle {SETTLE_MS} ms, then warmup {args.warmup}", file=sys.stderr,
          flush=True)
    def run_for(fn, ms=SETTLE_MS):
        """Untimed calls of fn for a fixed duration; returns (ms, calls)."""
        n, t0 = 0, time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < ms:
            for _ in range(10):
                fn()
            n += 10
            torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3, n

    settle_ms, settle_steps = run_for(case.decode)
    settle = {"ms": settle_ms, "steps": settle_steps,
              "note": "untimed decode steps of a fixed duration before the warmup steps (and "
                      "before the fused and graph legs): the first ~25 steps after an idle gap "
                      "run ~9% slower on this part"}
    for _ in range(args.warmup):
        case.decode()
    torch.cuda.synchronize()

    def timed_loop(fused):
        """K steps bracketed by synchronizations, with nothing else on the
        stream (a recorded HIP event costs the stream several microseconds)."""
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            case.decode(fused=fused)
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / args.steps

    def stage_loop(fused):
        """Per-kernel times: K more steps with a HIP event recorded on the
        launch stream at every stage boundary (these steps run slower than
        the timed ones; each stage interval is one kernel).  Returns the mean
        per stage and the p10/p50/p90 of the per-step and score-kernel times."""
        timer = qsa.Timer(args.steps)
        for _ in range(args.steps):
            case.decode(timer, fused=fused)
        torch.cuda.synchronize()
        stage = timer.read()
        timer.close()
        means = {name: sum(c[i] for c in stage) / len(stage)
                 for i, name in enumerate(qsa.STAGE_NAMES)}
        pct = lambda v: {f"p{q}": float(np.percentile(v, q)) for q in (10, 50, 90)}
        spread = {"step_ms": pct([sum(c) for c in stage]), "score_ms": pct([c[0] for c in stage])}
        return means, spread

    def step_loop():
        """K more steps with one event at every step boundary: the per-step
        spread next to the timed mean (each event adds a little to its step)."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(args.steps):
            case.decode()
            ev[i + 1].record()
        torch.cuda.synchronize()
        d = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
        return {"mean": float(np.mean(d)),
                **{f"p{q}": float(np.percentile(d, q)) for q in (10, 50, 90)},
                "note": "one HIP event per step boundary, K steps after the timed ones"}

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    ms_per_step = timed_loop(False)
    step_spread = step_loop()
    stage_ms, stage_spread = stage_loop(False)
    score_ms = stage_ms["score"]

    # the same step with the gather fused into the attention (no compact scratch)
    print(f"[bench] timing {args.steps} fused steps", file=sys.stderr, flush=True)
    ref_out = case.out.clone()
    run_for(lambda: case.decode(fused=True))
    for _ in range(args.warmup):
        case.decode(fused=True)
    fused_ms = timed_loop(True)
    fused_stage_ms, _ = stage_loop(True)
    assert torch.equal(case.out, ref_out), "fused path differs from the compact path"

    # the compact step captured once in a HIP graph and replayed K times (a
    # decode call enqueues kernel launches only, so it can be captured)
    print(f"[bench] timing {args.steps} graph replays", file=sys.stderr, flush=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        case.decode()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        case.decode()
    case.out.fill_(float("nan"))
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(case.out, ref_out), "graph replay differs from the eager step"
    run_for(graph.replay)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        graph.replay()
    stop.record()
    torch.cuda.synchronize()
    graph_ms = start.elapsed_time(stop) / args.steps
    assert torch.equal(case.out, ref_out), "graph replay differs from the eager step"
    del graph

    alg = algorithmic_bytes()
    step_bytes = sum(alg.values())
    overhead = implementation_overhead_bytes()
    score_bytes = score_roofline_bytes()
    achieved = score_bytes / (score_ms * 1e-3) / 1e9
    traffic = measured_traffic()
    stage_traffic = measured_step_traffic()
    step_traffic = None
    if stage_traffic:
        tb = sum(stage_traffic.values())
        step_traffic = {
            "bytes": tb, "over_algorithmic": tb / step_bytes,
            "over_implementation_bytes": tb / sum(stage_bytes().values()),
            "gbps_over_kernel_time": tb / (sum(stage_ms.values()) * 1e-3) / 1e9,
            "by_stage": stage_traffic,
            "source": "rocprofv3 FETCH_SIZE and WRITE_SIZE per kernel, scaled by a 1 GiB copy "
                      "(profiles/decode_32x262144_counters.md)"}
    print("[bench] context bandwidth", file=sys.stderr, flush=True)
    context = context_bandwidth()
    widths = case.width.cpu()
    assert int(widths.min()) == 2048 and int(widths.max()) == 2048, "unexpected widths"

    result = {
        "metric": METRIC,
        "value": rows / (ms_per_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "decode batch of 32 sequences x 262,144 visible tokens (65,536 groups), "
                        "budget 512 groups, indexer 16 heads x 128, attention 32 q / 4 KV heads "
                        "x 128, shared 8,388,608-slot K/V pool, random per-sequence slot maps",
            "batch": rows, "seq_len": spec.seq_lens[0], "budget_groups": spec.budget,
            "index_heads": spec.h_i, "index_dim": spec.d_i, "q_heads": spec.h_q,
            "kv_heads": spec.h_kv, "head_dim": spec.d, "kv_slots": data["kv_slots"],
        },
        "step_ms_spread": step_spread,
        "settle": settle,
        "step_algorithmic_bytes": step_bytes,
        "step_algorithmic_bytes_by_item": alg,
        "step_hbm_gbps": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "step_frac_of_peak": step_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "step_implementation_overhead_bytes": {**overhead, "total": sum(overhead.values()),
                                               "note": "moved by this implementation on top of "
                                                       "the method's bytes; not in "
                                                       "step_algorithmic_bytes"},
        "stage_ms": stage_ms,
        "stage_ms_note": "HIP events at every stage boundary, in a loop of its own after the "
                         "timed steps",
        "stage_spread": stage_spread,
        "step_traffic": step_traffic,
        "context_bandwidth": context,
        "roofline": {
            "kernel": "score_mfma_kernel<16,128>",
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": score_bytes,
            "algorithmic_bytes_note": "per group: its pooled key (128 floats) read and its score "
                                      "written; per row: its index query (16 x 128 floats)",
            "mean_launch_ms": score_ms,
            "timing": "HIP events on the launch stream around the kernel, averaged over the "
                      "per-stage loop's steps",
        },
        "graph": {
            "note": "the compact step captured in a HIP graph, K replays; bit-identical "
                    "outputs (context: value is the eager K steps)",
            "value": rows / (graph_ms * 1e-3),
            "ms_per_step": graph_ms,
        },
        "fused": {
            "note": "same step with resolve+gather fused into the attention kernel "
                    "(no compact scratch); bit-identical outputs",
            "value": rows / (fused_ms * 1e-3),
            "ms_per_step": fused_ms,
            "algorithmic_bytes": fused_algorithmic_bytes(),
            "frac_of_peak": fused_algorithmic_bytes() / (fused_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "hbm_gbps": fused_algorithmic_bytes() / (fused_ms * 1e-3) / 1e9,
            "stage_ms": fused_stage_ms,
        },
        "cpu_baseline": None,
    }
    print("[bench] dense leg", file=sys.stderr, flush=True)
    result["pool"] = pool
    result["dense"] = dense_leg(case)
    if not args.no_chunk:
        print("[bench] chunk leg", file=sys.stderr, flush=True)
        result["chunk"] = chunk_leg(args.seed, steps=5)
    if keep_raw:
        threads = len(os.sched_getaffinity(0))
        print(f"[bench] cpu baseline: oracle over {rows} rows, {threads} cores in the affinity "
              f"mask", file=sys.stderr, flush=True)
        cb, prep = cpu_baseline(data, list(range(rows)), threads)
        cb.pop("seconds", None)
        result["cpu_baseline"] = cb
        result["parity"] = parity_report(case, prep)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
