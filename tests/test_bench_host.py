"""Host-side checks of bench.py (no GPU): the one-GPU contract and the
algorithmic byte counts the roofline divides by."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_of_the_decode_step():
    """The method's bytes for one step of the 32 x 262,144 decode batch: the
    scope table's items, 1,898,446,848 B in all, and 1,361,575,936 B when the
    compact copy is fused away."""
    a = bench.algorithmic_bytes()
    B, G, d_i, h_i, h_q, d, W, kv_row = 32, 65536, 128, 16, 32, 128, 2048, 4 * 128 * 4
    assert a["pooled_keys"] == B * G * d_i * 4              # 1 GiB, read once
    assert a["scores"] == 2 * B * G * 4                      # written and read once
    assert a["kv_rows_read"] == 2 * B * W * kv_row           # selected K and V rows
    assert a["compact_write_read"] == 2 * 2 * B * W * kv_row
    # index q, attention q, out, a selection bitmap written and read, token IDs
    # written and read, slot-map entries
    assert a["small"] == (B * h_i * d_i * 4 + 2 * B * h_q * d * 4 + 2 * B * G // 8
                          + 2 * B * W * 4 + B * W * 4)
    assert sum(a.values()) == 1_898_446_848
    assert bench.fused_algorithmic_bytes() == 1_361_575_936
    # the scoring kernel's own bytes: pooled keys, scores written, index queries
    assert bench.score_roofline_bytes() == B * G * (d_i * 4 + 4) + B * h_i * d_i * 4
    # what each kernel moves, overhead included, is the method's bytes plus
    # the overhead up to the small per-row vectors counted per kernel
    over = sum(bench.implementation_overhead_bytes().values())
    assert abs(sum(bench.stage_bytes().values()) - (sum(a.values()) + over)) < 1 << 20
