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
    a = bench.algorithmic_bytes()
    B, G, d_i, h_i, W, kv_row = 32, 65536, 128, 16, 2048, 4 * 128 * 4
    # step 1 reads every pooled key once and writes one score and one
    # 16-group maximum per group (plus the index queries)
    assert a["score"] == B * G * d_i * 4 + B * h_i * d_i * 4 + B * G * 4 + B * (G // 16) * 4
    # steps 6-7 read and write each selected K and V row once
    assert a["resolve_gather"] >= 4 * B * W * kv_row
    # step 8 reads each compact row once
    assert a["attend_chunks"] >= 2 * B * W * kv_row
    # the fused variant drops the compact write and re-read: 2 x 256 MiB less
    assert sum(a.values()) - bench.fused_algorithmic_bytes() == \
        2 * 2 * B * W * kv_row + B * W * 4 * 2 + B * W * 4 - B * W * 4 * 2
