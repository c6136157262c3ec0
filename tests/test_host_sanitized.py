"""Host ASan/UBSan lane for libqsa.so's host side (the notes' host sanitizer
lanes, AFN-016 "A sparse mask is not sparse attention", capsule evidence):
api.cpp -- validation, workspace layout, launch chains, stage timer, byte
ledger -- is built with g++ -fsanitize=address,undefined against recording
stub launchers (tests/host_lane/) and driven through every validation path.
No GPU and no HIP runtime are involved: the stub touches no memory."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LANE = os.path.join(ROOT, "tests", "host_lane")
CSRC = os.path.join(ROOT, "top_sparse_attention_qsa_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_side_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_lane")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(LANE, "driver.cpp"), os.path.join(LANE, "stub_launch.cpp"),
                    os.path.join(CSRC, "api.cpp"), "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout, r.stdout
    assert r.stderr.strip() == "", r.stderr
