"""Host ASan/UBSan lane for the CPU oracle (the notes' host sanitizer lanes,
AFN-016 "A sparse mask is not sparse attention", capsule evidence): the
self-test driver is built with gcc -fsanitize=address,undefined and must run
clean."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_selftest_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_selftest")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-I", ORACLE,
                    os.path.join(ORACLE, "selftest.c"), os.path.join(ORACLE, "qsa_oracle.c"),
                    "-o", exe, "-lm"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle selftest: ok" in r.stdout
