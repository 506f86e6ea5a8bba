"""The CPU oracle and the library's host-compilable exact-rescoring header built with AddressSanitizer and
UndefinedBehaviorSanitizer (g++/gcc on the host; no GPU code is involved) and run by a small driver
(tests/native/sanitize_driver.cpp): every oracle routine on small inputs, and the header's exact dot products
and indexer scores bit-equal to the oracle's.  Any memory error or undefined behaviour aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="no host compiler")
def test_sanitized_oracle_and_exact_dot(tmp_path):
    obj = tmp_path / "oracle.o"
    exe = tmp_path / "sanitize_driver"
    subprocess.check_call(["gcc", "-std=c99", *SAN, "-ffp-contract=off", "-c", os.path.join(ROOT, "oracle", "oracle.c"),
                           "-o", str(obj)])
    subprocess.check_call(["g++", "-std=c++17", *SAN, "-ffp-contract=off",
                           "-I", os.path.join(ROOT, "compressed_sparse_kv_compressor_amd", "csrc"),
                           os.path.join(ROOT, "tests", "native", "sanitize_driver.cpp"), str(obj), "-lm", "-o", str(exe)])
    # (verify_asan_link_order=0: the environment may preload a library ahead of the sanitizer runtime)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "clean and equal" in r.stdout
