"""CPU tier: the host metadata code of libvlp (host_meta.cpp) built with the
host compiler under AddressSanitizer and UndefinedBehaviorSanitizer and run
through a fuzz driver (tests/native/host_meta_fuzz.cpp) that checks the
packing and ragged-grid invariants and every documented error path.  Any
out-of-bounds access, overflow or other undefined behaviour aborts the run."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CXX = shutil.which("g++")


@pytest.mark.skipif(CXX is None, reason="no host C++ compiler")
def test_host_metadata_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = tmp_path / "host_meta_fuzz"
    cmd = [CXX, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "tests", "native", "host_meta_fuzz.cpp"),
           os.path.join(ROOT, "variable_length_packed_pack_amd", "csrc", "host_meta.cpp"),
           "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    res = subprocess.run([str(exe), "3000"], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failed checks" in res.stdout
