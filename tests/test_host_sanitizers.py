"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The prefix cache's control plane (prefix_cache.cpp, plain C++ with no device
code) is compiled by g++ together with the randomised driver
tests/prefix_cache_stress.cpp and run: any out-of-bounds access, use after
free, leak or undefined behaviour aborts the run, and the driver checks the
C ABI's contract on every call.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _build(tmp_path, sources, name):
    exe = str(tmp_path / name)
    cmd = ["g++", "-std=c++17", "-O1", "-g", *SAN, *sources, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_prefix_cache_under_sanitizers(tmp_path):
    probe = tmp_path / "probe.cpp"
    probe.write_text("int main() { return 0; }\n")
    r = subprocess.run(["g++", *SAN, str(probe), "-o", str(tmp_path / "probe")], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("the sanitizer runtimes are not available: " + r.stderr[-300:])
    exe = _build(tmp_path, [os.path.join(ROOT, "mqa_attention_int8_amd", "csrc", "prefix_cache.cpp"),
                            os.path.join(ROOT, "tests", "prefix_cache_stress.cpp")], "stress")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "prefix cache stress ok" in r.stdout
