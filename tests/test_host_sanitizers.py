"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): kvq_api.cpp is built with g++ against tests/host_check/
kvq_launch_check.cpp, whose stubs stand in for the kernel launches and check
every launch's index ranges against the kvq_layout buffer sizes, the ring
liveness of the fp16 tokens an attention launch reads and the 32-bit offsets,
over a sweep of the supported shapes up to 2^25 tokens; its main program also
runs the validation paths of every entry point.  A planted mistake (a buffer
registered 16 bytes short) must make the checker abort."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_token_amd", "csrc")
CHECK = os.path.join(ROOT, "tests", "host_check", "kvq_launch_check.cpp")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path_factory.mktemp("host_check") / "kvq_launch_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(CSRC, "kvq_api.cpp"), CHECK, "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=600)
    return exe


def _run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([exe, *args], capture_output=True, text=True, timeout=600, env=env)


def test_host_code_under_sanitizers(checker):
    r = _run(checker)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "validation cases: ok" in r.stdout and "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr


@pytest.mark.parametrize("buf", ["k_codes", "v_scale", "k_zero", "v_resid", "k_sink", "workspace", "out"])
def test_planted_short_buffer_is_caught(checker, buf):
    r = _run(checker, "--shrink", buf)
    assert r.returncode != 0
    assert "CHECK FAILED" in r.stderr and "overrun " + buf in r.stderr, r.stderr[-2000:]
