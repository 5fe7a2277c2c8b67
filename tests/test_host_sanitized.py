"""The C-ABI's host code under the address and undefined-behaviour sanitizers
(CPU only; device code is never sanitized).

1. tests/host/plan_check.cpp: the planning arithmetic (stage lengths,
   workspace sizes, the receptive-field reach, the streaming tile grid and
   its batched groups) checked exhaustively over small sizes, built with g++
   -fsanitize=address,undefined.
2. The library's host sources (argument checks, decoder planning, the
   no-workspace AMP block's size checks, the launch profiler) built with
   hipcc -Xarch_host -fsanitize=address,undefined and linked with the
   regular kernel objects; tests/test_abi_host.py runs against that build in
   a child process with the sanitizer runtime preloaded."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_plan_arithmetic_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "bigvgan_waveform_decoder_amd", "csrc"),
           os.path.join(ROOT, "tests", "host", "plan_check.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120,
                       env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"})
    assert r.returncode == 0, r.stdout + r.stderr
    assert "plan_check ok" in r.stdout


def test_abi_host_tests_pass_on_the_host_sanitized_library():
    from bigvgan_waveform_decoder_amd import build as B
    try:
        B.hipcc()
        rt = B.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = B.build_host_sanitized()
    env = {**os.environ, "AVAE_LIB_PATH": lib, "LD_PRELOAD": rt,
           "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error" not in out
