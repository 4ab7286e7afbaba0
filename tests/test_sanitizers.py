"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Three programs are built with -fsanitize=address,undefined and any report
fails: the fp64 oracle driven over the kinds of inputs its pins use
(tests/sanitize/oracle_cases.c), the C entry points' argument checks with the
kernel launchers stubbed out (tests/sanitize/abi_cases.cpp), and the tile-copy
bounds walk of the fused kernel (tests/address_bounds.cpp)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, args=()):
    out = subprocess.run([*cmd, *args], capture_output=True, text=True, env=ENV)
    text = out.stdout + out.stderr
    print(text[-4000:])
    assert out.returncode == 0, text[-4000:]
    for marker in ("runtime error", "AddressSanitizer", "LeakSanitizer"):
        assert marker not in text, text[-4000:]
    return text


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_cases")
    subprocess.run(["gcc", *SAN, "-std=c99", "-fopenmp", "-ffp-contract=off",
                    os.path.join(ROOT, "oracle", "resolvent_oracle.c"),
                    os.path.join(ROOT, "tests", "sanitize", "oracle_cases.c"), "-o", exe, "-lm"],
                   check=True)
    assert "0 failures" in run([exe])


@pytest.mark.skipif(not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"),
                    reason="needs the HIP runtime headers for the entry points' types")
def test_entry_point_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_cases")
    csrc = os.path.join(ROOT, "gated_causal_attention_amd", "csrc")
    subprocess.run(["g++", *SAN, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
                    "-I", os.path.join(ROOT, "include"), "-I", csrc,
                    os.path.join(csrc, "resolvent_abi.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "abi_cases.cpp"), "-o", exe],
                   check=True)
    assert "0 failures" in run([exe])


def test_copy_bounds_under_sanitizers(tmp_path):
    exe = str(tmp_path / "address_bounds")
    subprocess.run(["g++", *SAN, "-std=c++17", "-I",
                    os.path.join(ROOT, "gated_causal_attention_amd", "csrc"),
                    os.path.join(ROOT, "tests", "address_bounds.cpp"), "-o", exe], check=True)
    shapes = []
    for n in (1, 63, 64, 65, 257, 1000):
        for d in (64, 128):
            shapes += [2, 2, n, d]
    run([exe, *map(str, shapes)])


def test_gcc_available():
    assert shutil.which("gcc") and shutil.which("g++")
