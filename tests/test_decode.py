"""CPU test of the task decode the tile kernel runs: tests/decode_check.cpp
compiles the library's lf_decode.h with g++ and checks every division by a
call constant and every band / global-row task decode (see that file)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_decode_check(tmp_path):
    exe = str(tmp_path / "decode_check")
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"),
                           "-I", os.path.join(ROOT, "sparse_long_sequence_lf_amd", "csrc"),
                           os.path.join(ROOT, "tests", "decode_check.cpp"), "-o", exe])
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(res.stdout)
    assert res.returncode == 0 and res.stdout.startswith("OK"), res.stdout
