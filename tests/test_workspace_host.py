"""CPU test of the library's per-stream workspace under stream capture:
tests/workspace_check.cpp compiles the host library (csrc/lf_host.cpp) with
g++ against stand-ins for the HIP runtime and the kernel launchers, and
checks that a captured call allocates nothing, that growth during capture
is refused, and that later eager calls neither overwrite nor free what a
captured graph uses (see that file)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_long_sequence_lf_amd", "csrc")


def test_workspace_under_capture(tmp_path):
    exe = str(tmp_path / "workspace_check")
    subprocess.check_call(["g++", "-O1", "-g", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-DLF_SOURCE_HASH=\"check\"",
                           "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                           os.path.join(ROOT, "tests", "workspace_check.cpp"), os.path.join(CSRC, "lf_host.cpp"),
                           "-o", exe])
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(res.stdout, res.stderr)
    assert res.returncode == 0 and res.stdout.startswith("OK"), res.stdout + res.stderr
