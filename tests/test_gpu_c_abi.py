"""The path driven from plain C on the GPU (tests/c/abi_gpu_roundtrip.c):
device memory from the HIP runtime's C API and every call through the C
ABI, no Python binding or torch involved.  With identity experts and exact
binary-fraction weights summing to 1 the combine must return x bit for bit
(separate calls with one- and two-launch layouts, the fused entry point,
the replica-aware fused entry point, and kernel times through
moe_time_next_launches)."""

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_c_program_round_trip(tmp_path):
    import combine_moe_dispatch_layout_amd as moe
    lib = moe.library_path()
    exe = tmp_path / "abi_gpu_roundtrip"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_gpu_roundtrip.c"), "-o", str(exe), lib,
                    f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib",
                    f"-Wl,-rpath,{os.path.dirname(lib)}"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    print(out.stdout)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.strip().endswith("ok")
