"""Native checks of host-side internals: the planner and the staging ring
(compiled with g++, CPU only)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_fused_worklist_equals_stepwise_plan(tmp_path):
    exe = tmp_path / "worklist_check"
    csrc = os.path.join(ROOT, "block_copy_amd", "csrc")
    subprocess.run(["g++", "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I" + os.path.join(ROOT, "include"), "-I" + csrc,
                    os.path.join(ROOT, "tests", "native", "worklist_check.cpp"),
                    os.path.join(csrc, "plan.cpp"), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok")


def test_planner_under_sanitizers(tmp_path):
    """The same check built with AddressSanitizer and UBSan (host code only)."""
    exe = tmp_path / "worklist_check_asan"
    csrc = os.path.join(ROOT, "block_copy_amd", "csrc")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I" + os.path.join(ROOT, "include"), "-I" + csrc,
                    os.path.join(ROOT, "tests", "native", "worklist_check.cpp"),
                    os.path.join(csrc, "plan.cpp"), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe), "250"], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr


def test_staging_ring_never_hands_out_bytes_in_use(tmp_path):
    exe = tmp_path / "ring_check"
    csrc = os.path.join(ROOT, "block_copy_amd", "csrc")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I" + csrc,
                    os.path.join(ROOT, "tests", "native", "ring_check.cpp"), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok")
