"""Host-side checks of the projection planner (CPU).

`plan_check.cpp` is compiled against the library's headers and linked to the
built libmoetail.so; it walks batch sizes 1..128, the shapes of the tail and
of the tests, and the tuning overrides, and checks every plan against what
its kernels assume (K covered by the slices, the LDS, units held per wave,
grid size).  Without a GPU the planner assumes 256 CUs, as on MI355X.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "expert_finalize_rmsnorm_amd")
LIB = os.path.join(PKG, "libmoetail.so")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_projection_plans_satisfy_kernel_assumptions(tmp_path):
    if not os.path.exists(LIB):
        pytest.fail("libmoetail.so is not built (run __graft_entry__.build())")
    exe = str(tmp_path / "plan_check")
    cmd = ["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(PKG, "csrc"),
           os.path.join(ROOT, "tests", "plan_check.cpp"), "-L" + PKG, "-lmoetail",
           "-Wl,-rpath," + PKG, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, HIP_VISIBLE_DEVICES="")  # the plans of the default 256 CUs
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-2000:]
    assert "0 failures" in r.stdout
