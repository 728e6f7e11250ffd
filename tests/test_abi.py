"""The host-side C ABI checks (tests/abi_host_checks.py), run in a child
process that sees no GPU.

Those checks hand fake device addresses to the real library and rely on its
validation refusing every call before a launch.  With HIP_VISIBLE_DEVICES
empty no kernel can launch, so a validation regression fails on the host
instead of faulting a device, also where this suite runs on a GPU machine.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_host_checks_without_a_device():
    env = dict(os.environ, HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join("tests", "abi_host_checks.py"),
                        "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-6000:] + r.stderr[-2000:]
    assert " passed" in r.stdout and " failed" not in r.stdout
