"""libgdn from plain C: compile tests/c/abi_check.c with gcc against include/gdn.h, link the
built library, run it (argument validation only, so no GPU is needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "gated_deltanet_recurrence_rule_amd")


def test_plain_c_program(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libgdn.so")):
        pytest.fail("libgdn.so is not built (run __graft_entry__.build())")
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "abi_check")
    cmd = [cc, "-std=c99", "-O1", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", os.path.join(ROOT, "tests", "c", "abi_check.c"), "-o", exe,
           "-L", LIBDIR, "-lgdn", "-Wl,-rpath," + LIBDIR]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all ok" in r.stdout
