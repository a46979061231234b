"""The C-ABI layer under AddressSanitizer, on the CPU.

The host units (argument checks, workspace plans, error strings, the fixed
scratch lookup's host side) are rebuilt with AddressSanitizer into a copy of
the library outside the package; tests/test_abi.py then runs in a child
process against that copy with the sanitizer's runtime preloaded.  Any
out-of-bounds or use-after-free access in the host code aborts the child
with a sanitizer report.  No GPU is touched: the ABI tests stop at the host
checks or at calls that need no device.
"""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "loglin_build", os.path.join(ROOT, "ssm_scan_amd", "csrc", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_abi_tests_clean_under_host_asan():
    b = _build_module()
    if not os.path.exists(os.path.join(b.BUILD_DIR, "loglin_inst_bf16_64.o")):
        pytest.skip("the library's objects are not built (run build() first)")
    lib = b.build_host_asan()
    rt = b.asan_runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ)
    env["LOGLIN_LIB"] = lib
    env["LD_PRELOAD"] = rt + ((":" + env["LD_PRELOAD"]) if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    res = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
         os.path.join(ROOT, "tests", "test_abi.py")],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in res.stdout, out[-2000:]
