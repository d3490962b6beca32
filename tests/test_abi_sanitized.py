"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's host side (argument checks, planning, workspace carving, status strings) is
rebuilt with both sanitizers, and the CPU ABI checks in test_abi.py run against it in a child
process with the ASan runtime preloaded.  Any sanitizer report stops the child with a non-zero
status; the report itself is printed because the child runs pytest without output capture.
No kernel is launched: those checks never reach a device call.
"""
import os
import subprocess
import sys

import pytest

from gated_delta_rule_73_amd import build as gbuild

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _toolchain_ready():
    try:
        rt = gbuild.asan_runtime()
    except Exception:
        return None
    return rt if rt and os.path.isabs(rt) and os.path.exists(rt) else None


@pytest.mark.slow
def test_abi_checks_clean_under_sanitizers():
    rt = _toolchain_ready()
    if rt is None:
        pytest.skip("no clang ASan runtime in this toolchain")
    lib = gbuild.build_sanitized()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        "GDR_LIBRARY": lib,
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "PYTHONPATH": ROOT + os.pathsep + env.get("PYTHONPATH", ""),
    })
    cmd = [sys.executable, "-m", "pytest", os.path.join(HERE, "test_abi.py"), "-q", "-x", "-s",
           "-p", "no:cacheprovider", "-m", "not gpu"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "runtime error:" not in out, out[-6000:]
    assert "AddressSanitizer" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in out, out[-2000:]
