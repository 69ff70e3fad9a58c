"""The C ABI's host code (argument checks, workspace sizing, split choice, error
reporting) built with AddressSanitizer and UndefinedBehaviorSanitizer and run on
the CPU over extreme shapes (tests/sanitize/host_checks.cpp). Only the host pass
is instrumented; the kernel launches are stubs and no call reaches the device,
so no GPU is involved."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "aware_flashbob_pass_amd", "csrc")


def _hipcc():
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.timeout(600)
def test_host_checks_under_asan_ubsan(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "host_checks")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    # api.cpp holds one device array (the fixed scratch of the no-allocation entry
    # point), so it is compiled for gfx950 as in the library; only the host pass is
    # instrumented (every -fsanitize is behind -Xarch_host)
    cmd = [hipcc, "-x", "hip", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-O1", "-g", "-std=c++17", *san,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "api.cpp"), os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out
    assert "ok: 0 failures" in out
    assert "runtime error" not in out and "AddressSanitizer" not in out
