"""The microbenchmarks and skeleton kernels behind the kernels' bound analysis
(aware_flashbob_pass_amd/csrc/microbench/probes_gen.py, run by `bench.py --microbench`)
generate and compile for gfx950 (no GPU needed)."""

import importlib.util
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEN = os.path.join(ROOT, "aware_flashbob_pass_amd", "csrc", "microbench", "probes_gen.py")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _gen():
    spec = importlib.util.spec_from_file_location("probes_gen", GEN)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_skeleton_lds_addresses_in_bounds():
    """Every LDS read of a skeleton stays inside its 64 KiB allocation (address register
    at most 1008 bytes, read width at most 16 bytes)."""
    import re
    mod = _gen()
    for name, (ins, _), _ in mod.SKELETONS:
        for x in ins:
            m = re.search(r"offset:(\d+)", x)
            if x.startswith("ds_read"):
                off = int(m.group(1)) if m else 0
                assert off + 1008 + 16 <= 65536, (name, x)


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="hipcc not available")
def test_probe_program_compiles(tmp_path):
    src = tmp_path / "microbench_probes.hip"
    src.write_text(_gen().render())
    res = subprocess.run([HIPCC, "-O3", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
                          "-packed-fp32-ops", "-c", str(src), "-o", str(tmp_path / "p.o")], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
