"""Build libflashbob.so (gfx950) in-tree with hipcc.

Usage: python -m aware_flashbob_pass_amd.build [--verbose] [--resource-usage]
Every call recompiles all sources (objects go to aware_flashbob_pass_amd/_build/).
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libflashbob.so")
ARCH = "gfx950"

SOURCES = ["attn_fwd.hip", "bob_pass1.hip", "bob_pass1_vgpr.hip", "pass1_q16.hip", "bob_pass2.hip", "bob_pass2_vgpr.hip",
           "attn_bwd.hip", "probes.hip", "api.cpp"]

# Packed fp32 VALU ops are disabled: the kernels are written with scalar fp32
# element-wise math and must not be auto-vectorised into v_pk_* forms.
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-result",
]


# Per-source extra flags. The statistics kernels are compiled without NaN
# semantics: their running row maxima then need no quieting (canonicalising)
# instruction in front of each v_max, which is about 16 VALU instructions per
# 32-key step. Maxima of finite values are exact either way. The one test for a
# non-finite value in that file (the lazy rescale trigger) compares bit patterns
# as integers, which that flag does not touch; api.cpp checks its arguments with
# NaN semantics intact. Inputs are assumed finite.
# The two-pass sweeps of pass 1 (16-bit: d = 64 in bob_pass1_vgpr.hip, the 16-query
# d = 128 kernel in pass1_q16.hip) and the non-causal d = 128 sweep of pass 2 take the
# matrix-core VGPR form for their score products (their accumulators are AGPR inline
# assembly); the flag applies to their whole files, which hold nothing else with
# matrix-core products (pass1_q16.hip's merge kernel has none).
EXTRA_FLAGS = {"attn_fwd.hip": ["-fno-honor-nans"], "bob_pass1_vgpr.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "bob_pass2_vgpr.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "pass1_q16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src, verbose, resource_usage):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if resource_usage and src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = res.stdout + res.stderr
    out = "\n".join(l for l in out.splitlines() if "unknown target feature" not in l and "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    return obj, out


def build(verbose=False, resource_usage=False, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose, resource_usage), SOURCES))
    logs = [log for _, log in results if log.strip()]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *[o for o, _ in results]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    return LIB, "\n".join(logs)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    args = ap.parse_args(argv)
    lib, log = build(args.verbose, args.resource_usage)
    if log and (args.verbose or args.resource_usage):
        print(log)
    print(lib)


if __name__ == "__main__":
    sys.exit(main())
