"""Write the expected column outputs gK[cols], gV[cols] of the two largest
workloads (one head each), computed by the fp64 oracle alone.

    python tests/golden/make_column_goldens.py [--procs 8]

At these sizes one N x N float64 matrix per head is 32 GiB (65,536 tokens) or
512 GiB (262,144 tokens), so the oracle's column routine (bob_cols_head) sweeps
all query rows in blocks: each block forms its rows' scalars D, alpha, E from
all keys in float64, then adds its exact contribution to the sampled columns.
This script only splits the query rows into contiguous ranges, evaluates them in
worker processes and adds the range results in range order (the oracle's own
row_range contract). Inputs come from the shared seeded generator (workload/);
the file records a SHA-256 of each input head so a test can confirm that it
regenerated the same tensors. Nothing here touches the HIP library.
"""

import argparse
import hashlib
import json
import multiprocessing as mp
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workload  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
# (workload, seed, head (b, h), number of random columns, column-sampling seed)
CASES = [("wide_64k", 0, (0, 0), 16, 64), ("endpoint_256k", 0, (0, 0), 16, 256)]
_ARRS = None


def head_arrays(w, seed, b, h):
    cpu = workload.make_inputs(w, seed)
    sha = {n: hashlib.sha256(cpu[n][b, h].contiguous().view(-1).view(torch_uint8()).numpy().tobytes()).hexdigest()
           for n in workload.INPUT_NAMES}
    arrs = [workload.to_f64(cpu[n][b, h]) for n in workload.INPUT_NAMES]
    return arrs, sha


def torch_uint8():
    import torch

    return torch.uint8


def sample_cols(N, count, seed):
    rng = np.random.default_rng(seed)
    cols = rng.choice(N, count, replace=False)
    return np.unique(np.concatenate([cols, [0, N - 1]])).astype(np.int64)


def _work(job):
    r0, r1, tau, causal, cols = job
    out = oracle.bob_cols_head(*_ARRS, tau, causal, cols, row_block=128, row_range=(r0, r1))
    return r0, out["gK"], out["gV"]


def run_case(name, seed, bh, ncols, col_seed, procs):
    global _ARRS
    w = workload.WORKLOADS[name]
    b, h = bh
    arrs, sha = head_arrays(w, seed, b, h)
    cols = sample_cols(w.N, ncols, col_seed)
    _ARRS = arrs  # shared with the forked workers
    chunk = max(128, w.N // (8 * procs))
    jobs = [(r0, min(w.N, r0 + chunk), w.scale, w.causal, cols) for r0 in range(0, w.N, chunk)]
    t0 = time.time()
    with mp.get_context("fork").Pool(procs) as pool:
        parts = dict((r0, (gk, gv)) for r0, gk, gv in pool.imap_unordered(_work, jobs))
    gk = np.zeros((len(cols), w.d))
    gv = np.zeros((len(cols), w.d))
    for r0 in sorted(parts):  # range order
        gk += parts[r0][0]
        gv += parts[r0][1]
    print(f"{name}: {len(cols)} columns in {time.time() - t0:.0f} s", flush=True)
    return {
        "workload": name, "seed": seed, "head": [b, h], "N": w.N, "d": w.d, "dtype": w.dtype,
        "causal": w.causal, "tau": w.scale, "cols": cols.tolist(), "inputs_sha256": sha,
        "gK": [[float(x) for x in row] for row in gk], "gV": [[float(x) for x in row] for row in gv],
        "source": "oracle.bob_cols_head (fp64), written by tests/golden/make_column_goldens.py",
    }


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--procs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--only", default=None)
    args = ap.parse_args(argv)
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    for name, seed, bh, ncols, col_seed in CASES:
        if args.only and name != args.only:
            continue
        res = run_case(name, seed, bh, ncols, col_seed, args.procs)
        path = os.path.join(HERE, f"{name}_columns.json")
        with open(path, "w") as f:
            json.dump(res, f, indent=0)
        print(f"wrote {path}", flush=True)


if __name__ == "__main__":
    main()
