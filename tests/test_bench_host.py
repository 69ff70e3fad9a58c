"""Host-side logic of bench.py (no GPU): the FLOP model, the transfer-ledger terms
the HBM summaries are compared with, and the one-GPU guard."""

import os
import subprocess
import sys

import bench
import workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_flop_unit_counts_key_query_pairs():
    w = workload.custom(2, 3, 100, 64, "bf16", False)
    assert bench.flop_unit(w) == 2.0 * 2 * 3 * 64 * 100 * 100
    wc = workload.custom(2, 3, 100, 64, "bf16", True)
    assert bench.flop_unit(wc) == 2.0 * 2 * 3 * 64 * (100 * 101 // 2)
    assert bench.UNITS["exec"] == bench.UNITS["stats"] + bench.UNITS["pass1"] + bench.UNITS["pass2"]
    assert bench.UNITS["two_pass"] == bench.UNITS["pass1"] + bench.UNITS["pass2"]


def test_ledger_fixed_terms_are_12Nd_plus_4N():
    """Review page, Strengths (Theorem 4.3): the fixed part is 12Nd + 4N elements per
    head; 16-bit tensors at 2 bytes, float32 row vectors at 4 bytes."""
    for N, d in ((1000, 64), (16384, 64), (65536, 128)):
        led = bench.ledger_terms(N, d)
        fixed = led["pass1"][0] + led["pass2"][0]
        assert fixed == 12 * N * d * 2 + 4 * N * 4
        # pass 1 reads Q, dO, UQ, O and L, D; writes gQ, gdO and alpha, E
        assert led["pass1"][0] == 6 * N * d * 2 + 4 * N * 4
        assert led["pass2"][0] == 6 * N * d * 2


def test_ledger_streamed_terms():
    """4dN^2/B_r (K, V, UK, UV per query tile) and (3d + 4)N^2/B_c (Q, dO, UQ and four
    row scalars per key tile), with the tiles of the kernels (128) unless given."""
    N, d = 16384, 64
    led = bench.ledger_terms(N, d)
    assert led["pass1"][1] == 4 * d * N * N / 128 * 2
    assert led["pass2"][1] == (3 * d * 2 + 4 * 4) * N * N / 128
    led64 = bench.ledger_terms(N, d, br=64, bc=64)
    assert led64["pass1"][1] == 2 * led["pass1"][1]
    assert led64["pass2"][1] == 2 * led["pass2"][1]
    two = bench.ledger_terms(N, d, BH=2)
    assert two["pass1"] == (2 * led["pass1"][0], 2 * led["pass1"][1])


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_trace_digest_selects_the_timed_launches(tmp_path, monkeypatch):
    """The trace digest takes each long_16k kernel's launches in launch order: the
    headline region is [W, W + K) and the roofline region [W + K, W + 2K) of pass 1,
    whatever else the run launched (other shapes, later regions)."""
    import csv
    import json

    W, K = 2, 3
    names = [bench.TRACE_KERNELS[n] for n in bench.KERNELS_PER_CALL["two_pass"]]
    rows, t = [], 1000
    for call in range(W + 3 * K):
        for i, n in enumerate(names):
            dur = 1000 * (i + 1) + (100 * call if "pass1_kernel" in n else 0)
            rows.append({"Kernel_Name": f"void fb::{n}(args)", "Start_Timestamp": t, "End_Timestamp": t + dur})
            t += dur + 10
        # an unrelated kernel of another shape in between
        rows.append({"Kernel_Name": "void fb::bob_pass1_kernel<fb::BF16, 64, true, 0>(args)",
                     "Start_Timestamp": t, "End_Timestamp": t + 5})
        t += 20
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "run_kernel_trace.csv", "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=list(rows[0]))
        wr.writeheader()
        wr.writerows(rows[::-1])  # any order: the digest sorts by start time
    log = tmp_path / "bench.out"
    line = {"warmup": W, "steps": K, "ms_per_step": 0.02, "roofline": {
        "algorithmic_flops_per_launch": 3.0e9, "peak": 2500.0, "avg_launch_ms": 0.0034, "frac": 0.35}}
    log.write_text("noise\n" + json.dumps(line) + "\n")
    out = tmp_path / "summary.md"
    monkeypatch.setattr(bench, "pass1_source_hash", lambda: "abc")
    bench.digest_trace(str(d), str(out), str(log))
    summary = json.loads((tmp_path / "summary.json").read_text())
    p1 = 3000 + 100 * (W + K + 1)  # mean of calls W+K .. W+2K-1
    assert summary["roofline_region"]["avg_us"] == p1 / 1000
    assert summary["headline_region"]["kernels"]["bob_pass1"]["avg_us"] == (3000 + 100 * (W + 1)) / 1000
    assert summary["headline_region"]["kernels"]["attn_fwd_stats"]["launches"] == K
    assert abs(summary["roofline_region"]["frac_of_peak"] - 3.0e9 / (p1 * 1e-9) / 1e12 / 2500.0) < 1e-4


def test_dispatch_model_of_causal_grids():
    """The dispatch model behind the shape-trace digest: causal query tiles stream
    (tile + 1) * 4 key steps, causal key tiles stream the queries from their own
    tile on, and 10 of the 16 wave-steps of a diagonal 128 x 128 block have work."""
    rows = bench._dispatch_steps("rows", 2, 512, True, 4, 1)
    assert len(rows) == 8
    assert sorted(j for j, _ in rows) == [4, 4, 8, 8, 12, 12, 16, 16]
    assert [j for j, _ in rows][:2] == [16, 16]  # heaviest tile first, over all heads
    cols = bench._dispatch_steps("cols", 2, 512, True, 4, 1)
    assert [j for j, _ in cols][:2] == [16, 16] and sorted(j for j, _ in cols) == [4, 4, 8, 8, 12, 12, 16, 16]
    for steps, frac in rows + cols:
        q = steps // 4 - 1  # tiles before the diagonal one
        assert abs(frac - (16 * q + 10) / (16 * q + 16)) < 1e-12
    full = bench._dispatch_steps("rows", 1, 512, False, 4, 2)
    assert [j for j, _ in full] == [8] * 8 and all(f == 1.0 for _, f in full)
    # greedy placement in order: the longest job bounds the makespan
    assert bench._makespan([32, 1, 1, 1], 2) == 32
    assert bench._makespan([3, 3, 2, 2, 2], 2) == 7  # in order: (3, 3) (5, 3) (5, 5) (7, 5)
    # the library's split rule: no split once the grid fills the target
    assert bench._auto_splits(96, 1024, 256, 8) == 1
    assert bench._auto_splits(1, 16384, 256, 128) == 2
    assert bench._auto_splits(1, 16384, 512, 128) == 4
