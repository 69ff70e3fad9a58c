"""Benchmark of exact backward-over-backward (BoB) attention on one MI355X.

One step = one whole BoB call (statistics kernel, pass 1, pass 2 and the split
reductions) over one batch of synthetic inputs already resident in HBM.
Default workload: one long head, B=1, H=1, N=16384, d=64, bf16, non-causal,
tau = 1/sqrt(d), all seven inputs i.i.d. N(0, 1) from seed 0.

FLOP model: one unit = one N x N x d contraction = 2 B H d n_pairs flops
(n_pairs = N^2, or N(N+1)/2 causal). The executed schedule is 21 units
(statistics 2 + pass 1 11 + pass 2 8); the materialised minimum is 12 units.
`value` is TFLOP/s on the executed 21 units; MFMA utilisation is that over the
bf16 dense peak (2.5 PFLOP/s).

Prints ONE JSON line (rank 0, one GPU). `--gpus` above 1 exits: this build
runs on one GPU.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "BoB ms/call + TFLOP/s (MFMA util) at N=16K,d=64 bf16; max N on 1 GPU"
PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3}
UNITS = {"stats": 2, "pass1": 11, "pass2": 8, "exec": 21, "two_pass": 19, "useful": 12, "four_pass_exec": 27}
PMC_SUMMARY = os.path.join(ROOT, "profiles", "bob_pass1_long16k_pmc.json")
TRACE_SUMMARY = os.path.join(ROOT, "profiles", "long16k_kernel_trace.md")
TRACE_JSON = os.path.join(ROOT, "profiles", "long16k_kernel_trace.json")
PASS1_SOURCES = ("bob_pass1_vgpr.hip", "pass1_kernel.hpp", "pass1_asm.hpp", "pass1_asm_loop.inc", "pass1_common.hpp",
                 "common.hpp", "kernels.hpp")
# library kernel names (fb_profile_start) of one call, in launch order
KERNELS_PER_CALL = {
    "two_pass": ("attn_fwd_stats", "attn_fwd_combine", "bob_pass1", "bob_pass1_combine", "bob_pass2",
                 "bob_pass2_reduce"),
    "four_pass": ("attn_fwd_stats", "attn_fwd_combine", "fourpass_alpha", "fourpass_energy", "fourpass_rows",
                  "bob_pass2", "bob_pass2_reduce"),
}
# the device kernel (rocprofv3 name prefix) behind each library name at long_16k (bf16, d = 64, non-causal)
TRACE_KERNELS = {
    "attn_fwd_stats": "attn_fwd_skew_kernel<fb::BF16, 64, false, true>",
    "attn_fwd_combine": "attn_fwd_combine_kernel<fb::BF16, 64, true>",
    "bob_pass1": "bob_pass1_kernel<fb::BF16, 64, false, 0, true, 1>",
    "bob_pass1_combine": "bob_pass1_combine_kernel<fb::BF16, 64>",
    "bob_pass2": "bob_pass2_kernel<fb::BF16, 64, false, false>",
    "bob_pass2_reduce": "bob_pass2_reduce_kernel<fb::BF16, 64>",
}


def flop_unit(w):
    pairs = w.N * (w.N + 1) // 2 if w.causal else w.N * w.N
    return 2.0 * w.B * w.H * w.d * pairs


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def pass1_source_hash():
    h = hashlib.sha256()
    for f in PASS1_SOURCES:
        with open(os.path.join(ROOT, "aware_flashbob_pass_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per pass-1 launch from the committed rocprofv3 counter summary,
    or None when the summary is missing or was taken from other kernel source."""
    try:
        with open(PMC_SUMMARY) as fh:
            s = json.load(fh)
    except (OSError, ValueError):
        return None
    if s.get("source_hash") != pass1_source_hash():
        return None
    return s.get("hbm_bytes_per_launch")


def trace_from_profile():
    """The committed trace digest of the default bench command, if it was taken
    from the current pass-1 sources: the dominant kernel's average duration over
    the launches of the roofline timed region."""
    try:
        with open(TRACE_JSON) as fh:
            s = json.load(fh)
    except (OSError, ValueError):
        return None
    if s.get("source_hash") != pass1_source_hash():
        return None
    return {"avg_ms": s["roofline_region"]["avg_us"] / 1e3}


def _csv_rows(directory, suffix):
    import csv
    import glob

    files = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    with open(files[0]) as fh:
        return list(csv.DictReader(fh))


def _per_kernel_mean(directory):
    agg = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        agg.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in agg.items()}


def digest_pmc(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, out):
    """HBM bytes per dispatch of each kernel: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) each scaled by the factor that makes the same counter read the true
    size of a plain 512 MiB device copy (bench.py --calibrate-copy 512)."""
    copy_bytes = 512 << 20
    f, w = _per_kernel_mean(fetch_dir), _per_kernel_mean(write_dir)
    cf, cw = _per_kernel_mean(copy_fetch_dir), _per_kernel_mean(copy_write_dir)
    copy_name = [k for k in cf if "copyBuffer" in k or "copy" in k.lower()][0]
    ff = copy_bytes / (cf[copy_name] * 1024)
    wf = copy_bytes / (cw[copy_name] * 1024)
    kernels = {}
    for k in f:
        short = k.replace("void fb::", "").split("(")[0]
        kernels[short] = {"fetch_kib": round(f[k], 1), "write_kib": round(w.get(k, 0.0), 1),
                          "hbm_bytes": int(f[k] * 1024 * ff + w.get(k, 0.0) * 1024 * wf)}
    p1 = [v for k, v in kernels.items() if k.startswith("bob_pass1_kernel<")]
    summary = {
        "workload": "long_16k: B=1,H=1,N=16384,d=64,bf16,non-causal",
        "source_hash": pass1_source_hash(),
        "copy_calibration": {"bytes": copy_bytes, "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
        "hbm_bytes_per_launch": p1[0]["hbm_bytes"] if p1 else None,
        "kernels": kernels,
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE -d <FETCH> -o run --output-format csv -- python3 bench.py --steps 5 --warmup 2 "
            "--no-cpu --no-endpoint --no-parity --settle-s 0",
            "rocprofv3 --pmc WRITE_SIZE -d <WRITE> -o run --output-format csv -- python3 bench.py --steps 5 --warmup 2 "
            "--no-cpu --no-endpoint --no-parity --settle-s 0",
            "rocprofv3 --pmc FETCH_SIZE -d <COPY_FETCH> -o run --output-format csv -- python3 bench.py --calibrate-copy 512",
            "rocprofv3 --pmc WRITE_SIZE -d <COPY_WRITE> -o run --output-format csv -- python3 bench.py --calibrate-copy 512",
            "python3 bench.py --digest-pmc <FETCH> <WRITE> <COPY_FETCH> <COPY_WRITE> " + os.path.relpath(out, ROOT),
        ],
    }
    with open(out, "w") as fh:
        json.dump(summary, fh, indent=1)
    print(json.dumps(summary, indent=1))


def _auto_splits(bh, n, target, tiles):
    """The library's default split count (api.cpp auto_splits), for the dispatch model."""
    blocks = tiles * bh
    if blocks >= target:
        return 1
    steps = (n + 31) // 32
    s = (target + blocks - 1) // blocks
    s = min(s, max(1, steps // 4))
    return max(1, min(s, 64))


def _dispatch_steps(kind, bh, n, causal, tiles, splits):
    """32-row steps of every workgroup of a launch, in dispatch order, with the
    fraction of its wave-steps whose wave is active (causal diagonal tiles idle
    some of the four waves). kind: 'rows' (statistics, pass 1: query tiles, keys
    streamed) or 'cols' (pass 2: key tiles, queries streamed)."""
    nst = (n + 31) // 32
    per_tile = 4 if tiles == (n + 127) // 128 else 2  # 32-row blocks per tile (128- or 64-row tiles)
    out = []
    for z in range(splits):
        for y in range(bh):
            for x in range(tiles):
                lin = x + tiles * y
                rank, head = lin // bh, lin % bh
                if causal:
                    tile = (tiles - 1 - rank) if kind == "rows" else rank
                else:
                    tile, head = x, y
                if kind == "rows":
                    span = min(nst, (tile + 1) * per_tile) if causal else nst
                    lo, hi = z * span // splits, (z + 1) * span // splits
                    first = 0
                else:
                    first = tile * per_tile if causal else 0
                    span = nst - first
                    lo, hi = first + z * span // splits, first + (z + 1) * span // splits
                steps = hi - lo
                if causal and steps > 0:
                    active = 0
                    for j in range(lo, hi):
                        if kind == "rows":
                            active += sum(1 for w in range(per_tile) if j <= tile * per_tile + w)
                        else:
                            active += sum(1 for w in range(per_tile) if j >= tile * per_tile + w)
                    frac = active / (steps * per_tile)
                else:
                    frac = 1.0
                out.append((steps, frac))
    return out


def _makespan(jobs, slots):
    import heapq

    h = [0.0] * slots
    for j in jobs:
        t = heapq.heappop(h)
        heapq.heappush(h, t + j)
    return max(h)


# kernel families of a BoB call (16-bit): name prefix, how its grid walks the sequence,
# and workgroups one compute unit holds (d = 64; d = 128 holds one of each)
SHAPE_KERNELS = (("statistics", "attn_fwd_skew_kernel<", "rows", 2),
                 ("statistics", "attn_fwd_kernel<", "rows", 2),
                 ("pass 1", "bob_pass1_kernel<", "rows", 1),
                 ("pass 1", "bob_pass1_q16_kernel<", "rows", 1),
                 ("pass 2", "bob_pass2_kernel<", "cols", 2))


def _shape_kernel_name(prefix, d, causal, names):
    c = "true" if causal else "false"
    for nm in names:
        if not nm.startswith(prefix):
            continue
        args = [a.strip() for a in nm[len(prefix):].rstrip(">").split(",")]
        if prefix.startswith("bob_pass1_q16"):
            if d == 128 and args[1] == c:
                return nm
        elif args[1] == str(d) and args[2] == c:
            return nm
    return None


def digest_shapes(trace_dir, bench_log, out):
    """Summarise the other shapes of a traced default bench run (its other_configs):
    per-kernel durations of each shape's timed calls (the last launches of kernels that
    only that shape uses), and for each kernel a dispatch model: the workgroups'
    32-row step counts in dispatch order, placed greedily on the compute units' slots,
    priced at the per-step time the same run measured on the 16,384-token head."""
    import statistics

    traced = None
    with open(bench_log) as fh:
        for line in fh:
            if line.startswith("{") and '"roofline"' in line:
                traced = json.loads(line)
    if traced is None or "other_configs" not in traced:
        raise SystemExit(f"no bench line with other_configs in {bench_log}")
    rows = _csv_rows(trace_dir, "kernel_trace.csv")
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    launches = {}
    for r in rows:
        n = r["Kernel_Name"].replace("void fb::", "").split("(")[0]
        launches.setdefault(n, []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    names = list(launches)
    W, K = traced["warmup"] + traced.get("settle_calls", 0), traced["steps"]

    # per-step time of each kernel family on the 16,384-token head (same run, headline calls)
    cfg = traced["config"]
    base = {}
    for fam, prefix, kind, per_cu in SHAPE_KERNELS:
        nm = _shape_kernel_name(prefix, cfg["d"], cfg["causal"], names)
        if nm is None or len(launches[nm]) < W + K:
            continue
        d_us = statistics.mean((e - s_) / 1e3 for s_, e in launches[nm][W:W + K])
        tiles = (cfg["N"] + 127) // 128
        target = {"statistics": 512, "pass 1": 256, "pass 2": 512}[fam]
        spl = _auto_splits(cfg["B"] * cfg["H"], cfg["N"], target, tiles)
        jobs = _dispatch_steps(kind, cfg["B"] * cfg["H"], cfg["N"], cfg["causal"], tiles, spl)
        base[fam] = d_us / _makespan([j for j, _ in jobs], 256 * per_cu)

    lines = ["# Kernel traces of the other shapes of the default bench run", "",
             "Commands (repository root, one MI355X): the default bench run under the kernel tracer (the same run as "
             "`profiles/long16k_kernel_trace.md`), then this digest.", "", "```",
             "rocprofv3 --kernel-trace --stats -d <TRACE> -o run --output-format csv -- python3 bench.py > <TRACED_STDOUT>",
             "python3 bench.py --digest-shapes <TRACE> <TRACED_STDOUT> " + os.path.relpath(out, ROOT), "```", "",
             "Each shape's timed calls are the last launches of the kernels that only that shape uses. The dispatch "
             "model lists every workgroup's 32-row steps in dispatch order (the kernels' own tile order: causal grids "
             "heaviest tile first), places them greedily on the compute units' workgroup slots, and prices a step at "
             "the per-step time of the same kernel on the 16,384-token head in the same run "
             f"(statistics {base.get('statistics', float('nan')):.3f} us, pass 1 {base.get('pass 1', float('nan')):.3f} us, "
             f"pass 2 {base.get('pass 2', float('nan')):.3f} us per step and slot). 'even' divides all steps evenly over "
             "the slots; 'greedy' is the model's makespan; 'active' is the share of wave-steps whose wave has work "
             "(causal diagonal tiles leave some of a workgroup's four waves waiting at its barriers).", ""]
    summary = {}
    for shape, oc in traced["other_configs"].items():
        B, H, N, d, causal, calls = oc["B"], oc["H"], oc["N"], oc["d"], oc["causal"], oc["calls"]
        bh = B * H
        lines += [f"## {shape}: B={B}, H={H}, N={N}, d={d}, bf16, {'causal' if causal else 'non-causal'}", "",
                  f"Bench line of the traced run: {oc['ms_per_call']} ms per call over {calls} calls.", "",
                  "| Kernel | Launches | Average (us) | Min (us) | Max (us) | workgroups | splits | even (us) | "
                  "greedy (us) | active | trace / greedy |", "|---|---|---|---|---|---|---|---|---|---|---|"]
        total, spans, rec = 0.0, [], {}
        first_last = []
        for fam, prefix, kind, per_cu in SHAPE_KERNELS:
            nm = _shape_kernel_name(prefix, d, causal, names)
            if nm is None:
                continue
            ls = launches[nm][-calls:]
            first_last.append(ls)
            du = [(e - s_) / 1e3 for s_, e in ls]
            avg = statistics.mean(du)
            total += avg
            q16 = "q16" in prefix
            tiles = (N + 63) // 64 if q16 else (N + 127) // 128
            slots = 256 * (1 if d == 128 else per_cu)
            target = {"statistics": 512, "pass 1": 256, "pass 2": 256 * (2 if d == 64 else 1)}[fam]
            spl = _auto_splits(bh, N, target, tiles)
            jobs = _dispatch_steps(kind, bh, N, causal, tiles, spl)
            steps = [j for j, _ in jobs]
            act = sum(j * f for j, f in jobs) / max(1, sum(steps))
            t_step = base.get(fam) if d == cfg["d"] and not q16 else None
            even = sum(steps) / slots * t_step if t_step else None
            greedy = _makespan(steps, slots) * t_step if t_step else None
            fmt = lambda v, p=1: "—" if v is None else f"{v:.{p}f}"  # noqa: E731
            lines.append(f"| `{nm}` | {len(du)} | {avg:.1f} | {min(du):.1f} | {max(du):.1f} | {len(jobs)} | {spl} | "
                         f"{fmt(even)} | {fmt(greedy)} | {act:.3f} | {fmt(avg / greedy if greedy else None, 2)} |")
            rec[fam] = {"kernel": nm, "launches": len(du), "avg_us": round(avg, 2), "workgroups": len(jobs),
                        "splits": spl, "even_us": None if even is None else round(even, 2),
                        "greedy_us": None if greedy is None else round(greedy, 2), "active_wave_steps": round(act, 4)}
        span = statistics.mean((max(ls[i][1] for ls in first_last) - min(ls[i][0] for ls in first_last)) / 1e3
                               for i in range(calls))
        lines += ["", f"Sum of the kernel averages: {total:.1f} us per call; first launch start to last launch end: "
                  f"{span:.1f} us per call (the difference is the gaps between launches).", ""]
        summary[shape] = {"kernels": rec, "sum_of_kernel_avg_us": round(total, 2), "first_to_last_us": round(span, 2),
                          "bench_ms_per_call": oc["ms_per_call"]}
    lines += ["```json", json.dumps({"per_step_us_long16k": {k: round(v, 4) for k, v in base.items()},
                                      "shapes": summary}, indent=1), "```", ""]
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print(f"wrote {out}")


def digest_trace(trace_dir, out, bench_log):
    """Summarise a rocprofv3 --kernel-trace run of the default `python3 bench.py`.

    The long_16k calls come first in the run: W warm-up calls, K headline calls (no
    library events), K calls with HIP events around pass 1 (the roofline region), then
    K calls per kernel of the breakdown. Launches of each long_16k kernel are taken in
    launch order, so the headline and roofline regions are launches [W, W + K) and
    [W + K, W + 2K) of that kernel; the bench line printed by the same traced run
    (bench_log) gives W, K and its own event timings for comparison."""
    import statistics

    traced = None
    with open(bench_log) as fh:
        for line in fh:
            if line.startswith("{") and '"roofline"' in line:
                traced = json.loads(line)
    if traced is None:
        raise SystemExit(f"no bench line in {bench_log}")
    W, K = traced["warmup"] + traced.get("settle_calls", 0), traced["steps"]
    rows = _csv_rows(trace_dir, "kernel_trace.csv")
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    launches = {}
    for r in rows:
        n = r["Kernel_Name"].replace("void fb::", "").split("(")[0]
        launches.setdefault(n, []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))

    def durations(name, lo, hi):
        return [(e - s_) / 1e3 for s_, e in launches.get(TRACE_KERNELS[name], [])[lo:hi]]

    def headline_span():
        first = launches[TRACE_KERNELS["attn_fwd_stats"]][W][0]
        last = launches[TRACE_KERNELS["bob_pass2_reduce"]][W + K - 1][1]
        return (last - first) / 1e3 / K

    table = []
    total = 0.0
    for name in KERNELS_PER_CALL["two_pass"]:
        d = durations(name, W, W + K)
        if not d:
            continue
        total += statistics.mean(d)
        table.append((name, TRACE_KERNELS[name], len(d), statistics.mean(d), min(d), max(d)))
    dom = durations("bob_pass1", W + K, W + 2 * K)
    dom_avg = statistics.mean(dom)
    flops = traced["roofline"]["algorithmic_flops_per_launch"]
    peak = traced["roofline"]["peak"]
    frac = flops / (dom_avg * 1e-6) / 1e12 / peak
    ev_us = traced["roofline"]["avg_launch_ms"] * 1e3
    span = headline_span()
    summary = {
        "workload": "long_16k: B=1,H=1,N=16384,d=64,bf16,non-causal",
        "source_hash": pass1_source_hash(),
        "warmup": W, "steps": K,
        "headline_region": {"kernels": {t[0]: {"launches": t[2], "avg_us": round(t[3], 2), "min_us": round(t[4], 2),
                                                "max_us": round(t[5], 2)} for t in table},
                            "sum_of_kernel_avg_us": round(total, 2), "first_to_last_us_per_call": round(span, 2),
                            "bench_ms_per_step": traced["ms_per_step"]},
        "roofline_region": {"kernel": "bob_pass1", "launches": len(dom), "avg_us": round(dom_avg, 2),
                            "min_us": round(min(dom), 2), "max_us": round(max(dom), 2),
                            "bench_event_avg_us": round(ev_us, 2), "flops_per_launch": flops,
                            "frac_of_peak": round(frac, 5), "peak_tflops": peak},
    }
    cmd = ("rocprofv3 --kernel-trace --stats -d <TRACE> -o run --output-format csv -- python3 bench.py "
           "> <TRACED_STDOUT>")
    lines = ["# Kernel trace: BoB call at long_16k (B=1, H=1, N=16384, d=64, bf16, non-causal)", "",
             "Commands (repository root, one MI355X): the default bench run under the kernel tracer, then this "
             "digest.", "", "```", cmd,
             "python3 bench.py --digest-trace <TRACE> " + os.path.relpath(out, ROOT) + " <TRACED_STDOUT>", "```", "",
             f"Pass-1 source hash ({' + '.join(PASS1_SOURCES)}): {pass1_source_hash()}", "",
             f"## Headline region (launches {W}..{W + K - 1} of each kernel: the {K} timed calls after "
             f"{traced['warmup']} warm-up and {traced.get('settle_calls', 0)} settle calls, no library events)",
             "", "| Library name | Kernel | Launches | Average (us) | Min (us) | Max (us) |", "|---|---|---|---|---|---|"]
    for name, kern, n, avg, mn, mx in table:
        lines.append(f"| {name} | `{kern}` | {n} | {avg:.1f} | {mn:.1f} | {mx:.1f} |")
    lines += ["", f"Sum of the kernel averages: {total:.1f} us per call; first statistics launch to last "
              f"reduction end: {span:.1f} us per call; the same traced run's bench line: "
              f"{traced['ms_per_step'] * 1e3:.1f} us per call (stream events around the {K} calls).", "",
              f"## Roofline region (launches {W + K}..{W + 2 * K - 1} of pass 1: HIP events around pass 1 only)", "",
              f"Trace average {dom_avg:.1f} us (min {min(dom):.1f}, max {max(dom):.1f}); the same launches timed by "
              f"the bench run's HIP events: {ev_us:.1f} us.",
              f"Pass 1 does 11 units = {flops:.4g} flop per launch, so the trace gives "
              f"{flops / (dom_avg * 1e-6) / 1e12:.1f} TFLOP/s = {frac:.3f} of the {peak:.0f} TFLOP/s bf16 dense peak "
              f"(the bench line of that run: {traced['roofline']['frac']:.3f}).", "",
              "Durations drift by several percent within one run and by up to ~10% between MI355X boxes "
              "of the pool (clock and power state), so an untraced run on another box reports its own figure; "
              "this file shows that the trace and the bench's events agree on the same launches.", "",
              "```json", json.dumps(summary, indent=1), "```"]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    with open(os.path.splitext(out)[0] + ".json", "w") as fh:
        json.dump(summary, fh, indent=1)
    print("\n".join(lines))


def ledger_terms(N, d, BH=1, br=128, bc=128, esz=2):
    """The pages' transfer ledger (review page, Strengths, Theorem 4.3; our reading of
    its garbled terms): Q = 12Nd + 4N + 4dN^2/B_r + (3d + 4)N^2/B_c elements per head,
    split here by pass and priced in bytes (16-bit tensors, float32 row vectors)."""
    p1_fixed = (4 * N * d + 2 * N * d) * esz + (2 * N + 2 * N) * 4   # Q, dO, UQ, O in; gQ, gdO out; L, D in; alpha, E out
    p1_stream = 4 * d * N * N / br * esz                               # K, V, UK, UV per query tile
    p2_fixed = (4 * N * d + 2 * N * d) * esz                           # K, V, UK, UV in; gK, gV out
    p2_stream = (3 * d * esz + 4 * 4) * N * N / bc                     # Q, dO, UQ and L, D, alpha, E per key tile
    return {"pass1": (BH * p1_fixed, BH * p1_stream), "pass2": (BH * p2_fixed, BH * p2_stream)}


def digest_ledger(out, copy_fetch, copy_write, *runs):
    """HBM bytes per dispatch (FETCH_SIZE x its copy factor + WRITE_SIZE x its copy
    factor) of each kernel of one BoB call, against the transfer ledger's terms.
    runs: WORKLOAD=FETCH_DIR,WRITE_DIR ..."""
    import workload as _wl

    copy_bytes = 512 << 20
    cf, cw = _per_kernel_mean(copy_fetch), _per_kernel_mean(copy_write)
    ck = [k for k in cf if "copy" in k.lower()][0]
    ff, wf = copy_bytes / (cf[ck] * 1024), copy_bytes / (cw[ck] * 1024)
    lines = ["# HBM bytes against the transfer ledger (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             "Commands (repository root, one MI355X; one counter per run; <W> is the workload):", "", "```",
             "rocprofv3 --pmc FETCH_SIZE -d <FETCH_W> -o run --output-format csv -- python3 bench.py --workload <W> "
             "--steps 1 --warmup 1 --no-cpu --no-endpoint --no-parity --no-breakdown --settle-s 0",
             "rocprofv3 --pmc WRITE_SIZE -d <WRITE_W> -o run --output-format csv -- python3 bench.py --workload <W> "
             "--steps 1 --warmup 1 --no-cpu --no-endpoint --no-parity --no-breakdown --settle-s 0",
             "rocprofv3 --pmc FETCH_SIZE -d <COPY_FETCH> -o run --output-format csv -- python3 bench.py --calibrate-copy 512",
             "rocprofv3 --pmc WRITE_SIZE -d <COPY_WRITE> -o run --output-format csv -- python3 bench.py --calibrate-copy 512",
             "python3 bench.py --digest-ledger " + os.path.relpath(out, ROOT) +
             " <COPY_FETCH> <COPY_WRITE> <W>=<FETCH_W>,<WRITE_W> ...", "```", "",
             f"Counter scale from a plain 512 MiB device copy: FETCH_SIZE x {ff:.3f}, WRITE_SIZE x {wf:.3f}.", "",
             "Ledger (per head, elements priced at 2 B for 16-bit tensors and 4 B for float32 row vectors, "
             "B_r = B_c = 128, the kernels' query and key tiles): pass 1 = 4Nd + 2N in, 2Nd + 2N out, "
             "4dN^2/B_r streamed; pass 2 = 4Nd in, 2Nd out, (3d + 4)N^2/B_c streamed. The statistics kernel "
             "and the split merges are outside the ledger. Measured bytes below the streamed term mean the "
             "re-streamed tiles were served by L2 / MALL, as the pages' own analysis expects of a real cache.", ""]
    for r in runs:
        name, dirs = r.split("=", 1)
        fdir, wdir = dirs.split(",")
        w = _wl.WORKLOADS[name]
        f, wr = _per_kernel_mean(fdir), _per_kernel_mean(wdir)
        led = ledger_terms(w.N, w.d, w.B * w.H)
        lines += [f"## {name}: B={w.B}, H={w.H}, N={w.N}, d={w.d}, {w.dtype}, "
                  f"{'causal' if w.causal else 'non-causal'}", "",
                  "| Kernel | read (MB) | written (MB) | HBM total (MB) | ledger fixed (MB) | ledger streamed (MB) | "
                  "HBM / (fixed + streamed) |", "|---|---|---|---|---|---|---|"]
        tot = 0.0
        for k in sorted(f):
            short = k.replace("void fb::", "").split("(")[0]
            rd, wb = f[k] * 1024 * ff, wr.get(k, 0.0) * 1024 * wf
            tot += rd + wb
            key = "pass1" if short.startswith("bob_pass1_kernel<") else "pass2" if short.startswith(
                "bob_pass2_kernel<") else None
            if key:
                fx, st = led[key]
                lines.append(f"| `{short}` | {rd / 1e6:.1f} | {wb / 1e6:.1f} | {(rd + wb) / 1e6:.1f} | {fx / 1e6:.1f} | "
                             f"{st / 1e6:.0f} | {(rd + wb) / (fx + st):.4f} |")
            else:
                lines.append(f"| `{short}` | {rd / 1e6:.1f} | {wb / 1e6:.1f} | {(rd + wb) / 1e6:.1f} | — | — | — |")
        fx = led["pass1"][0] + led["pass2"][0]
        st = led["pass1"][1] + led["pass2"][1]
        lines += ["", f"Per dispatch of every kernel of one call (averaged over the run's calls): {tot / 1e6:.1f} MB "
                  f"of HBM traffic; the ledger's fixed part 12Nd + 4N is {fx / 1e6:.1f} MB and its streamed part "
                  f"{st / 1e6:.0f} MB at B = 128.", ""]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def digest_reduction(out, copy_fetch, copy_write, *runs):
    """Pass 2's three split reductions at long_16k (bench.py --reduction 0/1/2):
    call time, per-kernel time and HBM bytes of the pass-2 kernels per mode.
    runs: MODE=FETCH_DIR,WRITE_DIR,BENCH_JSON ..."""
    copy_bytes = 512 << 20
    cf, cw = _per_kernel_mean(copy_fetch), _per_kernel_mean(copy_write)
    ck = [k for k in cf if "copy" in k.lower()][0]
    ff, wf = copy_bytes / (cf[ck] * 1024), copy_bytes / (cw[ck] * 1024)
    label = {"0": "split records + merge kernel (default)", "1": "float32 atomics + zero/convert kernels",
             "2": "split records, merged by the last workgroup of each key tile"}
    lines = ["# Pass 2's split reduction, measured: long_16k (B=1, H=1, N=16384, d=64, bf16, non-causal)", "",
             "Pass 2 runs 4 splits of the query range here (128 key tiles x 4 = 512 workgroups, two per CU). "
             "Commands (repository root, one MI355X; <M> = 0, 1, 2):", "", "```",
             "python3 bench.py --reduction <M> --no-cpu --no-endpoint --steps 40 > <BENCH_M>",
             "rocprofv3 --pmc FETCH_SIZE -d <FETCH_M> -o run --output-format csv -- python3 bench.py --reduction <M> "
             "--steps 5 --warmup 2 --no-cpu --no-endpoint --no-parity --no-breakdown --settle-s 0",
             "rocprofv3 --pmc WRITE_SIZE -d <WRITE_M> -o run --output-format csv -- python3 bench.py --reduction <M> "
             "--steps 5 --warmup 2 --no-cpu --no-endpoint --no-parity --no-breakdown --settle-s 0",
             "rocprofv3 --pmc FETCH_SIZE -d <COPY_FETCH> -o run --output-format csv -- python3 bench.py --calibrate-copy 512",
             "rocprofv3 --pmc WRITE_SIZE -d <COPY_WRITE> -o run --output-format csv -- python3 bench.py --calibrate-copy 512",
             "python3 bench.py --digest-reduction " + os.path.relpath(out, ROOT) +
             " <COPY_FETCH> <COPY_WRITE> <M>=<FETCH_M>,<WRITE_M>,<BENCH_M> ...", "```", "",
             f"Counter scale from a plain 512 MiB device copy: FETCH_SIZE x {ff:.3f}, WRITE_SIZE x {wf:.3f}.", "",
             "| Mode | call (ms) | ledger path (ms) | pass-2 kernels (us each, events around that kernel alone) | "
             "pass-2 HBM read (MB) | pass-2 HBM written (MB) |", "|---|---|---|---|---|---|"]
    for r in runs:
        mode, dirs = r.split("=", 1)
        fdir, wdir, bj = dirs.split(",")
        f, wr = _per_kernel_mean(fdir), _per_kernel_mean(wdir)
        with open(bj) as fh:
            b = json.loads([ln for ln in fh if ln.startswith("{")][-1])
        kern = {k: v["avg_ms"] * 1e3 for k, v in b["kernels"].items() if k.startswith("bob_pass2")}
        rd = sum(v for k, v in f.items() if "pass2" in k or "zero_f32" in k) * 1024 * ff
        wb = sum(v for k, v in wr.items() if "pass2" in k or "zero_f32" in k) * 1024 * wf
        ks = ", ".join(f"{k} {v:.1f}" for k, v in kern.items())
        lines.append(f"| {mode}: {label.get(mode, mode)} | {b['ms_per_step']:.4f} | {b['with_stats']['ms_per_call']:.4f} | "
                     f"{ks} | {rd / 1e6:.1f} | {wb / 1e6:.1f} |")
    lines += ["", "Mode 0 is kept. The atomic form adds about 8.4 million float32 atomic additions per call "
              "(64 per lane per split workgroup) at the L2; the last-workgroup form makes every split workgroup "
              "release its records at device scope (a write-back of its XCD's L2) and the last one acquire them "
              "(an invalidation), which costs more than the merge kernel it replaces. Modes 0 and 2 are "
              "deterministic and bitwise equal; mode 1 depends on the order of the atomic additions."]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


SQ_COMMAND = ("rocprofv3 --pmc {counters} -d <{tag}> -o run --output-format csv -- python3 bench.py --steps 5 "
              "--warmup 2 --no-cpu --no-endpoint --no-parity --settle-s 0")
KERNEL_UNITS = {"attn_fwd_kernel<": UNITS["stats"], "attn_fwd_skew_kernel<": UNITS["stats"],
                "bob_pass1_kernel<": UNITS["pass1"], "bob_pass2_kernel<": UNITS["pass2"]}


def digest_sq(out, trace_dir, *runs):
    """Matrix-core and issue counters per kernel (long_16k), from rocprofv3 --pmc
    runs given as DIR=COUNTER,COUNTER,...: per-dispatch means, the bf16 MFMA flops
    the hardware counted (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) against the FLOP
    model's units, and those flops over the kernel-trace average duration."""
    import math as _m

    w_unit = 2.0 * 64 * 16384 * 16384  # one unit at long_16k
    vals = {}
    cmds = []
    for r in runs:
        d, counters = r.split("=", 1)
        cmds.append(SQ_COMMAND.format(counters=counters.replace(",", " "), tag=os.path.basename(d.rstrip("/"))))
        for r2 in _csv_rows(d, "counter_collection.csv"):
            k = r2["Kernel_Name"].replace("void fb::", "").split("(")[0]
            vals.setdefault(k, {}).setdefault(r2["Counter_Name"], []).append(float(r2["Counter_Value"]))
    durs = {}
    for r in _csv_rows(trace_dir, "kernel_stats.csv"):
        durs[r["Name"].replace("void fb::", "").split("(")[0]] = float(r["AverageNs"]) * 1e-9
    names = sorted({c for v in vals.values() for c in v})
    lines = ["# Matrix-core and issue counters: BoB call at long_16k (B=1, H=1, N=16384, d=64, bf16, non-causal)", "",
             "Commands (repository root, one MI355X; one counter set per run):", "", "```"] + cmds + [
             "python3 bench.py --digest-sq " + os.path.relpath(out, ROOT) + " <TRACE> <DIR>=<COUNTERS> ...", "```", "",
             f"Pass-1 source hash ({' + '.join(PASS1_SOURCES)}): {pass1_source_hash()}", "",
             "Per-dispatch means over every launch of the run (warm-up, timed and ledger-path calls).", "",
             "| Kernel | " + " | ".join(names) + " |", "|---|" + "---|" * len(names)]
    for k in sorted(vals):
        lines.append(f"| `{k}` | " + " | ".join(f"{sum(vals[k].get(c, [_m.nan])) / max(1, len(vals[k].get(c, []))):.4g}"
                                                for c in names) + " |")
    lines += ["", "Derived. MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; model = the kernel's units x "
              f"{w_unit:.4g} flops; trace avg = the kernel-trace average of the same command. GRBM_GUI_ACTIVE "
              "sums the 8 XCDs, so the clock during the kernel is GRBM_GUI_ACTIVE / 8 / trace avg and the "
              "matrix cores' busy fraction is SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs). "
              "SQ_WAVE_CYCLES, SQ_ACTIVE_INST_VALU, SQ_WAIT_INST_LDS, SQ_WAIT_ANY (waiting at s_waitcnt) and "
              "SQ_WAIT_INST_ANY (waiting to issue) count in the same unit, so their ratios are fractions of the "
              "waves' resident time; SQ_LDS_BANK_CONFLICT over SQ_LDS_IDX_ACTIVE is the share of the LDS's busy "
              "cycles lost to bank conflicts.", "",
              "| Kernel | MFMA flops / dispatch | counted / model | trace avg (us) | counted TFLOP/s | clock (GHz) | "
              "MFMA busy | co-exec / MFMA busy | VALU active / wave | LDS wait / wave | waitcnt / wave | "
              "issue wait / wave | LDS bank conflict / LDS active |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]

    def mean(k, c):
        v = vals[k].get(c)
        return sum(v) / len(v) if v else _m.nan

    for k in sorted(vals):
        units = next((u for p, u in KERNEL_UNITS.items() if k.startswith(p)), None)
        if units is None or _m.isnan(mean(k, "SQ_INSTS_VALU_MFMA_MOPS_BF16")):
            continue
        fl = mean(k, "SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512
        t = durs.get(k, _m.nan)
        cyc = mean(k, "GRBM_GUI_ACTIVE") / 8
        lines.append(f"| `{k}` | {fl:.4g} | {fl / (units * w_unit):.3f} | {t * 1e6:.1f} | {fl / t / 1e12:.0f} | "
                     f"{cyc / t / 1e9:.2f} | {mean(k, 'SQ_VALU_MFMA_BUSY_CYCLES') / (cyc * 1024):.3f} | "
                     f"{mean(k, 'SQ_VALU_MFMA_COEXEC_CYCLES') / mean(k, 'SQ_VALU_MFMA_BUSY_CYCLES'):.3f} | "
                     f"{mean(k, 'SQ_ACTIVE_INST_VALU') / mean(k, 'SQ_WAVE_CYCLES'):.3f} | "
                     f"{mean(k, 'SQ_WAIT_INST_LDS') / mean(k, 'SQ_WAVE_CYCLES'):.3f} | "
                     f"{mean(k, 'SQ_WAIT_ANY') / mean(k, 'SQ_WAVE_CYCLES'):.3f} | "
                     f"{mean(k, 'SQ_WAIT_INST_ANY') / mean(k, 'SQ_WAVE_CYCLES'):.3f} | "
                     f"{mean(k, 'SQ_LDS_BANK_CONFLICT') / mean(k, 'SQ_LDS_IDX_ACTIVE'):.3f} |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_baseline(w, inputs, budget_s):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same
    workload: query rows [0, R) of head 0 against all N keys; extrapolate by N/R."""
    import numpy as np
    import threadpoolctl

    import oracle
    from workload import INPUT_NAMES, to_f64

    arrs = [to_f64(inputs[n][0, 0]) for n in INPUT_NAMES]
    threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
    rows = 256
    spent = 0.0
    t_per_row = None
    while True:
        t0 = time.perf_counter()
        oracle.bob_head(*arrs, w.scale, w.causal, row_block=256, row_range=(0, rows))
        dt = time.perf_counter() - t0
        spent += dt
        t_per_row = dt / rows
        if dt >= budget_s / 3 or rows >= w.N or spent >= budget_s:
            break
        rows = min(w.N, max(rows * 2, int(rows * (budget_s / 3) / max(dt, 1e-3))))
        rows = max(256, (rows // 256) * 256)
    full_s = t_per_row * w.N * w.B * w.H
    # causal rows do not get cheaper in the materialised oracle (it masks, it does not skip)
    tflops = UNITS["exec"] * flop_unit(w) / full_s / 1e12
    return {
        "value": tflops,
        "unit": "TFLOP/s",
        "ms_per_call": full_s * 1e3,
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"fp64 oracle on query rows 0..{rows - 1} of head 0 against all {w.N} keys "
                  f"({dt:.1f} s), time scaled by {w.N * w.B * w.H}/{rows} rows; same 21-unit FLOP model",
    }


def microbench(out_md):
    """Build and run the microbenchmarks and skeleton kernels of
    aware_flashbob_pass_amd/csrc/microbench/probes_gen.py (one HIP program, generated
    into a temporary directory) and print their figures as one JSON line; with a path,
    also write them as a summary."""
    import importlib.util
    import subprocess
    import tempfile

    here = os.path.dirname(os.path.abspath(__file__))
    gen = os.path.join(here, "aware_flashbob_pass_amd", "csrc", "microbench", "probes_gen.py")
    spec = importlib.util.spec_from_file_location("probes_gen", gen)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with tempfile.TemporaryDirectory() as tmp:
        src, exe = os.path.join(tmp, "microbench_probes.hip"), os.path.join(tmp, "microbench_probes")
        with open(src, "w") as fh:
            fh.write(mod.render())
        hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
        cmd = [hipcc, "-O3", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               src, "-o", exe]
        log("microbench: building")
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise SystemExit(f"microbench build failed:\n{res.stderr[-2000:]}")
        log("microbench: running")
        run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    figures = {}
    for line in run.stdout.splitlines():
        name, _, rest = line.partition(": ")
        parts = rest.split()
        if name != "status" and parts:
            figures[name] = {"value": float(parts[0]), "unit": " ".join(parts[1:])}
    status = next((l.split(": ", 1)[1] for l in run.stdout.splitlines() if l.startswith("status: ")), "missing")
    if run.returncode != 0 or status != "no error":
        raise SystemExit(f"microbench run failed (rc {run.returncode}, status {status}):\n{run.stdout}\n{run.stderr}")
    print(json.dumps({"microbench": figures}), flush=True)
    if out_md:
        rows = "\n".join(f"| `{k}` | {v['value']:g} | {v['unit']} |" for k, v in figures.items())
        text = (f"# Microbenchmarks and skeleton kernels (one MI355X)\n\n"
                f"Command (repository root): `python3 bench.py --microbench {out_md}`, which generates\n"
                f"`microbench_probes.hip` from `aware_flashbob_pass_amd/csrc/microbench/probes_gen.py` (its\n"
                f"docstring describes every probe), builds it with hipcc and runs it.\n\n"
                f"| Probe | Value | Unit |\n|---|---|---|\n{rows}\n")
        with open(out_md, "w") as fh:
            fh.write(text)


def alt_schedule_probe(args):
    """Decide the alternative schedule by measurement: forming gQ in pass 2 would remove
    pass 1's four gQ accumulating units (W_a UK, W_b K, W_a K, P K: 4 of its 11) and
    shrink its split merge, but pass 2 would have to add every (key tile, query tile)
    pair's 32 x d tile of gQ into float32 gQ with atomics. The probe kernel issues
    exactly those additions with pass 2's grid and split count and nothing else, so its
    time bounds the schedule's extra cost from below (the two extra accumulating units
    of pass 2 and its weight transposes are not counted); if the atomics hid entirely
    under pass 2's own work, pass 2 would still take at least the probe's time. The
    saving is bounded from above by 4/11 of pass 1 plus its whole merge kernel."""
    import torch

    import aware_flashbob_pass_amd as fb
    import workload

    w = workload.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    g = {k: v.to(dev) for k, v in workload.make_inputs(w, args.seed).items()}
    ws = torch.empty(max(1, fb.workspace_bytes(w.B, w.H, w.N, w.d, w.torch_dtype)), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(g["Q"]) for _ in range(4)]

    def step():
        fb.bob_attention(g["Q"], g["K"], g["V"], g["dO"], g["UQ"], g["UK"], g["UV"], tau=w.scale, causal=w.causal,
                         workspace=ws, out=outs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + args.settle_s
    while time.perf_counter() < t_end:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    kern = {}
    for name in ("bob_pass1", "bob_pass1_combine", "bob_pass2", "bob_pass2_reduce"):
        fb.profile_start(name)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        for k, (n, t) in fb.profile_stop().items():
            kern[k] = t / n
    bh = w.B * w.H
    tiles = (w.N + 127) // 128
    s2 = _auto_splits(bh, w.N, (2 if w.d == 64 else 1) * 256, tiles)  # pass 2's default split count
    gq = torch.zeros(bh * w.N * w.d, dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        fb.probe_gq_atomics(gq, w.B, w.H, w.N, w.d, s2)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        fb.probe_gq_atomics(gq, w.B, w.H, w.N, w.d, s2)
    stop.record()
    torch.cuda.synchronize()
    probe_ms = start.elapsed_time(stop) / args.steps
    counted = bool(torch.all(gq == float((args.warmup + args.steps) * tiles)).item())
    adds = bh * tiles * w.N * w.d
    saving = kern.get("bob_pass1", 0.0) * 4 / 11 + kern.get("bob_pass1_combine", 0.0)
    print(json.dumps({
        "metric": "alternative schedule (gQ in pass 2 with float32 atomics): atomics alone vs the most it saves",
        "workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal, "pass2_splits": s2,
        "atomic_adds_per_call": adds, "probe_gq_atomics_ms": round(probe_ms, 4),
        "atomic_adds_per_ns": round(adds / (probe_ms * 1e6), 2), "probe_counts_exact": counted,
        "kernels_ms": {k: round(v, 4) for k, v in kern.items()},
        "saving_upper_bound_ms": round(saving, 4),
        # atomics serialised after pass 2's work, and (second figure) hidden under it as
        # far as possible: pass 2 then takes at least the longer of the two
        "alternative_slower_by_at_least_ms": round(probe_ms - saving, 4),
        "alternative_slower_by_at_least_ms_if_overlapped": round(
            max(0.0, probe_ms - kern.get("bob_pass2", 0.0)) - saving, 4),
    }), flush=True)


def hutchinson_bench(args, name):
    """One Hutchinson sample of the attention Hessian diagonal, diag(H) ~ u * (H u)
    with Rademacher u, where H is the Hessian of <dO, O(Q, K, V)> in (Q, K, V):
    H u is BoB with U = u. Timed through the C ABI directly and through the
    autograd integration (forward, create_graph backward, Hessian-vector
    product), the way a Sophia-style optimizer samples it."""
    import torch

    import aware_flashbob_pass_amd as fb
    import workload

    w = workload.WORKLOADS[name]
    dev = torch.device("cuda:0")
    inp = {k: v.to(dev) for k, v in workload.make_inputs(w, args.seed).items()}
    shape = (w.B, w.H, w.N, w.d)
    u = [workload.rademacher(shape, args.seed + 100 + i, w.torch_dtype).to(dev) for i in range(3)]
    ws = torch.empty(max(1, fb.workspace_bytes(w.B, w.H, w.N, w.d, w.torch_dtype)), dtype=torch.uint8, device=dev)

    def direct():
        hu = fb.bob_attention(inp["Q"], inp["K"], inp["V"], inp["dO"], u[0], u[1], u[2], tau=w.scale,
                              causal=w.causal, workspace=ws)
        return [a * b for a, b in zip(u, hu[:3])]

    q, k, v = (inp[n].clone().requires_grad_(True) for n in ("Q", "K", "V"))

    def through_autograd():
        o = fb.attention(q, k, v, tau=w.scale, causal=w.causal)
        grads = torch.autograd.grad(o, (q, k, v), grad_outputs=inp["dO"], create_graph=True)
        hu = torch.autograd.grad(grads, (q, k, v), grad_outputs=tuple(u))
        return [a * b for a, b in zip(u, hu)]

    res = {}
    for label, fn in (("direct", direct), ("autograd", through_autograd)):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(args.steps):
            fn()
        stop.record()
        torch.cuda.synchronize()
        res[label] = start.elapsed_time(stop) / args.steps
    print(json.dumps({
        "metric": "Hutchinson Hessian-diagonal sample time, attention block", "value": round(res["autograd"], 5),
        "unit": "ms", "higher_is_better": False, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_direct_c_abi": round(res["direct"], 5), "ms_through_autograd": round(res["autograd"], 5),
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "probe": "rademacher"}}), flush=True)


def max_n_probe(fb, workload, dev, seed, per_call_s, total_s=None):
    """Largest N (a power of two from 262144 up; B = H = 1, d = 64, bf16, non-causal)
    whose call runs within the budget.

    Each size runs once (the library is warmed by a small call first). The next
    size is tried only if four times this call's time (the N^2 work) fits the
    per-call budget and, with `total_s`, what is left of the total budget, and if
    its buffers fit the free device memory. Each size is checked on two query rows
    against the oracle (gQ, gdO) and on the key / value shift invariants: sum_j gK_j
    = 0 and sum_j gV_j = 0 up to rounding, here at most 1e-3 of sum_j |gK_j| (|gV_j|)
    per head dimension. Memory per size: torch's peak allocation (inputs, outputs and
    the library workspace all come from torch) and the drop in the device's free
    memory (hipMemGetInfo) from before the inputs are allocated to after the call."""
    import numpy as np
    import torch

    import oracle

    wu = workload.custom(1, 1, 4096, 64, "bf16", False)
    gu = {k: v.to(dev) for k, v in workload.make_inputs(wu, seed).items()}
    fb.bob_attention(*[gu[k] for k in workload.INPUT_NAMES], tau=wu.scale, causal=False)
    torch.cuda.synchronize()
    del gu
    torch.cuda.empty_cache()
    records = []
    best = None
    spent = 0.0
    n = 262144
    while True:
        w = workload.custom(1, 1, n, 64, "bf16", False, name=f"probe_{n}")
        need = (fb.workspace_bytes(1, 1, n, 64, w.torch_dtype) + 11 * n * 64 * 2) * 1.1
        free0, _ = torch.cuda.mem_get_info(dev)
        if need > free0:
            log(f"max-n probe: N={n} needs {need / 2**30:.1f} GiB, {free0 / 2**30:.1f} GiB free; stop")
            break
        log(f"max-n probe: N={n}: generating inputs")
        cpu_in = workload.make_inputs(w, seed)
        torch.cuda.reset_peak_memory_stats(dev)
        base_alloc = torch.cuda.memory_allocated(dev)
        g = {k: v.to(dev) for k, v in cpu_in.items()}
        log(f"max-n probe: N={n}: call")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        out = fb.bob_attention(*[g[k] for k in workload.INPUT_NAMES], tau=w.scale, causal=False)
        torch.cuda.synchronize()
        t = time.perf_counter() - t0
        spent += t
        free1, _ = torch.cuda.mem_get_info(dev)
        finite = all(bool(torch.isfinite(o).all()) for o in out)
        shift = {}
        for name, o in (("gK", out[1]), ("gV", out[2])):
            x = o[0, 0].double()
            shift[name] = float((x.sum(0).abs() / x.abs().sum(0).clamp_min(1e-300)).max())
        rows = np.array([0, n - 1])
        arrs = [workload.to_f64(cpu_in[k][0, 0]) for k in workload.INPUT_NAMES]
        r = oracle.bob_rows_head(*arrs, w.scale, False, rows)
        errs = {}
        for name, o in (("gQ", out[0]), ("gdO", out[3])):
            got = o[0, 0, torch.as_tensor(rows, device=dev)].double().cpu().numpy()
            errs[name] = float(np.linalg.norm(got - r[name]) / np.linalg.norm(r[name]))
        ok = finite and max(errs.values()) <= 2e-2 and max(shift.values()) <= 1e-3 and t <= per_call_s
        rec = {"N": n, "s": round(t, 4), "tflops_21_units": round(UNITS["exec"] * 2.0 * 64 * n * n / t / 1e12, 1),
               "finite": finite, "row_rel_err": {k: round(v, 6) for k, v in errs.items()},
               "shift_sum_rel": {k: float(f"{v:.3g}") for k, v in shift.items()},
               "peak_alloc_bytes": int(torch.cuda.max_memory_allocated(dev) - base_alloc),
               "hbm_free_drop_bytes": int(free0 - free1), "ok": ok}
        log(f"max-n probe: {rec}")
        records.append(rec)
        del g, out, cpu_in, arrs
        torch.cuda.empty_cache()
        if not ok:
            break
        best = n
        if 4 * t > per_call_s or (total_s is not None and 4 * t > total_s - spent):
            break
        n *= 2
    return {"max_n_run": best, "per_call_budget_s": per_call_s, "total_budget_s": total_s, "d": 64,
            "dtype": "bf16", "probe": records}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_16k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--settle-s", type=float, default=0.25,
                    help="after the warm-up calls, untimed calls for this long (clock settle)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-endpoint", action="store_true",
                    help="skip the N=262144 feasibility call and the timings of the other multi-head shapes")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true",
                    help="skip the untimed pass with HIP events around every kernel (the kernels field is then empty)")
    ap.add_argument("--hutchinson", action="store_true",
                    help="time one Hutchinson Hessian-diagonal sample u * (H u) instead (default shape: gpt2_hessian)")
    ap.add_argument("--microbench", nargs="?", const="", default=None, metavar="OUT_MD",
                    help="build and run the microbenchmarks and skeleton kernels (optionally write a summary)")
    ap.add_argument("--alt-schedule-probe", action="store_true",
                    help="time the float32 atomics a gQ-in-pass-2 schedule needs against the pass-1 work it saves")
    ap.add_argument("--reduction", type=int, choices=(0, 1, 2), default=0,
                    help="pass 2's split reduction: 0 records + merge kernel, 1 float32 atomics, "
                         "2 last-workgroup merge (fb_set_reduction)")
    ap.add_argument("--schedule", choices=("two_pass", "four_pass"), default="two_pass",
                    help="four_pass times the ablation schedule (separate alpha, E and row-output sweeps)")
    ap.add_argument("--max-n-probe", action="store_true",
                    help="only find the largest N = 2^k >= 262144 (B = H = 1, d = 64, bf16) whose call finishes "
                         "within --max-n-budget seconds and passes sampled oracle rows and the key/value shift "
                         "invariants")
    ap.add_argument("--max-n-budget", type=float, default=60.0, help="seconds per call for the max-N probe")
    ap.add_argument("--max-n-total", type=float, default=20.0,
                    help="seconds of probe calls in the default run (the opt-in --max-n-probe has no total cap)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 times), to scale HBM counters")
    ap.add_argument("--digest-pmc", nargs=5, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE", "OUT"),
                    help="summarise rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs (csv dirs) into OUT (json)")
    ap.add_argument("--digest-ledger", nargs="+", metavar="OUT COPY_FETCH COPY_WRITE WORKLOAD=FETCH,WRITE",
                    help="summarise FETCH_SIZE / WRITE_SIZE runs per workload against the transfer ledger (markdown)")
    ap.add_argument("--digest-reduction", nargs="+", metavar="OUT COPY_FETCH COPY_WRITE MODE=FETCH,WRITE,BENCH",
                    help="summarise pass 2's three split reductions (timing json + FETCH/WRITE runs per mode)")
    ap.add_argument("--digest-sq", nargs="+", metavar="OUT TRACE_DIR DIR=COUNTERS",
                    help="summarise rocprofv3 --pmc runs of matrix-core / issue counters into OUT (markdown)")
    ap.add_argument("--digest-shapes", nargs=3, metavar=("TRACE_DIR", "BENCH_LOG", "OUT"),
                    help="summarise the other shapes (other_configs) of a traced default run into OUT (markdown)")
    ap.add_argument("--digest-trace", nargs=3, metavar=("TRACE_DIR", "OUT", "BENCH_LOG"),
                    help="summarise a rocprofv3 --kernel-trace --stats run (csv dir) into OUT (markdown)")
    args = ap.parse_args()
    if args.digest_pmc:
        digest_pmc(*args.digest_pmc)
        return
    if args.digest_trace:
        digest_trace(*args.digest_trace)
        return
    if args.digest_shapes:
        digest_shapes(*args.digest_shapes)
        return
    if args.digest_sq:
        digest_sq(*args.digest_sq)
        return
    if args.digest_ledger:
        digest_ledger(*args.digest_ledger)
        return
    if args.digest_reduction:
        digest_reduction(*args.digest_reduction)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the BoB path here is single-GPU; sharding is described, not built.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import aware_flashbob_pass_amd as fb
    import workload

    fb.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.max_n_probe:
        print(json.dumps(max_n_probe(fb, workload, dev, args.seed, args.max_n_budget)), flush=True)
        return
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4, "launches": 5}))
        return
    if args.hutchinson:
        hutchinson_bench(args, "gpt2_hessian" if args.workload == "long_16k" else args.workload)
        return
    if args.alt_schedule_probe:
        alt_schedule_probe(args)
        return
    if args.microbench is not None:
        microbench(args.microbench)
        return
    w = workload.WORKLOADS[args.workload]
    fb.set_reduction(args.reduction)
    log(f"bench: {w.describe()} steps={args.steps} warmup={args.warmup}")
    cpu_in = workload.make_inputs(w, args.seed)
    g = {k: v.to(dev) for k, v in cpu_in.items()}
    ws = torch.empty(max(1, fb.workspace_bytes(w.B, w.H, w.N, w.d, w.torch_dtype)), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(g["Q"]) for _ in range(4)]

    call = fb.bob_attention if args.schedule == "two_pass" else fb.bob_attention_fourpass

    def step():
        call(g["Q"], g["K"], g["V"], g["dO"], g["UQ"], g["UK"], g["UV"], tau=w.scale, causal=w.causal,
             workspace=ws, out=outs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The MI355X takes tens of milliseconds of sustained load to reach a steady clock
    # (pass 1 measured ~400 -> 460 -> 348 us over its first ~45 calls), so the warm-up
    # calls are followed by untimed calls until --settle-s seconds have passed.
    settle_calls = 0
    t_settle = time.perf_counter() + args.settle_s
    while time.perf_counter() < t_settle:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        settle_calls += 10
    log(f"bench: warmup done (+{settle_calls} settle calls)")

    # dominant kernel: pass 1 (11 units); for the four-pass ablation, its row-output sweep (9 units)
    dom, dom_units = ("bob_pass1", UNITS["pass1"]) if args.schedule == "two_pass" else ("fourpass_rows", 9)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed_calls(only=None):
        """K calls between two stream events; with `only`, the library also records HIP
        events around every launch of that kernel (on its launch stream)."""
        torch.cuda.synchronize()
        if only:
            fb.profile_start(only)
        start.record()
        for _ in range(args.steps):
            step()
        stop.record()
        torch.cuda.synchronize()
        rec = fb.profile_stop() if only else {}
        return start.elapsed_time(stop) / args.steps, rec

    # 1. the timed region of the headline: K whole calls, no library events
    ms, _ = timed_calls()
    log(f"bench: {ms:.4f} ms/call")
    # 2. the dominant kernel's launch duration for the roofline: K more calls with HIP
    #    events around that kernel only (the launch-ordered position of these launches is
    #    what the rocprofv3 trace digest selects)
    ms_dom_region, dom_timed = timed_calls(dom)
    # 3. per-kernel breakdown: K calls per kernel, each with events around that kernel alone
    #    (the kernel names of one call come from one call with events around every kernel)
    kernels = {}
    if not args.no_breakdown:
        fb.profile_start()
        step()
        torch.cuda.synchronize()
        names = list(fb.profile_stop())
        for name in names:
            _, rec = timed_calls(name)
            kernels.update(rec)
    # 4. per-call median and minimum: stream events around each call
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    per_call = sorted(e0.elapsed_time(e1) for e0, e1 in evs)

    # the ledger path: pass 1 + pass 2 from saved statistics (19 units), same inputs
    with_stats = None
    if args.schedule == "two_pass":
        o_s, l_s, d_s = fb.attn_fwd(g["Q"], g["K"], g["V"], tau=w.scale, causal=w.causal, do=g["dO"])

        def step_ws():
            fb.bob_attention_with_stats(g["Q"], g["K"], g["V"], g["dO"], g["UQ"], g["UK"], g["UV"], o_s, l_s, d_s,
                                        tau=w.scale, causal=w.causal, workspace=ws)

        for _ in range(2):
            step_ws()
        start.record()
        for _ in range(args.steps):
            step_ws()
        stop.record()
        torch.cuda.synchronize()
        ms_ws = start.elapsed_time(stop) / args.steps
        with_stats = {"ms_per_call": round(ms_ws, 5), "units": UNITS["two_pass"],
                      "tflops": round(UNITS["two_pass"] * flop_unit(w) / (ms_ws * 1e-3) / 1e12, 3)}
        del o_s, l_s, d_s

    unit = flop_unit(w)
    tflops = UNITS["exec"] * unit / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    kern = {k: {"launches": n, "avg_ms": t / max(n, 1)} for k, (n, t) in kernels.items()}
    n_dom, t_dom = dom_timed.get(dom, (0, float("nan")))
    p1 = {"avg_ms": t_dom / max(n_dom, 1)}
    p1_flops = dom_units * unit
    p1_tflops = p1_flops / (p1["avg_ms"] * 1e-3) / 1e12
    traffic = traffic_from_profile()
    if args.schedule != "two_pass" or w.name != "long_16k":
        traffic = None
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(p1_tflops, 3), "peak": peak,
                "unit": "TFLOP/s", "frac": round(p1_tflops / peak, 5), "traffic": traffic,
                "algorithmic_flops_per_launch": p1_flops, "avg_launch_ms": p1["avg_ms"],
                "launches_timed": n_dom}
    prof = trace_from_profile() if (args.schedule == "two_pass" and w.name == "long_16k") else None
    if prof:
        # the committed rocprofv3 trace of this same command (same pass-1 sources):
        # its average duration of the same launches, and the fraction it gives
        roofline["profile_avg_launch_ms"] = prof["avg_ms"]
        roofline["profile_frac"] = round(p1_flops / (prof["avg_ms"] * 1e-3) / 1e12 / peak, 5)
        roofline["profile"] = os.path.relpath(TRACE_SUMMARY, ROOT)

    result = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "tau": w.scale, "seed": args.seed, "schedule": args.schedule, "reduction": args.reduction},
        "roofline": roofline,
        "mfma_util": round(tflops / peak, 5),
        "settle_calls": settle_calls,
        "executed_units": UNITS["exec"] if args.schedule == "two_pass" else UNITS["four_pass_exec"],
        "ms_per_call_with_pass1_events": round(ms_dom_region, 5),
        "ms_per_call_median": round(per_call[len(per_call) // 2], 5),
        "ms_per_call_min": round(per_call[0], 5),
        "sum_of_kernel_ms_per_call": round(sum(v["avg_ms"] * v["launches"] for v in kern.values()) / args.steps, 5),
        "tflops_useful_12_units": round(UNITS["useful"] * unit / (ms * 1e-3) / 1e12, 3),
        "with_stats": with_stats,
        "kernels": kern,
        "peak_mem_bytes": int(torch.cuda.max_memory_allocated(dev)),
    }

    if not args.no_parity:
        import oracle

        rng = np.random.default_rng(123)
        rows = np.unique(np.concatenate([rng.choice(w.N, 32, replace=False), [0, w.N - 1]]))
        arrs = [workload.to_f64(cpu_in[n][0, 0]) for n in workload.INPUT_NAMES]
        r = oracle.bob_rows_head(*arrs, w.scale, w.causal, rows)
        errs = {}
        for name, o in (("gQ", outs[0]), ("gdO", outs[3])):
            got = o[0, 0, torch.as_tensor(rows, device=dev)].double().cpu().numpy()
            errs[name] = float(np.linalg.norm(got - r[name]) / np.linalg.norm(r[name]))
        result["parity_sampled_rows"] = {k: round(v, 6) for k, v in errs.items()}

    if not args.no_endpoint and args.schedule == "two_pass":
        # the other multi-head shapes, timed the same way (whole calls, inputs resident)
        others = {}
        for name, reps in (("gpt2_hessian", 20), ("wide_64k", 3)):
            wo = workload.WORKLOADS[name]
            log(f"bench: {wo.describe()}")
            go = {k: v.to(dev) for k, v in workload.make_inputs(wo, args.seed).items()}
            wso = torch.empty(max(1, fb.workspace_bytes(wo.B, wo.H, wo.N, wo.d, wo.torch_dtype)), dtype=torch.uint8,
                              device=dev)
            oo = [torch.empty_like(go["Q"]) for _ in range(4)]

            def step_o():
                fb.bob_attention(*[go[n] for n in workload.INPUT_NAMES], tau=wo.scale, causal=wo.causal,
                                 workspace=wso, out=oo)

            # the headline's protocol: warm-up calls, then untimed calls until the clock settles
            # (at least two calls of the 65,536-token shape)
            for _ in range(args.warmup):
                step_o()
            torch.cuda.synchronize()
            t_settle, n_settle = time.perf_counter() + args.settle_s, 0
            while time.perf_counter() < t_settle or n_settle < 2:
                step_o()
                torch.cuda.synchronize()
                n_settle += 1
            start.record()
            for _ in range(reps):
                step_o()
            stop.record()
            torch.cuda.synchronize()
            mo = start.elapsed_time(stop) / reps
            others[name] = {"ms_per_call": round(mo, 4), "calls": reps, "settle_calls": n_settle,
                            "tflops_21_units": round(UNITS["exec"] * flop_unit(wo) / (mo * 1e-3) / 1e12, 2),
                            "B": wo.B, "H": wo.H, "N": wo.N, "d": wo.d, "causal": wo.causal}
            del go, wso, oo
        result["other_configs"] = others

    if not args.no_endpoint:
        # the 262,144-token feasibility endpoint and, within a bounded total budget,
        # the doubling probe above it (the longest N whose call runs here)
        log("bench: feasibility endpoint and bounded max-N probe")
        del g, ws, outs
        torch.cuda.empty_cache()
        probe = max_n_probe(fb, workload, dev, args.seed, args.max_n_budget, args.max_n_total)
        we = workload.WORKLOADS["endpoint_256k"]
        _, total = torch.cuda.mem_get_info(dev)
        per_row = (fb.workspace_bytes(1, 1, we.N, we.d, we.torch_dtype) + 11 * we.N * we.d * 2) / we.N
        end = probe["probe"][0] if probe["probe"] else {}
        result["max_n"] = {
            "max_n_run": probe["max_n_run"], "total_budget_s": args.max_n_total,
            "per_call_budget_s": args.max_n_budget,
            "endpoint_256k": end,
            "probe": probe["probe"][1:],
            "mem_bound_n_estimate": int(total / per_row),
        }

    if not args.no_cpu:
        log("bench: cpu baseline (fp64 oracle sample)")
        result["cpu_baseline"] = cpu_baseline(w, cpu_in, args.cpu_budget)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
