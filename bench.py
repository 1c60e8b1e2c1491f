"""Benchmark: DiT denoiser block forwards per second at 4096 image + 34 text rows.

One step is one ``moss_block_forward`` (every step of the block: row join,
adaLN GEMV, two modulated RMSNorms, QKV projection, q/k norm + rotary pack,
attention, out projection with the first gated residual add in its epilogue,
up projection with the SiLU gate in its epilogue, down projection with the
second gated residual add in its epilogue) on one batch of seeded synthetic
inputs already resident in HBM: D = 3072, 24 heads x 128, MLP 12288, a 64x64
image grid plus 34 text rows (the 1024x1024 picture's shape on the
MOSS-Image transformer page, "Measured"), weights N(0, 0.02).
``--workload p1280|p1408|p1536`` times the larger pictures instead (5120,
5632 and 6144 image rows).

Each timed step has its own pair of HIP events on the launch stream;
``ms_per_step`` is the median over the steps (the pages report the median of
100 forwards), with p10 / p90 beside it, and ``value`` = 1000 / median.
Every timed step's output is compared on the GPU with the first one's (outside
the event pairs), and the line says whether all were byte-identical.

Prints one JSON line.  ``roofline`` is for the up projection (the largest
kernel, 43% of the block's flops), timed live with HIP events recorded by the
library around each of its launches inside the timed region.  Its ``traffic``
(HBM bytes per launch) comes from the committed FETCH_SIZE / WRITE_SIZE
counter summary under ``profiles/`` when that summary was taken on the GEMM
source as it is now, else it is null.  ``cpu_baseline`` times the float64
oracle on block forwards of the same workload.

After the main timing (unless ``--no-extras``) the line also carries: each
step's launch time inside block forwards (the library's probe) with its
fraction of the MFMA or HBM peak, warm and with the 256 MB Infinity Cache
flushed before every forward (``step_times_cold_cache``: a 512 MB fill, which
also leaves dirty lines for the forward's reads to evict;
``step_times_cold_read``: a 512 MB read, which does not); the modulation GEMV
and the norm each alone beside a torch kernel moving the same bytes
(``hbm_reference``); the up projection's product through this library and
through torch's linear, i.e. hipBLASLt (``gemm_reference``; alone with
``--gemm-reference``, for counter runs over both); the 24-block guidance-pair stack (two items of
4096 image + 34 text rows) in ms per call; the larger pictures (block and
attention time against the square of the row count); and the block replayed
from a captured HIP graph.

Counter runs: ``--copy-calibration`` adds one plain 256 MiB device copy before
the warm-up, so that each ``rocprofv3 --pmc`` run also records what the
counter reads for a known byte count.  ``--traffic-summary FETCH_DIR
WRITE_DIR`` (no GPU) turns the two runs' counter CSVs into the summary file.
``--counter-summary DIR...`` (no GPU) writes the MFMA / LDS / wait counter
summary from ``rocprofv3 --pmc`` CSV runs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
CALIB_BYTES = 256 << 20  # the plain device copy the counters are scaled by
PROBE_EVERY = 5  # the timed steps whose up projection the probe brackets: 0, 5, 10, ...
# the up projection with the SiLU gate epilogue: whole 256-row tiles (two LDS stages), then the 34 leftover rows
# as 64 x 64 tiles (four stages)
UP_KERNELS = ("gemm_nt_kernel<256, 256, 2, 4, 1, 2, 6, 3>", "gemm_nt_kernel<64, 64, 2, 1, 1, 4, 6, 4>")
GEMM_SOURCES = ("diffusion_transformer_denoiser_amd/csrc/gemm.hip", "diffusion_transformer_denoiser_amd/csrc/common.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_up_c2_traffic.md")
METRIC = "denoiser block-forwards/s and TFLOP/s at 4096+34 tokens; MFMA % of peak"


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="c2", choices=("c2", "p1280", "p1408", "p1536"),
                   help="the timed block: 4096 image rows (default) or a larger picture")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-extras", action="store_true",
                   help="skip the per-step, repeat-hash and 24-block stack measurements after the main timing")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run one plain 256 MiB device copy before the warm-up (for counter runs)")
    p.add_argument("--oracle-sweep", action="store_true",
                   help="time the float64 oracle on the c0-c3 blocks and two c4 blocks (CPU only), then exit")
    p.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="write the HBM traffic summary from two rocprofv3 --pmc CSV runs, then exit")
    p.add_argument("--trace-summary", metavar="DB",
                   help="print the per-kernel table of a rocprofv3 --kernel-trace database (results.db), then exit")
    p.add_argument("--gemm-reference", action="store_true",
                   help="time the up projection's product through this library and through torch's linear "
                        "(hipBLASLt) only, print one JSON line, then exit (for counter runs over both)")
    p.add_argument("--counter-summary", nargs="+", metavar="DIR",
                   help="write the MFMA / LDS / wait counter summary from rocprofv3 --pmc CSV runs, then exit")
    return p.parse_args()


def gemm_source_digest():
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per up-projection launch from the committed counter summary,
    or None when the GEMM source differs from the one the counters were taken on."""
    import re
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("gemm_source_sha256") != gemm_source_digest():
        return None
    return rec


def read_counter_csv(folder, counter):
    """(kernel name, grid size, value) per dispatch of one counter from a rocprofv3 CSV run."""
    import csv
    import glob
    paths = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if len(paths) != 1:
        raise SystemExit(f"{folder}: expected one counter_collection.csv, found {len(paths)}")
    rows = []
    with open(paths[0]) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                rows.append((r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])))
    return rows


def traffic_summary(fetch_dir, write_dir, geom):
    """Scale FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the up projection by
    what each counter reads for the plain 256 MiB copy, and write the summary."""
    per = {}
    for counter, folder in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = read_counter_csv(folder, counter)
        # the up projection's dispatches (its two kernels run nowhere else in a block forward): the
        # whole 256-row tiles, one workgroup per CU, then the 384 tail tiles of 64 x 64
        parts = [[v for name, grid, v in rows if kname in name] for kname in UP_KERNELS]
        copies = [v for name, _, v in rows if "copyBuffer" in name]
        if not parts[0] or not copies:
            raise SystemExit(f"{counter}: no up-projection dispatch or no copy dispatch in {folder}")
        calib_kib = max(copies)  # the 256 MiB copy moves far more than any upload chunk
        factor = CALIB_BYTES / (calib_kib * 1024.0)
        # one up projection = one dispatch of each of its kernels
        per_call = [sum(x) for x in zip(*[p for p in parts if p])]
        per[counter] = dict(dispatches=len(per_call), avg_kib=float(np.mean(per_call)), min_kib=min(per_call),
                            max_kib=max(per_call), calib_kib=calib_kib, factor=factor,
                            bytes=float(np.mean(per_call)) * 1024.0 * factor)
    m = geom.batch * geom.rows
    alg = 2 * (m * geom.d_model + 2 * geom.mlp_inner * geom.d_model + m * geom.mlp_inner)
    total = per["FETCH_SIZE"]["bytes"] + per["WRITE_SIZE"]["bytes"]
    rec = {"gemm_source_sha256": gemm_source_digest(), "kernels": list(UP_KERNELS),
           "fetch_bytes": round(per["FETCH_SIZE"]["bytes"]), "write_bytes": round(per["WRITE_SIZE"]["bytes"]),
           "traffic_bytes": round(total), "algorithmic_bytes": alg}
    lines = [
        "# Up projection (4130 x 24576 x 3072, SiLU gate epilogue) at 4096 image + 34 text rows: HBM traffic",
        "",
        "Commands (on one MI355X, from the repository root; one counter per run):",
        "",
        "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o run -- "
        "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-extras --copy-calibration",
        "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o run -- "
        "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-extras --copy-calibration",
        "    python3 bench.py --traffic-summary gpurun_out/pmc_fetch gpurun_out/pmc_write",
        "",
        "One up projection is one dispatch of each of " + " and ".join(f"`{k}`" for k in UP_KERNELS) + " "
        "(whole 256-row tiles, then the leftover rows); their counts are summed per projection.  "
        "Each counter is scaled by what it reads for one plain 256 MiB device copy "
        "(`__amd_rocclr_copyBuffer`) in the same run: factor = 268435456 B / (counter KiB x 1024).",
        "",
        "| counter | up projections | avg KiB | min KiB | max KiB | copy KiB | factor | bytes per projection |",
        "|---|---|---|---|---|---|---|---|",
    ]
    for c, d in per.items():
        lines.append(f"| {c} | {d['dispatches']} | {d['avg_kib']:.1f} | {d['min_kib']:.1f} | {d['max_kib']:.1f} | "
                     f"{d['calib_kib']:.1f} | {d['factor']:.3f} | {d['bytes'] / 1e6:.1f} MB |")
    # every kernel of the run, scaled the same way (context for the block's other steps)
    kinds = {}
    for counter, folder in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        for name, grid, v in read_counter_csv(folder, counter):
            short = name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
            if short.startswith("__amd") or short.startswith("at::"):
                continue
            kinds.setdefault((short, grid), {}).setdefault(counter, []).append(v * 1024.0 * per[counter]["factor"])
    lines += ["", "All of the library's kernels in the same runs (MB per dispatch, scaled):", "",
              "| kernel | grid (threads) | dispatches | fetch MB | write MB |", "|---|---|---|---|---|"]
    for (short, grid), d in kinds.items():
        f = d.get("FETCH_SIZE", [float("nan")])
        w = d.get("WRITE_SIZE", [float("nan")])
        lines.append(f"| {short} | {grid} | {len(f)} | {np.mean(f) / 1e6:.1f} | {np.mean(w) / 1e6:.1f} |")
    lines += [
        "",
        "FETCH_SIZE counts what the L2 caches fetch from beyond themselves; part of it is served by the "
        "256 MB Infinity Cache rather than HBM, so it is an upper bound on HBM reads.  The GEMM's excess "
        "over its algorithmic bytes is operand panels re-fetched by successive groups of concurrently "
        "running tiles on each XCD (a 4 MB L2 holds a k-slab of each panel, not whole panels).",
    ]
    lines += [
        "",
        f"HBM traffic per launch: {total / 1e6:.1f} MB against {alg / 1e6:.1f} MB algorithmic "
        f"(A {2 * m * geom.d_model / 1e6:.1f} MB + W {4 * geom.mlp_inner * geom.d_model / 1e6:.1f} MB read, "
        f"z {2 * m * geom.mlp_inner / 1e6:.1f} MB written): {total / alg:.2f}x.",
        "",
        "The record bench.py reads (null traffic once the GEMM source hash differs):",
        "",
        "```json",
        json.dumps(rec),
        "```",
        "",
    ]
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def trace_summary(db):
    """Per kernel of a rocprofv3 --kernel-trace database: shape, registers, LDS, dispatches and
    durations (the registers and LDS as the code object records them)."""
    import sqlite3
    c = sqlite3.connect(db)
    rows = c.execute(
        "select s.display_name, d.grid_size_x, d.grid_size_y, d.workgroup_size_x, s.arch_vgpr_count, "
        "s.accum_vgpr_count, s.group_segment_size, count(*), avg(d.end - d.start), min(d.end - d.start), "
        "max(d.end - d.start), sum(d.end - d.start) from rocpd_kernel_dispatch d join rocpd_info_kernel_symbol s "
        "on d.kernel_id = s.id group by s.display_name, d.grid_size_x, d.grid_size_y order by sum(d.end - d.start) desc"
    ).fetchall()
    total = sum(r[11] for r in rows)
    print("| kernel | grid (threads) | block | VGPR | AGPR | LDS B | calls | avg us | min us | max us | share |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for name, gx, gy, bx, vg, ag, lds, n, avg, mn, mx, tot in rows:
        short = name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        print(f"| {short} | {gx}x{gy} | {bx} | {vg} | {ag} | {lds} | {n} | {avg / 1e3:.1f} | {mn / 1e3:.1f} | "
              f"{mx / 1e3:.1f} | {100 * tot / total:.1f}% |")


COUNTER_FILE = os.path.join(ROOT, "profiles", "mfma_util_c2.md")
COUNTER_PASSES = (
    "GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY "
    "SQ_ACTIVE_INST_ANY SQ_INSTS_MFMA",
    "GRBM_GUI_ACTIVE SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS "
    "SQ_LDS_DATA_FIFO_FULL SQ_INSTS_VALU_MFMA_MOPS_BF16",
)


def counter_summary(dirs):
    """Per kernel of a block forward: the MFMA, wait and LDS counters of rocprofv3 --pmc runs (each
    with --kernel-trace, so every dispatch has its duration), averaged over the dispatches."""
    import csv
    import glob
    per = {}   # (kernel, grid) -> counter -> [values]
    dur = {}   # (kernel, grid) -> [ns]
    n_xcc, n_simd = 8, 1024
    for folder in dirs:
        cc = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
        kt = glob.glob(os.path.join(folder, "**", "*kernel_trace.csv"), recursive=True)
        ag = glob.glob(os.path.join(folder, "**", "*agent_info.csv"), recursive=True)
        if len(cc) != 1 or len(kt) != 1:
            raise SystemExit(f"{folder}: expected one counter_collection.csv and one kernel_trace.csv")
        for r in (csv.DictReader(open(ag[0])) if ag else []):
            if r.get("Agent_Type", r.get("Type", "")).upper().endswith("GPU"):
                n_xcc = int(r.get("Num_Xcc", n_xcc) or n_xcc)
                n_simd = int(r.get("Simd_Count", 0) or 0) or n_simd
        times = {r["Dispatch_Id"]: int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in csv.DictReader(open(kt[0]))}
        for r in csv.DictReader(open(cc[0])):
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
            if name.startswith("__amd") or name.startswith("at::"):
                continue
            key = (name, int(r["Grid_Size"]))
            per.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE" and r["Dispatch_Id"] in times:
                dur.setdefault(key, []).append(times[r["Dispatch_Id"]])
    lines = [
        "# MFMA, wait and LDS counters per kernel of a block forward at 4096 image + 34 text rows",
        "",
        "Commands (on one MI355X, from the repository root; one counter pass per run, each with the kernel",
        "trace so that every dispatch has its duration):",
        "",
    ]
    for i, ctrs in enumerate(COUNTER_PASSES):
        lines.append(f"    rocprofv3 --pmc {ctrs} --kernel-trace --output-format csv -d gpurun_out/pmc_sq{i} -o run "
                     "-- python3 bench.py --steps 10 --warmup 2 --no-cpu-baseline --no-extras")
    lines += ["    python3 bench.py --counter-summary " + " ".join(f"gpurun_out/pmc_sq{i}" for i in range(len(COUNTER_PASSES))),
              "",
              f"Values are per dispatch, averaged over the dispatches of each kernel ({n_xcc} XCDs, {n_simd} SIMDs).  "
              "`GRBM_GUI_ACTIVE` sums the XCDs' busy cycles, so the clock is GRBM_GUI_ACTIVE / XCDs / duration.  "
              "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs x SIMDs) (rocprofv3's MfmaUtil).  "
              "Wait = SQ_WAIT_ANY / SQ_WAVE_CYCLES (wave cycles at a wait count or barrier); issue-blocked = "
              "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES.  LDS busy = SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE / XCDs x CUs) "
              "(rocprofv3's LdsUtil); bank conflicts are cycles per LDS-active cycle.  MFMA TFLOP/s = "
              "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / duration.  The counters cover the collection window around a "
              "dispatch, a few microseconds longer than the kernel: for kernels of tens of microseconds the clock "
              "reads high (above the 2.4 GHz maximum) and the busy fractions are diluted by the same factor.",
              "",
              "| kernel | grid | dispatches | avg us | clock GHz | MFMA busy | wait | issue-blocked | LDS busy | "
              "bank conflict | MFMA TFLOP/s |",
              "|---|---|---|---|---|---|---|---|---|---|---|"]
    n_cu = n_simd // 4

    def avg(d, c):
        v = d.get(c)
        return float(np.mean(v)) if v else float("nan")

    order = sorted(per, key=lambda k: -float(np.mean(dur.get(k, [0]))))
    for key in order:
        d = per[key]
        us = float(np.mean(dur[key])) / 1e3 if key in dur else float("nan")
        gui = avg(d, "GRBM_GUI_ACTIVE") / n_xcc
        clock = gui / (us * 1e3) if us == us else float("nan")
        mfma = avg(d, "SQ_VALU_MFMA_BUSY_CYCLES") / (gui * n_simd)
        wait = avg(d, "SQ_WAIT_ANY") / avg(d, "SQ_WAVE_CYCLES")
        blocked = avg(d, "SQ_WAIT_INST_ANY") / avg(d, "SQ_WAVE_CYCLES")
        lds = avg(d, "SQ_LDS_IDX_ACTIVE") / (gui * n_cu)
        conf = avg(d, "SQ_LDS_BANK_CONFLICT") / max(avg(d, "SQ_LDS_IDX_ACTIVE"), 1.0)
        tf = avg(d, "SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512 / (us * 1e-6) / 1e12 if us == us else float("nan")
        lines.append(f"| {key[0]} | {key[1]} | {len(dur.get(key, []))} | {us:.1f} | {clock:.2f} | {100 * mfma:.1f}% | "
                     f"{100 * wait:.1f}% | {100 * blocked:.1f}% | {100 * lds:.1f}% | {conf:.3f} | {tf:.0f} |")
    lines.append("")
    with open(COUNTER_FILE, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def cpu_baseline(geom, acts, wbits, min_seconds=10.0, max_forwards=8):
    """Time the float64 oracle on whole block forwards of the same workload: repeated until about
    min_seconds of CPU work (at most max_forwards), so the sample is bounded but not one noisy call."""
    from oracle import dit_block as ob
    threads = len(os.sched_getaffinity(0))
    cos, sin = ob.rope_tables(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, geom.head_dim)
    x, txt, cond = ob.widen_bf16(acts["x"]), ob.widen_bf16(acts["txt"]), ob.widen_bf16(acts["cond"])
    w = ob.weights_f64(wbits)
    n = 0
    t0 = time.perf_counter()
    while n < max_forwards and (n == 0 or time.perf_counter() - t0 < min_seconds):
        ob.block_forward(x, txt, acts["txt_len"], cond, w, cos, sin, geom.eps)
        n += 1
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "block-forwards/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} full block forwards of this workload in float64 NumPy ({dt:.1f} s; BLAS threads = "
                      f"{threads} host cores)"}


# the steps that launch kernels of their own (the q/k norm and packing, the gated adds and the SiLU
# product run in GEMM epilogues)
PROBED = ("JOIN", "ADALN", "NORM1", "QKV", "ATTN", "OUT", "NORM2", "UP", "DOWN")
MFMA_STEPS = ("QKV", "ATTN", "OUT", "UP", "DOWN")
# algorithmic work per step at one block forward of this workload: (GFLOP, MB)
def step_work(geom):
    m, d, f = geom.batch * geom.rows, geom.d_model, geom.mlp_inner
    t = geom.rows
    return {
        # the row join runs in one pass with the first block's first norm: x/txt in, h (fp32) and a (bf16) out
        "JOIN": (0.0, (2 * m * d + 4 * m * d + 2 * m * d) / 1e6),
        "ADALN": (2 * geom.batch * 6 * d * d / 1e9, 2 * 6 * d * d / 1e6),
        "NORM1": (0.0, (4 * m * d + 2 * m * d) / 1e6),
        "QKV": (2 * m * 3 * d * d / 1e9, None),
        "ATTN": (4 * geom.batch * geom.n_heads * t * t * 128 / 1e9, None),
        "OUT": (2 * m * d * d / 1e9, None),
        "NORM2": (0.0, (4 * m * d + 2 * m * d) / 1e6),
        "UP": (2 * m * 2 * f * d / 1e9, None),
        "DOWN": (2 * m * d * f / 1e9, None),
    }


def read_flush(torch):
    """A 512 MB buffer whose sum, taken before a forward, leaves the 256 MB Infinity Cache holding
    clean lines of that buffer: the forward's weights then come from HBM, and it does not also pay
    for writing back a flush's dirty lines (a 512 MB fill does that)."""
    buf = torch.ones(128 << 20, dtype=torch.int32, device="cuda")
    return lambda: buf.sum()


def write_flush(torch):
    """A 512 MB fill before a forward (the cold-cache protocol as specified): it evicts the 256 MB
    Infinity Cache, and leaves it full of dirty lines that the next kernels' reads evict."""
    buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    return lambda: buf.fill_(1)


def per_step(torch, moss, step, geom, reps=5, cold=None):
    """Average launch time of each step inside block forwards (the library's probe); cold is None
    (warm), "write" (a 512 MB fill before each forward) or "read" (a 512 MB read before each)."""
    flush = {None: lambda t: None, "write": write_flush, "read": read_flush}[cold](torch)
    work = step_work(geom)
    res = {}
    for name in PROBED:
        moss.moss_probe_arm(name, reps)
        for _ in range(reps):
            if flush is not None:
                flush()
            step()
        torch.cuda.synchronize()
        ms = moss.moss_probe_collect(reps)
        if not ms:  # a step with no launch of its own in a single block (the first norm runs with the join)
            res[name.lower()] = None
            continue
        us = 1000.0 * float(np.mean(ms))
        gflop, mb = work[name]
        entry = {"us": round(us, 2)}
        if gflop:
            entry["tflops"] = round(gflop / us * 1e3, 1)
        if mb:
            entry["gb_s"] = round(mb / us * 1e3, 1)
        # the fraction of the peak that bounds the step: MFMA for the contractions, HBM for the rest
        if name in MFMA_STEPS:
            entry["mfma_frac"] = round(gflop / us * 1e3 / PEAK_BF16_TFLOPS, 4)
        elif mb:
            entry["hbm_frac"] = round(mb / us * 1e3 / PEAK_HBM_GBS, 4)
        res[name.lower()] = entry
    return res


def hbm_reference(torch, moss, geom, reps=15):
    """The block's modulation GEMV and modulated RMSNorm, each alone (through its single-step entry
    point), beside a torch kernel that moves the same bytes: a read-only sum of W_mod, a fp32 ->
    bf16 conversion copy of h.  Each is timed between events on the stream right after a 512 MB
    read flush (so the operands come from HBM), median of `reps`; the GEMV's entry point also runs
    SiLU(cond) first, so its own time comes from the library's probe around the GEMV launch."""
    d, m = geom.d_model, geom.batch * geom.rows
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    cond = torch.randn(geom.batch, d, generator=g, device="cuda").to(torch.bfloat16)
    w_mod = (torch.randn(6 * d, d, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    mod = torch.empty(geom.batch, 6 * d, dtype=torch.float32, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    h = torch.randn(m, d, generator=g, device="cuda")
    shift, scale = mod[:, :d], mod[:, d:2 * d]
    out16 = torch.empty(m, d, dtype=torch.bfloat16, device="cuda")
    red = torch.empty((), dtype=torch.float32, device="cuda")
    flush = read_flush(torch)

    def timed(fn):
        ts = []
        for _ in range(reps):
            flush()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(1000.0 * a.elapsed_time(b))
        return float(np.median(ts))

    def gemv_alone():
        # moss_k_adaln_gemv runs SiLU(cond) and then the GEMV: the library's probe brackets the GEMV
        ts = []
        for _ in range(reps):
            flush()
            moss.moss_probe_arm("ADALN", 1)
            moss.moss_k_adaln_gemv(geom.batch, d, cond, w_mod, mod, ws)
            torch.cuda.synchronize()
            ts.extend(moss.moss_probe_collect(1))
        return 1000.0 * float(np.median(ts))

    res = {}
    gemv_mb, norm_mb = 2 * 6 * d * d / 1e6, 6 * m * d / 1e6
    for name, ours, ref, mb, what in (
            ("adaln_gemv", lambda: moss.moss_k_adaln_gemv(geom.batch, d, cond, w_mod, mod, ws),
             lambda: torch.sum(w_mod, dim=(0, 1), dtype=torch.float32, out=red), gemv_mb,
             "torch sum of W_mod (reads the same bytes)"),
            ("mod_rmsnorm", lambda: moss.moss_k_mod_rmsnorm(geom.batch, geom.rows, d, geom.eps, h, shift, scale,
                                                            6 * d, out16),
             lambda: out16.copy_(h), norm_mb, "torch fp32 -> bf16 copy of h (reads and writes the same bytes)")):
        for _ in range(3):
            ours()
            ref()
        t_ours, t_ref = timed(ours), timed(ref)
        entry = {}
        if name == "adaln_gemv":
            entry["entry_point_us"] = round(t_ours, 2)  # both launches and the gap between them
            t_ours = gemv_alone()
        entry.update({"us": round(t_ours, 2), "hbm_frac": round(mb / t_ours * 1e3 / PEAK_HBM_GBS, 4),
                      "same_bytes_us": round(t_ref, 2), "same_bytes_hbm_frac": round(mb / t_ref * 1e3 / PEAK_HBM_GBS, 4),
                      "same_bytes_kernel": what})
        res[name] = entry
    del w_mod, h, out16
    torch.cuda.empty_cache()
    return res


def gemm_reference(torch, moss, geom, reps=20):
    """The up projection's product (rows x 2F x D) through this library's SiLU-gated GEMM and through
    torch.nn.functional.linear (hipBLASLt on ROCm) on the same bf16 operands, each timed between events
    on the stream, median of `reps` (the library's kernel also applies the SiLU gate and stores the
    half-width z; torch's linear stores all 2F columns of the plain product)."""
    d, f, m = geom.d_model, geom.mlp_inner, geom.batch * geom.rows
    g = torch.Generator(device="cuda")
    g.manual_seed(2)
    a = torch.randn(m, d, generator=g, device="cuda").to(torch.bfloat16)
    w = (torch.randn(2 * f, d, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    z = torch.empty(m, f, dtype=torch.bfloat16, device="cuda")

    def timed(fn):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(1000.0 * e0.elapsed_time(e1))
        return float(np.median(ts))

    t_ours = timed(lambda: moss.moss_k_gemm_silu(m, f, d, a, d, w, d, z, f))
    t_ref = timed(lambda: torch.nn.functional.linear(a, w))
    gflop = 2.0 * m * 2 * f * d / 1e9
    del a, w, z
    torch.cuda.empty_cache()
    return {"shape": [m, 2 * f, d], "us": round(t_ours, 1), "tflops": round(gflop / t_ours * 1e3, 1),
            "torch_linear_us": round(t_ref, 1), "torch_linear_tflops": round(gflop / t_ref * 1e3, 1),
            "torch_linear_kernel": "torch.nn.functional.linear (hipBLASLt), plain product, no epilogue"}


def timed_steps(torch, step, out, stream, steps):
    """Run `steps` steps, each between its own pair of events on the launch stream.  After each
    step (outside its events) its output is copied into a device ring; after the loop every copy
    is compared with the first.  Returns (per-step ms, ms per step over the whole loop, wall
    seconds, all outputs identical, sha256 of the first output)."""
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    loop0, loop1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ring = torch.empty((steps, *out.shape), dtype=out.dtype, device=out.device)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    loop0.record(stream)
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
        ring[i].copy_(out)
    loop1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    identical = all(torch.equal(ring[i], ring[0]) for i in range(1, steps))
    digest = hashlib.sha256(ring[0].cpu().numpy().tobytes()).hexdigest()[:16]
    del ring
    return ms, loop0.elapsed_time(loop1) / steps, wall, identical, digest


def larger_pictures(torch, moss, w, seed, reps=20, warm=20, settle=40):
    """Block and attention time at 4096 image rows and at the larger pictures of the CUDA port
    page's served-picture table (1280x1024, 1408x1024, 1536x1024: 5120, 5632 and 6144 image
    rows), with the attention time per square row relative to the 4096-row block."""
    from diffusion_transformer_denoiser_amd import synth

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()

    res = {}
    base = None
    for name in ("c2", "p1280", "p1408", "p1536"):
        geom = synth.CONFIGS[name]
        acts = synth.make_activations(geom, seed)
        dims = moss.make_dims(geom.batch, geom.n_img, geom.n_txt, geom.d_model, geom.mlp_inner, geom.eps)
        x, txt, cond = dev(acts["x"]), dev(acts["txt"]), dev(acts["cond"])
        rope = torch.empty(2, geom.rows, 64, dtype=torch.float32, device="cuda")
        moss.moss_rope_build(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, rope)
        ws = torch.empty(moss.moss_workspace_bytes(dims, 1), dtype=torch.uint8, device="cuda")
        out = torch.empty(geom.batch, geom.rows, geom.d_model, dtype=torch.int16, device="cuda")

        def step():
            moss.moss_block_forward(dims, x, txt, acts["txt_len"], cond, w, rope, out, ws)

        for _ in range(warm):
            step()
        ms, _, _, same, _ = timed_steps(torch, step, out, torch.cuda.current_stream(), reps)
        # the timed loop's copies into its output ring leave the caches full of dirty lines, and the
        # forwards after it pay to write them back (the 4096-row attention probe read 277 us on the
        # first, 233-238 after 10 plain forwards, 226-227 after 40, as the per-step probe does)
        for _ in range(settle):
            step()
        moss.moss_probe_arm("ATTN", 5)
        for _ in range(5):
            step()
        torch.cuda.synchronize()
        attn_us = 1000.0 * float(np.mean(moss.moss_probe_collect(5)))
        t = geom.rows
        attn_gflop = 4.0 * geom.batch * geom.n_heads * t * t * 128 / 1e9
        med = float(np.median(ms))
        per_t2 = attn_us / (t * t)
        if base is None:
            base = per_t2
        res[name] = {"image_rows": geom.n_img, "rows": t, "block_ms": round(med, 4),
                     "block_forwards_s": round(1000.0 / med, 2),
                     "block_tflops": round(geom.block_flops() / med / 1e9, 1),
                     "attention_us": round(attn_us, 2), "attention_tflops": round(attn_gflop / attn_us * 1e3, 1),
                     "attention_mfma_frac": round(attn_gflop / attn_us * 1e3 / PEAK_BF16_TFLOPS, 4),
                     "attention_us_per_t2_vs_4096_rows": round(per_t2 / base, 4),
                     "outputs_identical": same}
        del ws, out, x, txt, cond, rope
    torch.cuda.empty_cache()
    return res


def stack_timing(torch, moss, geom, seed, reps=3):
    """The 24-block guidance-pair stack (two items, 34 and 10 valid text rows): ms per call.
    Weights are drawn on the GPU with torch's seeded generator (same distributions as the
    host generator: N(0, 0.02) weights, 1 + N(0, 0.02) gains, bf16), to keep the bench short."""
    from diffusion_transformer_denoiser_amd import synth
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    d, f = geom.d_model, geom.mlp_inner

    def w(*shape, mean=0.0):
        return (torch.randn(*shape, generator=g, device="cuda") * 0.02 + mean).to(torch.bfloat16)

    blocks = [{"w_mod": w(6 * d, d), "w_qkv": w(3 * d, d), "q_gain": w(128, mean=1.0), "k_gain": w(128, mean=1.0),
               "w_out": w(d, d), "w_up": w(2 * f, d), "w_down": w(d, f)} for _ in range(geom.n_blocks)]
    acts = synth.make_activations(geom, seed)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()

    dims = moss.make_dims(geom.batch, geom.n_img, geom.n_txt, d, f, geom.eps)
    x, txt, cond = dev(acts["x"]), dev(acts["txt"]), dev(acts["cond"])
    rope = torch.empty(2, geom.rows, 64, dtype=torch.float32, device="cuda")
    moss.moss_rope_build(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, rope)
    ws = torch.empty(moss.moss_workspace_bytes(dims, geom.n_blocks), dtype=torch.uint8, device="cuda")
    out = torch.empty(geom.batch, geom.rows, d, dtype=torch.int16, device="cuda")

    def call():
        moss.moss_stack_forward(dims, blocks, x, txt, acts["txt_len"], cond, rope, out, ws)

    call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tflop = geom.n_blocks * geom.block_flops() / 1e12

    # the guidance pass with block 22 skipped on one branch (the CUDA port page, "What this changes"):
    # the block runs on item 0's rows alone
    skip = [[False, i == 22] for i in range(geom.n_blocks)]

    def call_skip():
        moss.moss_stack_forward_skip(dims, blocks, skip, x, txt, acts["txt_len"], cond, rope, out, ws)

    call_skip()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        call_skip()
    e1.record()
    torch.cuda.synchronize()
    skip_ms = e0.elapsed_time(e1) / reps

    # the whole denoiser forward around the same stack: timestep MLP, prompt and latent projections,
    # the 24 blocks, final norm and velocity projection
    enc_dim = synth.ENC_DIM
    ends = {"w_t1": w(d, 256), "w_t2": w(d, d), "w_txt": w(d, enc_dim), "w_in": w(d, 128), "w_fmod": w(2 * d, d),
            "w_final": w(128, d)}
    inp = synth.make_denoiser_inputs(geom, seed, enc_dim)
    lat, enc = dev(inp["latent"]), dev(inp["enc"])
    vel = torch.empty(geom.batch, geom.n_img, 128, dtype=torch.int16, device="cuda")
    del ws
    ws = torch.empty(moss.moss_denoiser_workspace_bytes(dims, geom.n_blocks), dtype=torch.uint8, device="cuda")

    def den():
        moss.moss_denoiser_forward(dims, blocks, lat, enc, inp["txt_len"], inp["t"], ends, enc_dim, rope, vel, ws)

    den()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        den()
    e1.record()
    torch.cuda.synchronize()
    den_ms = e0.elapsed_time(e1) / reps
    del blocks, ws, ends
    torch.cuda.empty_cache()
    return {"workload": "24-block stack, guidance pair: 2 items x (4096 image + 34 text rows; 34 and 10 valid)",
            "ms_per_call": round(ms, 3), "tflops": round(tflop / ms * 1e3, 1), "tflop_per_call": round(tflop, 2),
            "ms_per_call_block22_skipped_by_item1": round(skip_ms, 3),
            "calls_timed": reps, "denoiser_forward_ms": round(den_ms, 3),
            "denoiser_forward_note": "the same stack with the ends: timestep MLP, prompt (4096-wide) and latent "
                                     "(128-wide) projections, final norm and velocity projection"}


def oracle_sweep():
    """Time the float64 oracle on one block at each workload (c0-c3) and on two blocks of the
    24-block guidance pair (c4; the 24-block time is 12x that), on this host's cores."""
    import platform
    from diffusion_transformer_denoiser_amd import synth
    from oracle import dit_block as ob
    threads = len(os.sched_getaffinity(0))
    cpu = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    rows = []
    for name, n_blocks in (("c0", 1), ("c1", 1), ("c2", 1), ("c3", 1), ("c4", 2)):
        geom = synth.CONFIGS[name]
        acts = synth.make_activations(geom, 0)
        ws = [ob.weights_f64(synth.make_block_weights(geom, 0, i)) for i in range(n_blocks)]
        cos, sin = ob.rope_tables(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, geom.head_dim)
        x, txt, cond = ob.widen_bf16(acts["x"]), ob.widen_bf16(acts["txt"]), ob.widen_bf16(acts["cond"])
        t0 = time.perf_counter()
        ob.stack_forward(x, txt, acts["txt_len"], cond, ws, cos, sin, geom.eps)
        dt = time.perf_counter() - t0
        per_block = dt / n_blocks
        rows.append((name, geom.batch, geom.rows, n_blocks, dt, per_block, geom.block_flops() / per_block / 1e9))
        print(f"oracle {name}: {n_blocks} block(s) in {dt:.2f} s", file=sys.stderr, flush=True)
    print(f"float64 oracle on {threads} threads of {cpu}")
    print("| workload | batch | rows per item | blocks timed | seconds | seconds per block | GFLOP/s |")
    print("|---|---|---|---|---|---|---|")
    for name, b, r, n, dt, pb, gf in rows:
        print(f"| {name} | {b} | {r} | {n} | {dt:.2f} | {pb:.2f} | {gf:.1f} |")
    c4 = rows[-1]
    print(f"\nThe 24-block c4 stack would take about {24 * c4[5]:.0f} s (12 x the two blocks timed).")


def graph_timing(torch, step, stream, steps):
    """ms per block forward when one block is captured in a HIP graph and replayed
    (outside the main timed region); None if capture is not possible here."""
    try:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for _ in range(3):
            graph.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return round(e0.elapsed_time(e1) / steps, 4)
    except Exception as exc:  # noqa: BLE001 - reported, not fatal to the main measurement
        print(f"bench: graph capture unavailable: {exc}", file=sys.stderr, flush=True)
        return None


def main():
    args = parse()
    if args.oracle_sweep:
        oracle_sweep()
        return
    if args.traffic_summary:
        from diffusion_transformer_denoiser_amd import synth
        traffic_summary(*args.traffic_summary, synth.CONFIGS["c2"])
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the block forward is "
              "measured on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    import torch

    from diffusion_transformer_denoiser_amd import moss, synth

    assert torch.cuda.is_available(), "no GPU"
    torch.cuda.set_device(0)
    rc = moss.moss_device_check(0)
    if rc != moss.MOSS_OK:
        raise SystemExit(f"device 0: {moss.moss_status_string(rc)}")

    geom = synth.CONFIGS[args.workload]
    if args.gemm_reference:
        print(json.dumps({"gemm_reference": gemm_reference(torch, moss, geom)}))
        return
    acts = synth.make_activations(geom, args.seed)
    wbits = synth.make_block_weights(geom, args.seed, 0)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()

    dims = moss.make_dims(geom.batch, geom.n_img, geom.n_txt, geom.d_model, geom.mlp_inner, geom.eps)
    x, txt, cond = dev(acts["x"]), dev(acts["txt"]), dev(acts["cond"])
    wdev = {k: dev(v) for k, v in wbits.items()}  # kept alive for the whole run
    w = moss.make_weights(wdev)
    rope = torch.empty(2, geom.rows, 64, dtype=torch.float32, device="cuda")
    moss.moss_rope_build(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, rope)
    ws = torch.empty(moss.moss_workspace_bytes(dims, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty(geom.batch, geom.rows, geom.d_model, dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        # on torch's current stream (the capture stream while a graph is being recorded)
        moss.moss_block_forward(dims, x, txt, acts["txt_len"], cond, w, rope, out, ws)

    if args.copy_calibration:
        src = torch.ones(CALIB_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"bench: warmup {args.warmup} done; timing {args.steps} block forwards", file=sys.stderr, flush=True)

    # the up projection of every PROBE_EVERY-th timed step is bracketed by events (each record leaves
    # a few microseconds of stream time between kernels; spreading them keeps that out of most steps)
    n_probe = max(1, (args.steps + PROBE_EVERY - 1) // PROBE_EVERY)
    moss.moss_probe_arm("UP", n_probe, PROBE_EVERY)
    step_ms, loop_ms, wall, identical, digest = timed_steps(torch, step, out, stream, args.steps)
    up_ms = moss.moss_probe_collect(n_probe)
    med = float(np.median(step_ms))
    p10, p90 = (float(v) for v in np.percentile(step_ms, [10, 90]))

    graph_ms = graph_timing(torch, step, stream, min(args.steps, 50))
    extras = {}
    if not args.no_extras:
        print("bench: per-step times, 24-block stack, larger pictures", file=sys.stderr, flush=True)
        extras["step_times"] = per_step(torch, moss, step, geom)
        extras["step_times_cold_cache"] = per_step(torch, moss, step, geom, cold="write")
        extras["step_times_cold_read"] = per_step(torch, moss, step, geom, cold="read")
        extras["hbm_reference"] = hbm_reference(torch, moss, geom)
        extras["gemm_reference"] = gemm_reference(torch, moss, geom)
        extras["stack_c4"] = stack_timing(torch, moss, synth.CONFIGS["c4"], args.seed)
        extras["larger_pictures"] = larger_pictures(torch, moss, w, args.seed)

    value = 1000.0 / med
    flops = geom.block_flops()
    tflops = flops * value / 1e12
    m = geom.batch * geom.rows
    up_flops = 2.0 * m * (2 * geom.mlp_inner) * geom.d_model
    up_avg_ms = float(np.mean(up_ms)) if up_ms else float("nan")
    up_tflops = up_flops / (up_avg_ms / 1e3) / 1e12
    traffic = stored_traffic() if args.workload == "c2" else None
    names = {"c2": "4096 image + 34 text rows (64x64 grid)", "p1280": "5120 image + 34 text rows (64x80 grid)",
             "p1408": "5632 image + 34 text rows (64x88 grid)", "p1536": "6144 image + 34 text rows (64x96 grid)"}

    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "block-forwards/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med, 4),
        "ms_per_step_p10": round(p10, 4),
        "ms_per_step_p90": round(p90, 4),
        "ms_per_step_mean": round(float(np.mean(step_ms)), 4),
        "ms_per_step_loop": round(loop_ms, 4),
        "wall_ms_per_step": round(wall * 1000 / args.steps, 4),
        "timing": "median of the per-step HIP event pairs on the launch stream; p10 / p90 and the mean beside it; "
                  "loop = one event pair around all steps (includes the copy of each output for the comparison)",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) random-init weights)",
        "tflops": round(tflops, 2),
        "mfma_frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "block_gflop": round(flops / 1e9, 2),
        "output_sha256_16": digest,
        "timed_outputs_identical": identical,
        "graph_ms_per_step": graph_ms,
        **extras,
        "config": {"workload": f"single DiT denoiser block forward, {names[args.workload]}, D=3072, 24 heads x 128, "
                               "MLP inner 12288 SiLU-gated, batch 1",
                   "global_batch": 1, "seq_len": geom.rows, "parallelism": "single GPU"},
        "roofline": {"kernel": f"up projection GEMM with the SiLU gate epilogue ({m} x {2 * geom.mlp_inner} x "
                               f"{geom.d_model}; whole 256-row tiles, then the leftover rows as 64 x 64 tiles in a "
                               "second launch, timed together)",
                     "bound": "mfma",
                     "achieved": round(up_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(up_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic["traffic_bytes"] if traffic else None,
                     "traffic_unit": "HBM bytes per up projection (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "algorithmic_bytes": 2 * (m * geom.d_model + 2 * geom.mlp_inner * geom.d_model
                                               + m * geom.mlp_inner),
                     "launches_timed": len(up_ms), "avg_launch_ms": round(up_avg_ms, 5)},
    }
    if not args.no_cpu_baseline:
        print("bench: timing the float64 oracle on one block (CPU baseline)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(geom, acts, wbits)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
