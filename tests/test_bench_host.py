"""bench.py's host logic that turns rocprofv3 output into the committed summaries and into the bench
line's traffic figure (no GPU): FETCH_SIZE / WRITE_SIZE scaled by what they read for the plain
256 MiB copy, the up projection's two launches summed per projection, the source-hash guard on the
stored record, the counter formulas of the MFMA / wait summary, and the kernel-trace table.  Inputs
are small synthetic CSVs in rocprofv3's column layout and a database with the two tables the trace
summary reads."""
import csv
import json
import os
import re
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from diffusion_transformer_denoiser_amd import synth  # noqa: E402

COPY = "__amd_rocclr_copyBuffer"


def _full(short):
    return "void (anonymous namespace)::" + short + "(unsigned short const*, int, unsigned short const*, int)"


def _counter_csv(folder, rows):
    """rows: (dispatch id, kernel name, grid size, counter, value)"""
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writerows(rows)


def _record(path):
    return json.loads(re.search(r"```json\n(.*?)\n```", open(path).read(), re.S).group(1))


def test_traffic_record_scales_by_the_copy_and_sums_the_two_launches(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.md"))
    main, tail = (_full(k) for k in bench.UP_KERNELS)
    # three up projections; an upload copy of a few KiB beside the 256 MiB calibration copy
    f_main, f_tail = [700000.0, 710000.0, 720000.0], [50000.0, 51000.0, 52000.0]
    w_main, w_tail = [99000.0, 99100.0, 99200.0], [100.0, 110.0, 120.0]
    f_copy, w_copy = 131072.0, 262144.0  # what gfx950 reads for the 256 MiB copy (factors 2 and 1)
    for counter, folder, mv, tv, cv in (("FETCH_SIZE", "f", f_main, f_tail, f_copy),
                                        ("WRITE_SIZE", "w", w_main, w_tail, w_copy)):
        rows = [(0, COPY, 512, counter, 3.0), (1, COPY, 65536, counter, cv)]
        for i in range(3):
            rows += [(10 + 2 * i, main, 131072, counter, mv[i]), (11 + 2 * i, tail, 49152, counter, tv[i]),
                     (20 + i, _full("attn_fwd_kernel"), 208896, counter, 1234.0)]
        _counter_csv(str(tmp_path / folder), rows)
    geom = synth.CONFIGS["c2"]
    bench.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), geom)

    rec = _record(bench.TRAFFIC_FILE)
    fetch = np.mean(np.add(f_main, f_tail)) * 1024 * (bench.CALIB_BYTES / (f_copy * 1024))
    write = np.mean(np.add(w_main, w_tail)) * 1024 * (bench.CALIB_BYTES / (w_copy * 1024))
    assert rec["fetch_bytes"] == round(fetch) and rec["write_bytes"] == round(write)
    assert rec["traffic_bytes"] == round(fetch + write)
    m, d, f = geom.batch * geom.rows, geom.d_model, geom.mlp_inner
    assert rec["algorithmic_bytes"] == 2 * (m * d + 2 * f * d + m * f)  # A and W read, z written, bf16
    assert rec["kernels"] == list(bench.UP_KERNELS)
    assert rec["gemm_source_sha256"] == bench.gemm_source_digest()

    # the bench line takes the record only while the GEMM source is the one the counters were taken on
    assert bench.stored_traffic() == rec
    text = open(bench.TRAFFIC_FILE).read().replace(rec["gemm_source_sha256"], "0" * 64)
    open(bench.TRAFFIC_FILE, "w").write(text)
    assert bench.stored_traffic() is None


def test_counter_summary_formulas(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "COUNTER_FILE", str(tmp_path / "counters.md"))
    folder = tmp_path / "pass"
    os.makedirs(folder)
    n_xcc, n_simd = 8, 1024
    with open(folder / "run_agent_info.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Agent_Type", "Num_Xcc", "Simd_Count"])
        w.writerow(["GPU", n_xcc, n_simd])
    # one kernel, two dispatches of 100 us at 2.0 GHz: 50% MFMA busy, 25% waiting, 10% issue-blocked,
    # 1e8 MFMA mops (x 512 flops) per dispatch
    name, grid, dur_ns, ghz = _full("gemm_nt_kernel<256, 256, 2, 4, 1, 2, 6, 3>"), 131072, 100000, 2.0
    cycles = ghz * dur_ns  # per XCD
    per = {"GRBM_GUI_ACTIVE": n_xcc * cycles, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * cycles * n_simd,
           "SQ_WAVE_CYCLES": 4.0e7, "SQ_WAIT_ANY": 1.0e7, "SQ_WAIT_INST_ANY": 4.0e6,
           "SQ_LDS_IDX_ACTIVE": 0.2 * cycles * (n_simd // 4), "SQ_LDS_BANK_CONFLICT": 0.0,
           "SQ_INSTS_VALU_MFMA_MOPS_BF16": 1.0e8}
    rows = [(dsp, name, grid, c, v) for dsp in (1, 2) for c, v in per.items()]
    _counter_csv(str(folder), rows)
    with open(folder / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Start_Timestamp", "End_Timestamp"])
        w.writerows([(1, 1000, 1000 + dur_ns), (2, 5000000, 5000000 + dur_ns)])
    bench.counter_summary([str(folder)])

    row = [l for l in open(bench.COUNTER_FILE).read().splitlines() if l.startswith("| gemm_nt_kernel")]
    assert len(row) == 1
    cells = [c.strip() for c in row[0].strip("|").split("|")]
    assert cells[:4] == ["gemm_nt_kernel<256, 256, 2, 4, 1, 2, 6, 3>", str(grid), "2", "100.0"]
    assert cells[4] == "2.00"      # GRBM_GUI_ACTIVE / XCDs / duration
    assert cells[5] == "50.0%"     # MFMA busy cycles / (busy cycles per XCD x SIMDs)
    assert cells[6] == "25.0%"     # SQ_WAIT_ANY / SQ_WAVE_CYCLES
    assert cells[7] == "10.0%"     # SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES
    assert cells[8] == "20.0%"     # LDS busy
    assert cells[10] == "512"      # 1e8 mops x 512 flops / 100 us, in TFLOP/s


def test_trace_summary_groups_dispatches_by_kernel_and_grid(tmp_path, capsys):
    import sqlite3
    db = str(tmp_path / "trace.db")
    c = sqlite3.connect(db)
    c.execute("create table rocpd_info_kernel_symbol (id integer, display_name text, arch_vgpr_count integer, "
              "accum_vgpr_count integer, group_segment_size integer)")
    c.execute("create table rocpd_kernel_dispatch (kernel_id integer, grid_size_x integer, grid_size_y integer, "
              "workgroup_size_x integer, start integer, end integer)")
    c.executemany("insert into rocpd_info_kernel_symbol values (?, ?, ?, ?, ?)",
                  [(1, _full("gemm_nt_kernel<224, 256, 1, 8, 2, 2, 6, 3>"), 128, 0, 155648),
                   (2, _full("attn_fwd_kernel"), 104, 0, 98304)])
    # the 224-row launch at two shapes' worth of time (out 80 + 90 us, down 300 us) and the attention twice
    c.executemany("insert into rocpd_kernel_dispatch values (?, ?, ?, ?, ?, ?)",
                  [(1, 116736, 1, 512, 0, 80000), (1, 116736, 1, 512, 100000, 190000),
                   (1, 116736, 1, 512, 200000, 500000),
                   (2, 8704, 24, 512, 600000, 830000), (2, 8704, 24, 512, 900000, 1130000)])
    c.commit()
    c.close()
    bench.trace_summary(db)
    rows = [l for l in capsys.readouterr().out.splitlines() if l.startswith("| ") and not l.startswith("| kernel |")]
    cells = [[x.strip() for x in r.strip("|").split("|")] for r in rows]
    assert [r[0] for r in cells] == ["gemm_nt_kernel<224, 256, 1, 8, 2, 2, 6, 3>", "attn_fwd_kernel"]  # by total time
    gemm, attn = cells
    assert gemm[1:8] == ["116736x1", "512", "128", "0", "155648", "3", "156.7"]  # (80 + 90 + 300) / 3 us
    assert gemm[8:10] == ["80.0", "300.0"]
    assert attn[1] == "8704x24" and attn[6:8] == ["2", "230.0"]
    assert gemm[10] == f"{100 * 470 / 930:.1f}%" and attn[10] == f"{100 * 460 / 930:.1f}%"
