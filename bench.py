"""Benchmark: DiT denoiser block forwards per second at 4096 image + 34 text rows.

One step is one ``moss_block_forward`` (every step of the block: row join,
adaLN GEMV, two modulated RMSNorms, QKV / out / up / down projections, q/k
norm + rotary pack, attention, SiLU product, two gated adds) on one batch of
seeded synthetic inputs already resident in HBM: D = 3072, 24 heads x 128,
MLP 12288, a 64x64 image grid plus 34 text rows (the 1024x1024 picture's
shape on the MOSS-Image transformer page, "Measured"), weights N(0, 0.02).

Prints one JSON line.  ``roofline`` is for the up projection (the largest
kernel, 43% of the block's flops), timed live with HIP events recorded by the
library around each of its launches inside the timed region.  ``cpu_baseline``
times the float64 oracle on one block forward of the same workload.
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
METRIC = "denoiser block-forwards/s and TFLOP/s at 4096+34 tokens; MFMA % of peak"


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    p.add_argument("--seed", type=int, default=0)
    return p.parse_args()


def cpu_baseline(geom, acts, wbits):
    """Time the float64 oracle on one block forward of the same workload."""
    from oracle import dit_block as ob
    threads = len(os.sched_getaffinity(0))
    cos, sin = ob.rope_tables(geom.n_txt, geom.grid_h, geom.grid_w, geom.theta, geom.head_dim)
    x, txt, cond = ob.widen_bf16(acts["x"]), ob.widen_bf16(acts["txt"]), ob.widen_bf16(acts["cond"])
    w = ob.weights_f64(wbits)
    t0 = time.perf_counter()
    ob.block_forward(x, txt, acts["txt_len"], cond, w, cos, sin, geom.eps)
    dt = time.perf_counter() - t0
    return {"value": 1.0 / dt, "unit": "block-forwards/s", "cores": threads, "kind": "oracle",
            "sample": f"one full block forward of this workload in float64 NumPy ({dt:.1f} s; BLAS threads = "
                      f"{threads} host cores)"}


def main():
    args = parse()
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

    geom = synth.CONFIGS["c2"]
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
        moss.moss_block_forward(dims, x, txt, acts["txt_len"], cond, w, rope, out, ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"bench: warmup {args.warmup} done; timing {args.steps} block forwards", file=sys.stderr, flush=True)

    moss.moss_probe_arm("UP", args.steps)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    up_ms = moss.moss_probe_collect(args.steps)
    ms = ev0.elapsed_time(ev1) / args.steps
    digest = hashlib.sha256(out.cpu().numpy().tobytes()).hexdigest()[:16]

    value = 1000.0 / ms
    flops = geom.block_flops()
    tflops = flops * value / 1e12
    m = geom.batch * geom.rows
    up_flops = 2.0 * m * (2 * geom.mlp_inner) * geom.d_model
    up_avg_ms = float(np.mean(up_ms)) if up_ms else float("nan")
    up_tflops = up_flops / (up_avg_ms / 1e3) / 1e12

    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "block-forwards/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "wall_ms_per_step": round(wall * 1000 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) random-init weights)",
        "tflops": round(tflops, 2),
        "mfma_frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "block_gflop": round(flops / 1e9, 2),
        "output_sha256_16": digest,
        "config": {"workload": "single DiT denoiser block forward, 4096 image + 34 text rows (64x64 grid), "
                               "D=3072, 24 heads x 128, MLP inner 12288 SiLU-gated, batch 1",
                   "global_batch": 1, "seq_len": geom.rows, "parallelism": "single GPU"},
        "roofline": {"kernel": "up projection GEMM (4130 x 24576 x 3072)", "bound": "mfma",
                     "achieved": round(up_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(up_tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "launches_timed": len(up_ms), "avg_launch_ms": round(up_avg_ms, 5)},
    }
    if not args.no_cpu_baseline:
        print("bench: timing the float64 oracle on one block (CPU baseline)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(geom, acts, wbits)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
