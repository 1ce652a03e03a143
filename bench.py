"""Benchmark of the W4A16 decode path on one MI355X.

One step = one pass of the vocabulary-head workload: the batch-1 W4A16 GEMV of a
262144 x 1536 packed table (4-bit codes, group 32, bf16 steps) with a bf16
activation vector, plus the 4-bit row gather of 64 token ids from the same
table (the table serves both the output layer and the input lookup, as on the
dev.to page "Gemma 4 on a 4 GB GPU in Plain PyTorch", section "Step 2 - Keep
the Vocabulary Tables in 4-Bit").  Three copies of the table are rotated so that
the 256 MB Infinity Cache cannot hold the working set.

`value` = algorithmic HBM bytes of one step / measured step time (GB/s, 1e9 B).
Printed as ONE JSON line, with the dominant kernel's roofline and the CPU
oracle's time on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E bandwidth

V, K, NIDS = 262144, 1536, 64
COPIES = 3


def gbps(nbytes: float, seconds: float) -> float:
    """Effective bandwidth in GB/s (GB = 1e9 B): bytes moved / time."""
    return nbytes / seconds / 1e9


def w4_bytes(n: int, k: int) -> int:
    """Packed bytes of an n x k W4 matrix: codes (k/2 per row) + bf16 steps."""
    return n * (k // 2) + n * (k // 32) * 2


def gemv_bytes(n: int, k: int) -> int:
    """Algorithmic bytes of one GEMV: packed weights + 16-bit x + fp32 y."""
    return w4_bytes(n, k) + 2 * k + 4 * n


def gather_bytes(n_ids: int, k: int) -> int:
    """Algorithmic bytes of a row gather: the packed rows, the ids, bf16 out."""
    return w4_bytes(n_ids, k) + 4 * n_ids + 2 * n_ids * k


STEP_BYTES = gemv_bytes(V, K) + gather_bytes(NIDS, K)


def cpu_baseline(codes, steps, x, ids, min_seconds: float = 10.0):
    """The oracle, as it stands, on the same workload: the full vocabulary-head
    GEMV (OpenMP over rows) plus the gather, repeated for >= min_seconds."""
    import oracle
    import synth
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.gemv(codes, steps, V, K, x, synth.BF16, threads=True)
        oracle.gather(codes, steps, V, K, ids)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    per_step = el / reps
    return {"value": round(gbps(STEP_BYTES, per_step), 3), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{reps} full steps (262144x1536 GEMV + 64-row gather), "
                      f"{per_step:.3f} s per step"}


def probe_ceiling(w4, torch, nbytes: int = 2 << 30, reps: int = 10) -> float:
    """Plain streaming-read ceiling (GB/s) of this device."""
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    buf.fill_(1)
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        w4.w4_probe_stream(buf, out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        w4.w4_probe_stream(buf, out)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / reps
    del buf
    return gbps(nbytes, t)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(this path runs on one MI355X; see the design notes on sharding)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import bit_weight_only_02_amd as w4
    import synth

    torch.cuda.set_device(0)
    rng = np.random.default_rng(0)
    codes, steps = synth.w4_matrix(rng, V, K)
    x = synth.activations(rng, K, synth.BF16)
    ids = synth.token_ids(rng, NIDS, V)

    dcodes = [torch.from_numpy(codes.view(np.int32)).cuda()]
    dsteps = [torch.from_numpy(steps.view(np.int16)).cuda().view(torch.bfloat16)]
    for _ in range(COPIES - 1):
        dcodes.append(dcodes[0].clone())
        dsteps.append(dsteps[0].clone())
    dx = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    dids = torch.from_numpy(ids).cuda()
    y = torch.empty(V, dtype=torch.float32, device="cuda")
    g = torch.empty((NIDS, K), dtype=torch.bfloat16, device="cuda")

    def step(i, ev=None):
        c = i % COPIES
        if ev is not None:
            ev[0].record()
        w4.w4_gemv(dcodes[c], dsteps[c], dx, y)
        if ev is not None:
            ev[1].record()
        w4.w4_embed_gather(dcodes[c], dsteps[c], dids, g)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        step(i, evs[i])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_s = t_start.elapsed_time(t_end) / 1e3 / args.steps
    gemv_s = sum(a.elapsed_time(b) for a, b in evs) / 1e3 / args.steps

    ceiling = probe_ceiling(w4, torch)
    achieved = gbps(gemv_bytes(V, K), gemv_s)
    result = {
        "metric": "achieved HBM GB/s (% of peak) for W4A16 GEMV; us per 35-layer decode sweep",
        "value": round(gbps(STEP_BYTES, step_s), 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16/bf16 products, fp32 accumulate",
        "data": "synthetic (seeded; codes uniform 0..15, steps bf16(|N(0,0.02)|+1e-4), x ~ N(0,1))",
        "config": {"workload": "vocabulary-head W4A16 GEMV 262144x1536 (bf16 x, batch 1) + "
                               "4-bit row gather of 64 ids from the same table",
                   "table_copies_rotated": COPIES, "step_bytes": STEP_BYTES},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None, "kernel": "w4::gemv_kernel",
                     "bytes_per_launch": gemv_bytes(V, K),
                     "avg_launch_us": round(gemv_s * 1e6, 3)},
        "extra": {"gemv_weight_GBps": round(gbps(w4_bytes(V, K), gemv_s), 2),
                  "probe_read_ceiling_GBps": round(ceiling, 1),
                  "gemv_frac_of_probe": round(achieved / ceiling, 4),
                  "timed_wall_s": round(wall, 3)},
    }
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(codes, steps, x, ids)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
