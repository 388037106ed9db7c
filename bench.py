"""Benchmark of the IQ4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one pass of the hot path over resident synthetic inputs:
  * the verify-window matvec, W 4096 x 4096 in IQ4 blocks, one call at each of
    T = 1, 2, 3, 4 fp32 columns, each call on a different one of R weight copies
    (R * 9.4 MB > 2 x the 256 MB Infinity Cache, so the weights stream from HBM).

Prints ONE JSON line.  ``value`` = effective weight GB/s of the matvec calls
(total weight bytes / total kernel time, T = 1..4).  The roofline object is measured
live with HIP events on the launch stream; ``cpu_baseline`` times the CPU oracle on a
bounded sample of the same workload.
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

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def build_verify_inputs(torch, iq4, synth, copies: int):
    """W 4096 x 4096 quantised on the GPU (seed 102), packed, replicated `copies`
    times; X = 4 fp32 columns (seed 102)."""
    n = k = 4096
    w = torch.from_numpy(synth.weights_f32(synth.SEED_VERIFY, synth.TAG_WEIGHT, n, k)).cuda()
    blocks = torch.empty(n * k // 32 * 18, dtype=torch.uint8, device="cuda")
    iq4.iq4_quantize_blocks(w, n * k // 32, blocks)
    nbytes = iq4.iq4_packed_bytes(n, k)
    packed = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    iq4.iq4_pack_weights(blocks, n, k, packed[0])
    for p in packed[1:]:
        p.copy_(packed[0])
    x = torch.from_numpy(synth.acts_f32(synth.SEED_VERIFY, synth.TAG_X, 4, k)).cuda()
    y = torch.empty((4, n), dtype=torch.float32, device="cuda")
    wsb = iq4.iq4_qmv_workspace_size(n, k)
    ws = torch.zeros(max(wsb, 256), dtype=torch.uint8, device="cuda")
    del w
    return dict(n=n, k=k, packed=packed, x=x, y=y, wbytes=nbytes, ws=ws, wsb=wsb)


def cpu_baseline(min_seconds: float = 10.0):
    """The CPU oracle on the verify-window matvec, T = 1..4 per pass, repeated until
    `min_seconds` of work; returns GB/s of weight bytes like the GPU value."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = 1
    n = k = 4096
    w = synth.weights_f32(synth.SEED_VERIFY, synth.TAG_WEIGHT, n, k)
    blocks = oracle.encode_blocks(w.reshape(-1, 32))
    x = synth.acts_f32(synth.SEED_VERIFY, synth.TAG_X, 4, k)
    wbytes = blocks.size
    done_bytes, passes = 0, 0
    t0 = time.perf_counter()
    while True:
        for T in (1, 2, 3, 4):
            oracle.qmv(blocks, n, k, x[:T])
            done_bytes += wbytes
        passes += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or passes >= 50:
            break
    return {"value": done_bytes / el / 1e9, "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{passes} passes of the verify-window matvec (W 4096x4096, T=1..4), "
                      f"numpy float64, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--copies", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import dequant_matmul_iq4_amd as iq4
    import synth

    torch.cuda.set_device(0)
    log("building inputs")
    V = build_verify_inputs(torch, iq4, synth, args.copies)
    stream = torch.cuda.current_stream()
    n, k = V["n"], V["k"]

    it = [0]

    def mmvq(T):
        p = V["packed"][it[0] % len(V["packed"])]
        it[0] += 1
        iq4.iq4_qmv_multi(p, n, k, V["x"], k, T, V["y"], n, V["ws"], V["wsb"], stream)

    def step():
        for T in (1, 2, 3, 4):
            mmvq(T)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The timed region replays HIP graphs of the step's launches: per-launch CPU
    # overhead (several us) would otherwise hide kernels that take a few us.
    # One graph per T: R launches, each on the next weight copy (cold weights).
    R = len(V["packed"])
    graphs = {}
    for T in (1, 2, 3, 4):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=torch.cuda.Stream()):
            s2 = torch.cuda.current_stream()
            for r in range(R):
                iq4.iq4_qmv_multi(V["packed"][r], n, k, V["x"], k, T, V["y"], n, V["ws"], V["wsb"], s2)
        graphs[T] = g
    for T in (1, 2, 3, 4):  # warm replays
        graphs[T].replay()
    torch.cuda.synchronize()

    # K steps = K x (T = 1..4) launches, timed per T with events around graph replays
    reps = max(1, args.steps // R) if args.steps >= R else 1
    per_T = {}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    total_ms, total_launches = 0.0, 0
    for T in (1, 2, 3, 4):
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(reps):
            graphs[T].replay()
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end)
        per_T[T] = ms / (reps * R)  # ms per launch
        total_ms += ms
        total_launches += reps * R
    steps_timed = total_launches // 4
    ms_step = total_ms / steps_timed
    tot_ms = sum(per_T.values())
    wb = V["wbytes"]
    value = 4 * wb / (tot_ms * 1e-3) / 1e9
    alg = sum(wb + 2 * 4 * T * k for T in (1, 2, 3, 4))  # weights + X + Y
    achieved = alg / (tot_ms * 1e-3) / 1e9

    res = {
        "metric": "MMVQ effective weight GB/s at T=1..4; ms per 3,256-token MoE layer",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps_timed,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "verify-window MMVQ W 4096x4096 IQ4 (18 B/32 w), X fp32 T=1..4, "
                               f"{args.copies} rotating weight copies (cold)",
                   "mmvq_us_per_T": {str(T): round(per_T[T] * 1e3, 3) for T in per_T},
                   "mmvq_weight_gbs_per_T": {str(T): round(wb / (per_T[T] * 1e-3) / 1e9, 1) for T in per_T}},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "qmv_kernel (verify-window matvec, T=1..4 mean)"},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline()
    print(json.dumps(res))


if __name__ == "__main__":
    main()
