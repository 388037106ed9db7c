"""Benchmark of the IQ4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one pass over every step of the hot path, on resident synthetic inputs:
  1. verify-window matvec: W 4096 x 4096 IQ4, one call at each T = 1, 2, 3, 4 fp32
     columns, each call on the next of R weight copies (R x 9.4 MB > 2 x the 256 MB
     Infinity Cache, so weights stream from HBM);
  2. block decode of that matrix to binary16 (iq4_dequant_blocks);
  3. MoE decode step: 4 fp32 tokens, top-8 of 128 experts (hidden 2048, inter 768),
     rotating over eight expert banks (8 x 340 MB, cold); its reported per-step time
     comes from a graph of the eight steps replayed back to back;
  4. MoE prefill layer: 3,256 f16 tokens, Zipf(1.1)-skewed top-8 routing, same bank;
  5. long-prompt projection: 13,056 f16 tokens x W 14,336 x 4,096, 512-token chunks.
Besides the step: the verify-window matvec on 8-bit activations (the q8_1 decode
numerics) at T = 1..4 over the same weight copies, and the activation quantisation.

Prints ONE JSON line.  ``value`` = effective weight GB/s of the verify-window matvec
(total weight bytes of the T = 1..4 calls / their total time).  Launch times come from
HIP events around graph replays on the launch stream (many launches per replay, so
per-launch CPU overhead does not enter), medians of 5 interleaved rounds after >= 200 ms
of clock warm-up.  Beside the published peaks, each roofline states its rate against a
ceiling measured in the same run (a plain streaming read of the same bytes, a pure
matrix-core loop).  ``cpu_baseline`` times the CPU oracle on the matvec workload;
``cpu_baselines`` on every config (threads = the cores this process may use).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import ctypes
import statistics

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
F16_MFMA_PEAK_TFS = 2500.0  # MI355X dense f16 matrix throughput, published

HIDDEN, INTER, N_EXPERT, TOP_K = 2048, 768, 128, 8
N_BANKS = 8                 # expert banks the decode step rotates over

# HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE passes (each scaled by what
# the counter reads for a 256 MiB device copy), kept with a digest of the kernel's sources
# at the time: a kernel changed since then reports traffic null.  Commands and raw
# figures: profiles/<name>.txt.
MEASURED_TRAFFIC = {
    "dequant_staged_4096x4096_f16": (43046990, "23a9b127dfaa11ea", ("format.hip", "common.hpp")),
    "qmv_dense_4096x4096_T1-4": (9927972, "6a2fa7d6d7b1b8ad", ("qmv.hip", "qmv.hpp", "common.hpp")),
    "qmv_q8_4096x4096_T1-4": (9674811, "6a2fa7d6d7b1b8ad", ("qmv.hip", "qmv.hpp", "common.hpp")),
    "qmv_grouped_gateup_moe_decode_4tok": (59952873, "6a2fa7d6d7b1b8ad", ("qmv.hip", "qmv.hpp", "common.hpp")),
    "qmv_down_combine_moe_decode_4tok": (28656195, "6a2fa7d6d7b1b8ad", ("qmv.hip", "qmv.hpp", "common.hpp")),
    "xs_qmv_mfma_6144x2560_T1-4": (8760985, "83810f3202cde74d", ("xs.hip", "common.hpp")),
    "xs_qmv_mfma_2560x6144_T1-4": (9015365, "83810f3202cde74d", ("xs.hip", "common.hpp")),
    "xs_dequant_6144x2560_f16": (39844042, "83810f3202cde74d", ("xs.hip", "common.hpp")),
    "qgemm_gateup_moe_prefill_3256tok": (590123568, "91b289d98fd124c6", ("gemm.hip", "gemm.hpp", "common.hpp")),
    "qgemm_down_moe_prefill_3256tok": (400111105, "91b289d98fd124c6", ("gemm.hip", "gemm.hpp", "common.hpp")),
    "qgemm_dense_13056x4096x14336_chunk512": (94901830, "91b289d98fd124c6", ("gemm.hip", "gemm.hpp", "common.hpp")),
}


def measured_traffic(name):
    import hashlib
    nbytes, digest, files = MEASURED_TRAFFIC[name]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "dequant_matmul_iq4_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return nbytes if h.hexdigest()[:16] == digest else None


def sum_traffic(*names):
    parts = [measured_traffic(nm) for nm in names]
    return None if any(p is None for p in parts) else sum(parts)


def mean_traffic(*names):
    total = sum_traffic(*names)
    return None if total is None else total / len(names)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def quantize_pack(torch, iq4, w32, n, k):
    """float32 [n, k] on the GPU -> packed IQ4 tensor (and the row-block bytes)."""
    blocks = torch.empty(n * k // 32 * 18, dtype=torch.uint8, device="cuda")
    iq4.iq4_quantize_blocks(w32.contiguous(), n * k // 32, blocks)
    packed = torch.empty(iq4.iq4_packed_bytes(n, k), dtype=torch.uint8, device="cuda")
    iq4.iq4_pack_weights(blocks, n, k, packed)
    return packed, blocks


def build_bank(torch, iq4, synth, seed):
    """128 experts x (gate, up: 768 x 2048; down: 2048 x 768), packed, expert-major."""
    sg = iq4.iq4_packed_bytes(INTER, HIDDEN)
    sd = iq4.iq4_packed_bytes(HIDDEN, INTER)
    gate = torch.empty(N_EXPERT * sg, dtype=torch.uint8, device="cuda")
    up = torch.empty(N_EXPERT * sg, dtype=torch.uint8, device="cuda")
    down = torch.empty(N_EXPERT * sd, dtype=torch.uint8, device="cuda")
    for e in range(N_EXPERT):
        for which, dst, n, k, size in (("gate", gate, INTER, HIDDEN, sg), ("up", up, INTER, HIDDEN, sg),
                                       ("down", down, HIDDEN, INTER, sd)):
            w = synth.weights_f32_torch(seed, synth.tag_expert(e, which), n, k, device="cuda")
            p, _ = quantize_pack(torch, iq4, w, n, k)
            dst[e * size:(e + 1) * size].copy_(p)
    return gate, up, down


def route(torch, iq4, logits):
    n = logits.shape[0]
    ids = torch.empty((n, TOP_K), dtype=torch.int32, device="cuda")
    w = torch.empty((n, TOP_K), dtype=torch.float32, device="cuda")
    iq4.iq4_route_topk(logits.contiguous(), n, N_EXPERT, TOP_K, ids, w)
    return ids, w


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baselines(min_seconds: float = 8.0):
    """The CPU oracle (as it stands: numpy float64) timed on this host's cores, every
    config.  Threads = the cores this
    process may run on (len(os.sched_getaffinity(0))), the BLAS pool limited to that.
    Returns (headline entry for the verify-window matvec, per-config entries)."""
    import statistics
    import oracle
    import synth
    from threadpoolctl import threadpool_limits

    cores = len(os.sched_getaffinity(0))
    model = cpu_model()
    enc = lambda w: oracle.encode_blocks(w.reshape(-1, 32))  # noqa: E731
    per = {}
    with threadpool_limits(limits=cores):
        # verify-window matvec (the headline), T = 1..4 per pass, at least min_seconds
        n = k = 4096
        b2 = enc(synth.weights_f32(synth.SEED_VERIFY, synth.TAG_WEIGHT, n, k))
        x2 = synth.acts_f32(synth.SEED_VERIFY, synth.TAG_X, 4, k)
        done_bytes, passes, t0 = 0, 0, time.perf_counter()
        while True:
            for T in (1, 2, 3, 4):
                oracle.qmv(b2, n, k, x2[:T])
                done_bytes += b2.size
            passes += 1
            el = time.perf_counter() - t0
            if el >= min_seconds or passes >= 50:
                break
        head = {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
                "cpu": model,
                "sample": f"{passes} passes of the verify-window matvec (W 4096x4096, T=1..4): oracle decode + "
                          f"float64 product, {el:.1f} s"}

        def median_of(fn, runs=5):
            ts = []
            for _ in range(runs):
                a = time.perf_counter()
                fn()
                ts.append(time.perf_counter() - a)
            return statistics.median(ts)

        # plumbing matvec 512 x 2048, T = 1: median of 5
        b1 = enc(synth.weights_f32(synth.SEED_PLUMBING, synth.TAG_WEIGHT, 512, 2048))
        x1 = synth.acts_f32(synth.SEED_PLUMBING, synth.TAG_X, 1, 2048)
        t1 = median_of(lambda: oracle.qmv(b1, 512, 2048, x1))
        per["plumbing_matvec_512x2048"] = {"ms": round(t1 * 1e3, 3), "weight_gbs": round(b1.size / t1 / 1e9, 4),
                                           "runs": "median of 5"}
        per["verify_window_matvec_4096x4096_T1-4"] = {"weight_gbs": head["value"], "runs": head["sample"]}

        # The expert bank and the long-prompt weights are random valid blocks (a seeded
        # binary16 scale of the synthetic weights' magnitude and uniform 4-bit indices):
        # the oracle's time does not depend on the values, and encoding 600 M weights
        # would take minutes of its own.
        rng = np.random.default_rng(synth.SEED_EXPERTS)

        def random_blocks(nn, kk):
            nb = nn * kk // 32
            out = np.empty((nb, 18), dtype=np.uint8)
            d = (0.06 / 127 * (0.5 + rng.random(nb))).astype(np.float16)
            out[:, 0:2] = d.astype("<f2").view(np.uint8).reshape(nb, 2)
            out[:, 2:18] = rng.integers(0, 256, (nb, 16), dtype=np.uint8)
            return out
        gate = [random_blocks(INTER, HIDDEN) for _ in range(N_EXPERT)]
        up = [random_blocks(INTER, HIDDEN) for _ in range(N_EXPERT)]
        down = [random_blocks(HIDDEN, INTER) for _ in range(N_EXPERT)]
        # MoE decode step: 4 fp32 tokens: median of 3
        dl = synth.logits_normal(synth.SEED_DECODE, synth.TAG_LOGITS, 4, N_EXPERT)
        dids, dw = oracle.route_topk(dl, TOP_K)
        dx = synth.acts_f32(synth.SEED_DECODE, synth.TAG_X, 4, HIDDEN)
        t3 = median_of(lambda: oracle.moe(dx, dids, dw, gate, up, down, HIDDEN, INTER), runs=3)
        ubytes = len(np.unique(dids)) * 3 * (INTER * HIDDEN // 32 * 18)
        per["moe_decode_step_4tok"] = {"us": round(t3 * 1e6, 1), "weight_gbs": round(ubytes / t3 / 1e9, 4),
                                       "runs": "median of 3"}
        # MoE prefill layer: one full run
        pl = synth.logits_zipf_gumbel(synth.SEED_PREFILL, synth.TAG_GUMBEL, 3256, N_EXPERT)
        pids, pw = oracle.route_topk(pl, TOP_K)
        px = synth.acts_f16(synth.SEED_PREFILL, synth.TAG_X, 3256, HIDDEN)
        a = time.perf_counter()
        oracle.moe(px, pids, pw, gate, up, down, HIDDEN, INTER)
        t4 = time.perf_counter() - a
        flop4 = 3256 * TOP_K * 3 * 2 * HIDDEN * INTER
        per["moe_prefill_layer_3256tok"] = {"ms": round(t4 * 1e3, 1), "gflops": round(flop4 / t4 / 1e9, 2),
                                            "runs": "one full run"}
        del gate, up, down
        # long-prompt projection: one 512-token chunk, scaled by 25.5 (13,056 = 25.5 x 512)
        b5 = random_blocks(14336, 4096)
        x5 = synth.acts_f16(synth.SEED_LONG, synth.TAG_X, 512, 4096)
        a = time.perf_counter()
        oracle.gemm(b5, 14336, 4096, x5)
        t5 = time.perf_counter() - a
        flop5 = 2 * 512 * 14336 * 4096
        per["long_prompt_projection_13056x4096x14336"] = {
            "ms_estimated": round(t5 * 25.5 * 1e3, 1), "gflops": round(flop5 / t5 / 1e9, 2),
            "runs": "one 512-token chunk timed, scaled by 25.5 (the full run is 25.5 chunks)"}
    return head, {"cores": cores, "cpu": model, "kind": "oracle", "configs": per}


def roof(bound, achieved, peak, unit, kernel, traffic=None, ceiling=None):
    """achieved against the published peak, and against the measured ceiling of the same
    bound on this GPU (a plain streaming read, or a pure matrix-core loop)."""
    r = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": kernel}
    if ceiling:
        r["measured_ceiling"] = round(ceiling, 1)
        r["frac_of_measured_ceiling"] = round(achieved / ceiling, 4)
    return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--copies", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-shared", action="store_true",
                    help="skip the shared-expert MoE timings beside the step (keeps per-kernel profiles "
                         "to the step's own launches)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy a float32 buffer of MIB MiB three times (the known-size "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import dequant_matmul_iq4_amd as iq4
    import synth

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    if args.copy_calibration:
        nel = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(nel, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_calibration} MiB three times")
        return
    Ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    # ---- inputs ------------------------------------------------------------------------
    log("verify-window matvec inputs")
    n = k = 4096
    w = synth.weights_f32_torch(synth.SEED_VERIFY, synth.TAG_WEIGHT, n, k, device="cuda")
    p0, vblocks = quantize_pack(torch, iq4, w, n, k)
    del w
    R = args.copies
    vcopies = [p0] + [p0.clone() for _ in range(R - 1)]
    wb = iq4.iq4_packed_bytes(n, k)
    vx = synth.acts_f32_torch(synth.SEED_VERIFY, synth.TAG_X, 4, k, device="cuda")
    vy = torch.empty((4, n), dtype=torch.float32, device="cuda")
    vwsb = iq4.iq4_qmv_workspace_size(n, k)
    vws = torch.zeros(max(vwsb, 256), dtype=torch.uint8, device="cuda")
    deq_out = torch.empty(n * k, dtype=torch.float16, device="cuda")
    # 8-bit activations of the same four columns (the q8_1 decode numerics)
    vq = torch.empty((4, k), dtype=torch.int8, device="cuda")
    vd = torch.empty((4, k // 32), dtype=torch.int16, device="cuda")
    iq4.iq4_quantize_q8_1(vx, 4, k, k, vq, vd)

    # The decode step reads ~80 MB of one bank; rotating over 8 banks (2.7 GB) puts 7
    # other steps' reads between two uses of a bank, well past the 256 MB Infinity Cache.
    log(f"expert banks ({N_BANKS} x 128 experts)")
    banks = [build_bank(torch, iq4, synth, synth.SEED_EXPERTS + 1000 * i) for i in range(N_BANKS)]
    bank_a = banks[0]

    log("MoE decode and prefill inputs")
    dx = synth.acts_f32_torch(synth.SEED_DECODE, synth.TAG_X, 4, HIDDEN, device="cuda")
    dlog = synth.acts_f32_torch(synth.SEED_DECODE, synth.TAG_LOGITS, 4, N_EXPERT, device="cuda")
    d_ids, d_w = route(torch, iq4, dlog)
    d_out = torch.empty((4, HIDDEN), dtype=torch.float32, device="cuda")
    d_wsb = iq4.iq4_moe_workspace_size(4, TOP_K, N_EXPERT, HIDDEN, INTER, iq4.IQ4_F32)
    d_ws = torch.empty(d_wsb, dtype=torch.uint8, device="cuda")
    n_unique = int(torch.unique(d_ids).numel())

    NP = 3256
    px = synth.acts_f16_torch(synth.SEED_PREFILL, synth.TAG_X, NP, HIDDEN, device="cuda")
    plog = torch.from_numpy(synth.logits_zipf_gumbel(synth.SEED_PREFILL, synth.TAG_GUMBEL, NP, N_EXPERT)).cuda()
    p_ids, p_w = route(torch, iq4, plog)
    p_out = torch.empty((NP, HIDDEN), dtype=torch.float32, device="cuda")
    p_wsb = iq4.iq4_moe_workspace_size(NP, TOP_K, N_EXPERT, HIDDEN, INTER, iq4.IQ4_F16)
    p_ws = torch.empty(p_wsb, dtype=torch.uint8, device="cuda")
    counts = torch.bincount(p_ids.reshape(-1).long(), minlength=N_EXPERT)

    log("long-prompt projection inputs")
    LN, LK, LM, CH = 14336, 4096, 13056, 512
    lw = synth.weights_f32_torch(synth.SEED_LONG, synth.TAG_WEIGHT, LN, LK, device="cuda")
    lpacked, _ = quantize_pack(torch, iq4, lw, LN, LK)
    del lw
    lx = synth.acts_f16_torch(synth.SEED_LONG, synth.TAG_X, LM, LK, device="cuda")
    ly = torch.empty((LM, LN), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    # ---- the step's calls ----------------------------------------------------------------
    def mmvq(copy, T, s):
        iq4.iq4_qmv_multi(vcopies[copy % R], n, k, vx, k, T, vy, n, vws, vwsb, s)

    def mmvq_q8(copy, T, s):
        iq4.iq4_qmv_q8(vcopies[copy % R], n, k, vq, vd, T, vy, n, vws, vwsb, s)

    def quantize_q8(s):
        iq4.iq4_quantize_q8_1(vx, 4, k, k, vq, vd, s)

    def dequant(s):
        iq4.iq4_dequant_blocks(vblocks, n * k // 32, iq4.IQ4_F16, deq_out, s)

    def moe_decode(bank, s):
        g, u, d = bank
        iq4.iq4_moe_expert_gemm(dx, iq4.IQ4_F32, 4, HIDDEN, d_ids, d_w, TOP_K, N_EXPERT, HIDDEN, INTER,
                                g, u, d, d_out, HIDDEN, d_ws, d_wsb, 0, s)

    def moe_prefill(s):
        g, u, d = bank_a
        iq4.iq4_moe_expert_gemm(px, iq4.IQ4_F16, NP, HIDDEN, p_ids, p_w, TOP_K, N_EXPERT, HIDDEN, INTER,
                                g, u, d, p_out, HIDDEN, p_ws, p_wsb, 0, s)

    def dense(s):
        iq4.iq4_qgemm(lpacked, LN, LK, lx, LM, LK, ly, LN, CH, s)

    # The small calls are replayed from HIP graphs (their CPU launch cost would otherwise
    # exceed their GPU time); each step advances through the weight copies.
    def capture(fn):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.graph(g, stream=side):
            fn(torch.cuda.current_stream())
        stream.wait_stream(side)
        return g

    steps_per_cycle = R // 4
    mm_graphs = [capture(lambda s, i=i: [mmvq(4 * i + T - 1, T, s) for T in (1, 2, 3, 4)])
                 for i in range(steps_per_cycle)]
    dec_graphs = [capture(lambda s, b=b: moe_decode(b, s)) for b in banks]

    def step(i, ev=None):
        if ev:
            ev[0].record(stream)
        mm_graphs[i % steps_per_cycle].replay()
        if ev:
            ev[1].record(stream)
        dequant(stream)
        if ev:
            ev[2].record(stream)
        dec_graphs[i % N_BANKS].replay()
        if ev:
            ev[3].record(stream)
        moe_prefill(stream)
        if ev:
            ev[4].record(stream)
        dense(stream)
        if ev:
            ev[5].record(stream)

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps ---------------------------------------------------
    log(f"timing {args.steps} steps")
    evs = [[Ev() for _ in range(6)] for _ in range(args.steps)]
    start, end = Ev(), Ev()
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(i, evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    comp = {name: sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)) / args.steps
            for j, name in enumerate(("mmvq_4_calls", "dequant", "moe_decode", "moe_prefill", "dense"))}

    # ---- per-launch matvec durations: graphs of R launches per T, cold weights ----------
    # Clocks ramp over ~100 ms, so the graphs are first replayed for >= 200 ms; then 5
    # rounds, each replaying every T's graph in turn (interleaved), and the median per T.
    mm_T = {T: capture(lambda s, T=T: [mmvq(c, T, s) for c in range(R)]) for T in (1, 2, 3, 4)}
    hot_T = {T: capture(lambda s, T=T: [mmvq(0, T, s) for _ in range(R)]) for T in (1, 2, 3, 4)}
    t_end = time.perf_counter() + 0.2
    while time.perf_counter() < t_end:
        for g in mm_T.values():
            g.replay()
        torch.cuda.synchronize()

    def replay_ms(g, launches, reps=2):
        a, b = Ev(), Ev()
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (reps * launches)

    ROUNDS = 5
    rounds_T = {T: [] for T in mm_T}
    rounds_hot = {T: [] for T in hot_T}
    for _ in range(ROUNDS):
        for T in (1, 2, 3, 4):
            rounds_T[T].append(replay_ms(mm_T[T], R))
            rounds_hot[T].append(replay_ms(hot_T[T], R))
    per_T = {T: statistics.median(v) for T, v in rounds_T.items()}  # ms per launch
    per_T_hot = {T: statistics.median(v) for T, v in rounds_hot.items()}
    spread_T = {T: [round(min(v) * 1e3, 3), round(max(v) * 1e3, 3)] for T, v in rounds_T.items()}
    del mm_T, hot_T

    # ---- measured ceilings: a plain streaming read of the matvec's weight bytes (graphs
    # of R launches over the same cold copies, the fastest of a few launch shapes), and a
    # pure matrix-core loop (f16 16 x 16 x 32, two waves per SIMD, every CU) ---------------
    ceil = ctypes.CDLL(os.path.join(ROOT, "dequant_matmul_iq4_amd", "libiq4_ceilings.so"))
    ceil.iq4c_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p]
    ceil.iq4c_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    stream_best = None
    for nv in (1, 2, 4):
        grid = (wb // 16 + 256 * nv - 1) // (256 * nv)
        g = capture(lambda s, nv=nv, grid=grid: [ceil.iq4c_stream_read(vcopies[c].data_ptr(), wb // 16 * 16, nv, grid,
                                                                        sink.data_ptr(), s) for c in range(R)])
        g.replay()
        ms = statistics.median([replay_ms(g, R) for _ in range(ROUNDS)])
        stream_best = ms if stream_best is None else min(stream_best, ms)
    mfma_iters, mfma_grid = 4096, 512
    g = capture(lambda s: [ceil.iq4c_mfma_loop(mfma_iters, mfma_grid, sink.data_ptr(), s) for _ in range(4)])
    g.replay()
    mfma_ms = statistics.median([replay_ms(g, 4) for _ in range(ROUNDS)])
    mfma_ceiling_tfs = mfma_grid * 4 * mfma_iters * 8 * 16384 / (mfma_ms * 1e-3) / 1e12
    stream_ceiling_gbs = (wb // 16 * 16) / (stream_best * 1e-3) / 1e9
    del g

    # ---- the same for the 8-bit-activation matvec, and its activation quantisation -----
    def per_launch_ms(fn, launches):
        g = capture(fn)
        g.replay()
        torch.cuda.synchronize()
        a, b = Ev(), Ev()
        reps = 4
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (reps * launches)

    per_T_q8 = {T: per_launch_ms(lambda s, T=T: [mmvq_q8(c, T, s) for c in range(R)], R) for T in (1, 2, 3, 4)}
    quant_ms = per_launch_ms(lambda s: [quantize_q8(s) for _ in range(R)], R)
    # the block decode per launch, as the matvec: a graph of launches back to back over
    # 32 copies of the blocks (302 MB, past the 256 MB Infinity Cache)
    deq_copies = [vblocks] + [vblocks.clone() for _ in range(31)]
    deq_ms = per_launch_ms(lambda s: [iq4.iq4_dequant_blocks(c, n * k // 32, iq4.IQ4_F16, deq_out, s)
                                      for c in deq_copies], len(deq_copies))
    del deq_copies
    # ---- IQ4_XS super-block matvec on page 2's two shapes, cold (rotating copies past
    # twice the Infinity Cache), medians of 5 interleaved rounds; weights are random
    # valid super-blocks (uniform bytes, binary16 scales of the workload's magnitude):
    # the kernel's time does not depend on the values ----------------------------------
    log("IQ4_XS matvec")
    xs_gen = torch.Generator(device="cuda")
    xs_gen.manual_seed(synth.SEED_XS_Z)
    xs_T, xs_bytes, xs_deq_ms = {}, {}, None
    for name, (xn, xk) in (("6144x2560", (6144, 2560)), ("2560x6144", (2560, 6144))):
        xb = iq4.iq4_xs_bytes(xn, xk)
        nsb = xb // 136
        base = torch.randint(0, 256, (xb,), dtype=torch.uint8, device="cuda", generator=xs_gen)
        dsc = (torch.randn(nsb, device="cuda", generator=xs_gen) * 2e-4).half()
        base.view(nsb, 136)[:, 0:2] = dsc.view(torch.uint8).view(nsb, 2)
        n_copies = (2 * (256 << 20)) // xb + 1
        xs_copies = [base] + [base.clone() for _ in range(n_copies - 1)]
        xs_x = synth.acts_f32_torch(synth.SEED_XS_Z, synth.TAG_X, 4, xk, device="cuda")
        xs_y = torch.empty((4, xn), dtype=torch.float32, device="cuda")
        gs = {T: capture(lambda s, T=T: [iq4.iq4_xs_qmv_multi(c, xn, xk, xs_x, xk, T, xs_y, xn, s)
                                         for c in xs_copies]) for T in (1, 2, 3, 4)}
        t_end = time.perf_counter() + 0.1
        while time.perf_counter() < t_end:
            for g in gs.values():
                g.replay()
            torch.cuda.synchronize()
        rounds = {T: [] for T in gs}
        for _ in range(ROUNDS):
            for T in gs:
                rounds[T].append(replay_ms(gs[T], n_copies))
        xs_T[name] = {T: statistics.median(v) for T, v in rounds.items()}
        xs_bytes[name] = (xb, xn, xk)
        if name == "6144x2560":
            xs_out = torch.empty(nsb * 256, dtype=torch.float16, device="cuda")
            xs_deq_ms = per_launch_ms(lambda s: [iq4.iq4_xs_dequant(c, nsb, iq4.IQ4_F16, xs_out, s)
                                                 for c in xs_copies], n_copies)
            xs_deq_bytes = xb + nsb * 256 * 2
            del xs_out
        del gs, xs_copies, base
    xs_alg = sum(xb + 4 * T * (xn + xk) for xb, xn, xk in xs_bytes.values() for T in (1, 2, 3, 4))
    xs_achieved = xs_alg / (sum(sum(v.values()) for v in xs_T.values()) * 1e-3) / 1e9
    q8_alg = sum(wb + T * k + T * (k // 32) * 2 + 4 * T * n for T in (1, 2, 3, 4))  # W + codes + scales + Y
    q8_achieved = q8_alg / (sum(per_T_q8.values()) * 1e-3) / 1e9
    # ---- MoE decode step device time: one graph of N_BANKS steps back to back, so a
    # step's figure holds no graph-launch gap (the per-step events above include one) ---
    dec_all = capture(lambda s: [moe_decode(b, s) for b in banks])
    dec_all.replay()
    torch.cuda.synchronize()
    a, b = Ev(), Ev()
    reps = 4
    a.record(stream)
    for _ in range(reps):
        dec_all.replay()
    b.record(stream)
    torch.cuda.synchronize()
    dec_ms = a.elapsed_time(b) / (reps * N_BANKS)
    # ---- beside the step: the same layer with a shared expert (its weights: expert 0 of
    # the bank four steps away, so they are as cold as the routed ones) ---------------
    sgb, sdb = iq4.iq4_packed_bytes(INTER, HIDDEN), iq4.iq4_packed_bytes(HIDDEN, INTER)

    def shared_of(i):
        g, u, d = banks[(i + N_BANKS // 2) % N_BANKS]
        return g[:sgb], u[:sgb], d[:sdb]
    ds_wsb = iq4.iq4_moe_shared_workspace_size(4, TOP_K, N_EXPERT, HIDDEN, INTER, iq4.IQ4_F32)
    ps_wsb = iq4.iq4_moe_shared_workspace_size(NP, TOP_K, N_EXPERT, HIDDEN, INTER, iq4.IQ4_F16)
    ds_ws = torch.empty(0 if args.no_shared else ds_wsb, dtype=torch.uint8, device="cuda")
    ps_ws = torch.empty(0 if args.no_shared else ps_wsb, dtype=torch.uint8, device="cuda")

    def moe_decode_shared(i, s):
        (g, u, d), (sg, su, sd) = banks[i], shared_of(i)
        iq4.iq4_moe_expert_gemm_shared(dx, iq4.IQ4_F32, 4, HIDDEN, d_ids, d_w, TOP_K, N_EXPERT, HIDDEN, INTER,
                                       g, u, d, sg, su, sd, d_out, HIDDEN, ds_ws, ds_wsb, 0, s)

    def moe_prefill_shared(s):
        (g, u, d), (sg, su, sd) = bank_a, shared_of(0)
        iq4.iq4_moe_expert_gemm_shared(px, iq4.IQ4_F16, NP, HIDDEN, p_ids, p_w, TOP_K, N_EXPERT, HIDDEN, INTER,
                                       g, u, d, sg, su, sd, p_out, HIDDEN, ps_ws, ps_wsb, 0, s)
    dec_shared_ms = pre_shared_ms = float("nan")
    if not args.no_shared:
        dec_shared_ms = per_launch_ms(lambda s: [moe_decode_shared(i, s) for i in range(N_BANKS)], N_BANKS)
        pre_shared_ms = per_launch_ms(lambda s: [moe_prefill_shared(s) for _ in range(2)], 2)
    del ps_ws
    tot_ms = sum(per_T.values())
    value = 4 * wb / (tot_ms * 1e-3) / 1e9
    mm_alg = sum(wb + 2 * 4 * T * k for T in (1, 2, 3, 4))  # weights + X + Y per four calls
    mm_achieved = mm_alg / (tot_ms * 1e-3) / 1e9

    prefill_flop = NP * TOP_K * 3 * 2 * HIDDEN * INTER  # 245,819,768,832
    dense_flop = 2 * LM * LN * LK
    unique_bytes = n_unique * 3 * iq4.iq4_packed_bytes(INTER, HIDDEN)
    deq_bytes = n * k // 32 * 18 + n * k * 2

    res = {
        "metric": "MMVQ effective weight GB/s at T=1..4; ms per 3,256-token MoE layer",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "verify-window MMVQ (W 4096x4096 IQ4, 18 B per 32 weights; fp32 X, T=1..4; "
                        f"{R} rotating weight copies) + IQ4 decode + MoE decode (4 tokens) + MoE prefill "
                        "(3256 tokens, Zipf 1.1, top-8 of 128, hidden 2048, inter 768) + long-prompt "
                        "projection (13056 x 4096 x 14336, 512-token chunks)",
            "mmvq_us_per_call": {str(T): round(per_T[T] * 1e3, 3) for T in per_T},
            "mmvq_us_per_call_min_max_of_5_rounds": {str(T): spread_T[T] for T in spread_T},
            "mmvq_weight_gbs_per_T": {str(T): round(wb / (per_T[T] * 1e-3) / 1e9, 1) for T in per_T},
            "mmvq_hot_us_per_call": {str(T): round(per_T_hot[T] * 1e3, 3) for T in per_T_hot},
            "timing": "HIP events around graph replays of 64 launches on the launch stream; >= 200 ms of "
                      "replays first (clock ramp); medians of 5 interleaved rounds; cold = 64 rotating weight "
                      "copies (604 MB, past the 256 MB Infinity Cache), hot = one copy",
            "measured_ceilings": {
                "stream_read_us_9.4MB": round(stream_best * 1e3, 3),
                "stream_read_gbs": round(stream_ceiling_gbs, 1),
                "mfma_f16_tflops": round(mfma_ceiling_tfs, 1),
                "how": "plain 16-byte grid-stride read of the matvec's weight bytes over the same cold copies "
                       "(best of 3 launch shapes); v_mfma_f32_16x16x32_f16 loop, 8 independent accumulators "
                       "per wave, 512 workgroups of 4 waves",
            },
            "moe_prefill_ms_per_layer": round(comp["moe_prefill"], 4),
            "moe_prefill_tflops": round(prefill_flop / (comp["moe_prefill"] * 1e-3) / 1e12, 2),
            "moe_decode_us_per_step": round(dec_ms * 1e3, 2),
            "moe_decode_us_in_step": round(comp["moe_decode"] * 1e3, 2),
            "moe_decode_unique_experts": n_unique,
            "moe_decode_shared_us_per_step": None if args.no_shared else round(dec_shared_ms * 1e3, 2),
            "moe_prefill_shared_ms_per_layer": None if args.no_shared else round(pre_shared_ms, 4),
            "moe_prefill_shared_tflops": None if args.no_shared else
            round(prefill_flop * (TOP_K + 1) / TOP_K / (pre_shared_ms * 1e-3) / 1e12, 2),
            "mmvq_q8_us_per_call": {str(T): round(per_T_q8[T] * 1e3, 3) for T in per_T_q8},
            "mmvq_q8_weight_gbs_per_T": {str(T): round(wb / (per_T_q8[T] * 1e-3) / 1e9, 1) for T in per_T_q8},
            "quantize_q8_us_4x4096": round(quant_ms * 1e3, 3),
            "dense_ms_26_chunks": round(comp["dense"], 4),
            "dense_tflops": round(dense_flop / (comp["dense"] * 1e-3) / 1e12, 2),
            "xs_mmvq_us_per_call": {nm: {str(T): round(v * 1e3, 3) for T, v in d.items()} for nm, d in xs_T.items()},
            "xs_mmvq_weight_gbs_per_T": {nm: {str(T): round(xs_bytes[nm][0] / (v * 1e-3) / 1e9, 1)
                                              for T, v in d.items()} for nm, d in xs_T.items()},
            "xs_dequant_us_6144x2560_f16": round(xs_deq_ms * 1e3, 2),
            "dequant_us": round(deq_ms * 1e3, 2),
            "dequant_us_in_step": round(comp["dequant"] * 1e3, 2),
            "prefill_expert_tokens_max_min": [int(counts.max()), int(counts.min())],
            "component_ms_per_step": {kk: round(v, 4) for kk, v in comp.items()},
        },
        "roofline": roof("hbm", mm_achieved, HBM_PEAK_GBS, "GB/s",
                         "qmv_dense_kernel: verify-window matvec, bytes = W + X + Y per call, "
                         "mean over T=1..4; traffic = HBM bytes per launch",
                         traffic=measured_traffic("qmv_dense_4096x4096_T1-4"),
                         ceiling=stream_ceiling_gbs),
        "rooflines": {
            "moe_prefill_layer": roof("mfma", prefill_flop / (comp["moe_prefill"] * 1e-3) / 1e12,
                                      F16_MFMA_PEAK_TFS, "TFLOP/s",
                                      "gather + qgemm<gateup> + qgemm<down> + combine, f16 MFMA; "
                                      "traffic = HBM bytes of the two GEMM launches",
                                      traffic=sum_traffic("qgemm_gateup_moe_prefill_3256tok",
                                                          "qgemm_down_moe_prefill_3256tok"),
                                      ceiling=mfma_ceiling_tfs),
            "dense_projection": roof("mfma", dense_flop / (comp["dense"] * 1e-3) / 1e12, F16_MFMA_PEAK_TFS,
                                     "TFLOP/s", "qgemm<dense> x 26 chunks; traffic = HBM bytes of the 26 launches",
                                     traffic=sum_traffic(*["qgemm_dense_13056x4096x14336_chunk512"] * 26),
                                     ceiling=mfma_ceiling_tfs),
            "moe_decode_step": roof("hbm", unique_bytes / (dec_ms * 1e-3) / 1e9, HBM_PEAK_GBS,
                                    "GB/s", f"qmv<gateup> + qmv_down_combine (down product and ordered "
                                    f"combine in one launch), {n_unique} unique experts' weights; traffic = "
                                    "HBM bytes of the two launches",
                                    traffic=sum_traffic("qmv_grouped_gateup_moe_decode_4tok",
                                                        "qmv_down_combine_moe_decode_4tok")),
            "mmvq_q8": roof("hbm", q8_achieved, HBM_PEAK_GBS, "GB/s",
                            "qmv_q8_kernel: verify-window matvec on 8-bit activations, bytes = W + codes + "
                            "scales + Y per call, mean over T=1..4; traffic = HBM bytes per launch",
                            traffic=measured_traffic("qmv_q8_4096x4096_T1-4")),
            "xs_mmvq": roof("hbm", xs_achieved, HBM_PEAK_GBS, "GB/s",
                            "xs_qmv_mfma_kernel: IQ4_XS super-block matvec on the matrix cores, 6144x2560 and "
                            "2560x6144, bytes = W + X + Y per call, mean over both shapes and T=1..4 (cold copies); "
                            "traffic = HBM bytes per launch, mean over both shapes",
                            traffic=mean_traffic("xs_qmv_mfma_6144x2560_T1-4", "xs_qmv_mfma_2560x6144_T1-4"),
                            ceiling=stream_ceiling_gbs),
            "xs_dequant": roof("hbm", xs_deq_bytes / (xs_deq_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s",
                               "xs_dequant_kernel<f16>: 8.4 MB of super-blocks in, 31.5 MB of f16 out per launch "
                               "(graph of launches over cold copies); traffic = HBM bytes per launch",
                               traffic=measured_traffic("xs_dequant_6144x2560_f16")),
            "dequant": roof("hbm", deq_bytes / (deq_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s",
                            "dequant_staged_kernel<f16>: 9.4 MB of blocks in, 33.5 MB of f16 out, per launch "
                            "(graph of 32 launches over cold copies); traffic = HBM bytes per launch",
                            traffic=measured_traffic("dequant_staged_4096x4096_f16")),
        },
    }
    if not args.no_cpu_baseline:
        log("cpu baselines (oracle, every config)")
        res["cpu_baseline"], res["cpu_baselines"] = cpu_baselines()
    print(json.dumps(res))


if __name__ == "__main__":
    main()
