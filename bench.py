"""Benchmark of the fused all-reduce epilogue hot path on one MI355X.

Prints ONE JSON line.  Headline (`value`): GEMM + reduce-scatter epilogue on
the tp=4 share -- X [4096,2048] . W [2048,4096] bf16, R=4, owner segment of 1024
rows, three peer partials landed per 128x128 flag tile by an emulated-peer
producer on a second stream in shuffled order, their ready bits published
eight tiles per release -- as TFLOP/s of the whole step (2*M*N*K per step).
The same step with one release per tile is reported beside it.  Inputs are
resident in HBM before timing starts.

Also reported in the same run: the Lamport AR+RMSNorm consumer (8 x
[4096,7168]) and the weighted top-8 combine ([4096,8,7168]) as GB/s of
algorithmic bytes, each against the 8 TB/s HBM peak; the pre-staged tp=4
kernel; the push-ring form of the same GEMM (one hop: the producer landing the
upstream partials beside it, and pre-staged); the fp8 block-scaled form
(pre-staged, against the fp8 peak); the two-phase Lamport call; with --sweep
the tp=8 sweep (M = 256..8192, N=7168, K=2048) in the bf16 forms.

`cpu_baseline` times the CPU oracle (oracle/, test infrastructure) on a
bounded row sample of the headline workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--sweep] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published

LAMPORT_BYTES = 998_258_688 + 7168 * 2   # read 8P + write P + re-arm 8P (+ gamma)
LAMPORT_BYTES_NO_REARM = 528_482_304 + 7168 * 2
COMBINE_BYTES = 528_613_376              # read x + gate + write out
# The emulated peers publish their tiles' ready bits eight tiles per release.
# On one GPU an agent-scope release writes back the L2 of the XCD it runs on --
# the L2 the GEMM is using -- which a remote peer's release never does to this
# GPU; one release per tile costs the step ~17 us of that artifact.  The step
# with one release per tile is reported beside the headline.
PRODUCER_TILES_PER_RELEASE = 8

_side_stream = None


def side_stream(torch):
    """One second stream for every leg: streams share a few hardware queues,
    and a fresh stream per leg can land on the main stream's queue."""
    global _side_stream
    if _side_stream is None:
        _side_stream = torch.cuda.Stream()
    return _side_stream
# two-phase Lamport, one rank's call at [4096,7168]: phase A reads P and stores
# P (its part into 8 stagings), phase B reads P, re-arms P, writes out P (+gamma)
LAMPORT2_BYTES = 5 * 58_720_256 + 7168 * 2


class _HipEvents:
    """HIP events created with a flag torch does not expose: no system-scope
    fence when the record completes.  A default record costs several
    microseconds of cache writeback and invalidation on the measured path; the
    work these events order stays on this GPU, and each kernel already ends
    with a device-scope release of its own writes."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, flags):
        e = self.ct.c_void_p()
        if self.lib.hipEventCreateWithFlags(self.ct.byref(e), flags) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e

    def record(self, e, stream):
        if self.lib.hipEventRecord(e, self.ct.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def wait(self, stream, e):
        if self.lib.hipStreamWaitEvent(self.ct.c_void_p(stream.cuda_stream), e, 0) != 0:
            raise RuntimeError("hipStreamWaitEvent failed")

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        if self.lib.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, events):
        for e in events:
            self.lib.hipEventDestroy(e)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sweep", action="store_true", help="also time the tp=8 sweep and the pre-staged tp=4 kernel")
    ap.add_argument("--only", default=None, choices=[None, "gemm_rs", "gemm_rs_prestaged", "gemm_rs_ring",
                                                   "gemm_rs_ring_prestaged", "gemm_rs_fp8", "lamport", "lamport_2phase",
                                                   "combine"],
                    help="run a single path (used for per-kernel profiles; counter collection serializes "
                         "kernels, so the GEMM's counters are taken pre-staged, without the producer stream)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    return ap.parse_args()


def gemm_rs_concurrent(A, inputs, torch, steps, warmup, ring=False, producer_wgs=0, per_release=1):
    """tp=4 share; a producer stream lands the peers while the GEMM runs
    (ring=True: the push-ring hop, the producer landing the upstream partials).

    The main stream runs only the GEMMs, back to back.  Each consumes its
    ready_in bits (the owner tiles clear what they waited for), so ready_in is
    zero again when it ends and needs no clearing kernel.  The producer of step
    i, on the side stream, waits for GEMM i-1 to end (it reuses recv and
    ready_in) and then runs while GEMM i does; GEMM i's owner tiles wait for
    its bits.  ready_out is only ever OR-ed into.  The producer's waves share
    CUs with the GEMM's (the chosen tile leaves registers for them).

    Returns the wall time per step and the GEMM's average launch duration from
    HIP events recorded on its stream just before and after each launch.
    """
    dev = torch.device("cuda:0")
    if ring:  # push-ring hop: upstream partials of every segment but the chain one
        case = inputs.gemm_rs_ring_case(**dict(inputs.WORKLOADS[2], M=4096), seed=1002)
    else:
        case = inputs.workload_gemm_rs(2)
    M, N, K, R, owner = case["M"], case["N"], case["K"], case["R"], case["owner"]
    seg = M // R
    # segment whose partial does not arrive: the owner's own (direct sum) or
    # the one this rank starts (ring)
    absent = (owner + R - 1) % R if ring else owner
    parts = case["up"] if ring else case["recv"]

    def up(a):
        return torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)

    x, w = up(case["x"]), up(case["w"])
    src = [None if p == absent else up(parts[p]) for p in range(R)]
    recv = [None if p == absent else torch.zeros_like(src[p]) for p in range(R)]
    words = A.gemm_rs_flag_words(M, N, R)
    tiles = ((seg + 127) // 128) * ((N + 127) // 128)
    orders = [torch.from_numpy(inputs.producer_order(R, absent, tiles, 2000 + i)).to(dev) for i in range(4)]
    rin = torch.zeros((R, words), dtype=torch.int32, device=dev)
    rout = torch.zeros((R, words), dtype=torch.int32, device=dev)
    out = torch.empty((seg, N), dtype=torch.bfloat16, device=dev)
    send = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    main = torch.cuda.current_stream()
    side = side_stream(torch)
    tile = A.gemm_rs_pick_tile(M, N, K, R, owner, publish=True)
    n_ev = steps + warmup
    H = _HipEvents()
    ev_gs = [H.create(H.DISABLE_SYSTEM_FENCE) for _ in range(n_ev)]
    ev_ge = [H.create(H.DISABLE_SYSTEM_FENCE) for _ in range(n_ev)]

    def step(i):
        if i > 0:
            H.wait(side, ev_ge[i - 1])
        A.emu_peer_producer(src, recv, rin, orders[i % len(orders)], R, absent, M, N, workgroups=producer_wgs,
                            items_per_release=per_release, stream=side)
        H.record(ev_gs[i], main)
        if ring:
            A.gemm_rs_ring(x, w, recv, rin, out, send, R, owner, ready_out=rout,
                           tile=tile | A.TILE_CONSUME_READY, status=status, stream=main)
        else:
            A.gemm_rs_fused(x, w, recv, rin, out, R, owner, send=send, ready_out=rout,
                            tile=tile | A.TILE_CONSUME_READY, status=status, stream=main)
        H.record(ev_ge[i], main)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(warmup, warmup + steps):
        step(i)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    gemm_ms = sum(H.elapsed_ms(ev_gs[i], ev_ge[i]) for i in range(warmup, warmup + steps)) / steps
    H.destroy(ev_gs + ev_ge)
    if int(status.item()) != 0:
        raise RuntimeError("a readiness wait timed out during the benchmark")
    flops = 2.0 * M * N * K
    return dict(ms_per_step=wall * 1e3, tflops=flops / wall / 1e12, gemm_ms=gemm_ms,
                gemm_tflops=flops / (gemm_ms * 1e-3) / 1e12, tile=A.TILE_NAMES[tile], flops=flops,
                M=M, N=N, K=K, R=R)


def gemm_rs_prestaged(A, inputs, torch, steps, warmup, num, M=None, ring=False):
    """GEMM + reduce-scatter epilogue with every partial landed beforehand (all
    ready bits set): the kernel alone.  ring=True times the push-ring hop."""
    dev = torch.device("cuda:0")
    if ring:
        spec = dict(inputs.WORKLOADS[num])
        if M is not None:
            spec["M"] = M
        case = inputs.gemm_rs_ring_case(seed=1000 + num, **spec)
    else:
        case = inputs.workload_gemm_rs(num, M=M)
    M, N, K, R, owner = case["M"], case["N"], case["K"], case["R"], case["owner"]
    seg = M // R
    absent = (owner + R - 1) % R if ring else owner
    parts = case["up"] if ring else case["recv"]

    def up(a):
        return torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)

    x, w = up(case["x"]), up(case["w"])
    recv = [None if p == absent else up(parts[p]) for p in range(R)]
    words = A.gemm_rs_flag_words(M, N, R)
    tiles = ((seg + 127) // 128) * ((N + 127) // 128)
    import numpy as np
    full = np.zeros((R, words), np.uint32)
    for p in range(R):
        if p != absent:
            for t in range(tiles):
                full[p, t // 32] |= np.uint32(1 << (t % 32))
    rin = torch.from_numpy(full.view(np.int32)).to(dev)
    rout = torch.zeros((R, words), dtype=torch.int32, device=dev)
    out = torch.empty((seg, N), dtype=torch.bfloat16, device=dev)
    send = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    tile = A.gemm_rs_pick_tile(M, N, K, R, owner, publish=True)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def call():
        if ring:
            A.gemm_rs_ring(x, w, recv, rin, out, send, R, owner, ready_out=rout, tile=tile)
        else:
            A.gemm_rs_fused(x, w, recv, rin, out, R, owner, send=send, ready_out=rout, tile=tile)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    s.record()
    for _ in range(steps):
        call()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    flops = 2.0 * M * N * K
    byts = 2.0 * (M * K + K * N + (R - 1) * seg * N + seg * N + (M - seg) * N)
    return dict(M=M, N=N, K=K, R=R, tile=A.TILE_NAMES[tile], ms=ms, tflops=flops / ms / 1e9,
                frac_mfma=flops / ms / 1e9 / PEAK_BF16_TFLOPS, gbs=byts / ms / 1e6,
                frac_hbm=byts / ms / 1e6 / PEAK_HBM_GBS)


def lamport(A, inputs, torch, steps, warmup):
    dev = torch.device("cuda:0")
    case = inputs.lamport_case()
    S, M, N = case["S"], case["M"], case["N"]
    src = torch.from_numpy(case["src"].view("int16")).view(torch.bfloat16).to(dev)
    gamma = torch.from_numpy(case["gamma"].view("int16")).view(torch.bfloat16).to(dev)
    order = torch.from_numpy(case["order"]).to(dev)
    st = torch.empty((S, M, N), dtype=torch.bfloat16, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    A.lamport_prefill(st)   # arming: once, before any timing
    main = torch.cuda.current_stream()
    side = side_stream(torch)
    n = steps + warmup
    # fence-free HIP events on the consumer's stream, as for the GEMM
    H = _HipEvents()
    es = [H.create(H.DISABLE_SYSTEM_FENCE) for _ in range(n)]
    ee = [H.create(H.DISABLE_SYSTEM_FENCE) for _ in range(n)]
    for i in range(n):
        side.wait_stream(main)   # publish only into re-armed staging
        A.lamport_publish(src, st, order, stream=side)
        main.wait_stream(side)
        H.record(es[i], main)
        A.ar_rmsnorm_lamport(st, gamma, out, case["eps"], status=status, stream=main)
        H.record(ee[i], main)
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError("Lamport consumer timed out")
    ms = sum(H.elapsed_ms(es[i], ee[i]) for i in range(warmup, n)) / steps
    H.destroy(es + ee)
    return dict(ms=ms, gbs=LAMPORT_BYTES / ms / 1e6, frac_hbm=LAMPORT_BYTES / ms / 1e6 / PEAK_HBM_GBS,
                gbs_no_rearm_bytes=LAMPORT_BYTES_NO_REARM / ms / 1e6, S=S, M=M, N=N)


def gemm_rs_fp8_prestaged(A, inputs, torch, steps, warmup):
    """fp8 e4m3fn block-scaled GEMM + reduce-scatter epilogue on the tp=4 share
    (X [4096,2048], W^T [4096,2048], 1x128 / 128x128 fp32 scales, R=4), peer
    partials landed beforehand: the kernel alone."""
    import numpy as np
    dev = torch.device("cuda:0")
    M, N, K, R, owner = 4096, 4096, 2048, 4, 0
    case = inputs.gemm_rs_fp8_case(M, N, K, R, owner=owner, seed=1002)
    seg = M // R
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x, wt, xs, ws = u8(case["x"]), u8(case["wt"]), u8(case["xs"]), u8(case["ws"])
    recv = [None if q == owner else torch.from_numpy(case["recv"][q].view("int16")).view(torch.bfloat16).to(dev)
            for q in range(R)]
    words = A.gemm_rs_flag_words(M, N, R)
    tiles = ((seg + 127) // 128) * ((N + 127) // 128)
    full = np.zeros((R, words), np.uint32)
    for q in range(R):
        if q != owner:
            for t in range(tiles):
                full[q, t // 32] |= np.uint32(1 << (t % 32))
    rin = torch.from_numpy(full.view(np.int32)).to(dev)
    rout = torch.zeros((R, words), dtype=torch.int32, device=dev)
    out = torch.empty((seg, N), dtype=torch.bfloat16, device=dev)
    send = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def call():
        A.gemm_rs_fp8(x, xs, wt, ws, recv, rin, out, R, owner, send=send, ready_out=rout)

    for _ in range(warmup):
        call()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(steps):
        call()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    flops = 2.0 * M * N * K
    byts = M * K + N * K + 4.0 * (M + N // 128) * (K // 128) + 2.0 * ((R - 1) * seg * N + seg * N + (M - seg) * N)
    return dict(M=M, N=N, K=K, R=R, tile="256x256", ms=ms, tflops=flops / ms / 1e9,
                frac_mfma_fp8=flops / ms / 1e9 / PEAK_FP8_TFLOPS, gbs=byts / ms / 1e6,
                frac_hbm=byts / ms / 1e6 / PEAK_HBM_GBS)


def lamport_2phase(A, inputs, torch, steps, warmup):
    """Two-phase Lamport AR + RMSNorm on rank 0 of 8, [4096,7168]: the seven
    peers' phase A is emulated on a side stream after the previous call has
    re-armed (their stores then wait in rank 0's staging); only the call itself
    is timed: phase A of its own part (read P, store P across the 8 stagings)
    and phase B (read P, re-arm P, write out P)."""
    dev = torch.device("cuda:0")
    case = inputs.lamport_case()
    R, M, N = case["S"], case["M"], case["N"]
    ins = [torch.from_numpy(case["src"][r].view("int16")).view(torch.bfloat16).to(dev) for r in range(R)]
    gamma = torch.from_numpy(case["gamma"].view("int16")).view(torch.bfloat16).to(dev)
    stg = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    for t in stg:
        A.lamport_prefill(t)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    main = torch.cuda.current_stream()
    side = side_stream(torch)
    n = steps + warmup
    # fence-free HIP events on the consumer's stream, as for the GEMM
    H = _HipEvents()
    es = [H.create(H.DISABLE_SYSTEM_FENCE) for _ in range(n)]
    ee = [H.create(H.DISABLE_SYSTEM_FENCE) for _ in range(n)]
    for i in range(n):
        side.wait_stream(main)
        for d in range(1, R):
            A.emu_lamport_phase_a(ins, stg, d, stream=side)
        main.wait_stream(side)
        H.record(es[i], main)
        A.ar_rmsnorm_lamport_2phase(ins, stg, gamma, out, 0, case["eps"], status=status, stream=main)
        H.record(ee[i], main)
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError("two-phase Lamport call timed out")
    ms = sum(H.elapsed_ms(es[i], ee[i]) for i in range(warmup, n)) / steps
    H.destroy(es + ee)
    return dict(ms=ms, gbs=LAMPORT2_BYTES / ms / 1e6, frac_hbm=LAMPORT2_BYTES / ms / 1e6 / PEAK_HBM_GBS,
                R=R, M=M, N=N)


def combine(A, inputs, torch, steps, warmup):
    dev = torch.device("cuda:0")
    case = inputs.combine_case()
    x = torch.from_numpy(case["x"].view("int16")).view(torch.bfloat16).to(dev)
    gate = torch.from_numpy(case["gate"]).to(dev)
    out = torch.empty((case["T"], case["H"]), dtype=torch.bfloat16, device=dev)
    for _ in range(warmup):
        A.combine_reduce(x, gate, out)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(steps):
        A.combine_reduce(x, gate, out)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    return dict(ms=ms, gbs=COMBINE_BYTES / ms / 1e6, frac_hbm=COMBINE_BYTES / ms / 1e6 / PEAK_HBM_GBS,
                T=case["T"], E=case["E"], H=case["H"])


def cpu_baseline(inputs, budget_s=10.0):
    """The CPU oracle (oracle/, test infrastructure) on the headline workload.

    Row bands of the tp=4 GEMM-RS share are run back to back, wrapping around
    the 4096 rows, until about `budget_s` seconds of wall time on all host
    threads have been spent; the rate is FLOPs of the rows done / time."""
    import oracle
    case = inputs.workload_gemm_rs(2)
    M, N, K, R = case["M"], case["N"], case["K"], case["R"]
    oracle.gemm_rs(case["x"], case["w"], case["recv"], R, case["owner"], rows=(0, 16))   # load + warm
    rows, t_used, r0, band = 0, 0.0, 0, 64
    while t_used < budget_s:
        r1 = min(M, r0 + band)
        t = time.perf_counter()
        oracle.gemm_rs(case["x"], case["w"], case["recv"], R, case["owner"], rows=(r0, r1))
        dt = time.perf_counter() - t
        t_used += dt
        rows += r1 - r0
        # next band sized for ~1 s so the budget is not overshot by much
        band = max(16, min(M, int((r1 - r0) / max(dt, 1e-3))))
        r0 = 0 if r1 == M else r1
    flops = 2.0 * rows * N * K
    return {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%d rows (%.2f passes over the %d rows) of the tp=4 GEMM-RS share, %.1f s wall, %s" % (
                rows, rows / M, M, t_used, platform.processor() or platform.machine())}


COUNTERS_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "gemm_rs_tp4_counters.txt")
# the kernel body and the direct-form entry (the counters go stale when either changes)
KERNEL_SOURCES = [os.path.join(os.path.dirname(os.path.abspath(__file__)), "all_reduce_epilogues_amd", "csrc", f)
                  for f in ("gemm_rs_impl.h", "gemm_rs.hip")]


def kernel_source_digest():
    import hashlib
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(tile):
    """HBM-side bytes per launch of the GEMM kernel from the stored rocprofv3
    FETCH_SIZE / WRITE_SIZE passes (scaled by the copy-kernel calibration), or
    None when the kernel source or the tile has changed since they were taken."""
    try:
        with open(COUNTERS_FILE) as f:
            rec = dict(line.split(": ", 1) for line in f.read().splitlines()
                       if line and not line.startswith("#") and ": " in line)
        digest = kernel_source_digest()
    except OSError:
        return None
    if rec.get("source_sha256", "").strip() != digest or rec.get("tile", "").strip() != tile:
        return None
    return int(rec["bytes_per_launch"])


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py measures one GPU only (this path has no multi-GPU run); got --gpus %d" % a.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    import all_reduce_epilogues_amd as A
    from all_reduce_epilogues_amd import inputs
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs the MI355X GPU")
    A.lib()
    secondary = {}
    head = None
    if a.only in (None, "gemm_rs"):
        head = gemm_rs_concurrent(A, inputs, torch, a.steps, a.warmup, per_release=PRODUCER_TILES_PER_RELEASE)
        r1 = gemm_rs_concurrent(A, inputs, torch, a.steps, a.warmup, per_release=1)
        secondary["gemm_rs_tp4_step_one_release_per_tile"] = dict(
            ms_per_step=r1["ms_per_step"], tflops=r1["tflops"], kernel_ms=r1["gemm_ms"],
            frac_mfma=r1["gemm_tflops"] / PEAK_BF16_TFLOPS)
    if a.only in (None, "gemm_rs_ring"):
        r = gemm_rs_concurrent(A, inputs, torch, a.steps, a.warmup, ring=True, per_release=PRODUCER_TILES_PER_RELEASE)
        secondary["gemm_rs_ring_tp4_step"] = dict(ms_per_step=r["ms_per_step"], tflops=r["tflops"],
                                                  kernel_ms=r["gemm_ms"], kernel_tflops=r["gemm_tflops"],
                                                  frac_mfma=r["gemm_tflops"] / PEAK_BF16_TFLOPS, tile=r["tile"])
    if a.only in (None, "lamport"):
        secondary["lamport_ar_rmsnorm"] = lamport(A, inputs, torch, max(10, a.steps // 2), 3)
    if a.only in (None, "combine"):
        secondary["combine_reduce"] = combine(A, inputs, torch, max(10, a.steps // 2), 3)
    if a.only in (None, "lamport_2phase"):
        secondary["lamport_2phase_ar_rmsnorm"] = lamport_2phase(A, inputs, torch, max(10, a.steps // 2), 3)
    if a.only in (None, "gemm_rs", "gemm_rs_prestaged"):
        secondary["gemm_rs_tp4_prestaged"] = gemm_rs_prestaged(A, inputs, torch, a.steps, a.warmup, 2)
    if a.only in (None, "gemm_rs_fp8"):
        secondary["gemm_rs_fp8_tp4_prestaged"] = gemm_rs_fp8_prestaged(A, inputs, torch, a.steps, a.warmup)
    if a.only in (None, "gemm_rs_ring", "gemm_rs_ring_prestaged"):
        secondary["gemm_rs_ring_tp4_prestaged"] = gemm_rs_prestaged(A, inputs, torch, a.steps, a.warmup, 2,
                                                                    ring=True)
    if a.sweep:
        secondary["gemm_rs_tp8_sweep"] = [gemm_rs_prestaged(A, inputs, torch, a.steps, a.warmup, 3, M=m)
                                         for m in inputs.TP8_M_SWEEP]
        secondary["gemm_rs_ring_tp8_sweep"] = [gemm_rs_prestaged(A, inputs, torch, a.steps, a.warmup, 3, M=m,
                                                                 ring=True) for m in inputs.TP8_M_SWEEP]
    line = {
        "metric": "GEMM-RS TFLOP/s + % bf16 MFMA peak; combine/RMSNorm GB/s + % HBM peak",
        "value": head["tflops"] if head else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": head["ms_per_step"] if head else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gemm_rs tp4 share: X[4096,2048] x W[2048,4096] bf16, R=4, owner=0, "
                               "3 peer partials [1024,4096] landed per 128x128 flag tile by a producer "
                               "stream in shuffled order, their bits published 8 tiles per release; "
                               "send + ready_out published",
                   "M": 4096, "N": 4096, "K": 2048, "R": 4, "owner": 0,
                   "producer_tiles_per_release": PRODUCER_TILES_PER_RELEASE,
                   "tile": head["tile"] if head else None},
    }
    if head:
        achieved = head["flops"] / (head["gemm_ms"] * 1e-3) / 1e12
        line["roofline"] = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                            "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic(head["tile"]),
                            "kernel": "gemm_rs_kernel", "avg_kernel_ms": head["gemm_ms"]}
    line["secondary"] = secondary
    if not a.no_cpu and head:
        line["cpu_baseline"] = cpu_baseline(inputs)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
