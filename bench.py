"""Benchmark of the fused all-reduce epilogue hot path on one MI355X.

Prints ONE JSON line.  Headline (`value`): GEMM + reduce-scatter epilogue on
the tp=4 share -- X [4096,2048] . W [2048,4096] bf16, R=4, owner segment of 1024
rows, three peer partials landed per 128x128 flag tile by an emulated-peer
producer on a second stream in shuffled order, their ready bits published
eight tiles per release -- as TFLOP/s of the whole step (2*M*N*K per step).
One producer launch serves all the steps: a one-wave gate on the GEMM's
stream waits until every producer workgroup has started, then the GEMMs run
back to back, each step's tiles landing once the previous GEMM has ended.
The same step with one release per tile is reported beside it in `config`.
Inputs are resident in HBM before timing starts.

`secondary` holds every other workload, each timed launch by launch with HIP
events on the kernel's stream (median, min and p90 over --iters launches) and
carrying a `roofline` object (algorithmic work per launch over the median
launch time, against the MFMA or HBM peak) and, where the oracle has one, a
bounded `cpu_baseline`:
  gemm_rs_tiny          R=2, X[256,256], W[256,512] (launch-bound)
  gemm_rs_tp4_prestaged the headline's kernel with every partial landed
  gemm_plain_tp4        the same kernel with R=1 (the plain product), beside the library's
  gemm_rs_tp8_m{M}      R=8, X[M,2048], W[2048,7168], M = 256, 1024, 4096, 8192
  lamport_ar_rmsnorm    8 x [4096,7168] partials, RMSNorm over 7168
  combine_reduce        [4096,8,7168] top-8 weighted sum, register pipeline and
                        the LDS-staged pipeline
  lamport_2phase        rank 0 of 8 of the two-phase call at [4096,7168]
  gemm_rs_fp8_tp4       fp8 e4m3fn block-scaled GEMM-RS on the tp=4 share
  gemm_rs_ring_tp4      one push-ring hop: step with the producer, and pre-staged

`cpu_baseline` times the CPU oracle (oracle/, test infrastructure) on a
bounded row sample of the headline workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--iters I] [--sweep]
                       [--no-cpu] [--only LEG]
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

P_4096x7168 = 4096 * 7168 * 2                 # one [4096,7168] bf16 buffer
LAMPORT_BYTES = 17 * P_4096x7168 + 7168 * 2   # read 8P + write P + re-arm 8P (+ gamma)
LAMPORT_BYTES_NO_REARM = 9 * P_4096x7168 + 7168 * 2
COMBINE_BYTES = 8 * P_4096x7168 + 4096 * 8 * 4 + P_4096x7168   # read x + gate + write out
# two-phase Lamport, one rank's call at [4096,7168]: phase A reads P and stores
# P (its part into 8 stagings), phase B reads P, re-arms P, writes out P (+gamma)
LAMPORT2_BYTES = 5 * P_4096x7168 + 7168 * 2
# The emulated peers publish their tiles' ready bits eight tiles per release.
# On one GPU an agent-scope release writes back the L2 of the XCD it runs on --
# the L2 the GEMM is using -- which a remote peer's release never does to this
# GPU.  The step with one release per tile is reported beside the headline.
PRODUCER_TILES_PER_RELEASE = 8
# The producer lands its batches with 96 workgroups at a time (a link of
# bounded rate).  The gate between the producer and the GEMM waits until all
# of them have started, so a small persistent grid also keeps the gate short.
PRODUCER_WORKGROUPS = 96

LEGS = ("gemm_rs", "gemm_rs_tiny", "gemm_rs_prestaged", "gemm_plain", "gemm_rs_tp8", "lamport", "combine",
        "combine_lds", "lamport_2phase", "gemm_rs_fp8", "gemm_rs_ring", "gemm_rs_ring_prestaged")

_side_stream = None


def side_stream(torch):
    """The second stream of the legs whose emulated peers run before each
    timed call (Lamport, two-phase): an ordinary non-blocking stream, created
    once (streams share a few hardware queues, and a fresh one per leg can
    land on the main stream's queue)."""
    global _side_stream
    if _side_stream is None:
        _side_stream = torch.cuda.Stream()
    return _side_stream


def producer_stream(torch):
    """The stream of the producer that runs beside the GEMM: one with a
    hardware queue of its own (a producer that waits for the GEMM's signal
    must never sit in front of that GEMM in a shared queue).  It is a blocking
    stream, which the legacy default stream waits for, so those legs run
    their GEMMs on main_stream()."""
    import all_reduce_epilogues_amd as A
    return A.emu_stream()


_main_stream = None


def main_stream(torch):
    """A non-blocking stream for the consumer of the legs whose producer
    runs beside it (the legacy default stream would wait for the producer)."""
    global _main_stream
    if _main_stream is None:
        _main_stream = torch.cuda.Stream()
    return _main_stream


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

    def create(self, flags=DISABLE_SYSTEM_FENCE):
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


def stats(ms):
    """Median, min, p90 and mean of per-launch times (ms)."""
    s = sorted(ms)
    n = len(s)
    return dict(ms_median=s[n // 2], ms_min=s[0], ms_p90=s[min(n - 1, (9 * n) // 10)], ms_mean=sum(s) / n, iters=n)


def time_launches(torch, call, iters, warmup, before=None):
    """Times `call()` launch by launch with fence-free HIP events on the
    current stream; `before()` (untimed) runs ahead of every launch."""
    H = _HipEvents()
    main = torch.cuda.current_stream()
    n = iters + warmup
    es = [H.create() for _ in range(n)]
    ee = [H.create() for _ in range(n)]
    for i in range(n):
        if before is not None:
            before()
        H.record(es[i], main)
        call()
        H.record(ee[i], main)
    torch.cuda.synchronize()
    ms = [H.elapsed_ms(es[i], ee[i]) for i in range(warmup, n)]
    H.destroy(es + ee)
    return stats(ms)


def roofline(bound, work, st, peak, unit, traffic=None, kernel=None):
    """Roofline object: algorithmic work per launch over the median launch
    time (FLOP -> TFLOP/s, bytes -> GB/s), against `peak`."""
    t = st["ms_median"] * 1e-3
    achieved = work / t / (1e12 if unit == "TFLOP/s" else 1e9)
    r = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
         "traffic": traffic}
    if kernel:
        r["kernel"] = kernel
    return r


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="timed steps of the headline")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--iters", type=int, default=100, help="timed launches of every other workload")
    ap.add_argument("--sweep", action="store_true", help="also time the push-ring hop over the tp=8 sweep")
    ap.add_argument("--only", default=None, choices=[None, *LEGS],
                    help="run a single leg (used for per-kernel profiles; counter collection serializes "
                         "kernels, so the GEMM's counters are taken pre-staged, without the producer stream)")
    ap.add_argument("--m", type=int, default=None, help="with --only gemm_rs_tp8: one M of the sweep")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baselines")
    return ap.parse_args()


def _up(torch, a):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(a).view("int16")).view(torch.bfloat16).to(torch.device("cuda:0"))


def _ready_all(torch, R, absent, words, tiles):
    import numpy as np
    full = np.zeros((R, words), np.uint32)
    for p in range(R):
        if p != absent:
            for t in range(tiles):
                full[p, t // 32] |= np.uint32(1 << (t % 32))
    return torch.from_numpy(full.view(np.int32)).to(torch.device("cuda:0"))


def gemm_rs_concurrent(A, inputs, torch, steps, warmup, ring=False, producer_wgs=PRODUCER_WORKGROUPS,
                       per_release=1):
    """tp=4 share; a producer lands the peers while the GEMM runs (ring=True:
    the push-ring hop, the producer landing the upstream partials).

    One producer launch on the side stream serves all the steps of a phase
    (warm-up, then the timed steps): it is resident before the first GEMM (the
    one-wave gate on the main stream waits for all its workgroups to start),
    and step i's tiles start landing once the main stream has signalled that
    GEMM i-1 has ended (it reuses recv and ready_in); they land while GEMM i
    runs, whose owner tiles wait for their bits.  The main stream runs the
    GEMMs back to back with a one-thread signal kernel between them.  Each GEMM
    consumes its ready_in bits (the owner tiles clear what they waited for), so
    ready_in is zero again when it ends.  ready_out is only ever OR-ed into.

    Returns the wall time per step (the one producer launch and gate of the
    phase included) and the GEMM's launch durations from HIP events recorded
    on its stream just before and after each launch.
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
    x, w = _up(torch, case["x"]), _up(torch, case["w"])
    src = [None if p == absent else _up(torch, parts[p]) for p in range(R)]
    recv = [None if p == absent else torch.zeros_like(src[p]) for p in range(R)]
    words = A.gemm_rs_flag_words(M, N, R)
    tiles = ((seg + 127) // 128) * ((N + 127) // 128)
    import numpy as np
    orders = torch.from_numpy(np.stack([inputs.producer_order(R, absent, tiles, 2000 + i) for i in range(4)])).to(dev)
    rin = torch.zeros((R, words), dtype=torch.int32, device=dev)
    rout = torch.zeros((R, words), dtype=torch.int32, device=dev)
    out = torch.empty((seg, N), dtype=torch.bfloat16, device=dev)
    send = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    resident = torch.zeros(2, dtype=torch.int32, device=dev)
    go = torch.zeros(1, dtype=torch.int32, device=dev)
    main = main_stream(torch)
    side = producer_stream(torch)
    torch.cuda.synchronize()
    tile = (A.gemm_rs_ring_pick_tile if ring else A.gemm_rs_pick_tile)(M, N, K, R, owner, publish=True)
    n_ev = steps + warmup
    H = _HipEvents()
    ev_gs = [H.create() for _ in range(n_ev)]
    ev_ge = [H.create() for _ in range(n_ev)]

    def phase(first, n):
        with torch.cuda.stream(main):
            go.zero_()
        side.wait_stream(main)
        A.emu_peer_producer_steps(src, recv, rin, orders, R, absent, M, N, go, n, workgroups=producer_wgs,
                                  items_per_release=per_release, resident=resident, status=status, stream=side)
        A.emu_producer_gate(resident, status=status, stream=main)
        for s in range(n):
            i = first + s
            H.record(ev_gs[i], main)
            if ring:
                A.gemm_rs_ring(x, w, recv, rin, out, send, R, owner, ready_out=rout,
                               tile=tile | A.TILE_CONSUME_READY, status=status, stream=main)
            else:
                A.gemm_rs_fused(x, w, recv, rin, out, R, owner, send=send, ready_out=rout,
                                tile=tile | A.TILE_CONSUME_READY, status=status, stream=main)
            H.record(ev_ge[i], main)
            A.emu_signal(go, s + 1, stream=main)

    phase(0, warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    phase(warmup, steps)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    gemm = stats([H.elapsed_ms(ev_gs[i], ev_ge[i]) for i in range(warmup, warmup + steps)])
    H.destroy(ev_gs + ev_ge)
    if int(status.item()) != 0:
        raise RuntimeError("a readiness wait timed out during the benchmark")
    flops = 2.0 * M * N * K
    return dict(ms_per_step=wall * 1e3, tflops=flops / wall / 1e12, gemm=gemm, tile=A.TILE_NAMES[tile],
                flops=flops, M=M, N=N, K=K, R=R)


def gemm_rs_bytes(M, N, K, R):
    """Algorithmic bytes of one GEMM-RS call: X + W + (R-1) partials + out + send."""
    seg = M // R
    return 2.0 * (M * K + K * N + (R - 1) * seg * N + seg * N + (M - seg) * N)


def gemm_rs_prestaged(A, inputs, torch, iters, warmup, num, M=None, ring=False, counters=None):
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
    x, w = _up(torch, case["x"]), _up(torch, case["w"])
    recv = [None if p == absent else _up(torch, parts[p]) for p in range(R)]
    words = A.gemm_rs_flag_words(M, N, R)
    tiles = ((seg + 127) // 128) * ((N + 127) // 128)
    rin = _ready_all(torch, R, absent, words, tiles)
    rout = torch.zeros((R, words), dtype=torch.int32, device=dev)
    out = torch.empty((seg, N), dtype=torch.bfloat16, device=dev)
    send = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    tile = (A.gemm_rs_ring_pick_tile if ring else A.gemm_rs_pick_tile)(M, N, K, R, owner, publish=True)
    name = A.TILE_NAMES[tile]
    if not ring:
        # the direct form runs the automatic choice, which may also split the
        # owner rows into half-height tiles (row block -1 in the schedule)
        if any(wg[0] == -1 for wg in A.gemm_rs_schedule(M, N, K, R, owner, publish=True)):
            name += "+owner_half"

    def call():
        if ring:
            A.gemm_rs_ring(x, w, recv, rin, out, send, R, owner, ready_out=rout, tile=tile)
        else:
            A.gemm_rs_fused(x, w, recv, rin, out, R, owner, send=send, ready_out=rout, tile=A.TILE_AUTO)

    st = time_launches(torch, call, iters, warmup)
    flops = 2.0 * M * N * K
    byts = gemm_rs_bytes(M, N, K, R)
    t = st["ms_median"] * 1e-3
    # HBM-bound where the arithmetic intensity is below the ridge point
    hbm = flops / byts < (PEAK_BF16_TFLOPS * 1e12) / (PEAK_HBM_GBS * 1e9)
    traffic = measured_traffic(counters, name) if counters else None
    rf = (roofline("hbm", byts, st, PEAK_HBM_GBS, "GB/s", traffic, "gemm_rs_ring_kernel" if ring else "gemm_rs_kernel")
          if hbm else
          roofline("mfma", flops, st, PEAK_BF16_TFLOPS, "TFLOP/s", traffic,
                   "gemm_rs_ring_kernel" if ring else "gemm_rs_kernel"))
    res = dict(M=M, N=N, K=K, R=R, tile=name, **st, tflops=flops / t / 1e12,
               frac_mfma=flops / t / 1e12 / PEAK_BF16_TFLOPS, gbs=byts / t / 1e9,
               frac_hbm=byts / t / 1e9 / PEAK_HBM_GBS, roofline=rf)
    if not ring:
        res["library_gemm"] = library_gemm(torch, x, w, iters, warmup)
    return res


def gemm_plain(A, torch, iters, warmup, M=4096, N=4096, K=2048):
    """Context: the same kernel with R = 1 (no peers, no send: the plain
    product X.W into out) beside the library's plain product of the same
    shape, so the two mainloops compare directly."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(1010)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(dev)
    w = (torch.randn(K, N, generator=g) * 0.02).to(torch.bfloat16).to(dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    tile = A.gemm_rs_pick_tile(M, N, K, 1, 0)
    st = time_launches(torch, lambda: A.gemm_rs_fused(x, w, [None], None, out, 1, 0, tile=tile), iters, warmup)
    flops = 2.0 * M * N * K
    t = st["ms_median"] * 1e-3
    return dict(M=M, N=N, K=K, R=1, tile=A.TILE_NAMES[tile], **st, tflops=flops / t / 1e12,
                roofline=roofline("mfma", flops, st, PEAK_BF16_TFLOPS, "TFLOP/s", None, "gemm_rs_kernel"),
                library_gemm=library_gemm(torch, x, w, iters, warmup))


def library_gemm(torch, x, w, iters, warmup):
    """Context only: the plain product X.W of the same shape through
    torch.matmul (hipBLASLt), no reduce-scatter -- what a library GEMM alone
    takes on this GPU."""
    c = torch.empty((x.shape[0], w.shape[1]), dtype=torch.bfloat16, device=x.device)
    st = time_launches(torch, lambda: torch.matmul(x, w, out=c), iters, warmup)
    flops = 2.0 * x.shape[0] * x.shape[1] * w.shape[1]
    return dict(ms_median=st["ms_median"], ms_min=st["ms_min"], tflops=flops / (st["ms_median"] * 1e-3) / 1e12,
                note="torch.matmul (hipBLASLt) of X.W alone, same shape, no reduce-scatter epilogue")


def lamport(A, inputs, torch, iters, warmup, case):
    dev = torch.device("cuda:0")
    S, M, N = case["S"], case["M"], case["N"]
    src = _up(torch, case["src"])
    gamma = _up(torch, case["gamma"])
    order = torch.from_numpy(case["order"]).to(dev)
    st_buf = torch.empty((S, M, N), dtype=torch.bfloat16, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    A.lamport_prefill(st_buf)   # arming: once, before any timing
    main = torch.cuda.current_stream()
    side = side_stream(torch)

    def publish():   # the emulated peers land their partials into the re-armed staging (untimed)
        side.wait_stream(main)
        A.lamport_publish(src, st_buf, order, stream=side)
        main.wait_stream(side)

    st = time_launches(torch, lambda: A.ar_rmsnorm_lamport(st_buf, gamma, out, case["eps"], status=status),
                       iters, warmup, before=publish)
    if int(status.item()) != 0:
        raise RuntimeError("Lamport consumer timed out")
    t = st["ms_median"] * 1e-3
    return dict(**st, gbs=LAMPORT_BYTES / t / 1e9, frac_hbm=LAMPORT_BYTES / t / 1e9 / PEAK_HBM_GBS,
                gbs_no_rearm_bytes=LAMPORT_BYTES_NO_REARM / t / 1e9, S=S, M=M, N=N,
                roofline=roofline("hbm", LAMPORT_BYTES, st, PEAK_HBM_GBS, "GB/s",
                                  measured_traffic("lamport", "512x2"), "ar_rmsnorm_kernel"))


def gemm_rs_fp8_prestaged(A, inputs, torch, iters, warmup):
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
    recv = [None if q == owner else _up(torch, case["recv"][q]) for q in range(R)]
    words = A.gemm_rs_flag_words(M, N, R)
    rin = _ready_all(torch, R, owner, words, ((seg + 127) // 128) * ((N + 127) // 128))
    rout = torch.zeros((R, words), dtype=torch.int32, device=dev)
    out = torch.empty((seg, N), dtype=torch.bfloat16, device=dev)
    send = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    st = time_launches(torch, lambda: A.gemm_rs_fp8(x, xs, wt, ws, recv, rin, out, R, owner, send=send,
                                                    ready_out=rout), iters, warmup)
    flops = 2.0 * M * N * K
    byts = M * K + N * K + 4.0 * (M + N // 128) * (K // 128) + 2.0 * ((R - 1) * seg * N + seg * N + (M - seg) * N)
    t = st["ms_median"] * 1e-3
    return dict(M=M, N=N, K=K, R=R, tile="256x256", **st, tflops=flops / t / 1e12,
                frac_mfma_fp8=flops / t / 1e12 / PEAK_FP8_TFLOPS, gbs=byts / t / 1e9,
                frac_hbm=byts / t / 1e9 / PEAK_HBM_GBS,
                roofline=roofline("mfma", flops, st, PEAK_FP8_TFLOPS, "TFLOP/s",
                                  measured_traffic("gemm_rs_fp8", "256x256"), "gemm_rs_fp8_kernel"))


def lamport_2phase(A, inputs, torch, iters, warmup, case):
    """Two-phase Lamport AR + RMSNorm on rank 0 of 8, [4096,7168]: the seven
    peers' phase A is emulated on a side stream after the previous call has
    re-armed (their stores then wait in rank 0's staging); only the call itself
    is timed: phase A of its own part (read P, store P across the 8 stagings)
    and phase B (read P, re-arm P, write out P)."""
    dev = torch.device("cuda:0")
    R, M, N = case["S"], case["M"], case["N"]
    ins = [_up(torch, case["src"][r]) for r in range(R)]
    gamma = _up(torch, case["gamma"])
    stg = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    for t in stg:
        A.lamport_prefill(t)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    main = torch.cuda.current_stream()
    side = side_stream(torch)

    def peers():
        side.wait_stream(main)
        for d in range(1, R):
            A.emu_lamport_phase_a(ins, stg, d, stream=side)
        main.wait_stream(side)

    st = time_launches(torch, lambda: A.ar_rmsnorm_lamport_2phase(ins, stg, gamma, out, 0, case["eps"],
                                                                  status=status), iters, warmup, before=peers)
    if int(status.item()) != 0:
        raise RuntimeError("two-phase Lamport call timed out")
    t = st["ms_median"] * 1e-3
    return dict(**st, gbs=LAMPORT2_BYTES / t / 1e9, frac_hbm=LAMPORT2_BYTES / t / 1e9 / PEAK_HBM_GBS,
                R=R, M=M, N=N, roofline=roofline("hbm", LAMPORT2_BYTES, st, PEAK_HBM_GBS, "GB/s",
                                                 measured_traffic("lamport_2phase", "rank0of8"),
                                                 "lamport2_kernel"))


def combine(A, inputs, torch, iters, warmup, case, pipeline="registers"):
    dev = torch.device("cuda:0")
    x = _up(torch, case["x"])
    gate = torch.from_numpy(case["gate"]).to(dev)
    out = torch.empty((case["T"], case["H"]), dtype=torch.bfloat16, device=dev)
    st = time_launches(torch, lambda: A.combine_reduce(x, gate, out, pipeline=pipeline), iters, warmup)
    t = st["ms_median"] * 1e-3
    key = "combine" if pipeline == "registers" else "combine_lds"
    return dict(**st, gbs=COMBINE_BYTES / t / 1e9, frac_hbm=COMBINE_BYTES / t / 1e9 / PEAK_HBM_GBS,
                T=case["T"], E=case["E"], H=case["H"], pipeline=pipeline,
                roofline=roofline("hbm", COMBINE_BYTES, st, PEAK_HBM_GBS, "GB/s",
                                  measured_traffic(key, pipeline),
                                  "combine_regs_kernel" if pipeline == "registers" else "combine_kernel"))


# ---- CPU baselines: the oracle (test infrastructure) on bounded samples --------

def _cpu_note(what, done, total, unit_name, secs):
    return "%s: %d of %d %s, %.1f s wall, %s" % (what, done, total, unit_name, secs,
                                                   platform.processor() or platform.machine())


def cpu_baseline_gemm_rs(inputs, case, budget_s, what):
    """Row bands of a GEMM-RS case run back to back (wrapping around its M
    rows) until about `budget_s` of wall time; rate = FLOPs of the rows done /
    time (TFLOP/s)."""
    import oracle
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
            "sample": _cpu_note(what, rows, M, "rows (%.2f passes)" % (rows / M), t_used)}


def cpu_baseline_rows(fn, total, per_unit_bytes, budget_s, what, unit_name):
    """`fn((r0, r1))` over row/token bands until about `budget_s`; rate =
    algorithmic bytes of the units done / time (GB/s)."""
    import oracle
    fn((0, 1))
    done, t_used, r0, band = 0, 0.0, 0, 8
    while t_used < budget_s:
        r1 = min(total, r0 + band)
        t = time.perf_counter()
        fn((r0, r1))
        dt = time.perf_counter() - t
        t_used += dt
        done += r1 - r0
        band = max(1, min(total, int((r1 - r0) * 0.5 / max(dt, 1e-3))))
        r0 = 0 if r1 == total else r1
    return {"value": done * per_unit_bytes / t_used / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": _cpu_note(what, done, total, unit_name, t_used)}


# ---- stored HBM-traffic counters -------------------------------------------------

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "all_reduce_epilogues_amd", "csrc")
# counter record per workload: file under profiles/ and the kernel sources it was
# measured on (the record goes stale when one of them changes)
COUNTERS = {
    "gemm_rs_tp4": ("gemm_rs_tp4_counters.txt", ("gemm_rs_impl.h", "gemm_rs_kernel.h", "gemm_rs.hip")),
    "gemm_rs_tp8_m256": ("gemm_rs_tp8_m256_counters.txt",
                         ("gemm_rs_impl.h", "gemm_rs_kernel.h", "gemm_rs.hip", "gemm_rs_mixed.hip")),
    "gemm_rs_tp8_m8192": ("gemm_rs_tp8_m8192_counters.txt", ("gemm_rs_impl.h", "gemm_rs_kernel.h", "gemm_rs.hip")),
    "lamport": ("lamport_counters.txt", ("lamport.hip",)),
    "combine": ("combine_counters.txt", ("combine.hip",)),
    "combine_lds": ("combine_counters_lds.txt", ("combine.hip",)),
    "lamport_2phase": ("lamport_2phase_counters.txt", ("lamport.hip",)),
    "gemm_rs_fp8": ("gemm_rs_fp8_tp4_counters.txt", ("gemm_rs_impl.h", "gemm_rs_fp8.hip")),
}
COUNTERS_FILE = None   # (tests) one record file used for every key instead


def kernel_source_digest(key="gemm_rs_tp4"):
    import hashlib
    h = hashlib.sha256()
    for f in COUNTERS[key][1]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(key, tile):
    """HBM-side bytes per launch from the stored rocprofv3 FETCH_SIZE /
    WRITE_SIZE passes (scaled by the copy-kernel calibration), or None when
    there is no record, or the kernel sources or the launch shape (`tile`)
    have changed since it was taken."""
    path = COUNTERS_FILE or os.path.join(HERE, "profiles", COUNTERS[key][0])
    try:
        with open(path) as f:
            rec = dict(line.split(": ", 1) for line in f.read().splitlines()
                       if line and not line.startswith("#") and ": " in line)
        digest = kernel_source_digest(key)
    except (OSError, KeyError):
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
    run = lambda leg: a.only in (None, leg)
    secondary = {}
    head = r1 = None
    it, wu = a.iters, min(10, a.warmup if a.only else 10)
    if run("gemm_rs"):
        head = gemm_rs_concurrent(A, inputs, torch, a.steps, a.warmup, per_release=PRODUCER_TILES_PER_RELEASE)
        r1 = gemm_rs_concurrent(A, inputs, torch, a.steps, a.warmup, per_release=1)
    if run("gemm_rs_tiny"):
        secondary["gemm_rs_tiny"] = gemm_rs_prestaged(A, inputs, torch, it, wu, 1)
    if run("gemm_rs_prestaged") or run("gemm_rs"):
        secondary["gemm_rs_tp4_prestaged"] = gemm_rs_prestaged(A, inputs, torch, it, wu, 2, counters="gemm_rs_tp4")
    if run("gemm_plain"):
        secondary["gemm_plain_tp4"] = gemm_plain(A, torch, it, wu)
    if run("gemm_rs_tp8"):
        for m in ([a.m] if a.m else inputs.TP8_M_SWEEP):
            key = "gemm_rs_tp8_m%d" % m
            secondary[key] = gemm_rs_prestaged(A, inputs, torch, it, wu, 3, M=m,
                                               counters=key if key in COUNTERS else None)
    lam_case = None
    if run("lamport") or run("lamport_2phase"):
        lam_case = inputs.lamport_case()
    if run("lamport"):
        secondary["lamport_ar_rmsnorm"] = lamport(A, inputs, torch, it, wu, lam_case)
    comb_case = None
    if run("combine") or run("combine_lds"):
        comb_case = inputs.combine_case()
    if run("combine"):
        secondary["combine_reduce"] = combine(A, inputs, torch, it, wu, comb_case)
    if run("combine_lds"):
        secondary["combine_reduce_lds"] = combine(A, inputs, torch, it, wu, comb_case, pipeline="lds")
    if run("lamport_2phase"):
        secondary["lamport_2phase_ar_rmsnorm"] = lamport_2phase(A, inputs, torch, it, wu, lam_case)
    if run("gemm_rs_fp8"):
        secondary["gemm_rs_fp8_tp4_prestaged"] = gemm_rs_fp8_prestaged(A, inputs, torch, it, wu)
    if run("gemm_rs_ring"):
        r = gemm_rs_concurrent(A, inputs, torch, a.steps, a.warmup, ring=True, per_release=PRODUCER_TILES_PER_RELEASE)
        secondary["gemm_rs_ring_tp4_step"] = dict(ms_per_step=r["ms_per_step"], tflops=r["tflops"],
                                                  kernel=r["gemm"], tile=r["tile"])
    if run("gemm_rs_ring") or run("gemm_rs_ring_prestaged"):
        secondary["gemm_rs_ring_tp4_prestaged"] = gemm_rs_prestaged(A, inputs, torch, it, wu, 2, ring=True)
    if a.sweep:
        secondary["gemm_rs_ring_tp8_sweep"] = [gemm_rs_prestaged(A, inputs, torch, it, wu, 3, M=m, ring=True)
                                               for m in inputs.TP8_M_SWEEP]

    # CPU baselines (oracle, bounded samples of each workload; reported, never a target)
    cpu = None
    if not a.no_cpu:
        import oracle
        if head:
            cpu = cpu_baseline_gemm_rs(inputs, inputs.workload_gemm_rs(2), 10.0, "tp=4 GEMM-RS share")
        if "gemm_rs_tp8_m8192" in secondary:
            c8 = inputs.workload_gemm_rs(3, M=8192)
            base = cpu_baseline_gemm_rs(inputs, c8, 4.0, "tp=8 GEMM-RS, M=8192")
            for m in inputs.TP8_M_SWEEP:   # the oracle's rate does not depend on M; one sample serves the sweep
                if "gemm_rs_tp8_m%d" % m in secondary:
                    secondary["gemm_rs_tp8_m%d" % m]["cpu_baseline"] = base
        if lam_case is not None and "lamport_ar_rmsnorm" in secondary:
            c = lam_case
            secondary["lamport_ar_rmsnorm"]["cpu_baseline"] = cpu_baseline_rows(
                lambda rows: oracle.ar_rmsnorm(c["src"], c["gamma"], c["eps"], rows=rows), c["M"],
                LAMPORT_BYTES / c["M"], 4.0, "Lamport AR+RMSNorm, 8 x [4096,7168] (algorithmic bytes per row)",
                "rows")
        if comb_case is not None and "combine_reduce" in secondary:
            c = comb_case
            secondary["combine_reduce"]["cpu_baseline"] = cpu_baseline_rows(
                lambda tok: oracle.combine(c["x"], c["gate"], tokens=tok), c["T"], COMBINE_BYTES / c["T"], 4.0,
                "combine, [4096,8,7168] (algorithmic bytes per token)", "tokens")

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
                               "stream (96 workgroups) in shuffled order, their bits published 8 tiles per "
                               "release; one producer launch serves every step, resident before the first GEMM; "
                               "send + ready_out published",
                   "M": 4096, "N": 4096, "K": 2048, "R": 4, "owner": 0,
                   "producer_tiles_per_release": PRODUCER_TILES_PER_RELEASE,
                   "producer_workgroups": PRODUCER_WORKGROUPS,
                   "tile": head["tile"] if head else None},
    }
    if head:
        line["config"]["one_release_per_tile"] = {
            "tflops": r1["tflops"], "ms_per_step": r1["ms_per_step"], "kernel_ms_median": r1["gemm"]["ms_median"],
            "note": "the same step with the producer releasing after every tile"}
        g = head["gemm"]
        line["roofline"] = roofline("mfma", head["flops"], g, PEAK_BF16_TFLOPS, "TFLOP/s",
                                    measured_traffic("gemm_rs_tp4", head["tile"]), "gemm_rs_kernel")
        line["roofline"].update(kernel_ms_median=g["ms_median"], kernel_ms_min=g["ms_min"],
                                kernel_ms_p90=g["ms_p90"])
    line["secondary"] = secondary
    if cpu:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
