"""MI355X (gfx950) fused all-reduce epilogues -- Python binding of libarepi.so.

Thin ctypes layer over the C ABI declared in ``include/arepi.h``: it checks
torch dtype, shape, device and contiguity, takes raw pointers and forwards them
with the caller's (or the current) HIP stream.  Every step of the hot path runs
in the library's HIP kernels; there is no fallback of any kind, and every call
raises if ``libarepi.so`` is missing or a kernel launch is refused.

Names mirror the C entry points without the ``arepi_`` prefix:
  gemm_rs_fused, gemm_rs_supports, gemm_rs_flag_words, gemm_rs_pick_tile, gemm_rs_schedule,
  lamport_prefill, lamport_publish, ar_rmsnorm_lamport, ar_rmsnorm_lamport_noalloc,
  combine_reduce (and its
  LDS-staged variant via pipeline="lds"),
  emu_peer_producer, last_error, version.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libarepi.so")

OK, EINVAL, EUNSUPPORTED, ELAUNCH = 0, -1, -2, -3
SCOPE_AGENT, SCOPE_SYSTEM = 0, 1
STATUS_TIMEOUT = 1
(TILE_AUTO, TILE_256x256, TILE_128x256, TILE_128x128, TILE_64x128, TILE_32x256, TILE_256x256_S4,
 TILE_256x128_S3, TILE_128x256_S3, TILE_128x128_S4, TILE_256x256_W8, TILE_256x256_W8_K64,
 TILE_64x128_S4) = range(13)
TILE_PAIRED_ROWS = 0x200  # OR into an explicit tile: pair owner half-blocks with non-owner ones
TILE_CONSUME_READY = 0x400  # OR into any tile: owner tiles clear the ready_in bits they waited for
TILE_OWNER_FIRST = 0x800  # OR into a contiguous tile: the owner's row blocks first (partials already landed)
TILE_OWNER_HALF = 0x1000  # OR into 256x256_w8_k64 (or AUTO): owner rows as 128x256 tiles after the rest
LAMPORT_NOALLOC_BYTES = 32 * 1024 * 1024  # static staging of ar_rmsnorm_lamport_noalloc
TILE_NAMES = {TILE_256x256: "256x256", TILE_128x256: "128x256", TILE_128x128: "128x128",
              TILE_64x128: "64x128", TILE_32x256: "32x256", TILE_256x256_S4: "256x256_s4",
              TILE_256x128_S3: "256x128_s3", TILE_128x256_S3: "128x256_s3", TILE_128x128_S4: "128x128_s4", TILE_256x256_W8: "256x256_w8",
              TILE_256x256_W8_K64: "256x256_w8_k64", TILE_64x128_S4: "64x128_s4"}
TILE_DIMS = {TILE_256x256: (256, 256), TILE_128x256: (128, 256), TILE_128x128: (128, 128),
             TILE_64x128: (64, 128), TILE_32x256: (32, 256), TILE_256x256_S4: (256, 256),
             TILE_256x128_S3: (256, 128), TILE_128x256_S3: (128, 256), TILE_128x128_S4: (128, 128), TILE_256x256_W8: (256, 256),
             TILE_256x256_W8_K64: (256, 256), TILE_64x128_S4: (64, 128)}

_lock = threading.Lock()
_lib = None


class ArepiError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s (status %d)" % (msg, code))
        self.code = code


def lib():
    """Load libarepi.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libarepi.so is not built (expected at %s); run "
                               "`python -m all_reduce_epilogues_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, u32p, vp, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float
        sig = {
            "arepi_last_error": ([], ctypes.c_char_p),
            "arepi_version": ([], ctypes.c_char_p),
            "arepi_gemm_rs_supports": ([i64, i64, i64, i32, i32, i32, i32, i32, i32], i32),
            "arepi_gemm_rs_flag_words": ([i64, i64, i32, i32, i32], i64),
            "arepi_gemm_rs_pick_tile": ([i64, i64, i64, i32, i32, i32, i32, i32], i32),
            "arepi_gemm_rs_schedule": ([i64, i64, i64, i32, i32, i32, i32, i32, i32, vp, i64], i64),
            "arepi_gemm_rs_fused": ([vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, i32, i32, i32,
                                     u32p, i64, vp], i32),
            "arepi_gemm_rs_ring_supports": ([i64, i64, i64, i32, i32, i32, i32, i32, i32], i32),
            "arepi_gemm_rs_ring_pick_tile": ([i64, i64, i64, i32, i32, i32, i32, i32], i32),
            "arepi_gemm_rs_ring": ([vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, i32, i32, i32,
                                    u32p, i64, vp], i32),
            "arepi_gemm_rs_fp8_supports": ([i64, i64, i64, i32, i32, i32, i32, i32, i32], i32),
            "arepi_gemm_rs_fp8": ([vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, i32, i32, i32,
                                   u32p, i64, vp], i32),
            "arepi_lamport_prefill": ([vp, i64, vp], i32),
            "arepi_lamport_publish": ([vp, vp, vp, i32, i64, i64, i32, i32, i32, vp], i32),
            "arepi_ar_rmsnorm_lamport": ([vp, vp, vp, i64, i64, i32, f32, i32, u32p, i64, vp], i32),
            "arepi_ar_rmsnorm_lamport_noalloc": ([vp, vp, i64, i64, i32, f32, i32, u32p, i64, vp, vp], i32),
            "arepi_ar_rmsnorm_lamport_2phase": ([vp, vp, vp, vp, i64, i64, i32, i32, f32, i32, u32p, i64, vp],
                                                i32),
            "arepi_emu_lamport_phase_a": ([vp, vp, i64, i64, i32, i32, i32, vp], i32),
            "arepi_combine_reduce": ([vp, vp, vp, i64, i32, i64, vp], i32),
            "arepi_combine_reduce_lds": ([vp, vp, vp, i64, i32, i64, vp], i32),
            "arepi_emu_peer_producer": ([vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, i32, i32, i32, i32, vp,
                                         vp], i32),
            "arepi_emu_producer_gate": ([vp, u32p, i64, vp], i32),
            "arepi_emu_peer_producer_steps": ([vp, vp, vp, vp, i32, i64, i64, i64, i32, i32, i32, i32, i32, i32,
                                               i32, vp, vp, i32, i32, i64, u32p, i64, vp], i32),
            "arepi_emu_signal": ([vp, ctypes.c_uint32, vp], i32),
            "arepi_emu_stream_create": ([vp], i32),
            "arepi_emu_stream_destroy": ([vp], i32),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def last_error() -> str:
    return lib().arepi_last_error().decode()


def version() -> str:
    return lib().arepi_version().decode()


def _check(rc: int, what: str) -> int:
    if rc < 0:
        raise ArepiError(rc, "%s: %s" % (what, last_error()))
    return rc


# ---- tensor checks (before any pointer is taken) -------------------------------

def _torch():
    import torch
    return torch


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need(t, name, dtypes, shape=None, device=True):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s must have dtype %s, got %s" % (name, " or ".join(map(str, dtypes)), t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if device and t.device.type != "cuda":
        raise ValueError("%s must live on the GPU, got %s" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _bf16(t, name, shape=None):
    _need(t, name, (_torch().bfloat16,), shape)


def _flags(t, name, shape=None):
    torch = _torch()
    _need(t, name, (torch.int32, torch.uint32), shape)


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ---- GEMM + reduce-scatter --------------------------------------------------------

def gemm_rs_flag_words(M: int, N: int, R: int, flag_tile_m: int = 128, flag_tile_n: int = 128) -> int:
    return _check(lib().arepi_gemm_rs_flag_words(M, N, R, flag_tile_m, flag_tile_n), "gemm_rs_flag_words")


def gemm_rs_supports(M, N, K, R, owner, flag_tile_m=128, flag_tile_n=128, publish=False, tile=TILE_AUTO) -> int:
    """0 when supported, else the negative status (message in last_error())."""
    return lib().arepi_gemm_rs_supports(M, N, K, R, owner, flag_tile_m, flag_tile_n, int(publish), tile)


def gemm_rs_schedule(M, N, K, R, owner, flag_tile_m=128, flag_tile_n=128, publish=False, tile=TILE_AUTO):
    """Work assignment of gemm_rs_fused: list of (row block, column block, a0, a_rows, b0, b_rows)
    per workgroup in launch order (the rows it computes are [a0, a0+a_rows) and [b0, b0+b_rows));
    row block -1 marks the owner's half-height tiles (TILE_OWNER_HALF, or chosen by AUTO)."""
    n = _check(lib().arepi_gemm_rs_schedule(M, N, K, R, owner, flag_tile_m, flag_tile_n, int(publish), tile,
                                             None, 0), "gemm_rs_schedule")
    buf = (ctypes.c_int64 * (6 * n))()
    _check(lib().arepi_gemm_rs_schedule(M, N, K, R, owner, flag_tile_m, flag_tile_n, int(publish), tile,
                                        ctypes.cast(buf, ctypes.c_void_p), 6 * n), "gemm_rs_schedule")
    return [tuple(buf[6 * i:6 * i + 6]) for i in range(n)]


def gemm_rs_pick_tile(M, N, K, R, owner, flag_tile_m=128, flag_tile_n=128, publish=False) -> int:
    return _check(lib().arepi_gemm_rs_pick_tile(M, N, K, R, owner, flag_tile_m, flag_tile_n, int(publish)),
                  "gemm_rs_pick_tile")


def gemm_rs_fused(x, w, recv, ready_in, out, R: int, owner: int, send=None, ready_out=None,
                  flag_tile_m: int = 128, flag_tile_n: int = 128, scope: int = SCOPE_AGENT,
                  tile: int = TILE_AUTO, status=None, spin_limit: int = 0, stream=None):
    """out[M/R,N] = bf16(X.W owner rows + sum of peers' recv); see include/arepi.h."""
    _bf16(x, "x")
    M, K = x.shape
    _bf16(w, "w")
    if w.shape[0] != K:
        raise ValueError("w must be [K=%d, N], got %s" % (K, tuple(w.shape)))
    N = w.shape[1]
    if M % R:
        raise ValueError("M=%d is not a multiple of R=%d" % (M, R))
    seg = M // R
    _bf16(out, "out", (seg, N))
    if send is not None:
        _bf16(send, "send", (M, N))
    words = gemm_rs_flag_words(M, N, R, flag_tile_m, flag_tile_n)
    if ready_in is not None:
        _flags(ready_in, "ready_in", (R, words))
    if ready_out is not None:
        _flags(ready_out, "ready_out", (R, words))
    if status is not None:
        _flags(status, "status", (1,))
    ptrs = (ctypes.c_void_p * R)()
    if len(recv) != R:
        raise ValueError("recv must list R=%d buffers (entry owner may be None)" % R)
    for p in range(R):
        if p == owner or recv[p] is None:
            ptrs[p] = None
            continue
        _bf16(recv[p], "recv[%d]" % p, (seg, N))
        ptrs[p] = recv[p].data_ptr()
    rc = lib().arepi_gemm_rs_fused(_ptr(x), _ptr(w), ctypes.cast(ptrs, ctypes.c_void_p), _ptr(ready_in),
                                   _ptr(out), _ptr(send), _ptr(ready_out), M, N, K, R, owner,
                                   flag_tile_m, flag_tile_n, scope, tile, _ptr(status), spin_limit,
                                   _stream(stream))
    _check(rc, "gemm_rs_fused")


def gemm_rs_ring_supports(M, N, K, R, owner, flag_tile_m=128, flag_tile_n=128, publish=False,
                          tile=TILE_AUTO) -> int:
    """0 when the push-ring form supports the shape, else the negative status."""
    return lib().arepi_gemm_rs_ring_supports(M, N, K, R, owner, flag_tile_m, flag_tile_n, int(publish), tile)


def gemm_rs_ring_pick_tile(M, N, K, R, owner, flag_tile_m=128, flag_tile_n=128, publish=False) -> int:
    return _check(lib().arepi_gemm_rs_ring_pick_tile(M, N, K, R, owner, flag_tile_m, flag_tile_n, int(publish)),
                  "gemm_rs_ring_pick_tile")


def gemm_rs_ring(x, w, upstream, ready_in, out, send, R: int, owner: int, ready_out=None,
                 flag_tile_m: int = 128, flag_tile_n: int = 128, scope: int = SCOPE_AGENT,
                 tile: int = TILE_AUTO, status=None, spin_limit: int = 0, stream=None):
    """One hop of the push ring: out = bf16(X.W owner rows + upstream[owner]),
    send rows of segment d = bf16(X.W + upstream[d]) (the chain segment
    (owner-1) mod R without upstream); see include/arepi.h."""
    _bf16(x, "x")
    M, K = x.shape
    _bf16(w, "w")
    if w.shape[0] != K:
        raise ValueError("w must be [K=%d, N], got %s" % (K, tuple(w.shape)))
    N = w.shape[1]
    if M % R:
        raise ValueError("M=%d is not a multiple of R=%d" % (M, R))
    seg = M // R
    chain = (owner + R - 1) % R
    _bf16(out, "out", (seg, N))
    _bf16(send, "send", (M, N))
    words = gemm_rs_flag_words(M, N, R, flag_tile_m, flag_tile_n)
    if ready_in is not None:
        _flags(ready_in, "ready_in", (R, words))
    if ready_out is not None:
        _flags(ready_out, "ready_out", (R, words))
    if status is not None:
        _flags(status, "status", (1,))
    if len(upstream) != R:
        raise ValueError("upstream must list R=%d buffers (entry (owner-1) mod R may be None)" % R)
    ptrs = (ctypes.c_void_p * R)()
    for d in range(R):
        if (R > 1 and d == chain) or upstream[d] is None:
            ptrs[d] = None
            continue
        _bf16(upstream[d], "upstream[%d]" % d, (seg, N))
        ptrs[d] = upstream[d].data_ptr()
    rc = lib().arepi_gemm_rs_ring(_ptr(x), _ptr(w), ctypes.cast(ptrs, ctypes.c_void_p), _ptr(ready_in),
                                  _ptr(out), _ptr(send), _ptr(ready_out), M, N, K, R, owner,
                                  flag_tile_m, flag_tile_n, scope, tile, _ptr(status), spin_limit,
                                  _stream(stream))
    _check(rc, "gemm_rs_ring")


def gemm_rs_fp8_supports(M, N, K, R, owner, flag_tile_m=128, flag_tile_n=128, publish=False, tile=0) -> int:
    """0 when the fp8 block-scaled form supports the shape, else the negative status."""
    return lib().arepi_gemm_rs_fp8_supports(M, N, K, R, owner, flag_tile_m, flag_tile_n, int(publish), tile)


def gemm_rs_fp8(x, xs, wt, ws, recv, ready_in, out, R: int, owner: int, send=None, ready_out=None,
                flag_tile_m: int = 128, flag_tile_n: int = 128, scope: int = SCOPE_AGENT, tile: int = 0,
                status=None, spin_limit: int = 0, stream=None):
    """fp8 e4m3fn block-scaled GEMM + reduce-scatter epilogue; see include/arepi.h.

    x: torch.float8_e4m3fn (or uint8 bytes) [M,K]; xs: float32 [M,K/128];
    wt: e4m3fn [N,K] (W transposed); ws: float32 [ceil(N/128),K/128]."""
    torch = _torch()
    fp8 = (torch.float8_e4m3fn, torch.uint8)
    _need(x, "x", fp8)
    _need(wt, "wt", fp8)
    if x.dim() != 2 or wt.dim() != 2 or x.shape[1] != wt.shape[1]:
        raise ValueError("x must be [M,K] and wt [N,K]")
    M, K = x.shape
    N = wt.shape[0]
    if K % 128:
        raise ValueError("K=%d must be a multiple of 128" % K)
    _need(xs, "xs", (torch.float32,), (M, K // 128))
    _need(ws, "ws", (torch.float32,), ((N + 127) // 128, K // 128))
    if M % R:
        raise ValueError("M=%d is not a multiple of R=%d" % (M, R))
    seg = M // R
    _bf16(out, "out", (seg, N))
    if send is not None:
        _bf16(send, "send", (M, N))
    words = gemm_rs_flag_words(M, N, R, flag_tile_m, flag_tile_n)
    if ready_in is not None:
        _flags(ready_in, "ready_in", (R, words))
    if ready_out is not None:
        _flags(ready_out, "ready_out", (R, words))
    if status is not None:
        _flags(status, "status", (1,))
    ptrs = (ctypes.c_void_p * R)()
    if len(recv) != R:
        raise ValueError("recv must list R=%d buffers (entry owner may be None)" % R)
    for q in range(R):
        if q == owner or recv[q] is None:
            ptrs[q] = None
            continue
        _bf16(recv[q], "recv[%d]" % q, (seg, N))
        ptrs[q] = recv[q].data_ptr()
    rc = lib().arepi_gemm_rs_fp8(_ptr(x), _ptr(xs), _ptr(wt), _ptr(ws), ctypes.cast(ptrs, ctypes.c_void_p),
                                 _ptr(ready_in), _ptr(out), _ptr(send), _ptr(ready_out), M, N, K, R, owner,
                                 flag_tile_m, flag_tile_n, scope, tile, _ptr(status), spin_limit, _stream(stream))
    _check(rc, "gemm_rs_fp8")


def emu_peer_producer(src, recv, ready_in, order, R: int, owner: int, M: int, N: int,
                      flag_tile_m: int = 128, flag_tile_n: int = 128, scope: int = SCOPE_AGENT,
                      workgroups: int = 0, items_per_release: int = 1, resident=None, stream=None):
    """Test-only: land (peer, tile) items of src[p] into recv[p] and set their bits,
    items_per_release tiles per release (workgroups > 0: that many batches in
    flight at a time).  resident: int32 [2] (zero before first use) for
    emu_producer_gate."""
    seg = M // R
    torch = _torch()
    _need(order, "order", (torch.int32,))
    if order.dim() != 2 or order.shape[1] != 2:
        raise ValueError("order must be int32 [n_items, 2]")
    words = gemm_rs_flag_words(M, N, R, flag_tile_m, flag_tile_n)
    _flags(ready_in, "ready_in", (R, words))
    if resident is not None:
        _flags(resident, "resident", (2,))
    sp = (ctypes.c_void_p * R)()
    rp = (ctypes.c_void_p * R)()
    for p in range(R):
        if p == owner:
            continue
        _bf16(src[p], "src[%d]" % p, (seg, N))
        _bf16(recv[p], "recv[%d]" % p, (seg, N))
        sp[p] = src[p].data_ptr()
        rp[p] = recv[p].data_ptr()
    rc = lib().arepi_emu_peer_producer(ctypes.cast(sp, ctypes.c_void_p), ctypes.cast(rp, ctypes.c_void_p),
                                       _ptr(ready_in), _ptr(order), order.shape[0], M, N, R, owner,
                                       flag_tile_m, flag_tile_n, scope, workgroups, items_per_release,
                                       _ptr(resident), _stream(stream))
    _check(rc, "emu_peer_producer")


def _peer_arrays(src, recv, R, owner, seg, N, src_sets=0):
    sp = (ctypes.c_void_p * R)()
    rp = (ctypes.c_void_p * R)()
    for p in range(R):
        if p == owner:
            continue
        _bf16(src[p], "src[%d]" % p, (src_sets, seg, N) if src_sets else (seg, N))
        _bf16(recv[p], "recv[%d]" % p, (seg, N))
        sp[p] = src[p].data_ptr()
        rp[p] = recv[p].data_ptr()
    return ctypes.cast(sp, ctypes.c_void_p), ctypes.cast(rp, ctypes.c_void_p)


def emu_peer_producer_steps(src, recv, ready_in, orders, R: int, owner: int, M: int, N: int, go, steps: int,
                            flag_tile_m: int = 128, flag_tile_n: int = 128, scope: int = SCOPE_AGENT,
                            workgroups: int = 0, items_per_release: int = 1, resident=None, status=None,
                            spin_limit: int = 0, stream=None, credit: bool = False):
    """Test-only: the emulated peers of `steps` consecutive calls in one launch;
    step s lands orders[s % len(orders)] (orders: int32 [n_orders, n_items,
    2]).  go: uint32 [1], zero before the launch.  credit=False: step s starts
    once go[0] >= s (raise it with emu_signal after each call).  credit=True:
    go counts the producer's own landed steps, and each batch waits until its
    ready_in bits have been consumed (the consumer passes TILE_CONSUME_READY).
    src[p]: bf16 [M/R, N], the same every step, or [n_orders, M/R, N], set
    s % n_orders for step s."""
    torch = _torch()
    _need(orders, "orders", (torch.int32,))
    if orders.dim() != 3 or orders.shape[2] != 2:
        raise ValueError("orders must be int32 [n_orders, n_items, 2]")
    words = gemm_rs_flag_words(M, N, R, flag_tile_m, flag_tile_n)
    _flags(ready_in, "ready_in", (R, words))
    _flags(go, "go", (1,))
    some = next(src[p] for p in range(R) if p != owner)
    sets = orders.shape[0] if some.dim() == 3 else 0
    if resident is not None:
        _flags(resident, "resident", (2,))
    if status is not None:
        _flags(status, "status", (1,))
    sp, rp = _peer_arrays(src, recv, R, owner, M // R, N, sets)
    rc = lib().arepi_emu_peer_producer_steps(sp, rp, _ptr(ready_in), _ptr(orders), orders.shape[0], orders.shape[1],
                                             M, N, R, owner, flag_tile_m, flag_tile_n, scope, workgroups,
                                             items_per_release, _ptr(resident), _ptr(go), int(bool(credit)), steps,
                                             (M // R) * N if sets else 0, _ptr(status), spin_limit,
                                             _stream(stream))
    _check(rc, "emu_peer_producer_steps")


_emu_streams = {}


def _destroy_emu_streams():
    """At exit: finish and destroy the streams emu_stream() created."""
    if not _emu_streams:
        return
    torch = _torch()
    for dev, st in list(_emu_streams.items()):
        try:
            st.synchronize()
            lib().arepi_emu_stream_destroy(ctypes.c_void_p(st.cuda_stream))
        except Exception:
            pass
    _emu_streams.clear()


def emu_stream():
    """Test-only: a torch stream on a hardware queue of its own (see
    arepi_emu_stream_create), one per device, kept for the process."""
    torch = _torch()
    dev = torch.cuda.current_device()
    if dev not in _emu_streams:
        h = ctypes.c_void_p()
        _check(lib().arepi_emu_stream_create(ctypes.byref(h)), "emu_stream_create")
        if not _emu_streams:
            import atexit
            atexit.register(_destroy_emu_streams)
        _emu_streams[dev] = torch.cuda.ExternalStream(h.value, device=dev)
    return _emu_streams[dev]


def emu_signal(flag, value: int, stream=None):
    """Test-only: flag[0] = value once the work queued before it on `stream` has ended."""
    _flags(flag, "flag", (1,))
    _check(lib().arepi_emu_signal(_ptr(flag), value, _stream(stream)), "emu_signal")


def emu_producer_gate(resident, status=None, spin_limit: int = 0, stream=None):
    """Test-only: on the consumer's stream, between emu_peer_producer (issued
    first, with the same resident) and the consumer: returns once every
    producer workgroup has started, so the consumer cannot crowd it out."""
    _flags(resident, "resident", (2,))
    if status is not None:
        _flags(status, "status", (1,))
    _check(lib().arepi_emu_producer_gate(_ptr(resident), _ptr(status), spin_limit, _stream(stream)),
           "emu_producer_gate")


# ---- Lamport AR + RMSNorm ------------------------------------------------------------

def lamport_prefill(staging, stream=None):
    _bf16(staging, "staging")
    _check(lib().arepi_lamport_prefill(_ptr(staging), staging.numel(), _stream(stream)), "lamport_prefill")


def lamport_publish(src, staging, order, tile_m: int = 128, tile_n: int = 128, scope: int = SCOPE_AGENT,
                    stream=None):
    """Emulated producers: src [S,M,N] -> staging [S,M,N] in order[s] tile order."""
    _bf16(src, "src")
    S, M, N = src.shape
    _bf16(staging, "staging", (S, M, N))
    torch = _torch()
    tiles = -(-M // tile_m) * -(-N // tile_n)
    _need(order, "order", (torch.int32,), (S, tiles))
    _check(lib().arepi_lamport_publish(_ptr(src), _ptr(staging), _ptr(order), S, M, N, tile_m, tile_n, scope,
                                       _stream(stream)), "lamport_publish")


def ar_rmsnorm_lamport(staging, gamma, out, eps: float = 1e-6, scope: int = SCOPE_AGENT, status=None,
                       spin_limit: int = 0, stream=None):
    _bf16(staging, "staging")
    S, M, N = staging.shape
    _bf16(gamma, "gamma", (N,))
    _bf16(out, "out", (M, N))
    if status is not None:
        _flags(status, "status", (1,))
    _check(lib().arepi_ar_rmsnorm_lamport(_ptr(staging), _ptr(gamma), _ptr(out), M, N, S, float(eps), scope,
                                          _ptr(status), spin_limit, _stream(stream)), "ar_rmsnorm_lamport")


def ar_rmsnorm_lamport_noalloc(gamma, out, S: int, eps: float = 1e-6, scope: int = SCOPE_AGENT, status=None,
                               spin_limit: int = 0, stream=None) -> int:
    """ar_rmsnorm_lamport on the library's static staging (no allocation).
    out is bf16 [M,N] (M = 0 only sets the device up).  Returns the staging's
    device address on the current device, laid out [S][M][N] for this call,
    for the producers to publish into."""
    _bf16(out, "out")
    M, N = out.shape
    _bf16(gamma, "gamma", (N,))
    if status is not None:
        _flags(status, "status", (1,))
    addr = ctypes.c_void_p()
    _check(lib().arepi_ar_rmsnorm_lamport_noalloc(_ptr(gamma), _ptr(out) if M else None, M, N, S, float(eps),
                                                  scope, _ptr(status), spin_limit, ctypes.byref(addr),
                                                  _stream(stream)), "ar_rmsnorm_lamport_noalloc")
    return addr.value


# ---- combine --------------------------------------------------------------------------

def _rank_arrays(inputs, staging):
    R = len(inputs)
    if len(staging) != R or R < 1:
        raise ValueError("inputs and staging must list the same R >= 1 buffers")
    shape = tuple(inputs[0].shape)
    if len(shape) != 2:
        raise ValueError("inputs are [M,N]")
    ip = (ctypes.c_void_p * R)()
    sp = (ctypes.c_void_p * R)()
    for r in range(R):
        _bf16(inputs[r], "inputs[%d]" % r, shape)
        _bf16(staging[r], "staging[%d]" % r, shape)
        ip[r] = inputs[r].data_ptr()
        sp[r] = staging[r].data_ptr()
    return R, shape, ip, sp


def ar_rmsnorm_lamport_2phase(inputs, staging, gamma, out, rank: int, eps: float = 1e-6,
                              scope: int = SCOPE_AGENT, status=None, spin_limit: int = 0, stream=None):
    """Two-phase Lamport AR + RMSNorm on rank `rank`: reduce this rank's part of
    the R inputs into every rank's staging (phase A), then consume this rank's
    staging into out (phase B).  inputs/staging: lists of R bf16 [M,N] tensors
    (staging armed with lamport_prefill)."""
    R, (M, N), ip, sp = _rank_arrays(inputs, staging)
    _bf16(gamma, "gamma", (N,))
    _bf16(out, "out", (M, N))
    if status is not None:
        _flags(status, "status", (1,))
    rc = lib().arepi_ar_rmsnorm_lamport_2phase(ctypes.cast(ip, ctypes.c_void_p), ctypes.cast(sp, ctypes.c_void_p),
                                               _ptr(gamma), _ptr(out), M, N, R, rank, eps, scope, _ptr(status),
                                               spin_limit, _stream(stream))
    _check(rc, "ar_rmsnorm_lamport_2phase")


def emu_lamport_phase_a(inputs, staging, rank: int, scope: int = SCOPE_AGENT, stream=None):
    """Test-only: phase A of rank `rank` alone (stands in for a peer GPU)."""
    R, (M, N), ip, sp = _rank_arrays(inputs, staging)
    rc = lib().arepi_emu_lamport_phase_a(ctypes.cast(ip, ctypes.c_void_p), ctypes.cast(sp, ctypes.c_void_p),
                                         M, N, R, rank, scope, _stream(stream))
    _check(rc, "emu_lamport_phase_a")


def combine_reduce(x, gate, out, stream=None, pipeline: str = "registers"):
    """out[t,h] = bf16(sum_k gate[t,k] * x[t,k,h]).  pipeline="lds" selects the
    LDS-staged kernel (arepi_combine_reduce_lds) instead of the default."""
    _bf16(x, "x")
    T, E, H = x.shape
    torch = _torch()
    _need(gate, "gate", (torch.float32,), (T, E))
    _bf16(out, "out", (T, H))
    if pipeline == "registers":
        fn, name = lib().arepi_combine_reduce, "combine_reduce"
    elif pipeline == "lds":
        fn, name = lib().arepi_combine_reduce_lds, "combine_reduce_lds"
    else:
        raise ValueError("pipeline must be 'registers' or 'lds'")
    _check(fn(_ptr(x), _ptr(gate), _ptr(out), T, E, H, _stream(stream)), name)
