"""CPU oracle for the fused all-reduce epilogues (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and the
two share no code: this module loads ``oracle/liboracle.so`` (plain C, built with
gcc from ``oracle/oracle.c``) through ctypes and hands it numpy arrays.

What each function computes, and the page passage it follows, is stated in
``oracle.c``.  Arrays of bf16 are carried as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

SENTINEL_BF16 = 0x8000

# -O2 without fast-math and with contraction off: every multiply and add in the
# oracle is a separately rounded binary32 operation.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (no GPU code involved)."""
    with _lock:
        if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            tmp = _LIB + ".tmp%d" % os.getpid()
            subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
            os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    lib = ctypes.CDLL(_LIB)
    i64, i32, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_float
    vp = ctypes.c_void_p
    lib.oracle_gemm_rs.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i64, i64]
    lib.oracle_gemm_rs.restype = i32
    lib.oracle_gemm_rs_ring.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i64, i64]
    lib.oracle_gemm_rs_ring.restype = i32
    lib.oracle_flag_tiles.argtypes = [i64, i64, i32, i64, i64]
    lib.oracle_flag_tiles.restype = i64
    lib.oracle_flag_words.argtypes = [i64, i64, i32, i64, i64]
    lib.oracle_flag_words.restype = i64
    lib.oracle_ready_out.argtypes = [i64, i64, i32, i32, i64, i64, vp]
    lib.oracle_ready_out.restype = i32
    lib.oracle_lamport_canon.argtypes = [vp, vp, i64]
    lib.oracle_lamport_canon.restype = None
    lib.oracle_lamport_arm.argtypes = [vp, i64]
    lib.oracle_lamport_arm.restype = None
    lib.oracle_ar_rmsnorm.argtypes = [vp, vp, vp, i64, i64, i32, f32, i64, i64]
    lib.oracle_ar_rmsnorm.restype = i32
    lib.oracle_combine.argtypes = [vp, vp, vp, i64, i32, i64, i64, i64]
    lib.oracle_fp8_e4m3fn_to_f32.argtypes = [ctypes.c_uint8]
    lib.oracle_fp8_e4m3fn_to_f32.restype = ctypes.c_float
    lib.oracle_gemm_rs_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i64, i64]
    lib.oracle_gemm_rs_fp8.restype = i32
    lib.oracle_lamport_reduce.argtypes = [vp, vp, i64, i64, i32, i64, i64]
    lib.oracle_lamport_reduce.restype = i32
    lib.oracle_ar_rmsnorm_2phase.argtypes = [vp, vp, vp, i64, i64, i32, f32, i64, i64]
    lib.oracle_ar_rmsnorm_2phase.restype = i32
    lib.oracle_combine.restype = i32
    lib.oracle_bf16_from_f32.argtypes = [vp, vp, i64]
    lib.oracle_bf16_from_f32.restype = None
    lib.oracle_f32_from_bf16.argtypes = [vp, vp, i64]
    lib.oracle_f32_from_bf16.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i32
    _lib = lib
    return lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 arrays are passed as uint16 bit patterns, got %s" % a.dtype)
    return a


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def bf16_from_f32(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_bf16_from_f32(_p(x), _p(out), x.size)
    return out


def f32_from_bf16(b) -> np.ndarray:
    b = _u16(b)
    out = np.empty(b.shape, dtype=np.float32)
    _load().oracle_f32_from_bf16(_p(b), _p(out), b.size)
    return out


def gemm_rs(x, w, recv, R: int, owner: int, rows=None, want_send: bool = True):
    """GEMM + reduce-scatter epilogue of one rank.

    x: uint16 [M,K]; w: uint16 [K,N]; recv: list of R arrays uint16 [M/R,N]
    (recv[owner] may be None).  Returns (out [M/R,N], send [M,N] or None).
    ``rows=(r0, r1)`` computes only that band of the rank's local product;
    output rows outside it are left zero.
    """
    x, w = _u16(x), _u16(w)
    M, K = x.shape
    K2, N = w.shape
    if K2 != K:
        raise ValueError("x is [M,K] and w is [K,N]")
    if M % R:
        raise ValueError("M must be a multiple of R")
    seg = M // R
    keep = []
    ptrs = (ctypes.c_void_p * R)()
    for p in range(R):
        if p == owner or recv[p] is None:
            ptrs[p] = None
            continue
        rp = _u16(recv[p])
        if rp.shape != (seg, N):
            raise ValueError("recv[%d] must be [%d,%d]" % (p, seg, N))
        keep.append(rp)
        ptrs[p] = rp.ctypes.data
    out = np.zeros((seg, N), dtype=np.uint16)
    send = np.zeros((M, N), dtype=np.uint16) if want_send else None
    r0, r1 = (0, M) if rows is None else rows
    rc = _load().oracle_gemm_rs(_p(x), _p(w), ctypes.cast(ptrs, ctypes.c_void_p), _p(out),
                                _p(send) if send is not None else None, M, N, K, R, owner, r0, r1)
    if rc != 0:
        raise ValueError("oracle_gemm_rs rejected its arguments")
    return out, send


def gemm_rs_ring(x, w, upstream, R: int, owner: int, rows=None, want_send: bool = True):
    """Push-ring form of one rank's GEMM + reduce-scatter epilogue.

    upstream: list of R arrays uint16 [M/R,N]; upstream[d] is the running
    partial of segment d from the upstream rank (the entry of the segment this
    rank starts, (owner - 1) mod R, may be None).  Returns (out, send) like
    gemm_rs().
    """
    x, w = _u16(x), _u16(w)
    M, K = x.shape
    K2, N = w.shape
    if K2 != K:
        raise ValueError("x is [M,K] and w is [K,N]")
    if M % R:
        raise ValueError("M must be a multiple of R")
    seg = M // R
    chain = (owner + R - 1) % R
    keep = []
    ptrs = (ctypes.c_void_p * R)()
    for d in range(R):
        if R == 1 or d == chain or upstream[d] is None:
            if R > 1 and d != chain:
                raise ValueError("upstream[%d] is needed" % d)
            ptrs[d] = None
            continue
        ud = _u16(upstream[d])
        if ud.shape != (seg, N):
            raise ValueError("upstream[%d] must be [%d,%d]" % (d, seg, N))
        keep.append(ud)
        ptrs[d] = ud.ctypes.data
    out = np.zeros((seg, N), dtype=np.uint16)
    send = np.zeros((M, N), dtype=np.uint16) if want_send else None
    r0, r1 = (0, M) if rows is None else rows
    rc = _load().oracle_gemm_rs_ring(_p(x), _p(w), ctypes.cast(ptrs, ctypes.c_void_p), _p(out),
                                     _p(send) if send is not None else None, M, N, K, R, owner, r0, r1)
    if rc != 0:
        raise ValueError("oracle_gemm_rs_ring rejected its arguments")
    return out, send


def fp8_e4m3fn_to_f32(code: int) -> float:
    return float(_load().oracle_fp8_e4m3fn_to_f32(code))


def gemm_rs_fp8(x, xs, wt, ws, recv, R: int, owner: int, rows=None, want_send: bool = True):
    """fp8 block-scaled GEMM + reduce-scatter epilogue of one rank.

    x: uint8 [M,K] e4m3fn; xs: float32 [M,K/128]; wt: uint8 [N,K] (W
    transposed); ws: float32 [ceil(N/128),K/128]; recv as in gemm_rs()."""
    x = np.ascontiguousarray(x, dtype=np.uint8)
    wt = np.ascontiguousarray(wt, dtype=np.uint8)
    xs = np.ascontiguousarray(xs, dtype=np.float32)
    ws = np.ascontiguousarray(ws, dtype=np.float32)
    M, K = x.shape
    N, K2 = wt.shape
    if K2 != K or K % 128:
        raise ValueError("x is [M,K], wt is [N,K], K a multiple of 128")
    if xs.shape != (M, K // 128) or ws.shape != ((N + 127) // 128, K // 128):
        raise ValueError("xs must be [M,K/128] and ws [ceil(N/128),K/128]")
    if M % R:
        raise ValueError("M must be a multiple of R")
    seg = M // R
    keep = []
    ptrs = (ctypes.c_void_p * R)()
    for p in range(R):
        if p == owner or R == 1:
            ptrs[p] = None
            continue
        rp = _u16(recv[p])
        if rp.shape != (seg, N):
            raise ValueError("recv[%d] must be [%d,%d]" % (p, seg, N))
        keep.append(rp)
        ptrs[p] = rp.ctypes.data
    out = np.zeros((seg, N), dtype=np.uint16)
    send = np.zeros((M, N), dtype=np.uint16) if want_send else None
    r0, r1 = (0, M) if rows is None else rows
    rc = _load().oracle_gemm_rs_fp8(_p(x), _p(xs), _p(wt), _p(ws), ctypes.cast(ptrs, ctypes.c_void_p), _p(out),
                                    _p(send) if send is not None else None, M, N, K, R, owner, r0, r1)
    if rc != 0:
        raise ValueError("oracle_gemm_rs_fp8 rejected its arguments")
    return out, send


def flag_tiles(M: int, N: int, R: int, ftm: int, ftn: int) -> int:
    return int(_load().oracle_flag_tiles(M, N, R, ftm, ftn))


def flag_words(M: int, N: int, R: int, ftm: int, ftn: int) -> int:
    return int(_load().oracle_flag_words(M, N, R, ftm, ftn))


def ready_out(M: int, N: int, R: int, owner: int, ftm: int, ftn: int) -> np.ndarray:
    W = flag_words(M, N, R, ftm, ftn)
    words = np.zeros((R, W), dtype=np.uint32)
    if _load().oracle_ready_out(M, N, R, owner, ftm, ftn, _p(words)) != 0:
        raise ValueError("bad flag geometry")
    return words


def lamport_canon(src) -> np.ndarray:
    src = _u16(src)
    dst = np.empty_like(src)
    _load().oracle_lamport_canon(_p(src), _p(dst), src.size)
    return dst


def lamport_arm(n: int) -> np.ndarray:
    st = np.empty(n, dtype=np.uint16)
    _load().oracle_lamport_arm(_p(st), n)
    return st


def ar_rmsnorm(src, gamma, eps: float = 1e-6, rows=None) -> np.ndarray:
    """src: uint16 [S,M,N] partials as handed to the producers; gamma uint16 [N]."""
    src, gamma = _u16(src), _u16(gamma)
    S, M, N = src.shape
    if gamma.shape != (N,):
        raise ValueError("gamma must be [N]")
    out = np.zeros((M, N), dtype=np.uint16)
    r0, r1 = (0, M) if rows is None else rows
    if _load().oracle_ar_rmsnorm(_p(src), _p(gamma), _p(out), M, N, S, eps, r0, r1) != 0:
        raise ValueError("oracle_ar_rmsnorm rejected its arguments")
    return out


def lamport_reduce(x, rows=None) -> np.ndarray:
    """Phase A of the two-phase Lamport path: T = canon(bf16(sum over ranks)).
    x: uint16 [R,M,N] (the ranks' inputs).  Returns uint16 [M,N] (rows outside
    `rows` left zero)."""
    x = _u16(x)
    R, M, N = x.shape
    t = np.zeros((M, N), dtype=np.uint16)
    r0, r1 = (0, M) if rows is None else rows
    if _load().oracle_lamport_reduce(_p(x), _p(t), M, N, R, r0, r1) != 0:
        raise ValueError("oracle_lamport_reduce rejected its arguments")
    return t


def ar_rmsnorm_2phase(x, gamma, eps: float = 1e-6, rows=None) -> np.ndarray:
    """Two-phase Lamport AR + RMSNorm: RMSNorm of the bf16-rounded sum.
    x: uint16 [R,M,N]; gamma uint16 [N]."""
    x, gamma = _u16(x), _u16(gamma)
    R, M, N = x.shape
    if gamma.shape != (N,):
        raise ValueError("gamma must be [N]")
    out = np.zeros((M, N), dtype=np.uint16)
    r0, r1 = (0, M) if rows is None else rows
    if _load().oracle_ar_rmsnorm_2phase(_p(x), _p(gamma), _p(out), M, N, R, eps, r0, r1) != 0:
        raise ValueError("oracle_ar_rmsnorm_2phase rejected its arguments")
    return out


def combine(x, gate, tokens=None) -> np.ndarray:
    """x: uint16 [T,E,H]; gate: float32 [T,E]."""
    x = _u16(x)
    gate = np.ascontiguousarray(gate, dtype=np.float32)
    T, E, H = x.shape
    if gate.shape != (T, E):
        raise ValueError("gate must be [T,E]")
    out = np.zeros((T, H), dtype=np.uint16)
    t0, t1 = (0, T) if tokens is None else tokens
    if _load().oracle_combine(_p(x), _p(gate), _p(out), T, E, H, t0, t1) != 0:
        raise ValueError("oracle_combine rejected its arguments")
    return out
