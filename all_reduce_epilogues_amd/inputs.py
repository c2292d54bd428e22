"""Seeded synthetic inputs shared by the HIP path's tests/benchmark and the oracle.

This module holds no arithmetic of the method itself: it only draws random
numbers with a seeded CPU ``torch.Generator``, rounds fp32 samples to bf16 with
torch's own conversion, and hands back numpy arrays (bf16 as uint16 bit
patterns).  Both sides of a parity test receive exactly the same bits.

The shapes and distributions stand in for the pages' model workloads (the
DeepSeek-V4-Pro ``wo_b`` row-parallel projection, [M,7168] at TP8 with K=2048,
and AR+RMSNorm at n=7168); no dataset or checkpoint is involved.

Workloads (seed = 1000 + workload number unless given):
  1 gemm_rs tiny      R=2, X[256,256], W[256,512], recv [128,512], all U(-1,1)
  2 gemm_rs tp4       R=4, X[4096,2048] N(0,1), W[2048,4096] N(0,0.02),
                      recv [1024,4096] N(0,0.5); shuffled producer order
  3 gemm_rs tp8       R=8, X[M,2048] N(0,1), W[2048,7168] N(0,0.02),
                      recv [M/8,7168] N(0,0.5), M in {256,1024,4096,8192}
  4 lamport           8 partials [4096,7168] N(0,1), gamma [7168] N(1,0.1),
                      random 128x128 publication order per slot
  5 combine           x [4096,8,7168] N(0,1), gate softmax(N(0,1)) over 8, fp32
"""
from __future__ import annotations

import numpy as np
import torch


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.bfloat16).contiguous().view(torch.int16).numpy().view(np.uint16)


def normal_bf16(shape, std: float, g: torch.Generator, mean: float = 0.0) -> np.ndarray:
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return _bf16_bits(t)


def uniform_bf16(shape, lo: float, hi: float, g: torch.Generator) -> np.ndarray:
    t = torch.rand(*shape, generator=g, dtype=torch.float32)
    t.mul_(hi - lo).add_(lo)
    return _bf16_bits(t)


def gemm_rs_case(M: int, N: int, K: int, R: int, owner: int = 0, seed: int = 1002,
                 dist: str = "normal", x_std: float = 1.0, w_std: float = 0.02,
                 recv_std: float = 0.5) -> dict:
    """X_r [M,K], W_r [K,N] and the R-1 peer partials [M/R,N] (recv[owner] is None)."""
    if M % R:
        raise ValueError("M must be a multiple of R")
    g = _gen(seed)
    seg = M // R
    if dist == "uniform":
        x = uniform_bf16((M, K), -1.0, 1.0, g)
        w = uniform_bf16((K, N), -1.0, 1.0, g)
        recv = [None if p == owner else uniform_bf16((seg, N), -1.0, 1.0, g) for p in range(R)]
    elif dist == "normal":
        x = normal_bf16((M, K), x_std, g)
        w = normal_bf16((K, N), w_std, g)
        recv = [None if p == owner else normal_bf16((seg, N), recv_std, g) for p in range(R)]
    else:
        raise ValueError(dist)
    return dict(x=x, w=w, recv=recv, M=M, N=N, K=K, R=R, owner=owner, seed=seed)


def gemm_rs_ring_case(M: int, N: int, K: int, R: int, owner: int = 0, seed: int = 1002, **kw) -> dict:
    """X_r, W_r and the running partials received from upstream in the push
    ring: up[d] [M/R,N] for every segment d except the one this rank starts,
    (owner - 1) mod R, whose entry is None.  Same draws as gemm_rs_case with
    that segment in the owner's place."""
    c = gemm_rs_case(M, N, K, R, owner=(owner + R - 1) % R, seed=seed, **kw)
    c["up"] = c.pop("recv")
    c["owner"] = owner
    return c


def fp8_e4m3fn_codes(shape, std: float, g: torch.Generator) -> np.ndarray:
    """e4m3fn bytes of N(0, std) samples (torch's round-to-nearest conversion)."""
    t = torch.randn(*shape, generator=g, dtype=torch.float32) * std
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def gemm_rs_fp8_case(M: int, N: int, K: int, R: int, owner: int = 0, seed: int = 1002,
                     x_std: float = 2.0, w_std: float = 2.0, recv_std: float = 0.5) -> dict:
    """fp8 operands of the block-scaled GEMM + reduce-scatter: x [M,K] and wt
    [N,K] e4m3fn bytes, positive fp32 block scales xs [M,K/128] and ws
    [ceil(N/128),K/128] ~ U(0.02, 0.06), and the R-1 bf16 peer partials."""
    if M % R or K % 128:
        raise ValueError("M must be a multiple of R and K of 128")
    g = _gen(seed)
    seg = M // R
    x = fp8_e4m3fn_codes((M, K), x_std, g)
    wt = fp8_e4m3fn_codes((N, K), w_std, g)
    xs = (0.02 + 0.04 * torch.rand(M, K // 128, generator=g)).numpy().astype(np.float32)
    ws = (0.02 + 0.04 * torch.rand((N + 127) // 128, K // 128, generator=g)).numpy().astype(np.float32)
    recv = [None if p == owner else normal_bf16((seg, N), recv_std, g) for p in range(R)]
    return dict(x=x, xs=xs, wt=wt, ws=ws, recv=recv, M=M, N=N, K=K, R=R, owner=owner, seed=seed)


WORKLOADS = {
    1: dict(M=256, N=512, K=256, R=2, dist="uniform"),
    2: dict(M=4096, N=4096, K=2048, R=4, dist="normal"),
    3: dict(N=7168, K=2048, R=8, dist="normal"),  # M swept
}
TP8_M_SWEEP = (256, 1024, 4096, 8192)


def workload_gemm_rs(num: int, M: int | None = None, owner: int = 0, seed: int | None = None) -> dict:
    spec = dict(WORKLOADS[num])
    if M is not None:
        spec["M"] = M
    return gemm_rs_case(owner=owner, seed=(1000 + num) if seed is None else seed, **spec)


def producer_order(R: int, owner: int, tiles: int, seed: int) -> np.ndarray:
    """Shuffled (peer, flag tile) publication order for the emulated peers:
    int32 [n_items, 2] with every peer p != owner and tile t exactly once."""
    g = _gen(seed)
    peers = [p for p in range(R) if p != owner]
    items = np.array([(p, t) for p in peers for t in range(tiles)], dtype=np.int32).reshape(-1, 2)
    perm = torch.randperm(items.shape[0], generator=g).numpy()
    return np.ascontiguousarray(items[perm])


def lamport_case(S: int = 8, M: int = 4096, N: int = 7168, seed: int = 1004,
                 tile_m: int = 128, tile_n: int = 128) -> dict:
    """S partial buffers [S,M,N] N(0,1), gamma [N] N(1,0.1), and one random tile
    publication order per slot (int32 [S, tiles])."""
    g = _gen(seed)
    src = normal_bf16((S, M, N), 1.0, g)
    gamma = normal_bf16((N,), 0.1, g, mean=1.0)
    tiles = ((M + tile_m - 1) // tile_m) * ((N + tile_n - 1) // tile_n)
    order = np.stack([torch.randperm(tiles, generator=g).numpy().astype(np.int32) for _ in range(S)])
    return dict(src=src, gamma=gamma, order=np.ascontiguousarray(order), S=S, M=M, N=N,
                tile_m=tile_m, tile_n=tile_n, eps=1e-6, seed=seed)


def combine_case(T: int = 4096, E: int = 8, H: int = 7168, seed: int = 1005) -> dict:
    g = _gen(seed)
    x = normal_bf16((T, E, H), 1.0, g)
    logits = torch.randn(T, E, generator=g, dtype=torch.float32)
    gate = torch.softmax(logits, dim=-1).numpy().astype(np.float32)
    return dict(x=x, gate=np.ascontiguousarray(gate), T=T, E=E, H=H, seed=seed)
