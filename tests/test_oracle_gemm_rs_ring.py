"""Pins for the push-ring form of the GEMM + reduce-scatter oracle (CPU only).

  * with R = 2 the ring and the direct sum are the same computation: bit-exact;
  * a whole ring simulated on the CPU (every rank's hop computed by the oracle,
    the running partials handed downstream) must end, at every owner, with
    the full product of the K-split operands: bit for bit on small integers,
    where every partial sum is exact in bf16 and fp32;
  * the segment a rank starts is its bare partial, rounded once.
"""
import numpy as np
import pytest
import torch

import oracle


def bits(a):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def widen(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rand_bf16(rng, shape, scale=1.0):
    return bits(rng.standard_normal(shape) * scale)


@pytest.mark.parametrize("owner", [0, 1])
def test_two_ranks_ring_equals_direct(owner):
    rng = np.random.default_rng(7 + owner)
    M, N, K = 64, 40, 24
    x, w = rand_bf16(rng, (M, K)), rand_bf16(rng, (K, N), 0.1)
    peer = 1 - owner
    part = rand_bf16(rng, (M // 2, N), 0.5)
    recv = [None, None]
    recv[peer] = part
    up = [None, None]
    up[owner] = part  # the one upstream partial is the peer's
    d_out, d_send = oracle.gemm_rs(x, w, recv, 2, owner)
    r_out, r_send = oracle.gemm_rs_ring(x, w, up, 2, owner)
    assert np.array_equal(d_out, r_out) and np.array_equal(d_send, r_send)


def simulate_ring(xs, ws, R):
    """Every rank's hop in chain order; returns the owners' outputs and the
    running partials each rank sent."""
    M, N = xs[0].shape[0], ws[0].shape[1]
    seg = M // R
    outs = [None] * R
    sent = {}  # (rank, segment) -> bf16 [seg, N]
    for d in range(R):
        carry = None
        for hop in range(1, R + 1):
            r = (d + hop) % R
            up = [np.zeros((seg, N), np.uint16) for _ in range(R)]
            if carry is not None:
                up[d] = carry
            out, send = oracle.gemm_rs_ring(xs[r], ws[r], up, R, r, rows=(d * seg, (d + 1) * seg))
            if r == d:
                outs[d] = out
            else:
                carry = send[d * seg:(d + 1) * seg].copy()
                sent[(r, d)] = carry
    return outs, sent


@pytest.mark.parametrize("R", [3, 4, 5])
def test_simulated_ring_reaches_the_full_product_exactly(R):
    rng = np.random.default_rng(100 + R)
    M, N, Kr = 16 * R, 24, 8
    Xf = rng.integers(-2, 3, size=(M, R * Kr)).astype(np.float64)
    Wf = rng.integers(-2, 3, size=(R * Kr, N)).astype(np.float64)
    xs = [bits(Xf[:, r * Kr:(r + 1) * Kr]) for r in range(R)]
    ws = [bits(Wf[r * Kr:(r + 1) * Kr]) for r in range(R)]
    full = Xf @ Wf  # |values| <= R*Kr*4 < 256: every partial sum is exact in bf16
    outs, sent = simulate_ring(xs, ws, R)
    seg = M // R
    for d in range(R):
        assert np.array_equal(outs[d], bits(full[d * seg:(d + 1) * seg])), d
        # the chain's first rank sends its bare partial
        first = (d + 1) % R
        part = Xf[d * seg:(d + 1) * seg, first * Kr:(first + 1) * Kr] @ Wf[first * Kr:(first + 1) * Kr]
        assert np.array_equal(sent[(first, d)], bits(part))


def test_simulated_ring_matches_direct_sum_within_rounding():
    R, M, N, K = 4, 64, 48, 32
    rng = np.random.default_rng(5)
    xs = [rand_bf16(rng, (M, K)) for _ in range(R)]
    ws = [rand_bf16(rng, (K, N), 0.1) for _ in range(R)]
    outs, _ = simulate_ring(xs, ws, R)
    seg = M // R
    exact = sum(widen(xs[r]) @ widen(ws[r]) for r in range(R))
    for d in range(R):
        ref = exact[d * seg:(d + 1) * seg]
        got = widen(outs[d])
        # R-1 bf16 roundings of running partials plus the final one, each at most
        # 2^-8 relative to a partial sum bounded by the sum of |terms|
        bound = sum(np.abs(widen(xs[r]) @ widen(ws[r]))[d * seg:(d + 1) * seg] for r in range(R))
        assert np.all(np.abs(got - ref) <= R * 2.0 ** -8 * bound + 1e-6)


def test_a_dropped_upstream_add_is_caught():
    """The exact-integer pin fails if the owner skips its upstream partial."""
    R, M, N, Kr = 3, 48, 16, 8
    rng = np.random.default_rng(9)
    Xf = rng.integers(-2, 3, size=(M, R * Kr)).astype(np.float64)
    Wf = rng.integers(-2, 3, size=(R * Kr, N)).astype(np.float64)
    xs = [bits(Xf[:, r * Kr:(r + 1) * Kr]) for r in range(R)]
    ws = [bits(Wf[r * Kr:(r + 1) * Kr]) for r in range(R)]
    seg = M // R
    zero = [np.zeros((seg, N), np.uint16) for _ in range(R)]
    out, _ = oracle.gemm_rs_ring(xs[0], ws[0], zero, R, 0)
    assert not np.array_equal(out, bits((Xf @ Wf)[:seg]))


def test_rejects_missing_upstream():
    x = np.zeros((6, 8), np.uint16)
    w = np.zeros((8, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm_rs_ring(x, w, [None, None, None], 3, 0)
