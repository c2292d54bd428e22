"""Pins for the GEMM + reduce-scatter epilogue oracle (CPU only).

Each test fixes the oracle to something other than itself:
  * R = 1 reduces to a plain GEMM: compared with a float64 matmul;
  * exact-integer linearity: the owner segment must equal the full product
    X_full . W_full of the K-split operands, bit for bit;
  * brute force on tiny dyadic inputs, where every fp32 step is exact, against a
    Fraction triple loop;
  * the pages' two closed-form examples (tests/golden).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden


def widen(b):
    """bf16 bits -> float64 (independent of the oracle's own conversion)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_bf16_bits(a):
    """float -> bf16 bits through torch (used for exactly representable values
    or as an independent RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def rand_bf16(rng, shape, scale=1.0):
    return to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * scale)


def test_r1_equals_plain_gemm():
    rng = np.random.default_rng(1)
    M, N, K = 48, 80, 384
    x = rand_bf16(rng, (M, K))
    w = rand_bf16(rng, (K, N), 0.05)
    out, send = oracle.gemm_rs(x, w, [None], R=1, owner=0)
    ref = widen(x) @ widen(w)
    bound = np.abs(widen(x)) @ np.abs(widen(w))
    got = widen(out)
    # fp32 sum error (K * 2^-24 * sum|x||w|) plus one bf16 rounding (2^-8 relative)
    tol = 2.0 ** -8 * np.abs(ref) * 1.001 + 1.01 * K * 2.0 ** -24 * bound + 1e-30
    assert np.all(np.abs(got - ref) <= tol)
    # and almost every element is the correctly rounded exact product
    exact = to_bf16_bits(ref.astype(np.float32))
    assert np.mean(out == exact) > 0.98
    # R = 1 has no non-owner rows: send is untouched
    assert not send.any()


def test_transposed_operand_would_fail():
    """The R=1 pin is sensitive to operand orientation (teeth for the check above)."""
    rng = np.random.default_rng(2)
    M = N = K = 64
    x = rand_bf16(rng, (M, K))
    w = rand_bf16(rng, (K, N))
    out, _ = oracle.gemm_rs(x, w, [None], R=1, owner=0)
    wrong = widen(x) @ widen(w).T
    assert np.max(np.abs(widen(out) - wrong)) > 1.0


@pytest.mark.parametrize("R,owner", [(2, 0), (2, 1), (4, 0), (4, 2), (4, 3), (8, 0), (8, 7)])
def test_exact_integer_linearity(R, owner):
    rng = np.random.default_rng(100 + 10 * R + owner)
    M, N, Kr = 8 * R, 24, 16
    # integer entries in [-2, 2]: every partial |.| <= 64 and every total <= 256,
    # all exact in bf16 and in fp32
    Xf = rng.integers(-2, 3, size=(M, R * Kr))
    Wf = rng.integers(-2, 3, size=(R * Kr, N))
    seg = M // R
    parts = [Xf[:, p * Kr:(p + 1) * Kr] @ Wf[p * Kr:(p + 1) * Kr, :] for p in range(R)]
    recv = [None if p == owner else to_bf16_bits(parts[p][owner * seg:(owner + 1) * seg])
            for p in range(R)]
    x = to_bf16_bits(Xf[:, owner * Kr:(owner + 1) * Kr])
    w = to_bf16_bits(Wf[owner * Kr:(owner + 1) * Kr, :])
    out, send = oracle.gemm_rs(x, w, recv, R=R, owner=owner)
    full = Xf @ Wf
    assert np.array_equal(out, to_bf16_bits(full[owner * seg:(owner + 1) * seg]))
    # non-owner rows carry this rank's own partial; owner rows of send untouched
    mask = np.ones(M, dtype=bool)
    mask[owner * seg:(owner + 1) * seg] = False
    assert np.array_equal(send[mask], to_bf16_bits(parts[owner][mask]))
    assert not send[~mask].any()


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny_dyadic(seed):
    rng = np.random.default_rng(seed)
    R = int(rng.integers(1, 4))
    owner = int(rng.integers(0, R))
    seg = int(rng.integers(1, 4))
    M, N, K = R * seg, int(rng.integers(1, 9)), int(rng.integers(1, 9))
    # values k/16 with |k| <= 32: products are multiples of 2^-8 below 4, sums of
    # at most 8 of them plus 3 peers stay far inside fp32's 24 bits -> exact
    xs = rng.integers(-32, 33, size=(M, K))
    ws = rng.integers(-32, 33, size=(K, N))
    rs = [rng.integers(-32, 33, size=(seg, N)) for _ in range(R)]
    x = to_bf16_bits(xs / 16.0)
    w = to_bf16_bits(ws / 16.0)
    recv = [None if p == owner else to_bf16_bits(rs[p] / 16.0) for p in range(R)]
    out, send = oracle.gemm_rs(x, w, recv, R=R, owner=owner)
    for i in range(M):
        for n in range(N):
            acc = sum(Fraction(int(xs[i, k]), 16) * Fraction(int(ws[k, n]), 16) for k in range(K))
            d = i // seg
            if d == owner:
                li = i - owner * seg
                tot = acc + sum(Fraction(int(rs[p][li, n]), 16) for p in range(R) if p != owner)
                assert out[li, n] == to_bf16_bits(np.array([float(tot)]))[0], (i, n)
            else:
                assert send[i, n] == to_bf16_bits(np.array([float(acc)]))[0], (i, n)


@pytest.mark.parametrize("owner", [0, 1])
def test_golden_all_ones_two_ranks(owner):
    g = read_golden("gemm_ar_all_ones.txt")
    M, N, K, R = g["M"], g["N"], g["K"], g["ranks"]
    one = to_bf16_bits(np.array([g["operand_value"]]))[0]
    x = np.full((M, K), one, dtype=np.uint16)
    w = np.full((K, N), one, dtype=np.uint16)
    # the peer's partial is its own all-ones product, K everywhere
    peer = to_bf16_bits(np.full((M // R, N), float(K)))
    recv = [None if p == owner else peer for p in range(R)]
    out, _ = oracle.gemm_rs(x, w, recv, R=R, owner=owner, want_send=False)
    assert np.all(out == g["expected_output_bf16"])
    assert np.all(widen(out) == g["expected_output"])


def test_golden_rank_plus_one_closed_form():
    g = read_golden("self_test_rank_plus_one.txt")
    for R, expect in zip(g["world_sizes"], g["expected"]):
        for owner in range(R):
            M, N, K = 4 * R, 8, owner + 1
            # local partial = K = owner + 1 everywhere; peer p's partial = p + 1
            x = to_bf16_bits(np.ones((M, K)))
            w = to_bf16_bits(np.ones((K, N)))
            recv = [None if p == owner else to_bf16_bits(np.full((M // R, N), p + 1.0))
                    for p in range(R)]
            out, _ = oracle.gemm_rs(x, w, recv, R=R, owner=owner, want_send=False)
            assert np.all(widen(out) == expect), (R, owner)


def test_row_bands_compose_to_full():
    rng = np.random.default_rng(5)
    R, owner, M, N, K = 4, 2, 64, 40, 96
    x = rand_bf16(rng, (M, K))
    w = rand_bf16(rng, (K, N), 0.1)
    recv = [None if p == owner else rand_bf16(rng, (M // R, N), 0.5) for p in range(R)]
    out, send = oracle.gemm_rs(x, w, recv, R=R, owner=owner)
    out2 = np.zeros_like(out)
    send2 = np.zeros_like(send)
    for r0 in range(0, M, 24):
        o, s = oracle.gemm_rs(x, w, recv, R=R, owner=owner, rows=(r0, min(M, r0 + 24)))
        out2 |= o
        send2 |= s
    assert np.array_equal(out, out2) and np.array_equal(send, send2)


def _order_case(A_hi, A_lo, peers, R, owner):
    """Local partial A = A_hi + A_lo (K=2, exact), peers given as floats."""
    M, N = R, 1
    x = to_bf16_bits(np.ones((M, 2)))
    w = to_bf16_bits(np.array([[A_hi], [A_lo]]))
    recv = [None if p == owner else to_bf16_bits(np.array([[peers[p]]])) for p in range(R)]
    out, _ = oracle.gemm_rs(x, w, recv, R=R, owner=owner, want_send=False)
    return int(out[0, 0])


def test_sum_is_sequential_not_grouped():
    """Local partial 1 + 2^-8 (a bf16 tie) plus two peers of 2^-24: adding them
    one at a time rounds back to the tie (-> 0x3F80); summing the peers first
    would step one fp32 ulp past it (-> 0x3F81)."""
    assert _order_case(1.0, 2.0 ** -8, [0.0, 2.0 ** -24, 2.0 ** -24], R=3, owner=0) == 0x3F80


def test_peers_are_added_in_ascending_rank():
    """Local partial 1 + 3*2^-8 (a bf16 tie that rounds up).  Adding rank 0's
    -2^-23 and then rank 2's +2^-24 lands back on the tie (-> 0x3F82); the
    reverse order ends one fp32 ulp below it (-> 0x3F81)."""
    assert _order_case(1.0, 3 * 2.0 ** -8, [-(2.0 ** -23), 0.0, 2.0 ** -24], R=3, owner=1) == 0x3F82


def test_rejects_bad_arguments():
    x = np.zeros((6, 4), np.uint16)
    w = np.zeros((4, 4), np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm_rs(x, w, [None] * 4, R=4, owner=0)  # 6 rows do not split 4 ways
    with pytest.raises(ValueError):
        oracle.gemm_rs(x, np.zeros((5, 4), np.uint16), [None, None], R=2, owner=0)
