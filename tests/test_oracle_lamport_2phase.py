"""Pins for the two-phase Lamport AR + RMSNorm oracle (CPU only).

  * one rank: the reduced tensor is the canonicalised input and the result is
    the one-slot consumer's, bit for bit;
  * exact integers: when every sum is exact in bf16 the two-phase result is
    the one-shot result, bit for bit, and T is the integer sum;
  * rounding before the norm: a hand-worked row whose sum is a bf16 tie --
    T rounds to even, and the normalised output then differs from the
    one-shot path by a value worked out here in float64;
  * all -0.0 inputs reduce to +0.0, never to the sentinel;
  * random inputs: T within half a bf16 ulp of the float64 sum (plus fp32
    rounding), the output within the parity tolerance of a float64 RMSNorm of T.
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


def test_one_rank_is_the_one_slot_consumer():
    rng = np.random.default_rng(1)
    x = bits(rng.standard_normal((1, 6, 40)))
    x.reshape(-1)[::7] = 0x8000  # -0.0 inputs
    g = bits(1 + 0.1 * rng.standard_normal(40))
    t = oracle.lamport_reduce(x)
    assert np.array_equal(t, oracle.lamport_canon(x[0]))
    assert np.array_equal(oracle.ar_rmsnorm_2phase(x, g), oracle.ar_rmsnorm(x, g))


@pytest.mark.parametrize("R", [2, 3, 8])
def test_exact_integers_match_the_one_shot_path(R):
    rng = np.random.default_rng(10 + R)
    xi = rng.integers(-16, 17, size=(R, 5, 64))
    x = bits(xi)
    g = bits(1 + 0.1 * rng.standard_normal(64))
    t = oracle.lamport_reduce(x)
    tot = xi.sum(axis=0)
    assert np.array_equal(widen(t), np.where(tot == 0, 0.0, tot))  # exact, and +0.0 for zero
    assert not np.any(t == oracle.SENTINEL_BF16)
    assert np.array_equal(oracle.ar_rmsnorm_2phase(x, g), oracle.ar_rmsnorm(x, g))


def test_sum_is_rounded_before_the_norm():
    # ranks 0 and 1; row [256 + 1, 16 + 0]: 257 is a tie between 256 and 258 in
    # bf16 (spacing 2 there) and rounds to the even 256.
    x = np.zeros((2, 1, 2), np.uint16)
    x[0, 0] = bits([256.0, 16.0])
    x[1, 0] = bits([1.0, 0.0])
    g = bits([1.0, 1.0])
    t = oracle.lamport_reduce(x)
    assert np.array_equal(widen(t[0]), [256.0, 16.0])
    # float64 RMSNorm of T, then bf16: 16 / sqrt((256^2 + 16^2) / 2) = 0.08820..., which
    # rounds to 181 * 2^-11; the unrounded sum would give 16 / 182.08... = 0.08787... -> 180 * 2^-11
    two = widen(oracle.ar_rmsnorm_2phase(x, g)[0])
    one = widen(oracle.ar_rmsnorm(x, g)[0])
    assert two[1] == 181 * 2.0 ** -11
    assert one[1] == 180 * 2.0 ** -11
    ref = 256.0 / np.sqrt((256.0 ** 2 + 16.0 ** 2) / 2 + 1e-6)
    assert abs(two[0] - ref) <= 2.0 ** -7  # one bf16 ulp at 1.41


def test_negative_zeros_reduce_to_positive_zero():
    x = np.full((4, 2, 8), 0x8000, np.uint16)
    t = oracle.lamport_reduce(x)
    assert np.all(t == 0)
    x[1, 0, 3] = bits([-3.0])[0]
    x[2, 0, 3] = bits([3.0])[0]  # cancels to +0.0 under round-to-nearest
    assert oracle.lamport_reduce(x)[0, 3] == 0


def test_random_inputs_against_float64():
    rng = np.random.default_rng(7)
    R, M, N = 8, 12, 1024
    x = bits(rng.standard_normal((R, M, N)))
    g = bits(1 + 0.1 * rng.standard_normal(N))
    t = widen(oracle.lamport_reduce(x))
    s64 = widen(x).sum(axis=0)
    # fp32 accumulation of 8 terms + one bf16 rounding
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(s64), 2.0 ** -126))) - 7)
    assert np.all(np.abs(t - s64) <= 0.5 * ulp + 8 * 2.0 ** -24 * widen(x).__abs__().sum(axis=0) + 1e-30)
    y = widen(oracle.ar_rmsnorm_2phase(x, g))
    ref = t / np.sqrt((t * t).mean(axis=1, keepdims=True) + 1e-6) * widen(g)
    assert np.all(np.abs(y - ref) <= 1e-2 * np.abs(ref) + 1e-3)
    # sampled rows equal the full call
    part = oracle.ar_rmsnorm_2phase(x, g, rows=(3, 7))
    full = oracle.ar_rmsnorm_2phase(x, g)
    assert np.array_equal(part[3:7], full[3:7]) and not part[:3].any() and not part[7:].any()
