"""Pins for the oracle's bf16 conversions (CPU only).

Widening must be the exact 16-bit shift; narrowing must be IEEE
round-to-nearest-even, checked against torch's own fp32 -> bf16 conversion
(a library routine) on random bit patterns and against hand-worked ties.
"""
import numpy as np
import pytest
import torch

import oracle


def test_widen_is_exact_shift_for_every_pattern():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.f32_from_bf16(b)
    assert np.array_equal(f.view(np.uint32), b.astype(np.uint32) << 16)


def test_rne_matches_torch_on_random_patterns():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2**32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    # add exact ties and near-ties, which random patterns rarely hit
    hi = rng.integers(0, 2**16, size=50_000, dtype=np.uint64).astype(np.uint32) << 16
    u = np.concatenate([u, hi | 0x8000, hi | 0x7FFF, hi | 0x8001])
    f = u.view(np.float32)
    ours = oracle.bf16_from_f32(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(ours[~nan], ref[~nan])
    # NaN stays a quiet NaN with its sign
    on = ours[nan].astype(np.uint32)
    assert np.all((on & 0x7F80) == 0x7F80) and np.all((on & 0x007F) != 0)
    assert np.array_equal(on >> 15, (u[nan] >> 31))


@pytest.mark.parametrize("bits,expect", [
    (0x3F800000, 0x3F80),  # 1.0
    (0x3F808000, 0x3F80),  # 1 + 2^-8: exact tie, even neighbour kept
    (0x3F818000, 0x3F82),  # tie with odd lower neighbour rounds up
    (0x3F808001, 0x3F81),  # just above half
    (0x3F807FFF, 0x3F80),  # just below half
    (0x7F7FFFFF, 0x7F80),  # largest fp32 rounds to +inf
    (0x7F7F7FFF, 0x7F7F),  # stays finite
    (0x80000000, 0x8000),  # -0.0 keeps its sign
    (0x80000001, 0x8000),  # smallest negative subnormal rounds to -0.0
    (0x807FFFFF, 0x8080),  # largest negative subnormal rounds to -2^-126
    (0x00008000, 0x0000),  # positive subnormal tie -> 0
    (0x7F800000, 0x7F80),  # +inf
    (0xFF800000, 0xFF80),  # -inf
])
def test_rne_hand_worked_cases(bits, expect):
    f = np.array([bits], dtype=np.uint32).view(np.float32)
    assert int(oracle.bf16_from_f32(f)[0]) == expect
