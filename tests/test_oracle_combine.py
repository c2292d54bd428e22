"""Pins for the weighted top-k combine oracle (CPU only)."""
import numpy as np
import torch

import oracle


def widen(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_bf16_bits(a):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_one_hot_gate_selects_the_expert():
    rng = np.random.default_rng(21)
    T, E, H = 16, 8, 136
    x = to_bf16_bits(rng.standard_normal((T, E, H)))
    pick = rng.integers(0, E, size=T)
    gate = np.zeros((T, E), np.float32)
    gate[np.arange(T), pick] = 1.0
    out = oracle.combine(x, gate)
    assert np.array_equal(out, x[np.arange(T), pick])


def test_uniform_gate_over_identical_rows_is_identity():
    rng = np.random.default_rng(22)
    T, E, H = 8, 8, 64
    row = to_bf16_bits(rng.standard_normal((T, 1, H)))
    x = np.repeat(row, E, axis=1)
    gate = np.full((T, E), 1.0 / E, np.float32)
    assert np.array_equal(oracle.combine(x, gate), row[:, 0])


def test_matches_float64_brute_force():
    rng = np.random.default_rng(23)
    T, E, H = 32, 8, 96
    x = to_bf16_bits(rng.standard_normal((T, E, H)))
    gate = torch.softmax(torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32)), -1).numpy()
    out = widen(oracle.combine(x, gate))
    xw = widen(x)
    g64 = gate.astype(np.float64)
    ref = np.zeros((T, H))
    mag = np.zeros((T, H))
    for t in range(T):
        for k in range(E):
            ref[t] += g64[t, k] * xw[t, k]
            mag[t] += abs(g64[t, k] * xw[t, k])
    tol = 2.0 ** -8 * np.abs(ref) * 1.001 + 2 * E * 2.0 ** -24 * mag + 1e-30
    assert np.all(np.abs(out - ref) <= tol)


def test_scaling_the_gate_by_two_doubles_the_output_exactly():
    rng = np.random.default_rng(24)
    T, E, H = 8, 8, 64
    x = to_bf16_bits(rng.standard_normal((T, E, H)))
    gate = rng.random((T, E)).astype(np.float32)
    a = widen(oracle.combine(x, gate))
    b = widen(oracle.combine(x, gate * 2))
    assert np.array_equal(b, 2 * a)
