"""Pins for the Lamport sentinel, canonicalisation and AR + RMSNorm oracle (CPU only)."""
import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden


def widen(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_bf16_bits(a):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_sentinel_is_negative_zero():
    g = read_golden("lamport_sentinel.txt")
    assert oracle.SENTINEL_BF16 == g["sentinel_bf16"]
    assert np.float32(-0.0).view(np.uint32) == g["sentinel_f32"]
    assert to_bf16_bits(np.array([-0.0]))[0] == g["sentinel_bf16"]
    assert np.all(oracle.lamport_arm(1000) == g["sentinel_bf16"])


def test_canonicalisation_over_every_pattern():
    g = read_golden("lamport_sentinel.txt")
    allp = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    c = oracle.lamport_canon(allp)
    changed = np.nonzero(c != allp)[0]
    assert list(changed) == [g["sentinel_bf16"]]
    assert c[g["sentinel_bf16"]] == g["canonical_zero_bf16"]
    assert not np.any(c == g["sentinel_bf16"])


def reference_rmsnorm_f64(src, gamma, eps):
    s = widen(src).sum(axis=0)  # slot sum in float64 (sign of zero irrelevant)
    ms = np.mean(s * s, axis=-1, keepdims=True)
    return s / np.sqrt(ms + eps) * widen(gamma)


def test_ar_rmsnorm_matches_float64_textbook():
    rng = np.random.default_rng(11)
    S, M, N = 8, 12, 7168
    src = to_bf16_bits(rng.standard_normal((S, M, N)))
    gamma = to_bf16_bits(1.0 + 0.1 * rng.standard_normal(N))
    out = oracle.ar_rmsnorm(src, gamma, 1e-6)
    ref = reference_rmsnorm_f64(src, gamma, 1e-6)
    got = widen(out)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) * 1.01 + 1e-6)
    assert np.mean(out == to_bf16_bits(ref)) > 0.97


def test_ar_rmsnorm_matches_torch_rms_norm():
    rng = np.random.default_rng(12)
    S, M, N = 4, 9, 1024
    src = to_bf16_bits(rng.standard_normal((S, M, N)))
    gamma = to_bf16_bits(1.0 + 0.1 * rng.standard_normal(N))
    s = torch.from_numpy(widen(src).sum(axis=0))
    y = torch.nn.functional.rms_norm(s, [N], weight=torch.from_numpy(widen(gamma)), eps=1e-6)
    got = widen(oracle.ar_rmsnorm(src, gamma, 1e-6))
    assert np.allclose(got, y.numpy(), rtol=1e-2, atol=1e-3)


@pytest.mark.parametrize("c", [0.0625, 0.5, 1.0, 3.0, -2.0, 100.0])
def test_constant_row_normalises_to_unit(c):
    N = 512
    src = to_bf16_bits(np.full((1, 2, N), c))
    gamma = to_bf16_bits(np.ones(N))
    out = oracle.ar_rmsnorm(src, gamma, 1e-6)
    assert np.all(widen(out) == np.sign(c))


def test_sentinel_words_count_as_positive_zero():
    rng = np.random.default_rng(13)
    S, M, N = 3, 4, 256
    src = to_bf16_bits(rng.standard_normal((S, M, N)))
    src[:, :, ::7] = 0x8000
    clean = src.copy()
    clean[clean == 0x8000] = 0x0000
    gamma = to_bf16_bits(np.ones(N))
    assert np.array_equal(oracle.ar_rmsnorm(src, gamma, 1e-6), oracle.ar_rmsnorm(clean, gamma, 1e-6))


def test_row_bands_compose():
    rng = np.random.default_rng(14)
    src = to_bf16_bits(rng.standard_normal((2, 10, 64)))
    gamma = to_bf16_bits(np.ones(64))
    full = oracle.ar_rmsnorm(src, gamma, 1e-6)
    part = oracle.ar_rmsnorm(src, gamma, 1e-6, rows=(3, 7))
    assert np.array_equal(part[3:7], full[3:7]) and not part[:3].any() and not part[7:].any()
