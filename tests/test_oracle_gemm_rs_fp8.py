"""Pins for the fp8 block-scaled GEMM + reduce-scatter oracle (CPU only).

  * the e4m3fn decoding equals torch's float8_e4m3fn for all 256 codes;
  * the block-scaled product equals a float64 product of the dequantised
    operands (X~[m,k] = dec(x)*xs[m,k/128], W~[n,k] = dec(wt)*ws[n/128,k/128]),
    with scales that differ per K block, per row and per 128-column block, so
    a swapped or shifted scale index fails;
  * doubling one row's scales doubles that row exactly;
  * the all-ones two-rank example of the pages (1024; 4096 from e4m3fnuz bytes);
  * exact-integer K-split linearity of the epilogue, bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden


def widen(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dec_table():
    return np.array([oracle.fp8_e4m3fn_to_f32(c) for c in range(256)], dtype=np.float64)


def test_decode_matches_torch_for_every_code():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    got = dec_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def rand_fp8(rng, shape, scale=1.0):
    v = torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32))
    return v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def dequant(x, xs, wt, ws):
    t = dec_table()
    M, K = x.shape
    N = wt.shape[0]
    xd = t[x] * np.repeat(xs.astype(np.float64), 128, axis=1)
    wsr = np.repeat(np.repeat(ws.astype(np.float64), 128, axis=0)[:N], 128, axis=1)
    wd = t[wt] * wsr
    return xd, wd


@pytest.mark.parametrize("M,N,K", [(64, 200, 256), (40, 384, 512)])
def test_block_scaled_product_equals_dequantised_float64(M, N, K):
    rng = np.random.default_rng(M + N)
    x, wt = rand_fp8(rng, (M, K), 2.0), rand_fp8(rng, (N, K), 2.0)
    xs = rng.uniform(0.01, 0.1, size=(M, K // 128)).astype(np.float32)
    ws = rng.uniform(0.01, 0.1, size=((N + 127) // 128, K // 128)).astype(np.float32)
    out, _ = oracle.gemm_rs_fp8(x, xs, wt, ws, [None], 1, 0)
    xd, wd = dequant(x, xs, wt, ws)
    c64 = xd @ wd.T
    bound = np.abs(xd) @ np.abs(wd).T * (K + 2 * (K // 128) + 4) * 2.0 ** -24
    got = widen(out)
    assert np.all(np.abs(got - c64) <= 2.0 ** -8 * np.abs(c64) + bound)
    # the same with the scale of the second K block moved to the first fails
    xs2 = xs.copy()
    xs2[:, [0, 1]] = xs2[:, [1, 0]]
    bad = widen(oracle.gemm_rs_fp8(x, xs2, wt, ws, [None], 1, 0)[0])
    assert np.any(np.abs(bad - c64) > 2.0 ** -8 * np.abs(c64) + bound)


def test_row_scale_is_linear():
    rng = np.random.default_rng(3)
    M, N, K = 16, 136, 256
    x, wt = rand_fp8(rng, (M, K)), rand_fp8(rng, (N, K))
    xs = rng.uniform(0.5, 1.0, size=(M, K // 128)).astype(np.float32)
    ws = rng.uniform(0.5, 1.0, size=((N + 127) // 128, K // 128)).astype(np.float32)
    a, _ = oracle.gemm_rs_fp8(x, xs, wt, ws, [None], 1, 0)
    xs2 = xs.copy()
    xs2[5] *= 2
    b, _ = oracle.gemm_rs_fp8(x, xs2, wt, ws, [None], 1, 0)
    assert np.array_equal(widen(b[5]), 2 * widen(a[5]))
    assert np.array_equal(np.delete(a, 5, 0), np.delete(b, 5, 0))


def test_all_ones_two_ranks_and_the_fnuz_bytes():
    g = read_golden("fp8_one_encodings.txt")
    M, N, K = 64, 128, g["K"]  # the value does not depend on M or N
    for byte, expect in ((g["e4m3fn_one"], g["expected_e4m3fn"]), (g["e4m3fnuz_one"], g["result_of_fnuz_bytes"])):
        x = np.full((M, K), byte, np.uint8)
        wt = np.full((N, K), byte, np.uint8)
        xs = np.ones((M, K // 128), np.float32)
        ws = np.ones((1, K // 128), np.float32)
        # the peer's partial is what the same operands give on that rank
        peer_val = expect / g["ranks"]
        peer = np.full((M // 2, N), np.float32(peer_val).view(np.uint32) >> 16, np.uint16)
        out, _ = oracle.gemm_rs_fp8(x, xs, wt, ws, [None, peer], 2, 0)
        assert np.all(widen(out) == expect), (hex(byte), np.unique(widen(out)))


@pytest.mark.parametrize("R,owner", [(2, 1), (4, 0), (4, 3)])
def test_exact_integer_k_split_linearity(R, owner):
    # small integers halved / quartered are exact in e4m3fn; power-of-two scales undo that exactly
    rng = np.random.default_rng(20 + R)
    M, N, Kr = 16 * R, 136, 128
    Xf = (rng.integers(-2, 3, size=(M, R * Kr)) * (rng.random((M, R * Kr)) < 0.25)).astype(np.float32)
    Wf = (rng.integers(-2, 3, size=(R * Kr, N)) * (rng.random((R * Kr, N)) < 0.25)).astype(np.float32)
    # every partial and total is an integer of magnitude <= 256: exact in bf16
    assert max(np.abs(Xf @ Wf).max(), max(np.abs(Xf[:, p * Kr:(p + 1) * Kr] @ Wf[p * Kr:(p + 1) * Kr]).max()
                                          for p in range(R))) <= 256
    enc = lambda a: torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    seg = M // R
    bits = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    parts = [Xf[:, p * Kr:(p + 1) * Kr] @ Wf[p * Kr:(p + 1) * Kr] for p in range(R)]
    x = enc(np.ascontiguousarray(Xf[:, owner * Kr:(owner + 1) * Kr] / 2))
    wt = enc(np.ascontiguousarray(Wf[owner * Kr:(owner + 1) * Kr].T / 4))
    xs = np.full((M, 1), 2.0, np.float32)
    ws = np.full(((N + 127) // 128, 1), 4.0, np.float32)
    recv = [None if p == owner else bits(parts[p][owner * seg:(owner + 1) * seg]) for p in range(R)]
    out, send = oracle.gemm_rs_fp8(x, xs, wt, ws, recv, R, owner)
    assert np.array_equal(out, bits((Xf @ Wf)[owner * seg:(owner + 1) * seg]))
    mask = np.ones(M, bool)
    mask[owner * seg:(owner + 1) * seg] = False
    assert np.array_equal(send[mask], bits(parts[owner])[mask])
