"""GPU parity of arepi_gemm_rs_fp8 (e4m3fn block-scaled GEMM + reduce-scatter
epilogue) against the CPU oracle.

bf16 outputs within |d| <= 1e-2|ref| + 1e-3 (the GPU applies the scales as a
running rescale, the oracle as the plain block sum); ready_out bit-exact;
exact-integer and all-ones cases bit-exact.
"""
import numpy as np
import pytest
import torch

import all_reduce_epilogues_amd as A
import oracle
from all_reduce_epilogues_amd import inputs
from conftest import read_golden
from gpu_util import (assert_bf16_close, device, flag_words_all_set, from_dev_bf16, from_dev_u32, to_dev_bf16,
                      to_dev_u32)

pytestmark = pytest.mark.gpu

SENTINEL_FILL = 0x7FC1


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device())


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device())


def run(case, publish=True, ftm=128, ftn=128, ready_in=None, status=None, spin_limit=0, tile=0, stream=None,
        recv_dev=None):
    dev = device()
    M, N, R, owner = case["M"], case["N"], case["R"], case["owner"]
    seg = M // R
    recv = recv_dev if recv_dev is not None else [
        None if q == owner else to_dev_bf16(case["recv"][q]) for q in range(R)]
    tiles = oracle.flag_tiles(M, N, R, ftm, ftn)
    rin_np = flag_words_all_set(R, owner, tiles) if ready_in is None else ready_in
    rin = to_dev_u32(rin_np) if not torch.is_tensor(rin_np) else rin_np
    out = torch.full((seg, N), SENTINEL_FILL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    send = torch.full((M, N), SENTINEL_FILL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    rout = torch.zeros(rin.shape, dtype=torch.int32, device=dev) if publish else None
    A.gemm_rs_fp8(dev_u8(case["x"]), dev_f32(case["xs"]), dev_u8(case["wt"]), dev_f32(case["ws"]), recv, rin, out, R,
                  owner, send=send, ready_out=rout, flag_tile_m=ftm, flag_tile_n=ftn, tile=tile, status=status,
                  spin_limit=spin_limit, stream=stream)
    torch.cuda.synchronize()
    return dict(out=from_dev_bf16(out), send=from_dev_bf16(send),
                ready_out=from_dev_u32(rout) if rout is not None else None)


def check(case, res, ftm=128, ftn=128, rows=None, what=""):
    M, N, R, owner = case["M"], case["N"], case["R"], case["owner"]
    seg = M // R
    if rows is None:
        ref_out, ref_send = oracle.gemm_rs_fp8(case["x"], case["xs"], case["wt"], case["ws"], case["recv"], R, owner)
        assert_bf16_close(res["out"], ref_out, what + " out")
        mask = np.ones(M, bool)
        mask[owner * seg:(owner + 1) * seg] = False
        assert_bf16_close(res["send"][mask], ref_send[mask], what + " send")
        assert np.all(res["send"][~mask] == SENTINEL_FILL), what + " owner rows of send were written"
    else:
        for r0, r1 in rows:
            ref_out, ref_send = oracle.gemm_rs_fp8(case["x"], case["xs"], case["wt"], case["ws"], case["recv"], R,
                                                   owner, rows=(r0, r1))
            for i in range(r0, r1):
                if owner * seg <= i < (owner + 1) * seg:
                    assert_bf16_close(res["out"][i - owner * seg], ref_out[i - owner * seg], "%s out %d" % (what, i))
                else:
                    assert_bf16_close(res["send"][i], ref_send[i], "%s send %d" % (what, i))
    if res["ready_out"] is not None:
        assert np.array_equal(res["ready_out"], oracle.ready_out(M, N, R, owner, ftm, ftn)), what + " ready_out"


@pytest.mark.parametrize("M,N,K,R,owner,ftm,ftn", [
    (256, 512, 256, 2, 0, 128, 128),   # the tiny workload's shape
    (200, 520, 384, 2, 1, 32, 64),     # ragged M tile and N tail
    (96, 264, 128, 4, 2, 24, 8),       # one K block
    (640, 384, 512, 1, 0, 128, 128),   # one rank: the plain block-scaled GEMM
    (512, 1032, 256, 8, 4, 64, 128),   # R=8, several segments per tile
])
def test_matches_oracle(M, N, K, R, owner, ftm, ftn):
    case = inputs.gemm_rs_fp8_case(M, N, K, R, owner=owner, seed=70 + M + N + K)
    print("fp8 %s" % ((M, N, K, R, owner),), flush=True)
    pub = A.gemm_rs_fp8_supports(M, N, K, R, owner, ftm, ftn, publish=True) == 0
    res = run(case, ftm=ftm, ftn=ftn, publish=pub)
    check(case, res, ftm, ftn, what="fp8 %s" % ((M, N, K, R, owner),))


def test_zero_scale_blocks_with_zero_data_add_nothing():
    """A quantiser gives an all-zero block a zero scale.  Such blocks (the
    first, a middle and the last K block of some rows; every block of one row;
    a -0.0 scale; a zero column-block scale) must add nothing, as in the
    oracle's plain sum of s_b * d_b, and leave the other blocks' sum finite."""
    M, N, K, R, owner = 512, 1032, 512, 4, 1
    case = inputs.gemm_rs_fp8_case(M, N, K, R, owner=owner, seed=81)
    x, xs, wt, ws = case["x"].copy(), case["xs"].copy(), case["wt"].copy(), case["ws"].copy()
    seg = M // R
    zero_blocks = {seg + 0: [0], seg + 5: [2], seg + 9: [3], seg + 17: [0, 1, 2, 3], 3: [1], 300: [0, 3]}
    for row, blocks in zero_blocks.items():
        for b in blocks:
            xs[row, b] = 0.0
            x[row, b * 128:(b + 1) * 128] = 0
    xs[seg + 33, 2] = -0.0
    x[seg + 33, 256:384] = 0
    ws[1, 3] = 0.0          # columns 128..255, last K block
    wt[128:256, 384:512] = 0
    ws[8, 0] = 0.0          # the ragged last column block (1024..1031), first K block
    wt[1024:1032, 0:128] = 0
    case.update(x=x, xs=xs, wt=wt, ws=ws)
    res = run(case)
    check(case, res, what="fp8 zero-scale blocks")
    out = (res["out"].astype(np.uint32) << 16).view(np.float32)
    assert np.isfinite(out).all()


def test_all_ones_two_ranks_golden():
    g = read_golden("fp8_one_encodings.txt")
    M, N, K, R = g["M"], g["N"], g["K"], g["ranks"]
    one = g["e4m3fn_one"]
    case = dict(M=M, N=N, K=K, R=R, owner=0, x=np.full((M, K), one, np.uint8),
                xs=np.ones((M, K // 128), np.float32), wt=np.full((N, K), one, np.uint8),
                ws=np.ones(((N + 127) // 128, K // 128), np.float32),
                recv=[None, np.full((M // R, N), 0x4400, np.uint16)])  # the peer's partial, 512
    res = run(case)
    assert np.all((res["out"].astype(np.uint32) << 16).view(np.float32) == g["expected_e4m3fn"])


@pytest.mark.parametrize("R,owner", [(2, 1), (4, 3)])
def test_exact_integer_k_split_linearity(R, owner):
    rng = np.random.default_rng(40 + R)
    M, N, Kr = 32 * R, 264, 128
    Xf = (rng.integers(-2, 3, size=(M, R * Kr)) * (rng.random((M, R * Kr)) < 0.25)).astype(np.float32)
    Wf = (rng.integers(-2, 3, size=(R * Kr, N)) * (rng.random((R * Kr, N)) < 0.25)).astype(np.float32)
    assert np.abs(Xf @ Wf).max() <= 256
    enc = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bits = lambda a: (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    seg = M // R
    parts = [Xf[:, q * Kr:(q + 1) * Kr] @ Wf[q * Kr:(q + 1) * Kr] for q in range(R)]
    case = dict(M=M, N=N, K=Kr, R=R, owner=owner, x=enc(Xf[:, owner * Kr:(owner + 1) * Kr] / 2),
                xs=np.full((M, 1), 2.0, np.float32), wt=enc(Wf[owner * Kr:(owner + 1) * Kr].T / 4),
                ws=np.full(((N + 127) // 128, 1), 4.0, np.float32),
                recv=[None if q == owner else bits(parts[q][owner * seg:(owner + 1) * seg]) for q in range(R)])
    res = run(case)
    assert np.array_equal(res["out"], bits((Xf @ Wf)[owner * seg:(owner + 1) * seg]))


def test_tp4_share_prestaged_and_concurrent_producer():
    case = inputs.gemm_rs_fp8_case(4096, 4096, 2048, 4, owner=0, seed=1002)
    M, N, R, owner = 4096, 4096, 4, 0
    seg = M // R
    pre = run(case)
    rows = [(0, 64), (seg - 64, seg)] + [(d * seg + o, d * seg + o + 8) for d in range(1, R) for o in (0, 509)]
    check(case, pre, rows=rows, what="fp8 tp4")
    dev = device()
    tiles = oracle.flag_tiles(M, N, R, 128, 128)
    order = torch.from_numpy(inputs.producer_order(R, owner, tiles, 77)).to(dev)
    src = [None if q == owner else to_dev_bf16(case["recv"][q]) for q in range(R)]
    recv = [None if q == owner else torch.zeros_like(src[q]) for q in range(R)]
    rin = torch.zeros((R, A.gemm_rs_flag_words(M, N, R)), dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    resident = torch.zeros(2, dtype=torch.int32, device=device())
    A.emu_peer_producer(src, recv, rin, order, R, owner, M, N, resident=resident, stream=side)
    A.emu_producer_gate(resident, status=status, stream=torch.cuda.current_stream())
    conc = run(case, ready_in=rin, recv_dev=recv, status=status, tile=A.TILE_CONSUME_READY,
               stream=torch.cuda.current_stream())
    assert int(status.item()) == 0
    assert np.array_equal(conc["out"], pre["out"]) and np.array_equal(conc["send"], pre["send"])
    assert not from_dev_u32(rin).any(), "consumed bits must be cleared"


@pytest.mark.parametrize("M,owner", [(256, 0), (1024, 6)])
def test_tp8_shapes(M, owner):
    """The tp=8 wide shape (N=7168, K=2048, eight ranks) in the fp8 form."""
    case = inputs.gemm_rs_fp8_case(M, 7168, 2048, 8, owner=owner, seed=1003)
    R, seg = 8, M // 8
    res = run(case)
    rows = [(owner * seg, (owner + 1) * seg)]
    rows += [(d * seg, d * seg + min(8, seg)) for d in range(R) if d != owner]
    check(case, res, rows=rows, what="fp8 tp8 M=%d" % M)
