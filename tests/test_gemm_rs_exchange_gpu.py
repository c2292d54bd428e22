"""Two ranks of the direct-form GEMM-RS exchanging through each other's
buffers on one GPU: rank r's recv[1-r] is rank (1-r)'s send rows of segment r
and rank r's ready_in row 1-r is rank (1-r)'s ready_out row r, the two calls
running at once on two streams.

With tiles of 256 rows and segments of 128, every workgroup holds owner rows
and rows of the other segment: it must publish those before it waits, or the
two ranks would each wait for the other's publication (the cycle the
readiness protocol of DeepGEMM PR #1, "Fused ring RS: per-tile bitmask +
drain-ring with owner-boundary flush", has to avoid).  Waits are bounded by a
small poll budget, so a cycle shows as a timeout status, not a hang.

Expected values come from the CPU oracle: each rank's out is its own partial
plus the peer's send rows, within the bf16 tolerance.
"""
import numpy as np
import pytest
import torch

import all_reduce_epilogues_amd as A
import oracle
from all_reduce_epilogues_amd import inputs
from gpu_util import assert_bf16_close, device, from_dev_bf16, from_dev_u32, to_dev_bf16

pytestmark = pytest.mark.gpu

SPIN = 1 << 16  # polls before a wait gives up
NAN_FILL = 0x7FC1
_streams = []


def two_streams():
    """Two streams created one after the other, once: consecutive streams get
    separate hardware queues, so the two ranks' kernels can run at once."""
    if not _streams:
        _streams.extend([torch.cuda.Stream(), torch.cuda.Stream()])
    return _streams


def exchange(M, N, K, tile, seed):
    """Runs both ranks at once; returns (status, cases, outs, sends, routs)."""
    dev = device()
    R, seg = 2, M // 2
    cases = [inputs.gemm_rs_case(M, N, K, R, owner=r, seed=seed + r) for r in range(R)]
    W = A.gemm_rs_flag_words(M, N, R)
    # flag words: rank r's ready_out rows are fl[r][W:2W] (segment 0) and
    # fl[r][2W:3W] (segment 1); the peer's ready_in is a window of the same
    # words whose row r is this rank's publication for segment (1 - r)
    fl = [torch.zeros(4 * W, dtype=torch.int32, device=dev) for _ in range(R)]
    rout = [fl[r][W:3 * W].view(R, W) for r in range(R)]
    rin = [fl[1][0:2 * W].view(R, W), fl[0][2 * W:4 * W].view(R, W)]  # row 1-r = peer's row r
    sends = [torch.full((M, N), NAN_FILL, dtype=torch.int16, device=dev).view(torch.bfloat16) for _ in range(R)]
    outs = [torch.full((seg, N), NAN_FILL, dtype=torch.int16, device=dev).view(torch.bfloat16) for _ in range(R)]
    recv = [[None, sends[1][0:seg]], [sends[0][seg:2 * seg], None]]
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    xs = [to_dev_bf16(c["x"]) for c in cases]
    ws = [to_dev_bf16(c["w"]) for c in cases]
    torch.cuda.synchronize()
    streams = two_streams()
    for r in range(R):
        A.gemm_rs_fused(xs[r], ws[r], recv[r], rin[r], outs[r], R, r, send=sends[r], ready_out=rout[r],
                        tile=tile, status=status, spin_limit=SPIN, stream=streams[r])
    torch.cuda.synchronize()
    return (int(status.item()), cases, [from_dev_bf16(o) for o in outs], [from_dev_bf16(s) for s in sends],
            [from_dev_u32(t) for t in rout])


def check(M, N, cases, outs, sends, routs):
    R, seg = 2, M // 2
    local = [oracle.gemm_rs(c["x"], c["w"], [None, None], 1, 0)[0] for c in cases]  # each rank's partial C_r
    tiles = oracle.flag_tiles(M, N, R, 128, 128)
    for r in range(R):
        q = 1 - r
        # rank r sent its partial of segment q and published every flag tile of it
        assert_bf16_close(sends[r][q * seg:(q + 1) * seg], local[r][q * seg:(q + 1) * seg], "send of rank %d" % r)
        assert np.array_equal(routs[r], oracle.ready_out(M, N, R, r, 128, 128)), "ready_out of rank %d" % r
        # and owns the sum of its partial and the peer's pushed rows
        recv = [None, None]
        recv[q] = sends[q][r * seg:(r + 1) * seg]
        ref, _ = oracle.gemm_rs(cases[r]["x"], cases[r]["w"], recv, R, r)
        assert_bf16_close(outs[r], ref, "out of rank %d" % r)
    assert tiles >= 1


def test_two_ranks_exchange_with_tiles_over_both_segments():
    # control: 512 rows (segments of 256), tile rows 256 -- no workgroup holds
    # both segments, so no ordering can cycle; if even this times out the two
    # streams did not run at once and the exchange cannot be observed
    st, cases, outs, sends, routs = exchange(512, 512, 256, A.TILE_256x256_W8_K64, seed=500)
    if st:
        pytest.skip("the two ranks' kernels did not run concurrently (streams on one hardware queue)")
    check(512, 512, cases, outs, sends, routs)
    # every workgroup holds owner rows and the other segment's rows
    for tile in (A.TILE_256x256_W8_K64, A.TILE_256x256_W8, A.TILE_256x256):
        st, cases, outs, sends, routs = exchange(256, 512, 256, tile, seed=600 + tile)
        print("tile %s status %d" % (A.TILE_NAMES[tile], st), flush=True)
        assert st == 0, "readiness wait timed out with tile %s: a wait ahead of a publication" % A.TILE_NAMES[tile]
        check(256, 512, cases, outs, sends, routs)
    # the control again, after the mixed ones
    st, cases, outs, sends, routs = exchange(512, 512, 256, A.TILE_256x256_W8_K64, seed=501)
    assert st == 0


def test_two_ranks_exchange_paired_half_blocks():
    # paired rows pair each owner half-block with a half-block of the other
    # segment in one workgroup
    st, cases, outs, sends, routs = exchange(512, 512, 256, A.TILE_256x256_W8_K64 | A.TILE_PAIRED_ROWS, seed=700)
    assert st == 0, "readiness wait timed out in the paired layout"
    check(512, 512, cases, outs, sends, routs)
