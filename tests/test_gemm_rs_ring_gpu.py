"""GPU parity of arepi_gemm_rs_ring (one hop of the push-ring reduce-scatter)
against the CPU oracle's ring form.

Inputs come from the seeded generators; expected values only from oracle/.
bf16 outputs within |d| <= 1e-2|ref| + 1e-3; ready_out bit-exact; exact-integer
cases bit-exact.
"""
import numpy as np
import pytest
import torch

import all_reduce_epilogues_amd as A
import oracle
from all_reduce_epilogues_amd import inputs
from gpu_util import assert_bf16_close, device, from_dev_bf16, from_dev_u32, to_dev_bf16, to_dev_u32

pytestmark = pytest.mark.gpu

SENTINEL_FILL = 0x7FC1  # a NaN pattern no correct output produces


def chain_of(R, owner):
    return (owner + R - 1) % R


def ready_all(R, skip, tiles):
    """Every flag tile of every segment except `skip` published (built directly)."""
    W = (tiles + 31) // 32
    words = np.zeros((R, W), dtype=np.uint32)
    for d in range(R):
        if d == skip and R > 1:
            continue
        for t in range(tiles):
            words[d, t // 32] |= np.uint32(1 << (t % 32))
    return words


def run(case, tile=A.TILE_AUTO, publish=True, ftm=128, ftn=128, ready_in=None, status=None, spin_limit=0,
        stream=None):
    dev = device()
    M, N, R, owner = case["M"], case["N"], case["R"], case["owner"]
    seg = M // R
    chain = chain_of(R, owner)
    x, w = to_dev_bf16(case["x"]), to_dev_bf16(case["w"])
    up = [None if (R > 1 and d == chain) or case["up"][d] is None else to_dev_bf16(case["up"][d])
          for d in range(R)]
    tiles = oracle.flag_tiles(M, N, R, ftm, ftn)
    rin_np = ready_all(R, chain, tiles) if ready_in is None else ready_in
    rin = to_dev_u32(rin_np)
    out = torch.full((seg, N), SENTINEL_FILL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    send = torch.full((M, N), SENTINEL_FILL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    rout = torch.zeros(rin.shape, dtype=torch.int32, device=dev) if publish else None
    A.gemm_rs_ring(x, w, up, rin, out, send, R, owner, ready_out=rout, flag_tile_m=ftm, flag_tile_n=ftn,
                   tile=tile, status=status, spin_limit=spin_limit, stream=stream)
    torch.cuda.synchronize()
    res = dict(out=from_dev_bf16(out), send=from_dev_bf16(send),
               ready_out=from_dev_u32(rout) if rout is not None else None, ready_in=from_dev_u32(rin))
    assert np.array_equal(res["ready_in"], rin_np), "ready_in must be read-only"
    return res


def check(case, res, ftm=128, ftn=128, rows=None, what="", ref=None):
    M, N, R, owner = case["M"], case["N"], case["R"], case["owner"]
    seg = M // R
    if rows is None:
        ref_out, ref_send = ref if ref is not None else oracle.gemm_rs_ring(case["x"], case["w"], case["up"], R,
                                                                          owner)
        assert_bf16_close(res["out"], ref_out, what + " out")
        mask = np.ones(M, bool)
        mask[owner * seg:(owner + 1) * seg] = False
        assert_bf16_close(res["send"][mask], ref_send[mask], what + " send")
        assert np.all(res["send"][~mask] == SENTINEL_FILL), what + " owner rows of send were written"
    else:
        for r0, r1 in rows:
            ref_out, ref_send = oracle.gemm_rs_ring(case["x"], case["w"], case["up"], R, owner, rows=(r0, r1))
            for i in range(r0, r1):
                if owner * seg <= i < (owner + 1) * seg:
                    li = i - owner * seg
                    assert_bf16_close(res["out"][li], ref_out[li], "%s out row %d" % (what, i))
                else:
                    assert_bf16_close(res["send"][i], ref_send[i], "%s send row %d" % (what, i))
    if res["ready_out"] is not None:
        assert np.array_equal(res["ready_out"], oracle.ready_out(M, N, R, owner, ftm, ftn)), what + " ready_out"


def tiles_for(case, ftm, ftn):
    for t in sorted(A.TILE_NAMES):
        if A.gemm_rs_ring_supports(case["M"], case["N"], case["K"], case["R"], case["owner"], ftm, ftn,
                                   publish=False, tile=t) != 0:
            continue
        pub = A.gemm_rs_ring_supports(case["M"], case["N"], case["K"], case["R"], case["owner"], ftm, ftn,
                                      publish=True, tile=t) == 0
        yield t, pub


@pytest.mark.parametrize("owner", [0, 1])
def test_tiny_workload_every_tile(owner):
    case = inputs.gemm_rs_ring_case(256, 512, 256, 2, owner=owner, seed=1001, dist="uniform")
    ref = oracle.gemm_rs_ring(case["x"], case["w"], case["up"], 2, owner)
    for tile, pub in tiles_for(case, 128, 128):
        print("ring tiny owner=%d tile=%s publish=%s" % (owner, A.TILE_NAMES[tile], pub), flush=True)
        res = run(case, tile=tile, publish=pub)
        check(case, res, what="ring tiny/%s" % A.TILE_NAMES[tile], ref=ref)


@pytest.mark.parametrize("M,N,K,R,owner,ftm,ftn", [
    (208, 520, 200, 2, 1, 32, 64),    # ragged M tile, N and K tails
    (96, 72, 8, 4, 2, 24, 8),         # K smaller than one k-step, 24-row segments
    (192, 264, 136, 3, 0, 64, 8),     # R=3, owner 0: chain segment is the last
    (640, 384, 328, 1, 0, 128, 128),  # R=1: a plain GEMM
    (512, 1032, 72, 8, 4, 128, 128),  # 64-row segments, several per tile
    (256, 7168, 256, 8, 0, 128, 128), # 32-row segments at the model width
])
def test_ragged_shapes_every_tile(M, N, K, R, owner, ftm, ftn):
    case = inputs.gemm_rs_ring_case(M, N, K, R, owner=owner, seed=17 + M + N + K)
    ref = oracle.gemm_rs_ring(case["x"], case["w"], case["up"], R, owner)
    for tile, pub in tiles_for(case, ftm, ftn):
        print("ring ragged %s tile=%s publish=%s" % ((M, N, K, R, owner), A.TILE_NAMES[tile], pub), flush=True)
        res = run(case, tile=tile, publish=pub, ftm=ftm, ftn=ftn)
        check(case, res, ftm, ftn, what="ring ragged/%s" % A.TILE_NAMES[tile], ref=ref)


@pytest.mark.parametrize("owner", [0, 1])
def test_two_ranks_ring_is_the_direct_sum_bit_for_bit(owner):
    """With R = 2 the ring hop and the direct sum do the same arithmetic on the
    same accumulators: identical bits from the two GPU entry points on the same
    compute tile (both calls without ready_out, so the automatic choice is the
    same too).  The tiles cover the fold of the partial inside the K loop
    (two-stage tiles) and the add after it (four-stage tiles)."""
    dev = device()
    M, N, K, R = 512, 1024, 512, 2
    case = inputs.gemm_rs_ring_case(M, N, K, R, owner=owner, seed=77)
    part = case["up"][owner]
    for tile in (A.TILE_AUTO, A.TILE_128x128_S4, A.TILE_256x256_W8, A.TILE_256x256_W8_K64, A.TILE_64x128,
                 A.TILE_128x128):
        ring = run(case, tile=tile, publish=False)
        recv = [None, None]
        recv[1 - owner] = to_dev_bf16(part)
        rin = to_dev_u32(ready_all(R, owner, oracle.flag_tiles(M, N, R, 128, 128)))
        out = torch.empty((M // R, N), dtype=torch.bfloat16, device=dev)
        send = torch.full((M, N), SENTINEL_FILL, dtype=torch.int16, device=dev).view(torch.bfloat16)
        A.gemm_rs_fused(to_dev_bf16(case["x"]), to_dev_bf16(case["w"]), recv, rin, out, R, owner, send=send,
                        tile=tile)
        torch.cuda.synchronize()
        assert np.array_equal(ring["out"], from_dev_bf16(out)), A.TILE_NAMES.get(tile, "auto")
        assert np.array_equal(ring["send"], from_dev_bf16(send)), A.TILE_NAMES.get(tile, "auto")


@pytest.mark.parametrize("R", [2, 3, 4, 8])
def test_whole_ring_on_the_gpu_ends_with_the_full_product(R):
    """Every hop of a whole ring run on the GPU, the running partials handed
    from rank to rank: with small integers every partial sum is exact, so each
    owner's output must equal its rows of the full product bit for bit, and
    every hop must equal the oracle's hop bit for bit."""
    rng = np.random.default_rng(900 + R)
    M, N, Kr = 32 * R, 264, 16
    seg = M // R
    Xf = rng.integers(-2, 3, size=(M, R * Kr))
    Wf = rng.integers(-2, 3, size=(R * Kr, N))

    def bits(a):
        return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)

    xs = [bits(Xf[:, r * Kr:(r + 1) * Kr]) for r in range(R)]
    ws = [bits(Wf[r * Kr:(r + 1) * Kr]) for r in range(R)]
    full = bits(Xf @ Wf)
    zeros = np.zeros((seg, N), np.uint16)
    for d in range(R):
        carry = None
        for hop in range(1, R + 1):
            r = (d + hop) % R
            chain = chain_of(R, r)
            up = [None if dd == chain else (carry if (dd == d and carry is not None) else zeros)
                  for dd in range(R)]
            case = dict(M=M, N=N, K=Kr, R=R, owner=r, x=xs[r], w=ws[r], up=up)
            res = run(case)
            ref_out, ref_send = oracle.gemm_rs_ring(xs[r], ws[r], up, R, r, rows=(d * seg, (d + 1) * seg))
            if r == d:
                assert np.array_equal(res["out"], ref_out), (R, d)
                assert np.array_equal(res["out"], full[d * seg:(d + 1) * seg]), (R, d)
            else:
                got = res["send"][d * seg:(d + 1) * seg]
                assert np.array_equal(got, ref_send[d * seg:(d + 1) * seg]), (R, d, r)
                carry = got


def test_tp4_workload_prestaged_and_concurrent_producer():
    case = inputs.gemm_rs_ring_case(4096, 4096, 2048, 4, owner=0, seed=1002)
    M, N, R, owner = case["M"], case["N"], case["R"], case["owner"]
    seg = M // R
    chain = chain_of(R, owner)
    pre = run(case)
    rows = [(0, seg)] + [(d * seg + o, d * seg + o + 16) for d in range(1, R) for o in (0, 509, seg - 16)]
    check(case, pre, rows=rows, what="ring tp4 prestaged")
    # concurrent: the emulated producer lands every upstream partial (all
    # segments but the chain one) in a shuffled tile order while the GEMM runs
    dev = device()
    tiles = oracle.flag_tiles(M, N, R, 128, 128)
    x, w = to_dev_bf16(case["x"]), to_dev_bf16(case["w"])
    src = [None if d == chain else to_dev_bf16(case["up"][d]) for d in range(R)]
    for seed, groups in ((21, 0), (22, 24)):
        print("ring tp4 concurrent seed=%d groups=%d" % (seed, groups), flush=True)
        order = torch.from_numpy(inputs.producer_order(R, chain, tiles, seed)).to(dev)
        up = [None if d == chain else torch.zeros_like(src[d]) for d in range(R)]
        rin = torch.zeros((R, A.gemm_rs_flag_words(M, N, R)), dtype=torch.int32, device=dev)
        out = torch.empty((seg, N), dtype=torch.bfloat16, device=dev)
        send = torch.full((M, N), SENTINEL_FILL, dtype=torch.int16, device=dev).view(torch.bfloat16)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        main = torch.cuda.current_stream()
        resident = torch.zeros(2, dtype=torch.int32, device=dev)
        A.emu_peer_producer(src, up, rin, order, R, chain, M, N, workgroups=groups, resident=resident,
                            stream=side)
        A.emu_producer_gate(resident, status=status, stream=main)
        A.gemm_rs_ring(x, w, up, rin, out, send, R, owner, status=status, stream=main)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "a readiness wait timed out"
        assert np.array_equal(from_dev_bf16(out), pre["out"]), "result depends on arrival order"
        assert np.array_equal(from_dev_bf16(send), pre["send"]), "result depends on arrival order"


@pytest.mark.parametrize("M,owner", [(256, 0), (1024, 5), (8192, 0)])
def test_tp8_workload_sweep(M, owner):
    case = inputs.gemm_rs_ring_case(M, 7168, 2048, 8, owner=owner, seed=1003)
    R = 8
    seg = M // R
    res = run(case)
    rows = [(owner * seg, (owner + 1) * seg)]
    rows += [(d * seg, d * seg + min(8, seg)) for d in range(R) if d != owner]
    rows += [(d * seg + seg - min(8, seg), d * seg + seg) for d in range(R) if d != owner]
    check(case, res, rows=rows, what="ring tp8 M=%d" % M)


def test_consume_ready_leaves_ready_in_clear():
    """Two hops in a row share one ready_in that only the kernel clears."""
    dev = device()
    M, N, K, R, owner = 1024, 2048, 256, 4, 2
    case = inputs.gemm_rs_ring_case(M, N, K, R, owner=owner, seed=333)
    ref = oracle.gemm_rs_ring(case["x"], case["w"], case["up"], R, owner)
    chain = chain_of(R, owner)
    seg = M // R
    tiles = oracle.flag_tiles(M, N, R, 128, 128)
    x, w = to_dev_bf16(case["x"]), to_dev_bf16(case["w"])
    src = [None if d == chain else to_dev_bf16(case["up"][d]) for d in range(R)]
    up = [None if d == chain else torch.zeros_like(src[d]) for d in range(R)]
    rin = torch.zeros((R, A.gemm_rs_flag_words(M, N, R)), dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    for call, seed in enumerate((41, 42)):
        print("ring consume call %d" % call, flush=True)
        for d in range(R):
            if d != chain:
                up[d].zero_()
        out = torch.full((seg, N), SENTINEL_FILL, dtype=torch.int16, device=dev).view(torch.bfloat16)
        send = torch.full((M, N), SENTINEL_FILL, dtype=torch.int16, device=dev).view(torch.bfloat16)
        rout = torch.zeros_like(rin)
        order = torch.from_numpy(inputs.producer_order(R, chain, tiles, seed)).to(dev)
        torch.cuda.synchronize()
        resident = torch.zeros(2, dtype=torch.int32, device=dev)
        A.emu_peer_producer(src, up, rin, order, R, chain, M, N, workgroups=16 * call, resident=resident,
                            stream=side)
        A.emu_producer_gate(resident, status=status, stream=main)
        A.gemm_rs_ring(x, w, up, rin, out, send, R, owner, ready_out=rout, tile=A.TILE_CONSUME_READY,
                       status=status, stream=main)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "a readiness wait timed out"
        assert not from_dev_u32(rin).any(), "ready_in bits left set"
        res = dict(out=from_dev_bf16(out), send=from_dev_bf16(send), ready_out=from_dev_u32(rout))
        check(case, res, what="ring consume call %d" % call, ref=ref)


def test_one_producer_launch_feeds_consecutive_hops():
    """The push-ring hop fed by one multi-step producer launch (on a stream
    with a hardware queue of its own) over three consecutive calls, each
    consuming its bits: every call equals the pre-staged hop."""
    R, owner = 4, 1
    M, N, K = 1024, 1024, 512
    case = inputs.gemm_rs_ring_case(M, N, K, R, owner=owner, seed=88)
    chain = (owner + R - 1) % R
    dev = device()
    tile = A.TILE_256x256_W8_K64
    pre = run(case, tile=tile, publish=False)
    seg = M // R
    tiles = oracle.flag_tiles(M, N, R, 128, 128)
    orders = torch.from_numpy(np.stack([inputs.producer_order(R, chain, tiles, 60 + i) for i in range(2)])).to(dev)
    x, w = to_dev_bf16(case["x"]), to_dev_bf16(case["w"])
    src = [None if p == chain else to_dev_bf16(case["up"][p]) for p in range(R)]
    up = [None if p == chain else torch.zeros_like(src[p]) for p in range(R)]
    rin = torch.zeros((R, A.gemm_rs_flag_words(M, N, R)), dtype=torch.int32, device=dev)
    go = torch.zeros(1, dtype=torch.int32, device=dev)
    resident = torch.zeros(2, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    outs = [torch.empty((seg, N), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    send = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    main = torch.cuda.Stream()  # the producer's stream is a blocking one
    torch.cuda.synchronize()
    print("ring hop, multi-step producer", flush=True)
    A.emu_peer_producer_steps(src, up, rin, orders, R, chain, M, N, go, 3, workgroups=16, items_per_release=4,
                              resident=resident, status=status, stream=A.emu_stream())
    A.emu_producer_gate(resident, status=status, stream=main)
    for s in range(3):
        A.gemm_rs_ring(x, w, up, rin, outs[s], send, R, owner, tile=tile | A.TILE_CONSUME_READY, status=status,
                       stream=main)
        A.emu_signal(go, s + 1, stream=main)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "a wait timed out"
    for s in range(3):
        assert np.array_equal(from_dev_bf16(outs[s]), pre["out"]), "call %d" % s
    assert not rin.any().item()


def test_timeout_reports_status_and_finishes():
    M, N, K, R, owner = 256, 512, 256, 2, 0
    case = inputs.gemm_rs_ring_case(M, N, K, R, owner=owner, seed=5)
    tiles = oracle.flag_tiles(M, N, R, 128, 128)
    rin = ready_all(R, chain_of(R, owner), tiles)
    rin[owner, 0] &= ~np.uint32(1 << 2)  # one upstream tile of the owner segment never lands
    status = torch.zeros(1, dtype=torch.int32, device=device())
    res = run(case, ready_in=rin, status=status, spin_limit=2000)
    assert int(status.item()) & A.STATUS_TIMEOUT
    # the chain segment's send rows do not depend on the missing tile
    _, ref_send = oracle.gemm_rs_ring(case["x"], case["w"], case["up"], R, owner)
    assert_bf16_close(res["send"][128:], ref_send[128:], "send after timeout")
