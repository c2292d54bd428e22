"""GPU parity of arepi_gemm_rs_fused against the CPU oracle.

Inputs come from the seeded generators; expected values only from oracle/.
bf16 outputs within |d| <= 1e-2|ref| + 1e-3; ready_out bit-exact; ready_in
unchanged; owner rows of `send` untouched.
"""
import numpy as np
import pytest
import torch

import all_reduce_epilogues_amd as A
import oracle
from all_reduce_epilogues_amd import inputs
from conftest import read_golden
from gpu_util import (assert_bf16_close, device, flag_words_all_set, from_dev_bf16, from_dev_u32,
                      to_dev_bf16, to_dev_u32)

pytestmark = pytest.mark.gpu

SENTINEL_FILL = 0x7FC1  # a NaN pattern no correct output produces


def run(case, tile=A.TILE_AUTO, publish=True, ftm=128, ftn=128, stream=None, status=None, spin_limit=0,
        ready_in=None, want_send=True):
    dev = device()
    M, N, R, owner = case["M"], case["N"], case["R"], case["owner"]
    seg = M // R
    x = to_dev_bf16(case["x"])
    w = to_dev_bf16(case["w"])
    recv = [None if p == owner else to_dev_bf16(case["recv"][p]) for p in range(R)]
    tiles = oracle.flag_tiles(M, N, R, ftm, ftn)
    rin_np = flag_words_all_set(R, owner, tiles) if ready_in is None else ready_in
    rin = to_dev_u32(rin_np)
    out = torch.full((seg, N), 0, dtype=torch.int16, device=dev).fill_(SENTINEL_FILL).view(torch.bfloat16)
    send = None
    if want_send:
        send = torch.full((M, N), SENTINEL_FILL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    rout = torch.zeros(rin.shape, dtype=torch.int32, device=dev) if (publish and want_send) else None
    A.gemm_rs_fused(x, w, recv, rin, out, R, owner, send=send, ready_out=rout, flag_tile_m=ftm,
                    flag_tile_n=ftn, tile=tile, status=status, spin_limit=spin_limit, stream=stream)
    torch.cuda.synchronize()
    res = dict(out=from_dev_bf16(out), send=from_dev_bf16(send) if send is not None else None,
               ready_out=from_dev_u32(rout) if rout is not None else None, ready_in=from_dev_u32(rin))
    assert np.array_equal(res["ready_in"], rin_np), "ready_in must be read-only"
    return res


def check_against_oracle(case, res, ftm=128, ftn=128, rows=None, what="", ref=None):
    M, N, R, owner = case["M"], case["N"], case["R"], case["owner"]
    seg = M // R
    if rows is None:
        ref_out, ref_send = ref if ref is not None else oracle.gemm_rs(case["x"], case["w"], case["recv"], R, owner)
        assert_bf16_close(res["out"], ref_out, what + " out")
        if res["send"] is not None:
            mask = np.ones(M, bool)
            mask[owner * seg:(owner + 1) * seg] = False
            assert_bf16_close(res["send"][mask], ref_send[mask], what + " send")
            assert np.all(res["send"][~mask] == SENTINEL_FILL), what + " owner rows of send were written"
    else:
        for r0, r1 in rows:
            ref_out, ref_send = oracle.gemm_rs(case["x"], case["w"], case["recv"], R, owner, rows=(r0, r1))
            for i in range(r0, r1):
                if owner * seg <= i < (owner + 1) * seg:
                    li = i - owner * seg
                    assert_bf16_close(res["out"][li], ref_out[li], "%s out row %d" % (what, i))
                elif res["send"] is not None:
                    assert_bf16_close(res["send"][i], ref_send[i], "%s send row %d" % (what, i))
    if res["ready_out"] is not None:
        assert np.array_equal(res["ready_out"], oracle.ready_out(M, N, R, owner, ftm, ftn)), what + " ready_out"


def tiles_to_try(case, ftm, ftn):
    """Every tile, and its paired-half-blocks form where that is a different row layout."""
    for base in sorted(A.TILE_NAMES):
        variants = [base]
        if A.TILE_DIMS[base][0] >= 64:
            variants.append(base | A.TILE_PAIRED_ROWS)
        for t in variants:
            pub = A.gemm_rs_supports(case["M"], case["N"], case["K"], case["R"], case["owner"], ftm, ftn,
                                     publish=True, tile=t) == 0
            yield t, pub


def tile_name(t):
    base = t & 0xff
    return A.TILE_NAMES.get(base, "auto") + ("/paired" if t & A.TILE_PAIRED_ROWS else "") + \
        ("/owner-half" if t & A.TILE_OWNER_HALF else "")


@pytest.mark.parametrize("owner", [0, 1])
def test_tiny_workload_every_tile(owner):
    case = inputs.workload_gemm_rs(1, owner=owner)
    for tile, pub in tiles_to_try(case, 128, 128):
        print("tiny workload owner=%d tile=%s publish=%s" % (owner, tile_name(tile), pub), flush=True)
        res = run(case, tile=tile, publish=pub)
        check_against_oracle(case, res, what="tiny/%s" % tile_name(tile))


@pytest.mark.parametrize("M,N,K,R,owner,ftm,ftn", [
    (200, 520, 200, 2, 1, 32, 64),    # ragged M tile, N and K tails
    (96, 72, 8, 4, 2, 24, 8),         # K smaller than one k-step
    (24, 8, 16, 8, 7, 3, 8),          # one pack wide, 3-row segments
    (192, 264, 136, 3, 1, 64, 8),     # R=3
    (640, 384, 328, 1, 0, 128, 128),  # R=1: a plain GEMM
    (520, 1032, 72, 8, 4, 128, 128),  # 65-row segments straddling every tile
])
def test_ragged_shapes_every_tile(M, N, K, R, owner, ftm, ftn):
    case = inputs.gemm_rs_case(M, N, K, R, owner=owner, seed=7 + M + N + K)
    for tile, pub in tiles_to_try(case, ftm, ftn):
        print("ragged %s tile=%s publish=%s" % ((M, N, K, R, owner), tile_name(tile), pub), flush=True)
        res = run(case, tile=tile, publish=pub, ftm=ftm, ftn=ftn)
        check_against_oracle(case, res, ftm, ftn, what="ragged/%s" % tile_name(tile))


@pytest.mark.parametrize("M,N,K,R,owner,ftm,ftn", [
    (512, 520, 136, 4, 1, 64, 64),     # half-blocks of 128 / 64 rows, N tail
    (384, 264, 72, 3, 2, 128, 8),      # R=3: one non-owner half-block left unpaired
    (640, 1032, 200, 5, 3, 64, 128),   # R=5: pure, single and owner-paired blocks
    (2048, 7168, 256, 8, 5, 128, 128), # R=8 at the model width
])
def test_paired_half_blocks_every_tile(M, N, K, R, owner, ftm, ftn):
    case = inputs.gemm_rs_case(M, N, K, R, owner=owner, seed=11 + M + N + K)
    ref = oracle.gemm_rs(case["x"], case["w"], case["recv"], R, owner)
    for tile, pub in tiles_to_try(case, ftm, ftn):
        print("paired %s tile=%s publish=%s" % ((M, N, K, R, owner), tile_name(tile), pub), flush=True)
        res = run(case, tile=tile, publish=pub, ftm=ftm, ftn=ftn)
        check_against_oracle(case, res, ftm, ftn, what="paired/%s" % tile_name(tile), ref=ref)


@pytest.mark.parametrize("M,N,K,R,owner,ftm,ftn", [
    (200, 520, 200, 2, 1, 32, 64),       # ragged M tile, N and K tails
    (520, 1032, 72, 8, 4, 128, 128),     # segments straddling every tile
    (4096, 7168, 256, 8, 3, 128, 128),   # several rounds of workgroups at the model width
])
def test_owner_first_order_every_tile(M, N, K, R, owner, ftm, ftn):
    """AREPI_TILE_OWNER_FIRST changes only the order of the workgroups."""
    case = inputs.gemm_rs_case(M, N, K, R, owner=owner, seed=13 + M + N + K)
    ref = oracle.gemm_rs(case["x"], case["w"], case["recv"], R, owner)
    for base in [A.TILE_AUTO] + sorted(A.TILE_NAMES):
        tile = base | A.TILE_OWNER_FIRST
        pub = A.gemm_rs_supports(M, N, K, R, owner, ftm, ftn, publish=True, tile=tile) == 0
        print("owner-first %s tile=%s publish=%s" % ((M, N, K, R, owner), tile_name(base), pub), flush=True)
        res = run(case, tile=tile, publish=pub, ftm=ftm, ftn=ftn)
        check_against_oracle(case, res, ftm, ftn, what="owner-first/%s" % tile_name(base), ref=ref)


@pytest.mark.parametrize("M,N,K,R,owner", [
    (512, 520, 136, 2, 1),      # N tail, K tail, one 256-row segment
    (2048, 1032, 200, 8, 7),    # last segment owns, N tail
    (4096, 7168, 256, 8, 3),    # two rounds of workgroups at the model width
    (384, 520, 72, 3, 2),       # R=3, 128-row segments: the 128x256 tile's 64-row owner tiles
    (1024, 7168, 256, 8, 5),    # the tp=8 M=1024 shape
])
def test_owner_half_tiles(M, N, K, R, owner):
    """AREPI_TILE_OWNER_HALF: the owner rows as half-height workgroups after
    the others, the same arithmetic per element."""
    case = inputs.gemm_rs_case(M, N, K, R, owner=owner, seed=17 + M + N + K)
    ref = oracle.gemm_rs(case["x"], case["w"], case["recv"], R, owner)
    for tile in (A.TILE_256x256_W8_K64 | A.TILE_OWNER_HALF, A.TILE_128x256 | A.TILE_OWNER_HALF,
                 A.TILE_AUTO | A.TILE_OWNER_HALF):
        if A.gemm_rs_supports(M, N, K, R, owner, publish=True, tile=tile) != 0:
            continue  # AUTO picks another tile for this shape
        print("owner-half %s tile=%s" % ((M, N, K, R, owner), tile_name(tile)), flush=True)
        res = run(case, tile=tile, publish=True)
        check_against_oracle(case, res, what="owner-half %#x" % tile, ref=ref)


def test_golden_all_ones_two_ranks_on_gpu():
    g = read_golden("gemm_ar_all_ones.txt")
    M, N, K, R = g["M"], g["N"], g["K"], g["ranks"]
    ones = np.full((M, K), 0x3F80, np.uint16)
    case = dict(M=M, N=N, K=K, R=R, owner=0, x=ones, w=np.full((K, N), 0x3F80, np.uint16),
                recv=[None, np.full((M // R, N), 0x4400, np.uint16)])  # peer partial = 512
    res = run(case)
    assert np.all(res["out"] == g["expected_output_bf16"])


def test_golden_rank_plus_one_on_gpu():
    g = read_golden("self_test_rank_plus_one.txt")
    for R, expect in zip(g["world_sizes"], g["expected"]):
        owner = R - 1
        K = 8 * (owner + 1)  # local partial = K/8 * 8 ones... = owner + 1 via w = 1/8
        M, N = 16 * R, 64
        x = np.full((M, K), 0x3F80, np.uint16)                 # 1.0
        w = np.full((K, N), 0x3E00, np.uint16)                 # 0.125
        recv = [None if p == owner else
                np.full((M // R, N), np.float32(p + 1).view(np.uint32) >> 16, np.uint16) for p in range(R)]
        res = run(dict(M=M, N=N, K=K, R=R, owner=owner, x=x, w=w, recv=recv))
        vals = (res["out"].astype(np.uint32) << 16).view(np.float32)
        assert np.all(vals == expect), (R, np.unique(vals))


@pytest.mark.parametrize("R,owner", [(2, 0), (4, 3), (8, 5)])
def test_exact_integer_linearity_on_gpu(R, owner):
    rng = np.random.default_rng(500 + R)
    M, N, Kr = 64 * R, 136, 16
    Xf = rng.integers(-2, 3, size=(M, R * Kr))
    Wf = rng.integers(-2, 3, size=(R * Kr, N))
    seg = M // R

    def bits(a):
        return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)

    parts = [Xf[:, p * Kr:(p + 1) * Kr] @ Wf[p * Kr:(p + 1) * Kr] for p in range(R)]
    case = dict(M=M, N=N, K=Kr, R=R, owner=owner, x=bits(Xf[:, owner * Kr:(owner + 1) * Kr]),
                w=bits(Wf[owner * Kr:(owner + 1) * Kr]),
                recv=[None if p == owner else bits(parts[p][owner * seg:(owner + 1) * seg]) for p in range(R)])
    res = run(case)
    assert np.array_equal(res["out"], bits((Xf @ Wf)[owner * seg:(owner + 1) * seg]))


def test_tp4_workload_prestaged_and_concurrent_producer():
    case = inputs.workload_gemm_rs(2)
    M, N, R, owner = case["M"], case["N"], case["R"], case["owner"]
    seg = M // R
    pre = run(case)
    # owner segment in full, send rows sampled from every segment
    rows = [(0, seg)] + [(d * seg + o, d * seg + o + 16) for d in range(1, R) for o in (0, 509, seg - 16)]
    check_against_oracle(case, pre, rows=rows, what="tp4 prestaged")
    rerun = run(case)
    assert np.array_equal(pre["out"], rerun["out"]) and np.array_equal(pre["send"], rerun["send"])

    # concurrent: an emulated-peer producer on a second stream lands the peer
    # partials in a shuffled tile order while the GEMM runs
    dev = device()
    tiles = oracle.flag_tiles(M, N, R, 128, 128)
    for seed, groups, per_release in ((11, 0, 1), (12, 0, 1), (13, 24, 1), (14, 0, 8), (15, 16, 4)):
        order = torch.from_numpy(inputs.producer_order(R, owner, tiles, seed)).to(dev)
        src = [None if p == owner else to_dev_bf16(case["recv"][p]) for p in range(R)]
        recv = [None if p == owner else torch.zeros_like(src[p]) for p in range(R)]
        rin = torch.zeros((R, A.gemm_rs_flag_words(M, N, R)), dtype=torch.int32, device=dev)
        out = torch.empty((seg, N), dtype=torch.bfloat16, device=dev)
        send = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        rout = torch.zeros_like(rin)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        x, w = to_dev_bf16(case["x"]), to_dev_bf16(case["w"])
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        main = torch.cuda.current_stream()
        resident = torch.zeros(2, dtype=torch.int32, device=dev)
        A.emu_peer_producer(src, recv, rin, order, R, owner, M, N, workgroups=groups,
                            items_per_release=per_release, resident=resident, stream=side)
        A.emu_producer_gate(resident, status=status, stream=main)
        A.gemm_rs_fused(x, w, recv, rin, out, R, owner, send=send, ready_out=rout, status=status, stream=main)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "a readiness wait timed out"
        assert np.array_equal(from_dev_bf16(out), pre["out"]), "result depends on arrival order"
        assert np.array_equal(from_dev_u32(rin), flag_words_all_set(R, owner, tiles))


@pytest.mark.parametrize("M", [1024, 4096])
def test_owner_half_tiles_with_a_concurrent_producer(M):
    """tp=8 shapes where the automatic choice runs the owner rows as
    half-height tiles: the peers' partials land tile by tile in a shuffled
    order while the GEMM runs, so the half-height owner workgroups really
    wait; the result equals the pre-staged one bit for bit."""
    case = inputs.workload_gemm_rs(3, M=M, owner=3)
    N, R, owner = case["N"], case["R"], case["owner"]
    seg = M // R
    assert any(wg[0] == -1 for wg in A.gemm_rs_schedule(M, N, case["K"], R, owner, publish=True))
    pre = run(case)
    dev = device()
    tiles = oracle.flag_tiles(M, N, R, 128, 128)
    order = torch.from_numpy(inputs.producer_order(R, owner, tiles, 70 + M)).to(dev)
    src = [None if p == owner else to_dev_bf16(case["recv"][p]) for p in range(R)]
    recv = [None if p == owner else torch.zeros_like(src[p]) for p in range(R)]
    rin = torch.zeros((R, A.gemm_rs_flag_words(M, N, R)), dtype=torch.int32, device=dev)
    out = torch.empty((seg, N), dtype=torch.bfloat16, device=dev)
    send = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    rout = torch.zeros_like(rin)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    resident = torch.zeros(2, dtype=torch.int32, device=dev)
    x, w = to_dev_bf16(case["x"]), to_dev_bf16(case["w"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    print("owner-half tp=8 M=%d, concurrent producer" % M, flush=True)
    A.emu_peer_producer(src, recv, rin, order, R, owner, M, N, workgroups=48, items_per_release=4,
                        resident=resident, stream=side)
    A.emu_producer_gate(resident, status=status, stream=main)
    A.gemm_rs_fused(x, w, recv, rin, out, R, owner, send=send, ready_out=rout, status=status, stream=main)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "a readiness wait timed out"
    assert np.array_equal(from_dev_bf16(out), pre["out"])
    assert np.array_equal(from_dev_u32(rout), oracle.ready_out(M, N, R, owner, 128, 128))


def test_gate_lets_the_producer_finish_beside_a_register_full_gemm():
    """The 4-wave 256x256 tile at R = 4 allocates all 512 registers per SIMD
    lane, so no producer wave fits beside it on a compute unit.  The gate,
    queued between the producer and the GEMM, holds the GEMM back until every
    producer workgroup has started; the producer never waits, so every
    owner-tile wait is met and the result equals the pre-staged one.  The gate
    leaves resident at zero for the next step."""
    case = inputs.workload_gemm_rs(2)
    M, N, R, owner = case["M"], case["N"], case["R"], case["owner"]
    seg = M // R
    dev = device()
    pre = run(case, tile=A.TILE_256x256)
    tiles = oracle.flag_tiles(M, N, R, 128, 128)
    x, w = to_dev_bf16(case["x"]), to_dev_bf16(case["w"])
    src = [None if p == owner else to_dev_bf16(case["recv"][p]) for p in range(R)]
    resident = torch.zeros(2, dtype=torch.int32, device=dev)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    for seed, groups in ((21, 16), (22, 0)):
        print("gate seed %d workgroups %d" % (seed, groups), flush=True)
        order = torch.from_numpy(inputs.producer_order(R, owner, tiles, seed)).to(dev)
        recv = [None if p == owner else torch.zeros_like(src[p]) for p in range(R)]
        rin = torch.zeros((R, A.gemm_rs_flag_words(M, N, R)), dtype=torch.int32, device=dev)
        out = torch.empty((seg, N), dtype=torch.bfloat16, device=dev)
        send = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        rout = torch.zeros_like(rin)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        A.emu_peer_producer(src, recv, rin, order, R, owner, M, N, workgroups=groups, resident=resident,
                            stream=side)
        A.emu_producer_gate(resident, status=status, stream=main)
        A.gemm_rs_fused(x, w, recv, rin, out, R, owner, send=send, ready_out=rout, tile=A.TILE_256x256,
                        status=status, stream=main)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "a wait timed out"
        assert np.array_equal(from_dev_bf16(out), pre["out"])
        assert not resident.any().item(), "the gate must leave resident at zero"


def test_one_producer_launch_feeds_consecutive_calls():
    """One multi-step producer launch, on a stream with a hardware queue of its
    own, lands the peers of four consecutive GEMM-RS calls (step s once the
    call before has signalled its end); each call consumes its bits.  Every
    call equals the pre-staged result, and ready_in and resident end zero."""
    case = inputs.workload_gemm_rs(2)
    M, N, R, owner = case["M"], case["N"], case["R"], case["owner"]
    seg = M // R
    dev = device()
    pre = run(case)
    tiles = oracle.flag_tiles(M, N, R, 128, 128)
    orders = torch.from_numpy(np.stack([inputs.producer_order(R, owner, tiles, 40 + i) for i in range(3)])).to(dev)
    x, w = to_dev_bf16(case["x"]), to_dev_bf16(case["w"])
    src = [None if p == owner else to_dev_bf16(case["recv"][p]) for p in range(R)]
    recv = [None if p == owner else torch.zeros_like(src[p]) for p in range(R)]
    rin = torch.zeros((R, A.gemm_rs_flag_words(M, N, R)), dtype=torch.int32, device=dev)
    rout = torch.zeros_like(rin)
    send = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    outs = [torch.empty((seg, N), dtype=torch.bfloat16, device=dev) for _ in range(4)]
    go = torch.zeros(1, dtype=torch.int32, device=dev)
    resident = torch.zeros(2, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    # the producer's stream synchronises with the legacy default stream (it is
    # a blocking stream), so the consumer runs on a non-blocking one
    side = A.emu_stream()
    main = torch.cuda.Stream()
    torch.cuda.synchronize()
    print("multi-step producer, 4 steps", flush=True)
    A.emu_peer_producer_steps(src, recv, rin, orders, R, owner, M, N, go, 4, workgroups=96, items_per_release=8,
                              resident=resident, status=status, stream=side)
    A.emu_producer_gate(resident, status=status, stream=main)
    for s in range(4):
        A.gemm_rs_fused(x, w, recv, rin, outs[s], R, owner, send=send, ready_out=rout,
                        tile=A.TILE_CONSUME_READY, status=status, stream=main)
        A.emu_signal(go, s + 1, stream=main)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "a wait timed out"
    for s in range(4):
        assert np.array_equal(from_dev_bf16(outs[s]), pre["out"]), "call %d" % s
    assert not rin.any().item() and not resident.any().item()
    assert int(go.item()) == 4


def test_credit_producer_feeds_consecutive_calls_with_changing_partials():
    """Credits instead of signals: the producer lands step s's partials into a
    slot as soon as the call before has consumed its bit (the owner tiles
    clear a bit only after reading the data under it), with no signal between
    the calls.  The steps alternate between two different sets of partials,
    so a slot refilled before the call before had read it would show up as
    the other set's data in that call's output.  Every call equals the
    pre-staged result of its set; ready_in and resident end zero."""
    case = inputs.workload_gemm_rs(2)
    M, N, K, R, owner = case["M"], case["N"], case["K"], case["R"], case["owner"]
    seg = M // R
    dev = device()
    other = inputs.gemm_rs_case(M, N, K, R, owner=owner, seed=4242)
    case_b = dict(case, recv=other["recv"])
    pre = [run(case)["out"], run(case_b)["out"]]
    assert not np.array_equal(pre[0], pre[1])
    tiles = oracle.flag_tiles(M, N, R, 128, 128)
    orders = torch.from_numpy(np.stack([inputs.producer_order(R, owner, tiles, 60 + i) for i in range(2)])).to(dev)
    x, w = to_dev_bf16(case["x"]), to_dev_bf16(case["w"])
    src = [None if p == owner else torch.stack([to_dev_bf16(case["recv"][p]), to_dev_bf16(other["recv"][p])])
           for p in range(R)]
    recv = [None if p == owner else torch.zeros((seg, N), dtype=torch.bfloat16, device=dev) for p in range(R)]
    rin = torch.zeros((R, A.gemm_rs_flag_words(M, N, R)), dtype=torch.int32, device=dev)
    rout = torch.zeros_like(rin)
    send = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    steps = 6
    outs = [torch.empty((seg, N), dtype=torch.bfloat16, device=dev) for _ in range(steps)]
    resident = torch.zeros(2, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    count = torch.zeros(1, dtype=torch.int32, device=dev)
    side = A.emu_stream()
    main = torch.cuda.Stream()
    torch.cuda.synchronize()
    print("credit producer, %d steps, two alternating sets" % steps, flush=True)
    A.emu_peer_producer_steps(src, recv, rin, orders, R, owner, M, N, count, steps, workgroups=96,
                              items_per_release=8, resident=resident, status=status, stream=side, credit=True)
    A.emu_producer_gate(resident, status=status, stream=main)
    for s in range(steps):
        A.gemm_rs_fused(x, w, recv, rin, outs[s], R, owner, send=send, ready_out=rout,
                        tile=A.TILE_CONSUME_READY, status=status, stream=main)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "a wait timed out"
    for s in range(steps):
        assert np.array_equal(from_dev_bf16(outs[s]), pre[s % 2]), "call %d" % s
    assert not rin.any().item() and not resident.any().item()
    assert int(count.item()) == 96 * steps


def test_credit_producer_gives_up_on_unconsumed_bits():
    """Every bit is still set (nothing consumed it): each batch's bounded wait
    for its credit gives up, the producer reports the time-out and finishes
    without touching recv."""
    case = inputs.workload_gemm_rs(1)
    M, N, R, owner = case["M"], case["N"], case["R"], case["owner"]
    dev = device()
    tiles = oracle.flag_tiles(M, N, R, 128, 128)
    orders = torch.from_numpy(np.stack([inputs.producer_order(R, owner, tiles, 51)])).to(dev)
    src = [None if p == owner else to_dev_bf16(case["recv"][p]) for p in range(R)]
    recv = [None if p == owner else torch.zeros_like(src[p]) for p in range(R)]
    full = flag_words_all_set(R, owner, tiles)
    rin = to_dev_u32(full)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    count = torch.zeros(1, dtype=torch.int32, device=dev)
    A.emu_peer_producer_steps(src, recv, rin, orders, R, owner, M, N, count, 2, status=status, spin_limit=2000,
                              stream=A.emu_stream(), credit=True)
    torch.cuda.synchronize()
    assert int(status.item()) & A.STATUS_TIMEOUT
    assert np.array_equal(from_dev_u32(rin), full)
    for p in range(R):
        if p != owner:
            assert not recv[p].view(torch.int16).any().item()


def test_multi_step_producer_gives_up_when_no_signal_comes():
    """Step 0 lands at once; step 1 waits for a signal the host never sends:
    the producer's bounded wait gives up, reports the time-out and the kernel
    finishes, with step 0's bits set."""
    case = inputs.workload_gemm_rs(1)
    M, N, R, owner = case["M"], case["N"], case["R"], case["owner"]
    dev = device()
    tiles = oracle.flag_tiles(M, N, R, 128, 128)
    orders = torch.from_numpy(np.stack([inputs.producer_order(R, owner, tiles, 50)])).to(dev)
    src = [None if p == owner else to_dev_bf16(case["recv"][p]) for p in range(R)]
    recv = [None if p == owner else torch.zeros_like(src[p]) for p in range(R)]
    rin = torch.zeros((R, A.gemm_rs_flag_words(M, N, R)), dtype=torch.int32, device=dev)
    go = torch.zeros(1, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    A.emu_peer_producer_steps(src, recv, rin, orders, R, owner, M, N, go, 2, status=status, spin_limit=2000,
                              stream=A.emu_stream())
    torch.cuda.synchronize()
    assert int(status.item()) & A.STATUS_TIMEOUT
    assert np.array_equal(from_dev_u32(rin), flag_words_all_set(R, owner, tiles))
    for p in range(R):
        if p != owner:
            assert torch.equal(recv[p], src[p])


def test_gate_times_out_when_no_producer_announces():
    """Nothing ever starts on `resident`: the gate's bounded wait gives up,
    reports the time-out and finishes."""
    dev = device()
    resident = torch.zeros(2, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    A.emu_producer_gate(resident, status=status, spin_limit=2000)
    torch.cuda.synchronize()
    assert int(status.item()) & A.STATUS_TIMEOUT


@pytest.mark.parametrize("M,owner,tile", [(256, 0, A.TILE_AUTO), (1024, 0, A.TILE_AUTO), (1024, 7, A.TILE_AUTO),
                                          (4096, 0, A.TILE_AUTO), (8192, 0, A.TILE_AUTO),
                                          (4096, 5, A.TILE_OWNER_FIRST), (8192, 0, A.TILE_OWNER_FIRST),
                                          (4096, 2, A.TILE_OWNER_HALF), (8192, 7, A.TILE_OWNER_HALF)])
def test_tp8_workload_sweep(M, owner, tile):
    case = inputs.workload_gemm_rs(3, M=M, owner=owner)
    R = 8
    seg = M // R
    res = run(case, tile=tile)
    rows = [(owner * seg, (owner + 1) * seg)]
    rows += [(d * seg, d * seg + min(8, seg)) for d in range(R) if d != owner]
    rows += [(d * seg + seg - min(8, seg), d * seg + seg) for d in range(R) if d != owner]
    check_against_oracle(case, res, rows=rows, what="tp8 M=%d tile=%#x" % (M, tile))


def test_timeout_reports_status_and_finishes():
    case = inputs.workload_gemm_rs(1)
    R, owner = case["R"], case["owner"]
    tiles = oracle.flag_tiles(case["M"], case["N"], R, 128, 128)
    rin = flag_words_all_set(R, owner, tiles)
    rin[1, 0] &= ~np.uint32(1 << 2)  # one peer tile never lands
    status = torch.zeros(1, dtype=torch.int32, device=device())
    res = run(case, ready_in=rin, status=status, spin_limit=2000)
    assert int(status.item()) & A.STATUS_TIMEOUT
    # send rows do not depend on the missing tile
    _, ref_send = oracle.gemm_rs(case["x"], case["w"], case["recv"], R, owner)
    assert_bf16_close(res["send"][128:], ref_send[128:], "send after timeout")


@pytest.mark.parametrize("M,N,K,R,owner,ftm,ftn,tile", [
    (2048, 2048, 512, 4, 0, 128, 128, A.TILE_AUTO),
    (2048, 1032, 200, 8, 7, 128, 128, A.TILE_256x256_W8_K64 | A.TILE_OWNER_HALF),
    (1024, 7168, 256, 8, 3, 128, 128, A.TILE_256x256_W8 | A.TILE_PAIRED_ROWS),
    (640, 1032, 200, 5, 3, 64, 128, A.TILE_AUTO),
    (384, 264, 72, 3, 2, 32, 8, A.TILE_128x128_S4),
])
def test_consume_ready_leaves_ready_in_clear_for_the_next_call(M, N, K, R, owner, ftm, ftn, tile):
    """With AREPI_TILE_CONSUME_READY the owner tiles clear the bits they waited
    for: two calls in a row, each fed by the emulated producer on a second
    stream, share one ready_in that nothing else clears; both match the oracle
    and ready_in ends all zero."""
    dev = device()
    case = inputs.gemm_rs_case(M, N, K, R, owner=owner, seed=900 + M + R)
    ref = oracle.gemm_rs(case["x"], case["w"], case["recv"], R, owner)
    seg = M // R
    tiles = oracle.flag_tiles(M, N, R, ftm, ftn)
    x, w = to_dev_bf16(case["x"]), to_dev_bf16(case["w"])
    src = [None if p == owner else to_dev_bf16(case["recv"][p]) for p in range(R)]
    recv = [None if p == owner else torch.zeros_like(src[p]) for p in range(R)]
    rin = torch.zeros((R, A.gemm_rs_flag_words(M, N, R, ftm, ftn)), dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    resident = torch.zeros(2, dtype=torch.int32, device=dev)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    for call, seed in enumerate((31, 32)):
        print("consume %s tile=%s call %d" % ((M, N, K, R, owner, ftm, ftn), tile_name(tile), call), flush=True)
        for p in range(R):
            if p != owner:
                recv[p].zero_()
        out = torch.full((seg, N), SENTINEL_FILL, dtype=torch.int16, device=dev).view(torch.bfloat16)
        send = torch.full((M, N), SENTINEL_FILL, dtype=torch.int16, device=dev).view(torch.bfloat16)
        rout = torch.zeros_like(rin)
        order = torch.from_numpy(inputs.producer_order(R, owner, tiles, seed)).to(dev)
        torch.cuda.synchronize()
        A.emu_peer_producer(src, recv, rin, order, R, owner, M, N, flag_tile_m=ftm, flag_tile_n=ftn,
                            workgroups=16 * call, resident=resident, stream=side)
        A.emu_producer_gate(resident, status=status, stream=main)
        A.gemm_rs_fused(x, w, recv, rin, out, R, owner, send=send, ready_out=rout, flag_tile_m=ftm,
                        flag_tile_n=ftn, tile=tile | A.TILE_CONSUME_READY, status=status, stream=main)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "a readiness wait timed out"
        assert not from_dev_u32(rin).any(), "ready_in bits left set"
        res = dict(out=from_dev_bf16(out), send=from_dev_bf16(send), ready_out=from_dev_u32(rout))
        check_against_oracle(case, res, ftm, ftn, what="consume call %d" % call, ref=ref)
