"""GPU parity of the two-phase Lamport AR + RMSNorm (arepi_ar_rmsnorm_lamport_2phase)
against the CPU oracle.

The peers' phase A is emulated on the same GPU (arepi_emu_lamport_phase_a),
always submitted before the call it feeds.  Checks: out within
|d| <= 1e-2|ref| + 1e-3 of the oracle; every other rank's staging holds the
oracle's reduced tensor bit for bit (phase A); this rank's staging is all
0x8000 again (re-armed).
"""
import numpy as np
import pytest
import torch

import all_reduce_epilogues_amd as A
import oracle
from all_reduce_epilogues_amd import inputs
from gpu_util import assert_bf16_close, device, from_dev_bf16, to_dev_bf16

pytestmark = pytest.mark.gpu


def setup(x, gamma):
    R, M, N = x.shape
    ins = [to_dev_bf16(x[r]) for r in range(R)]
    stg = [torch.empty((M, N), dtype=torch.bfloat16, device=device()) for _ in range(R)]
    for s in stg:
        A.lamport_prefill(s)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=device())
    return ins, stg, to_dev_bf16(gamma), out


def run(x, gamma, rank, eps=1e-6, concurrent=False, status=None, spin_limit=0, peers=True):
    R = x.shape[0]
    ins, stg, g, out = setup(x, gamma)
    torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream() if concurrent else main
    if peers:
        for d in range(R):
            if d != rank:
                A.emu_lamport_phase_a(ins, stg, d, stream=side)
    if not concurrent:
        torch.cuda.synchronize()
    A.ar_rmsnorm_lamport_2phase(ins, stg, g, out, rank, eps, status=status, spin_limit=spin_limit, stream=main)
    torch.cuda.synchronize()
    return from_dev_bf16(out), [from_dev_bf16(s) for s in stg]


def check(x, gamma, rank, out, stg, eps=1e-6, what=""):
    t = oracle.lamport_reduce(x)
    assert_bf16_close(out, oracle.ar_rmsnorm_2phase(x, gamma, eps), what + " out")
    assert np.all(stg[rank] == oracle.SENTINEL_BF16), what + " staging of this rank not re-armed"
    for d in range(x.shape[0]):
        if d != rank:
            assert np.array_equal(stg[d], t), what + " staging[%d] != reduced tensor" % d


@pytest.mark.parametrize("R,M,N,rank", [
    (1, 3, 64, 0),        # one rank: reduce is the identity
    (2, 5, 1000, 1),      # parts split rows; N not a multiple of the pack block
    (3, 7, 2056, 1),      # R that does not divide the pack count
    (8, 64, 7168, 5),     # model width
    (4, 33, 16384, 0),    # widest row, 8 packs per thread
    (8, 1, 8, 7),         # one pack in all: seven ranks own empty parts
])
def test_matches_oracle(R, M, N, rank):
    case = inputs.lamport_case(R, M, N, seed=300 + R + M)
    x, gamma = case["src"], case["gamma"]
    print("2phase R=%d M=%d N=%d rank=%d" % (R, M, N, rank), flush=True)
    out, stg = run(x, gamma, rank)
    check(x, gamma, rank, out, stg, what="2phase %s" % ((R, M, N, rank),))


def test_sentinel_inputs_and_exact_sums():
    """-0.0 everywhere in some elements (they must reduce to +0.0, never to
    the sentinel) and small integers (exact sums: the result equals the
    one-shot oracle's)."""
    rng = np.random.default_rng(5)
    R, M, N = 4, 16, 1024
    xi = rng.integers(-8, 9, size=(R, M, N)).astype(np.float32)
    x = (xi.view(np.uint32) >> 16).astype(np.uint16)
    x[:, :, ::17] = 0x8000
    gamma = inputs.lamport_case(1, 1, N, seed=6)["gamma"]
    out, stg = run(x, gamma, rank=2)
    check(x, gamma, 2, out, stg, what="integers")
    assert not np.any(stg[0] == 0x8000)
    assert_bf16_close(out, oracle.ar_rmsnorm(x, gamma), "vs one-shot")


def test_concurrent_peers_give_identical_bits():
    case = inputs.lamport_case(8, 512, 7168, seed=31)
    x, gamma = case["src"], case["gamma"]
    seq, _ = run(x, gamma, rank=3)
    status = torch.zeros(1, dtype=torch.int32, device=device())
    conc, stg = run(x, gamma, rank=3, concurrent=True, status=status)
    assert int(status.item()) == 0
    assert np.array_equal(seq, conc)
    assert np.all(stg[3] == oracle.SENTINEL_BF16)


def test_repeated_calls_stay_armed_and_identical():
    case = inputs.lamport_case(8, 128, 7168, seed=41)
    x, gamma = case["src"], case["gamma"]
    ins, stg, g, out = setup(x, gamma)
    status = torch.zeros(1, dtype=torch.int32, device=device())
    first = None
    for it in range(50):
        for d in range(1, 8):
            A.emu_lamport_phase_a(ins, stg, d)
        A.ar_rmsnorm_lamport_2phase(ins, stg, g, out, 0, status=status)
        if it in (0, 49):
            got = from_dev_bf16(out)
            first = got if first is None else first
            assert np.array_equal(got, first)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.all(from_dev_bf16(stg[0]) == oracle.SENTINEL_BF16)
    assert_bf16_close(first, oracle.ar_rmsnorm_2phase(x, gamma), "after 50 calls")


def test_full_workload_matches_oracle():
    case = inputs.lamport_case()  # 8 x [4096, 7168]
    x, gamma = case["src"], case["gamma"]
    out, stg = run(x, gamma, rank=0)
    check(x, gamma, 0, out, stg, what="full")


def test_missing_peers_time_out_and_finish():
    case = inputs.lamport_case(4, 8, 256, seed=51)
    status = torch.zeros(1, dtype=torch.int32, device=device())
    out, stg = run(case["src"], case["gamma"], rank=1, status=status, spin_limit=200, peers=False)
    assert int(status.item()) & A.STATUS_TIMEOUT
    assert np.all(stg[1] == oracle.SENTINEL_BF16), "every pack is re-armed even after a timeout"
