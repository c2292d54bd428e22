"""GPU parity of the Lamport AR + RMSNorm path against the CPU oracle.

Bit-exact: armed staging is all 0x8000; after publication staging equals the
canonicalised sources; after consumption staging is all 0x8000 again.
Tolerance: the normalised output, |d| <= 1e-2|ref| + 1e-3.
"""
import numpy as np
import pytest
import torch

import all_reduce_epilogues_amd as A
import oracle
from all_reduce_epilogues_amd import inputs
from gpu_util import assert_bf16_close, device, from_dev_bf16, to_dev_bf16

pytestmark = pytest.mark.gpu


def armed(S, M, N):
    st = torch.empty((S, M, N), dtype=torch.bfloat16, device=device())
    A.lamport_prefill(st)
    return st


def publish_and_consume(case, sequential=True, status=None):
    S, M, N = case["S"], case["M"], case["N"]
    dev = device()
    src = to_dev_bf16(case["src"])
    gamma = to_dev_bf16(case["gamma"])
    order = torch.from_numpy(case["order"]).to(dev)
    st = armed(S, M, N)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    if sequential:
        A.lamport_publish(src, st, order, case["tile_m"], case["tile_n"])
        torch.cuda.synchronize()
        published = from_dev_bf16(st)
        A.ar_rmsnorm_lamport(st, gamma, out, case["eps"], status=status)
    else:
        # Streams are spread over a few hardware queues, and two streams can
        # share one, which runs its work in submission order: the publisher is
        # submitted first so that a shared queue serialises the pair instead of
        # leaving the consumer to wait for work queued behind it.  On separate
        # queues the consumer starts while the publisher is still landing tiles.
        side = torch.cuda.Stream()
        published = None
        A.lamport_publish(src, st, order, case["tile_m"], case["tile_n"], stream=side)
        A.ar_rmsnorm_lamport(st, gamma, out, case["eps"], status=status)
    torch.cuda.synchronize()
    return dict(out=from_dev_bf16(out), staging=from_dev_bf16(st), published=published)


def test_prefill_arms_every_word():
    st = torch.zeros(1000003, dtype=torch.bfloat16, device=device())
    A.lamport_prefill(st)
    torch.cuda.synchronize()
    assert np.all(from_dev_bf16(st) == oracle.SENTINEL_BF16)


@pytest.mark.parametrize("S,M,N,tile", [(8, 64, 7168, 128), (3, 5, 1000, 128), (1, 1, 8, 128),
                                        (8, 3, 16384, 64), (5, 33, 2056, 32)])
def test_publish_consume_matches_oracle(S, M, N, tile):
    case = inputs.lamport_case(S, M, N, seed=40 + S + M, tile_m=tile, tile_n=tile)
    res = publish_and_consume(case)
    assert np.array_equal(res["published"], oracle.lamport_canon(case["src"])), "publication bits"
    assert np.all(res["staging"] == oracle.SENTINEL_BF16), "consumer must re-arm every pack"
    assert_bf16_close(res["out"], oracle.ar_rmsnorm(case["src"], case["gamma"], case["eps"]), "rmsnorm")


def test_sentinel_words_in_the_data_are_canonicalised():
    case = inputs.lamport_case(8, 16, 1024, seed=77)
    src = case["src"].copy()
    rng = np.random.default_rng(3)
    idx = rng.integers(0, src.size, size=5000)
    src.reshape(-1)[idx] = 0x8000          # -0.0 produced by a peer
    src.reshape(-1)[idx[:50] + 1] = 0x8001  # smallest negative subnormal stays as is
    case["src"] = src
    status = torch.zeros(1, dtype=torch.int32, device=device())
    res = publish_and_consume(case, status=status)
    assert int(status.item()) == 0
    assert not np.any(res["published"] == 0x8000)
    assert np.array_equal(res["published"], oracle.lamport_canon(src))
    assert_bf16_close(res["out"], oracle.ar_rmsnorm(src, case["gamma"], case["eps"]), "rmsnorm")


def test_concurrent_publication_gives_identical_bits():
    case = inputs.lamport_case(8, 1024, 7168, seed=91)  # publication outlasts the consumer's start
    seq = publish_and_consume(case)
    status = torch.zeros(1, dtype=torch.int32, device=device())
    conc = publish_and_consume(case, sequential=False, status=status)
    assert int(status.item()) == 0
    assert np.array_equal(seq["out"], conc["out"])
    assert np.all(conc["staging"] == oracle.SENTINEL_BF16)


def test_unpublished_staging_times_out_and_finishes():
    dev = device()
    st = armed(2, 4, 64)
    gamma = torch.ones(64, dtype=torch.bfloat16, device=dev)
    out = torch.empty((4, 64), dtype=torch.bfloat16, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    A.ar_rmsnorm_lamport(st, gamma, out, status=status, spin_limit=200)
    torch.cuda.synchronize()
    assert int(status.item()) & A.STATUS_TIMEOUT


def test_repeated_iterations_stay_armed_and_identical():
    case = inputs.lamport_case(8, 64, 7168, seed=5)
    dev = device()
    src = to_dev_bf16(case["src"])
    gamma = to_dev_bf16(case["gamma"])
    order = torch.from_numpy(case["order"]).to(dev)
    st = armed(8, 64, 7168)
    out = torch.empty((64, 7168), dtype=torch.bfloat16, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    first = None
    for it in range(200):
        A.lamport_publish(src, st, order)
        A.ar_rmsnorm_lamport(st, gamma, out, status=status)
        if it in (0, 199):
            got = from_dev_bf16(out)
            first = got if first is None else first
            assert np.array_equal(got, first)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.all(from_dev_bf16(st) == oracle.SENTINEL_BF16)


def test_full_workload_matches_oracle():
    case = inputs.lamport_case()  # 8 x [4096, 7168]
    res = publish_and_consume(case)
    assert np.all(res["staging"] == oracle.SENTINEL_BF16)
    assert_bf16_close(res["out"], oracle.ar_rmsnorm(case["src"], case["gamma"], case["eps"]), "full rmsnorm")
