"""GPU parity of the no-allocation Lamport consumer
(arepi_ar_rmsnorm_lamport_noalloc, staging held in a static device array)
against the consumer on a caller-owned staging, called through the C ABI.

Two calls in a row, the second with fewer rows: each publishes the same
seeded partials into both stagings, and the two outputs must be identical bit
for bit (same kernel, same summation order); each is also held to the parity
tolerance against the oracle.  After each call the used part of the static
staging must be armed (all 0x8000) again, since the next call reads it.
"""
import ctypes

import numpy as np
import pytest
import torch

import all_reduce_epilogues_amd as A
import oracle
from all_reduce_epilogues_amd import inputs
from gpu_util import assert_bf16_close, device, from_dev_bf16, to_dev_bf16

pytestmark = pytest.mark.gpu


def _hip_runtime():
    """The HIP runtime this process already loaded (the one the library uses)."""
    with open("/proc/self/maps") as f:
        paths = {line.split()[-1] for line in f if "libamdhip64.so" in line}
    assert paths, "HIP runtime not loaded"
    hip = ctypes.CDLL(sorted(paths)[0])
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    hip.hipMemcpy.restype = ctypes.c_int
    return hip


def _read_words(addr, n):
    """n bf16 words at device address addr, copied to the host."""
    host = np.empty(n, dtype=np.uint16)
    rc = _hip_runtime().hipMemcpy(host.ctypes.data, addr, 2 * n, 2)  # hipMemcpyDeviceToHost
    assert rc == 0, "hipMemcpy failed: %d" % rc
    return host


def _publish_raw(src, addr, order, case):
    """arepi_lamport_publish into a raw device address."""
    rc = A.lib().arepi_lamport_publish(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(addr),
                                       ctypes.c_void_p(order.data_ptr()), case["S"], case["M"], case["N"],
                                       case["tile_m"], case["tile_n"], A.SCOPE_AGENT,
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, A.last_error()


def test_noalloc_matches_caller_staging_on_two_calls():
    dev = device()
    S, N = 8, 7168
    seen = set()
    for M, seed in ((256, 71), (40, 72)):  # the second call is smaller
        case = inputs.lamport_case(S, M, N, seed=seed)
        src = to_dev_bf16(case["src"])
        gamma = to_dev_bf16(case["gamma"])
        order = torch.from_numpy(case["order"]).to(dev)

        # existing entry point, caller-owned staging
        st = torch.empty((S, M, N), dtype=torch.bfloat16, device=dev)
        A.lamport_prefill(st)
        A.lamport_publish(src, st, order, case["tile_m"], case["tile_n"])
        ref = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        A.ar_rmsnorm_lamport(st, gamma, ref, case["eps"])

        # no-allocation entry point: set-up call (M = 0) returns the address
        empty = torch.empty((0, N), dtype=torch.bfloat16, device=dev)
        addr = A.ar_rmsnorm_lamport_noalloc(gamma, empty, S)
        torch.cuda.synchronize()
        assert addr and addr % 256 == 0
        seen.add(addr)
        _publish_raw(src, addr, order, case)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        assert A.ar_rmsnorm_lamport_noalloc(gamma, out, S, case["eps"], status=status) == addr
        torch.cuda.synchronize()

        assert int(status.item()) == 0, "no wait may time out: publication finished first"
        got, want = from_dev_bf16(out), from_dev_bf16(ref)
        assert np.array_equal(got, want), "M=%d: differs from the caller-staging consumer" % M
        assert_bf16_close(got, oracle.ar_rmsnorm(case["src"], case["gamma"], case["eps"]), "M=%d oracle" % M)
        assert np.all(_read_words(addr, S * M * N) == oracle.SENTINEL_BF16), "static staging re-armed"
    assert len(seen) == 1, "one static staging per device"


def test_noalloc_refuses_sizes_beyond_the_static_staging():
    dev = device()
    N, S = 7168, 8
    rows = A.LAMPORT_NOALLOC_BYTES // (S * N * 2)
    gamma = torch.empty(N, dtype=torch.bfloat16, device=dev)
    out = torch.empty((rows + 1, N), dtype=torch.bfloat16, device=dev)
    with pytest.raises(A.ArepiError, match="static staging"):
        A.ar_rmsnorm_lamport_noalloc(gamma, out, S)
