"""GPU parity of arepi_combine_reduce against the CPU oracle."""
import numpy as np
import pytest
import torch

import all_reduce_epilogues_amd as A
import oracle
from all_reduce_epilogues_amd import inputs
from gpu_util import assert_bf16_close, device, from_dev_bf16, to_dev_bf16

pytestmark = pytest.mark.gpu


PIPELINES = ["registers", "lds"]


def run(x_np, gate_np, pipeline="registers"):
    dev = device()
    T, E, H = x_np.shape
    x = to_dev_bf16(x_np)
    gate = torch.from_numpy(np.ascontiguousarray(gate_np, np.float32)).to(dev)
    out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=dev)
    A.combine_reduce(x, gate, out, pipeline=pipeline)
    torch.cuda.synchronize()
    return from_dev_bf16(out)


@pytest.mark.parametrize("pipeline", PIPELINES)
@pytest.mark.parametrize("T,E,H", [(1, 8, 7168), (37, 3, 520), (5, 16, 8), (64, 1, 4096), (300, 8, 1032),
                                   (2, 5, 512), (33, 12, 2056)])
def test_shapes_match_oracle(T, E, H, pipeline):
    case = inputs.combine_case(T, E, H, seed=60 + T + E)
    got = run(case["x"], case["gate"], pipeline)
    assert_bf16_close(got, oracle.combine(case["x"], case["gate"]), "combine %s %s" % (pipeline, (T, E, H)))


def test_both_pipelines_give_identical_bits():
    case = inputs.combine_case(257, 8, 7168, seed=64)
    assert np.array_equal(run(case["x"], case["gate"], "registers"), run(case["x"], case["gate"], "lds"))


def test_empty_token_batch_is_a_no_op():
    dev = device()
    x = torch.empty((0, 8, 64), dtype=torch.bfloat16, device=dev)
    g = torch.empty((0, 8), dtype=torch.float32, device=dev)
    out = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    A.combine_reduce(x, g, out)
    torch.cuda.synchronize()


def test_one_hot_gate_is_bit_exact():
    case = inputs.combine_case(96, 8, 1536, seed=61)
    rng = np.random.default_rng(0)
    pick = rng.integers(0, 8, size=96)
    gate = np.zeros((96, 8), np.float32)
    gate[np.arange(96), pick] = 1.0
    got = run(case["x"], gate)
    assert np.array_equal(got, case["x"][np.arange(96), pick])


def test_uniform_gate_over_identical_rows_is_bit_exact():
    case = inputs.combine_case(32, 8, 2048, seed=62)
    x = np.repeat(case["x"][:, :1], 8, axis=1)
    got = run(x, np.full((32, 8), 0.125, np.float32))
    assert np.array_equal(got, x[:, 0])


@pytest.mark.parametrize("pipeline", PIPELINES)
def test_full_workload_matches_oracle(pipeline):
    case = inputs.combine_case()  # [4096, 8, 7168]
    got = run(case["x"], case["gate"], pipeline)
    assert_bf16_close(got, oracle.combine(case["x"], case["gate"]), "combine full " + pipeline)
