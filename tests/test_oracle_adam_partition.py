"""Pins of the oracle's optimiser step, bf16 refresh and stage partition."""
import os

import numpy as np
import pytest
import torch

from oracle import adam as A
from oracle import partition as PT

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(11)


# ---------------------------------------------------------------- Adam
def test_adam_first_step_closed_form():
    """From zero state, t = 1: mhat = g and vhat = g^2, so theta1 = theta0 - lr g/(|g| + eps)."""
    th = rng.standard_normal(1000).astype(np.float32)
    g = (rng.standard_normal(1000) * 10.0 ** rng.uniform(-6, 1, 1000)).astype(np.float32)
    m = np.zeros_like(th); v = np.zeros_like(th)
    t0 = th.copy()
    A.adam_update(th, g, m, v, 1, lr=1e-3)
    expect = t0.astype(np.float64) - 1e-3 * g / (np.abs(g.astype(np.float64)) + 1e-8)
    np.testing.assert_allclose(th, expect, rtol=0, atol=4 * np.spacing(np.abs(t0)).max())
    # (1 - b1) is formed in fp64 from the float32 b1 and rounded once
    np.testing.assert_array_equal(m, np.float32(1.0 - float(np.float32(0.9))) * g)


def test_adam_matches_torch_optimizer_over_steps():
    th = rng.standard_normal(512).astype(np.float32)
    m = np.zeros_like(th); v = np.zeros_like(th)
    p = torch.nn.Parameter(torch.tensor(th.astype(np.float64)))
    opt = torch.optim.Adam([p], lr=1e-3, betas=(0.9, 0.999), eps=1e-8)
    for t in range(1, 6):
        g = rng.standard_normal(512).astype(np.float32)
        A.adam_update(th, g, m, v, t, lr=1e-3)
        p.grad = torch.tensor(g.astype(np.float64))
        opt.step()
        np.testing.assert_allclose(th, p.detach().numpy(), rtol=0, atol=2e-6)


def test_adam_zero_gradient_keeps_parameter_at_step_one():
    th = rng.standard_normal(16).astype(np.float32)
    t0 = th.copy()
    A.adam_update(th, np.zeros_like(th), np.zeros_like(th), np.zeros_like(th), 1)
    np.testing.assert_array_equal(th, t0)


def test_bf16_round_matches_torch_rne():
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 3.4e38, -3.4e38, 1e-40, np.inf, -np.inf,
                                  1.00390625, 1.01171875, 1.0 + 2 ** -8 + 2 ** -20], np.float32)])
    ours = A.bf16_round(x)
    ref = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    nan = A.bf16_round(np.array([np.nan], np.float32))
    assert np.isnan(A.bf16_to_f32(nan))[0]


# ---------------------------------------------------------------- partition
def _golden_partition():
    d = {}
    for line in open(os.path.join(GOLDEN, "partition_12layer.txt")):
        if line.strip() and not line.startswith("#"):
            k, *vals = line.split()
            d[k] = [int(v) for v in vals]
    return d


@pytest.mark.parametrize("n_gpus", [1, 2, 4, 8])
def test_partition_user_guide_example(n_gpus):
    g = _golden_partition()
    L = g["L"][0]
    lf, lb, tmax, J = PT.partition_bruteforce(g["t_f"], g["t_b"], [1] * L, [1] * L, 100, n_gpus, 4)
    assert lf == g["forward_stage_lengths"]
    assert lb == g["backward_stage_lengths"]
    assert tmax == g["t_max"][0]
    assert J == (4 * 16 + n_gpus * (n_gpus - 1)) * 3


def test_partition_memory_cap_forces_short_stages():
    # equal times, memory 5 per layer, cap 10: at most two layers per stage in either pass
    lf, lb, tmax, J = PT.partition_bruteforce([1] * 6, [1] * 6, [5] * 6, [5] * 6, 10, 2, 1)
    assert max(lf) <= 2 and max(lb) <= 2
    assert PT.partition_bruteforce([1] * 3, [1] * 3, [5, 11, 5], [5, 5, 5], 10, 1, 1) is None


def test_partition_single_layer_and_objective_by_hand():
    assert PT.partition_bruteforce([7], [9], [1], [1], 5, 1, 3) == ([1], [1], 9, 3 * 2 * 9)
    # two layers, N=1, M=1, t_f = (1, 2), t_b = (2, 3). By hand:
    #   f[2] b[2]: S=2, t=5 -> 10;  f[2] b[1,1]: S=3, t=3 -> 9;  f[1,1] b[1,1]: S=4, t=3 -> 12
    lf, lb, tmax, J = PT.partition_bruteforce([1, 2], [2, 3], [1, 1], [1, 1], 9, 1, 1)
    assert (lf, lb, tmax, J) == ([2], [1, 1], 3, 9)


def test_stage_bounds():
    assert PT.stage_bounds([3, 3, 3, 3], 12, False) == [0, 3, 6, 9]
    assert PT.stage_bounds([1, 2], 3, True) == [2, 1]
