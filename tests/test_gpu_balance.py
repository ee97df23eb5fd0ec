"""Router-bias balancing update and expert depth usage on the GPU, against
the oracle (exact: integer load comparisons, one float32 add per entry)."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import rdt_oracle as ro
from rdt_inputs import get_config
from rdt_gpu_run import run_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,E,rows", [(1, 4, 1), (8, 16, 1), (16, 64, 16), (5, 64, 16), (12, 300, 3), (0, 8, 2)])
def test_bias_update_matches_oracle(T, E, rows):
    import torch

    import recurrent_depth_transformer_amd as rdt
    rng = np.random.default_rng(T * 1000 + E)
    counts = rng.integers(0, 50, size=(T, E)).astype(np.int32)
    if T:
        counts[0, : E // 2] = counts[0, E // 2: 2 * (E // 2)]   # plant exact ties with the mean
    bias = rng.standard_normal((rows, E)).astype(np.float32)
    want = ro.router_bias_update(counts.reshape(T, E), bias, 0.125)
    bd = torch.from_numpy(bias).cuda()
    rdt.router_bias_update(torch.from_numpy(counts.reshape(T, E)).cuda(), bd, 0.125)
    np.testing.assert_array_equal(bd.cpu().numpy(), want)
    dep = rdt.expert_depths(torch.from_numpy(counts.reshape(T, E)).cuda())
    assert dep.cpu().numpy().tolist() == ro.expert_depths(counts.reshape(T, E)).tolist()


def test_balancing_step_after_a_forward():
    """The counts a forward dumps feed the update directly; depth usage of
    the wide MoE workload is read from the same dump."""
    import torch

    import recurrent_depth_transformer_amd as rdt
    cfg = get_config("wide_small")
    res, inputs, _, W = run_gpu(cfg)
    counts = torch.from_numpy(res["expert_counts"]).cuda()
    bias0 = W["router_bias"].clone()
    rdt.router_bias_update(counts, W["router_bias"], 1e-3)
    want = ro.router_bias_update(res["expert_counts"], bias0.cpu().numpy(), 1e-3)
    np.testing.assert_array_equal(W["router_bias"].cpu().numpy(), want)
    dep = rdt.expert_depths(counts).cpu().numpy()
    assert dep.tolist() == ro.expert_depths(res["expert_counts"]).tolist()
    assert dep.max() <= cfg["T"]


def test_bias_update_argument_errors():
    import torch

    import recurrent_depth_transformer_amd as rdt
    c = torch.zeros(2, 4, dtype=torch.int32, device="cuda")
    with pytest.raises(rdt.RdtError):
        rdt.router_bias_update(c, torch.zeros(1, 4, device="cuda"), float("nan"))
    with pytest.raises(rdt.RdtError):
        rdt.router_bias_update(c, torch.zeros(1, 4, device="cuda"), -1.0)
    with pytest.raises(rdt.RdtError):
        rdt.router_bias_update(c, torch.zeros(1, 5, device="cuda"), 0.1)
