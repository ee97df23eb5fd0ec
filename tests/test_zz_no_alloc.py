"""rdt_recurrent_forward_noalloc (static per-device scratch, nothing
allocated) against rdt_recurrent_forward with a caller workspace: two calls in
a row on one GPU, the second with a smaller input, and the refusal of a config
whose workspace exceeds the scratch."""
import numpy as np
import pytest

from rdt_inputs import get_config, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _pair(cfg):
    import torch

    from recurrent_depth_transformer_amd import RecurrentBlock, device_weights
    inp = make_inputs(cfg)
    W = device_weights(inp, cfg, "cuda")
    T = cfg["T"]
    blk = RecurrentBlock(cfg, graph=True)
    ref = blk.forward(W["h0"], W["e"], W, T=T)
    out = torch.empty_like(W["h0"])
    loops = torch.empty(W["h0"].shape[0], dtype=torch.int32, device="cuda")
    got = blk.forward_noalloc(W["h0"], W["e"], W, T=T, out=out, aux={"loops": loops})
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy(), loops.cpu().numpy()


@pytest.mark.parametrize("first,second", [("act_small", "gqa_small")])
def test_noalloc_matches_workspace_forward_twice(first, second):
    # the second call is smaller (fewer tokens, narrower rows) and runs after
    # the first has left its contents in the shared scratch
    a = get_config(first)
    b = get_config(second, batch=1, seq=40)
    assert a["batch"] * a["seq"] * a["dim"] > b["batch"] * b["seq"] * b["dim"]
    for cfg in (a, b):
        ref, got, loops = _pair(cfg)
        print(f"[noalloc] {cfg['name']}: {cfg['batch']}x{cfg['seq']} dim {cfg['dim']} T={cfg['T']} "
              f"max|diff|={float(np.max(np.abs(ref - got))):.3e}", flush=True)
        assert np.all(np.isfinite(got))
        np.testing.assert_array_equal(got, ref)
        assert loops.min() >= 1 and loops.max() <= cfg["T"]


def test_noalloc_refuses_a_workspace_above_the_scratch():
    import torch

    from recurrent_depth_transformer_amd import NOALLOC_SCRATCH_BYTES, RdtError, RecurrentBlock, device_weights
    cfg = get_config("gqa_small", batch=16, seq=512)
    blk = RecurrentBlock(cfg)
    assert blk.workspace_size(cfg["T"]) > NOALLOC_SCRATCH_BYTES
    inp = make_inputs(get_config("gqa_small"))
    N, D = cfg["batch"] * cfg["seq"], cfg["dim"]
    W = device_weights(inp, get_config("gqa_small"), "cuda")
    h0 = torch.zeros(N, D, dtype=torch.float32, device="cuda")
    out = torch.empty_like(h0)
    with pytest.raises(RdtError) as ei:
        blk.forward_noalloc(h0, h0, W, T=cfg["T"], out=out)
    assert "RDT_E_WORKSPACE" in str(ei.value) and "scratch" in str(ei.value)
