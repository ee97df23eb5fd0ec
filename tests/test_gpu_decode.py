"""Prefill + one-token decode with the per-loop cache (GPU).

A prefill of the first S0 positions followed by decode steps at S0..S-1 must
reproduce the full-sequence forward: causal attention makes position p depend
only on positions <= p, loop by loop. Checked two ways: against librdt's own
full forward (same kernels, so the states agree bit for bit) and against the
oracle's full forward, forced to the GPU's routing and halting.
"""
from __future__ import annotations

import numpy as np
import pytest

from oracle import rdt_oracle as ro
from rdt_inputs import get_config, make_inputs
from rdt_gpu_run import rms, run_gpu

pytestmark = pytest.mark.gpu
TOL = 2e-2
N_DEC = 3


def _aux(B_rows, T, cfg, torch):
    k = cfg["top_k"]
    return dict(loops=torch.empty(B_rows, dtype=torch.int32, device="cuda"),
                route_idx=torch.empty(T, B_rows, k, dtype=torch.int32, device="cuda"))


def _prefill_decode(cfg, inputs, W, T):
    import torch

    from recurrent_depth_transformer_amd import RecurrentBlock
    B, S, D = cfg["batch"], cfg["seq"], cfg["dim"]
    S0 = S - N_DEC
    blk = RecurrentBlock(dict(cfg, seq=S0))
    h0 = W["h0"].view(B, S, D)
    e = W["e"].view(B, S, D)
    cache = blk.new_cache(T, S)
    aux0 = _aux(B * S0, T, cfg, torch)
    out0 = blk.prefill(h0[:, :S0].contiguous().view(B * S0, D), e[:, :S0].contiguous().view(B * S0, D), W, T,
                       cache, S, aux=aux0)
    dec, dec_aux = [], []
    for p in range(S0, S):
        a = _aux(B, T, cfg, torch)
        dec.append(blk.decode_step(h0[:, p].contiguous(), e[:, p].contiguous(), W, T, p, cache, S, aux=a))
        dec_aux.append(a)
    torch.cuda.synchronize()
    h = np.zeros((B, S, D), np.float32)
    h[:, :S0] = out0.cpu().numpy().reshape(B, S0, D)
    loops = np.zeros((B, S), np.int32)
    loops[:, :S0] = aux0["loops"].cpu().numpy().reshape(B, S0)
    idx = np.zeros((T, B, S, cfg["top_k"]), np.int32)
    idx[:, :, :S0] = aux0["route_idx"].cpu().numpy().reshape(T, B, S0, -1)
    for j, p in enumerate(range(S0, S)):
        h[:, p] = dec[j].cpu().numpy()
        loops[:, p] = dec_aux[j]["loops"].cpu().numpy()
        idx[:, :, p] = dec_aux[j]["route_idx"].cpu().numpy().reshape(T, B, -1)
    return h.reshape(B * S, D), loops.reshape(-1), idx.reshape(T, B * S, -1), S0


# widths that are multiples of 8 but not of the k-stages, row chunks or tiles
RAGGED = {"ragged_gqa": dict(base="gqa_small", dim=328, expert_dim=200),
          "ragged_mla": dict(base="mla_small", dim=200, expert_dim=136),
          "three_chunk_gqa": dict(base="gqa_small", dim=640, expert_dim=200),
          "ragged_heads_mla": dict(base="mla_small", qk_nope_head_dim=40, v_head_dim=24)}


@pytest.mark.parametrize("name", ["tiny", "tiny_bf16", "gqa_small", "mla_small", "act_small", "wide_small",
                                  "dreamer_tiny", "dreamer_small", "parallel_small"] + sorted(RAGGED))
def test_prefill_then_decode_matches_full_forward(name):
    if name in RAGGED:
        over = dict(RAGGED[name])
        cfg = get_config(over.pop("base"), **over)
    else:
        cfg = get_config(name)
    T = cfg["T"]
    full, inputs, _, W = run_gpu(cfg, T=T)
    h, loops, idx, S0 = _prefill_decode(cfg, inputs, W, T)
    B, S, D = cfg["batch"], cfg["seq"], cfg["dim"]
    print(f"[decode] {name}: prefill {S0}, decode {N_DEC}, T={T}", flush=True)
    # same kernels, same per-row arithmetic: identical states
    assert np.array_equal(loops, full["loops"])
    assert np.array_equal(idx, full["route_idx"])
    np.testing.assert_array_equal(h, full["h"])
    # against the oracle's full-sequence forward, forced to the GPU's decisions
    ref = ro.forward(cfg, inputs, T=T, forced_idx=idx, forced_loops=loops if cfg["act"] else None)
    err = np.max(np.abs(h - ref["h"]))
    scale = rms(ref["h"])
    print(f"[decode] {name}: max|dh| {err:.3e}, rms {scale:.3f}, ratio {err / scale:.3e}", flush=True)
    assert err <= TOL * scale


@pytest.mark.parametrize("name,seq", [("tiny", 520), ("gqa_small", 600), ("mla_small", 560)])
def test_long_cache_decode_against_oracle(name, seq):
    """Caches of 256 positions or more are cut into key ranges merged after the
    attention launch, so the decoded rows round differently from the
    single-pass forward: they are checked against the oracle's full forward,
    forced to the GPU's routing, and the prefilled rows still equal the
    forward bit for bit."""
    cfg = get_config(name, seq=seq)
    T = cfg["T"]
    full, inputs, _, W = run_gpu(cfg, T=T)
    h, loops, idx, S0 = _prefill_decode(cfg, inputs, W, T)
    B, S, D = cfg["batch"], cfg["seq"], cfg["dim"]
    hp = h.reshape(B, S, D)
    np.testing.assert_array_equal(hp[:, :S0], full["h"].reshape(B, S, D)[:, :S0])
    ref = ro.forward(cfg, inputs, T=T, forced_idx=idx)
    err = np.max(np.abs(h - ref["h"]))
    scale = rms(ref["h"])
    print(f"[decode] {name} seq {seq}: max|dh| {err:.3e}, ratio {err / scale:.3e}", flush=True)
    assert err <= TOL * scale


def test_decode_graph_replay_reuses_one_graph_across_positions():
    """Decode steps at different positions replay one captured graph (the
    position is read from the workspace): graph and eager give equal states."""
    import torch

    from recurrent_depth_transformer_amd import RecurrentBlock, device_weights
    cfg = get_config("gqa_small")
    T, B, S, D = cfg["T"], cfg["batch"], cfg["seq"], cfg["dim"]
    inputs = make_inputs(cfg)
    W = device_weights(inputs, cfg)
    outs = []
    for graph in (True, False):
        blk = RecurrentBlock(dict(cfg, seq=S - N_DEC), graph=graph)
        cache = blk.new_cache(T, S)
        h0, e = W["h0"].view(B, S, D), W["e"].view(B, S, D)
        blk.prefill(h0[:, :S - N_DEC].contiguous().view(-1, D), e[:, :S - N_DEC].contiguous().view(-1, D), W, T,
                    cache, S)
        o = [blk.decode_step(h0[:, p].contiguous(), e[:, p].contiguous(), W, T, p, cache, S).clone()
             for p in range(S - N_DEC, S)]
        torch.cuda.synchronize()
        outs.append(torch.stack(o).cpu().numpy())
    assert np.array_equal(outs[0], outs[1])


def test_decode_argument_errors():
    import torch

    from recurrent_depth_transformer_amd import RdtError, RecurrentBlock, device_weights
    cfg = get_config("tiny")
    T, B, D = cfg["T"], cfg["batch"], cfg["dim"]
    W = device_weights(make_inputs(cfg), cfg)
    blk = RecurrentBlock(cfg)
    cache = blk.new_cache(T, 40)
    x = torch.zeros(B, D, device="cuda")
    with pytest.raises(RdtError):
        blk.decode_step(x, x.clone(), W, T, 40, cache, 40)          # pos == max_seq
    with pytest.raises(RdtError):
        blk.decode_step(x, x.clone(), W, T, -1, cache, 40)          # negative pos
    with pytest.raises(RdtError):
        blk.decode_step(x, x.clone(), W, 0, 0, cache, 40)           # T = 0
    h0 = torch.zeros(B * cfg["seq"], D, device="cuda")
    with pytest.raises(RdtError):
        blk.prefill(h0, h0.clone(), W, T, cache, cfg["seq"] - 1)    # max_seq < seq
