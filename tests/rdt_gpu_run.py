"""Helpers for GPU tests: run librdt with dumps and bring the results back."""
from __future__ import annotations

import numpy as np

from rdt_inputs import make_inputs, n_tokens


def run_gpu(cfg: dict, inputs: dict | None = None, T: int | None = None, dumps: bool = True,
            graph: bool = True, weights=None, block=None):
    import torch

    from recurrent_depth_transformer_amd import RecurrentBlock, device_weights

    T = cfg["T"] if T is None else T
    if inputs is None:
        inputs = make_inputs(cfg)
    W = device_weights(inputs, cfg, "cuda") if weights is None else weights
    blk = block or RecurrentBlock(dict(cfg, max_T=max(T, cfg["T"])), graph=graph)
    N, D, k, E = n_tokens(cfg), cfg["dim"], cfg["top_k"], cfg["n_experts"]
    aux = make_aux(cfg, N, T) if dumps else None
    out = blk.forward(W["h0"], W["e"], W, T=T, aux=aux)
    torch.cuda.synchronize()
    res = dict(h=out.float().cpu().numpy())
    if dumps:
        res.update(aux_to_numpy(aux))
    return res, inputs, blk, W


def make_aux(cfg: dict, N: int, T: int) -> dict:
    """Device buffers for every per-loop dump of N rows."""
    import torch
    D, k, E = cfg["dim"], cfg["top_k"], cfg["n_experts"]
    store = torch.float32 if cfg["dtype"] == "f32" else torch.bfloat16
    return dict(
        loops=torch.empty(N, dtype=torch.int32, device="cuda"),
        route_idx=torch.empty(max(T, 1), N, k, dtype=torch.int32, device="cuda"),
        route_gap=torch.empty(max(T, 1), N, dtype=torch.float32, device="cuda"),
        expert_counts=torch.empty(max(T, 1), E, dtype=torch.int32, device="cuda"),
        act_cum=torch.empty(max(T, 1), N, dtype=torch.float32, device="cuda"),
        n2_dump=torch.empty(max(T, 1), N, D, dtype=store, device="cuda"),
        a_dump=torch.empty(max(T, 1), N, D, dtype=torch.float32, device="cuda"),
        h_dump=torch.empty(T + 1, N, D, dtype=torch.float32, device="cuda"),
    )


def aux_to_numpy(aux: dict) -> dict:
    import torch
    return {k_: (v.float().cpu().numpy() if v.dtype == torch.bfloat16 else v.cpu().numpy()) for k_, v in aux.items()}


def rms(x):
    return float(np.sqrt(np.mean(np.square(np.asarray(x, np.float64)))))


def check_routing_teacher_forced(cfg, inputs, res, T, oracle_mod, active_rows_per_loop=None):
    """Oracle router on the GPU's own n2 dump, loop by loop. Returns
    (mismatches, near_ties, compared)."""
    ro = oracle_mod
    k, E = cfg["top_k"], cfg["n_experts"]
    mism = near = comp = 0
    for t in range(T):
        idx_g = res["route_idx"][t]
        rows = np.nonzero(idx_g[:, 0] >= 0)[0]
        if rows.size == 0:
            continue
        n2 = res["n2_dump"][t][rows].astype(np.float64)
        bias = inputs["router_bias"][min(t, cfg["n_bias_rows"] - 1)]
        idx_o, _, gap_o, _ = ro.route(n2, inputs["Wr"], bias, k)
        ok = gap_o >= 1e-3
        same = np.all(np.sort(idx_o, 1) == np.sort(idx_g[rows], 1), axis=1)
        mism += int(np.sum(~same & ok))
        near += int(np.sum(~ok))
        comp += int(np.sum(ok))
        cnt = np.bincount(idx_g[rows].ravel(), minlength=E)[:E]
        assert np.array_equal(cnt, res["expert_counts"][t]), f"loop {t}: counts disagree with route_idx"
        assert np.all(np.diff(np.sort(idx_g[rows], 1), axis=1) > 0), "repeated expert in a token's top-k"
    return mism, near, comp
