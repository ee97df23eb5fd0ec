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


def prefix_inputs(inp: dict, cfg: dict, b: int, P: int):
    """Inputs of the first P positions of sequence b as a one-sequence workload."""
    S = cfg["seq"]
    sub = dict(inp)
    sub["e"] = inp["e"][b * S:b * S + P]
    sub["h0"] = inp["h0"][b * S:b * S + P]
    return dict(cfg, batch=1, seq=P), sub


def rms(x):
    return float(np.sqrt(np.mean(np.square(np.asarray(x, np.float64)))))


def check_routing_teacher_forced(cfg, inputs, res, T, oracle_mod, stats=None):
    """Oracle router on the GPU's own n2 dump, loop by loop (routing
    teacher-forced). Rows of loop t are the tokens the GPU ran in loop t
    (loops > t); every other row must carry no routing (-1).

    Checked exactly, excluding near-tie tokens (gap between the k-th and the
    (k+1)-th selection score < 1e-3 in the oracle):
      * the chosen experts in order (descending selection score); a token whose
        set matches but whose order differs must have two chosen experts
        within 1e-3 of each other (counted as order ties);
      * the per-expert counts: the GPU's counts equal the oracle's counts over
        the clear tokens plus the GPU's own choices for the near-tie tokens.
    Returns (mismatches, near_ties, compared); stats (a dict) receives the
    order ties and the per-loop near-tie counts."""
    ro = oracle_mod
    k, E = cfg["top_k"], cfg["n_experts"]
    N = res["route_idx"].shape[1]
    loops = res["loops"] if "loops" in res else np.full(N, T)
    mism = near = comp = order_ties = 0
    per_loop = []
    for t in range(T):
        idx_g = res["route_idx"][t]
        rows = np.nonzero(loops > t)[0]
        idle = np.setdiff1d(np.arange(N), rows)
        assert np.all(idx_g[idle] == -1), f"loop {t}: routing written for a token that did not run"
        if rows.size == 0:
            per_loop.append(0)
            continue
        g = idx_g[rows]
        assert np.all(g >= 0) and np.all(g < E), f"loop {t}: missing routing for a running token"
        assert np.all(np.diff(np.sort(g, 1), axis=1) > 0), "repeated expert in a token's top-k"
        n2 = res["n2_dump"][t][rows].astype(np.float64)
        bias = inputs["router_bias"][min(t, cfg["n_bias_rows"] - 1)]
        idx_o, _, gap_o, sel = ro.route(n2, inputs["Wr"], bias, k)
        ok = gap_o >= 1e-3
        same_set = np.all(np.sort(idx_o, 1) == np.sort(g, 1), axis=1)
        same_order = np.all(idx_o == g, axis=1)
        # adjacent gaps among the chosen experts (oracle scores, descending)
        ssel = np.take_along_axis(sel.astype(np.float64), idx_o, axis=1)
        inner_tie = np.any(ssel[:, :-1] - ssel[:, 1:] < 1e-3, axis=1) if k > 1 else np.zeros(rows.size, bool)
        mism += int(np.sum(~same_set & ok))
        bad_order = same_set & ~same_order & ok
        assert np.all(inner_tie[bad_order]), f"loop {t}: experts in a different order without a near tie"
        order_ties += int(np.sum(bad_order))
        near += int(np.sum(~ok))
        comp += int(np.sum(ok))
        per_loop.append(int(np.sum(~ok)))
        cnt_g = np.bincount(g.ravel(), minlength=E)[:E]
        assert np.array_equal(cnt_g, res["expert_counts"][t]), f"loop {t}: counts disagree with route_idx"
        want = np.bincount(idx_o[ok].ravel(), minlength=E)[:E] + np.bincount(g[~ok].ravel(), minlength=E)[:E]
        if np.all(same_set[ok]):
            assert np.array_equal(res["expert_counts"][t], want), f"loop {t}: counts disagree with the oracle"
    if stats is not None:
        stats.update(order_ties=order_ties, near_ties_per_loop=per_loop)
    return mism, near, comp


def check_halting(cfg, inputs, res, T):
    """ACT halting decisions against the oracle's rule, recomputed in float64
    from the GPU's own states h_{t+1} (cumulative sum in float32, halt when it
    reaches the threshold). Tokens within 1e-3 of the threshold are excluded.
    Also checks the running sums the GPU dumped. Returns (wrong, near)."""
    thr = np.float32(cfg["act_threshold"])
    N = res["loops"].shape[0]
    cum = np.zeros(N, np.float32)
    bad = near = 0
    w = inputs["w_halt"].astype(np.float64)
    for t in range(T):
        act_rows = np.nonzero(res["loops"] > t)[0]
        if act_rows.size == 0:
            continue
        z = res["h_dump"][t + 1][act_rows].astype(np.float64) @ w
        cum[act_rows] = (cum[act_rows] + (1 / (1 + np.exp(-z))).astype(np.float32)).astype(np.float32)
        halt_o = cum[act_rows] >= thr
        halt_g = res["loops"][act_rows] == t + 1
        if t == T - 1:  # loops == T also means the token ran out of loops
            halt_g = halt_g & (res["act_cum"][t][act_rows] >= thr)
        clear = np.abs(cum[act_rows] - thr) >= 1e-3
        bad += int(np.sum((halt_o != halt_g) & clear))
        near += int(np.sum(~clear))
        np.testing.assert_allclose(res["act_cum"][t][act_rows], cum[act_rows], rtol=1e-4, atol=1e-4)
    return bad, near
