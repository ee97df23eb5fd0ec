"""Parity at the workloads' full sizes, in the launch configuration bench.py times
(graph mode, same shapes).

* Routing of every running row, every loop, teacher-forced on the GPU's router
  input: experts in order and per-expert counts against the oracle (near-tie
  tokens excluded and reported).
* ACT: halting decisions of every token against the oracle's rule from the
  GPU's own states.
* On sampled rows, the loop update h_t -> h_{t+1} from the GPU's own state.
* End to end after all T loops, max|dh_T| <= 2e-2 RMS(h_T), with routing and
  halting forced to the GPU's choices: the whole batch for gqa; for the larger
  workloads the first PREFIX positions of the first and of the last sequence.
  Causal attention and per-token routing and halting make those positions
  independent of the later ones, so the float64 oracle run on the prefix alone
  gives exactly their states."""
import numpy as np
import pytest

from oracle import rdt_oracle as ro
from rdt_inputs import get_config

from rdt_gpu_run import (aux_to_numpy, check_halting, check_routing_teacher_forced, make_aux, prefix_inputs, rms,
                         run_gpu)

pytestmark = pytest.mark.gpu

TOL = 2e-2
PREFIX = 256


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _loops_to_check(T):
    return sorted({0, T // 2, T - 1})


def end_to_end_prefix(name, cfg, inp, res, T, P=PREFIX):
    """Worst max|dh_T| / RMS(h_T) over the prefixes of the first and last sequence."""
    S, B = cfg["seq"], cfg["batch"]
    worst = 0.0
    for b in sorted({0, B - 1}):
        rows = b * S + np.arange(P)
        cp, sub = prefix_inputs(inp, cfg, b, P)
        fl = res["loops"][rows] if cfg["act"] else None
        ref = ro.forward(cp, sub, T=T, forced_idx=res["route_idx"][:, rows], forced_loops=fl)
        if cfg["act"]:
            assert np.array_equal(ref["loops"], res["loops"][rows])
        err = float(np.max(np.abs(res["h"][rows] - ref["h"])))
        scale = rms(ref["h"])
        worst = max(worst, err / scale)
        print(f"[fullsize] {name} end to end, sequence {b} positions 0..{P - 1}: "
              f"max|dh_T|/rms={err / scale:.3e}", flush=True)
    return worst


@pytest.mark.parametrize("name", ["gqa", "mla", "wide_moe", "act"])
def test_fullsize(name):
    cfg = get_config(name)
    T = cfg["T"]
    N = cfg["batch"] * cfg["seq"]
    print(f"[fullsize] {name}: running the GPU forward with dumps", flush=True)
    res, inp, *_ = run_gpu(cfg, T=T)
    assert np.all(np.isfinite(res["h"]))
    if cfg["act"]:
        assert res["loops"].min() >= 1 and res["loops"].max() <= T
        bad, near_h = check_halting(cfg, inp, res, T)
        print(f"[fullsize] act: halting decisions wrong={bad} near-threshold={near_h}; executed token-loops="
              f"{int(res['loops'].sum())} of {N * T}, mean depth {res['loops'].mean():.2f}", flush=True)
        assert bad == 0
    stats = {}
    mism, near, comp = check_routing_teacher_forced(cfg, inp, res, T, ro, stats)
    print(f"[fullsize] {name}: routing mismatches={mism} near_ties={near} compared={comp} "
          f"order_ties={stats['order_ties']} near_ties_per_loop={stats['near_ties_per_loop']}", flush=True)
    assert mism == 0
    rng = np.random.default_rng(123)
    d_r = cfg["head_dim"] if cfg["attn"] == "gqa" else cfg["qk_rope_head_dim"]
    tables = ro.rope_tables(cfg["seq"], d_r, cfg["rope_base"])
    for t in _loops_to_check(T):
        active = np.nonzero(res["loops"] > t)[0]
        if active.size == 0:
            continue
        ends = [b * cfg["seq"] + cfg["seq"] - 1 for b in range(cfg["batch"])]
        pick = np.concatenate([rng.choice(active, size=min(40, active.size), replace=False),
                               np.intersect1d(ends, active)])
        rows = np.unique(pick)
        hn, a, _ = ro.step_rows(cfg, inp, res["h_dump"][t], inp["e"], t, rows, res["route_idx"][t][rows],
                                tables=tables)
        err = np.max(np.abs(res["h_dump"][t + 1][rows] - hn))
        scale = rms(res["h_dump"][t + 1][active])
        aerr = np.max(np.abs(res["a_dump"][t][rows] - a)) / max(rms(a), 1e-30)
        print(f"[fullsize] {name} loop {t}: rows={rows.size} max|dh|/rms={err / scale:.3e} "
              f"attn-branch rel={aerr:.3e} active={active.size}", flush=True)
        assert err <= TOL * scale
    if name == "gqa":  # small enough for a full float64 forward with routing forced
        ref = ro.forward(cfg, inp, T=T, forced_idx=res["route_idx"])
        err = np.max(np.abs(res["h"] - ref["h"]))
        print(f"[fullsize] gqa end-to-end max|dh|/rms={err / rms(ref['h']):.3e}", flush=True)
        assert err <= TOL * rms(ref["h"])
    else:
        assert end_to_end_prefix(name, cfg, inp, res, T) <= TOL


@pytest.mark.parametrize("name", ["dreamer", "dreamer_parallel"])
def test_fullsize_dreamer(name):
    """The Dreamer workloads at the size bench.py times (sequential sublayers;
    parallel sublayers with depth-wise LoRA, whose attention branch runs on a
    second stream): routing of every row
    teacher-forced each loop, and on sampled rows of the first sequence the
    loop update from the GPU's own states (depth attention over the token's
    loops 0..t, sequence attention over its sequence)."""
    cfg = get_config(name)
    T, S = cfg["T"], cfg["seq"]
    print(f"[fullsize] {name}: running the GPU forward with dumps", flush=True)
    res, inp, *_ = run_gpu(cfg, T=T)
    assert np.all(np.isfinite(res["h"]))
    mism, near, comp = check_routing_teacher_forced(cfg, inp, res, T, ro)
    print(f"[fullsize] {name}: routing mismatches={mism} near_ties={near} compared={comp}", flush=True)
    assert mism == 0
    rng = np.random.default_rng(321)
    tables = ro.rope_tables(S, cfg["head_dim"], cfg["rope_base"])
    rows = np.unique(np.concatenate([rng.choice(S, size=40, replace=False), [S - 1]]))
    for t in _loops_to_check(T):
        hn, d, a, _ = ro.step_rows_depth(cfg, inp, res["h_dump"][:t + 1], inp["e"], t, T, rows,
                                         res["route_idx"][t][rows], tables=tables)
        err = np.max(np.abs(res["h_dump"][t + 1][rows] - hn))
        scale = rms(res["h_dump"][t + 1])
        print(f"[fullsize] {name} loop {t}: rows={rows.size} max|dh|/rms={err / scale:.3e}", flush=True)
        assert err <= TOL * scale


@pytest.mark.parametrize("name", ["gqa", "mla", "dreamer"])
def test_fullsize_decode_last_position(name):
    """At the sizes bench.py times: prefill seq-1 positions (the same kernels as
    the full forward: equal bit for bit), then decode the last position. The
    decode step cuts the cached keys into ranges (one workgroup each, merged
    afterwards), so it is checked against the oracle loop by loop from the
    GPU's own states: the cached positions' states come from the prefill dumps,
    the new token's from the decode dumps, routing teacher-forced."""
    import torch

    from recurrent_depth_transformer_amd import RecurrentBlock
    cfg = get_config(name)
    B, S, D, T = cfg["batch"], cfg["seq"], cfg["dim"], cfg["T"]
    full, inp, _, W = run_gpu(cfg, dumps=False)
    blk = RecurrentBlock(dict(cfg, seq=S - 1))
    cache = blk.new_cache(T, S)
    h0, e = W["h0"].view(B, S, D), W["e"].view(B, S, D)
    aux_p, aux_d = make_aux(cfg, B * (S - 1), T), make_aux(cfg, B, T)
    pre = blk.prefill(h0[:, :S - 1].contiguous().view(-1, D), e[:, :S - 1].contiguous().view(-1, D), W, T, cache, S,
                      aux=aux_p)
    last = blk.decode_step(h0[:, S - 1].contiguous(), e[:, S - 1].contiguous(), W, T, S - 1, cache, S, aux=aux_d)
    torch.cuda.synchronize()
    hf = full["h"].reshape(B, S, D)
    print(f"[fullsize-decode] {name}: prefill {S - 1} x {B}, decode position {S - 1}", flush=True)
    np.testing.assert_array_equal(pre.cpu().numpy().reshape(B, S - 1, D), hf[:, :S - 1])
    dp, dd = aux_to_numpy(aux_p), aux_to_numpy(aux_d)
    last = last.cpu().numpy()
    np.testing.assert_array_equal(last, dd["h_dump"][T])

    def states(t):   # every token's state at the start of loop t, token order b*S + s
        x = np.concatenate([dp["h_dump"][t].reshape(B, S - 1, D), dd["h_dump"][t][:, None]], axis=1)
        return x.reshape(B * S, D)

    seqs = [0] if cfg.get("da_heads", 0) else list(range(B))   # depth attention runs per sequence
    rows = np.array([b * S + S - 1 for b in seqs])
    d_r = cfg["head_dim"] if cfg["attn"] == "gqa" else cfg["qk_rope_head_dim"]
    tables = ro.rope_tables(S, d_r, cfg["rope_base"])
    for t in _loops_to_check(T):
        idx = dd["route_idx"][t][seqs]
        # the decode token's routing from its own router input
        n2 = dd["n2_dump"][t][seqs].astype(np.float64)
        idx_o, _, gap_o, _ = ro.route(n2, inp["Wr"], inp["router_bias"][min(t, cfg["n_bias_rows"] - 1)], cfg["top_k"])
        same = np.all(np.sort(idx_o, 1) == np.sort(idx, 1), axis=1)
        assert np.all(same | (gap_o < 1e-3))
        if cfg.get("da_heads", 0):
            hn, _, _, _ = ro.step_rows_depth(cfg, inp, [states(u) for u in range(t + 1)], inp["e"], t, T, rows, idx,
                                             tables=tables)
        else:
            hn, _, _ = ro.step_rows(cfg, inp, states(t), inp["e"], t, rows, idx, tables=tables)
        g = dd["h_dump"][t + 1][seqs]
        err = float(np.max(np.abs(g - hn))) / rms(g)
        print(f"[fullsize-decode] {name} loop {t}: max|dh|/rms={err:.3e}", flush=True)
        assert err <= TOL
    dev = float(np.max(np.abs(last - hf[:, S - 1]))) / rms(hf[:, S - 1])
    print(f"[fullsize-decode] {name}: decode vs full forward max|dh|/rms={dev:.3e}", flush=True)


def test_expert_tiles_ragged_many_rows():
    """The 256x256 expert tiles at widths off their blocks: 256 sequences of 128
    tokens, dim 328 and expert width 200 (k-blocks of 64 and column tiles of
    128 / 256 end part-way), 8 experts top-4, so experts see ~16 384 rows and
    both projections have over four rounds of 256x256 tiles (the rule that
    selects them). Routing of every row teacher-forced each loop; end to end
    on the first and last sequence against the oracle with routing forced."""
    import bench
    cfg = get_config("gqa_small", batch=256, seq=128, dim=328, expert_dim=200, n_experts=8, top_k=4, T=2)
    T, N = cfg["T"], cfg["batch"] * cfg["seq"]
    mt = N * cfg["top_k"] // 256 + cfg["n_experts"] // 2
    assert mt * -(-cfg["expert_dim"] // 128) >= 1024 and mt * -(-cfg["dim"] // 256) >= 1024
    assert bench.gate_up_kernel(cfg) == "k_grouped_gemm<bf16,256,256,0,2,8>"
    print(f"[tiles] ragged 256x256 expert tiles: {N} tokens, dim 328, F 200", flush=True)
    res, inp, *_ = run_gpu(cfg, T=T)
    assert np.all(np.isfinite(res["h"]))
    stats = {}
    mism, near, comp = check_routing_teacher_forced(cfg, inp, res, T, ro, stats)
    print(f"[tiles] routing mismatches={mism} near_ties={near} compared={comp}", flush=True)
    assert mism == 0
    assert end_to_end_prefix("ragged_tiles", cfg, inp, res, T, P=cfg["seq"]) <= TOL


@pytest.mark.parametrize("heads,kv,hd", [(15, 5, 128), (30, 6, 64)])
def test_query_projection_big_tiles_ragged(heads, kv, hd):
    """The query projection on 256x256 tiles with RoPE in the per-wave
    epilogue: 129 sequences of 257 tokens (33 153 rows, the last row tile
    part-filled) and 1920 query columns (the last column tile holds one
    128-wide head, or two 64-wide ones), over four rounds of tiles (the rule
    that selects them); 128-wide heads permute their weight rows so a lane
    holds both members of a rotation pair. End to end on the first and last
    sequence against the oracle with routing forced."""
    cfg = get_config("gqa_small", batch=129, seq=257, dim=256, n_heads=heads, n_kv_heads=kv, head_dim=hd, T=2)
    T, N = cfg["T"], cfg["batch"] * cfg["seq"]
    tiles = -(-N // 256) * -(-heads * hd // 256)
    assert tiles >= 1024 and N % 256 and (heads * hd) % 256
    print(f"[tiles] query projection on 256x256 tiles: {N} tokens, {heads} heads of {hd}", flush=True)
    res, inp, *_ = run_gpu(cfg, T=T)
    assert np.all(np.isfinite(res["h"]))
    stats = {}
    mism, near, comp = check_routing_teacher_forced(cfg, inp, res, T, ro, stats)
    print(f"[tiles] routing mismatches={mism} near_ties={near} compared={comp}", flush=True)
    assert mism == 0
    assert end_to_end_prefix(f"q_tiles_{hd}", cfg, inp, res, T, P=cfg["seq"]) <= TOL
