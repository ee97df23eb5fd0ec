"""Pins of the CPU oracle to facts outside itself: closed forms, library special
cases, invariants and a float64 scalar brute force. CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as Fnn

import oracle
from oracle import brute
from oracle import rdt_oracle as ro
from rdt_inputs import get_config, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny(name="tiny", **kw):
    cfg = get_config(name, **kw)
    return cfg, make_inputs(cfg)


# ---------------------------------------------------------------------------
# injection: closed form with the block switched off
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "mla_small", "act_small", "wide_small"])
def test_injection_closed_form(name):
    cfg, W = _tiny(name)
    if cfg["attn"] == "mla" or cfg["dim"] > 64:
        cfg["seq"] = 8
        cfg = dict(cfg, batch=1)
        W["e"] = W["e"][:8]
        W["h0"] = W["h0"][:8] * 0.5 + 0.25
    W["Wo"] = np.zeros_like(W["Wo"])
    W["Wd"] = np.zeros_like(W["Wd"])
    if cfg["n_shared_experts"]:
        W["Wsd"] = np.zeros_like(W["Wsd"])
    if cfg["lora_rank"]:
        W["lora_up"] = np.zeros_like(W["lora_up"])
    cfg["act"] = False
    T = 7
    out = ro.forward(cfg, W, T=T)["h"]
    A = W["A"].astype(np.float64)
    B = W["B"].astype(np.float64)
    h0 = W["h0"].astype(np.float64)
    e = W["e"].astype(np.float64)
    closed = A ** T * h0 + B * e * (1 - A ** T) / (1 - A)
    np.testing.assert_allclose(out, closed, rtol=1e-12, atol=1e-12)
    # contraction towards the fixed point h* = B e / (1 - A)
    hstar = B * e / (1 - A)
    rho = oracle.spectral_radius(A)
    assert np.all(np.abs(out - hstar) <= rho ** T * np.abs(h0 - hstar) + 1e-12)


def test_spectral_radius_and_guard():
    facts = json.load(open(os.path.join(GOLDEN, "pages_facts.json")))
    assert facts["injection_A_is_per_channel"]["value"]
    A = np.array([0.3, -0.97, 0.5])
    assert oracle.spectral_radius(A) == pytest.approx(0.97)
    # diagonal matrix: eigenvalues are the entries
    assert oracle.spectral_radius(A) == pytest.approx(np.max(np.abs(np.linalg.eigvals(np.diag(A)))))
    cfg, W = _tiny()
    W["A"] = W["A"].copy()
    W["A"][3] = 1.0
    with pytest.raises(ValueError):
        ro.forward(cfg, W, T=1)


# ---------------------------------------------------------------------------
# elementary closed forms
# ---------------------------------------------------------------------------
def test_rmsnorm_closed_form():
    x = np.full((2, 16), 3.0)
    g = np.linspace(0.5, 2.0, 16)
    y = oracle.rmsnorm(x, g, eps=0.0)
    np.testing.assert_allclose(y, np.broadcast_to(g, (2, 16)), rtol=1e-15)
    x = np.array([[3.0, 4.0]])  # rms = sqrt(12.5)
    y = oracle.rmsnorm(x, np.ones(2), eps=0.0)
    np.testing.assert_allclose(y, [[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]], rtol=1e-15)


def test_attention_uniform_query_is_prefix_mean():
    rng = np.random.default_rng(1)
    S, d = 9, 4
    v = rng.standard_normal((S, d))
    k = rng.standard_normal((S, d))
    o = ro.attention_causal(np.zeros((S, d)), k, v, 0.5)
    ref = np.cumsum(v, axis=0) / np.arange(1, S + 1)[:, None]
    np.testing.assert_allclose(o, ref, rtol=1e-13, atol=1e-14)
    # first query only sees itself
    o = ro.attention_causal(rng.standard_normal((S, d)), k, v, 1.0)
    np.testing.assert_allclose(o[0], v[0], rtol=1e-14)


def test_swiglu_hand_value():
    # silu(1) = 1 / (1 + e^-1) = 0.7310585786300049; (2*0.5)=1, (2*3)=6, *0.25
    y = ro.swiglu(np.array([[2.0]]), np.array([[0.5]]), np.array([[3.0]]), np.array([[0.25]]))
    assert y[0, 0] == pytest.approx(0.7310585786300049 * 6 * 0.25, rel=1e-15)


def test_rope_is_relative():
    rng = np.random.default_rng(2)
    d = 32
    cos, sin = ro.rope_tables(64, d, 10000.0)
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))

    def score(i, j):
        qi = ro.apply_rope(q, np.array([i]), cos, sin)
        kj = ro.apply_rope(k, np.array([j]), cos, sin)
        return float(np.sum(qi * kj))

    for (i, j, s) in [(5, 2, 7), (10, 10, 30), (3, 0, 40)]:
        assert score(i, j) == pytest.approx(score(i + s, j + s), rel=1e-10, abs=1e-12)
    # rotation preserves the norm; position 0 is the identity
    x = rng.standard_normal((3, 2, d))
    r = ro.apply_rope(x, np.array([0, 7, 33]), cos, sin)
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_allclose(r[0], x[0], rtol=0, atol=0)


def test_rope_matches_complex_rotation():
    # half-split rotation = multiplying (x1 + i x2) by exp(i * pos * theta)
    rng = np.random.default_rng(3)
    d, S = 16, 20
    cos, sin = ro.rope_tables(S, d, 10000.0)
    x = rng.standard_normal((S, 3, d))
    pos = np.arange(S)
    ref = torch.view_as_complex(torch.stack([torch.tensor(x[..., :d // 2]),
                                             torch.tensor(x[..., d // 2:])], -1).contiguous())
    theta = torch.tensor(10000.0, dtype=torch.float64) ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    rot = torch.polar(torch.ones(S, d // 2, dtype=torch.float64), torch.arange(S, dtype=torch.float64)[:, None] * theta)
    z = ref * rot[:, None, :]
    y = np.concatenate([z.real.numpy(), z.imag.numpy()], -1)
    np.testing.assert_allclose(ro.apply_rope(x, pos, cos, sin), y, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# attention: GQA special cases against torch SDPA
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("H,KV", [(4, 4), (4, 1), (8, 2), (6, 3)])
def test_gqa_against_sdpa(H, KV):
    rng = np.random.default_rng(H * 10 + KV)
    Bt, S, d = 2, 11, 8
    q = rng.standard_normal((Bt * S, H, d))
    k = rng.standard_normal((Bt * S, KV, d))
    v = rng.standard_normal((Bt * S, KV, d))
    o = ro.gqa_attention(q, k, v, Bt, S)
    tq = torch.tensor(q).view(Bt, S, H, d).transpose(1, 2)
    tk = torch.tensor(k).view(Bt, S, KV, d).transpose(1, 2).repeat_interleave(H // KV, dim=1)
    tv = torch.tensor(v).view(Bt, S, KV, d).transpose(1, 2).repeat_interleave(H // KV, dim=1)
    ref = Fnn.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    ref = ref.transpose(1, 2).reshape(Bt * S, H, d).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# router and MoE
# ---------------------------------------------------------------------------
def test_moe_k_equals_E_is_dense_softmax_mixture():
    cfg, W = _tiny(top_k=4)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((13, cfg["dim"]))
    idx, gates, gap, _ = ro.route(x, W["Wr"], np.zeros(4), 4)
    assert np.all(np.isinf(gap))
    np.testing.assert_allclose(gates.sum(1), 1.0, rtol=1e-14)
    m = ro.moe(x, idx, gates, W, 0)
    # dense mixture through einsum over all experts at once
    logits = torch.tensor(x) @ torch.tensor(W["Wr"], dtype=torch.float64).T
    p = torch.softmax(logits, dim=1)
    Wg = torch.tensor(W["Wg"], dtype=torch.float64)
    Wu = torch.tensor(W["Wu"], dtype=torch.float64)
    Wd = torch.tensor(W["Wd"], dtype=torch.float64)
    tx = torch.tensor(x)
    hid = Fnn.silu(torch.einsum("nd,efd->nef", tx, Wg)) * torch.einsum("nd,efd->nef", tx, Wu)
    y = torch.einsum("nef,edf->ned", hid, Wd)
    ref = (p[:, :, None] * y).sum(1).numpy()
    np.testing.assert_allclose(m, ref, rtol=1e-10, atol=1e-13)


def test_router_forced_bias_selects_set():
    cfg, W = _tiny("wide_small")
    rng = np.random.default_rng(5)
    x = rng.standard_normal((40, cfg["dim"]))
    E, k = cfg["n_experts"], cfg["top_k"]
    chosen = [1, 6, 9, 14]
    bias = np.zeros(E)
    bias[chosen] = 1e4
    idx, gates, gap, _ = ro.route(x, W["Wr"], bias, k)
    assert all(sorted(r) == chosen for r in idx.tolist())
    counts = np.bincount(idx.ravel(), minlength=E)
    assert set(counts.tolist()) <= {0, 40}
    # the bias moves selection only: gates are the plain softmax at those experts
    p = torch.softmax(torch.tensor(x) @ torch.tensor(W["Wr"], dtype=torch.float64).T, 1).numpy()
    np.testing.assert_allclose(gates, np.take_along_axis(p, idx, 1), rtol=1e-14)


def test_router_invariants_and_ties():
    rng = np.random.default_rng(6)
    E, k, n, D = 16, 4, 200, 32
    Wr = rng.standard_normal((E, D)).astype(np.float32)
    x = rng.standard_normal((n, D))
    idx, gates, gap, sel = ro.route(x, Wr, np.zeros(E), k)
    assert all(len(set(r)) == k for r in idx.tolist())
    assert np.all(gates > 0) and np.all(gates.sum(1) <= 1 + 1e-12)
    assert np.all(gap >= 0)
    srt = np.sort(sel, axis=1)[:, ::-1]
    np.testing.assert_array_equal(np.take_along_axis(sel, idx, 1), srt[:, :k])
    # exact ties go to the lower expert index
    Wt = np.zeros((6, 4), np.float32)
    Wt[2] = Wt[4] = Wt[5] = [1, 0, 0, 0]
    idx, _, gap, _ = ro.route(np.array([[1.0, 0, 0, 0]]), Wt, np.zeros(6), 2)
    assert idx.tolist() == [[2, 4]] and gap[0] == 0.0


# ---------------------------------------------------------------------------
# the whole block: T=1 against an independent torch block, brute force
# ---------------------------------------------------------------------------
def _torch_block_gqa(cfg, W):
    """Independent single block: torch library RMSNorm, SDPA with GQA, complex
    RoPE, torch.topk routing; returns A h0 + B e + a + m."""
    t = lambda a: torch.tensor(np.asarray(a), dtype=torch.float64)
    Bt, S, D = cfg["batch"], cfg["seq"], cfg["dim"]
    H, KV, d = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    h, e = t(W["h0"]), t(W["e"])
    u = h + e
    n1 = Fnn.rms_norm(u, (D,), t(W["g1"]), eps=cfg["norm_eps"])
    q = (n1 @ t(W["Wq"]).T).view(Bt, S, H, d)
    k = (n1 @ t(W["Wk"]).T).view(Bt, S, KV, d)
    v = (n1 @ t(W["Wv"]).T).view(Bt, S, KV, d)
    theta = torch.tensor(cfg["rope_base"], dtype=torch.float64) ** (
        -torch.arange(0, d, 2, dtype=torch.float64) / d)
    rot = torch.polar(torch.ones(S, d // 2, dtype=torch.float64),
                      torch.arange(S, dtype=torch.float64)[:, None] * theta)[None, :, None, :]

    def rope(x):
        z = torch.view_as_complex(torch.stack([x[..., :d // 2], x[..., d // 2:]], -1).contiguous()) * rot
        return torch.cat([z.real, z.imag], -1)

    q, k = rope(q), rope(k)
    o = Fnn.scaled_dot_product_attention(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2),
                                         is_causal=True, enable_gqa=True)
    o = o.transpose(1, 2).reshape(Bt * S, H * d)
    a = o @ t(W["Wo"]).T
    x = u + a
    n2 = Fnn.rms_norm(x, (D,), t(W["g2"]), eps=cfg["norm_eps"])
    logits = n2 @ t(W["Wr"]).T
    p = torch.softmax(logits, -1)
    top = torch.topk(logits + t(W["router_bias"][0]), cfg["top_k"], dim=-1).indices
    m = torch.zeros_like(n2)
    for n in range(n2.shape[0]):
        for ex in top[n].tolist():
            hid = Fnn.silu(n2[n] @ t(W["Wg"][ex]).T) * (n2[n] @ t(W["Wu"][ex]).T)
            m[n] += p[n, ex] * (hid @ t(W["Wd"][ex]).T)
        for s in range(cfg["n_shared_experts"]):
            hid = Fnn.silu(n2[n] @ t(W["Wsg"][s]).T) * (n2[n] @ t(W["Wsu"][s]).T)
            m[n] += hid @ t(W["Wsd"][s]).T
    return (t(W["A"]) * h + t(W["B"]) * e + a + m).numpy()


@pytest.mark.parametrize("name", ["tiny", "tiny_bf16"])
def test_T1_equals_single_torch_block(name):
    cfg, W = _tiny(name)
    out = ro.forward(cfg, W, T=1)["h"]
    ref = _torch_block_gqa(cfg, W)
    np.testing.assert_allclose(out, ref, rtol=1e-9, atol=1e-11)


def test_T0_is_identity():
    cfg, W = _tiny()
    np.testing.assert_array_equal(ro.forward(cfg, W, T=0)["h"], W["h0"].astype(np.float64))


def _tiny_mla():
    cfg = get_config("mla_small", batch=2, seq=12, dim=48, n_heads=3, q_lora_rank=24,
                     kv_lora_rank=16, qk_rope_head_dim=8, qk_nope_head_dim=8,
                     v_head_dim=12, n_experts=4, top_k=2, expert_dim=32)
    return cfg, make_inputs(cfg)


@pytest.mark.parametrize("which", ["gqa", "mla", "act_lora", "shared_bias"])
def test_brute_force_matches_oracle(which):
    if which == "gqa":
        cfg, W = _tiny()
        cfg["batch"], cfg["seq"] = 2, 16
    elif which == "mla":
        cfg, W = _tiny_mla()
    elif which == "act_lora":
        cfg = get_config("act_small", batch=2, seq=10, dim=32, n_heads=4, n_kv_heads=2,
                         head_dim=8, n_experts=4, top_k=2, expert_dim=24, lora_rank=4,
                         n_lora=2, halt_std=0.3)
        W = make_inputs(cfg)
    else:
        cfg = get_config("wide_small", batch=1, seq=12, dim=32, n_heads=4, n_kv_heads=1,
                         head_dim=8, n_experts=6, top_k=3, expert_dim=16, n_bias_rows=2)
        W = make_inputs(cfg)
    T = 3
    res = ro.forward(cfg, W, T=T)
    hb, loops = brute.forward(cfg, W, T)
    np.testing.assert_allclose(res["h"], np.array(hb), rtol=1e-10, atol=1e-11)
    np.testing.assert_array_equal(res["loops"], np.array(loops))
    if which == "act_lora":
        assert 0 < res["loops"].min() and res["loops"].min() < T  # some tokens halted


@pytest.mark.parametrize("name", ["act_small", "mla_small", "wide_small"])
def test_causal_prefix_equals_full_forward(name):
    """The full-size end-to-end check runs the oracle on a causal prefix of one
    sequence: with routing and halting forced, the first P positions of any
    sequence come out of the whole forward as from the prefix alone (up to
    float64 summation order)."""
    from rdt_gpu_run import prefix_inputs
    cfg = get_config(name)
    W = make_inputs(cfg)
    T, P, S = cfg["T"], 23, cfg["seq"]
    full = oracle.forward(cfg, W, T=T, record=True)
    forced = np.stack(full["idx"])
    loops = full["loops"] if cfg["act"] else None
    for b in (0, cfg["batch"] - 1):
        rows = b * S + np.arange(P)
        cp, sub = prefix_inputs(W, cfg, b, P)
        ref = oracle.forward(cp, sub, T=T, forced_idx=forced[:, rows],
                             forced_loops=None if loops is None else loops[rows])
        # (record=True keeps h per loop; BLAS blocking differs with the row count)
        np.testing.assert_allclose(ref["h"], full["h"][-1][rows], rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(ref["loops"], full["loops"][rows])


# ---------------------------------------------------------------------------
# invariants of the loop
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "act_small"])
def test_causality(name):
    cfg, W = _tiny(name)
    if name == "act_small":
        cfg.update(batch=2, seq=24)
        N = 48
        for key in ("e", "h0"):
            W[key] = W[key][:N]
    S = cfg["seq"]
    base = ro.forward(cfg, W, T=3)
    j = S - 5
    W2 = dict(W)
    W2["e"] = W["e"].copy()
    W2["h0"] = W["h0"].copy()
    W2["e"][j] += 3.0
    W2["h0"][j] -= 2.0
    pert = ro.forward(cfg, W2, T=3)
    # equal up to float64 rounding: BLAS may block the per-expert products
    # differently once token j's expert choice changes the row counts
    np.testing.assert_allclose(pert["h"][:j], base["h"][:j], rtol=1e-12, atol=1e-13)
    assert not np.allclose(pert["h"][j], base["h"][j])
    np.testing.assert_array_equal(pert["loops"][:j], base["loops"][:j])
    if cfg["batch"] > 1:  # other sequences are untouched too
        np.testing.assert_allclose(pert["h"][S:], base["h"][S:], rtol=1e-12, atol=1e-13)


def test_router_counts_over_loops():
    cfg, W = _tiny("wide_small")
    res = ro.forward(cfg, W, T=4, record=True)
    N, k = cfg["batch"] * cfg["seq"], cfg["top_k"]
    sets = []
    for t in range(4):
        assert res["counts"][t].sum() == k * N
        np.testing.assert_array_equal(res["counts"][t],
                                      np.bincount(res["idx"][t].ravel(), minlength=cfg["n_experts"]))
        sets.append(res["idx"][t])
    # the per-loop offset makes selections differ across iterations
    assert any(not np.array_equal(np.sort(sets[0], 1), np.sort(s, 1)) for s in sets[1:])


# ---------------------------------------------------------------------------
# ACT and LoRA special cases
# ---------------------------------------------------------------------------
def test_act_threshold_fact():
    facts = json.load(open(os.path.join(GOLDEN, "pages_facts.json")))
    assert get_config("act")["act_threshold"] == facts["act_threshold"]["value"]
    assert get_config("act")["T"] <= facts["max_loop_iters_upper"]["value"]
    assert get_config("wide_moe")["T"] <= facts["max_loop_iters_upper"]["value"]


def _act_cut(cfg, W, n=32):
    cfg = dict(cfg, batch=2, seq=n // 2)
    W = dict(W)
    W["e"] = W["e"][:n]
    W["h0"] = W["h0"][:n]
    return cfg, W


def test_act_zero_w_halts_after_two_loops():
    cfg, W = _tiny("act_small")
    cfg, W = _act_cut(cfg, W)
    W["w_halt"] = np.zeros_like(W["w_halt"])
    res = ro.forward(cfg, W, T=6)
    assert np.all(res["loops"] == 2)
    np.testing.assert_array_equal(res["cum"], np.float32(1.0))
    plain = ro.forward(dict(cfg, act=False), W, T=2)
    np.testing.assert_array_equal(res["h"], plain["h"])


def test_act_unreachable_threshold_is_plain_loop():
    cfg, W = _tiny("act_small")
    cfg, W = _act_cut(cfg, W)
    res = ro.forward(dict(cfg, act_threshold=1e9), W, T=5)
    plain = ro.forward(dict(cfg, act=False), W, T=5)
    np.testing.assert_array_equal(res["h"], plain["h"])
    assert np.all(res["loops"] == 5)


def test_act_halted_rows_frozen():
    cfg, W = _tiny("act_small")
    cfg, W = _act_cut(cfg, W, 48)
    W["w_halt"] = W["w_halt"] * 8
    res = ro.forward(cfg, W, T=6, record=True)
    assert res["loops"].min() < 6
    for n in range(48):
        L = res["loops"][n]
        for t in range(L, 6):
            np.testing.assert_array_equal(res["h"][t + 1][n], res["h"][L][n])


def test_lora_zero_up_is_plain_and_merge():
    cfg, W = _tiny("act_small")
    cfg, W = _act_cut(cfg, W)
    cfg["act"] = False
    W0 = dict(W, lora_up=np.zeros_like(W["lora_up"]))
    np.testing.assert_array_equal(ro.forward(cfg, W0, T=3)["h"],
                                  ro.forward(dict(cfg, lora_rank=0), W, T=3)["h"])
    # merged output projection W_o + B_t A_t with adapter index min(t, n_lora-1)
    T = cfg["n_lora"] + 2
    ref = ro.forward(cfg, W, T=T)["h"]
    h = W["h0"].astype(np.float64)
    A, B = W["A"].astype(np.float64), W["B"].astype(np.float64)
    for t in range(T):
        tl = min(t, cfg["n_lora"] - 1)
        Wm = dict(W, Wo=(torch.tensor(W["Wo"], dtype=torch.float64)
                         + torch.tensor(W["lora_up"][tl], dtype=torch.float64)
                         @ torch.tensor(W["lora_down"][tl], dtype=torch.float64)).numpy())
        st = ro.block_step(dict(cfg, lora_rank=0), Wm, h, W["e"], t,
                           np.ones(h.shape[0], bool))
        h = A * h + B * W["e"] + st["a"] + st["m"]
    np.testing.assert_allclose(ref, h, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# MLA
# ---------------------------------------------------------------------------
def test_mla_kv_saving_in_pages_range():
    facts = json.load(open(os.path.join(GOLDEN, "pages_facts.json")))
    lo, hi = facts["mla_kv_saving_range"]["value"]
    cfg = get_config("mla")
    H, nope, r, v = cfg["n_heads"], cfg["qk_nope_head_dim"], cfg["qk_rope_head_dim"], cfg["v_head_dim"]
    full = H * ((nope + r) + v) * 2
    ratio = full / oracle.kv_cache_bytes_per_token(cfg)
    assert ratio == pytest.approx(16.0)
    assert lo <= ratio <= hi
    g = get_config("gqa")
    full_mha = 2 * g["n_heads"] * g["head_dim"] * 2
    assert full_mha / oracle.kv_cache_bytes_per_token(g) == g["n_heads"] / g["n_kv_heads"]


def test_mla_explicit_equals_absorbed_numpy():
    cfg, W = _tiny_mla()
    N = cfg["batch"] * cfg["seq"]
    rng = np.random.default_rng(7)
    n1 = rng.standard_normal((N, cfg["dim"]))
    pos = np.arange(N) % cfg["seq"]
    cos, sin = ro.rope_tables(cfg["seq"], cfg["qk_rope_head_dim"], cfg["rope_base"])
    o = ro.mla_attention_explicit(cfg, W, n1, pos, cos, sin)
    # absorbed: q_lat = q_nope Wuk_h, scores over the latent, o = (P c_kv) Wuv_h^T
    H, kvl, r = cfg["n_heads"], cfg["kv_lora_rank"], cfg["qk_rope_head_dim"]
    nope, vd = cfg["qk_nope_head_dim"], cfg["v_head_dim"]
    t = lambda a: torch.tensor(np.asarray(a), dtype=torch.float64)
    tn1 = t(n1)
    cq = Fnn.rms_norm(tn1 @ t(W["Wdq"]).T, (cfg["q_lora_rank"],), t(W["gq"]), eps=1e-6)
    q = (cq @ t(W["Wuq"]).T).view(N, H, nope + r)
    lat = tn1 @ t(W["Wdkv"]).T
    ckv = Fnn.rms_norm(lat[:, :kvl], (kvl,), t(W["gkv"]), eps=1e-6)
    kpe = t(ro.apply_rope(lat[:, None, kvl:].numpy(), pos, cos, sin))[:, 0]
    qpe = t(ro.apply_rope(q[..., nope:].numpy(), pos, cos, sin))
    qlat = torch.einsum("nhi,hic->nhc", q[..., :nope], t(W["Wuk"]).view(H, nope, kvl))
    S = cfg["seq"]
    out = torch.zeros(N, H, vd, dtype=torch.float64)
    for b in range(cfg["batch"]):
        sl = slice(b * S, (b + 1) * S)
        sc = (torch.einsum("qhc,kc->hqk", qlat[sl], ckv[sl])
              + torch.einsum("qhr,kr->hqk", qpe[sl], kpe[sl])) / math.sqrt(nope + r)
        P = torch.softmax(sc.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), -math.inf), -1)
        olat = torch.einsum("hqk,kc->qhc", P, ckv[sl])
        out[sl] = torch.einsum("qhc,hvc->qhv", olat, t(W["Wuv"]).view(H, vd, kvl))
    np.testing.assert_allclose(o, out.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("name", ["tiny", "mla_small", "act_small", "wide_small"])
def test_step_rows_matches_block_step(name):
    cfg, W = _tiny(name)
    if cfg["batch"] * cfg["seq"] > 64:
        cfg.update(batch=2, seq=20)
        W["e"], W["h0"] = W["e"][:40], W["h0"][:40]
    N = cfg["batch"] * cfg["seq"]
    rng = np.random.default_rng(11)
    h = W["h0"].astype(np.float64) + 0.3 * rng.standard_normal(W["h0"].shape)
    t = 1
    full = ro.block_step(cfg, W, h, W["e"], t, np.ones(N, bool))
    rows = np.unique(np.minimum([0, 3, cfg["seq"] - 1, N - 1, cfg["seq"] + 2], N - 1))
    hn, a, n2 = ro.step_rows(cfg, W, h, W["e"], t, rows, full["idx"][rows])
    ref = np.asarray(W["A"], np.float64) * h[rows] + np.asarray(W["B"], np.float64) * W["e"][rows] \
        + full["a"][rows] + full["m"][rows]
    np.testing.assert_allclose(a, full["a"][rows], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(n2, full["n2"][rows], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(hn, ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("name", ["dreamer_tiny", "dreamer_small"])
@pytest.mark.parametrize("par", [0, 1])
def test_step_rows_depth_matches_forward(name, par):
    """The per-row Dreamer loop update equals the full forward's loop update
    (block_step with depth attention) on the same states."""
    cfg, W = _tiny(name)
    cfg["parallel"] = par
    T = 3
    N = cfg["batch"] * cfg["seq"]
    rec = ro.forward(cfg, W, T=T, record=True)
    S = cfg["seq"]
    rows = np.unique(np.minimum([0, 3, S - 1, N - 1, S + 2], N - 1))
    for t in (0, T - 1):
        hn, d, a, n2 = ro.step_rows_depth(cfg, W, rec["h"][:t + 1], W["e"], t, T, rows, rec["idx"][t][rows])
        np.testing.assert_allclose(n2, rec["n2"][t][rows], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(hn, rec["h"][t + 1][rows], rtol=1e-10, atol=1e-11)


# ---------------------------------------------------------------------------
# router-bias balancing and expert depth usage (between forwards)
# ---------------------------------------------------------------------------
def test_bias_update_hand_worked():
    # loop 0 uses bias row 0, loops 1 and 2 share row 1 (row min(t, rows - 1))
    counts = np.array([[5, 1, 0, 2],     # row 0: mean 2 -> over, under, under, at
                       [2, 2, 2, 2],
                       [0, 4, 4, 0]])    # row 1: [2, 6, 6, 2], mean 4
    bias = np.array([[0.5, -0.25, 0.0, 1.0], [0.0, 0.0, 0.0, 0.0]], np.float32)
    got = oracle.router_bias_update(counts, bias, 0.25)
    want = np.array([[0.25, 0.0, 0.25, 1.0], [0.25, -0.25, -0.25, 0.25]], np.float32)
    np.testing.assert_array_equal(got, want)
    assert got.dtype == np.float32


def test_bias_update_balanced_and_unused_rows_unchanged():
    bias = np.random.default_rng(3).standard_normal((4, 6)).astype(np.float32)
    counts = np.full((2, 6), 7)          # balanced; rows 2 and 3 see no loop
    np.testing.assert_array_equal(oracle.router_bias_update(counts, bias, 0.1), bias)


def test_bias_update_revives_dead_experts():
    """Troubleshooting item 5: without the bias adjustment the router keeps
    choosing the first two experts; repeated updates bring every expert into
    use and flatten the load."""
    rng = np.random.default_rng(11)
    E, k, D, n = 8, 2, 32, 512
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    n2 = rng.standard_normal((n, D)) + 2.0 * u
    Wr = 0.1 * rng.standard_normal((E, D))
    Wr[:2] += 3.0 * u                     # experts 0 and 1 dominate every token
    bias = np.zeros((1, E), np.float32)

    def load(b):
        idx, *_ = oracle.route(n2, Wr, b[0].astype(np.float64), k)
        return np.bincount(idx.ravel(), minlength=E)

    c0 = load(bias)
    assert c0[0] + c0[1] >= 0.9 * n * k          # the other six share under 10 %
    for _ in range(300):
        bias = oracle.router_bias_update(load(bias)[None, :], bias, 0.05)
    c = load(bias)
    assert 0.5 * c.mean() < c.min() <= c.max() < 1.5 * c.mean()
    assert np.all(bias[0, :2] < 0) and np.all(bias[0, 2:] > 0)


def test_expert_depths_counts_loops_with_tokens():
    rng = np.random.default_rng(5)
    counts = rng.integers(0, 3, size=(9, 7)) * (rng.random((9, 7)) < 0.6)
    want = [sum(1 for t in range(9) if counts[t, e] > 0) for e in range(7)]
    assert oracle.expert_depths(counts).tolist() == want


# ---------------------------------------------------------------------------
# Dreamer variants: depth attention, parallel sublayers, max-score shared expert
# ---------------------------------------------------------------------------
def _complex_depth_rope(x, pos, pos_rev, base):
    """Independent form: pair (x_i, x_{i+d/2}) as the complex number
    x_i + 1j x_{i+d/2}, multiplied by exp(1j p_i theta_i)."""
    d = x.shape[-1]
    h = d // 2
    z = x[..., :h] + 1j * x[..., h:]
    th = base ** (-2.0 * np.arange(h) / d)
    p = np.array([pos if i < h // 2 else pos_rev for i in range(h)], dtype=np.float64)
    z = z * np.exp(1j * p * th)
    return np.concatenate([z.real, z.imag], axis=-1)


def test_depth_rope_matches_complex_rotation():
    x = np.random.default_rng(1).standard_normal((5, 3, 16))
    for pos, rev in [(0, 7), (3, 4), (7, 0)]:
        np.testing.assert_allclose(oracle.depth_rope(x, pos, rev, 10000.0),
                                   _complex_depth_rope(x, pos, rev, 10000.0), rtol=1e-12, atol=1e-12)


def _depth_setup(seed=2, N=3, D=16, Hd=4, KVd=2, dd=8):
    rng = np.random.default_rng(seed)
    cfg = dict(da_heads=Hd, da_kv_heads=KVd, da_head_dim=dd, rope_base=10000.0)
    W = {"Wq_da": rng.standard_normal((Hd * dd, D)) * 0.3, "Wk_da": rng.standard_normal((KVd * dd, D)) * 0.3,
         "Wv_da": rng.standard_normal((KVd * dd, D)) * 0.3, "Wo_da": rng.standard_normal((D, Hd * dd)) * 0.3}
    states = rng.standard_normal((6, N, D))          # RMSNorm outputs of loops 0..5
    return cfg, W, states


def test_depth_attention_brute_force():
    """Scalar loops over tokens, heads and depths, complex-number rotations."""
    cfg, W, states = _depth_setup()
    T, N = 5, states.shape[1]
    Hd, KVd, dd = cfg["da_heads"], cfg["da_kv_heads"], cfg["da_head_dim"]
    hist = {"k": [], "v": []}
    for t in range(T):
        got = oracle.depth_attention(cfg, W, states[t], t, T, hist)
        want = np.zeros_like(got)
        for n in range(N):
            o = np.zeros(Hd * dd)
            for i in range(Hd):
                j = i * KVd // Hd
                q = _complex_depth_rope((states[t, n] @ W["Wq_da"].T)[i * dd:(i + 1) * dd], t, T - 1 - t, 1e4)
                sc, vs = [], []
                for tau in range(t + 1):
                    kk = _complex_depth_rope((states[tau, n] @ W["Wk_da"].T)[j * dd:(j + 1) * dd], tau,
                                             T - 1 - tau, 1e4)
                    sc.append(float(q @ kk) / np.sqrt(dd))
                    vs.append((states[tau, n] @ W["Wv_da"].T)[j * dd:(j + 1) * dd])
                w = np.exp(np.array(sc) - max(sc))
                w /= w.sum()
                o[i * dd:(i + 1) * dd] = sum(wi * vi for wi, vi in zip(w, vs))
            want[n] = W["Wo_da"] @ o
        np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_depth_attention_first_loop_passes_values():
    """At loop 0 a token has one depth state: attention returns its value."""
    cfg, W, states = _depth_setup()
    got = oracle.depth_attention(cfg, W, states[0], 0, 4, {"k": [], "v": []})
    Hd, KVd, dd = cfg["da_heads"], cfg["da_kv_heads"], cfg["da_head_dim"]
    v = (states[0] @ W["Wv_da"].T).reshape(-1, KVd, dd)
    o = np.concatenate([v[:, i * KVd // Hd] for i in range(Hd)], axis=1)
    np.testing.assert_allclose(got, o @ W["Wo_da"].T, rtol=1e-12, atol=1e-12)


def test_depth_attention_relative_in_both_halves():
    """Scores depend on depth offsets only (the reversed half on the negated
    offset), so the output does not depend on the loop count T."""
    cfg, W, states = _depth_setup()
    outs = []
    for T in (5, 9):
        hist = {"k": [], "v": []}
        outs.append([oracle.depth_attention(cfg, W, states[t], t, T, hist) for t in range(5)])
    np.testing.assert_allclose(np.array(outs[0]), np.array(outs[1]), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("variant", ["sequential", "parallel", "parallel_no_depth", "plain_shared_weight",
                                     "parallel_lora"])
def test_brute_force_matches_oracle_dreamer(variant):
    """The Dreamer block composition inside the loop, against the scalar brute
    force: depth attention -> sequence attention -> experts on the running
    residual, the parallel variant (every sublayer reads RMSNorm(h + e)), and
    the shared expert weighted by the largest router probability. All weights
    are nonzero, so a sublayer that reads the wrong residual, a dropped depth
    term or a wrong shared weight changes h_T by far more than the tolerance."""
    # weights ~N(0, 0.15): every sublayer moves the state by tens of percent
    over = dict(batch=1, seq=12, T=4, w_std=0.15)
    if variant == "parallel":
        over["parallel"] = 1
    elif variant == "parallel_no_depth":
        over.update(parallel=1, da_heads=0, da_kv_heads=0, da_head_dim=0)
    elif variant == "plain_shared_weight":
        over["shared_scale"] = 0
    elif variant == "parallel_lora":
        over.update(parallel=1, lora_rank=8, n_lora=2)
    cfg = get_config("dreamer_tiny", **over)
    W = make_inputs(cfg)
    T = cfg["T"]
    res = oracle.forward(cfg, W, T=T)
    hb, loops = brute.forward(cfg, W, T)
    hb = np.array(hb)
    np.testing.assert_allclose(res["h"], hb, rtol=1e-10, atol=1e-11)
    assert np.all(res["loops"] == T) and np.all(np.array(loops) == T)
    # the pin is sensitive to the composition: the other sublayer wiring moves h_T
    other = dict(cfg, parallel=0 if cfg.get("parallel", 0) else 1)
    hb_other = np.array(brute.forward(other, W, T)[0])
    assert np.max(np.abs(hb_other - hb)) > 1e-2 * np.max(np.abs(hb))


def test_parallel_equals_sequential_without_attention_output():
    base = get_config("parallel_small", T=2)
    W = make_inputs(base)
    W["Wo"] = np.zeros_like(W["Wo"])
    W["Wo_da"] = np.zeros_like(W["Wo_da"])
    seq = oracle.forward(dict(base, parallel=0), W)["h"]
    par = oracle.forward(base, W)["h"]
    np.testing.assert_allclose(par, seq, rtol=1e-13, atol=1e-13)
    W2 = make_inputs(base)
    assert not np.allclose(oracle.forward(dict(base, parallel=0), W2)["h"], oracle.forward(base, W2)["h"])


def test_shared_expert_scaled_by_max_score_dense():
    """k = E: the MoE is the dense softmax mixture plus max(p) times the
    shared expert (einsum over all experts, written independently)."""
    cfg = get_config("dreamer_tiny", top_k=4, T=1)
    W = make_inputs(cfg)
    rng = np.random.default_rng(4)
    n2 = rng.standard_normal((10, cfg["dim"]))
    p = np.exp(n2 @ W["Wr"].astype(np.float64).T)
    p /= p.sum(1, keepdims=True)

    def ffn(x, g, u, dn):
        a = x @ g.T
        return (a / (1 + np.exp(-a)) * (x @ u.T)) @ dn.T
    ys = np.stack([ffn(n2, W["Wg"][e], W["Wu"][e], W["Wd"][e]) for e in range(4)], 1)
    want = np.einsum("ne,ned->nd", p, ys) + p.max(1)[:, None] * ffn(n2, W["Wsg"][0], W["Wsu"][0], W["Wsd"][0])
    idx = np.tile(np.arange(4), (10, 1))
    got = oracle.moe(n2, idx, p, W, 1, p.max(1))
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_depth_attention_rejected_with_act():
    cfg = get_config("dreamer_tiny", act=True)
    W = make_inputs(cfg)
    W["w_halt"] = np.zeros(cfg["dim"], np.float32)
    with pytest.raises(ValueError):
        oracle.forward(cfg, W)
