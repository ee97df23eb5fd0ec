"""Float64 NumPy oracle of the recurrent block's T-loop (test infrastructure only).

Every function states the passage it follows. "techbriefly" is the page
"Projeto OpenMythos afirma que Claude Mythos e um transformador de profundidade
recorrente"; "openclawapi" is "Introducao ao OpenMythos" (its Passo sections and
troubleshooting list); "Dreamer summary" is the gist.science summary of
"Depth-Recurrent Attention Mixtures" (its Metodologia section).

Readings taken where the pages are silent (each one is listed in the design doc):
  R1 the block consumes u = h_t + e and returns only its residual branch a + m;
  R2 sequential pre-norm block: RMSNorm -> attention, RMSNorm -> MoE;
  R3 RMSNorm eps 1e-6, gains given as inputs (ones);
  R4 half-split RoPE (pair i with i + d/2), positions 0..S-1 per sequence;
  R5 query head i reads kv head floor(i*KV/H); scale 1/sqrt(qk head dim);
  R6 MLA: RMSNorm on both latents, one rope key per token shared by all heads;
  R7 router: float64 logits, gates = softmax over all experts (no renorm),
     selection on logits + bias row min(t, rows-1), decided in float32, ties to
     the lower expert index; dropless experts; shared experts weight 1;
  R8 depth-wise LoRA on the attention output projection, scale 1, adapter
     index min(t, n_lora-1);
  R9 ACT: p = sigmoid(w . h_{t+1}) after each update, cumulative in float32,
     halt when c >= threshold; a halted token's state is frozen, it still
     serves as key/value, and it leaves the router, experts and update.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------
# elementary pieces
# ----------------------------------------------------------------------------
def rmsnorm(x, g, eps=1e-6):
    """RMSNorm on the residual stream (Dreamer summary, Metodologia; reading R3):
    x / sqrt(mean(x^2) + eps) * g along the last axis."""
    x = np.asarray(x, F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, F64)


def rope_tables(seq, d_r, base):
    """Rotary angles precomputed up to the sequence length (openclawapi Passo 2,
    max_seq_len is the RoPE precompute bound): theta_i = base^(-2i/d_r)."""
    i = np.arange(d_r // 2, dtype=F64)
    inv_freq = np.power(F64(base), -2.0 * i / d_r)
    ang = np.arange(seq, dtype=F64)[:, None] * inv_freq[None, :]
    return np.cos(ang), np.sin(ang)


def apply_rope(x, pos, cos, sin):
    """Rotate x [n, heads, d_r] at positions pos [n] (reading R4: element i pairs
    with element i + d_r/2)."""
    x = np.asarray(x, F64)
    half = x.shape[-1] // 2
    c = cos[pos][:, None, :]
    s = sin[pos][:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def depth_rope(x, pos, pos_rev, base):
    """Depth RoPE (Dreamer summary, depth attention: rotary encoding of the
    depth, with one half reversed to carry the distance to the maximum depth).
    Reading: half-split pairs (i, i + d/2) as in R4; pairs i < d/4 rotate by
    the depth pos, pairs d/4 <= i < d/2 by the reversed depth pos_rev =
    T - 1 - pos. x [n, heads, d]."""
    x = np.asarray(x, F64)
    d = x.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=F64)
    inv_freq = np.power(F64(base), -2.0 * i / d)
    p = np.where(np.arange(half) < half // 2, F64(pos), F64(pos_rev))
    ang = p * inv_freq
    c, sn = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * sn, x1 * sn + x2 * c], axis=-1)


def softmax(z, axis=-1):
    z = np.asarray(z, F64)
    z = z - np.max(z, axis=axis, keepdims=True)
    p = np.exp(z)
    return p / np.sum(p, axis=axis, keepdims=True)


def attention_causal(q, k, v, scale):
    """Causal softmax attention of one head of one sequence: q [S, dq], k [S, dq],
    v [S, dv] -> [S, dv]; key j is visible to query i iff j <= i."""
    s = (np.asarray(q, F64) @ np.asarray(k, F64).T) * scale
    S = s.shape[0]
    s[np.triu(np.ones((S, S), dtype=bool), 1)] = -np.inf
    return softmax(s, axis=1) @ np.asarray(v, F64)


def gqa_attention(q, k, v, batch, seq):
    """Grouped-query attention (openclawapi Passo 5; bigsaas MLA vs GQA section):
    q [N, H, d], k/v [N, KV, d]; query head i reads kv head floor(i*KV/H) (R5)."""
    N, H, d = q.shape
    KV = k.shape[1]
    o = np.empty((N, H, v.shape[2]), F64)
    for b in range(batch):
        sl = slice(b * seq, (b + 1) * seq)
        for i in range(H):
            j = (i * KV) // H
            o[sl, i] = attention_causal(q[sl, i], k[sl, j], v[sl, j], 1.0 / np.sqrt(d))
    return o


def mla_attention_explicit(cfg, W, n1, pos, cos, sin):
    """Multi-latent attention with K and V reconstructed explicitly (openclawapi
    Passo 5: kv_lora_rank / q_lora_rank latents, qk_rope_head_dim and
    qk_nope_head_dim per head, v_head_dim; each step rebuilds K/V from the latent
    by a linear projection). Readings R4-R6. Returns o [N, H, v]."""
    H = cfg["n_heads"]
    ql, kvl = cfg["q_lora_rank"], cfg["kv_lora_rank"]
    r, nope, vd = cfg["qk_rope_head_dim"], cfg["qk_nope_head_dim"], cfg["v_head_dim"]
    eps = cfg["norm_eps"]
    N = n1.shape[0]
    cq = rmsnorm(n1 @ W["Wdq"].astype(F64).T, W["gq"], eps)
    q = (cq @ W["Wuq"].astype(F64).T).reshape(N, H, nope + r)
    lat = n1 @ W["Wdkv"].astype(F64).T
    ckv = rmsnorm(lat[:, :kvl], W["gkv"], eps)
    kpe = apply_rope(lat[:, None, kvl:], pos, cos, sin)           # [N, 1, r]
    q_pe = apply_rope(q[..., nope:], pos, cos, sin)                 # [N, H, r]
    k_nope = (ckv @ W["Wuk"].astype(F64).T).reshape(N, H, nope)
    v = (ckv @ W["Wuv"].astype(F64).T).reshape(N, H, vd)
    k = np.concatenate([k_nope, np.broadcast_to(kpe, (N, H, r))], axis=-1)
    qf = np.concatenate([q[..., :nope], q_pe], axis=-1)
    o = np.empty((N, H, vd), F64)
    B, S = cfg["batch"], cfg["seq"]
    for b in range(B):
        sl = slice(b * S, (b + 1) * S)
        for i in range(H):
            o[sl, i] = attention_causal(qf[sl, i], k[sl, i], v[sl, i],
                                        1.0 / np.sqrt(nope + r))
    return o


def swiglu(x, wg, wu, wd):
    """One expert FFN: (silu(x Wg^T) * (x Wu^T)) Wd^T, no biases (expert width
    expert_dim, openclawapi Passo 2; SwiGLU activation as the workload states)."""
    x = np.asarray(x, F64)
    g = x @ wg.astype(F64).T
    u = x @ wu.astype(F64).T
    hmid = g / (1.0 + np.exp(-g)) * u
    return hmid @ wd.astype(F64).T


def route(n2, Wr, bias_row, k):
    """Top-k router (techbriefly: an MoE layer picks a subset of experts per token;
    openclawapi item 5 / Dreamer summary: a bias vector steers selection).
    Reading R7. Returns idx [n, k] int64 (descending selection score), gates
    [n, k] float64, gap [n] float32 (k-th minus (k+1)-th selection score; +inf
    when k equals the expert count), sel [n, E] float32."""
    logits = np.asarray(n2, F64) @ Wr.astype(F64).T
    p = softmax(logits, axis=1)
    sel = (logits + np.asarray(bias_row, F64)[None, :]).astype(np.float32)
    order = np.argsort(-sel, axis=1, kind="stable")
    idx = order[:, :k]
    rows = np.arange(sel.shape[0])[:, None]
    gates = p[rows, idx]
    E = sel.shape[1]
    if k < E:
        gap = (sel[rows[:, 0], order[:, k - 1]] - sel[rows[:, 0], order[:, k]])
    else:
        gap = np.full(sel.shape[0], np.inf, np.float32)
    return idx, gates, gap.astype(np.float32), sel


def moe(n2, idx, gates, W, n_shared, shared_w=None):
    """Sparse MoE output: sum over a token's selected experts of gate * expert(x),
    plus every always-on shared expert at weight 1 (openclawapi Passo 2,
    n_shared_experts; reading R7) or, with shared_w [n], at that per-token weight
    (Dreamer summary, routing: the shared expert scaled by the maximum score)."""
    n2 = np.asarray(n2, F64)
    m = np.zeros_like(n2)
    E = W["Wg"].shape[0]
    for e in range(E):
        rows, slot = np.nonzero(idx == e)
        if rows.size == 0:
            continue
        y = swiglu(n2[rows], W["Wg"][e], W["Wu"][e], W["Wd"][e])
        m[rows] += gates[rows, slot][:, None] * y
    for s in range(n_shared):
        y = swiglu(n2, W["Wsg"][s], W["Wsu"][s], W["Wsd"][s])
        m += y if shared_w is None else np.asarray(shared_w, F64)[:, None] * y
    return m


def depth_attention(cfg, W, nd, t, T, hist):
    """Dreamer depth attention at loop t (Dreamer summary, Metodologia: the
    sequence dimension is the batch and depth is the sequence; the depth KV can
    be dropped after each token). Every token attends over its own loop states
    0..t: q from loop t, keys and values of loops 0..t (kept in hist, to which
    this loop's are appended). GQA head map and 1/sqrt(d) scale as R5; depth
    RoPE as depth_rope with T the loop count of the forward. nd [N, D] is
    RMSNorm(u) * g_da. Returns the sublayer output [N, D] (after Wo_da)."""
    N = nd.shape[0]
    Hd, KVd, dd = cfg["da_heads"], cfg["da_kv_heads"], cfg["da_head_dim"]
    base = cfg["rope_base"]
    q = (nd @ W["Wq_da"].astype(F64).T).reshape(N, Hd, dd)
    k = (nd @ W["Wk_da"].astype(F64).T).reshape(N, KVd, dd)
    v = (nd @ W["Wv_da"].astype(F64).T).reshape(N, KVd, dd)
    q = depth_rope(q, t, T - 1 - t, base)
    k = depth_rope(k, t, T - 1 - t, base)
    hist["k"].append(k)
    hist["v"].append(v)
    K = np.stack(hist["k"], axis=2)              # [N, KVd, t+1, dd]
    V = np.stack(hist["v"], axis=2)
    o = np.empty((N, Hd, dd))
    for i in range(Hd):
        j = (i * KVd) // Hd
        sc = np.einsum("nd,ntd->nt", q[:, i], K[:, j]) / np.sqrt(dd)
        p = softmax(sc, axis=1)
        o[:, i] = np.einsum("nt,ntd->nd", p, V[:, j])
    return o.reshape(N, Hd * dd) @ W["Wo_da"].astype(F64).T


def spectral_radius(A):
    """rho(A) for the per-channel A (openclawapi Passo 6 returns A with shape
    (dim,)): a diagonal matrix's eigenvalues are its entries, so rho = max |A_i|."""
    return float(np.max(np.abs(np.asarray(A, F64))))


def kv_cache_bytes_per_token(cfg, elem_bytes=2):
    """Cached bytes per token per loop step: GQA keeps KV heads of K and V
    (openclawapi Passo 5: the cache shrinks by n_heads/n_kv_heads); MLA keeps the
    kv latent plus the shared rope key (Passo 5: about 10-20x smaller)."""
    if cfg["attn"] == "gqa":
        return 2 * cfg["n_kv_heads"] * cfg["head_dim"] * elem_bytes
    return (cfg["kv_lora_rank"] + cfg["qk_rope_head_dim"]) * elem_bytes


# ----------------------------------------------------------------------------
# one loop iteration and the T-loop
# ----------------------------------------------------------------------------
def _attn_out(cfg, W, n1, pos, cos, sin):
    N = n1.shape[0]
    if cfg["attn"] == "gqa":
        H, KV, d = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
        q = (n1 @ W["Wq"].astype(F64).T).reshape(N, H, d)
        k = (n1 @ W["Wk"].astype(F64).T).reshape(N, KV, d)
        v = (n1 @ W["Wv"].astype(F64).T).reshape(N, KV, d)
        q = apply_rope(q, pos, cos, sin)
        k = apply_rope(k, pos, cos, sin)
        o = gqa_attention(q, k, v, cfg["batch"], cfg["seq"])
    else:
        o = mla_attention_explicit(cfg, W, n1, pos, cos, sin)
    return o.reshape(N, -1)


def block_step(cfg, W, h, e, t, active, forced_idx=None, tables=None, depth=None, T=None):
    """Residual branch of one recurrent-block iteration (reading R1/R2):
    u = h + e; a = attention-out-projection(RMSNorm(u)) [+ depth-wise LoRA];
    x = u + a; n2 = RMSNorm(x); m = MoE(n2). Attention runs on every token (keys
    of halted tokens use their frozen state); the router and experts run on the
    active rows only.

    Dreamer variants (Dreamer summary, Metodologia): with depth attention
    (cfg da_heads > 0; needs depth = {"k": [], "v": []} carried across loops
    and T) the sublayers run DA -> SA -> EA, each on RMSNorm of the running
    residual: d = DA(RMSNorm(u) g_da), a = SA(RMSNorm(u + d) g1), m =
    MoE(RMSNorm(u + d + a) g2), branch d + a + m. With cfg parallel every
    sublayer reads RMSNorm(u) (own gains). With cfg shared_scale the shared
    expert is weighted by the token's maximum router probability.

    Returns a dict with a (the whole residual branch except m: d + a), d, n2,
    m [N, D] (rows of inactive tokens of m are zero), idx [N, k] (-1 when
    inactive), gates, gap, counts."""
    N, D = h.shape
    S = cfg["seq"]
    eps = cfg["norm_eps"]
    par = bool(cfg.get("parallel", 0))
    pos = np.arange(N) % S
    if tables is None:
        d_r = cfg["head_dim"] if cfg["attn"] == "gqa" else cfg["qk_rope_head_dim"]
        tables = rope_tables(S, d_r, cfg["rope_base"])
    cos, sin = tables
    u = np.asarray(h, F64) + np.asarray(e, F64)
    d = np.zeros((N, D), F64)
    if cfg.get("da_heads", 0):
        if depth is None or T is None:
            raise ValueError("depth attention needs the depth history and T")
        d = depth_attention(cfg, W, rmsnorm(u, W["g_da"], eps), t, T, depth)
    u1 = u if par else u + d
    n1 = rmsnorm(u1, W["g1"], eps)
    o = _attn_out(cfg, W, n1, pos, cos, sin)
    a = o @ W["Wo"].astype(F64).T
    if cfg["lora_rank"]:
        # depth-wise LoRA on the output projection (techbriefly; openclawapi
        # lora_rank and advanced direction 1); reading R8
        tl = min(t, cfg["n_lora"] - 1)
        a = a + (o @ W["lora_down"][tl].astype(F64).T) @ W["lora_up"][tl].astype(F64).T
    x = u if par else u1 + a
    n2 = rmsnorm(x, W["g2"], eps)

    k = cfg["top_k"]
    E = cfg["n_experts"]
    act_rows = np.nonzero(active)[0]
    bias_row = W["router_bias"][min(t, cfg["n_bias_rows"] - 1)]
    idx_a, gates_a, gap_a, _ = route(n2[act_rows], W["Wr"], bias_row, k)
    logits = n2[act_rows] @ W["Wr"].astype(F64).T
    p_all = softmax(logits, axis=1)
    if forced_idx is not None:
        idx_a = np.asarray(forced_idx, np.int64)[act_rows]
        gates_a = p_all[np.arange(act_rows.size)[:, None], idx_a]
    sw = p_all.max(axis=1) if cfg.get("shared_scale", 0) else None
    m_a = moe(n2[act_rows], idx_a, gates_a, W, cfg["n_shared_experts"], sw)
    m = np.zeros((N, D), F64)
    m[act_rows] = m_a
    idx = np.full((N, k), -1, np.int64)
    idx[act_rows] = idx_a
    gates = np.zeros((N, k), F64)
    gates[act_rows] = gates_a
    gap = np.full(N, np.nan, np.float32)
    gap[act_rows] = gap_a
    counts = np.bincount(idx_a.reshape(-1), minlength=E)[:E].astype(np.int64)
    return dict(a=d + a, d=d, n2=n2, m=m, idx=idx, gates=gates, gap=gap, counts=counts)


def forward(cfg, W, h0=None, e=None, T=None, forced_idx=None, forced_loops=None,
            record=False):
    """The T-loop (techbriefly: h_{t+1} = A h_t + B e + Transformer(h_t, e), the
    same weights reused every iteration, up to 16 iterations; openclawapi
    Passo 3: the loop count is chosen at call time and may exceed the trained
    count). A and B are per-channel (openclawapi Passo 6).

    forced_idx: optional [T, N, k] expert indices used instead of the router's
    own choice (gates are still this oracle's softmax at those indices).
    forced_loops: optional [N]; token n takes exactly min(T, loops[n]) updates.

    Returns dict(h [N, D] float64, loops [N] int64, and with record=True the
    per-loop lists idx, gap, counts, cum, n2, h).
    """
    e = np.asarray(W["e"] if e is None else e, F64)
    h = np.array(W["h0"] if h0 is None else h0, F64)
    T = cfg["T"] if T is None else int(T)
    if T < 0:
        raise ValueError("T must be >= 0")
    if spectral_radius(W["A"]) >= 1.0:
        raise ValueError("unstable injection: rho(A) >= 1")
    if cfg.get("da_heads", 0) and cfg["act"]:
        raise ValueError("depth attention with ACT halting is not defined here")
    depth = {"k": [], "v": []}
    A = np.asarray(W["A"], F64)[None, :]
    Bv = np.asarray(W["B"], F64)[None, :]
    N = h.shape[0]
    d_r = cfg["head_dim"] if cfg["attn"] == "gqa" else cfg["qk_rope_head_dim"]
    tables = rope_tables(cfg["seq"], d_r, cfg["rope_base"])
    active = np.ones(N, dtype=bool)
    loops = np.zeros(N, np.int64)
    cum = np.zeros(N, np.float32)
    thr = np.float32(cfg["act_threshold"])
    rec = dict(idx=[], gap=[], counts=[], cum=[], n2=[], h=[h.copy()])
    for t in range(T):
        if forced_loops is not None:
            active = np.asarray(forced_loops) > t
        if not active.any():
            if record:
                k = cfg["top_k"]
                rec["idx"].append(np.full((N, k), -1, np.int64))
                rec["gap"].append(np.full(N, np.nan, np.float32))
                rec["counts"].append(np.zeros(cfg["n_experts"], np.int64))
                rec["cum"].append(cum.copy())
                rec["n2"].append(np.zeros_like(h))
                rec["h"].append(h.copy())
            continue
        fi = None if forced_idx is None else forced_idx[t]
        st = block_step(cfg, W, h, e, t, active, fi, tables, depth, T)
        rows = np.nonzero(active)[0]
        # LTI injection plus the block's residual branch (techbriefly loop update)
        h[rows] = A * h[rows] + Bv * e[rows] + st["a"][rows] + st["m"][rows]
        loops[rows] += 1
        if cfg["act"]:
            # ACT halting (techbriefly; openclawapi item 4, threshold 0.99); R9
            z = h[rows] @ np.asarray(W["w_halt"], F64)
            p = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
            cum[rows] = (cum[rows] + p).astype(np.float32)
            if forced_loops is None:
                active = active.copy()
                active[rows[cum[rows] >= thr]] = False
        if record:
            rec["idx"].append(st["idx"])
            rec["gap"].append(st["gap"])
            rec["counts"].append(st["counts"])
            rec["cum"].append(cum.copy())
            rec["n2"].append(st["n2"])
            rec["h"].append(h.copy())
    out = dict(h=h, loops=loops, cum=cum)
    if record:
        out.update(rec)
    return out


def step_rows(cfg, W, h, e, t, rows, forced_idx_rows, tables=None):
    """One loop update h_{t+1}[rows] for a sample of active tokens, given the
    state h of every token (same definitions as block_step and forward; keys
    and values come from every token of the sequence, queries only from the
    sampled rows). forced_idx_rows: [len(rows), k] expert indices. Returns
    (h_new_rows, a_rows, n2_rows). Not defined for the Dreamer variants (depth
    attention needs every earlier loop's state of the token)."""
    if cfg.get("da_heads", 0) or cfg.get("parallel", 0) or cfg.get("shared_scale", 0):
        raise NotImplementedError("step_rows covers the sequential block without depth attention")
    h = np.asarray(h, F64)
    e = np.asarray(e, F64)
    rows = np.asarray(rows)
    N, D = h.shape
    S, eps = cfg["seq"], cfg["norm_eps"]
    H = cfg["n_heads"]
    if tables is None:
        d_r = cfg["head_dim"] if cfg["attn"] == "gqa" else cfg["qk_rope_head_dim"]
        tables = rope_tables(S, d_r, cfg["rope_base"])
    cos, sin = tables
    pos_all = np.arange(N) % S
    u = h + e
    n1 = rmsnorm(u, W["g1"], eps)
    o = np.empty((rows.size, cfg["n_heads"] * (cfg["head_dim"] if cfg["attn"] == "gqa" else cfg["v_head_dim"])))
    if cfg["attn"] == "gqa":
        KV, d = cfg["n_kv_heads"], cfg["head_dim"]
        k = apply_rope((n1 @ W["Wk"].astype(F64).T).reshape(N, KV, d), pos_all, cos, sin)
        v = (n1 @ W["Wv"].astype(F64).T).reshape(N, KV, d)
        q = apply_rope((n1[rows] @ W["Wq"].astype(F64).T).reshape(rows.size, H, d), pos_all[rows], cos, sin)
        for r, n in enumerate(rows):
            b0 = (n // S) * S
            for i in range(H):
                j = (i * KV) // H
                s = (k[b0:n + 1, j] @ q[r, i]) / np.sqrt(d)
                p = softmax(s)
                o[r, i * d:(i + 1) * d] = p @ v[b0:n + 1, j]
    else:
        ql, kvl = cfg["q_lora_rank"], cfg["kv_lora_rank"]
        nr, nope, vd = cfg["qk_rope_head_dim"], cfg["qk_nope_head_dim"], cfg["v_head_dim"]
        lat = n1 @ W["Wdkv"].astype(F64).T
        ckv = rmsnorm(lat[:, :kvl], W["gkv"], eps)
        kpe = apply_rope(lat[:, None, kvl:], pos_all, cos, sin)[:, 0]
        kn = (ckv @ W["Wuk"].astype(F64).T).reshape(N, H, nope)
        vv = (ckv @ W["Wuv"].astype(F64).T).reshape(N, H, vd)
        cq = rmsnorm(n1[rows] @ W["Wdq"].astype(F64).T, W["gq"], eps)
        q = (cq @ W["Wuq"].astype(F64).T).reshape(rows.size, H, nope + nr)
        qpe = apply_rope(q[..., nope:], pos_all[rows], cos, sin)
        for r, n in enumerate(rows):
            b0 = (n // S) * S
            for i in range(H):
                s = (kn[b0:n + 1, i] @ q[r, i, :nope] + kpe[b0:n + 1] @ qpe[r, i]) / np.sqrt(nope + nr)
                p = softmax(s)
                o[r, i * vd:(i + 1) * vd] = p @ vv[b0:n + 1, i]
    a = o @ W["Wo"].astype(F64).T
    if cfg["lora_rank"]:
        tl = min(t, cfg["n_lora"] - 1)
        a = a + (o @ W["lora_down"][tl].astype(F64).T) @ W["lora_up"][tl].astype(F64).T
    x = u[rows] + a
    n2 = rmsnorm(x, W["g2"], eps)
    idx = np.asarray(forced_idx_rows, np.int64)
    p = softmax(n2 @ W["Wr"].astype(F64).T, axis=1)
    gates = p[np.arange(rows.size)[:, None], idx]
    m = moe(n2, idx, gates, W, cfg["n_shared_experts"])
    h_new = np.asarray(W["A"], F64) * h[rows] + np.asarray(W["B"], F64) * e[rows] + a + m
    return h_new, a, n2


def step_rows_depth(cfg, W, h_hist, e, t, T, rows, forced_idx_rows, tables=None):
    """step_rows for the Dreamer block with depth attention (GQA sequence
    attention; sequential or parallel sublayers; optional max-score shared
    expert), same definitions as block_step. h_hist[tau] is the state of every
    token at the start of loop tau for tau = 0..t: depth attention at loop t
    needs a token's own states of loops 0..t, and sequence attention needs the
    keys and values of every token of the sampled rows' sequences, so depth
    attention runs on those sequences only. Returns (h_new_rows, d_rows,
    a_rows, n2_rows) for loop t."""
    if not cfg.get("da_heads", 0) or cfg["attn"] != "gqa":
        raise NotImplementedError("step_rows_depth covers depth attention with GQA sequence attention")
    e = np.asarray(e, F64)
    rows = np.asarray(rows)
    S, eps = cfg["seq"], cfg["norm_eps"]
    par = bool(cfg.get("parallel", 0))
    if tables is None:
        tables = rope_tables(S, cfg["head_dim"], cfg["rope_base"])
    cos, sin = tables
    seqs = np.unique(rows // S)
    R = (seqs[:, None] * S + np.arange(S)[None, :]).reshape(-1)   # tokens of those sequences
    where = {int(n): i for i, n in enumerate(R)}
    hist = {"k": [], "v": []}
    for tau in range(t + 1):
        u_tau = np.asarray(h_hist[tau], F64)[R] + e[R]
        d = depth_attention(cfg, W, rmsnorm(u_tau, W["g_da"], eps), tau, T, hist)
    h = np.asarray(h_hist[t], F64)
    u = h[R] + e[R]
    u1 = u if par else u + d
    n1 = rmsnorm(u1, W["g1"], eps)
    H, KV, dh = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    pos = R % S
    k = apply_rope((n1 @ W["Wk"].astype(F64).T).reshape(R.size, KV, dh), pos, cos, sin)
    v = (n1 @ W["Wv"].astype(F64).T).reshape(R.size, KV, dh)
    loc = np.array([where[int(n)] for n in rows])
    q = apply_rope((n1[loc] @ W["Wq"].astype(F64).T).reshape(rows.size, H, dh), pos[loc], cos, sin)
    o = np.empty((rows.size, H * dh))
    for r, n in enumerate(rows):
        i0 = loc[r] - (int(n) % S)                # the sequence's first token in R
        for i in range(H):
            j = (i * KV) // H
            sc = (k[i0:loc[r] + 1, j] @ q[r, i]) / np.sqrt(dh)
            o[r, i * dh:(i + 1) * dh] = softmax(sc) @ v[i0:loc[r] + 1, j]
    a = o @ W["Wo"].astype(F64).T
    if cfg["lora_rank"]:
        tl = min(t, cfg["n_lora"] - 1)
        a = a + (o @ W["lora_down"][tl].astype(F64).T) @ W["lora_up"][tl].astype(F64).T
    x = u[loc] if par else u1[loc] + a
    n2 = rmsnorm(x, W["g2"], eps)
    idx = np.asarray(forced_idx_rows, np.int64)
    p = softmax(n2 @ W["Wr"].astype(F64).T, axis=1)
    gates = p[np.arange(rows.size)[:, None], idx]
    sw = p.max(axis=1) if cfg.get("shared_scale", 0) else None
    m = moe(n2, idx, gates, W, cfg["n_shared_experts"], sw)
    d_rows = d[loc]
    h_new = np.asarray(W["A"], F64) * h[rows] + np.asarray(W["B"], F64) * e[rows] + d_rows + a + m
    return h_new, d_rows, a, n2


# ----------------------------------------------------------------------------
# between forwards: router-bias balancing and expert depth usage
# ----------------------------------------------------------------------------
def bias_row_counts(counts, rows):
    """Tokens per expert seen by each router-bias row: loop t selects with row
    min(t, rows-1), so row r sums the counts of those loops. counts: [T, E]."""
    counts = np.asarray(counts, np.int64)
    T, E = counts.shape
    out = np.zeros((rows, E), np.int64)
    for t in range(T):
        out[min(t, rows - 1)] += counts[t]
    return out


def router_bias_update(counts, bias, gamma):
    """Auxiliary-loss-free load balancing (openclawapi troubleshooting item 5:
    DeepSeekMoE-style dynamic adjustment of router_bias; Dreamer summary,
    routing: top-k with a balancing bias vector as in DeepSeek-V3). Reading:
    every expert below the mean load of its bias row gains gamma, every expert
    above it loses gamma, an expert at the mean keeps its bias. The load
    comparison is exact (integers); the bias is stored and updated in float32.
    counts [T, E] int, bias [rows, E] -> new bias [rows, E] float32."""
    bias = np.asarray(bias, np.float32)
    rows, E = bias.shape
    c = bias_row_counts(counts, rows)
    total = c.sum(axis=1, keepdims=True)
    # sign(mean - c_e) with mean = total / E, compared as total vs E * c_e
    s = np.sign(total - E * c).astype(np.float32)
    return (bias + np.float32(gamma) * s).astype(np.float32)


def expert_depths(counts):
    """Number of loop iterations (depths) in which each expert received at
    least one token (Dreamer summary, expert diversity: share of experts used
    at several depths). counts [T, E] -> [E] int."""
    return (np.asarray(counts) > 0).sum(axis=0).astype(np.int64)
