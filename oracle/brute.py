"""Float64 scalar-loop brute force of the recurrent block (test infrastructure only).

A second, deliberately different evaluation of the same loop for tiny inputs:
plain Python loops over scalars (no BLAS, no NumPy reductions), dense routing
computed by a full sort per token, and -- for multi-latent attention -- the
absorbed form (query latents q_nope Wuk, attention over the shared latent,
then the per-head value up-projection) where the NumPy oracle reconstructs K and
V explicitly. Agreement of the two to float64 rounding pins the oracle's
indexing, head mapping, rope pairing and associativity.

It follows the same readings R1-R9 as rdt_oracle (listed there), and for the
Dreamer block variants (gist.science summary of "Depth-Recurrent Attention
Mixtures", Metodologia) the same readings of depth attention (every token
attends over its own states of loops 0..t; rotary encoding of the depth with
one half of the pairs at the reversed depth), of the sublayer order (depth
attention, then sequence attention, then experts, each behind an RMSNorm of
the running residual, or all three on RMSNorm(h + e) in the parallel variant)
and of the shared expert scaled by the token's largest router probability.
Here the depth rotation is written with complex numbers and the depth history
is kept per token as lists, where the NumPy oracle stacks per-loop arrays.
"""
from __future__ import annotations

import cmath
import math


def _dot(a, b):
    s = 0.0
    for x, y in zip(a, b):
        s += x * y
    return s


def _matvec(Wrows, x):
    """Wrows: list of rows (each a list); returns [W x]."""
    return [_dot(r, x) for r in Wrows]


def _rms(x, g, eps):
    s = 0.0
    for v in x:
        s += v * v
    inv = 1.0 / math.sqrt(s / len(x) + eps)
    return [v * inv * gg for v, gg in zip(x, g)]


def _rot(x, p, base):
    """Half-split rotary rotation of one vector at position p."""
    d = len(x)
    half = d // 2
    out = [0.0] * d
    for i in range(half):
        ang = p * base ** (-2.0 * i / d)
        c, s = math.cos(ang), math.sin(ang)
        out[i] = x[i] * c - x[i + half] * s
        out[i + half] = x[i] * s + x[i + half] * c
    return out


def _rows(M):
    return [list(map(float, r)) for r in M]


def _silu(z):
    return z / (1.0 + math.exp(-z))


def _depth_rot(x, p_lo, p_hi, base):
    """Depth rotation of one head vector as complex multiplication: element i
    and element i + d/2 form the complex number x_i + 1j*x_{i+d/2}, rotated by
    the angle p * base^(-2i/d), with p = p_lo for the first d/4 pairs and
    p = p_hi (the reversed depth) for the others."""
    d = len(x)
    half = d // 2
    out = [0.0] * d
    for i in range(half):
        p = p_lo if i < half // 2 else p_hi
        z = complex(x[i], x[i + half]) * cmath.exp(1j * p * base ** (-2.0 * i / d))
        out[i], out[i + half] = z.real, z.imag
    return out


def forward(cfg, W, T):
    """Brute-force T-loop. Returns (h as nested lists, loops list)."""
    B, S, D = cfg["batch"], cfg["seq"], cfg["dim"]
    N = B * S
    H = cfg["n_heads"]
    eps = cfg["norm_eps"]
    base = cfg["rope_base"]
    E, k, Se = cfg["n_experts"], cfg["top_k"], cfg["n_shared_experts"]
    A = list(map(float, W["A"]))
    Bv = list(map(float, W["B"]))
    e = _rows(W["e"])
    h = _rows(W["h0"])
    g1, g2 = list(map(float, W["g1"])), list(map(float, W["g2"]))
    Wo = _rows(W["Wo"])
    Wr = _rows(W["Wr"])
    experts = [(_rows(W["Wg"][x]), _rows(W["Wu"][x]), _rows(W["Wd"][x])) for x in range(E)]
    shared = [(_rows(W["Wsg"][x]), _rows(W["Wsu"][x]), _rows(W["Wsd"][x])) for x in range(Se)]
    if cfg["attn"] == "gqa":
        KV, d = cfg["n_kv_heads"], cfg["head_dim"]
        Wq, Wk, Wv = _rows(W["Wq"]), _rows(W["Wk"]), _rows(W["Wv"])
    else:
        ql, kvl = cfg["q_lora_rank"], cfg["kv_lora_rank"]
        r, nope, vd = cfg["qk_rope_head_dim"], cfg["qk_nope_head_dim"], cfg["v_head_dim"]
        Wdq, Wuq, Wdkv = _rows(W["Wdq"]), _rows(W["Wuq"]), _rows(W["Wdkv"])
        Wuk, Wuv = _rows(W["Wuk"]), _rows(W["Wuv"])
        gq, gkv = list(map(float, W["gq"])), list(map(float, W["gkv"]))
    Hd = cfg.get("da_heads", 0)
    par = bool(cfg.get("parallel", 0))
    smax_shared = bool(cfg.get("shared_scale", 0))
    if Hd:
        KVd, dd = cfg["da_kv_heads"], cfg["da_head_dim"]
        Wq_da, Wk_da, Wv_da = _rows(W["Wq_da"]), _rows(W["Wk_da"]), _rows(W["Wv_da"])
        Wo_da = _rows(W["Wo_da"])
        g_da = list(map(float, W["g_da"]))
        keys_of = [[] for _ in range(N)]      # per token: its depth keys of loops 0..t
        vals_of = [[] for _ in range(N)]
    active = [True] * N
    loops = [0] * N
    cum = [0.0] * N
    thr = cfg["act_threshold"]

    for t in range(T):
        u = [[h[n][c] + e[n][c] for c in range(D)] for n in range(N)]
        dep = [[0.0] * D for _ in range(N)]
        if Hd:
            # depth attention: the token's own states over the loops so far
            for n in range(N):
                x = _rms(u[n], g_da, eps)
                qv, kv, vv_ = _matvec(Wq_da, x), _matvec(Wk_da, x), _matvec(Wv_da, x)
                q_heads = [_depth_rot(qv[i * dd:(i + 1) * dd], t, T - 1 - t, base) for i in range(Hd)]
                keys_of[n].append([_depth_rot(kv[j * dd:(j + 1) * dd], t, T - 1 - t, base)
                                   for j in range(KVd)])
                vals_of[n].append([vv_[j * dd:(j + 1) * dd] for j in range(KVd)])
                cat = []
                for i in range(Hd):
                    j = (i * KVd) // Hd
                    sc = [_dot(q_heads[i], keys_of[n][tau][j]) / math.sqrt(dd) for tau in range(t + 1)]
                    mx = max(sc)
                    wts = [math.exp(s_ - mx) for s_ in sc]
                    z = sum(wts)
                    acc = [0.0] * dd
                    for tau in range(t + 1):
                        for c in range(dd):
                            acc[c] += wts[tau] / z * vals_of[n][tau][j][c]
                    cat += acc
                dep[n] = _matvec(Wo_da, cat)
        # the sequence attention reads RMSNorm(u + d), or RMSNorm(u) in parallel
        u1 = u if par else [[u[n][c] + dep[n][c] for c in range(D)] for n in range(N)]
        n1 = [_rms(u1[n], g1, eps) for n in range(N)]
        o = [[0.0] * 0 for _ in range(N)]
        if cfg["attn"] == "gqa":
            q = [_matvec(Wq, n1[n]) for n in range(N)]
            kk = [_matvec(Wk, n1[n]) for n in range(N)]
            vv = [_matvec(Wv, n1[n]) for n in range(N)]
            for n in range(N):
                p = n % S
                for i in range(H):
                    q[n][i * d:(i + 1) * d] = _rot(q[n][i * d:(i + 1) * d], p, base)
                for j in range(KV):
                    kk[n][j * d:(j + 1) * d] = _rot(kk[n][j * d:(j + 1) * d], p, base)
            for n in range(N):
                b0 = (n // S) * S
                out = []
                for i in range(H):
                    j = (i * KV) // H
                    qi = q[n][i * d:(i + 1) * d]
                    sc = [_dot(qi, kk[m][j * d:(j + 1) * d]) / math.sqrt(d)
                          for m in range(b0, n + 1)]
                    mx = max(sc)
                    w = [math.exp(s - mx) for s in sc]
                    z = sum(w)
                    acc = [0.0] * d
                    for wi, m in zip(w, range(b0, n + 1)):
                        vm = vv[m][j * d:(j + 1) * d]
                        for c in range(d):
                            acc[c] += wi / z * vm[c]
                    out += acc
                o[n] = out
        else:
            # absorbed multi-latent attention
            lat = [_matvec(Wdkv, n1[n]) for n in range(N)]
            ckv = [_rms(lat[n][:kvl], gkv, eps) for n in range(N)]
            kpe = [_rot(lat[n][kvl:], n % S, base) for n in range(N)]
            cq = [_rms(_matvec(Wdq, n1[n]), gq, eps) for n in range(N)]
            qfull = [_matvec(Wuq, cq[n]) for n in range(N)]
            scale = 1.0 / math.sqrt(nope + r)
            for n in range(N):
                b0 = (n // S) * S
                out = []
                for i in range(H):
                    qh = qfull[n][i * (nope + r):(i + 1) * (nope + r)]
                    qn, qp = qh[:nope], _rot(qh[nope:], n % S, base)
                    # q_lat[c] = sum_j qn[j] * Wuk[i*nope + j][c]
                    qlat = [0.0] * kvl
                    for jj in range(nope):
                        row = Wuk[i * nope + jj]
                        for c in range(kvl):
                            qlat[c] += qn[jj] * row[c]
                    sc = [(_dot(qlat, ckv[m]) + _dot(qp, kpe[m])) * scale
                          for m in range(b0, n + 1)]
                    mx = max(sc)
                    w = [math.exp(s - mx) for s in sc]
                    z = sum(w)
                    olat = [0.0] * kvl
                    for wi, m in zip(w, range(b0, n + 1)):
                        for c in range(kvl):
                            olat[c] += wi / z * ckv[m][c]
                    out += [_dot(Wuv[i * vd + jj], olat) for jj in range(vd)]
                o[n] = out
        a = [_matvec(Wo, o[n]) for n in range(N)]
        if cfg["lora_rank"]:
            tl = min(t, cfg["n_lora"] - 1)
            Ld, Lu = _rows(W["lora_down"][tl]), _rows(W["lora_up"][tl])
            for n in range(N):
                z = _matvec(Ld, o[n])
                add = _matvec(Lu, z)
                a[n] = [x + y for x, y in zip(a[n], add)]
        bias = list(map(float, W["router_bias"][min(t, cfg["n_bias_rows"] - 1)]))
        for n in range(N):
            if not active[n]:
                continue
            # the experts read RMSNorm(u + d + a), or RMSNorm(u) in parallel
            x = list(u[n]) if par else [u1[n][c] + a[n][c] for c in range(D)]
            n2 = _rms(x, g2, eps)
            logits = _matvec(Wr, n2)
            mx = max(logits)
            ex = [math.exp(l - mx) for l in logits]
            zs = sum(ex)
            prob = [v / zs for v in ex]
            # full sort of (-score, index); the score is rounded to float32 the
            # way the oracle and the kernels decide
            import struct
            f32 = [struct.unpack("f", struct.pack("f", l + bb))[0]
                   for l, bb in zip(logits, bias)]
            order = sorted(range(E), key=lambda ee: (-f32[ee], ee))
            m = [0.0] * D
            for ee in order[:k]:
                wg, wu, wd = experts[ee]
                hid = [_silu(_dot(wg[f], n2)) * _dot(wu[f], n2) for f in range(len(wg))]
                y = _matvec(wd, hid)
                for c in range(D):
                    m[c] += prob[ee] * y[c]
            sw = max(prob) if smax_shared else 1.0
            for (wg, wu, wd) in shared:
                hid = [_silu(_dot(wg[f], n2)) * _dot(wu[f], n2) for f in range(len(wg))]
                y = _matvec(wd, hid)
                for c in range(D):
                    m[c] += sw * y[c]
            h[n] = [A[c] * h[n][c] + Bv[c] * e[n][c] + dep[n][c] + a[n][c] + m[c] for c in range(D)]
            loops[n] += 1
        if cfg["act"]:
            import numpy as _np  # only for float32 accumulation of the halting sum
            w = list(map(float, W["w_halt"]))
            for n in range(N):
                if not active[n]:
                    continue
                p = 1.0 / (1.0 + math.exp(-_dot(w, h[n])))
                cum[n] = float(_np.float32(_np.float32(cum[n]) + _np.float32(p)))
                if cum[n] >= float(_np.float32(thr)):
                    active[n] = False
    return h, loops
