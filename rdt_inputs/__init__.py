"""Seeded synthetic inputs for the recurrent-depth block.

This module only draws numbers: it holds the workload shapes and the random
distributions they are drawn from, and nothing of the method's arithmetic.
Both the CPU oracle and the GPU path take their inputs from here.

Workloads (shapes and distributions as the recurrent-block workloads state them;
where a distribution is left open the fallback is: A ~ U(0.5, 0.95),
B ~ U(0, 0.5), e ~ N(0, 1), h0 = e, projection weights ~ N(0, 0.02), RMSNorm
gains = 1, router bias = 0):

  tiny      fp32, 1x32 tokens, D 64, GQA 4/2 heads of 16, 4 experts top-2 F 128, T 4
  gqa       bf16, 1x512, D 1024, GQA 16/4 heads of 64, 8 experts top-2 F 2816, T 3
  mla       bf16, 4x2048, D 1024, MLA 16 heads, kv latent 128 + rope 32, q latent 384,
            nope 64 / v 64, 16 experts top-2 F 1408, T 8, A ~ U(0.6, 0.98)
  wide_moe  bf16, 2x4096, D 2048, GQA 16/4 heads of 128, 64 experts top-8 + 1 shared,
            F 1024, T 16; router weights ~ N(0, 1/D) and a per-loop N(0,1) offset
  act       bf16, 8x2048, D 1024, GQA 16/4 of 64, 32 experts top-4 F 1408, T <= 16,
            depth-wise LoRA rank 16 per loop on the attention output (~ N(0, 0.01)),
            ACT halting with w ~ N(0, 0.05), threshold 0.99

  dreamer   bf16, 4x2048, D 1024, GQA 16/4 of 64, depth attention 16/4 of 64, 16 experts
            top-2 + 1 shared weighted by the max router probability, F 1408, T 8
  dreamer_parallel  the same with parallel sublayers (every sublayer reads
            RMSNorm(h + e)) and depth-wise LoRA of rank 16 on the attention output

The ``*_small`` workloads keep each family's structure at sizes a CPU reference
finishes in seconds, with sequence lengths and widths that leave ragged tiles.

Draw order is fixed: A, B, e, then the weights in struct field order, then the
router bias, then the LoRA factors, then the halting vector, then the depth
attention weights (Wq_da, Wk_da, Wv_da, Wo_da). bf16 workloads round
every drawn weight once to bfloat16 (round to nearest even) and hand both sides
those exact values as float32 arrays.
"""
from __future__ import annotations

import copy
import numpy as np

__all__ = ["WORKLOADS", "get_config", "make_inputs", "round_bf16", "bf16_bits",
           "n_tokens"]

_BASE = dict(
    batch=1, seq=32, dim=64, attn="gqa", n_heads=4, n_kv_heads=2, head_dim=16,
    q_lora_rank=0, kv_lora_rank=0, qk_rope_head_dim=0, qk_nope_head_dim=0,
    v_head_dim=0, rope_base=10000.0, norm_eps=1e-6,
    n_experts=4, n_shared_experts=0, top_k=2, expert_dim=128,
    n_bias_rows=1, lora_rank=0, n_lora=0, act=False, act_threshold=0.99,
    parallel=0, shared_scale=0, da_heads=0, da_kv_heads=0, da_head_dim=0,
    dtype="f32", T=4, seed=0,
    # distributions
    a_range=(0.5, 0.95), b_range=(0.0, 0.5), w_std=0.02, router_std=None,
    bias_std=0.0, lora_std=0.01, halt_std=0.05,
)


def _cfg(**kw):
    c = copy.deepcopy(_BASE)
    for k, v in kw.items():
        if k not in c:
            raise KeyError(k)
        c[k] = v
    return c


WORKLOADS = {
    # ---- full-size workloads ----
    "tiny": _cfg(batch=1, seq=32, dim=64, n_heads=4, n_kv_heads=2, head_dim=16,
                 n_experts=4, top_k=2, expert_dim=128, T=4, dtype="f32",
                 a_range=(0.5, 0.9)),
    "gqa": _cfg(batch=1, seq=512, dim=1024, n_heads=16, n_kv_heads=4, head_dim=64,
                n_experts=8, top_k=2, expert_dim=2816, T=3, dtype="bf16"),
    "mla": _cfg(batch=4, seq=2048, dim=1024, attn="mla", n_heads=16, n_kv_heads=16,
                head_dim=0, q_lora_rank=384, kv_lora_rank=128, qk_rope_head_dim=32,
                qk_nope_head_dim=64, v_head_dim=64, n_experts=16, top_k=2,
                expert_dim=1408, T=8, dtype="bf16", a_range=(0.6, 0.98)),
    "wide_moe": _cfg(batch=2, seq=4096, dim=2048, n_heads=16, n_kv_heads=4,
                     head_dim=128, n_experts=64, n_shared_experts=1, top_k=8,
                     expert_dim=1024, T=16, dtype="bf16", n_bias_rows=16,
                     router_std="1/sqrt(D)", bias_std=1.0),
    "act": _cfg(batch=8, seq=2048, dim=1024, n_heads=16, n_kv_heads=4, head_dim=64,
                n_experts=32, top_k=4, expert_dim=1408, T=16, dtype="bf16",
                lora_rank=16, n_lora=16, act=True),
    # ---- reduced-size workloads of each family (ragged tails on purpose) ----
    "tiny_bf16": _cfg(batch=1, seq=32, dim=64, n_heads=4, n_kv_heads=2, head_dim=16,
                      n_experts=4, top_k=2, expert_dim=128, T=4, dtype="bf16",
                      a_range=(0.5, 0.9)),
    "gqa_small": _cfg(batch=2, seq=80, dim=256, n_heads=8, n_kv_heads=2, head_dim=32,
                      n_experts=8, top_k=2, expert_dim=352, T=3, dtype="bf16"),
    "mla_small": _cfg(batch=2, seq=72, dim=256, attn="mla", n_heads=4, n_kv_heads=4,
                      head_dim=0, q_lora_rank=96, kv_lora_rank=64,
                      qk_rope_head_dim=32, qk_nope_head_dim=32, v_head_dim=32,
                      n_experts=8, top_k=2, expert_dim=160, T=3, dtype="bf16",
                      a_range=(0.6, 0.98)),
    "wide_small": _cfg(batch=2, seq=100, dim=256, n_heads=4, n_kv_heads=1,
                       head_dim=128, n_experts=16, n_shared_experts=1, top_k=4,
                       expert_dim=128, T=4, dtype="bf16", n_bias_rows=4,
                       router_std="1/sqrt(D)", bias_std=1.0),
    "act_small": _cfg(batch=3, seq=70, dim=256, n_heads=4, n_kv_heads=2, head_dim=64,
                      n_experts=8, top_k=2, expert_dim=192, T=8, dtype="bf16",
                      lora_rank=8, n_lora=4, act=True),
    # ---- Dreamer block variants (depth attention, parallel sublayers,
    # shared expert scaled by the max router score) ----
    "dreamer": _cfg(batch=4, seq=2048, dim=1024, n_heads=16, n_kv_heads=4, head_dim=64,
                    da_heads=16, da_kv_heads=4, da_head_dim=64, n_experts=16,
                    n_shared_experts=1, shared_scale=1, top_k=2, expert_dim=1408, T=8,
                    dtype="bf16"),
    "dreamer_small": _cfg(batch=2, seq=72, dim=256, n_heads=4, n_kv_heads=2, head_dim=64,
                          da_heads=4, da_kv_heads=2, da_head_dim=32, n_experts=8,
                          n_shared_experts=1, shared_scale=1, top_k=2, expert_dim=192,
                          T=6, dtype="bf16"),
    "parallel_small": _cfg(batch=2, seq=68, dim=256, n_heads=8, n_kv_heads=2, head_dim=32,
                           da_heads=4, da_kv_heads=4, da_head_dim=64, parallel=1,
                           n_experts=16, n_shared_experts=1, shared_scale=1, top_k=4,
                           expert_dim=160, T=4, dtype="bf16"),
    "dreamer_parallel": _cfg(batch=4, seq=2048, dim=1024, n_heads=16, n_kv_heads=4, head_dim=64,
                             da_heads=16, da_kv_heads=4, da_head_dim=64, parallel=1, n_experts=16,
                             n_shared_experts=1, shared_scale=1, top_k=2, expert_dim=1408, T=8,
                             lora_rank=16, n_lora=8, dtype="bf16"),
    "parallel_lora_small": _cfg(batch=2, seq=66, dim=256, n_heads=8, n_kv_heads=2, head_dim=32,
                                da_heads=4, da_kv_heads=2, da_head_dim=32, parallel=1, n_experts=8,
                                n_shared_experts=1, shared_scale=1, top_k=2, expert_dim=160, T=5,
                                lora_rank=16, n_lora=3, dtype="bf16"),
    "parallel_act_small": _cfg(batch=3, seq=70, dim=256, n_heads=4, n_kv_heads=2, head_dim=64,
                               parallel=1, n_experts=8, top_k=2, expert_dim=192, T=8,
                               lora_rank=8, n_lora=4, act=True, dtype="bf16"),
    "dreamer_tiny": _cfg(batch=1, seq=32, dim=64, n_heads=4, n_kv_heads=2, head_dim=16,
                         da_heads=2, da_kv_heads=1, da_head_dim=16, n_experts=4,
                         n_shared_experts=1, shared_scale=1, top_k=2, expert_dim=128, T=5,
                         dtype="f32", a_range=(0.5, 0.9)),
}


def get_config(name: str, **overrides) -> dict:
    """A copy of a named workload, with optional field overrides."""
    c = copy.deepcopy(WORKLOADS[name])
    c["name"] = name
    for k, v in overrides.items():
        if k not in c:
            raise KeyError(k)
        c[k] = v
    return c


def n_tokens(cfg: dict) -> int:
    return int(cfg["batch"]) * int(cfg["seq"])


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 out."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are exact bfloat16 numbers."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not representable in bfloat16")
    return (u >> 16).astype(np.uint16)


def weight_shapes(cfg: dict) -> list[tuple[str, tuple[int, ...]]]:
    """(name, shape) of every projection weight, in struct field order."""
    D, H = cfg["dim"], cfg["n_heads"]
    E, F, Se = cfg["n_experts"], cfg["expert_dim"], cfg["n_shared_experts"]
    out = []
    if cfg["attn"] == "gqa":
        d, KV = cfg["head_dim"], cfg["n_kv_heads"]
        out += [("Wq", (H * d, D)), ("Wk", (KV * d, D)), ("Wv", (KV * d, D)),
                ("Wo", (D, H * d))]
    else:
        ql, kvl = cfg["q_lora_rank"], cfg["kv_lora_rank"]
        r, nope, v = cfg["qk_rope_head_dim"], cfg["qk_nope_head_dim"], cfg["v_head_dim"]
        out += [("Wdq", (ql, D)), ("Wuq", (H * (nope + r), ql)),
                ("Wdkv", (kvl + r, D)), ("Wuk", (H * nope, kvl)),
                ("Wuv", (H * v, kvl)), ("Wo", (D, H * v))]
    out += [("Wr", (E, D)), ("Wg", (E, F, D)), ("Wu", (E, F, D)), ("Wd", (E, D, F))]
    if Se:
        out += [("Wsg", (Se, F, D)), ("Wsu", (Se, F, D)), ("Wsd", (Se, D, F))]
    return out


def attn_out_dim(cfg: dict) -> int:
    """Width of the concatenated attention output that feeds the output projection."""
    if cfg["attn"] == "gqa":
        return cfg["n_heads"] * cfg["head_dim"]
    return cfg["n_heads"] * cfg["v_head_dim"]


def make_inputs(cfg: dict) -> dict:
    """Draw every input of one workload from PCG64 with the workload's seed.

    Returns a dict of float32 numpy arrays: A, B [D]; e, h0 [N, D]; g1, g2 [D];
    the projection weights; router_bias [n_bias_rows, E]; lora_down [n_lora, r, Hv],
    lora_up [n_lora, D, r] when lora_rank > 0; w_halt [D] when ACT is on; and
    gq [q_lora_rank], gkv [kv_lora_rank] for MLA.
    """
    rng = np.random.default_rng(int(cfg.get("seed", 0)))
    D, N = cfg["dim"], n_tokens(cfg)
    bf16 = cfg["dtype"] == "bf16"
    rnd = round_bf16 if bf16 else (lambda a: np.ascontiguousarray(a, np.float32))

    out = {}
    lo, hi = cfg["a_range"]
    out["A"] = rng.uniform(lo, hi, size=D).astype(np.float32)
    lo, hi = cfg["b_range"]
    out["B"] = rng.uniform(lo, hi, size=D).astype(np.float32)
    out["e"] = rng.standard_normal((N, D), dtype=np.float32)
    out["h0"] = out["e"].copy()
    out["g1"] = np.ones(D, np.float32)
    out["g2"] = np.ones(D, np.float32)
    if cfg["attn"] == "mla":
        out["gq"] = np.ones(cfg["q_lora_rank"], np.float32)
        out["gkv"] = np.ones(cfg["kv_lora_rank"], np.float32)
    for name, shape in weight_shapes(cfg):
        std = cfg["w_std"]
        if name == "Wr" and cfg["router_std"] is not None:
            std = 1.0 / np.sqrt(D)
        w = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
        out[name] = rnd(w)
    E = cfg["n_experts"]
    if cfg["bias_std"]:
        b = rng.standard_normal((cfg["n_bias_rows"], E), dtype=np.float32)
        out["router_bias"] = (b * np.float32(cfg["bias_std"])).astype(np.float32)
    else:
        out["router_bias"] = np.zeros((cfg["n_bias_rows"], E), np.float32)
    if cfg["lora_rank"]:
        r, L, Hv = cfg["lora_rank"], cfg["n_lora"], attn_out_dim(cfg)
        s = np.float32(cfg["lora_std"])
        out["lora_down"] = rnd(rng.standard_normal((L, r, Hv), dtype=np.float32) * s)
        out["lora_up"] = rnd(rng.standard_normal((L, D, r), dtype=np.float32) * s)
    if cfg["act"]:
        out["w_halt"] = (rng.standard_normal(D, dtype=np.float32)
                         * np.float32(cfg["halt_std"])).astype(np.float32)
    if cfg["da_heads"]:
        Hd, KVd, dd = cfg["da_heads"], cfg["da_kv_heads"], cfg["da_head_dim"]
        out["g_da"] = np.ones(D, np.float32)
        for name, shape in [("Wq_da", (Hd * dd, D)), ("Wk_da", (KVd * dd, D)),
                            ("Wv_da", (KVd * dd, D)), ("Wo_da", (D, Hd * dd))]:
            w = rng.standard_normal(shape, dtype=np.float32) * np.float32(cfg["w_std"])
            out[name] = rnd(w)
    return out
