"""CPU oracle for the recurrent-depth block -- TEST INFRASTRUCTURE ONLY.

A plain, slow float64 NumPy implementation of what the GPU path computes, used to
check it. Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product path never does, and this package imports
nothing from the product.

Sources (the web pages on OpenMythos and on depth-recurrent attention mixtures):
  * techbriefly, "Projeto OpenMythos ...": the Prelude / Recurrent Block / Coda
    split, the loop update h_{t+1} = A h_t + B e + Transformer(h_t, e), one MoE
    layer per iteration with a different expert selection per iteration,
    multi-latent attention, spectral radius of A below 1, ACT halting and
    depth-wise LoRA adapters.
  * openclawapi, "Introducao ao OpenMythos", Passo 2 (config fields: heads,
    kv heads, experts, shared experts, experts per token, expert_dim, lora_rank),
    Passo 5 (MLA latent ranks, decoupled rope/nope head dims; GQA kv heads),
    Passo 6 (A is a per-channel vector; rho(A) < 1 is asserted), troubleshooting
    item 4 (act_threshold 0.99: a position leaves once it has accumulated 99%),
    item 5 (router bias, DeepSeek-style balancing).
  * gist.science summary of "Depth-Recurrent Attention Mixtures", Metodologia:
    RMSNorm on the residual stream, sequential attention -> expert sublayers,
    top-k routing with a bias vector, an always-on shared expert.

Pinned by tests/test_oracle_pins.py (closed form of the injection, T=1 against an
independent torch block, GQA = MHA, k = E dense MoE, MLA explicit = absorbed,
float64 scalar brute force, causality, RoPE relativity, router invariants, ACT
special cases, LoRA merge; the router-bias update on hand-worked counts and
on the dead-expert case of troubleshooting item 5). Parity unpinned: nothing on the pages prints a value
of a full random-weight block, so beyond those pins the oracle is its own
reference.
"""
from .rdt_oracle import (  # noqa: F401
    rmsnorm, rope_tables, apply_rope, attention_causal, gqa_attention,
    mla_attention_explicit, swiglu, route, moe, block_step, forward,
    spectral_radius, kv_cache_bytes_per_token, step_rows,
    bias_row_counts, router_bias_update, expert_depths, depth_rope, depth_attention,
)
