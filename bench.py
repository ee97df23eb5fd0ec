#!/usr/bin/env python3
"""Recurrent-block throughput on one MI355X.

One step = one rdt_recurrent_forward: the whole T-loop of the recurrent block
(RMSNorm, causal attention, output projection, router, grouped SwiGLU experts,
combine + LTI injection) over one batch of seeded synthetic inputs that are
already resident in HBM, replayed as a captured HIP graph.

Default workload: the GQA recurrent block -- batch 1, seq 512, dim 1024, 16/4
heads of 64, 8 experts top-2 with SwiGLU hidden 2816, T = 3, bf16 weights and
activations with fp32 accumulation and fp32 state.

Prints one JSON line. `value` is token-loops per second (batch*seq*T tokens
through one loop each, per forward); `roofline` describes the dominant kernel
(the grouped gate/up expert GEMM), timed with HIP events around its launches on
the stream they run on; `cpu_baseline` times the float64 CPU oracle on the
host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "recurrent-block token-loops/sec at 1 MI355X; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
DOMINANT_STAGE = "expert_gate_up"
DOMINANT_SOURCES = ["rdt_gemm.hip", "rdt_device.h"]


def describe(cfg: dict) -> str:
    att = (f"GQA {cfg['n_heads']}/{cfg['n_kv_heads']} heads of {cfg['head_dim']}" if cfg["attn"] == "gqa"
           else f"MLA {cfg['n_heads']} heads, kv latent {cfg['kv_lora_rank']}+rope {cfg['qk_rope_head_dim']}, "
                f"q latent {cfg['q_lora_rank']}")
    moe = f"{cfg['n_experts']} experts top-{cfg['top_k']}"
    if cfg["n_shared_experts"]:
        moe += f" + {cfg['n_shared_experts']} shared"
    extra = ""
    if cfg["lora_rank"]:
        extra += f", depth-wise LoRA r{cfg['lora_rank']}"
    if cfg["act"]:
        extra += f", ACT halting at {cfg['act_threshold']}"
    if cfg.get("da_heads"):
        extra += f", depth attention {cfg['da_heads']}/{cfg['da_kv_heads']} of {cfg['da_head_dim']}"
    if cfg.get("parallel"):
        extra += ", parallel sublayers"
    if cfg.get("shared_scale"):
        extra += ", shared expert weighted by the max router probability"
    return (f"{cfg['name']}: batch {cfg['batch']}, seq {cfg['seq']}, dim {cfg['dim']}, {att}, {moe}, "
            f"SwiGLU hidden {cfg['expert_dim']}, T={cfg['T']}{extra}, {cfg['dtype']}")


def flops_per_token_loop(cfg: dict) -> dict:
    """Algorithmic FLOPs of one token through one loop (causal attention counts
    the average (S+1)/2 visible keys; MLA is counted in absorbed form)."""
    D, H, S = cfg["dim"], cfg["n_heads"], cfg["seq"]
    keys = (S + 1) / 2.0
    f = {}
    if cfg["attn"] == "gqa":
        d, KV = cfg["head_dim"], cfg["n_kv_heads"]
        f["qkv"] = 2 * D * (H + 2 * KV) * d
        f["attention"] = 2 * 2 * H * d * keys
        hv = H * d
    else:
        ql, kvl, nr = cfg["q_lora_rank"], cfg["kv_lora_rank"], cfg["qk_rope_head_dim"]
        nope, vd = cfg["qk_nope_head_dim"], cfg["v_head_dim"]
        f["qkv"] = 2 * D * (ql + kvl + nr) + 2 * ql * H * (nope + nr) + 2 * H * nope * kvl
        f["attention"] = 2 * H * (kvl + nr) * keys + 2 * H * kvl * keys + 2 * H * kvl * vd
        hv = H * vd
    f["out_proj"] = 2 * hv * D + (2 * cfg["lora_rank"] * (hv + D) if cfg["lora_rank"] else 0)
    f["router"] = 2 * D * cfg["n_experts"]
    f["experts"] = (cfg["top_k"] + cfg["n_shared_experts"]) * 6 * D * cfg["expert_dim"]
    return f


def gate_up_kernel(cfg: dict) -> str:
    """Name of the gate/up launch the library picks for this workload: fp32
    128x128; bf16 64x64 under 64 rows per expert, 160x128 up to 128, else
    192x128 (the tile rule of the library's host code)."""
    if cfg["dtype"] == "f32":
        return "k_grouped_gemm<f32,128,128,0,2,4>"
    rows = cfg["batch"] * cfg["seq"] * cfg["top_k"] / cfg["n_experts"]
    if rows < 64:
        return "k_grouped_gemm<bf16,64,64,0,3,4>"
    return "k_grouped_gemm<bf16,160,128,0,2,4>" if rows <= 128 else "k_grouped_gemm<bf16,192,128,0,2,4>"


def gate_up_bytes(cfg: dict, counts_per_loop, elt: int) -> float:
    """Algorithmic HBM bytes of the grouped gate/up GEMM, averaged per launch:
    the gate and up matrices of every expert that received a row (and of every
    shared expert), the routed rows read once, the SwiGLU output written once."""
    D, F = cfg["dim"], cfg["expert_dim"]
    tot = 0.0
    for counts in counts_per_loop:
        rows = int(sum(counts))
        n_tok = rows // cfg["top_k"]
        used = sum(1 for c in counts if c > 0) + cfg["n_shared_experts"]
        all_rows = rows + cfg["n_shared_experts"] * n_tok
        tot += used * 2 * F * D * elt + all_rows * D * elt + all_rows * F * elt
    return tot / max(1, len(counts_per_loop))


def decode_step_bytes(cfg: dict, route_idx, pos: int, elt: int) -> float:
    """Algorithmic HBM bytes of one decode step (one token per sequence through
    T loops): per loop the attention and router weights, the gate/up/down
    matrices of every expert some token chose (and the shared experts), the
    cached keys/values of positions 0..pos, and the state rows."""
    D, F, B, T = cfg["dim"], cfg["expert_dim"], cfg["batch"], cfg["T"]
    H, KV, d = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    attn_w = (H * d + 2 * KV * d) * D + D * H * d
    tot = 0.0
    for t in range(T):
        used = len({int(x) for x in route_idx[t].reshape(-1) if x >= 0}) + cfg["n_shared_experts"]
        tot += (attn_w + cfg["n_experts"] * D) * elt + used * 3 * F * D * elt
        tot += B * (pos + 1) * 2 * KV * d * elt + B * D * 4 * 4
    return tot


def depth_attention_bytes(cfg: dict, elt: int) -> float:
    """Algorithmic bytes of one depth-attention launch, averaged over loops:
    every token reads its query, the keys and values of loops 0..t and writes
    its output (mean t + 1 = (T + 1) / 2)."""
    N, T = cfg["batch"] * cfg["seq"], cfg["T"]
    Hd, KVd, dd = cfg["da_heads"], cfg["da_kv_heads"], cfg["da_head_dim"]
    return N * (2 * Hd * dd + (T + 1) / 2 * 2 * KVd * dd) * elt


def source_hash(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "recurrent_depth_transformer_amd", "csrc", n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str):
    """Per-launch HBM bytes of the dominant kernel from committed rocprofv3
    counter runs, or None when absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"expert_gate_up_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_hash") != source_hash(DOMINANT_SOURCES):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(cfg: dict, inputs: dict, T: int, budget_s: float):
    """Time the float64 CPU oracle on this host (repeats of the full forward
    until the budget is used, at least one)."""
    import numpy as np  # noqa: F401
    from oracle import rdt_oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(p.get("num_threads", 1)) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    runs, t_used = 0, 0.0
    while runs == 0 or (t_used < budget_s and runs < 50):
        t0 = time.perf_counter()
        rdt_oracle.forward(cfg, inputs, T=T)
        t_used += time.perf_counter() - t0
        runs += 1
    N = cfg["batch"] * cfg["seq"]
    return {"value": N * T * runs / t_used, "unit": "token-loops/s", "cores": threads, "kind": "oracle",
            "sample": f"{runs} full forward(s) of the {cfg['name']} workload (T={T}, {N} tokens) in float64 "
                      f"NumPy, {t_used:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gqa")
    ap.add_argument("--profile-steps", type=int, default=10, help="eager forwards timed per stage")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stages", action="store_true", help="also print the per-stage breakdown to stderr")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the decode-step and depth-attention (dreamer workload) measurements")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (calibrates HBM counters) and exit")
    args = ap.parse_args()
    if args.copy_probe:
        import torch
        x = torch.empty(args.copy_probe // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe, "launches": 3}))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import recurrent_depth_transformer_amd as rdt
    from rdt_inputs import get_config, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    cfg = get_config(args.workload)
    T, N = cfg["T"], cfg["batch"] * cfg["seq"]
    inputs = make_inputs(cfg)
    W = rdt.device_weights(inputs, cfg, "cuda")
    blk = rdt.RecurrentBlock(cfg, graph=True)
    out = torch.empty_like(W["h0"])
    ws = blk.workspace(T)
    stream = torch.cuda.current_stream()
    print(f"[bench] {describe(cfg)}; warmup {args.warmup}, steps {args.steps}", file=sys.stderr, flush=True)

    # executed token-loops (ACT halts tokens early) and per-loop expert counts
    loops = torch.empty(N, dtype=torch.int32, device="cuda")
    counts = torch.empty(T, cfg["n_experts"], dtype=torch.int32, device="cuda")
    blk.forward(W["h0"], W["e"], W, T=T, out=out, workspace=ws, aux={"loops": loops, "expert_counts": counts})
    torch.cuda.synchronize()
    executed = int(loops.sum().item())
    counts_np = counts.cpu().numpy()

    for _ in range(args.warmup):
        blk.forward(W["h0"], W["e"], W, T=T, out=out, workspace=ws)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        blk.forward(W["h0"], W["e"], W, T=T, out=out, workspace=ws)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    value = executed / (ms * 1e-3)
    print(f"[bench] {ms:.4f} ms per forward (wall {wall * 1e3 / args.steps:.4f} ms)", file=sys.stderr, flush=True)
    # spread of single steps (an event pair around each forward, after the timed run)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a_, b_ in evs:
        a_.record(stream)
        blk.forward(W["h0"], W["e"], W, T=T, out=out, workspace=ws)
        b_.record(stream)
    torch.cuda.synchronize()
    single = np.array([a_.elapsed_time(b_) for a_, b_ in evs])
    step_ms = {"median": round(float(np.median(single)), 5), "p10": round(float(np.percentile(single, 10)), 5),
               "p90": round(float(np.percentile(single, 90)), 5)}

    # per-stage device time: kernels launched one by one with HIP events around
    # each launch on the launch stream
    acc = {}
    for _ in range(max(1, args.profile_steps)):
        _, st = blk.profile_forward(W["h0"], W["e"], W, T=T, out=out, workspace=ws)
        for k, (t_ms, n) in st.items():
            a = acc.setdefault(k, [0.0, 0])
            a[0] += t_ms
            a[1] += n
    stage_avg = {k: (v[0] / v[1] if v[1] else 0.0, v[1] // max(1, args.profile_steps)) for k, v in acc.items()}
    if args.stages:
        for k, (avg, n) in stage_avg.items():
            print(f"[stage] {k:16s} {avg * 1e3:9.2f} us/launch x {n}", file=sys.stderr)

    elt = 4 if cfg["dtype"] == "f32" else 2
    fl = flops_per_token_loop(cfg)
    flops = sum(fl.values()) * executed
    peak_tf = PEAK_F32_TFLOPS if cfg["dtype"] == "f32" else PEAK_BF16_TFLOPS
    gu_ms = stage_avg[DOMINANT_STAGE][0]
    gu_bytes = gate_up_bytes(cfg, counts_np, elt)
    achieved = gu_bytes / (gu_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic_from_profiles(args.workload),
                "kernel": gate_up_kernel(cfg) + " (expert gate/up + SwiGLU)",
                "avg_launch_us": round(gu_ms * 1e3, 2), "algorithmic_bytes_per_launch": int(gu_bytes)}

    calibration = None if args.no_extras else machine_calibration(stream)

    extras = None
    if not args.no_extras:
        extras = {"decode": bench_decode(args, cfg, W, stream), "dreamer": bench_dreamer(args)}

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, inputs, T, args.cpu_budget)

    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "token-loops/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg["dtype"],
        "data": "synthetic (seeded PCG64 draws, random-init weights)",
        "config": {"workload": describe(cfg), "batch": cfg["batch"], "seq": cfg["seq"], "dim": cfg["dim"],
                   "T": T, "token_loops_per_step": executed, "parallelism": "single GPU"},
        "mfma_peak_frac": round(flops / (ms * 1e-3) / (peak_tf * 1e12), 5),
        "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "stages_us": {k: round(v[0] * 1e3, 2) for k, v in stage_avg.items() if v[1]},
        "step_ms": step_ms,
        "calibration": calibration,
        "extras": extras,
    }
    print(json.dumps(res), flush=True)


def _time(fn, steps: int, warmup: int, stream) -> float:
    """Mean milliseconds of fn() over `steps` calls after `warmup` calls,
    HIP events on `stream`."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def machine_calibration(stream) -> dict:
    """What this MI355X delivers outside librdt, as context for the roofline
    fractions (which use the published peaks): a 1 GiB device-to-device copy
    (read + write bytes per second) and torch's library bf16 GEMM at
    8192 x 8192 x 8192."""
    import torch
    x = torch.empty(1 << 29, dtype=torch.float16, device="cuda")
    y = torch.empty_like(x)
    copy_ms = _time(lambda: y.copy_(x), 10, 2, stream)
    a = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda")
    c = torch.empty(8192, 8192, dtype=torch.bfloat16, device="cuda")
    mm_ms = _time(lambda: torch.matmul(a, b, out=c), 5, 2, stream)
    del x, y, a, b, c
    torch.cuda.empty_cache()
    return {"copy_GBps": round(2 * (1 << 30) / (copy_ms * 1e-3) / 1e9, 1),
            "library_bf16_gemm_TFLOPs": round(2 * 8192 ** 3 / (mm_ms * 1e-3) / 1e12, 1)}


def bench_decode(args, cfg: dict, W: dict, stream) -> dict:
    """One-token decode step on the bench workload: prefill seq-1 positions,
    then time steps at the last position (each step rewrites the same cache
    row, so every step does the same work)."""
    import torch

    import recurrent_depth_transformer_amd as rdt
    B, S, D, T = cfg["batch"], cfg["seq"], cfg["dim"], cfg["T"]
    blk = rdt.RecurrentBlock(dict(cfg, seq=S - 1), graph=True)
    cache = blk.new_cache(T, S)
    h0, e = W["h0"].view(B, S, D), W["e"].view(B, S, D)
    blk.prefill(h0[:, :S - 1].contiguous().view(-1, D), e[:, :S - 1].contiguous().view(-1, D), W, T, cache, S)
    ht, et = h0[:, S - 1].contiguous(), e[:, S - 1].contiguous()
    out = torch.empty_like(ht)
    ridx = torch.empty(T, B, cfg["top_k"], dtype=torch.int32, device="cuda")
    blk.decode_step(ht, et, W, T, S - 1, cache, S, out=out, aux={"route_idx": ridx})
    torch.cuda.synchronize()
    ms = _time(lambda: blk.decode_step(ht, et, W, T, S - 1, cache, S, out=out), args.steps, args.warmup, stream)
    elt = 4 if cfg["dtype"] == "f32" else 2
    nbytes = decode_step_bytes(cfg, ridx.cpu().numpy(), S - 1, elt)
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"{cfg['name']}: {B} sequence(s), one token at position {S - 1} after a {S - 1}-token "
                        f"prefill, T={T}, per-loop KV cache",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(B / (ms * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                         "kernel": "whole decode step (weights, chosen experts, cache)",
                         "algorithmic_bytes_per_step": int(nbytes)},
            "cache_bytes": blk.cache_size(T, S)}


def bench_dreamer(args) -> dict:
    """Forward throughput of the full-size Dreamer workload (depth attention,
    max-score shared expert) and the roofline of the depth-attention kernel."""
    import torch

    import recurrent_depth_transformer_amd as rdt
    from rdt_inputs import get_config, make_inputs
    cfg = get_config("dreamer")
    T, N = cfg["T"], cfg["batch"] * cfg["seq"]
    W = rdt.device_weights(make_inputs(cfg), cfg, "cuda")
    blk = rdt.RecurrentBlock(cfg, graph=True)
    out = torch.empty_like(W["h0"])
    ws = blk.workspace(T)
    stream = torch.cuda.current_stream()
    steps = max(3, args.steps // 10)
    ms = _time(lambda: blk.forward(W["h0"], W["e"], W, T=T, out=out, workspace=ws), steps, 2, stream)
    _, st = blk.profile_forward(W["h0"], W["e"], W, T=T, out=out, workspace=ws)
    da_ms, da_n = st["depth_attention"]
    da_us = da_ms / max(1, da_n) * 1e3
    elt = 2
    nbytes = depth_attention_bytes(cfg, elt)
    achieved = nbytes / (da_us * 1e-6) / 1e9
    return {"workload": describe(cfg), "ms_per_step": round(ms, 4),
            "value": round(N * T / (ms * 1e-3), 1), "unit": "token-loops/s",
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                         "kernel": "k_depth_attention (Dreamer depth attention)", "avg_launch_us": round(da_us, 2),
                         "algorithmic_bytes_per_launch": int(nbytes)},
            "stages_us": {k: round(v[0] / v[1] * 1e3, 2) for k, v in st.items() if v[1]}}


if __name__ == "__main__":
    main()
