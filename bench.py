#!/usr/bin/env python3
"""Recurrent-block throughput on one MI355X.

One step = one rdt_recurrent_forward: the whole T-loop of the recurrent block
(RMSNorm, causal attention, output projection, router, grouped SwiGLU experts,
combine + LTI injection) over one batch of seeded synthetic inputs that are
already resident in HBM, replayed as a captured HIP graph.

Default workload (the largest recurrent-block configuration that fits one GPU):
wide_moe -- batch 2, seq 4096, dim 2048, GQA 16/4 heads of 128, 64 routed
experts top-8 plus one shared expert with SwiGLU hidden 1024, T = 16, bf16
weights and activations with fp32 accumulation and fp32 state.

Prints one JSON line. `value` is token-loops per second (tokens through one
loop each, per forward); `roofline` describes the dominant kernel (the grouped
gate/up expert GEMM, MFMA-bound), timed with HIP events around its launches on
the stream they run on; `kernels` gives the same for the other kernels (the
router and the combine against HBM bandwidth); `extras` measures the other
workloads; `cpu_baseline` times the float64 CPU oracle on the host's cores.
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
        # the query absorb and the value up-projection run inside the bf16
        # attention launch, so they are counted with it (fp32 runs the absorb
        # as a launch of its own)
        f["qkv"] = 2 * D * (ql + kvl + nr) + 2 * ql * H * (nope + nr)
        f["attention"] = 2 * H * nope * kvl + 2 * H * (kvl + nr) * keys + 2 * H * kvl * keys + 2 * H * kvl * vd
        hv = H * vd
    f["out_proj"] = 2 * hv * D + (2 * cfg["lora_rank"] * (hv + D) if cfg["lora_rank"] else 0)
    f["router"] = 2 * D * cfg["n_experts"]
    f["experts"] = (cfg["top_k"] + cfg["n_shared_experts"]) * 6 * D * cfg["expert_dim"]
    return f


def gate_up_kernel(cfg: dict) -> str:
    """Name of the gate/up launch the library picks for this workload: fp32
    128x128; bf16 64x64 under 64 rows per expert, 160x128 up to 128, the
    eight-wave 256x256 ping-pong tile from 256 rows when the launch has at
    least four rounds of such tiles over 256 CUs, else 192x128 (the tile rule
    of the library's host code)."""
    if cfg["dtype"] == "f32":
        return "k_grouped_gemm<f32,128,128,0,2,4>"
    rows = cfg["batch"] * cfg["seq"] * cfg["top_k"] / cfg["n_experts"]
    if rows < 64:
        return "k_grouped_gemm<bf16,64,64,0,3,4>"
    n_tok = cfg["batch"] * cfg["seq"]
    mt = n_tok * cfg["top_k"] // 256 + cfg["n_experts"] // 2 + cfg["n_shared_experts"] * -(-n_tok // 256)
    if rows >= 256 and mt * -(-cfg["expert_dim"] // 128) >= 4 * 256:
        return "k_grouped_gemm<bf16,256,256,0,2,8>"
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


def gate_up_flops(cfg: dict, counts_per_loop) -> float:
    """Algorithmic FLOPs of the grouped gate/up GEMM, averaged per launch: every
    routed row and every shared-expert row costs gate and up projections,
    2 * 2 * D * F."""
    D, F = cfg["dim"], cfg["expert_dim"]
    tot = 0.0
    for counts in counts_per_loop:
        rows = int(sum(counts))
        tot += 4.0 * D * F * (rows + cfg["n_shared_experts"] * (rows // cfg["top_k"]))
    return tot / max(1, len(counts_per_loop))


def down_flops(cfg: dict, counts_per_loop) -> float:
    """Algorithmic FLOPs of the grouped down projection per launch (2 * D * F per row)."""
    return gate_up_flops(cfg, counts_per_loop) / 2.0


def active_rows(cfg: dict, counts_per_loop):
    """Tokens that ran each loop (routed rows / top-k)."""
    return [int(sum(c)) // cfg["top_k"] for c in counts_per_loop]


def router_bytes(cfg: dict, counts_per_loop, elt: int) -> float:
    """Algorithmic HBM bytes of the fused second RMSNorm + router launch per
    loop, averaged: per running token it reads h, e and the attention-branch
    output a (float32), writes n2 (storage type), and writes k expert indices,
    gates and slots (int32/float32) plus the top-k gap (float32); the router
    weights E x D are read once."""
    D, E, k = cfg["dim"], cfg["n_experts"], cfg["top_k"]
    extra = 4 * D if cfg.get("da_heads") and not cfg.get("parallel") else 0   # depth-attention output
    tot = 0.0
    for n in active_rows(cfg, counts_per_loop):
        tot += n * (12 * D + extra + elt * D + 12 * k + 4) + E * D * elt
    return tot / max(1, len(counts_per_loop))


def combine_bytes(cfg: dict, counts_per_loop, elt: int, ksplit: int = 1) -> float:
    """Algorithmic HBM bytes of the combine + injection launch per loop,
    averaged: per running token it reads h, e, a (float32), its k routed
    expert outputs and the shared experts' outputs (storage type, or float32
    partial sums per K slice), and its k indices, slots and gates; it writes h'
    (float32) and the next loop's RMSNorm(h' + e) (storage type; not after the
    last loop); with ACT it reads and writes the halting sum."""
    D, k, Se, T = cfg["dim"], cfg["top_k"], cfg["n_shared_experts"], len(counts_per_loop)
    ybytes = D * (k + Se) * (4 * ksplit if ksplit > 1 else elt)
    tot = 0.0
    for t, n in enumerate(active_rows(cfg, counts_per_loop)):
        per = 12 * D + ybytes + 12 * k + 4 * D + (elt * D if t + 1 < T else 0) + (8 if cfg["act"] else 0)
        if cfg.get("da_heads"):
            per += 4 * D
        tot += n * per
    return tot / max(1, T)


def host_info() -> dict:
    """Threads the BLAS pools use, the CPU model and the BLAS library."""
    info = {"cpu_count": os.cpu_count(), "cpu_model": None, "blas": None, "threads": os.cpu_count() or 1}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        import numpy as np
        from threadpoolctl import threadpool_info
        np.ones((2, 2)) @ np.ones((2, 2))
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if pools:
            info["threads"] = max(int(p.get("num_threads", 1)) for p in pools)
            info["blas"] = ", ".join(f"{p.get('internal_api')} {p.get('version')}" for p in pools)
    except Exception:
        pass
    return info


def cpu_baseline(cfg: dict, inputs: dict) -> dict:
    """Time the float64 CPU oracle on this host: one loop (T = 1) of the
    workload over every token (a bounded sample of the T-loop; token-loops per
    second do not depend on the loop index)."""
    from oracle import rdt_oracle
    hi = host_info()
    N = cfg["batch"] * cfg["seq"]
    t0 = time.perf_counter()
    rdt_oracle.forward(cfg, inputs, T=1)
    dt = time.perf_counter() - t0
    return {"value": round(N / dt, 1), "unit": "token-loops/s", "cores": hi["threads"], "kind": "oracle",
            "sample": f"one loop (T=1) of the {cfg['name']} workload over all {N} tokens in float64 NumPy, "
                      f"{dt:.1f} s",
            "cpu_model": hi["cpu_model"], "cpu_count": hi["cpu_count"], "blas": hi["blas"]}


def unforced_routing(cfg: dict, inputs: dict, route_idx, h_gpu, P: int = 64) -> dict:
    """For information: the float64 oracle run unforced on the first P
    positions of sequence 0 (causal, so they do not depend on later ones)
    against the GPU's routing of the same tokens: the share of (token, loop)
    pairs whose expert set differs, and max|dh_T| / RMS over the tokens whose
    routing never differed."""
    import numpy as np
    from oracle import rdt_oracle
    T = route_idx.shape[0]
    sub = dict(inputs)
    sub["e"], sub["h0"] = inputs["e"][:P], inputs["h0"][:P]
    ref = rdt_oracle.forward(dict(cfg, batch=1, seq=P), sub, T=T, record=True)
    flips = np.zeros(P, bool)
    pairs = 0
    for t in range(T):
        go, gg = ref["idx"][t], route_idx[t][:P]
        run = (go[:, 0] >= 0) & (gg[:, 0] >= 0)
        diff = run & ~np.all(np.sort(go, 1) == np.sort(gg, 1), axis=1)
        flips |= diff
        pairs += int(np.sum(diff))
    hT = ref["h"][-1]
    keep = ~flips
    scale = float(np.sqrt(np.mean(hT ** 2)))
    dev = float(np.max(np.abs(h_gpu[:P][keep] - hT[keep]))) / scale if keep.any() else None
    return {"tokens": P, "loops": T, "flip_rate": round(pairs / (P * T), 5),
            "tokens_ever_flipped": int(flips.sum()),
            "max_dh_over_rms_unflipped": None if dev is None else round(dev, 6)}


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


class Run:
    """One workload on the device: weights, a graph-mode block, its workspace,
    and one forward with the per-loop counts (and routing dumps) recorded."""

    def __init__(self, name: str, routing_dumps: bool = False):
        import torch

        import recurrent_depth_transformer_amd as rdt
        from rdt_inputs import get_config, make_inputs
        self.cfg = cfg = get_config(name)
        self.T, self.N = cfg["T"], cfg["batch"] * cfg["seq"]
        self.inputs = make_inputs(cfg)
        self.W = rdt.device_weights(self.inputs, cfg, "cuda")
        self.blk = rdt.RecurrentBlock(cfg, graph=True)
        self.out = torch.empty_like(self.W["h0"])
        self.ws = self.blk.workspace(self.T)
        self.stream = torch.cuda.current_stream()
        T, N = self.T, self.N
        aux = {"loops": torch.empty(N, dtype=torch.int32, device="cuda"),
               "expert_counts": torch.empty(T, cfg["n_experts"], dtype=torch.int32, device="cuda")}
        if routing_dumps:
            aux["route_idx"] = torch.empty(T, N, cfg["top_k"], dtype=torch.int32, device="cuda")
            aux["route_gap"] = torch.empty(T, N, dtype=torch.float32, device="cuda")
        self.blk.forward(self.W["h0"], self.W["e"], self.W, T=T, out=self.out, workspace=self.ws, aux=aux)
        torch.cuda.synchronize()
        self.executed = int(aux["loops"].sum().item())
        self.counts = aux["expert_counts"].cpu().numpy()
        self.route_idx = aux["route_idx"].cpu().numpy() if routing_dumps else None
        self.route_gap = aux["route_gap"].cpu().numpy() if routing_dumps else None
        self.h = self.out.cpu().numpy() if routing_dumps else None

    def step(self):
        self.blk.forward(self.W["h0"], self.W["e"], self.W, T=self.T, out=self.out, workspace=self.ws)

    def stages(self, n: int) -> dict:
        """{stage: (mean device ms per launch, launches per forward)} from n
        kernel-by-kernel forwards with HIP events around every launch."""
        acc = {}
        for _ in range(max(1, n)):
            _, st = self.blk.profile_forward(self.W["h0"], self.W["e"], self.W, T=self.T, out=self.out,
                                             workspace=self.ws)
            for k, (t_ms, c) in st.items():
                a = acc.setdefault(k, [0.0, 0])
                a[0] += t_ms
                a[1] += c
        return {k: (v[0] / v[1] if v[1] else 0.0, v[1] // max(1, n)) for k, v in acc.items()}


def kernel_figures(cfg: dict, counts, stage_avg: dict, elt: int, peak_tf: float) -> dict:
    """Per-kernel roofline figures from the per-stage launch times: the GEMMs
    and attention against the MFMA peak, the router and combine against HBM.
    A stage's time per loop is its mean launch time times its launches per
    loop (the MLA attention stage also holds the query absorb and the value
    up-projection; their FLOPs are counted with it)."""
    fl = flops_per_token_loop(cfg)
    rows = active_rows(cfg, counts)
    mean_rows = sum(rows) / max(1, len(rows))
    T = max(1, len(counts))
    out = {}

    def per_loop_us(stage):
        avg_ms, n = stage_avg.get(stage, (0.0, 0))
        return avg_ms * 1e3 * n / T, n / T

    def mfma(stage, flops):
        us, lpl = per_loop_us(stage)
        if us <= 0:
            return
        out[stage] = {"bound": "mfma", "us_per_loop": round(us, 2), "launches_per_loop": round(lpl, 3),
                      "algorithmic_flops_per_loop": int(flops),
                      "achieved_TFLOPs": round(flops / (us * 1e-6) / 1e12, 1),
                      "frac": round(flops / (us * 1e-6) / 1e12 / peak_tf, 4)}

    def hbm(stage, nbytes):
        us, lpl = per_loop_us(stage)
        if us <= 0:
            return
        out[stage] = {"bound": "hbm", "us_per_loop": round(us, 2), "launches_per_loop": round(lpl, 3),
                      "algorithmic_bytes_per_loop": int(nbytes),
                      "achieved_GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                      "frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}

    mfma("expert_gate_up", gate_up_flops(cfg, counts))
    mfma("expert_down", down_flops(cfg, counts))
    mfma("qkv", fl["qkv"] * mean_rows)
    mfma("attention", fl["attention"] * mean_rows)
    mfma("out_proj", fl["out_proj"] * mean_rows)
    hbm("router", router_bytes(cfg, counts, elt))
    hbm("combine", combine_bytes(cfg, counts, elt, ksplit_of(cfg)))
    return out


def ksplit_of(cfg: dict) -> int:
    """K slices of the down projection the library picks (bf16: at most 32
    64-wide stages per slice; fp32 does not slice)."""
    if cfg["dtype"] == "f32":
        return 1
    stages = (cfg["expert_dim"] + 63) // 64
    return (stages + 31) // 32


def measure_extra(name: str, steps: int, stream) -> dict:
    """Forward throughput of another workload and its per-kernel figures."""
    r = Run(name)
    ms = _time(r.step, steps, 3, r.stream)
    st = r.stages(2)
    elt = 4 if r.cfg["dtype"] == "f32" else 2
    peak = PEAK_F32_TFLOPS if r.cfg["dtype"] == "f32" else PEAK_BF16_TFLOPS
    flops = sum(flops_per_token_loop(r.cfg).values()) * r.executed
    res = {"workload": describe(r.cfg), "ms_per_step": round(ms, 4), "value": round(r.executed / (ms * 1e-3), 1),
           "unit": "token-loops/s", "token_loops_per_step": r.executed,
           "mfma_peak_frac": round(flops / (ms * 1e-3) / (peak * 1e12), 5),
           "kernels": kernel_figures(r.cfg, r.counts, st, elt, peak),
           "stages_us": {k: round(v[0] * 1e3, 2) for k, v in st.items() if v[1]}}
    if r.cfg["act"]:
        res["nominal_token_loops_per_step"] = r.N * r.T
    if r.cfg.get("da_heads"):
        da_us = st["depth_attention"][0] * 1e3
        nbytes = depth_attention_bytes(r.cfg, elt)
        achieved = nbytes / (da_us * 1e-6) / 1e9
        res["depth_attention"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                                  "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                                  "avg_launch_us": round(da_us, 2), "algorithmic_bytes_per_launch": int(nbytes)}
    del r
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wide_moe")
    ap.add_argument("--profile-steps", type=int, default=4, help="eager forwards timed per stage")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stages", action="store_true", help="also print the per-stage breakdown to stderr")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other workloads, the decode step and the machine calibration")
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

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    run = Run(args.workload, routing_dumps=True)
    cfg, T, N = run.cfg, run.T, run.N
    stream = run.stream
    print(f"[bench] {describe(cfg)}; warmup {args.warmup}, steps {args.steps}", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        run.step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        run.step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    value = run.executed / (ms * 1e-3)
    print(f"[bench] {ms:.4f} ms per forward (wall {wall * 1e3 / args.steps:.4f} ms)", file=sys.stderr, flush=True)
    # spread of single steps (an event pair around each forward, after the timed run)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a_, b_ in evs:
        a_.record(stream)
        run.step()
        b_.record(stream)
    torch.cuda.synchronize()
    single = np.array([a_.elapsed_time(b_) for a_, b_ in evs])
    step_ms = {"median": round(float(np.median(single)), 5), "p10": round(float(np.percentile(single, 10)), 5),
               "p90": round(float(np.percentile(single, 90)), 5)}

    # per-stage device time: kernels launched one by one with HIP events around
    # each launch on the launch stream
    stage_avg = run.stages(args.profile_steps)
    if args.stages:
        for k, (avg, n) in stage_avg.items():
            print(f"[stage] {k:16s} {avg * 1e3:9.2f} us/launch x {n}", file=sys.stderr)

    elt = 4 if cfg["dtype"] == "f32" else 2
    fl = flops_per_token_loop(cfg)
    flops = sum(fl.values()) * run.executed
    peak_tf = PEAK_F32_TFLOPS if cfg["dtype"] == "f32" else PEAK_BF16_TFLOPS
    kernels = kernel_figures(cfg, run.counts, stage_avg, elt, peak_tf)
    gu = kernels[DOMINANT_STAGE]   # one launch per loop
    roofline = {"bound": "mfma", "achieved": gu["achieved_TFLOPs"], "peak": peak_tf, "unit": "TFLOP/s",
                "frac": gu["frac"], "traffic": traffic_from_profiles(args.workload),
                "kernel": gate_up_kernel(cfg) + " (expert gate/up + SwiGLU)",
                "avg_launch_us": gu["us_per_loop"], "algorithmic_flops_per_launch": gu["algorithmic_flops_per_loop"],
                "algorithmic_bytes_per_launch": int(gate_up_bytes(cfg, run.counts, elt))}
    gaps = run.route_gap
    routing = {"near_ties_per_loop": [int(np.sum(gaps[t][np.isfinite(gaps[t])] < 1e-3)) for t in range(T)],
               "routed_tokens_per_loop": [int(x) for x in active_rows(cfg, run.counts)]}

    calibration = extras = None
    if not args.no_extras:
        calibration = machine_calibration(stream)
        extras = {}
        for name in ["gqa", "mla", "act", "dreamer", "dreamer_parallel"]:
            if name == args.workload:
                continue
            print(f"[bench] extra workload {name}", file=sys.stderr, flush=True)
            extras[name] = measure_extra(name, max(5, args.steps // 3), stream)
        print("[bench] decode step (gqa)", file=sys.stderr, flush=True)
        extras["decode"] = bench_decode(args, "gqa")

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, run.inputs)
        print("[bench] unforced routing on a causal prefix (oracle)", file=sys.stderr, flush=True)
        routing["unforced"] = unforced_routing(cfg, run.inputs, run.route_idx, run.h)

    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "token-loops/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg["dtype"],
        "data": "synthetic (seeded PCG64 draws, random-init weights)",
        "config": {"workload": describe(cfg), "batch": cfg["batch"], "seq": cfg["seq"], "dim": cfg["dim"],
                   "T": T, "token_loops_per_step": run.executed, "parallelism": "single GPU"},
        "mfma_peak_frac": round(flops / (ms * 1e-3) / (peak_tf * 1e12), 5),
        "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "routing": routing,
        "stages_us": {k: round(v[0] * 1e3, 2) for k, v in stage_avg.items() if v[1]},
        "step_ms": step_ms,
        "calibration": calibration,
        "extras": extras,
    }
    print(json.dumps(res), flush=True)


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


def bench_decode(args, name: str) -> dict:
    """One-token decode step: prefill seq-1 positions, then time steps at the
    last position (each step rewrites the same cache row, so every step does
    the same work)."""
    import torch

    import recurrent_depth_transformer_amd as rdt
    from rdt_inputs import get_config, make_inputs
    cfg = get_config(name)
    W = rdt.device_weights(make_inputs(cfg), cfg, "cuda")
    stream = torch.cuda.current_stream()
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


if __name__ == "__main__":
    main()
