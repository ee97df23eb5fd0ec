"""GPU parity of librdt against the CPU oracle (needs an MI355X)."""
import numpy as np
import pytest

from oracle import rdt_oracle as ro
from rdt_inputs import get_config, make_inputs, n_tokens

from rdt_gpu_run import check_halting, check_routing_teacher_forced, rms, run_gpu

pytestmark = pytest.mark.gpu

TOL = 2e-2  # max |dh| <= TOL * RMS(h_T) after T loops, routing and halting forced


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from recurrent_depth_transformer_amd import load_library
    load_library()


def _report(name, **kw):
    print(f"[parity] {name}: " + ", ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


@pytest.mark.parametrize("name", ["tiny", "gqa_small", "wide_small", "act_small", "mla_small", "dreamer_small",
                                  "parallel_small"])
def test_closed_form_injection(name):
    cfg = get_config(name)
    inp = make_inputs(cfg)
    inp["Wo"] = np.zeros_like(inp["Wo"])
    if cfg["da_heads"]:
        inp["Wo_da"] = np.zeros_like(inp["Wo_da"])
    inp["Wd"] = np.zeros_like(inp["Wd"])
    if cfg["n_shared_experts"]:
        inp["Wsd"] = np.zeros_like(inp["Wsd"])
    if cfg["lora_rank"]:
        inp["lora_up"] = np.zeros_like(inp["lora_up"])
    cfg["act"] = False
    T = 5
    res, *_ = run_gpu(cfg, inp, T=T, dumps=False)
    A, B = inp["A"].astype(np.float64), inp["B"].astype(np.float64)
    closed = A ** T * inp["h0"] + B * inp["e"] * (1 - A ** T) / (1 - A)
    err = np.max(np.abs(res["h"] - closed))
    _report(f"closed-form {name}", max_abs=err)
    assert err <= 1e-5 * max(1.0, np.max(np.abs(closed)))


@pytest.mark.parametrize("name", ["tiny", "tiny_bf16", "gqa_small", "wide_small", "act_small", "mla_small",
                                  "dreamer_tiny", "dreamer_small", "parallel_small", "parallel_lora_small",
                                  "parallel_act_small"])
def test_end_to_end_forced(name):
    cfg = get_config(name)
    T = cfg["T"]
    res, inp, *_ = run_gpu(cfg, T=T)
    mism, near, comp = check_routing_teacher_forced(cfg, inp, res, T, ro)
    forced_loops = res["loops"] if cfg["act"] else None
    ref = ro.forward(cfg, inp, T=T, forced_idx=res["route_idx"], forced_loops=forced_loops)
    err = np.max(np.abs(res["h"] - ref["h"]))
    scale = rms(ref["h"])
    _report(name, max_abs=f"{err:.3e}", rms=f"{scale:.3f}", ratio=f"{err / scale:.3e}",
            route_mismatch=mism, near_ties=near, compared=comp,
            loops_mean=float(np.mean(res["loops"])))
    assert mism == 0
    assert err <= TOL * scale
    if cfg["act"]:
        # halting decisions from the GPU's own states, loop by loop
        bad, _ = check_halting(cfg, inp, res, T)
        assert bad == 0
        assert 0 < res["loops"].min() <= res["loops"].max() <= T


# fp32 versions of the MLA, ACT (with depth-wise LoRA) and Dreamer workloads:
# the fp32 attention (V transposed in LDS, no transpose reads), the fp32 GEMM
# main loop with the LoRA second K phase, and the fp32 router and combine,
# against the oracle at a tolerance fp32 arithmetic can meet.
F32_VARIANTS = {
    "mla_f32": dict(base="mla_small", dtype="f32"),
    "act_f32": dict(base="act_small", dtype="f32"),
    "dreamer_f32": dict(base="dreamer_small", dtype="f32"),
}


@pytest.mark.parametrize("name", sorted(F32_VARIANTS))
def test_fp32_variants_forced(name):
    over = dict(F32_VARIANTS[name])
    cfg = get_config(over.pop("base"), **over)
    T = cfg["T"]
    res, inp, *_ = run_gpu(cfg, T=T)
    mism, near, comp = check_routing_teacher_forced(cfg, inp, res, T, ro)
    ref = ro.forward(cfg, inp, T=T, forced_idx=res["route_idx"], forced_loops=res["loops"] if cfg["act"] else None)
    err = np.max(np.abs(res["h"] - ref["h"]))
    scale = rms(ref["h"])
    _report(name, ratio=f"{err / scale:.3e}", route_mismatch=mism, near_ties=near, compared=comp)
    assert mism == 0
    assert err <= 1e-4 * scale


# The limits of the block: the widest row (dim 4096: 16 float4 per lane and
# more than one router k-chunk), the most routed experts (64) with top-8, the
# pages' maximum of 16 loops, and a ragged sequence length. In bf16 over 16
# loops at this width the rounding of the bf16 operands compounds (each loop
# adds 3e-3..7e-3 of RMS, measured), so the bf16 cases check every loop from
# the GPU's own state; the fp32 case also checks the end state.
LIMITS = {
    "wide_max": dict(base="wide_small", dim=4096, seq=37, n_experts=64, top_k=8, expert_dim=64, T=16,
                     n_bias_rows=16),
    "wide_max_f32": dict(base="wide_small", dim=4096, seq=37, n_experts=64, top_k=8, expert_dim=64, T=16,
                         n_bias_rows=16, dtype="f32"),
    "act_max": dict(base="act_small", dim=4096, seq=37, T=16),
    "mla_max": dict(base="mla_small", dim=4096, seq=37, T=16),
}


@pytest.mark.parametrize("name", sorted(LIMITS))
def test_size_limits_forced(name):
    over = dict(LIMITS[name])
    cfg = get_config(over.pop("base"), **over)
    T = cfg["T"]
    res, inp, *_ = run_gpu(cfg, T=T)
    mism, near, comp = check_routing_teacher_forced(cfg, inp, res, T, ro)
    assert mism == 0
    worst = 0.0
    for t in range(T):
        act = np.nonzero(res["loops"] > t)[0]
        if act.size == 0:
            break
        hn, _, _ = ro.step_rows(cfg, inp, res["h_dump"][t], inp["e"], t, act, res["route_idx"][t][act])
        g = res["h_dump"][t + 1][act]
        worst = max(worst, float(np.max(np.abs(g - hn))) / rms(g))
    _report(name, worst_loop_ratio=f"{worst:.3e}", route_mismatch=mism, near_ties=near, compared=comp)
    assert worst <= TOL
    if cfg["dtype"] == "f32":
        ref = ro.forward(cfg, inp, T=T, forced_idx=res["route_idx"], forced_loops=res["loops"] if cfg["act"] else None)
        err = np.max(np.abs(res["h"] - ref["h"]))
        _report(name, end_ratio=f"{err / rms(ref['h']):.3e}")
        assert err <= 1e-4 * rms(ref["h"])


# Degenerate cases of the method: every expert chosen (k = E: the dense softmax
# mixture, no next-best score), a single expert, one-token sequences (attention
# over one key), one loop.
DEGENERATE = {
    "dense_mixture": dict(base="gqa_small", top_k=8),
    "single_expert": dict(base="gqa_small", n_experts=1, top_k=1),
    "one_token_sequences": dict(base="gqa_small", batch=5, seq=1),
    "one_loop": dict(base="act_small", T=1),
}


# Widths that are multiples of 8 but not of the 64-wide k-stages, the 256- and
# 512-column row chunks or the output tiles: partial last chunks in the row
# kernels, K tails in every GEMM, partial column tiles.
RAGGED = {
    "ragged_width": dict(base="gqa_small", dim=328, expert_dim=200),
    "ragged_width_mla": dict(base="mla_small", dim=200, expert_dim=136),
    "ragged_width_depth": dict(base="dreamer_small", dim=200, expert_dim=120),
    "ragged_width_act": dict(base="act_small", dim=136, expert_dim=264),
    # three 256-column chunks, run by the four-chunk instantiations
    "three_chunk_width": dict(base="gqa_small", dim=640, expert_dim=200),
    # MLA head widths off the MFMA blocks: a half-empty last k-step of the
    # query absorb (nope 40) and a half-empty last block of value columns (24)
    "ragged_heads_mla": dict(base="mla_small", qk_nope_head_dim=40, v_head_dim=24),
}


@pytest.mark.parametrize("name", sorted(RAGGED))
def test_ragged_widths_forced(name):
    test_degenerate_forced(name)


@pytest.mark.parametrize("name", sorted(DEGENERATE))
def test_degenerate_forced(name):
    over = dict(DEGENERATE[name] if name in DEGENERATE else RAGGED[name])
    cfg = get_config(over.pop("base"), **over)
    T = cfg["T"]
    res, inp, *_ = run_gpu(cfg, T=T)
    mism, near, comp = check_routing_teacher_forced(cfg, inp, res, T, ro)
    ref = ro.forward(cfg, inp, T=T, forced_idx=res["route_idx"], forced_loops=res["loops"] if cfg["act"] else None)
    err = np.max(np.abs(res["h"] - ref["h"]))
    _report(name, ratio=f"{err / rms(ref['h']):.3e}", route_mismatch=mism, near_ties=near, compared=comp)
    assert mism == 0
    assert err <= TOL * rms(ref["h"])
    if cfg["top_k"] == cfg["n_experts"]:
        assert np.all(np.isinf(res["route_gap"]))           # no expert left out: no gap
        assert np.all(res["expert_counts"] == cfg["batch"] * cfg["seq"])


def test_k_sliced_down_projection():
    """An expert hidden width of 2112 (33 stages of 64) cuts the down
    projection into two K slices of 17 and 16 stages whose float partial sums
    the combine adds; end to end against the oracle, and prefill + decode
    still equal the forward bit for bit (the slice count is the config's)."""
    cfg = get_config("gqa_small", expert_dim=2112)
    T = cfg["T"]
    res, inp, *_ = run_gpu(cfg, T=T)
    mism, near, comp = check_routing_teacher_forced(cfg, inp, res, T, ro)
    ref = ro.forward(cfg, inp, T=T, forced_idx=res["route_idx"])
    err = np.max(np.abs(res["h"] - ref["h"]))
    _report("k_sliced", ratio=f"{err / rms(ref['h']):.3e}", route_mismatch=mism, near_ties=near)
    assert mism == 0
    assert err <= TOL * rms(ref["h"])


def test_combine_odd_and_long_top_k():
    """Top-11 of 16 experts plus a shared expert, with two K slices: the
    combine gathers the first eight choices in pairs and the rest one at a
    time, the last pair has one member (odd k), and the shared expert's two
    slices are added after them. End to end against the oracle."""
    cfg = get_config("gqa_small", n_experts=16, top_k=11, expert_dim=2112, n_shared_experts=1)
    T = cfg["T"]
    res, inp, *_ = run_gpu(cfg, T=T)
    mism, near, comp = check_routing_teacher_forced(cfg, inp, res, T, ro)
    ref = ro.forward(cfg, inp, T=T, forced_idx=res["route_idx"])
    err = np.max(np.abs(res["h"] - ref["h"]))
    _report("top11_of_16", ratio=f"{err / rms(ref['h']):.3e}", route_mismatch=mism, near_ties=near)
    assert mism == 0
    assert err <= TOL * rms(ref["h"])


def test_act_zero_halting_vector_halts_after_two_loops():
    """w = 0 gives p = 1/2 every loop: the cumulative sum reaches 1.0 >= 0.99
    at the second loop, so every token runs exactly two loops whatever T."""
    cfg = get_config("act_small", T=6)
    inp = make_inputs(cfg)
    inp["w_halt"] = np.zeros_like(inp["w_halt"])
    res, *_ = run_gpu(cfg, inp, T=6)
    assert np.all(res["loops"] == 2)
    np.testing.assert_array_equal(res["act_cum"][1], np.ones_like(res["act_cum"][1]))
    ref = ro.forward(cfg, inp, T=6)
    assert np.all(ref["loops"] == 2)
    assert np.max(np.abs(res["h"] - ref["h"])) <= TOL * rms(ref["h"])


@pytest.mark.parametrize("name", ["gqa_small", "act_small", "dreamer_small", "parallel_lora_small",
                                  "parallel_act_small"])
def test_graph_matches_eager_bitwise(name):
    """Graph replay against kernels launched one by one; for the parallel
    block both run the attention branch on the second stream, and the
    profiling forward (one stream) gives the same bits as well."""
    cfg = get_config(name)
    r1, inp, blk, W = run_gpu(cfg, dumps=False, graph=True)
    r2, *_ = run_gpu(cfg, inp, dumps=False, graph=False, weights=W)
    assert np.array_equal(r1["h"], r2["h"])
    if cfg.get("parallel"):
        out, stages = blk.profile_forward(W["h0"], W["e"], W, T=cfg["T"])
        assert np.array_equal(out.cpu().numpy(), r1["h"])
        for _ in range(3):   # replays with the host synchronising in between
            r3, *_ = run_gpu(cfg, inp, dumps=False, weights=W, block=blk)
            assert np.array_equal(r3["h"], r1["h"])


def test_repeat_runs_bitwise():
    cfg = get_config("wide_small")
    r1, inp, blk, W = run_gpu(cfg, dumps=True)
    r2, *_ = run_gpu(cfg, inp, dumps=True, weights=W, block=blk)
    for k in ("h", "route_idx", "expert_counts", "loops"):
        assert np.array_equal(r1[k], r2[k]), k


def test_T0_and_extrapolation():
    cfg = get_config("gqa_small")
    r0, inp, blk, W = run_gpu(cfg, T=0, dumps=False)
    assert np.array_equal(r0["h"], inp["h0"])
    # more loops than the workload's T (depth extrapolation); LoRA-free so any T is fine
    res, *_ = run_gpu(cfg, inp, T=cfg["T"] + 2, dumps=True, weights=W)
    ref = ro.forward(cfg, inp, T=cfg["T"] + 2, forced_idx=res["route_idx"])
    assert np.max(np.abs(res["h"] - ref["h"])) <= TOL * rms(ref["h"])


def test_error_paths():
    import torch

    from recurrent_depth_transformer_amd import RdtError, RecurrentBlock
    cfg = get_config("tiny")
    inp = make_inputs(cfg)
    inp["A"] = inp["A"].copy()
    inp["A"][5] = 1.0
    with pytest.raises(RdtError) as ei:
        run_gpu(cfg, inp, dumps=False)
    assert "RDT_E_UNSTABLE" in str(ei.value)
    inp = make_inputs(cfg)
    _, _, blk, W = run_gpu(cfg, inp, dumps=False)
    with pytest.raises(RdtError) as ei:
        blk.forward(W["h0"], W["e"], W, T=-1)
    assert "RDT_E_INVALID" in str(ei.value)
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(RdtError) as ei:
        blk.forward(W["h0"], W["e"], W, T=2, workspace=small)
    assert "RDT_E_WORKSPACE" in str(ei.value)
    W2 = dict(W)
    W2["Wq"] = None
    with pytest.raises(RdtError) as ei:
        blk.forward(W["h0"], W["e"], W2, T=1)
    assert "RDT_E_INVALID" in str(ei.value)
    # out may alias h0 exactly
    h = W["h0"].clone()
    blk.forward(h, W["e"], W, T=2, out=h)
    ref = blk.forward(W["h0"], W["e"], W, T=2)
    torch.cuda.synchronize()
    assert torch.equal(h, ref)


def test_act_many_sequences_compaction():
    """ACT with more sequences than one compaction workgroup has threads
    (1100 sequences of 2 tokens): every sequence's offset in the compacted
    active list must be right, or its tokens get another sequence's keys.
    End to end against the oracle with halting forced to the GPU's, and the
    halting decisions from the GPU's own states."""
    cfg = get_config("act_small", batch=1100, seq=2, dim=64, n_heads=4, n_kv_heads=2, head_dim=16,
                     n_experts=4, top_k=2, expert_dim=32, lora_rank=8, n_lora=2, T=5, halt_std=0.3)
    T = cfg["T"]
    res, inp, *_ = run_gpu(cfg, T=T)
    mism, near, comp = check_routing_teacher_forced(cfg, inp, res, T, ro)
    ref = ro.forward(cfg, inp, T=T, forced_idx=res["route_idx"], forced_loops=res["loops"])
    err = np.max(np.abs(res["h"] - ref["h"]))
    scale = rms(ref["h"])
    bad, _ = check_halting(cfg, inp, res, T)
    _report("act_many_sequences", ratio=f"{err / scale:.3e}", route_mismatch=mism, near_ties=near,
            loops=np.bincount(res["loops"], minlength=T + 1).tolist())
    assert mism == 0 and bad == 0
    assert res["loops"].min() < T   # some tokens halted early
    assert err <= TOL * scale
