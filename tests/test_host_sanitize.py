"""The host-only planning code (config validation, workspace layout) built
with the address and undefined-behaviour sanitizers and run over every named
workload, their decode plans and a sweep of edge shapes (CPU only)."""
import os
import shutil
import subprocess

import pytest

from rdt_inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "recurrent_depth_transformer_amd", "csrc")

DRIVER = r'''
#include "rdt_plan.h"
#include <cstdio>
#include <cstdlib>
using namespace rdt;
// argv: batch seq dim attn H KV d ql kvl nr nope vd E Se k F r L act dtype da_h da_kv da_d par T
int main(int argc, char** argv) {
  if (argc != 25) return 2;
  int v[24];
  for (int i = 0; i < 24; ++i) v[i] = atoi(argv[i + 1]);
  rdt_config c{};
  c.batch = v[0]; c.seq = v[1]; c.dim = v[2]; c.attn_type = v[3]; c.n_heads = v[4]; c.n_kv_heads = v[5];
  c.head_dim = v[6]; c.q_lora_rank = v[7]; c.kv_lora_rank = v[8]; c.qk_rope_head_dim = v[9];
  c.qk_nope_head_dim = v[10]; c.v_head_dim = v[11]; c.n_experts = v[12]; c.n_shared_experts = v[13];
  c.top_k = v[14]; c.expert_dim = v[15]; c.lora_rank = v[16]; c.n_lora = v[17]; c.act_enabled = v[18];
  c.dtype = v[19]; c.da_heads = v[20]; c.da_kv_heads = v[21]; c.da_head_dim = v[22]; c.parallel_block = v[23];
  c.rope_base = 1e4f; c.norm_eps = 1e-6f; c.n_bias_rows = 1; c.act_threshold = 0.99f; c.max_T = 16;
  std::string why;
  const rdt_status st = validate_config(c, &why);
  if (st != RDT_OK) { printf("invalid %d %s\n", (int)st, why.c_str()); return 0; }
  size_t last = 0;
  for (int T = 0; T <= 16; ++T) {
    const Plan p = make_plan(c, T);
    if (p.total < last || p.total % 256) { printf("bad total\n"); return 1; }
    last = p.total;
    const Plan d = make_decode_plan(c, T, 4096);
    if (d.total < 256) { printf("bad decode total\n"); return 1; }
  }
  printf("ok %zu\n", last);
  return 0;
}
'''


def _args(c):
    mla = c["attn"] == "mla"
    return [c["batch"], c["seq"], c["dim"], 1 if mla else 0, c["n_heads"], c["n_kv_heads"], c["head_dim"],
            c["q_lora_rank"], c["kv_lora_rank"], c["qk_rope_head_dim"], c["qk_nope_head_dim"], c["v_head_dim"],
            c["n_experts"], c["n_shared_experts"], c["top_k"], c["expert_dim"], c["lora_rank"], c["n_lora"],
            int(c["act"]), 0 if c["dtype"] == "f32" else 1, c["da_heads"], c["da_kv_heads"], c["da_head_dim"],
            int(c["parallel"])]


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_plan_under_address_and_ub_sanitizers(tmp_path):
    drv = tmp_path / "drv.cpp"
    drv.write_text(DRIVER)
    exe = tmp_path / "drv"
    r = subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        "-I", os.path.join(ROOT, "include"), "-I", CSRC, str(drv), os.path.join(CSRC, "rdt_plan.cpp"),
                        "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    cases = [_args(c) for c in WORKLOADS.values()]
    base = _args(WORKLOADS["gqa_small"])
    edge = []
    for i, val in [(0, 0), (0, 1100), (1, 1), (2, 4104), (2, 4096), (12, 65), (14, 9), (15, 7), (6, 48)]:
        a = list(base)
        a[i] = val
        edge.append(a)
    for a in cases + edge:
        out = subprocess.run([str(exe)] + [str(x) for x in a], capture_output=True, text=True, timeout=60)
        assert out.returncode == 0, (a, out.stdout, out.stderr)
        assert out.stdout.startswith("ok") or out.stdout.startswith("invalid"), (a, out.stdout)
        assert "runtime error" not in out.stderr and "AddressSanitizer" not in out.stderr, out.stderr
