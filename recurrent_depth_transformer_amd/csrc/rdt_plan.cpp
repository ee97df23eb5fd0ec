// Config validation and workspace planning (host-only C++).
#include "rdt_plan.h"

#include <stdio.h>

namespace rdt {

// Smallest tile heights the grouped expert GEMMs use (kept in step with the
// host orchestration; this file does not include the HIP headers). Taller
// tiles need fewer tiles, so these bound the grid from above.

static rdt_status fail(std::string* why, rdt_status st, const char* msg) {
  if (why) *why = msg;
  return st;
}

rdt_status validate_config(const rdt_config& c, std::string* why) {
  if (c.batch <= 0 || c.seq <= 0 || c.dim <= 0) return fail(why, RDT_E_INVALID, "batch, seq and dim must be positive");
  if (c.n_heads <= 0) return fail(why, RDT_E_INVALID, "n_heads must be positive");
  if (c.n_experts <= 0 || c.top_k <= 0) return fail(why, RDT_E_INVALID, "n_experts and top_k must be positive");
  if (c.top_k > c.n_experts) return fail(why, RDT_E_INVALID, "top_k exceeds n_experts");
  if (c.expert_dim <= 0) return fail(why, RDT_E_INVALID, "expert_dim must be positive");
  if (c.n_shared_experts < 0) return fail(why, RDT_E_INVALID, "n_shared_experts is negative");
  if (c.n_bias_rows < 0) return fail(why, RDT_E_INVALID, "n_bias_rows is negative");
  if (c.lora_rank < 0 || c.n_lora < 0) return fail(why, RDT_E_INVALID, "lora_rank and n_lora must be >= 0");
  if (c.lora_rank > 0 && c.n_lora <= 0) return fail(why, RDT_E_INVALID, "lora_rank > 0 needs n_lora >= 1");
  if (c.max_T < 0) return fail(why, RDT_E_INVALID, "max_T is negative");
  if (!(c.norm_eps >= 0.f)) return fail(why, RDT_E_INVALID, "norm_eps must be >= 0");
  if (!(c.rope_base > 0.f)) return fail(why, RDT_E_INVALID, "rope_base must be positive");
  if (c.dtype != RDT_F32 && c.dtype != RDT_BF16) return fail(why, RDT_E_INVALID, "unknown dtype");
  if (c.act_enabled && !(c.act_threshold > 0.f)) return fail(why, RDT_E_INVALID, "act_threshold must be positive");
  if (c.attn_type == RDT_ATTN_GQA) {
    if (c.n_kv_heads <= 0 || c.n_heads % c.n_kv_heads)
      return fail(why, RDT_E_INVALID, "n_heads must be a positive multiple of n_kv_heads");
    if (c.head_dim <= 0 || (c.head_dim & 1)) return fail(why, RDT_E_INVALID, "head_dim must be positive and even");
    if (c.head_dim != 16 && c.head_dim != 32 && c.head_dim != 64 && c.head_dim != 128)
      return fail(why, RDT_E_UNSUPPORTED, "head_dim must be 16, 32, 64 or 128");
  } else if (c.attn_type == RDT_ATTN_MLA) {
    if (c.q_lora_rank <= 0 || c.kv_lora_rank <= 0 || c.qk_rope_head_dim <= 0 || c.qk_nope_head_dim <= 0 ||
        c.v_head_dim <= 0)
      return fail(why, RDT_E_INVALID, "MLA ranks and head widths must be positive");
    if (c.qk_rope_head_dim & 1) return fail(why, RDT_E_INVALID, "qk_rope_head_dim must be even");
    const int dq = c.kv_lora_rank + c.qk_rope_head_dim;
    if (!((dq == 160 && c.kv_lora_rank == 128) || (dq == 96 && c.kv_lora_rank == 64)))
      return fail(why, RDT_E_UNSUPPORTED, "MLA latent must be kv_lora_rank 128 + rope 32 or 64 + 32");
    if (c.q_lora_rank % 8 || c.qk_nope_head_dim % 8 || c.v_head_dim % 8 || c.qk_rope_head_dim % 8)
      return fail(why, RDT_E_UNSUPPORTED, "MLA widths must be multiples of 8");
  } else {
    return fail(why, RDT_E_INVALID, "unknown attn_type");
  }
  if (c.dim % 8) return fail(why, RDT_E_UNSUPPORTED, "dim must be a multiple of 8");
  if (c.dim > 4096) return fail(why, RDT_E_UNSUPPORTED, "dim above 4096");
  if (c.expert_dim % 8) return fail(why, RDT_E_UNSUPPORTED, "expert_dim must be a multiple of 8");
  if (c.n_experts > 64) return fail(why, RDT_E_UNSUPPORTED, "more than 64 routed experts");
  if (c.lora_rank % 8) return fail(why, RDT_E_UNSUPPORTED, "lora_rank must be a multiple of 8");
  const long long N = (long long)c.batch * c.seq;
  if (N * (c.top_k + c.n_shared_experts) > (1ll << 30)) return fail(why, RDT_E_UNSUPPORTED, "too many token rows");
  if (c.parallel_block != 0 && c.parallel_block != 1) return fail(why, RDT_E_INVALID, "parallel_block must be 0 or 1");
  if (c.shared_scale != 0 && c.shared_scale != 1) return fail(why, RDT_E_INVALID, "shared_scale must be 0 or 1");
  if (c.da_heads < 0) return fail(why, RDT_E_INVALID, "da_heads is negative");
  if (c.da_heads > 0) {
    if (c.da_kv_heads <= 0 || c.da_heads % c.da_kv_heads)
      return fail(why, RDT_E_INVALID, "da_heads must be a positive multiple of da_kv_heads");
    if (c.da_head_dim != 16 && c.da_head_dim != 32 && c.da_head_dim != 64 && c.da_head_dim != 128)
      return fail(why, RDT_E_UNSUPPORTED, "da_head_dim must be 16, 32, 64 or 128");
    if (c.act_enabled) return fail(why, RDT_E_UNSUPPORTED, "depth attention with ACT halting");
    if (c.max_T > 64) return fail(why, RDT_E_UNSUPPORTED, "depth attention needs max_T <= 64");
  }
  return RDT_OK;
}

static size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

Plan make_plan(const rdt_config& c, int T, int counters) {
  Plan p{};
  p.B = c.batch; p.S = c.seq; p.N = c.batch * c.seq; p.D = c.dim;
  p.H = c.n_heads; p.E = c.n_experts; p.Se = c.n_shared_experts; p.k = c.top_k;
  p.F = c.expert_dim; p.r = c.lora_rank; p.L = c.n_lora; p.T = T;
  p.elt = c.dtype == RDT_F32 ? 4 : 2;
  p.mla = c.attn_type == RDT_ATTN_MLA;
  if (p.mla) {
    p.KV = 1; p.d = 0;
    p.ql = c.q_lora_rank; p.kvl = c.kv_lora_rank; p.nr = c.qk_rope_head_dim;
    p.nope = c.qk_nope_head_dim; p.vd = c.v_head_dim;
    p.dq = p.kvl + p.nr; p.dv = p.kvl; p.hv = p.H * p.vd; p.dr = p.nr;
  } else {
    p.KV = c.n_kv_heads; p.d = c.head_dim;
    p.dq = p.d; p.dv = p.d; p.hv = p.H * p.d; p.dr = p.d;
  }
  const size_t N = p.N, D = p.D, e = p.elt;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += up256(bytes); return o; };
  p.cosb = take((size_t)p.S * (p.dr / 2) * 4);
  p.sinb = take((size_t)p.S * (p.dr / 2) * 4);
  p.n1 = take(N * D * e);
  if (p.mla) {
    p.cq_raw = take(N * p.ql * 4);
    p.lat_raw = take(N * (p.kvl + p.nr) * 4);
    p.cqn = take(N * p.ql * e);
    p.latent = take(N * (p.kvl + p.nr) * e);
    p.qfull = take(N * p.H * (p.nope + p.nr) * e);
    p.qattn = take(N * p.H * (p.kvl + p.nr) * e);
    p.olat = take(N * p.H * p.kvl * e);
    p.wukT = take((size_t)p.H * p.kvl * p.nope * e);
  } else {
    p.q = take(N * p.H * p.d * e);
    p.k_ = take(N * p.KV * p.d * e);
    p.v_ = take(N * p.KV * p.d * e);
  }
  p.o = take(N * p.hv * e);
  p.z = take(N * (p.r > 0 ? p.r : 1) * e);
  p.a = take(N * D * 4);
  p.n2 = take(N * D * e);
  p.idx = take(N * p.k * 4);
  p.gates = take(N * p.k * 4);
  p.gap = take(N * 4);
  p.att_cnt = counters;
  // decode key-range counters, the ACT compaction arrival counters, then two
  // loops' expert counts (alternate loops)
  p.cnt = take((size_t)(counters + kCompactCounters + 2 * p.E) * 4);
  p.slot = take(N * p.k * 4);
  p.pcap = take((size_t)p.E * N * 4);
  p.hmid = take(N * (p.k + p.Se) * p.F * e);
  // The down projection's K loop (F / 64 stages per tile) is latency-bound
  // once it is long: it is cut into slices of at most 32 stages, each written
  // as a float partial sum that the combine adds in slice order. The count
  // depends on the config only, so prefill, decode and the full forward sum
  // every row the same way.
  p.ksplit = c.dtype == RDT_BF16 ? ((p.F + 63) / 64 + 31) / 32 : 1;
  p.y = take(N * (p.k + p.Se) * D * (p.ksplit > 1 ? 4 * (size_t)p.ksplit : e));
  const size_t Tp = (size_t)(T > 0 ? T : 0) + 1;
  p.lists = take(Tp * N * 4);
  p.ncount = take(Tp * 4);
  p.seg = take(Tp * (p.B + 1) * 4);
  p.cum = take(N * 4);
  p.wgmask = take((size_t)((N + 3) / 4) * 4);   // ACT compaction: one mask per combine workgroup
  p.wgtmp = take((size_t)((N + 3) / 4) * 4);
  p.pos = take(4);
  p.smax = take(N * 4);
  p.da = c.da_heads > 0;
  if (p.da) {
    p.Hd = c.da_heads; p.KVd = c.da_kv_heads; p.dd = c.da_head_dim;
    p.da_nd = take(N * D * e);
    p.da_q = take(N * p.Hd * p.dd * e);
    p.da_k = take(Tp * N * p.KVd * p.dd * e);
    p.da_v = take(Tp * N * p.KVd * p.dd * e);
    p.da_out = take(N * p.Hd * p.dd * e);
    p.da_buf = take(N * D * 4);
    p.da_cos = take(Tp * (p.dd / 2) * 4);
    p.da_sin = take(Tp * (p.dd / 2) * 4);
  }
  p.rope_len = p.S;
  p.total = off;
  return p;
}

Plan make_decode_plan(const rdt_config& c, int T, int max_seq) {
  rdt_config d = c;
  d.seq = 1;
  const int att_split = max_seq / 128 < 1 ? 1 : (max_seq / 128 > 8 ? 8 : max_seq / 128);
  Plan p = make_plan(d, T, att_split > 1 ? c.batch * c.n_heads : 0);
  size_t off = p.total;
  auto take = [&](size_t bytes) { size_t o = off; off += up256(bytes); return o; };
  p.cosb = take((size_t)max_seq * (p.dr / 2) * 4);
  p.sinb = take((size_t)max_seq * (p.dr / 2) * 4);
  p.rope_len = max_seq;
  // one workgroup per 128 cached positions, at most 8, per sequence and head
  // group (measured in place: 4 ranges for the gqa decode, 8 for the MLA one)
  p.att_split = att_split;
  if (p.att_split > 1) {
    const size_t rows = (size_t)p.att_split * p.B * p.H;
    p.att_po = take(rows * p.dv * 4);
    p.att_pm = take(rows * 4);
    p.att_pl = take(rows * 4);
  }
  p.total = off;
  return p;
}

size_t cache_bytes(const rdt_config& c, int T, int max_seq) {
  if (T <= 0 || max_seq <= 0) return 0;
  const size_t elt = c.dtype == RDT_F32 ? 4 : 2;
  const size_t row = c.attn_type == RDT_ATTN_MLA ? (size_t)(c.kv_lora_rank + c.qk_rope_head_dim)
                                                 : (size_t)2 * c.n_kv_heads * c.head_dim;
  return (size_t)T * c.batch * max_seq * row * elt;
}

}  // namespace rdt
