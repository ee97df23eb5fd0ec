// Host-only planning for librdt: config validation and the device workspace
// layout. No HIP dependency, so it builds and tests with a plain C++ compiler.
#pragma once
#include <stddef.h>
#include <string>

#include "../../include/rdt.h"

namespace rdt {

// Arrival counters of the ACT compaction inside the combine launch (one
// counter of finished sub-counters, then 64 sub-counters).
constexpr int kCompactCounters = 65;

struct Plan {
  // shapes
  int B, S, N, D, H, KV, d, E, Se, k, F, r, L, T;
  int mla;                  // 1 for multi-latent attention
  int ql, kvl, nr, nope, vd;
  int dq;                   // per-head query/key width seen by attention
  int dv;                   // per-head value width seen by attention
  int hv;                   // width of the concatenated attention output
  int dr;                   // rope width
  int elt;                  // bytes per stored element (2 or 4)
  // workspace byte offsets
  size_t cosb, sinb, n1, q, k_, v_, o, z, a, n2;
  size_t cq_raw, lat_raw, cqn, latent, qfull, qattn, olat, wukT;
  size_t idx, gates, gap, cnt, slot, pcap;
  size_t hmid, y;
  int ksplit;                // K slices of the expert down projection (y then holds
                            // ksplit float partial sums, [ksplit][N*(k+Se)][D])
  size_t lists, ncount, seg, cum;
  size_t wgmask, wgtmp;     // ACT compaction inside the combine: [ceil(N/4)] ints each
  size_t pos;               // decode position (one int, written before each step)
  int rope_len;             // positions in the RoPE tables
  size_t smax;              // [N] float: maximum router probability per row
  // depth attention (Dreamer): norm output, queries, per-loop keys/values
  // [T+1][N][KVd*dd], attention output, projected output (float), depth RoPE
  int da, Hd, KVd, dd;
  size_t da_nd, da_q, da_k, da_v, da_out, da_buf, da_cos, da_sin;
  // decode attention: key ranges per step and their partial results
  int att_split;
  size_t att_po, att_pm, att_pl;
  // ints in front of the expert counts (cnt), cleared with them by the first
  // RMSNorm of a call: decode attention counts finished key ranges per
  // (sequence, head group) there, so the last range merges the partials;
  // ints att_cnt .. att_cnt + kCompactCounters - 1 of the region are the ACT
  // compaction's arrival counters, and the two loops' counts follow them
  int att_cnt;
  size_t total;
};

// RDT_OK, RDT_E_INVALID or RDT_E_UNSUPPORTED; *why receives a message.
rdt_status validate_config(const rdt_config& c, std::string* why);

// Layout for loop counts up to T (T >= 0). Requires a validated config.
Plan make_plan(const rdt_config& c, int T, int counters = 0);
// Plan of one decoding step: batch slots of one token each, RoPE tables for
// max_seq positions.
Plan make_decode_plan(const rdt_config& c, int T, int max_seq);
// Bytes of the per-loop cache for T loops and max_seq positions (0 if invalid).
size_t cache_bytes(const rdt_config& c, int T, int max_seq);

}  // namespace rdt
