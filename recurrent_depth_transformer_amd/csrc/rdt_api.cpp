// librdt C-ABI: argument checks, the rho(A) guard, the per-loop launch plan and
// the cache of captured HIP graphs.
//
// One forward enqueues, per loop t (h_{t+1} = A h_t + B e + Block(h_t, e)):
//   RMSNorm(h + e) (first loop only; later loops get it from the combine
//   kernel) -> Q/K/V (GQA, RoPE in the epilogue) or the MLA latent chain ->
//   causal flash attention -> output projection (+ depth-wise LoRA as a second
//   K phase) -> one kernel for RMSNorm, router softmax/top-k and the stable
//   expert permutation -> grouped SwiGLU gate/up -> grouped down -> combine +
//   injection (+ ACT halting and the stable compaction of the active list, +
//   the next loop's first RMSNorm).
// Data-dependent sizes (active tokens, rows per expert) stay on the device;
// grids are sized for the worst case and idle workgroups exit at once, so the
// whole T-loop is a static graph.
#include <hip/hip_runtime.h>
#include <math.h>

#include <cmath>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/rdt.h"
#include "rdt_launch.h"
#include "rdt_plan.h"

using namespace rdt;

static thread_local std::string g_err;

static rdt_status set_err(rdt_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

#define HIPCHK(x)                                                                                \
  do {                                                                                           \
    hipError_t e_ = (x);                                                                         \
    if (e_ != hipSuccess) return set_err(RDT_E_HIP, std::string(#x) + ": " + hipGetErrorString(e_)); \
  } while (0)

struct GraphKey {
  const void* ptrs[48];
  int T, max_seq, decode;
  bool operator==(const GraphKey& o) const {
    return T == o.T && max_seq == o.max_seq && decode == o.decode && memcmp(ptrs, o.ptrs, sizeof(ptrs)) == 0;
  }
};

struct GraphEntry {
  GraphKey key;
  hipGraph_t graph;
  hipGraphExec_t exec;
};

// A pointers whose rho(A) < 1 was confirmed (the newest kRhoSlots, fixed
// storage so that checking allocates nothing).
constexpr int kRhoSlots = 8;

struct rdt_handle {
  rdt_config cfg;
  int device;
  hipStream_t cap;
  hipStream_t side;          // the parallel block's attention branch
  hipEvent_t ev_fork, ev_join;
  int graph_mode;
  const float* checked_A[kRhoSlots];
  int n_checked;
  std::vector<GraphEntry> graphs;
};

// Scratch of rdt_recurrent_forward_noalloc: one copy of this array on every
// device the library runs on, held until the process ends. Host code never
// passes the array's name to a kernel (on the host it stands for a host-side
// shadow, not a device address); it uses the device address that
// hipGetSymbolAddress returned for the device, looked up once per device when
// the first handle on that device is created.
static __device__ __align__(256) char scratch[RDT_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static hipError_t scratch_setup(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[device]) return hipSuccess;
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));   // the current device's copy
  if (e != hipSuccess) return e;
  if (!ptr) return hipErrorInvalidSymbol;
  g_scratch_ptr[device] = ptr;
  return hipSuccess;
}

static void* scratch_of(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  return g_scratch_ptr[device];
}

extern "C" const char* rdt_last_error(void) { return g_err.c_str(); }
extern "C" const char* rdt_version(void) { return "librdt 0.1 gfx950"; }

extern "C" rdt_status rdt_config_default(rdt_config* c) {
  if (!c) return set_err(RDT_E_INVALID, "null config");
  memset(c, 0, sizeof(*c));
  c->attn_type = RDT_ATTN_GQA;
  c->rope_base = 10000.f;
  c->norm_eps = 1e-6f;
  c->n_bias_rows = 1;
  c->act_threshold = 0.99f;
  c->dtype = RDT_BF16;
  c->max_T = 16;
  return RDT_OK;
}

extern "C" rdt_status rdt_config_validate(const rdt_config* c) {
  if (!c) return set_err(RDT_E_INVALID, "null config");
  std::string why;
  rdt_status st = validate_config(*c, &why);
  if (st != RDT_OK) return set_err(st, why);
  return RDT_OK;
}

extern "C" rdt_status rdt_spectral_radius(const float* A, int32_t dim, float* rho) {
  if (!A || !rho || dim <= 0) return set_err(RDT_E_INVALID, "rdt_spectral_radius: bad arguments");
  float m = 0.f;
  for (int i = 0; i < dim; ++i) {
    const float v = fabsf(A[i]);
    if (!(v <= m)) m = v;  // NaN propagates
  }
  *rho = m;
  return RDT_OK;
}

extern "C" rdt_status rdt_create(const rdt_config* c, rdt_handle** out) {
  if (!out) return set_err(RDT_E_INVALID, "null output handle");
  *out = nullptr;
  rdt_status st = rdt_config_validate(c);
  if (st != RDT_OK) return st;
  rdt_handle* h = new (std::nothrow) rdt_handle();
  if (!h) return set_err(RDT_E_INVALID, "out of host memory");
  h->cfg = *c;
  h->graph_mode = 1;
  h->n_checked = 0;
  if (hipGetDevice(&h->device) != hipSuccess ||
      hipStreamCreateWithFlags(&h->cap, hipStreamNonBlocking) != hipSuccess) {
    delete h;
    return set_err(RDT_E_HIP, "rdt_create: cannot create the capture stream");
  }
  h->side = nullptr; h->ev_fork = nullptr; h->ev_join = nullptr;
  if (c->parallel_block &&
      (hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking) != hipSuccess ||
       hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming) != hipSuccess ||
       hipEventCreateWithFlags(&h->ev_join, hipEventDisableTiming) != hipSuccess)) {
    if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
    if (h->side) (void)hipStreamDestroy(h->side);
    (void)hipStreamDestroy(h->cap);
    delete h;
    return set_err(RDT_E_HIP, "rdt_create: cannot create the branch stream");
  }
  // the device address of this device's scratch array (first handle only)
  hipError_t se = scratch_setup(h->device);
  if (se != hipSuccess) {
    (void)hipStreamDestroy(h->cap);
    delete h;
    return set_err(RDT_E_HIP, std::string("rdt_create: scratch address lookup failed: ") + hipGetErrorString(se));
  }
  *out = h;
  return RDT_OK;
}

extern "C" void rdt_destroy(rdt_handle* h) {
  if (!h) return;
  for (auto& g : h->graphs) {
    (void)hipGraphExecDestroy(g.exec);
    (void)hipGraphDestroy(g.graph);
  }
  if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
  if (h->ev_join) (void)hipEventDestroy(h->ev_join);
  if (h->side) (void)hipStreamDestroy(h->side);
  (void)hipStreamDestroy(h->cap);
  delete h;
}

extern "C" size_t rdt_workspace_size(const rdt_handle* h, int32_t T) {
  if (!h || T < 0 || T > h->cfg.max_T) return 0;
  return make_plan(h->cfg, T).total;
}

extern "C" rdt_status rdt_set_graph_mode(rdt_handle* h, int32_t enabled) {
  if (!h) return set_err(RDT_E_INVALID, "null handle");
  h->graph_mode = enabled != 0;
  return RDT_OK;
}

// ------------------------------------------------------------------ enqueue
struct Fwd {
  const rdt_config* c;
  Plan P;
  const float* h0;
  const float* e;
  const rdt_weights* w;
  int T;
  float* out;
  rdt_aux aux;
  char* ws;
  // per-loop cache: prefill writes positions 0..S-1, a decode step (decode = 1,
  // one token per sequence, position read from the workspace) appends one row
  char* cache = nullptr;
  int max_seq = 0;
  int decode = 0;
  // second stream and fork / join events for the parallel block's branches
  // (null: one stream)
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
};

// Event pairs around launches (rdt_profile_forward only).
struct Prof {
  struct Rec { int stage; hipEvent_t a, b; };
  std::vector<Rec> recs;
  int cur = -1;
  ~Prof() {
    for (auto& r : recs) { (void)hipEventDestroy(r.a); (void)hipEventDestroy(r.b); }
  }
};

static hipError_t prof_begin(Prof* p, int stage, hipStream_t s) {
  Prof::Rec r{stage, nullptr, nullptr};
  hipError_t e = hipEventCreate(&r.a);
  if (e == hipSuccess) e = hipEventCreate(&r.b);
  if (e != hipSuccess) return e;
  p->recs.push_back(r);
  return hipEventRecord(r.a, s);
}
static hipError_t prof_end(Prof* p, hipStream_t s) { return hipEventRecord(p->recs.back().b, s); }

#define LAUNCH(STG, X)                                   \
  do {                                                   \
    if (prof) HIPCHK(prof_begin(prof, (STG), s));        \
    HIPCHK(X);                                           \
    if (prof) HIPCHK(prof_end(prof, s));                 \
  } while (0)

template <typename P>
static P* at(char* ws, size_t off) { return reinterpret_cast<P*>(ws + off); }

static const char* elt_ptr(const void* base, long long elems, int elt) {
  return reinterpret_cast<const char*>(base) + elems * elt;
}

// Under ACT, tokens halt: from the third loop on the gathered projections
// usually see a small share of the rows (act workload: 8258 of 16384 at loop
// 2, under 2000 from loop 10), and 128x128 tiles then leave most CUs idle
// while each tile walks its K stages. 64x64 tiles from loop 2 on: act forward
// 7.94 -> 7.63 ms; in loops where every token is still active they cost ~3 %
// (loop 1 measured with them: 1.222 -> 1.263 ms).
constexpr int kActSmallTilesFrom = 2;

static void pick_tile(long long M, long long N, int min_bn, int* bm, int* bn) {
  auto tiles = [&](int m, int n) { return ((M + m - 1) / m) * ((N + n - 1) / n); };
  *bm = 128;
  *bn = 128;
  if (tiles(128, 128) >= 256) return;
  if (tiles(64, 128) >= 256 || min_bn > 64) { *bm = 64; return; }
  *bm = 64;
  *bn = 64;
}

// bf16 dense GEMMs with square 64 or 128 tiles run eight waves per workgroup:
// one wave keeps only a few direct-to-LDS loads in flight, so twice the waves
// stream a tile about 1.5x faster. Measured in place against four waves:
// forwards 1-6 % faster (MLA -4 %, ACT -5 %, Dreamer -2 % with 128x128 tiles
// instead of 128x192 ones), one-token decode -3 %.
//
// A projection with one weight segment (rows stored in place or scattered to
// their token, RoPE over 64- or 128-wide heads or none, no depth RoPE, no
// cache rows) that fills whole rounds of 256x256 tiles over 256 CUs, or at
// least four, runs on the 256x256 ping-pong tiles of the expert GEMMs with a
// per-wave epilogue (wide MoE: the output projection and the query projection,
// 256 tiles each).
static bool big_tiles_ok(const DenseGemm& g) {
  const GemmSeg& s0 = g.seg[0];
  if (g.dtype != DT_BF16 || g.bm != 128 || g.bn != 128 || g.A2 || g.batch > 1 || g.epi != EPI_STORE ||
      g.nseg != 1 || s0.row_mul)
    return false;
  if (s0.rope && (g.drope || (g.rope_dim != 64 && g.rope_dim != 128) || s0.ncols % g.rope_dim)) return false;
  const long long tiles = (long long)((g.M + 255) / 256) * ((s0.ncols + 255) / 256);
  return tiles >= 256 && (tiles % 256 == 0 || tiles >= 4 * 256);
}

static hipError_t dense_gemm(DenseGemm& g, hipStream_t s) {
  if (big_tiles_ok(g)) g.bm = g.bn = 256;
  if (g.dtype == DT_BF16 && g.bm == g.bn && (g.bm == 64 || g.bm == 128 || g.bm == 256)) g.nw = 8;
  return launch_dense_gemm(g, s);
}

static rdt_status enqueue(const Fwd& f, hipStream_t s, Prof* prof = nullptr) {
  const rdt_config& c = *f.c;
  const Plan& P = f.P;
  char* ws = f.ws;
  const int N = P.N, D = P.D, dt = c.dtype == RDT_F32 ? DT_F32 : DT_BF16, elt = P.elt;
  const rdt_weights& w = *f.w;
  const bool act = c.act_enabled != 0;

  // T > 0: the first loop's RMSNorm kernel copies h0 into out as it reads it
  if (f.out != f.h0 && f.T == 0)
    LAUNCH(RDT_STAGE_OTHER, hipMemcpyAsync(f.out, f.h0, (size_t)N * D * 4, hipMemcpyDeviceToDevice, s));
  if (f.aux.h_dump) LAUNCH(RDT_STAGE_OTHER, launch_copy_f32(f.aux.h_dump, f.h0, (long long)N * D, s));
  if (f.T == 0) {
    if (f.aux.loops) LAUNCH(RDT_STAGE_OTHER, launch_fill_i32(f.aux.loops, 0, N, s));
    return RDT_OK;
  }
  float* cosb = at<float>(ws, P.cosb);
  float* sinb = at<float>(ws, P.sinb);
  // the RoPE tables are built by the first loop's RMSNorm kernel
  int* pos_dev = f.decode ? at<int>(ws, P.pos) : nullptr;
  // decode without ACT: the cached keys are cut into P.att_split ranges, one
  // workgroup each; the last range of each (sequence, head group) to finish
  // merges them (counted in P.att_cnt ints in front of the expert counts)
  auto set_split = [&](AttnArgs& aa) {
    aa.nsplit = (f.decode && !act && P.att_split > 1) ? P.att_split : 1;
    if (aa.nsplit > 1) {
      aa.part_o = at<float>(ws, P.att_po);
      aa.part_m = at<float>(ws, P.att_pm);
      aa.part_l = at<float>(ws, P.att_pl);
      aa.split_cnt = at<int>(ws, P.cnt);
    }
  };
  // loop t's cache: GQA keys then values, or MLA latents (rows b*max_seq + p)
  const size_t crow = P.mla ? (size_t)(P.kvl + P.nr) : (size_t)P.KV * P.d;  // elements per row
  const size_t cplane = (size_t)P.B * f.max_seq * crow * elt;                 // bytes per array per loop
  auto cache_at = [&](int t, int which) { return f.cache + ((size_t)t * (P.mla ? 1 : 2) + which) * cplane; };
  // rows of this call's K/V (or latent) buffer -> cache rows
  auto append = [&](int t, int which, const char* src, hipStream_t st) -> hipError_t {
    if (!f.cache) return hipSuccess;
    const int s_in = f.decode ? 1 : P.S;
    return launch_rows_scatter(cache_at(t, which), (long long)crow * elt, src, (long long)crow * elt,
                               (int)(crow * elt), N, s_in, f.max_seq, pos_dev, st);
  };
  if (P.mla) LAUNCH(RDT_STAGE_OTHER, launch_head_transpose(dt, at<char>(ws, P.wukT), w.Wuk, P.H, P.nope, P.kvl, s));

  int* lists = at<int>(ws, P.lists);
  int* ncount = at<int>(ws, P.ncount);
  int* segs = at<int>(ws, P.seg);
  float* cum = at<float>(ws, P.cum);
  if (act) {
    LAUNCH(RDT_STAGE_OTHER, launch_iota(lists, N, ncount, N, segs, P.B, P.S, s));
    LAUNCH(RDT_STAGE_OTHER, launch_fill_f32(cum, 0.f, N, s));
    LAUNCH(RDT_STAGE_OTHER, launch_fill_i32(at<int>(ws, P.wgmask), 0, (N + 3) / 4, s));
  }
  const int k = P.k, E = P.E;
  if (f.aux.loops) LAUNCH(RDT_STAGE_OTHER, launch_fill_i32(f.aux.loops, 0, N, s));
  if (f.aux.route_idx) LAUNCH(RDT_STAGE_OTHER, launch_fill_i32(f.aux.route_idx, -1, (long long)f.T * N * k, s));
  if (f.aux.route_gap) LAUNCH(RDT_STAGE_OTHER, launch_fill_f32(f.aux.route_gap, NAN, (long long)f.T * N, s));
  if (f.aux.act_cum) LAUNCH(RDT_STAGE_OTHER, launch_fill_f32(f.aux.act_cum, NAN, (long long)f.T * N, s));
  if (act && f.aux.n2_dump) {
    if (dt == DT_F32) LAUNCH(RDT_STAGE_OTHER, launch_fill_f32((float*)f.aux.n2_dump, 0.f, (long long)f.T * N * D, s));
    else LAUNCH(RDT_STAGE_OTHER, launch_fill_u16((uint16_t*)f.aux.n2_dump, 0, (long long)f.T * N * D, s));
  }
  if (act && f.aux.a_dump) LAUNCH(RDT_STAGE_OTHER, launch_fill_f32(f.aux.a_dump, 0.f, (long long)f.T * N * D, s));

  char* n1 = at<char>(ws, P.n1);
  // Dreamer variants: depth attention buffers, parallel sublayers, shared scale
  const bool par = c.parallel_block != 0;
  // concurrent branches need the handle's second stream; the profiling
  // forward keeps one stream so that its events time single launches
  const bool fork = par && f.side && !prof;
  hipStream_t sa = fork ? f.side : s;

  float* smax = (c.shared_scale && P.Se > 0) ? at<float>(ws, P.smax) : nullptr;
  char* nd = P.da ? at<char>(ws, P.da_nd) : nullptr;
  char* dq = P.da ? at<char>(ws, P.da_q) : nullptr;
  char* dk = P.da ? at<char>(ws, P.da_k) : nullptr;
  char* dvb = P.da ? at<char>(ws, P.da_v) : nullptr;
  char* dout = P.da ? at<char>(ws, P.da_out) : nullptr;
  float* dbuf = P.da ? at<float>(ws, P.da_buf) : nullptr;
  float* dcos = P.da ? at<float>(ws, P.da_cos) : nullptr;
  float* dsin = P.da ? at<float>(ws, P.da_sin) : nullptr;

  char* o = at<char>(ws, P.o);
  char* z = at<char>(ws, P.z);
  float* abuf = at<float>(ws, P.a);
  char* n2 = at<char>(ws, P.n2);
  int* idx = at<int>(ws, P.idx);
  float* gates = at<float>(ws, P.gates);
  float* gap = at<float>(ws, P.gap);
  int* cnt2 = at<int>(ws, P.cnt) + P.att_cnt + kCompactCounters;  // per-expert counts of even / odd loops
  int* slot = at<int>(ws, P.slot);
  int* pcap = at<int>(ws, P.pcap);
  char* hmid = at<char>(ws, P.hmid);
  char* ybuf = at<char>(ws, P.y);
  // loop 0's expert counts are cleared by the first RMSNorm kernel; each
  // loop's combine clears the next loop's
  // Expert GEMM tiles (measured on MI355X): gate/up 192x128 with a two-stage
  // ring (two workgroups per CU); 160x128 when experts see 64-128 rows on
  // average (one row tile still covers an expert 25 % above the average, and
  // each CU that runs two tiles streams 10 % fewer bytes: gqa forward -2.4 %
  // in place, while the large workloads were 1-2 % slower with it); or 64x64
  // with a three-stage ring when
  // experts see under 64 rows (decode: narrow tiles give more workgroups;
  // 64x128 was 2-4 % slower per step); down 192x128 with a two-stage ring
  // when experts see many rows (measured in place: 0.3-1.5 % faster forwards
  // than 128x128), 64x32 for decode, else 64x64 with a three-stage ring.
  const long long rows_per_expert = (long long)N * k / E;
  const bool bf = dt == DT_BF16;
  // Experts that see 256 rows or more on average: 256x256 ping-pong tiles
  // (eight waves, one workgroup per CU; see rdt_gemm.hip) for a projection
  // that yields at least four rounds of such tiles over 256 CUs. With fewer,
  // the last round leaves CUs idle and two 192x128 workgroups per CU do better
  // (measured on the MLA expert shape: down projection, about 544 tiles, 123
  // against 105 us; wide MoE, 2560 tiles each: gate/up 683 against 799 us,
  // down 352 against 412 us).
  auto pp_rounds_ok = [&](int outw, int ncols) {
    const long long mt = (long long)N * k / 256 + E / 2 + (long long)P.Se * ((N + 255) / 256);
    return bf && rows_per_expert >= 256 && mt * ((ncols + outw - 1) / outw) >= 4 * 256;
  };
  const bool pp_gu = pp_rounds_ok(128, P.F), pp_dn = pp_rounds_ok(256, D) && P.ksplit <= 1;
  const int gu_bm = pp_gu ? 256 : bf ? (rows_per_expert < 64 ? 64 : rows_per_expert <= 128 ? 160 : 192) : GU_BM;
  const int gu_bn = pp_gu ? 256 : bf && rows_per_expert < 64 ? 64 : GU_BN;
  const int dn_bm = (rows_per_expert >= 256 && bf) ? 128 : 64;
  // grid bound of a grouped GEMM with bm-row tiles: sum_e ceil(c_e / bm) over
  // the routed experts is at most N*k/bm + E; each shared expert adds ceil(N/bm)
  auto max_mtiles = [&](int bm) {
    return (int)((long long)N * k / bm + E + (long long)P.Se * ((N + bm - 1) / bm));
  };

  for (int t = 0; t < f.T; ++t) {
    const int* cur = act ? lists + (size_t)t * N : nullptr;
    const int* ncur = act ? ncount + t : nullptr;
    const int tp = t > 0 ? t - 1 : 0;
    const int* prev = act ? lists + (size_t)tp * N : nullptr;
    const int* nprev = act ? ncount + tp : nullptr;
    const int* seg = act ? segs + (size_t)t * (P.B + 1) : nullptr;

    // a1: u = h + e, n1 = RMSNorm(u) * g1 (tokens whose state changed last loop)
    //     (after the first loop the combine kernel of the previous loop wrote it)
    //     With depth attention the first norm feeds it (gain g_da) and the
    //     attention input is normalised after it.
    if (t == 0) {
      NormArgs n1a{};
      n1a.dtype = dt; n1a.h = f.out; n1a.e = f.e; n1a.a = nullptr; n1a.g = P.da ? w.g_da : w.g1;
      n1a.eps = c.norm_eps; n1a.D = D;
      n1a.rows = prev; n1a.ndev = nprev; n1a.n = N; n1a.out = P.da ? nd : n1; n1a.out_scatter = 1; n1a.dump = nullptr;
      // per-forward set-up in the same launch: h0 -> out, RoPE tables, counts
      n1a.h = f.h0;
      n1a.h_copy = f.out != f.h0 ? f.out : nullptr;
      n1a.rope_cos[0] = cosb; n1a.rope_sin[0] = sinb; n1a.rope_S[0] = P.rope_len; n1a.rope_dr[0] = P.dr;
      if (P.da) { n1a.rope_cos[1] = dcos; n1a.rope_sin[1] = dsin; n1a.rope_S[1] = f.T; n1a.rope_dr[1] = P.dd; }
      n1a.rope_base = c.rope_base;
      // split counters, the compaction arrival counters, loop 0's counts
      n1a.zero = at<int>(ws, P.cnt); n1a.zero_n = P.att_cnt + kCompactCounters + E;
      LAUNCH(RDT_STAGE_NORM1, launch_norm(n1a, s));
    }
    // Parallel block (every sublayer reads RMSNorm(h + e)): the sequence-
    // attention branch runs on a second stream, forked here and joined before
    // the combine, beside the depth-attention and MoE branches on `s`.
    if (fork) {
      HIPCHK(hipEventRecord(f.ev_fork, s));
      HIPCHK(hipStreamWaitEvent(f.side, f.ev_fork, 0));
    }
    if (P.da) {
      // Dreamer depth attention: q, k, v of this loop (depth RoPE at t and at
      // the reversed depth T-1-t), keys/values kept per loop, attention over
      // loops 0..t of the same token, output projection into dbuf (float)
      const int qw = P.Hd * P.dd, kw = P.KVd * P.dd;
      const size_t lpl = (size_t)N * kw;  // elements per loop in dk / dv
      DenseGemm g{};
      g.dtype = dt; g.A = nd; g.lda = D; g.K = D; g.batch = 1; g.epi = EPI_STORE;
      g.rows = nullptr; g.gather = 0; g.M = N; g.Mdev = nullptr;
      g.nseg = 3;
      g.seg[0] = GemmSeg{w.Wq_da, qw, dq, qw, 0, 1, 0};
      g.seg[1] = GemmSeg{w.Wk_da, kw, dk + (size_t)t * lpl * elt, kw, 1, 1, 0};
      g.seg[2] = GemmSeg{w.Wv_da, kw, dvb + (size_t)t * lpl * elt, kw, 1, 0, 0};
      g.cosb = dcos; g.sinb = dsin; g.rope_dim = P.dd; g.seq = 1;
      g.drope = 1; g.dpos0 = t; g.dpos1 = f.T - 1 - t;
      pick_tile(N, qw + 2 * kw, P.dd, &g.bm, &g.bn);
      LAUNCH(RDT_STAGE_QKV, dense_gemm(g, s));
      DepthAttnArgs da{};
      da.dtype = dt; da.q = dq; da.k = dk; da.v = dvb; da.o = dout; da.lstride = (long long)lpl;
      da.n = N; da.H = P.Hd; da.KV = P.KVd; da.dd = P.dd; da.t = t; da.scale = 1.f / sqrtf((float)P.dd);
      LAUNCH(RDT_STAGE_DEPTH_ATTN, launch_depth_attention(da, s));
      DenseGemm gdo{};
      gdo.dtype = dt; gdo.A = dout; gdo.lda = qw; gdo.K = qw; gdo.batch = 1; gdo.epi = EPI_STORE;
      gdo.rows = nullptr; gdo.gather = 0; gdo.M = N; gdo.Mdev = nullptr;
      gdo.nseg = 1; gdo.seg[0] = GemmSeg{w.Wo_da, D, dbuf, D, 0, 0, 1};
      pick_tile(N, D, 16, &gdo.bm, &gdo.bn);
      LAUNCH(RDT_STAGE_OPROJ, dense_gemm(gdo, s));
      // sequence-attention input: RMSNorm(u + d) (sequential) or RMSNorm(u) (parallel)
      NormArgs n1a{};
      n1a.dtype = dt; n1a.h = f.out; n1a.e = f.e; n1a.a = par ? nullptr : dbuf; n1a.g = w.g1; n1a.eps = c.norm_eps;
      n1a.D = D; n1a.rows = nullptr; n1a.ndev = nullptr; n1a.n = N; n1a.out = n1; n1a.out_scatter = 1;
      LAUNCH(RDT_STAGE_NORM1, launch_norm(n1a, sa));
    }

    // a2-a4: attention
    if (!P.mla) {
      const int Hd = P.H * P.d, KVd = P.KV * P.d;
      char* q = at<char>(ws, P.q);
      char* kb = at<char>(ws, P.k_);
      char* vb = at<char>(ws, P.v_);
      GemmSeg sq{w.Wq, Hd, q, Hd, act ? 0 : 1, 1, 0};
      GemmSeg sk{w.Wk, KVd, kb, KVd, 1, 1, 0};
      GemmSeg sv{w.Wv, KVd, vb, KVd, 1, 0, 0};
      // one-token decode without ACT: k and v go straight into the cache rows
      const bool direct = f.decode && !act;
      if (direct) {
        sk.C = cache_at(t, 0); sk.row_mul = f.max_seq;
        sv.C = cache_at(t, 1); sv.row_mul = f.max_seq;
      }
      DenseGemm g{};
      g.dtype = dt; g.A = n1; g.lda = D; g.K = D; g.batch = 1;
      g.cosb = cosb; g.sinb = sinb; g.rope_dim = P.d; g.seq = P.S; g.epi = EPI_STORE; g.pos_dev = pos_dev;
      g.M = N;
      if (!act) {
        g.rows = nullptr; g.gather = 0; g.Mdev = nullptr;
        // the query projection alone when it fills the 256x256 tiles (wide
        // MoE: 114 against 140 us per loop for q, k and v on 128x128 tiles),
        // else q, k and v in one launch
        DenseGemm gq = g;
        gq.nseg = 1; gq.seg[0] = sq; gq.bm = gq.bn = 128;
        if (big_tiles_ok(gq)) {
          LAUNCH(RDT_STAGE_QKV, dense_gemm(gq, sa));
          g.nseg = 2; g.seg[0] = sk; g.seg[1] = sv;
          pick_tile(N, 2 * KVd, P.d, &g.bm, &g.bn);
        } else {
          g.nseg = 3; g.seg[0] = sq; g.seg[1] = sk; g.seg[2] = sv;
          pick_tile(N, Hd + 2 * KVd, P.d, &g.bm, &g.bn);
        }
        LAUNCH(RDT_STAGE_QKV, dense_gemm(g, sa));
      } else {
        DenseGemm gq = g;
        gq.rows = cur; gq.gather = 1; gq.Mdev = ncur; gq.nseg = 1; gq.seg[0] = sq;
        pick_tile(N, Hd, P.d, &gq.bm, &gq.bn);
        if (t >= kActSmallTilesFrom && bf) gq.bm = gq.bn = 64;
        LAUNCH(RDT_STAGE_QKV, dense_gemm(gq, sa));
        DenseGemm gkv = g;
        gkv.rows = prev; gkv.gather = 1; gkv.Mdev = nprev; gkv.nseg = 2; gkv.seg[0] = sk; gkv.seg[1] = sv;
        pick_tile(N, 2 * KVd, P.d, &gkv.bm, &gkv.bn);
        if (t >= kActSmallTilesFrom && bf) gkv.bm = gkv.bn = 64;
        LAUNCH(RDT_STAGE_QKV, dense_gemm(gkv, sa));
      }
      if (f.cache && !direct) {
        LAUNCH(RDT_STAGE_QKV, append(t, 0, kb, sa));
        LAUNCH(RDT_STAGE_QKV, append(t, 1, vb, sa));
      }
      AttnArgs aa{};
      aa.dtype = dt; aa.dqk = P.d; aa.dv = P.d;
      aa.q = q; aa.q_ld = Hd; aa.q_hs = P.d;
      aa.k = f.decode ? cache_at(t, 0) : kb; aa.k_ld = KVd; aa.k_hs = P.d;
      aa.v = f.decode ? cache_at(t, 1) : vb; aa.v_ld = KVd; aa.v_hs = P.d;
      aa.o = o; aa.o_ld = Hd; aa.o_hs = P.d;
      aa.H = P.H; aa.KV = P.KV; aa.rows = cur; aa.seg = seg; aa.B = P.B;
      aa.S = f.decode ? f.max_seq : P.S; aa.dec = f.decode; aa.dec_pos = pos_dev;
      aa.scale = 1.f / sqrtf((float)P.d);
      // ACT late loops: the running tokens of a sequence are spread over its
      // positions, so a 32-row query slice walks the keys of its last token
      // for all 32; 16-row slices halve that (act attention 66 -> 60 us per loop)
      aa.narrow = act && t >= kActSmallTilesFrom;
      set_split(aa);
      LAUNCH(RDT_STAGE_ATTN, launch_attention(aa, sa));
    } else {
      const int W = P.kvl + P.nr, qw = P.nope + P.nr;
      char* cq_raw = at<char>(ws, P.cq_raw);
      char* lat_raw = at<char>(ws, P.lat_raw);
      char* cqn = at<char>(ws, P.cqn);
      char* latent = at<char>(ws, P.latent);
      char* qfull = at<char>(ws, P.qfull);
      char* qattn = at<char>(ws, P.qattn);
      char* olat = at<char>(ws, P.olat);
      char* wukT = at<char>(ws, P.wukT);
      // down projections of the query and kv latents (fp32 for the norms)
      DenseGemm g1{};
      g1.dtype = dt; g1.A = n1; g1.lda = D; g1.K = D; g1.batch = 1; g1.epi = EPI_STORE;
      g1.rows = prev; g1.gather = act ? 1 : 0; g1.M = N; g1.Mdev = nprev;
      g1.nseg = 2;
      g1.seg[0] = GemmSeg{w.Wdq, P.ql, cq_raw, P.ql, 1, 0, 1};
      g1.seg[1] = GemmSeg{w.Wdkv, W, lat_raw, W, 1, 0, 1};
      pick_tile(N, P.ql + W, 16, &g1.bm, &g1.bn);
      LAUNCH(RDT_STAGE_QKV, dense_gemm(g1, sa));
      MlaNormArgs mn{};
      mn.dtype = dt; mn.cq_raw = (const float*)cq_raw; mn.ql = P.ql; mn.lat_raw = (const float*)lat_raw;
      mn.kvl = P.kvl; mn.nr = P.nr; mn.gq = w.gq; mn.gkv = w.gkv; mn.eps = c.norm_eps;
      mn.rows = prev; mn.ndev = nprev; mn.n = N; mn.cqn = cqn; mn.latent = latent;
      mn.cosb = cosb; mn.sinb = sinb; mn.S = P.S; mn.pos_dev = pos_dev;
      LAUNCH(RDT_STAGE_QKV, launch_mla_norm(mn, sa));
      if (f.cache) LAUNCH(RDT_STAGE_QKV, append(t, 0, latent, sa));
      // query up-projection (compacted rows)
      DenseGemm g2{};
      g2.dtype = dt; g2.A = cqn; g2.lda = P.ql; g2.K = P.ql; g2.batch = 1; g2.epi = EPI_STORE;
      g2.rows = cur; g2.gather = act ? 1 : 0; g2.M = N; g2.Mdev = ncur;
      g2.nseg = 1; g2.seg[0] = GemmSeg{w.Wuq, P.H * qw, qfull, P.H * qw, 0, 0, 0};
      pick_tile(N, P.H * qw, 16, &g2.bm, &g2.bn);
      LAUNCH(RDT_STAGE_QKV, dense_gemm(g2, sa));
      AttnArgs aa{};
      aa.dtype = dt; aa.dqk = W; aa.dv = P.kvl;
      const char* lat_src = f.decode ? cache_at(t, 0) : latent;
      aa.k = lat_src; aa.k_ld = W; aa.k_hs = 0;
      aa.v = lat_src; aa.v_ld = W; aa.v_hs = 0;
      aa.o = olat; aa.o_ld = P.H * P.kvl; aa.o_hs = P.kvl;
      aa.H = P.H; aa.KV = 1; aa.rows = cur; aa.seg = seg; aa.B = P.B;
      aa.S = f.decode ? f.max_seq : P.S; aa.dec = f.decode; aa.dec_pos = pos_dev;
      aa.scale = 1.f / sqrtf((float)(P.nope + P.nr));
      aa.narrow = act && t >= kActSmallTilesFrom;
      set_split(aa);
      // value up-projection per head: o[h] = o_lat[h] . Wuv[h]^T
      DenseGemm g4{};
      g4.dtype = dt; g4.A = olat; g4.lda = P.H * P.kvl; g4.a_bstride = P.kvl; g4.K = P.kvl; g4.epi = EPI_STORE;
      g4.rows = cur; g4.gather = 0; g4.M = N; g4.Mdev = ncur; g4.batch = P.H;
      g4.nseg = 1; g4.seg[0] = GemmSeg{w.Wuv, P.vd, o, P.hv, 0, 0, 0};
      g4.b_bstride = (long long)P.vd * P.kvl; g4.c_bstride = P.vd;
      pick_tile(N, (long long)P.vd * P.H, 16, &g4.bm, &g4.bn);
      if (bf) {
        // bf16: the attention kernel forms q from q_nope and q_pe (absorb and
        // RoPE) and, outside key-range splits, applies Wuv itself
        aa.qn = qfull; aa.qn_ld = P.H * qw; aa.qn_hs = qw; aa.nope = P.nope;
        aa.wukT = wukT; aa.cosb = cosb; aa.sinb = sinb;
        aa.wuv = w.Wuv; aa.vd = P.vd; aa.ov = o; aa.ov_ld = P.hv;
        LAUNCH(RDT_STAGE_ATTN, launch_attention(aa, sa));
        if (aa.nsplit > 1) LAUNCH(RDT_STAGE_ATTN, dense_gemm(g4, sa));
      } else {
        // absorb: q_lat[h] = q_nope[h] . Wuk[h]  (per head, B = Wuk[h]^T)
        DenseGemm g3{};
        g3.dtype = dt; g3.A = qfull; g3.lda = P.H * qw; g3.a_bstride = qw; g3.K = P.nope; g3.epi = EPI_STORE;
        g3.rows = cur; g3.gather = 0; g3.M = N; g3.Mdev = ncur; g3.batch = P.H;
        g3.nseg = 1; g3.seg[0] = GemmSeg{wukT, P.kvl, qattn, P.H * W, 0, 0, 0};
        g3.b_bstride = (long long)P.kvl * P.nope; g3.c_bstride = W;
        pick_tile(N, (long long)P.kvl * P.H, 16, &g3.bm, &g3.bn);
        LAUNCH(RDT_STAGE_QKV, dense_gemm(g3, sa));
        QRopeArgs qr{};
        qr.dtype = dt; qr.src = qfull; qr.src_ld = P.H * qw; qr.src_hs = qw; qr.src_off = P.nope;
        qr.dst = qattn; qr.dst_ld = P.H * W; qr.dst_hs = W; qr.dst_off = P.kvl;
        qr.H = P.H; qr.nr = P.nr; qr.rows = cur; qr.ndev = ncur; qr.n = N;
        qr.cosb = cosb; qr.sinb = sinb; qr.S = P.S; qr.pos_dev = pos_dev;
        LAUNCH(RDT_STAGE_QKV, launch_qrope(qr, sa));
        aa.q = qattn; aa.q_ld = P.H * W; aa.q_hs = W;
        LAUNCH(RDT_STAGE_ATTN, launch_attention(aa, sa));
        LAUNCH(RDT_STAGE_ATTN, dense_gemm(g4, sa));
      }
    }

    // a5: output projection (+ depth-wise LoRA as a second K phase)
    const int tl = P.r > 0 ? (t < P.L - 1 ? t : P.L - 1) : 0;
    if (P.r > 0) {
      DenseGemm gz{};
      gz.dtype = dt; gz.A = o; gz.lda = P.hv; gz.K = P.hv; gz.batch = 1; gz.epi = EPI_STORE;
      gz.rows = cur; gz.gather = 0; gz.M = N; gz.Mdev = ncur;
      gz.nseg = 1;
      gz.seg[0] = GemmSeg{elt_ptr(w.lora_down, (long long)tl * P.r * P.hv, elt), P.r, z, P.r, 0, 0, 0};
      gz.bm = 128; gz.bn = 64;
      if ((N + 127) / 128 < 256) gz.bm = 64;
      LAUNCH(RDT_STAGE_OPROJ, dense_gemm(gz, sa));
    }
    DenseGemm go{};
    go.dtype = dt; go.A = o; go.lda = P.hv; go.K = P.hv; go.batch = 1; go.epi = EPI_STORE;
    go.rows = cur; go.gather = 0; go.M = N; go.Mdev = ncur;
    go.nseg = 1; go.seg[0] = GemmSeg{w.Wo, D, abuf, D, 0, 0, 1};
    if (P.r > 0) {
      go.A2 = z; go.lda2 = P.r; go.B2 = elt_ptr(w.lora_up, (long long)tl * D * P.r, elt); go.K2 = P.r;
    }
    pick_tile(N, D, 16, &go.bm, &go.bn);
    if (act && t >= kActSmallTilesFrom && bf) go.bm = go.bn = 64;
    LAUNCH(RDT_STAGE_OPROJ, dense_gemm(go, sa));
    if (fork) HIPCHK(hipEventRecord(f.ev_join, sa));

    // a5-a6: x = u + a, n2 = RMSNorm(x) * g2 (compacted rows), router softmax /
    // top-k, and the stable expert permutation, in one kernel
    NormRouteArgs nr{};
    NormArgs& n2a = nr.norm;
    // parallel block: the MoE reads RMSNorm(u); sequential: RMSNorm(u [+ d] + a)
    n2a.dtype = dt; n2a.h = f.out; n2a.e = f.e; n2a.a = par ? nullptr : abuf; n2a.a2 = (P.da && !par) ? dbuf : nullptr;
    n2a.g = w.g2; n2a.eps = c.norm_eps; n2a.D = D;
    n2a.rows = cur; n2a.ndev = ncur; n2a.n = N; n2a.out = n2; n2a.out_scatter = 0;
    n2a.dump = f.aux.n2_dump ? (void*)elt_ptr(f.aux.n2_dump, (long long)t * N * D, elt) : nullptr;
    nr.Wr = w.Wr; nr.E = E; nr.k = k; nr.smax = smax;
    nr.bias = w.router_bias && c.n_bias_rows > 0
                  ? w.router_bias + (size_t)(t < c.n_bias_rows - 1 ? t : c.n_bias_rows - 1) * E
                  : nullptr;
    nr.idx = idx; nr.gates = gates; nr.gap = gap;
    nr.dump_idx = f.aux.route_idx ? f.aux.route_idx + (size_t)t * N * k : nullptr;
    nr.dump_gap = f.aux.route_gap ? f.aux.route_gap + (size_t)t * N : nullptr;
    int* cnt = cnt2 + (t & 1) * E;
    nr.cnt = cnt; nr.slot = slot; nr.pcap = pcap; nr.cap = N;
    LAUNCH(RDT_STAGE_ROUTER, launch_norm_route(nr, s));

    // a7: grouped SwiGLU experts
    GroupedGemm gu{};
    gu.dtype = dt; gu.kind = 0; gu.A = n2; gu.lda = D;
    gu.cnt = cnt; gu.pcap = pcap; gu.cap = N; gu.ndev = ncur; gu.n_static = N;
    gu.E = E; gu.Se = P.Se; gu.k = k; gu.W1 = w.Wg; gu.W2 = w.Wu; gu.S1 = w.Wsg; gu.S2 = w.Wsu;
    gu.N = P.F; gu.K = D; gu.C = hmid; gu.ldc = P.F;
    gu.bm = gu_bm; gu.bn = gu_bn; gu.ns = gu_bm == 64 ? 3 : 2; gu.max_mtiles = max_mtiles(gu.bm);
    LAUNCH(RDT_STAGE_EXPERT_GU, launch_grouped_gemm(gu, s));
    GroupedGemm gd{};
    gd.dtype = dt; gd.kind = 1; gd.A = hmid; gd.lda = P.F;
    gd.cnt = cnt; gd.pcap = pcap; gd.cap = N; gd.ndev = ncur; gd.n_static = N;
    gd.E = E; gd.Se = P.Se; gd.k = k; gd.W1 = w.Wd; gd.W2 = nullptr; gd.S1 = w.Wsd; gd.S2 = nullptr;
    gd.N = D; gd.K = P.F; gd.C = ybuf; gd.ldc = D;
    const long long ystride = (long long)N * (k + P.Se) * D;
    gd.ksplit = P.ksplit; gd.part = P.ksplit > 1 ? reinterpret_cast<float*>(ybuf) : nullptr; gd.pstride = ystride;
    // many rows per expert: large tiles; few rows: small tiles, deeper ring
    if (pp_dn) { gd.bm = 256; gd.bn = 256; gd.ns = 2; }
    else if (dn_bm == 128) { gd.bm = 192; gd.bn = 128; gd.ns = 2; }
    else { gd.bm = 64; gd.bn = rows_per_expert < 64 && bf ? 32 : 64; gd.ns = 3; }
    gd.max_mtiles = max_mtiles(gd.bm);
    LAUNCH(RDT_STAGE_EXPERT_DOWN, launch_grouped_gemm(gd, s));

    // a8: combine + LTI injection (+ ACT)
    CombineArgs ca{};
    ca.dtype = dt; ca.h = f.out; ca.e = f.e; ca.a = abuf; ca.A = w.A; ca.B = w.B;
    ca.Y = ybuf; ca.ksplit = P.ksplit; ca.Yp = reinterpret_cast<const float*>(ybuf); ca.ystride = ystride;
    ca.gates = gates; ca.idx = idx; ca.slot = slot; ca.cnt = cnt; ca.E = E;
    ca.cnt_next = cnt2 + ((t + 1) & 1) * E;
    ca.counts_dump = f.aux.expert_counts ? f.aux.expert_counts + (size_t)t * E : nullptr;
    ca.k = k; ca.Se = P.Se; ca.D = D;
    ca.rows = cur; ca.ndev = ncur; ca.n = N;
    ca.act = act; ca.w_halt = w.w_halt; ca.thr = c.act_threshold; ca.cum = cum; ca.loops = f.aux.loops; ca.t = t;
    ca.cum_dump = f.aux.act_cum ? f.aux.act_cum + (size_t)t * N : nullptr;
    ca.a_dump = f.aux.a_dump ? f.aux.a_dump + (size_t)t * N * D : nullptr;
    ca.n1_out = t + 1 < f.T ? (P.da ? nd : n1) : nullptr; ca.g1 = P.da ? w.g_da : w.g1; ca.eps = c.norm_eps;
    ca.d = P.da ? dbuf : nullptr; ca.smax = smax;
    if (act) {   // the stable compaction of the active list runs inside the combine launch
      ca.seg_in = seg; ca.rows_out = lists + (size_t)(t + 1) * N; ca.n_out = ncount + t + 1;
      ca.seg_out = segs + (size_t)(t + 1) * (P.B + 1); ca.nseq = P.B;
      ca.wg_mask = at<int>(ws, P.wgmask); ca.wg_tmp = at<int>(ws, P.wgtmp); ca.done = at<int>(ws, P.cnt) + P.att_cnt;
    }
    if (fork) HIPCHK(hipStreamWaitEvent(s, f.ev_join, 0));   // the attention branch has written a
    LAUNCH(RDT_STAGE_COMBINE, launch_combine(ca, s));
    if (f.aux.h_dump) LAUNCH(RDT_STAGE_OTHER, launch_copy_f32(f.aux.h_dump + (size_t)(t + 1) * N * D, f.out, (long long)N * D, s));
  }
  return RDT_OK;
}

static bool misaligned(const void* p, size_t a) { return p && (reinterpret_cast<uintptr_t>(p) % a) != 0; }

static rdt_status check_weights(const rdt_config& c, const rdt_weights* w) {
  if (!w) return set_err(RDT_E_INVALID, "null weights");
  const void* need[32];
  const char* names[32];
  int n = 0;
  auto req = [&](const void* p, const char* nm) { need[n] = p; names[n] = nm; ++n; };
  req(w->g1, "g1"); req(w->g2, "g2"); req(w->Wo, "Wo"); req(w->Wr, "Wr");
  req(w->Wg, "Wg"); req(w->Wu, "Wu"); req(w->Wd, "Wd"); req(w->A, "A"); req(w->B, "B");
  if (c.attn_type == RDT_ATTN_GQA) {
    req(w->Wq, "Wq"); req(w->Wk, "Wk"); req(w->Wv, "Wv");
  } else {
    req(w->Wdq, "Wdq"); req(w->gq, "gq"); req(w->Wuq, "Wuq"); req(w->Wdkv, "Wdkv");
    req(w->gkv, "gkv"); req(w->Wuk, "Wuk"); req(w->Wuv, "Wuv");
  }
  if (c.n_shared_experts > 0) { req(w->Wsg, "Wsg"); req(w->Wsu, "Wsu"); req(w->Wsd, "Wsd"); }
  if (c.lora_rank > 0) { req(w->lora_down, "lora_down"); req(w->lora_up, "lora_up"); }
  if (c.act_enabled) req(w->w_halt, "w_halt");
  if (c.da_heads > 0) {
    req(w->Wq_da, "Wq_da"); req(w->Wk_da, "Wk_da"); req(w->Wv_da, "Wv_da"); req(w->Wo_da, "Wo_da");
    req(w->g_da, "g_da");
  }
  for (int i = 0; i < n; ++i) {
    if (!need[i]) return set_err(RDT_E_INVALID, std::string("null weight pointer: ") + names[i]);
    if (misaligned(need[i], 16)) return set_err(RDT_E_INVALID, std::string("weight not 16-byte aligned: ") + names[i]);
  }
  if (misaligned(w->router_bias, 4)) return set_err(RDT_E_INVALID, "router_bias misaligned");
  return RDT_OK;
}

// rho(A) < 1 for the per-channel A, checked once per A pointer: the first call
// with a pointer copies A to the host (a stack buffer; dim <= 4096 is
// validated) and waits for it. A rewritten in place under the same pointer is
// not checked again.
static rdt_status check_rho(rdt_handle* h, const float* A, hipStream_t s) {
  for (int i = 0; i < h->n_checked && i < kRhoSlots; ++i)
    if (h->checked_A[i] == A) return RDT_OK;
  float host[4096];
  const int dim = h->cfg.dim;
  if (dim > 4096) return set_err(RDT_E_UNSUPPORTED, "dim above 4096");
  HIPCHK(hipMemcpyAsync(host, A, (size_t)dim * 4, hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  float rho = 0.f;
  rdt_spectral_radius(host, dim, &rho);
  if (!(rho < 1.f)) {
    char buf[96];
    snprintf(buf, sizeof buf, "unstable injection: rho(A) = %.6g >= 1", (double)rho);
    return set_err(RDT_E_UNSTABLE, buf);
  }
  h->checked_A[h->n_checked % kRhoSlots] = A;
  h->n_checked += 1;
  return RDT_OK;
}

// Argument checks shared by the forward entry points; fills *f. `rows` is the
// number of state rows (batch*seq for a forward, batch for a decode step).
static rdt_status prepare(rdt_handle* h, const float* h0, const float* e, const rdt_weights* w, int32_t T,
                          float* out, const rdt_aux* aux, void* ws, size_t ws_bytes, Fwd& f, bool decode = false,
                          int max_seq = 0) {
  if (!h) return set_err(RDT_E_INVALID, "null handle");
  const rdt_config& c = h->cfg;
  if (T < 0 || T > c.max_T) return set_err(RDT_E_INVALID, "T must be in [0, max_T]");
  if (!h0 || !e || !out) return set_err(RDT_E_INVALID, "null h0, e or out");
  if (misaligned(h0, 16) || misaligned(e, 16) || misaligned(out, 16))
    return set_err(RDT_E_INVALID, "h0, e and out must be 16-byte aligned");
  const size_t bytes = (size_t)c.batch * (decode ? 1 : c.seq) * c.dim * 4;
  auto overlap = [&](const void* a, const void* b) {
    const char* x = (const char*)a;
    const char* y = (const char*)b;
    return x < y + bytes && y < x + bytes;
  };
  if (out != h0 && overlap(out, h0)) return set_err(RDT_E_INVALID, "out partially overlaps h0");
  if (overlap(out, e)) return set_err(RDT_E_INVALID, "out overlaps e");
  rdt_status st = check_weights(c, w);
  if (st != RDT_OK) return st;
  f = Fwd{};
  f.c = &h->cfg;
  f.P = decode ? make_decode_plan(c, T, max_seq) : make_plan(c, T);
  if (!ws || ws_bytes < f.P.total) return set_err(RDT_E_WORKSPACE, "workspace missing or too small");
  if (misaligned(ws, 256)) return set_err(RDT_E_INVALID, "workspace must be 256-byte aligned");
  f.h0 = h0; f.e = e; f.w = w; f.T = T; f.out = out; f.ws = (char*)ws;
  f.side = h->side; f.ev_fork = h->ev_fork; f.ev_join = h->ev_join;
  f.decode = decode ? 1 : 0;
  f.max_seq = max_seq;
  if (aux) f.aux = *aux;
  return RDT_OK;
}

// Cache arguments of rdt_prefill / rdt_decode_step.
static rdt_status check_cache(rdt_handle* h, int32_t T, void* cache, int32_t max_seq, int32_t need_seq) {
  if (max_seq <= 0 || max_seq < need_seq) return set_err(RDT_E_INVALID, "max_seq too small");
  if (T < 1) return set_err(RDT_E_INVALID, "a cache needs T >= 1");
  if (!cache) return set_err(RDT_E_INVALID, "null cache");
  if (misaligned(cache, 256)) return set_err(RDT_E_INVALID, "cache must be 256-byte aligned");
  if ((long long)h->cfg.batch * max_seq > (1ll << 30)) return set_err(RDT_E_UNSUPPORTED, "cache too long");
  return RDT_OK;
}

// Enqueue f on s: replay (capturing on first use) the HIP graph of this
// argument set, or launch the kernels one by one when graphs are off.
static rdt_status launch(rdt_handle* h, const Fwd& f, hipStream_t s) {
  if (!h->graph_mode || f.T == 0) return enqueue(f, s);
  GraphKey key{};
  int nk = 0;
  const void* const* wv = reinterpret_cast<const void* const*>(f.w);
  for (size_t i = 0; i < sizeof(rdt_weights) / sizeof(void*); ++i) key.ptrs[nk++] = wv[i];
  const void* const* av = reinterpret_cast<const void* const*>(&f.aux);
  for (size_t i = 0; i < sizeof(rdt_aux) / sizeof(void*); ++i) key.ptrs[nk++] = av[i];
  key.ptrs[nk++] = f.h0; key.ptrs[nk++] = f.e; key.ptrs[nk++] = f.out; key.ptrs[nk++] = f.ws;
  key.ptrs[nk++] = f.cache;
  key.T = f.T; key.max_seq = f.max_seq; key.decode = f.decode;
  for (auto& g : h->graphs)
    if (g.key == key) {
      HIPCHK(hipGraphLaunch(g.exec, s));
      return RDT_OK;
    }
  HIPCHK(hipStreamBeginCapture(h->cap, hipStreamCaptureModeThreadLocal));
  rdt_status st = enqueue(f, h->cap);
  hipGraph_t graph = nullptr;
  hipError_t ce = hipStreamEndCapture(h->cap, &graph);
  if (st != RDT_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return st;
  }
  if (ce != hipSuccess) return set_err(RDT_E_HIP, std::string("graph capture failed: ") + hipGetErrorString(ce));
  hipGraphExec_t exec = nullptr;
  ce = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (ce != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return set_err(RDT_E_HIP, std::string("graph instantiate failed: ") + hipGetErrorString(ce));
  }
  if (h->graphs.size() >= 16) {
    (void)hipGraphExecDestroy(h->graphs.front().exec);
    (void)hipGraphDestroy(h->graphs.front().graph);
    h->graphs.erase(h->graphs.begin());
  }
  h->graphs.push_back(GraphEntry{key, graph, exec});
  HIPCHK(hipGraphLaunch(exec, s));
  return RDT_OK;
}

static const char* kStageNames[RDT_N_STAGES] = {"norm1", "qkv", "attention", "out_proj", "norm2", "router",
                                                "permute", "expert_gate_up", "expert_down", "combine",
                                                "compact", "other", "depth_attention"};

extern "C" const char* rdt_stage_name(int32_t stage) {
  return (stage >= 0 && stage < RDT_N_STAGES) ? kStageNames[stage] : "";
}

extern "C" rdt_status rdt_profile_forward(rdt_handle* h, const float* h0, const float* e, const rdt_weights* w,
                                          int32_t T, float* out, const rdt_aux* aux, void* ws, size_t ws_bytes,
                                          void* stream, float* stage_ms, int32_t* stage_launches, int32_t n_stages) {
  if (!stage_ms || !stage_launches || n_stages < RDT_N_STAGES)
    return set_err(RDT_E_INVALID, "rdt_profile_forward: stage arrays missing or too short");
  Fwd f;
  rdt_status st = prepare(h, h0, e, w, T, out, aux, ws, ws_bytes, f);
  if (st != RDT_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  st = check_rho(h, w->A, s);
  if (st != RDT_OK) return st;
  Prof prof;
  st = enqueue(f, s, &prof);
  HIPCHK(hipStreamSynchronize(s));
  if (st != RDT_OK) return st;
  for (int i = 0; i < n_stages; ++i) { stage_ms[i] = 0.f; stage_launches[i] = 0; }
  for (auto& r : prof.recs) {
    float ms = 0.f;
    HIPCHK(hipEventElapsedTime(&ms, r.a, r.b));
    stage_ms[r.stage] += ms;
    stage_launches[r.stage] += 1;
  }
  return RDT_OK;
}

extern "C" rdt_status rdt_recurrent_forward(rdt_handle* h, const float* h0, const float* e, const rdt_weights* w,
                                            int32_t T, float* out, const rdt_aux* aux, void* ws, size_t ws_bytes,
                                            void* stream) {
  Fwd f;
  rdt_status st = prepare(h, h0, e, w, T, out, aux, ws, ws_bytes, f);
  if (st != RDT_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  st = check_rho(h, w->A, s);
  if (st != RDT_OK) return st;
  return launch(h, f, s);
}

extern "C" rdt_status rdt_recurrent_forward_noalloc(rdt_handle* h, const float* h0, const float* e,
                                                    const rdt_weights* w, int32_t T, float* out,
                                                    const rdt_aux* aux, void* stream) {
  if (!h) return set_err(RDT_E_INVALID, "null handle");
  void* ws = scratch_of(h->device);
  if (!ws) return set_err(RDT_E_HIP, "no scratch address for this handle's device");
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != h->device)
    return set_err(RDT_E_INVALID, "the handle's device must be current");
  if (T >= 0 && T <= h->cfg.max_T) {
    const size_t need = make_plan(h->cfg, T).total;
    if (need > (size_t)RDT_NOALLOC_SCRATCH_BYTES) {
      char buf[160];
      snprintf(buf, sizeof buf, "rdt_recurrent_forward_noalloc: this config needs %zu workspace bytes; the static "
               "scratch holds %zu (use rdt_recurrent_forward with a workspace)", need,
               (size_t)RDT_NOALLOC_SCRATCH_BYTES);
      return set_err(RDT_E_WORKSPACE, buf);
    }
  }
  Fwd f;
  rdt_status st = prepare(h, h0, e, w, T, out, aux, ws, (size_t)RDT_NOALLOC_SCRATCH_BYTES, f);
  if (st != RDT_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  st = check_rho(h, w->A, s);
  if (st != RDT_OK) return st;
  return enqueue(f, s);   // launched one by one: instantiating a graph would allocate
}

extern "C" size_t rdt_cache_size(const rdt_config* cfg, int32_t T, int32_t max_seq) {
  if (!cfg || validate_config(*cfg, nullptr) != RDT_OK || T > cfg->max_T) return 0;
  return cache_bytes(*cfg, T, max_seq);
}

extern "C" rdt_status rdt_prefill(rdt_handle* h, const float* h0, const float* e, const rdt_weights* w, int32_t T,
                                  float* out, const rdt_aux* aux, void* cache, int32_t max_seq, void* ws,
                                  size_t ws_bytes, void* stream) {
  if (!h) return set_err(RDT_E_INVALID, "null handle");
  rdt_status st = check_cache(h, T, cache, max_seq, h->cfg.seq);
  if (st != RDT_OK) return st;
  Fwd f;
  st = prepare(h, h0, e, w, T, out, aux, ws, ws_bytes, f);
  if (st != RDT_OK) return st;
  f.cache = (char*)cache;
  f.max_seq = max_seq;
  hipStream_t s = (hipStream_t)stream;
  st = check_rho(h, w->A, s);
  if (st != RDT_OK) return st;
  return launch(h, f, s);
}

extern "C" size_t rdt_decode_workspace_size(const rdt_handle* h, int32_t T, int32_t max_seq) {
  if (!h || T < 0 || T > h->cfg.max_T || max_seq <= 0) return 0;
  return make_decode_plan(h->cfg, T, max_seq).total;
}

extern "C" rdt_status rdt_decode_step(rdt_handle* h, const float* h0, const float* e, const rdt_weights* w,
                                      int32_t T, int32_t pos, void* cache, int32_t max_seq, float* out,
                                      const rdt_aux* aux, void* ws, size_t ws_bytes, void* stream) {
  if (!h) return set_err(RDT_E_INVALID, "null handle");
  rdt_status st = check_cache(h, T, cache, max_seq, 1);
  if (st != RDT_OK) return st;
  if (pos < 0 || pos >= max_seq) return set_err(RDT_E_INVALID, "pos must be in [0, max_seq)");
  Fwd f;
  st = prepare(h, h0, e, w, T, out, aux, ws, ws_bytes, f, true, max_seq);
  if (st != RDT_OK) return st;
  f.cache = (char*)cache;
  hipStream_t s = (hipStream_t)stream;
  st = check_rho(h, w->A, s);
  if (st != RDT_OK) return st;
  // the position lives in the workspace, so one captured graph serves every step
  HIPCHK(launch_fill_i32(reinterpret_cast<int*>(f.ws + f.P.pos), pos, 1, s));
  return launch(h, f, s);
}

extern "C" rdt_status rdt_router_bias_update(const int32_t* expert_counts, int32_t T, int32_t E, float* router_bias,
                                             int32_t rows, float gamma, void* stream) {
  if ((!expert_counts && T > 0) || !router_bias) return set_err(RDT_E_INVALID, "null counts or bias");
  if (T < 0 || E <= 0 || rows <= 0) return set_err(RDT_E_INVALID, "T must be >= 0, E and rows positive");
  if (!(gamma >= 0.f) || !std::isfinite(gamma)) return set_err(RDT_E_INVALID, "gamma must be finite and >= 0");
  HIPCHK(launch_bias_update(expert_counts, T, E, router_bias, rows, gamma, (hipStream_t)stream));
  return RDT_OK;
}

extern "C" rdt_status rdt_expert_depths(const int32_t* expert_counts, int32_t T, int32_t E, int32_t* depths,
                                        void* stream) {
  if ((!expert_counts && T > 0) || !depths) return set_err(RDT_E_INVALID, "null counts or depths");
  if (T < 0 || E <= 0) return set_err(RDT_E_INVALID, "T must be >= 0 and E positive");
  HIPCHK(launch_expert_depths(expert_counts, T, E, depths, (hipStream_t)stream));
  return RDT_OK;
}
