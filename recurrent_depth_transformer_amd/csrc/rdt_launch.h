// Internal launch interface between the host orchestration (rdt_api.cpp) and
// the HIP kernels (rdt_gemm.hip, rdt_attention.hip, rdt_rows.hip). Plain
// structs of device pointers and sizes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rdt {

enum { DT_F32 = 0, DT_BF16 = 1 };

// Tiles of the fp32 grouped expert GEMMs (the bf16 tiles are chosen per
// launch from the rows per expert; gate/up columns hold gate and up halves).
constexpr int GU_BM = 128;
constexpr int GU_BN = 128;
constexpr int DN_BM = 64;
constexpr int DN_BN = 128;
constexpr int MAX_EXPERTS = 64;

// ---------------------------------------------------------------- dense GEMM
// C[i, :] = A[row(i), :K] . B^T (+ A2[i, :K2] . B2^T), fp32 accumulation.
// B is split by output column into up to three segments, each with its own
// weight matrix and destination.
struct GemmSeg {
  const void* B;   // [ncols, K] row-major (row stride K)
  int ncols;
  void* C;         // destination base
  int ldc;         // destination row stride in elements
  int scatter;     // 1: destination row = token id of row i; 0: row i
  int rope;        // apply half-split RoPE per head of width rope_dim
  int out_f32;     // write float instead of the storage type
  int row_mul;     // nonzero: destination row = token id * row_mul + *pos_dev
                   // (one-token decode writing straight into a per-loop cache)
};

enum { EPI_STORE = 0, EPI_ROUTER = 1 };

struct RouterEpi {
  const float* bias;     // [E] selection bias row, may be null
  int E, k;
  int* idx;              // [n, k] compacted
  float* gates;          // [n, k]
  float* gap;            // [n]
  int* dump_idx;         // [N, k] by token, may be null
  float* dump_gap;       // [N] by token, may be null
};

struct DenseGemm {
  int dtype;
  const void* A; int lda; long long a_bstride;
  const int* rows;       // token id of compacted row i (null: identity)
  int gather;            // A row = rows[i] (1) or i (0)
  int M; const int* Mdev;
  int K;
  int nseg; GemmSeg seg[3];
  long long b_bstride, c_bstride;
  int batch;
  const void* A2; int lda2; const void* B2; int K2;   // optional second K phase
  const float* cosb; const float* sinb; int rope_dim; int seq;
  int epi;
  RouterEpi router;
  const int* pos_dev;    // RoPE at position *pos_dev for every row (one-token decode), else token % seq
  int drope, dpos0, dpos1; // depth RoPE: pairs below rope_dim/4 at dpos0, the rest at dpos1
  int bm, bn;            // tile shape (64 or 128 each)
  int ns;                // bf16 pipeline stages (2..4; 0 = default)
  int nw;                // bf16 waves per workgroup: 8 (64x64 and 128x128 tiles), else 4
};
hipError_t launch_dense_gemm(const DenseGemm& g, hipStream_t s);

// --------------------------------------------------------------- grouped GEMM
// Experts 0..E-1 (routed) and E..E+Se-1 (shared, every active row). Routed
// expert g received cnt[g] rows, listed in pcap[g * cap + 0 .. cnt[g] - 1]
// (any order). Output rows are grouped by expert: routed expert g starts at
// the exclusive prefix sum of cnt, shared expert s at n*k + s*n. Every
// workgroup rebuilds the prefix sums and the tile schedule (ceil(rows / bm)
// tiles per expert) from cnt.
struct GroupedGemm {
  int dtype;
  int kind;              // 0: gate/up + SwiGLU, 1: down projection
  const void* A; int lda;
  const int* cnt; const int* pcap; int cap;
  const int* ndev; int n_static;
  int E, Se, k;
  const void* W1; const void* W2;  // routed weights (gate/up: Wg, Wu; down: Wd)
  const void* S1; const void* S2;  // shared weights (gate/up: Wsg, Wsu; down: Wsd)
  int N, K;
  void* C; int ldc;
  int max_mtiles;
  int bm, bn, ns;        // tile rows, columns, stages
  // down projection only: ksplit > 1 cuts K into ksplit slices of whole
  // 64-wide stages; slice s writes its float partial sums to
  // part + s * pstride (row-major, ldc) instead of C
  int ksplit; float* part; long long pstride;
};
hipError_t launch_grouped_gemm(const GroupedGemm& g, hipStream_t s);

// ------------------------------------------------------------------ attention
struct AttnArgs {
  int dtype;
  int dqk, dv;           // per-head q/k width and v width
  const void* q; int q_ld, q_hs;
  const void* k; int k_ld, k_hs;
  const void* v; int v_ld, v_hs;
  void* o; int o_ld, o_hs;
  int H, KV;
  const int* rows;       // token id of compacted query row (null: identity)
  const int* seg;        // [B+1] start of each sequence in the query list (null: b*S)
  int B, S;
  float scale;           // softmax scale (multiplies q.k)
  // one-token decode: query row i is slot s = rows[i] (or i) at position
  // *dec_pos, its keys are rows s*S .. s*S + *dec_pos of the K/V cache (S is
  // the cache length), and sequence b of the grid is slot b
  int dec; const int* dec_pos;
  // decode only, nsplit > 1: the keys are cut into nsplit ranges of whole
  // tiles, one workgroup each; range r writes its unnormalised output and its
  // running max / sum (exp2 domain) for query row i, head h to
  // part_o[((r * nq + i) * H + h) * dv + d], part_m / part_l[(r * nq + i) * H + h]
  // (nq = B query rows). split_cnt[b * (H / heads per workgroup) + group]
  // (zero on entry, left zero) counts the finished ranges; the last one
  // forms o from all of them
  int nsplit; float* part_o; float* part_m; float* part_l; int* split_cnt;
  int narrow;            // 16-row query slices even where the launch has blocks to spare
  // bf16 absorbed MLA (v == k): the kernel forms its queries itself, and
  // outside key-range splits also the value up-projection. Query row i of
  // head h is [q_nope Wuk[h] | RoPE(q_pe)] with q_nope = qn[i*qn_ld + h*qn_hs
  // + (0..nope)], q_pe the 32 values after it, wukT[h] = Wuk[h]^T ([dv][nope]
  // per head) and the RoPE factors of position p at cosb/sinb[p*16 + j]; q
  // is then unused. Without a split, row i of head h is written as
  // o_lat Wuv[h]^T to ov[i*ov_ld + h*vd + (0..vd)] (wuv: [H][vd][dv]) and o
  // is unused; with one, o receives o_lat as for any other head.
  const void* qn; int qn_ld, qn_hs, nope;
  const void* wukT; const float* cosb; const float* sinb;
  const void* wuv; int vd; void* ov; int ov_ld;
};
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);

// ---------------------------------------------------------------- row kernels
struct NormArgs {
  int dtype;
  const float* h; const float* e; const float* a;  // a optional: x = h + e + a[i]
  const float* a2;       // optional second addend (row i), used by the router kernel
  const float* g; float eps; int D;
  const int* rows; const int* ndev; int n;
  void* out; int out_scatter;
  void* dump;            // optional copy of the output scattered by token
  // first-loop extras, all optional: write the h rows read to h_copy (the
  // forward's output buffer), fill up to two RoPE tables (positions 0..S-1,
  // rotary width dr) from extra workgroups, clear zero[0..zero_n)
  float* h_copy;
  float* rope_cos[2]; float* rope_sin[2]; int rope_S[2], rope_dr[2]; float rope_base;
  int* zero; int zero_n;
};
hipError_t launch_norm(const NormArgs& a, hipStream_t s);

struct CombineArgs {
  int dtype;
  float* h; const float* e; const float* a; const float* A; const float* B;
  const void* Y; const float* gates;
  // routed output row of (i, j): exclusive prefix of cnt at expert idx[i][j],
  // plus slot[i][j]
  const int* idx; const int* slot; const int* cnt; int E;
  int* cnt_next;         // zeroed by workgroup 0 for the next loop's router
  int* counts_dump;      // [E] copy of cnt (may be null)
  int k, Se, D;
  const int* rows; const int* ndev; int n;
  int act; const float* w_halt; float thr; float* cum; int* loops; int t;
  float* cum_dump;       // [N] by token, may be null
  float* a_dump;         // [N, D] by token, may be null
  void* n1_out;          // optional: next loop's RMSNorm(h' + e) * g1 by token
  const float* g1; float eps;
  const float* d;        // optional depth-attention output (row i), added to h'
  const float* smax;     // optional: shared experts weighted by smax[i] (else 1)
  // ksplit > 1: the expert outputs are ksplit float partial sums at
  // Yp + s * ystride (row-major, D), added in slice order; Y is unused
  int ksplit; const float* Yp; long long ystride;
  // ACT compaction (act and rows_out set): the tokens of this launch's list
  // (rows, *ndev of them, in token order) whose halting sum stays below thr
  // go, in the same order, to rows_out (count to *n_out); seg_out[b] is the
  // first position in rows_out of sequence b's tokens (seg_in: the same for
  // the input list), b = 0..nseq. Scratch: wg_mask [grid] (zero on entry,
  // left zero), wg_tmp [grid], done [65] (zero on entry, left zero).
  const int* seg_in; int* rows_out; int* n_out; int* seg_out; int nseq;
  int* wg_mask; int* wg_tmp; int* done;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);



// Second RMSNorm + router + top-k + expert slots. Each pick (i, j) of expert
// e takes slot[i][j] = a unique index below cnt[e] (an atomic reservation per
// workgroup and expert); pcap[e * cap + slot] = i. cnt must be zero on entry.
struct NormRouteArgs {
  NormArgs norm;         // x = h + e (+ a2[i]) (+ a[i]); out = n2 (compacted rows), dump by token
  const void* Wr; int E, k; const float* bias;
  int* idx; float* gates; float* gap; int* dump_idx; float* dump_gap;
  float* smax;           // optional [n]: maximum router probability of row i
  int* cnt; int* slot; int* pcap; int cap;
};
hipError_t launch_norm_route(const NormRouteArgs& a, hipStream_t s);


// -------------------------------------------------------- depth attention
// Row i (token tok = i) and query head h attend over the token's own keys and
// values of loops 0..t: k[tau][tok], v[tau][tok] with loop stride `lstride`
// elements; online softmax in loop order.
struct DepthAttnArgs {
  int dtype;
  const void* q; const void* k; const void* v; void* o;
  long long lstride;     // elements between loops in k and v
  int n, H, KV, dd, t;
  float scale;
};
hipError_t launch_depth_attention(const DepthAttnArgs& a, hipStream_t s);

// ------------------------------------------------------------- MLA helpers
struct MlaNormArgs {
  int dtype;
  const float* cq_raw; int ql;        // [N, ql] by token
  const float* lat_raw; int kvl, nr;  // [N, kvl+nr] by token
  const float* gq; const float* gkv; float eps;
  const int* rows; const int* ndev; int n;
  void* cqn; void* latent;            // T [N, ql], T [N, kvl+nr] by token
  const float* cosb; const float* sinb; int S;
  const int* pos_dev;                 // RoPE at position *pos_dev for every row (decode)
};
hipError_t launch_mla_norm(const MlaNormArgs& a, hipStream_t s);

struct QRopeArgs {
  int dtype;
  const void* src; int src_ld, src_hs, src_off;   // q_pe of row i head h at src + i*ld + h*hs + off
  void* dst; int dst_ld, dst_hs, dst_off;
  int H, nr;
  const int* rows; const int* ndev; int n;
  const float* cosb; const float* sinb; int S;
  const int* pos_dev;
};
hipError_t launch_qrope(const QRopeArgs& a, hipStream_t s);

// ------------------------------------------------------- between forwards
hipError_t launch_bias_update(const int* counts, int T, int E, float* bias, int rows, float gamma, hipStream_t s);
hipError_t launch_expert_depths(const int* counts, int T, int E, int* depths, hipStream_t s);

// ------------------------------------------------------------------ utilities
hipError_t launch_rope_tables(float* cosb, float* sinb, int S, int dr, float base, hipStream_t s);
hipError_t launch_fill_i32(int* p, int v, long long n, hipStream_t s);
hipError_t launch_fill_f32(float* p, float v, long long n, hipStream_t s);
hipError_t launch_fill_u16(uint16_t* p, uint16_t v, long long n, hipStream_t s);
hipError_t launch_iota(int* p, int n, int* count, int count_val, int* seg, int B, int S, hipStream_t s);
hipError_t launch_copy_f32(float* dst, const float* src, long long n, hipStream_t s);
// dst row (r / s_in) * s_out + r % s_in + pos0 <- src row r, for r < nrows,
// with pos0 = *pos_dev (or 0 when null): copies rows of `bytes` bytes (a
// multiple of 16) between strided buffers. Appends per-token K/V or latent
// rows to a per-loop cache.
hipError_t launch_rows_scatter(void* dst, long long dst_ld, const void* src, long long src_ld, int bytes, int nrows,
                               int s_in, int s_out, const int* pos_dev, hipStream_t s);
// dst[h][c][i] = src[h*rows + i][c]: per-head transpose of an [H*rows, cols] matrix
hipError_t launch_head_transpose(int dtype, void* dst, const void* src, int H, int rows, int cols,
                                 hipStream_t s);

}  // namespace rdt
