/*
 * librdt -- recurrent-depth transformer block on AMD Instinct MI355X (gfx950).
 *
 * One call runs the shared recurrent block T times under the LTI injection
 *     h_{t+1} = A (.) h_t + B (.) e + Block(h_t, e)
 * (techbriefly, "Projeto OpenMythos ...": Prelude / Recurrent Block / Coda, the
 * loop update, an MoE layer per iteration, multi-latent attention, rho(A) < 1,
 * ACT halting and depth-wise LoRA). A and B are per-channel vectors
 * (openclawapi, "Introducao ao OpenMythos", Passo 6: get_A() has shape (dim,)).
 * Block(h, e) is the residual branch of a pre-norm transformer block on
 * u = h + e: RMSNorm -> causal GQA or MLA attention -> output projection
 * (+ depth-wise LoRA) -> RMSNorm -> top-k routed SwiGLU mixture of experts
 * (+ always-on shared experts).
 *
 * Conventions for every entry point:
 *   - Device pointers are plain HIP device addresses owned by the caller and
 *     borrowed for the duration of the call (and of the asynchronous work it
 *     enqueues). The library never frees them.
 *   - Row-major layouts; token n = b * seq + s. Weights use the [out, in]
 *     layout of a linear layer.
 *   - "T-type" means the storage type chosen by rdt_config.dtype: float32 for
 *     RDT_F32, bfloat16 (raw 16-bit) for RDT_BF16. RMSNorm gains, A, B, the
 *     router bias and the halting vector are always float32.
 *   - Status codes: RDT_OK (0) or a negative rdt_status. No C++ exception
 *     crosses this boundary. rdt_last_error() describes the last failure of the
 *     calling thread.
 */
#ifndef RDT_H_
#define RDT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rdt_status {
  RDT_OK = 0,
  RDT_E_INVALID = -1,     /* bad argument: null/misaligned pointer, bad shape, T < 0 */
  RDT_E_UNSUPPORTED = -2, /* valid for the method, not supported by these kernels */
  RDT_E_UNSTABLE = -3,    /* rho(A) >= 1 (never clipped) */
  RDT_E_WORKSPACE = -4,   /* workspace missing or smaller than rdt_workspace_size */
  RDT_E_HIP = -5          /* a HIP runtime call failed */
} rdt_status;

typedef enum rdt_attn_type { RDT_ATTN_GQA = 0, RDT_ATTN_MLA = 1 } rdt_attn_type;
typedef enum rdt_dtype { RDT_F32 = 0, RDT_BF16 = 1 } rdt_dtype;

/*
 * Shapes and options of one recurrent block (the MythosConfig fields of
 * openclawapi Passo 2 and Passo 5, plus act_threshold from its troubleshooting
 * item 4). Plain value type, owned by the caller.
 *
 *   batch, seq, dim       tokens are batch*seq rows of width dim
 *   attn_type             RDT_ATTN_GQA or RDT_ATTN_MLA
 *   n_heads, n_kv_heads   query heads; kv heads (GQA; n_heads % n_kv_heads == 0)
 *   head_dim              GQA head width: 16, 32, 64 or 128
 *   q_lora_rank, kv_lora_rank, qk_rope_head_dim, qk_nope_head_dim, v_head_dim
 *                         MLA latent widths and per-head widths
 *   rope_base             RoPE base (half-split rotation, positions 0..seq-1)
 *   norm_eps              RMSNorm epsilon
 *   n_experts, top_k      routed experts and experts per token (top_k <= n_experts <= 64)
 *   n_shared_experts      always-on experts (weight 1, or see shared_scale)
 *   expert_dim            SwiGLU hidden width of every expert
 *   n_bias_rows           rows of the router selection bias; loop t uses row min(t, rows-1)
 *   lora_rank, n_lora     depth-wise LoRA on the attention output projection;
 *                         loop t uses adapter min(t, n_lora-1); rank 0 disables it
 *   act_enabled, act_threshold
 *                         ACT halting: after its update a token adds
 *                         sigmoid(w_halt . h) to its cumulative sum and halts once the
 *                         sum reaches the threshold; a halted token keeps its state
 *   dtype                 RDT_F32 or RDT_BF16 storage of weights and activations
 *   max_T                 largest loop count a workspace is planned for
 * Dreamer block variants (Dreamer summary, Metodologia), all 0 by default:
 *   parallel_block        1: attention and the MoE both read RMSNorm(h + e) (own
 *                         gains) instead of running one after the other
 *   shared_scale          1: shared experts weighted by the token's maximum router
 *                         probability instead of 1
 *   da_heads, da_kv_heads, da_head_dim
 *                         depth attention before sequence attention: every token
 *                         attends over its own states of loops 0..t (depth as the
 *                         sequence), with depth RoPE whose second half of rotary
 *                         pairs uses the reversed depth T-1-t; da_heads = 0 turns
 *                         it off. da_head_dim 16, 32, 64 or 128; not combinable with
 *                         ACT; max_T <= 64
 */
typedef struct rdt_config {
  int32_t batch, seq, dim;
  int32_t attn_type;
  int32_t n_heads, n_kv_heads, head_dim;
  int32_t q_lora_rank, kv_lora_rank, qk_rope_head_dim, qk_nope_head_dim, v_head_dim;
  float rope_base, norm_eps;
  int32_t n_experts, n_shared_experts, top_k, expert_dim;
  int32_t n_bias_rows;
  int32_t lora_rank, n_lora;
  int32_t act_enabled;
  float act_threshold;
  int32_t dtype;
  int32_t max_T;
  int32_t parallel_block;
  int32_t shared_scale;
  int32_t da_heads, da_kv_heads, da_head_dim;
} rdt_config;

/*
 * Device pointers to the block's parameters (all borrowed). Shapes use
 * D = dim, H = n_heads, KV = n_kv_heads, d = head_dim, E = n_experts,
 * Se = n_shared_experts, F = expert_dim, r = lora_rank, L = n_lora,
 * ql/kvl = q/kv latent rank, nr = qk_rope_head_dim, nn = qk_nope_head_dim,
 * vd = v_head_dim, Hv = H*d (GQA) or H*vd (MLA).
 *
 *   g1, g2            float [D]       RMSNorm gains before attention / before the MoE
 *   GQA: Wq [H*d, D], Wk [KV*d, D], Wv [KV*d, D]                         T-type
 *   MLA: Wdq [ql, D], gq float [ql], Wuq [H*(nn+nr), ql] (per head: nn
 *        no-rope rows then nr rope rows), Wdkv [kvl+nr, D] (latent rows then
 *        the shared rope-key rows), gkv float [kvl], Wuk [H*nn, kvl],
 *        Wuv [H*vd, kvl]                                                  T-type
 *   Wo                [D, Hv]         T-type
 *   Wr                [E, D]          T-type router
 *   router_bias float [n_bias_rows, E] selection-only bias (may be null = 0)
 *   Wg, Wu [E, F, D]; Wd [E, D, F]    T-type routed experts
 *   Wsg, Wsu [Se, F, D]; Wsd [Se, D, F] shared experts (null when Se = 0)
 *   lora_down [L, r, Hv]; lora_up [L, D, r]  T-type (null when r = 0)
 *   w_halt float [D]  ACT halting vector (null unless ACT)
 *   A, B float [D]    injection diagonals; rho(A) = max |A_i| must be < 1
 *   depth attention (null unless da_heads > 0; Hd = da_heads, KVd = da_kv_heads,
 *   dd = da_head_dim): Wq_da [Hd*dd, D], Wk_da [KVd*dd, D], Wv_da [KVd*dd, D],
 *   Wo_da [D, Hd*dd] T-type; g_da float [D] its RMSNorm gain
 */
typedef struct rdt_weights {
  const float* g1;
  const float* g2;
  const void* Wq;
  const void* Wk;
  const void* Wv;
  const void* Wdq;
  const float* gq;
  const void* Wuq;
  const void* Wdkv;
  const float* gkv;
  const void* Wuk;
  const void* Wuv;
  const void* Wo;
  const void* Wr;
  const float* router_bias;
  const void* Wg;
  const void* Wu;
  const void* Wd;
  const void* Wsg;
  const void* Wsu;
  const void* Wsd;
  const void* lora_down;
  const void* lora_up;
  const float* w_halt;
  const float* A;
  const float* B;
  const void* Wq_da;
  const void* Wk_da;
  const void* Wv_da;
  const void* Wo_da;
  const float* g_da;
} rdt_weights;

/*
 * Optional device outputs (each pointer may be null). N = batch*seq,
 * k = top_k. Rows of tokens that did not take loop t hold -1 (route_idx),
 * NaN (route_gap, act_cum) or 0 (n2_dump, a_dump).
 *   loops         int32 [N]        updates each token took (T without ACT)
 *   route_idx     int32 [T, N, k]  selected experts, descending selection score
 *   route_gap     float [T, N]     k-th minus (k+1)-th selection score (+inf if k = E)
 *   expert_counts int32 [T, E]     tokens routed to each expert in loop t
 *   act_cum       float [T, N]     cumulative halting sum after loop t (ACT only)
 *   n2_dump       T-type [T, N, D] router input (second RMSNorm output)
 *   a_dump        float [T, N, D]  attention branch a (output projection + LoRA)
 *   h_dump        float [T+1, N, D] state before loop 0 and after every loop
 */
typedef struct rdt_aux {
  int32_t* loops;
  int32_t* route_idx;
  float* route_gap;
  int32_t* expert_counts;
  float* act_cum;
  void* n2_dump;
  float* a_dump;
  float* h_dump;
} rdt_aux;

typedef struct rdt_handle rdt_handle;

/* Fill *cfg with defaults: norm_eps 1e-6, rope_base 1e4, act_threshold 0.99
 * (openclawapi troubleshooting item 4), n_bias_rows 1, max_T 16 (techbriefly:
 * up to 16 iterations), dtype bf16, GQA; shapes zero. RDT_E_INVALID on null. */
rdt_status rdt_config_default(rdt_config* cfg);

/* Check a config without touching the GPU. RDT_E_INVALID for shapes the method
 * cannot have (non-positive sizes, n_heads % n_kv_heads != 0, top_k > n_experts,
 * odd rope width, ...); RDT_E_UNSUPPORTED for valid shapes these kernels do not
 * cover (head_dim not in {16,32,64,128}, n_experts > 64, widths not a multiple
 * of 8, ...). */
rdt_status rdt_config_validate(const rdt_config* cfg);

/* Create a handle for one config on the current HIP device. The handle owns a
 * private capture stream and the cache of captured graphs; it allocates no
 * device memory. The first handle on a device also looks up the device address
 * of that device's static scratch (rdt_recurrent_forward_noalloc); RDT_E_HIP if
 * that fails. *out is set to null on failure. */
rdt_status rdt_create(const rdt_config* cfg, rdt_handle** out);

/* Destroy a handle (null is a no-op). Work it enqueued must have finished. */
void rdt_destroy(rdt_handle* h);

/* Bytes of device workspace one forward needs for loop counts up to T
 * (0 on a null handle or T > max_T). Sized for the worst case: every token
 * active and any expert imbalance. */
size_t rdt_workspace_size(const rdt_handle* h, int32_t T);

/* rho(A) of the per-channel injection A (host array of dim floats):
 * max_i |A_i|, the spectral radius of diag(A) (openclawapi Passo 6).
 * RDT_E_INVALID on null pointers or dim <= 0. */
rdt_status rdt_spectral_radius(const float* A_host, int32_t dim, float* rho);

/* Use captured HIP graphs for the T-loop (enabled != 0, the default) or launch
 * the kernels one by one. Both produce bit-identical results. A graph is
 * captured once per set of pointers (inputs, weights, out, aux, workspace) and
 * T and replayed while they repeat; the handle keeps the last 16. A caller that
 * passes a new out (or workspace) address every call captures every call:
 * reuse the buffers to replay. */
rdt_status rdt_set_graph_mode(rdt_handle* h, int32_t enabled);

/*
 * Run T loops of the recurrent block: out = h_T starting from h0.
 *   h0, e, out  float [batch*seq, dim] device, 16-byte aligned. out may alias h0
 *               exactly; any other overlap is RDT_E_INVALID.
 *   w           parameters (see rdt_weights); aux optional outputs (may be null).
 *   T           loop count, 0 <= T <= max_T (T may exceed the count the weights
 *               were trained for: openclawapi Passo 3, depth extrapolation).
 *               T = 0 copies h0 to out.
 *   ws, ws_bytes device workspace of at least rdt_workspace_size(h, T) bytes,
 *               256-byte aligned; its contents need not be preserved between calls.
 *   stream      hipStream_t to enqueue on (null = the default stream).
 * The work is enqueued asynchronously; the call returns without waiting, except
 * that the first call with a given A pointer copies A to the host once to check
 * rho(A) < 1 (RDT_E_UNSTABLE otherwise; the weights are never clipped,
 * openclawapi troubleshooting item 3). The check is made once per A pointer
 * (the handle remembers the last 8): values rewritten in place under a pointer
 * already checked are not checked again. Kernel faults surface at the caller's
 * next synchronisation. Not thread-safe for one handle.
 */
rdt_status rdt_recurrent_forward(rdt_handle* h, const float* h0, const float* e,
                                 const rdt_weights* w, int32_t T, float* out,
                                 const rdt_aux* aux, void* ws, size_t ws_bytes,
                                 void* stream);

/* Bytes of the static scratch behind rdt_recurrent_forward_noalloc (one copy
 * per device, 32 MiB). */
#define RDT_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * rdt_recurrent_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The workspace is a static device array of
 * RDT_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs on
 * until the process ends; this call allocates nothing (no hipMalloc, no graph
 * instantiation: the kernels are launched one by one on `stream`).
 *   Arguments, layouts and results as for rdt_recurrent_forward; the handle's
 *   device must be current.
 *   RDT_E_WORKSPACE when the config's workspace for T loops
 *   (rdt_workspace_size) exceeds RDT_NOALLOC_SCRATCH_BYTES, before anything is
 *   enqueued; the other errors as for rdt_recurrent_forward.
 * Every call on one device shares that device's scratch: calls whose work
 * overlaps on a device (other streams, other threads, other handles) race and
 * must be serialised by the caller. The scratch keeps the last call's contents;
 * the forward clears what it needs before use. As for rdt_recurrent_forward,
 * the first call with a new A pointer waits for a copy of A to check rho(A),
 * so a caller that captures graphs makes one call before capture.
 */
rdt_status rdt_recurrent_forward_noalloc(rdt_handle* h, const float* h0, const float* e,
                                         const rdt_weights* w, int32_t T, float* out,
                                         const rdt_aux* aux, void* stream);

/*
 * Per-loop key/value cache for incremental decoding. Generation keeps one cache
 * per loop iteration, and MLA caches the compressed kv latent instead of full
 * keys and values (openclawapi Passo 4 and troubleshooting item 1; bigsaas,
 * MLA vs GQA). Device memory owned by the caller, in the storage type of
 * cfg.dtype:
 *   GQA  for each loop t < T: K[t] then V[t], each [batch * max_seq,
 *        n_kv_heads * head_dim]; row b * max_seq + p holds the key (after RoPE)
 *        and the value of position p of sequence b as loop t computed them.
 *   MLA  for each loop t < T: L[t] [batch * max_seq, kv_lora_rank +
 *        qk_rope_head_dim]: the RMS-normalised kv latent, then the rotated
 *        shared rope key.
 * Rows of positions not yet written are never read. Returns the byte size for
 * T loops and max_seq positions per sequence (0 on a null or invalid config,
 * T < 1, T > max_T or max_seq < 1).
 */
size_t rdt_cache_size(const rdt_config* cfg, int32_t T, int32_t max_seq);

/*
 * rdt_recurrent_forward over the cfg.seq prompt tokens of every sequence that
 * also writes each loop's keys and values (MLA: latents) of positions
 * 0..seq-1 into `cache` (rdt_cache_size(cfg, T, max_seq) bytes, 256-byte
 * aligned, max_seq >= seq, T >= 1). Other arguments, workspace and errors are
 * those of rdt_recurrent_forward.
 */
rdt_status rdt_prefill(rdt_handle* h, const float* h0, const float* e, const rdt_weights* w,
                       int32_t T, float* out, const rdt_aux* aux, void* cache, int32_t max_seq,
                       void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of rdt_decode_step for T loops and caches of max_seq
 * positions (0 on a null handle, T > max_T or max_seq < 1). */
size_t rdt_decode_workspace_size(const rdt_handle* h, int32_t T, int32_t max_seq);

/*
 * One decoding step: one new token per sequence, at position pos, runs T loops
 * (openclawapi Passo 4: generation with a per-loop cache). In loop t the
 * token's key and value (MLA: latent) go to row b * max_seq + pos of the loop-t
 * cache and the token attends to rows b * max_seq + 0..pos of it. A prefill of
 * positions 0..pos-1 (or earlier steps) followed by this step therefore gives
 * the state rdt_recurrent_forward computes for that position on the whole
 * sequence (causal attention).
 *   h0, e, out  float [batch, dim] device, 16-byte aligned: the new token of
 *               each sequence; out may alias h0 exactly.
 *   T           loops, 1 <= T <= max_T, the T the cache was filled with.
 *   pos         0 <= pos < max_seq; positions below pos must already be cached.
 *   cache       as for rdt_prefill (same T and max_seq).
 *   aux         optional dumps as for rdt_recurrent_forward, batch rows.
 *   ws          at least rdt_decode_workspace_size(h, T, max_seq) bytes.
 * With ACT a token that halts keeps its frozen key and value in the caches of
 * the remaining loops, so later tokens still see it. Errors as for
 * rdt_recurrent_forward, plus RDT_E_INVALID for pos or max_seq out of range or
 * a null or misaligned cache.
 */
rdt_status rdt_decode_step(rdt_handle* h, const float* h0, const float* e, const rdt_weights* w,
                           int32_t T, int32_t pos, void* cache, int32_t max_seq, float* out,
                           const rdt_aux* aux, void* ws, size_t ws_bytes, void* stream);

/*
 * Auxiliary-loss-free load balancing between forwards (openclawapi
 * troubleshooting item 5: the router bias must be adjusted dynamically in the
 * DeepSeekMoE style or the router settles on a few experts; Dreamer summary,
 * routing: a balancing bias vector as in DeepSeek-V3). For every bias row r,
 * c_e is the number of tokens expert e received in the loops that select with
 * row r (loop t uses row min(t, rows - 1)); an expert below the row's mean
 * load gains gamma, one above it loses gamma, one at the mean is unchanged.
 *   expert_counts  int32 [T, E] device, e.g. rdt_aux.expert_counts of a forward
 *                  (may be null when T = 0: nothing changes)
 *   router_bias    float [rows, E] device, updated in place
 *   gamma          step, finite and >= 0
 * Enqueued on `stream`; deterministic. RDT_E_INVALID on null pointers,
 * T < 0, E <= 0, rows <= 0 or a bad gamma.
 */
rdt_status rdt_router_bias_update(const int32_t* expert_counts, int32_t T, int32_t E,
                                  float* router_bias, int32_t rows, float gamma, void* stream);

/*
 * Expert depth usage (Dreamer summary, expert diversity: how many depths use
 * each expert): depths[e] = number of loops t < T with expert_counts[t][e] > 0.
 *   expert_counts int32 [T, E] device; depths int32 [E] device (written).
 * Enqueued on `stream`. RDT_E_INVALID on null pointers, T < 0 or E <= 0.
 */
rdt_status rdt_expert_depths(const int32_t* expert_counts, int32_t T, int32_t E, int32_t* depths,
                             void* stream);

/* Stages of one loop iteration, for rdt_profile_forward. */
typedef enum rdt_stage {
  RDT_STAGE_NORM1 = 0,    /* u = h + e, RMSNorm */
  RDT_STAGE_QKV = 1,      /* q/k/v projections (+RoPE); MLA latent projections and norms
                             (fp32 MLA: also the query absorb and the query RoPE) */
  RDT_STAGE_ATTN = 2,     /* causal flash attention (bf16 MLA: with the query absorb, the
                             query RoPE and the value up-projection; fp32 MLA: with the
                             value up-projection) */
  RDT_STAGE_OPROJ = 3,    /* output projection (+ depth-wise LoRA) */
  RDT_STAGE_NORM2 = 4,    /* reserved: x = u + a and its RMSNorm run inside the router launch */
  RDT_STAGE_ROUTER = 5,   /* x = u + a, RMSNorm, router logits, softmax, top-k, expert slots */
  RDT_STAGE_PERMUTE = 6,  /* reserved: per-expert counts and slots are taken inside the router launch */
  RDT_STAGE_EXPERT_GU = 7,   /* grouped gate/up GEMM + SwiGLU */
  RDT_STAGE_EXPERT_DOWN = 8, /* grouped down GEMM */
  RDT_STAGE_COMBINE = 9,  /* MoE combine + LTI injection (+ ACT halting and compaction) */
  RDT_STAGE_COMPACT = 10, /* reserved: the ACT active-list compaction runs inside the combine */
  RDT_STAGE_OTHER = 11,   /* per-forward set-up, fills and dump copies */
  RDT_STAGE_DEPTH_ATTN = 12, /* Dreamer depth attention over a token's own loop states */
  RDT_N_STAGES = 13
} rdt_stage;

/*
 * Profiling variant of rdt_recurrent_forward (same arguments and result):
 * launches the kernels one by one on `stream` with a HIP event pair around
 * each launch, waits for completion, and writes for every rdt_stage the summed
 * device time in milliseconds (stage_ms) and the number of launches
 * (stage_launches); both arrays hold n_stages >= RDT_N_STAGES entries (host
 * memory). RDT_E_INVALID on null arrays or n_stages < RDT_N_STAGES.
 */
rdt_status rdt_profile_forward(rdt_handle* h, const float* h0, const float* e,
                               const rdt_weights* w, int32_t T, float* out,
                               const rdt_aux* aux, void* ws, size_t ws_bytes,
                               void* stream, float* stage_ms, int32_t* stage_launches,
                               int32_t n_stages);

/* Short name of a stage ("" when out of range). */
const char* rdt_stage_name(int32_t stage);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* rdt_last_error(void);

/* Library version string. */
const char* rdt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RDT_H_ */
