/*
 * spd.h - C ABI of the single-GPU Speculative Pipeline Decoding (SPD) hot path.
 *
 * The method (arXiv 2605.30852, as summarised on the pith.science review
 * page, "What carries the argument" and "Core claim"; aiqbench abstract):
 * the target LLM is cut into n pipeline stages so that n tokens of ONE
 * sequence advance at once, each in a different stage; a Pipeline Draft
 * Module (PDM) reads the pipeline's input states, concatenates hidden states
 * at anchor depths B, projects k*d -> d, and runs Ls decoder layers plus the
 * LM head to draft the next token while the step runs; the token leaving the
 * last stage verifies the next position (greedy match, or rejection sampling
 * as in Leviathan et al. 2023 at temperature > 0), and a rejection truncates
 * the KV cache, flushes the pipeline and reseeds it. On one GPU every step
 * runs all n stage slices as grouped launches (the "depth staircase").
 *
 * Conventions
 *   - Every call returns SPD_OK or a negative SPD_E_* code; no exception ever
 *     crosses this boundary. spd_last_error() then holds a message.
 *   - Ownership: the caller owns the weights (device memory), the workspace
 *     (device memory of spd_workspace_bytes() bytes) and the HIP stream; the
 *     library borrows them until spd_destroy(). The library owns the handle
 *     and a few pinned host staging buffers that it allocates in spd_init().
 *     No step call allocates memory.
 *   - Call order: spd_init -> spd_prefill -> (spd_step -> spd_verify_commit)*.
 *     Any other order returns SPD_E_STATE and changes nothing.
 *   - A handle is used from one host thread and one stream.
 *   - Host pointers are marked [host]; all others are device pointers.
 */
#ifndef SPD_H
#define SPD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct spd_handle spd_handle;   /* opaque, library-owned */

enum {
  SPD_OK = 0,
  SPD_E_ARG = -1,       /* null or out-of-range argument */
  SPD_E_CONFIG = -2,    /* configuration the library does not support */
  SPD_E_STATE = -3,     /* call out of order */
  SPD_E_CAPACITY = -4,  /* a position would reach max_ctx, or workspace too small */
  SPD_E_DEVICE = -5     /* a HIP runtime call failed */
};

enum { SPD_F32 = 0, SPD_BF16 = 1 };                 /* weight (and KV cache) storage */
enum { SPD_FILL_CLAMP = 0, SPD_FILL_ZERO = 1 };      /* anchors not computed yet */
enum { SPD_LAYER_SOFTMAX = 0, SPD_LAYER_LINEAR = 1 };
enum { SPD_SPEC_INPUT = 0, SPD_SPEC_OUTPUT = 1 };     /* which states the PDM reads */
enum { SPD_KV_AUTO = 0, SPD_KV_F32 = 1 };             /* KV cache storage */

/*
 * Model and SPD configuration. Free parameters in the pages' notation
 * (pith.science review, "Assumptions & free parameters"): anchors B, pipeline
 * width n, speculation layers Ls, temperature T.
 *   n_layers = L; n_stages = n (1 <= n <= L);
 *   stage_layers [host, n entries, each >= 1, sum = L] or NULL for the default split
 *     (the first L mod n stages get ceil(L/n) layers);
 *   anchors [host, k entries]: depths b in [0, L], strictly ascending, anchors[0] == 0;
 *     anchor b is the residual stream after b target layers (b = 0: embedding);
 *   pdm_layers = Ls >= 1 (Ls > L/n is allowed: the PDM is then simply not
 *     latency-masked, which the pages state as the condition Ls <= L/n);
 *   layer_kind [host, L entries] SPD_LAYER_* or NULL for all softmax. A linear
 *     layer has n_q_heads heads of head_dim with an hd x hd fp32 state per head,
 *     S <- gamma_h S + k^ v^T, o = S^T q^ (q^, k^ unit-normalised, gamma_h =
 *     1 - 2^-(5 + h mod 8), no RoPE); the state after each position is kept in a
 *     ring of n + 1 slots, so a rejection restores it without a copy. PDM layers
 *     are always softmax;
 *   anchor_fill: how a PDM row fills anchors deeper than its current depth:
 *     SPD_FILL_CLAMP repeats the deepest computed anchor (default), SPD_FILL_ZERO uses 0;
 *   max_ctx: KV capacity in positions; every in-flight position must stay below it;
 *   speculate_from: SPD_SPEC_INPUT (0, the method's early start, pith.science review
 *     "Core claim"): the PDM reads the step's input states and runs alongside the step
 *     on a second stream. SPD_SPEC_OUTPUT (1, the input- vs output-state ablation its
 *     referee summary mentions): the PDM runs after the step's target layers on the
 *     states they produced, one stage deeper (the exiting token at depth L, whose PDM
 *     row becomes permanent in the same step), on the caller's stream.
 *   kv_dtype: SPD_KV_AUTO (0) stores the target and PDM KV caches in the weight dtype
 *     (bf16 keys and values, rounded to nearest even, for bf16 weights); SPD_KV_F32 (1)
 *     stores them in fp32 with bf16 weights too: twice the KV bytes, and no bf16
 *     rounding of K and V, whose one-ulp flips deep, wide models amplify in the logits.
 *   draft_width: W, candidates the PDM proposes per draft position (0 or 1: a chain;
 *     at most 4; any other value is SPD_E_CONFIG). The pith.science review lists W = 1 and 4 among the paper's free
 *     parameters ("Assumptions & free parameters"). With W > 1 each draft position
 *     carries the PDM's W best candidates (largest logits at T = 0; at T > 0 the W
 *     largest log q + Gumbel scores, a draw without replacement from q), ranked best
 *     first; rank 0 (the spine) is the token the next positions build on, ranks 1..W-1
 *     (siblings) run through the same layers at the same position, each attending to
 *     the cache plus its own key. Verification tests them in rank order (see
 *     spd_sampling); an accepted sibling becomes the token at its position, keeping
 *     the layers it has run, and the positions after it are flushed. Needs softmax
 *     layers only, SPD_SPEC_INPUT, top_p >= 1 and forced_mode 0.
 * Limits: d_model, d_ffn, n_q_heads*head_dim multiples of 8; head_dim in
 * {16, 32, 64, 80, 128}; n_q_heads a multiple of n_kv_heads with at most 16 query
 * heads per KV head; n <= 16; k <= 8; Ls <= 16.
 */
typedef struct {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, d_ffn, vocab;
  int32_t dtype;                  /* SPD_F32 | SPD_BF16 */
  float rope_theta, rms_eps;
  const uint8_t* layer_kind;      /* [host] */
  int32_t n_stages;
  const int32_t* stage_layers;    /* [host] */
  int32_t n_anchors;
  const int32_t* anchors;         /* [host] */
  int32_t pdm_layers;
  int32_t anchor_fill;
  int32_t max_ctx;
  int32_t speculate_from;         /* SPD_SPEC_INPUT | SPD_SPEC_OUTPUT */
  int32_t kv_dtype;               /* SPD_KV_AUTO | SPD_KV_F32 */
  int32_t draft_width;            /* W: candidates per draft position, 1..4 (0 means 1;
                                     other values: SPD_E_CONFIG) */
} spd_model_config;

/*
 * Weights: device pointers owned by the caller, row-major, K (input) dimension
 * contiguous. Matrices are stored in cfg.dtype; RMSNorm gains are float32.
 *   embed   [V][d]        lm_head [V][d]   (tied: the PDM uses the same head)
 *   final_norm [d] f32    pdm_final_norm [d] f32
 *   pdm_proj [d][k*d]     input order: anchor 0's d values, then anchor 1's, ...
 *   layers  [host] array of 7*L device pointers, per layer in this order:
 *     attn_norm [d] f32,
 *     w_qkv  softmax layer: [(hq + 2 hkv) hd][d], q rows then k rows then v rows;
 *            linear layer:  [3 hq hd][d]
 *     w_o [d][hq hd], ffn_norm [d] f32, w_gate [F][d], w_up [F][d], w_down [d][F]
 *   pdm_layers [host] array of 7*Ls pointers, same order (softmax layers).
 */
typedef struct {
  const void* embed;
  const void* lm_head;
  const float* final_norm;
  const void* const* layers;
  const void* pdm_proj;
  const void* const* pdm_layers;
  const float* pdm_final_norm;
} spd_weights;

/*
 * Sampling. temperature == 0: greedy drafts and greedy verification
 * (lossless: the committed stream is the target's greedy stream).
 * temperature > 0: drafts d ~ q = softmax(z_pdm/T), target p = softmax(z/T);
 * accept iff u*q(d) < p(d), else commit y ~ max(0, p - q) (normalised).
 * 0 < top_p < 1 (temperature > 0) restricts both q and p to their top-p sets and
 * renormalises: the smallest prefix of the tokens in order of decreasing
 * probability, lower id first on ties, whose mass reaches top_p (Holtzman et al.
 * 2019); drafts and the first token are drawn from that set. top_p >= 1 disables the
 * filter; top_p <= 0 or NaN is SPD_E_ARG. Random numbers are a pure function of (seed, stream, position,
 * index): SplitMix64 output function, u = ((x >> 41) + 0.5) * 2^-23.
 * forced_mode = 1 (temperature 0 only) replaces each draft at position x by
 * forced_ref[x - P0] with probability forced_p, else by (forced_ref[x - P0] + 1) mod V,
 * where P0 is the prompt length given to spd_prefill; positions past the end
 * of forced_ref keep the PDM's draft. forced_ref [host] holds ids in [0, V) (else
 * spd_init returns SPD_E_ARG); spd_init copies it, and spd_prefill uploads it.
 * If a rejection finds no token with p > q in floating point (the residual
 * max(0, p - q) has no mass), the committed token is the target's argmax and the
 * decision is flagged as a near-tie.
 * Draft trees (draft_width W > 1): at T = 0 the committed token is the target's argmax
 * and the accepted candidate is the one equal to it, if any. At T > 0 the candidates
 * c_0..c_{W-1} are tested in rank order by recursive rejection sampling: round i
 * proposes from q_i, q with c_0..c_{i-1} removed and renormalised, against r_i, where
 * r_0 = p and r_{i+1} = max(0, r_i - q_i) normalised; c_i is accepted iff
 * u_i q_i(c_i) < r_i(c_i) with u_i the stream-2 number of (v, i); if every round rejects,
 * y is drawn from r_W. A residual without mass ends the rounds as above.
 */
typedef struct {
  float temperature;
  float top_p;
  uint64_t seed;
  int32_t forced_mode;
  float forced_p;
  const int32_t* forced_ref;      /* [host] */
  int32_t forced_ref_len;
} spd_sampling;

/* Bytes of device workspace spd_init needs for this configuration (0 on invalid config). */
size_t spd_workspace_bytes(const spd_model_config* cfg);

/*
 * Validate the configuration, carve the caller's workspace, bind the weight
 * pointers, and precompute the RoPE table. hip_stream is a hipStream_t (NULL:
 * the null stream). The workspace must stay valid and unused by the caller
 * until spd_destroy. Errors: SPD_E_ARG (NULL pointers, bad sampling values, a
 * forced_ref id outside [0, V)), SPD_E_CONFIG, SPD_E_CAPACITY (ws_bytes too small),
 * SPD_E_DEVICE.
 */
int spd_init(const spd_model_config* cfg, const spd_weights* w, const spd_sampling* s,
             void* d_workspace, size_t ws_bytes, void* hip_stream, spd_handle** out);

/*
 * Run the target over the prompt [host, len token ids in [0, V), any length below
 * max_ctx: it is uploaded through the pinned staging in 512 KiB pieces] in chunks,
 * writing the target KV cache, the anchor states of every prompt position, the
 * PDM KV cache over the verified prefix (its depth-maximised features: all
 * anchors), and the first generated token (greedy, or sampled at T > 0).
 * Blocking. Afterwards the pipeline holds one token (position len, stage 0).
 * Errors: SPD_E_ARG (bad ids, len < 1), SPD_E_CAPACITY (len >= max_ctx),
 * SPD_E_STATE (already prefilled: call spd_reset first), SPD_E_DEVICE.
 */
int spd_prefill(spd_handle* h, const int32_t* prompt, int32_t len, int32_t* first_token);

/*
 * spd_prefill for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same prefill, with
 * the same arguments, results and errors, except that its chunk activation buffers live
 * in a 32 MiB array of the library's own device memory instead of the caller's workspace
 * (one array per GPU, held until the process ends), so the prompt is processed in chunks
 * of as many rows as the array holds (at most the regular 512). It calls no allocating
 * routine. Every call on a GPU shares that GPU's array, so calls on two handles of one GPU
 * that overlap in time race on it. Extra errors: SPD_E_CAPACITY when even 16 prompt rows
 * of this model do not fit the array; SPD_E_DEVICE when its address could not be obtained
 * at spd_init.
 */
int spd_prefill_static_scratch(spd_handle* h, const int32_t* prompt, int32_t len,
                               int32_t* first_token);

/*
 * Enqueue one pipeline step on the stream and return at once: embed the
 * stage-0 token; the PDM drafts the next token from the step's input states;
 * every in-flight token runs its stage's layers; if the oldest token leaves the
 * last stage, its logits verify the following position. Nothing is committed
 * until spd_verify_commit. Errors: SPD_E_STATE (a step is pending or no
 * prefill), SPD_E_CAPACITY (the newest position reached max_ctx), SPD_E_DEVICE.
 */
int spd_step(spd_handle* h);

/*
 * Lookahead (on != 0; off by default). A step in which no token leaves the last
 * stage (a refill step) verifies nothing, so the state of the step after it is
 * fixed when it is enqueued. With lookahead on, spd_step enqueues that following
 * step as well, right behind the pending one, so the GPU starts it as soon as the
 * pending one ends instead of waiting for the host's next spd_step; the next
 * spd_step then only takes it over. Results are bit for bit those of a run
 * without lookahead; the call order stays init -> prefill -> (step -> verify)*.
 * While a step runs ahead, the buffers that spd_debug_copy reads may already hold
 * its values, and spd_timing_enable returns SPD_E_STATE; lookahead is skipped
 * while timing is enabled. The review of the paper (pith.science, "What carries
 * the argument") describes the pipeline this keeps fed: one token enters stage 0
 * per step. Errors: SPD_E_ARG (NULL handle).
 */
int spd_lookahead(spd_handle* h, int on);

/*
 * Wait for the pending step (polling its end-of-step event; the verdict kernels
 * write their result to pinned host memory) and apply its verdict: on accept the ring shifts
 * and the draft enters stage 0; on reject every layer's KV length becomes the
 * verified position v, the pipeline is flushed and reseeded with the
 * corrected token at v. This is the only per-step device-to-host wait.
 *   verified: 1 if a token left the last stage this step (else a refill step)
 *   position: v, the position whose token was committed (verified == 1)
 *   token: the committed token y; accepted: 1 if y is the draft
 *   draft_token: the draft that stood at v before verification
 *   new_draft: the token drafted this step, for position newest + 1
 *   newest: position of this step's stage-0 token
 *   flags: bit 0 near-tie in the verify decision (top-2 gap < 1e-3, or
 *     |u q(d) - p(d)| < 1e-3 q(d)); bit 1 near-tie in the draft selection
 *   committed_total: N after this step; inflight: tokens in flight now
 *   accepted_index: rank of the accepted candidate at v (0: the spine; > 0 a sibling,
 *     with draft_width > 1), -1 when nothing was accepted or nothing verified
 */
typedef struct {
  int32_t verified, position, token, accepted, draft_token, flags;
  int32_t committed_total, inflight, new_draft, newest;
  int32_t accepted_index;
} spd_commit;
int spd_verify_commit(spd_handle* h, spd_commit* out);

/* Counters of Eq. (9): K steps, N committed tokens (the prefill's first token
 * excluded), alpha = N/K, s0 = alpha * n. */
typedef struct { int64_t K, N, accepted, rejected; double alpha, s0; } spd_stats;
int spd_get_stats(const spd_handle* h, spd_stats* out);

/* Current KV lengths: per_layer [host, L] for the target, *pdm_len for the
 * PDM's permanent rows (positions with full depth). Either may be NULL. */
int spd_get_kv_lens(const spd_handle* h, int32_t* per_layer, int32_t* pdm_len);

/* Copy one internal buffer to host memory for parity checks; bytes must equal
 * the buffer's size (spd_debug_size). Synchronises the stream. Not for the hot loop. */
enum {
  SPD_DBG_TARGET_LOGITS = 1,   /* f32 [V]: last target head output (prefill row or exit) */
  SPD_DBG_DRAFT_LOGITS = 2,    /* f32 [V]: last PDM head output (raw logits) */
  SPD_DBG_H_RING = 3,          /* f32 [n+1][W][d]: residual of position p's candidate b in
                                  row (p mod (n+1)) W + b (b = 0: the token) */
  SPD_DBG_ANCHORS = 4,         /* f32 [n+1][W][k][d]: anchors, rows as SPD_DBG_H_RING */
  SPD_DBG_PDM_ROWS = 5,        /* f32 [n+1][d]: PDM residual rows of the last step */
  SPD_DBG_TARGET_KV = 6,       /* KV dtype [softmax layers][2][hkv][max_ctx][hd] */
  SPD_DBG_PDM_KV = 7,          /* KV dtype [Ls][2][hkv][max_ctx][hd] */
  SPD_DBG_TOKENS = 8,          /* i32 [n+1][W]: candidate b of position p in row
                                  (p mod (n+1)) W + b */
  SPD_DBG_TOP_P = 9            /* [1 + (n+1)] x {f32 zb, i32 id_cut, f32 lse, i32 0}: top-p
                                  sets (top_p < 1, T > 0) of the last target row, then of the
                                  draft of position p in entry 1 + p mod (n+1); a set is the
                                  tokens with z > zb or z == zb and id <= id_cut, and lse is
                                  log sum over it of exp(z / T). Zero until computed. */
};
size_t spd_debug_size(const spd_handle* h, int32_t what);
int spd_debug_copy(const spd_handle* h, int32_t what, void* host_dst, size_t bytes);

/*
 * Measurement. When enabled, the first and last launch of every operation of a
 * step carry HIP start / stop events bound to their dispatch packets
 * (hipExtLaunchKernelGGL), on the stream the operation runs on, so a duration is
 * the kernels' own; spd_verify_commit accumulates per launch kind:
 * the number of launches, their total duration and their algorithmic HBM
 * bytes (weights read once, KV rows read once). Kinds, in order: 0 embed,
 * 1 PDM projection GEMV, 2 QKV GEMV, 3 attention, 4 linear attention, 5 O GEMV,
 * 6 gate/up GEMV, 7 down GEMV, 8 LM-head GEMV, 9 vocabulary stats, 10 verify,
 * 11 residual sample, then the PDM's own launches: 12 QKV GEMV, 13 attention,
 * 14 O GEMV, 15 gate/up GEMV, 16 down GEMV; 17 top-p sets (top_p < 1 only); 18 the PDM
 * feature gather after the target layers (SPD_SPEC_OUTPUT only).
 * Kinds 0-11 and 17 except 1 run on the
 * caller's stream; the PDM's run on a second, library-owned stream that forks
 * after the embedding and joins before the LM head, so their durations overlap.
 * Enabling or disabling clears the totals; a pending step gives SPD_E_STATE.
 * on = 2 also runs the PDM's launches on the caller's stream, one after another with
 * the target's, so that no launch shares the GPU with another (per-layer costs for
 * spd_timing_read_layers); 1 keeps the two streams.
 */
int spd_timing_enable(spd_handle* h, int on);
int spd_timing_read(const spd_handle* h, int32_t kind, int64_t* count, double* total_ms,
                    double* bytes);
/*
 * Per-layer time, for planning stages (pith.science review of the paper: the referee's
 * remarks on its Appendix C.1, non-uniform stage partitioning). While timing is enabled, the launches of a
 * sub-layer round that carries a single token (every round at n = 1; the first rounds
 * after a reseed at n > 1) serve one target layer alone; their durations add up per
 * layer. total_ms [host, L] receives each layer's total kernel time and passes [host, L]
 * the number of such single-token passes through it; the mean per pass is the cost of
 * one token through that layer, which is one pipeline stage's unit of work when each
 * stage has a GPU of its own. SPD_E_ARG for NULL arguments.
 */
int spd_timing_read_layers(const spd_handle* h, double* total_ms, int64_t* passes);

/*
 * Non-uniform stage partitioning (pith.science review of the paper: the referee's
 * remarks on its Appendix C.1, and on the compute imbalance of mixed attention layers
 * that its Section 6 admits). Splits n_layers layers, in order,
 * into n_stages contiguous stages of at least one layer each, minimising the largest
 * stage cost, where a stage's cost is the sum of layer_cost [host, n_layers] over its
 * layers, added in double from its first layer upward. Among the splits that reach that
 * minimum, it maximises the smallest stage cost; among those, the first stage takes as
 * many layers as it can, then the second, and so on (with equal costs this is the
 * default split: the first L mod n stages one layer larger). Writes stage_layers
 * [host, n_stages], suitable for spd_model_config's stage_layers. Host only; no device
 * or handle is needed. SPD_E_ARG for NULL pointers,
 * n_stages outside [1, n_layers], n_layers outside [1, 4096], or a cost that is
 * negative, infinite or NaN.
 */
int spd_balance_stages(int32_t n_layers, const float* layer_cost, int32_t n_stages,
                       int32_t* stage_layers);

/* Return to the post-init state (no prefill); device buffers are reused. */
int spd_reset(spd_handle* h);
/* Message of the last failed call on this handle ("" if none); valid until the next call. */
const char* spd_last_error(const spd_handle* h);
/* Message of the last spd_init failure (no handle exists then). */
const char* spd_init_error(void);
/* Release the handle and its pinned buffers; the caller's buffers are untouched. NULL is a no-op. */
void spd_destroy(spd_handle* h);

#ifdef __cplusplus
}
#endif
#endif /* SPD_H */
