/*
 * libspecverify -- the verify step of speculative / Chain-of-Draft decoding on
 * AMD Instinct MI355X (gfx950).
 *
 * One call verifies a batch of B requests.  Request b drafted gamma_b tokens;
 * the caller supplies the target model's logits for the gamma_b + 1 positions
 * behind the draft, the draft model's logits for the gamma_b drafted positions,
 * the drafted token ids and host-drawn uniforms.  The call returns, per
 * request, the accepted prefix of the draft followed by one more token.
 *
 * Modes (what each computes is defined by the passages cited):
 *
 *   SV_MODE_STOCHASTIC  Modified rejection sampling -- "大模型推理的投机采样"
 *       page, section "核心算法数学原理": with p = softmax(target_i / T) and
 *       q = softmax(draft_i / T), draft token x_i is accepted when
 *       u_accept_i <= alpha_i = min(1, p(x_i) / q(x_i)); at the first rejection
 *       j the slot is redrawn from max(0, p_j - q_j) / norm and the remaining
 *       drafts are discarded.  When all gamma_b drafts are accepted a bonus
 *       token is drawn from p_gamma (target row gamma_b).  Each request uses
 *       one uniform u_resample[b] for its terminal draw, by inverse CDF in
 *       ascending token order: y* = min{y : C_y > u * C_{V-1}}.
 *   SV_MODE_GREEDY      Greedy verification -- Gemma-4 MTP drafter page,
 *       section 2.3: x_i is accepted while it equals argmax(target_i) (lowest
 *       index on ties); the first mismatching slot (or slot gamma_b) gets the
 *       target row's argmax.
 *   SV_MODE_NKL         Normalised-KL filter -- "Chain of Draft" page, section
 *       3.2: nkl_i = KL(q_i || p_i) / ln V at the request's temperature; x_i is
 *       accepted while nkl_i < delta; the first failing slot (or slot gamma_b)
 *       gets argmax(target row).
 *   SV_MODE_BLOCK       Block accept -- "Chain of Draft" page, section 3.3
 *       (Block-Accept Mode) and section 2.2 (block mode: runs of >= 3 agreeing
 *       tokens): position i agrees when x_i == argmax(target_i) (lowest index
 *       on ties).  The first longest run of consecutive agreeing positions, if
 *       it has at least cfg->block_min_len positions and ends at e, keeps the
 *       drafted tokens x_0..x_{e-1} (those before the run too) and slot e gets
 *       argmax(target_e); with no such run slot 0 gets argmax(target_0) and
 *       nothing is accepted.  (The page's strict token-by-token policy is
 *       SV_MODE_GREEDY.)
 *   SV_MODE_TREE_GREEDY Greedy tree verification -- "Parallel Drafting" page,
 *       section 2.2 (tree drafts), Gemma-4 MTP page, section 6.2 (keep the
 *       longest accepted path): node n with parent pi(n) is accepted iff pi(n)
 *       is accepted and its token equals argmax(target row of pi(n)); the
 *       output is the path to the deepest accepted node (lowest node id on
 *       equal depth) followed by that node's argmax.
 *
 * Packed (ragged) layout.  t_off[b] = sum_{b'<b}(gamma_b' + 1),
 * d_off[b] = sum_{b'<b} gamma_b'.  Target row t_off[b] + i holds position i of
 * request b (i = 0..gamma_b); draft row d_off[b] + i holds drafted position i
 * (i = 0..gamma_b - 1).  Tree mode: request b is a tree of N_b = gamma_b + 1
 * nodes, node 0 the root; target row t_off[b] + n belongs to node n;
 * draft_tokens[d_off[b] + n - 1] and tree_parents[d_off[b] + n - 1] are node
 * n's token and parent (0 <= parent < n).
 *
 * Memory.  Every array argument is DEVICE memory, row-major and packed.  The
 * caller owns all buffers (including the workspace); the library allocates
 * nothing and only enqueues work on cfg->stream.  Outputs are valid once that
 * stream has been synchronised.  Calls on different streams must use
 * different workspaces.  Host-side state is limited to cached device
 * attributes (compute-unit counts, kernel occupancies) and a call counter
 * whose values ("epochs", never 0 or 0xFFFFFFFF) tag what a call leaves in
 * its workspace.
 *
 * Workspace.  Its contents need no initialisation and need not be preserved
 * between calls: a call reads only what the same call wrote, apart from the
 * per-request arrival counters, which it first claims for itself (a word that
 * carries another call's epoch, or any other bytes, is replaced).  One
 * workspace may serve successive calls of any entry point and any
 * configuration on one stream, as long as it is large enough for each.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPECVERIFY_VERSION 10300 /* 1.3.0: consensus across drafts (spec_consensus) */

/* status codes */
#define SV_OK 0
#define SV_EINVAL (-1)       /* bad argument (returned before any work is enqueued) */
#define SV_EUNSUPPORTED (-2) /* valid but unsupported request (e.g. max_gamma above SV_MAX_GAMMA) */
#define SV_EWORKSPACE (-3)   /* workspace missing or smaller than spec_verify_workspace_size() */
#define SV_EHIP (-4)         /* a HIP launch failed; spec_verify_status_string(SV_EHIP) names it */

/* modes */
#define SV_MODE_STOCHASTIC 0
#define SV_MODE_GREEDY 1
#define SV_MODE_NKL 2
#define SV_MODE_TREE_GREEDY 3
#define SV_MODE_BLOCK 4

/* logit element types */
#define SV_DTYPE_F32 0
#define SV_DTYPE_BF16 1

#define SV_MAX_GAMMA 4096 /* largest accepted cfg->max_gamma (tree: nodes - 1) */

/* Phase events (optional, for timing): cfg->phase_events points to
 * SV_NUM_PHASE_EVENTS hipEvent_t handles created by the caller, all on
 * cfg->stream: [0] is recorded before the first kernel and [3] after the last;
 * [1] and [2] take the start and end timestamps of the row-statistics
 * dispatch itself (the streaming pass over the logits). */
#define SV_NUM_PHASE_EVENTS 4

typedef struct sv_config {
  uint32_t struct_size;     /* = sizeof(sv_config); other values are rejected */
  int32_t batch;            /* B > 0 */
  int32_t vocab;            /* V > 0 */
  int32_t dtype;            /* SV_DTYPE_F32 or SV_DTYPE_BF16 (both logit arrays) */
  int32_t max_gamma;        /* bound on gamma_per_req[b]; 0 <= max_gamma <= SV_MAX_GAMMA */
  int32_t wait_polls;       /* >= 0; 0 = default.  How often a helper of the single dispatch
                               polls for a statistics partial that another workgroup of the same
                               dispatch writes before it computes that partial itself (results
                               do not depend on it) */
  int64_t total_draft_rows; /* sum_b gamma_per_req[b], known on the host (sizes the grids) */
  void* stream;             /* hipStream_t to enqueue on; NULL = the default stream */
  void* workspace;          /* device scratch, >= spec_verify_workspace_size(cfg) bytes, 256-byte aligned;
                               contents need no initialisation (see "Workspace" above) */
  uint64_t workspace_bytes;
  /* optional diagnostics (device pointers, NULL = not written) */
  float* out_p_x;           /* [total_draft_rows] p_i(x_i) (stochastic and NKL modes) */
  float* out_q_x;           /* [total_draft_rows] q_i(x_i) (stochastic and NKL modes) */
  float* out_resid_mass;    /* [B] stochastic: sum_y max(0, p_j - q_j) after a rejection, 1 for a bonus */
  int32_t* out_tree_node;   /* [B] tree mode: id of the deepest accepted node */
  void* phase_events;       /* optional hipEvent_t[SV_NUM_PHASE_EVENTS] (see above) */
  /* NKL mode, optional: position-adaptive threshold ("Chain of Draft" page, section 4.3).
   * nkl_position: device int32 [total_draft_rows], the 0-based position of each draft token
   * in the generated sequence (NULL = the constant threshold delta for every token).  Token i
   * is then accepted while nkl_i < min(nkl_delta_max, delta * (1 + nkl_alpha * log2(pos_i + 1))),
   * evaluated in float64.  nkl_alpha and nkl_delta_max must be finite when nkl_position is set;
   * a negative position is a data error of its request. */
  const int32_t* nkl_position;
  float nkl_alpha;
  float nkl_delta_max;
  /* block-accept mode: the shortest run of agreeing positions that is kept (>= 0; 0 = 3, the
   * page's min_block_len) */
  int32_t block_min_len;
} sv_config;

/*
 * Verifies one batch.
 *
 * target_logits  [sum(gamma+1)][V] of cfg->dtype (bf16 = IEEE bfloat16 bit patterns).
 * draft_logits   [sum(gamma)][V]; read in stochastic and NKL modes only (may be NULL otherwise;
 *                greedy, block and tree modes read target rows only).
 * draft_tokens   int32 [sum(gamma)]; must lie in [0, V).
 * gamma_per_req  int32 [B]; 0 <= gamma_b <= cfg->max_gamma.
 * temperature    float32 [B]; > 0 and finite (stochastic and NKL modes; may be NULL otherwise).
 * u_accept       float32 [sum(gamma)] in [0, 1) (stochastic mode; may be NULL otherwise).
 * u_resample     float32 [B] in [0, 1) (stochastic mode; may be NULL otherwise).
 * mode           SV_MODE_*.
 * delta          NKL threshold (NKL mode; must be finite there).
 * tree_parents   int32 [sum(gamma)] (tree mode; may be NULL otherwise).
 * out_tokens     int32 [sum(gamma+1)], same offsets as the target rows: accepted tokens, then the
 *                terminal token, then -1 in the unused slots.
 * out_num_accepted int32 [B]: number of accepted draft tokens (tree: depth of the deepest accepted node;
 *                block: the kept prefix e).
 * out_nkl        float32 [sum(gamma)]: nkl_i for every drafted position (required in NKL mode;
 *                in stochastic mode written when non-NULL).
 * cfg            see sv_config.
 *
 * Synchronous errors (nothing enqueued): SV_EINVAL for a NULL pointer the mode needs, B <= 0,
 * V <= 0, an unknown mode or dtype, a non-finite delta in NKL mode, a struct_size mismatch,
 * total_draft_rows outside [0, B*max_gamma], or misaligned pointers (logits: element size;
 * int32/float32 arrays: 4 bytes); SV_EUNSUPPORTED for max_gamma > SV_MAX_GAMMA or more than
 * 2^31-1 rows; SV_EWORKSPACE; SV_EHIP.
 * Data errors (found on the device, no host sync): a request with a token outside [0, V), a
 * gamma_b above max_gamma, a temperature <= 0 or non-finite, a uniform outside [0, 1) or a bad
 * parent gets out_num_accepted[b] = -1 and -1 in all its token slots; other requests are not
 * affected.  A negative gamma_b, or sum(gamma) != total_draft_rows, makes the packed layout
 * undefined: every out_num_accepted[b] is set to -1 and no token slot is written.
 * Logits are expected to be finite.
 */
int spec_verify(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                const int32_t* gamma_per_req, const float* temperature, const float* u_accept,
                const float* u_resample, int32_t mode, float delta, const int32_t* tree_parents,
                int32_t* out_tokens, int32_t* out_num_accepted, float* out_nkl, const sv_config* cfg);

/* Workspace bytes spec_verify needs for this configuration (any mode); 0 for an invalid cfg.
 * Reads batch, vocab, dtype, max_gamma and total_draft_rows only.  The workspace holds
 * per-chunk partial results, arrival counters and per-request records; it needs no
 * initialisation and may be reused by successive calls on the same stream (see
 * "Workspace" above).  spec_sample_rows and spec_topk_rows need the size for batch =
 * rows and total_draft_rows = 0. */
size_t spec_verify_workspace_size(const sv_config* cfg);

/* Static description of a status code.  For SV_EHIP it includes the HIP error of the
 * most recent failed launch on the calling thread. */
const char* spec_verify_status_string(int status);

/* SPECVERIFY_VERSION of the loaded library. */
int spec_verify_version(void);

/* 1 if spec_verify would run this configuration as one kernel dispatch (batch
 * <= 1024 and a short statistics pass, in the stochastic mode with out_nkl ==
 * NULL (with_nkl == 0), the greedy mode, or the tree and block modes with
 * max_gamma <= 256; never in the NKL mode), 0 if as separate kernels,
 * SV_EINVAL for an invalid cfg or mode.  Reads batch, vocab, dtype, max_gamma,
 * total_draft_rows and the device's compute-unit count (the current device);
 * enqueues nothing.  For timing and
 * profiling tools: phase_events [1] and [2] bracket that single dispatch, or
 * else the row-statistics dispatch. */
int spec_verify_single_dispatch(const sv_config* cfg, int32_t mode, int32_t with_nkl);

/*
 * spec_verify without a caller-provided workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The arguments and results are those of spec_verify; cfg->workspace and cfg->workspace_bytes
 * are ignored.  The scratch is a fixed array of SV_NOALLOC_SCRATCH_BYTES in the library's own
 * device memory, one copy per GPU, held until the process ends; its device address is looked
 * up once per device on the first call (the current device, which must own cfg->stream).  The
 * call allocates nothing.  A configuration whose spec_verify_workspace_size() exceeds
 * SV_NOALLOC_SCRATCH_BYTES returns SV_EWORKSPACE before anything is enqueued.  Every call on a
 * GPU shares that GPU's array: calls that overlap on one GPU (two streams, or two threads) race
 * and give undefined results; successive calls on one stream are fine.  Nothing in the array
 * must start at a particular value (see "Workspace" above), so it is never cleared.
 */
#define SV_NOALLOC_SCRATCH_BYTES (16u << 20)
int spec_verify_noalloc(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                        const int32_t* gamma_per_req, const float* temperature, const float* u_accept,
                        const float* u_resample, int32_t mode, float delta, const int32_t* tree_parents,
                        int32_t* out_tokens, int32_t* out_num_accepted, float* out_nkl, const sv_config* cfg);

/*
 * Draft-side sampling, the drafter's step before verification: one token per row, drawn from
 * softmax(logits_r / temperature[r]) by the inverse CDF with the uniform u[r],
 *     y_r = min{ y : C_y > u_r * S }   (C_y: cumulative mass in ascending token order, S: total),
 * the same rule as the verify step's bonus draw (draft tokens "drawn from the draft softmax";
 * the "投机采样" page's draft loop draws x_i ~ q_i).
 *
 * logits       [cfg->batch][cfg->vocab] of cfg->dtype, device, row-major (cfg->batch = rows).
 * temperature  float32 [rows], > 0 and finite.
 * u            float32 [rows] in [0, 1).
 * out_tokens   int32 [rows]: the drawn token, or -1 for a row whose temperature or uniform is
 *              invalid (a data error, found on the device; other rows are not affected).
 * cfg          batch, vocab, dtype, stream, workspace (>= spec_verify_workspace_size(cfg) with
 *              total_draft_rows = 0; no initialisation needed) and phase_events ([1] and [2]
 *              bracket the sampling dispatch).  The other fields are not read.
 * Synchronous errors: SV_EINVAL (NULL or misaligned pointer, B <= 0, V <= 0, bad dtype or
 * struct_size), SV_EUNSUPPORTED (grid above 2^31 - 1), SV_EWORKSPACE, SV_EHIP.
 * Asynchronous on cfg->stream, like spec_verify.
 */
int spec_sample_rows(const void* logits, const float* temperature, const float* u, int32_t* out_tokens,
                     const sv_config* cfg);

/*
 * Top-k of each row, for the children of a tree-draft node (the node's k children are the top-k
 * tokens of its draft row: "Parallel Drafting" page, section 2.2 tree draft): the k indices with
 * the largest logits, largest first, the lower index first among equal logits (-0 == +0).
 *
 * logits   [cfg->batch][cfg->vocab] of cfg->dtype, device, row-major (cfg->batch = rows);
 *          finite values.
 * k        1 <= k <= min(16, vocab).
 * out_idx  int32 [rows][k].
 * cfg      as for spec_sample_rows (batch, vocab, dtype, stream, workspace, phase_events).
 * Synchronous errors: SV_EINVAL (NULL or misaligned pointer, B <= 0, V <= 0, bad dtype or
 * struct_size, k out of range), SV_EUNSUPPORTED, SV_EWORKSPACE, SV_EHIP.
 */
int spec_topk_rows(const void* logits, int32_t k, int32_t* out_idx, const sv_config* cfg);

/*
 * Consensus across several drafts ("Chain of Draft" page, section 4.4, Consensus-Aware Accept:
 * the pairwise NKL distance matrix of the drafts; a pair below 0.1 is a consensus, every pair
 * above 0.15 a divergence).  Request b has gamma_b positions; each position holds num_drafts
 * draft rows (one per draft model), all at the request's temperature.  Per position:
 *     M[a][b] = KL(q_a || q_b) / ln V    (q_a = softmax(row a / T); 0 when V == 1),
 *     distance of a pair a < b = (M[a][b] + M[b][a]) / 2,
 *     pair  = a * num_drafts + b of the closest pair (lowest (a, b) on ties),
 *     state = 1 (consensus) if that distance < delta_c, 2 (divergence) if it is > delta_d (so
 *             every pair is), else 0.
 * One read of the rows gives each KL value with an error estimate; positions where an estimate
 * exceeds 1e-5 of its value, or where a threshold or a near tie of the closest pair lies within
 * the estimates, are recomputed in the exact form (sum_y q_a (e^w - 1 - w), w = ln(q_b / q_a),
 * no cancellation) by a second read of their rows.
 *
 * draft_logits [total_draft_rows][num_drafts][V] of cfg->dtype: the drafts of one position are
 *              consecutive rows (position n, draft a: row n * num_drafts + a).
 * num_drafts   2 .. 4.
 * gamma_per_req int32 [B] (positions per request), temperature float32 [B].
 * out_nkl      float32 [total_draft_rows][num_drafts][num_drafts] (may be NULL).
 * out_state, out_pair int32 [total_draft_rows].
 * cfg          batch, vocab, dtype, max_gamma, total_draft_rows (= sum of gamma), stream,
 *              workspace (>= spec_consensus_workspace_size(cfg, num_drafts); no initialisation
 *              needed), phase_events ([1] and [2] take the start and end of the pass over
 *              all the rows).
 * Data errors: a request whose temperature is not > 0 and finite gets state -1, pair -1 and
 * NaN in out_nkl at its positions; a negative gamma or sum(gamma) != total_draft_rows gives -1
 * everywhere.  Synchronous errors: SV_EINVAL (NULL or misaligned pointer, bad cfg, num_drafts
 * out of range, non-finite threshold), SV_EUNSUPPORTED, SV_EWORKSPACE, SV_EHIP.
 */
int spec_consensus(const void* draft_logits, int32_t num_drafts, const int32_t* gamma_per_req,
                   const float* temperature, float delta_c, float delta_d, float* out_nkl, int32_t* out_state,
                   int32_t* out_pair, const sv_config* cfg);

/* Workspace bytes of spec_consensus (0 for an invalid cfg or num_drafts). */
size_t spec_consensus_workspace_size(const sv_config* cfg, int32_t num_drafts);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
