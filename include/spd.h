/*
 * spd.h -- C ABI of libspd: one speculative-pipeline-decoding (SPD) engine on
 * one MI355X (gfx950).
 *
 * Citation tags (section names are those on each page):
 *   [RB] paper.rainbus.top summary of arXiv 2605.30852 "Speculative Pipeline
 *        Decoding: Higher-Accuracy and Zero-Bubble Speculation via Pipeline
 *        Parallelism" -- sections "core method", "method steps" (1-6).
 *   [TW] techwalker.com article on the same paper -- sections 3-6, 8.
 *   [PL] paperlayer.ai summary of arXiv 2605.30852v3 "Speculative Pipeline
 *        Decoding: Higher-Accuracy Drafting with Hidden Latency via Pipeline
 *        Parallelism" -- sections 3.1-3.4, A.1-A.3.
 *   [YB] ybb.press speculative-decoding blog -- sections 2.1-2.2.
 *
 * What the engine computes.  The L-layer target decoder is split into n
 * stages of L/n layers ([RB] core method).  Up to n tokens of ONE sequence
 * are in flight at depths 0..n-1; every cycle each of them advances through
 * its own stage -- on one GPU the n stages run as one stage-grouped batched
 * decode ([RB] method step 1, [PL] 3.1).  Concurrently, on a second stream,
 * the pipeline draft module (PDM) builds the depth-staircase feature sequence
 * from anchor hidden states (f(k) = max{i : b_i <= lmax(k)}, lmax(k) =
 * min(L, k L/n), [RB] core method, [PL] 3.2), runs Ls <= L/n causal decoder
 * layers and an LM head, and predicts the one next token from the pre-step
 * state ([RB] method step 4, [PL] 3.3).  The token leaving the last stage
 * verifies its successor ([RB] method step 5, [TW] 6); a rejection truncates
 * every layer's KV cache, flushes the in-flight states and re-seeds stage 0
 * with the corrected token (the three-step rollback, [RB] method step 5,
 * [PL] 3.4).  The emitted sequence equals the target's greedy decoding
 * (greedy mode) or is distributed as its temperature sampling (sample mode,
 * rejection rule of [YB] 2.1).
 *
 * Conventions.  All calls return SPD_OK (0) or a negative SPD_E* code;
 * nothing throws across the ABI.  Positions are 0-indexed; token ids int32;
 * greedy ties resolve to the lowest id.  A handle is used by one host thread
 * at a time.  Device pointers are HIP device memory on the current device;
 * "stream" arguments are hipStream_t values passed as void*.  The library
 * never allocates device memory: the caller owns every device buffer
 * (weights, workspace, policy arrays) and both streams, all of which must
 * outlive the handle.  The handle itself is host memory owned by the library.
 */
#ifndef SPD_H
#define SPD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* entry points are the library's only exported symbols */
#if defined(__GNUC__) || defined(__clang__)
#define SPD_API __attribute__((visibility("default")))
#else
#define SPD_API
#endif

#define SPD_MAX_LAYERS 64
#define SPD_MAX_PDM_LAYERS 8
#define SPD_MAX_ANCHORS 8
#define SPD_MAX_STAGES 16
#define SPD_MAX_VOCAB (1 << 20)
#define SPD_MAX_TOPK 64
#define SPD_MAX_WIDTH 4

/* return codes */
#define SPD_OK 0
#define SPD_EINVAL (-1)  /* invalid argument or configuration */
#define SPD_ESTATE (-2)  /* call not valid in the engine's current state */
#define SPD_ECTX (-3)    /* sequence would exceed max_ctx */
#define SPD_EHIP (-4)    /* a HIP runtime call failed (see spd_sync status) */
#define SPD_EDEVICE (-5) /* a device-side invariant check failed */
#define SPD_ESCRATCH (-6) /* the configuration needs more scratch than the static scratch array holds */

/* storage types of weights and KV cache */
#define SPD_DTYPE_F32 0
#define SPD_DTYPE_BF16 1

/* verification mode */
#define SPD_MODE_GREEDY 0 /* accept iff draft == argmax ([TW] 6) */
#define SPD_MODE_SAMPLE 1 /* accept w.p. min(1, P/Q), else redraw from max(0,P-Q) ([YB] 2.1) */

/* Draft-module schedule ([PL] §3.3; the scheduling ablation of [PL] §4).
 * PRE: the draft module reads the features of the trailing positions as they
 *   stand before this cycle's stage step (the just-verified position at depth
 *   n, in-flight tokens at depths a-1..0) and runs concurrently with it.
 * POST: it reads them after the stage step (in-flight tokens at depths a..1;
 *   an exiting token at depth n, whose draft-module key/values are committed
 *   in the same cycle) and therefore runs after the stage step and the
 *   verification, on the stage stream: drafting is serial again.  The tokens
 *   entering the pipeline follow the same rules in both schedules. */
#define SPD_SCHED_PRE 0
#define SPD_SCHED_POST 1

/* draft policy */
#define SPD_DRAFT_NATURAL 0 /* the PDM's own prediction */
#define SPD_DRAFT_FORCED 1  /* seeded forced acceptance (test harness device, greedy only) */

/* columns of the per-position uniform table */
#define SPD_U_TARGET 0
#define SPD_U_DRAFT 1
#define SPD_U_ACCEPT 2
#define SPD_U_RESAMPLE 3
#define SPD_U_FORCE 4
#define SPD_U_COUNT 5

/* device-side check flags (spd_status.flags, spd_cycle_rec.flags) */
#define SPD_FLAG_KVLEN 1u     /* a KV append found len != position */
#define SPD_FLAG_OCCUPANCY 2u /* occupancy left 1..n */
#define SPD_FLAG_CTX 4u       /* a position reached max_ctx */
#define SPD_FLAG_IDLE 8u      /* record of a cycle enqueued after generation ended */
#define SPD_FLAG_NODRAFT 16u  /* the verified successor had no draft */
#define SPD_FLAG_BADTOKEN 32u /* an argmax / draw found no valid id (non-finite logits); id 0 used */

/*
 * Model and engine shape.  The target layer is pre-norm: RMSNorm (gain
 * attn_norm), q/k/v projection, rotate-half RoPE (theta_i = rope_base^(-2i/hd)),
 * grouped-query attention over the layer's KV cache, output projection +
 * residual, RMSNorm (ffn_norm), SwiGLU (silu(gate) * up), down projection +
 * residual; no biases.  The PDM layers have the same shape with their own
 * weights.  Constraints checked by spd_init ([RB] core method): n_stages
 * divides n_layers and is at most SPD_MAX_STAGES (the draft module batches
 * up to n_stages + 1 rows); pdm_layers <= n_layers / n_stages (for a
 * non-uniform split see stage_layers); anchors strictly
 * increasing with anchors[0] == 0 and anchors[n_anchors-1] <= n_layers;
 * n_heads % n_kv_heads == 0; head_dim in {64, 128}; d_model, d_ffn and
 * n_heads*head_dim multiples of 256; max_ctx <= 32768; 2 <= vocab <=
 * SPD_MAX_VOCAB; schedule one of SPD_SCHED_* (SPD_SCHED_POST needs n_stages >= 2);
 * 0 <= top_k <= min(SPD_MAX_TOPK, vocab).  With n_stages = 1 every token exits in
 * the cycle it enters and verifies the draft made in that cycle: the draft
 * module then runs ahead of the stage step on the stage stream.
 */
typedef struct spd_config {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ffn, vocab;
  int32_t n_stages;   /* n */
  int32_t pdm_layers; /* Ls */
  int32_t n_anchors;  /* m */
  int32_t anchors[SPD_MAX_ANCHORS]; /* b_i: anchor i = residual after b_i layers (b_0 = 0: embedding) */
  int32_t dtype;      /* SPD_DTYPE_*: matrices and KV cache; norm gains are always fp32 */
  int32_t max_ctx;    /* KV capacity in positions; must cover prompt + max_new + n_stages */
  int32_t max_new;    /* G: generation stops once G tokens are emitted (the first from prefill) */
  int32_t mode;       /* SPD_MODE_* */
  float rms_eps;      /* RMSNorm epsilon */
  float rope_base;    /* RoPE base */
  float temperature;  /* sample mode only */
  int32_t schedule;   /* SPD_SCHED_* */
  int32_t attn_period; /* hybrid target ([RB] limitations, [TW] §11: one standard and three
                          linear-attention layers per block of four): layer l uses softmax
                          attention iff attn_period == 0 or l % attn_period == attn_period - 1,
                          else causal linear attention with feature map elu + 1 over the same
                          q/k/v (o = phi(q)^T S / phi(q)^T z, S = sum phi(k) v^T, z = sum phi(k),
                          per kv head, fp32 state).  0 <= attn_period <= n_layers.  With linear
                          layers spd_rollback accepts only lengths whose state is still held:
                          the last n_stages + 1 positions, or the prefill length. */
  int32_t top_k;      /* sample mode: only the top_k largest logits keep their weight, in the
                         target's P and the draft module's Q alike (equal logits rank by the lower
                         id; selection before the temperature); 0 = the whole vocabulary.
                         0 <= top_k <= min(SPD_MAX_TOPK, vocab).  [RB] reproducibility assessment:
                         the evaluation decodes with top-k 50, top-p 1.0 (no nucleus cut). */
  int32_t stage_layers[SPD_MAX_STAGES]; /* non-uniform split ([RB] limitations and future
                         work: splits such as "5+4;9;9;9" -- a 5-layer first stage beside the
                         4-layer draft module, then three 9-layer stages -- to fit 4- or
                         8-GPU nodes): stage k runs the next stage_layers[k] layers, so a token
                         at depth k has run stage_layers[0] + ... + stage_layers[k-1] layers,
                         which takes the place of k * n_layers / n_stages in the anchor
                         patterns.  All zero: the uniform split.  Otherwise entries
                         0..n_stages-1 are >= 1 and sum to n_layers, the rest are 0, and
                         pdm_layers is at most the longest stage (the cycle lasts as long as
                         its longest stage). */
  int32_t draft_width; /* draft tree ([RB] prerequisites "draft tree": keep the top-W branches by
                         cumulative probability; [PL] appendix B widens each SPD draft step into a
                         width-4 tree).  0 or 1: one draft per cycle (a chain).  W in 2..
                         SPD_MAX_WIDTH: the tokens in flight form a tree of at most W nodes per
                         position (one at the oldest); every cycle the draft module runs on
                         every node's pre-step features (each row attending to its own
                         ancestors), scores each pair (leaf, token) among the leaves' W most
                         likely tokens by cum(leaf) + log Q_leaf(token) -- cum summing log Q
                         along the leaf's in-flight path -- and the next cycle enters the best W
                         whose leaf survived verification; the exiting node keeps the child that
                         matches the target's argmax and prunes the others, and the three-step
                         rollback runs only when no child matches.  Each leaf owns a KV lane (a
                         full cache copy): a node's key/values go to its descendants' lanes, so
                         every node attends to committed prefix + ancestors + itself.  Needs
                         greedy mode, the pre-step schedule, 2 <= n_stages, attn_period = 0,
                         uniform stages, and 2 + (n_stages - 1) * W <= 32 draft rows. */
} spd_config;

/* Device pointers of one decoder layer.  Row-major, output features first:
 * w_qkv [(Hq+2Hkv)*hd, d] (q rows, then k rows, then v rows); w_o [d, Hq*hd];
 * w_gu [2F, d] (gate rows 0..F-1, up rows F..2F-1); w_down [d, F];
 * attn_norm, ffn_norm [d] fp32.  Matrices are in config.dtype. */
typedef struct spd_layer_weights {
  const void *attn_norm, *w_qkv, *w_o, *ffn_norm, *w_gu, *w_down;
} spd_layer_weights;

/* embed [V, d]; final_norm [d] fp32; lm_head [V, d]; fc[f] [d, (f+1)*d] maps
 * the concatenation of anchors 0..f (in anchor order) to a PDM feature;
 * pdm[] the PDM layers; pdm_final_norm [d] fp32; pdm_lm_head [V, d]. */
typedef struct spd_weights {
  const void *embed;
  spd_layer_weights layers[SPD_MAX_LAYERS];
  const void *final_norm, *lm_head;
  const void *fc[SPD_MAX_ANCHORS];
  spd_layer_weights pdm[SPD_MAX_PDM_LAYERS];
  const void *pdm_final_norm, *pdm_lm_head;
} spd_weights;

/* One record per enqueued cycle, written on the device and copied to the
 * caller's host buffer by spd_cycle.  kv_len[] holds every target layer's KV
 * length after the cycle (after any rollback truncation); with a draft tree,
 * the committed length (the tree's in-flight key/values live in its lanes),
 * the same in every layer.  With a draft tree, draft / pdm_argmax are the
 * best-ranked candidate's token and the draft module's top token of the
 * rank-0 leaf. */
typedef struct spd_cycle_rec {
  int32_t cycle;        /* engine cycle index */
  int32_t t;            /* position of the newest in-flight token (this cycle's seed) */
  int32_t occupancy;    /* a: tokens in flight after entry (1..n) */
  int32_t pending_row;  /* 1 if the just-verified position's full-depth feature was cached this cycle */
  int32_t pdm_argmax;   /* PDM prediction for position t+1 (argmax, or sampled draw) */
  int32_t draft;        /* draft for position t+1 after the draft policy */
  int32_t exit_pos;     /* position j that left the pipeline, or -1 */
  int32_t target_token; /* token emitted at j+1 (argmax or sampled), or -1 */
  int32_t accepted;     /* 1 accepted, 0 rejected (rollback), -1 no exit */
  int32_t pdm_len;      /* PDM committed length after the cycle */
  int32_t emitted;      /* tokens emitted so far (including the prefill token) */
  uint32_t flags;       /* SPD_FLAG_* */
  int32_t kv_len[SPD_MAX_LAYERS];
  /* draft tree (draft_width >= 2; a chain fills the first entries): */
  int32_t nodes;        /* nodes in flight after entry */
  int32_t n_new;        /* nodes that entered this cycle (at position t), in rank order: */
  int32_t new_parent[SPD_MAX_WIDTH]; /* rank of each one's parent at t-1 (-1: re-seeded) */
  int32_t new_token[SPD_MAX_WIDTH];
  int32_t accepted_rank; /* rank of the kept child at exit_pos+1, or -1 */
} spd_cycle_rec;

typedef struct spd_status {
  int32_t cycles;     /* cycles executed on the device */
  int32_t emitted;    /* tokens emitted (including the prefill token) */
  int32_t done;       /* 1 once emitted == max_new */
  int32_t t;          /* newest position of the last executed cycle */
  int32_t occupancy;  /* occupancy of the last executed cycle */
  int32_t pdm_len;    /* PDM committed length */
  uint32_t flags;     /* accumulated SPD_FLAG_* bits */
  int32_t hip_error;  /* last hipError_t seen by the handle (0 = none) */
} spd_status;

typedef struct spd_handle spd_t;

/* Bytes of device workspace spd_init needs for `cfg` (KV caches of target
 * and PDM, in-flight slots, anchor store, scratch, logits, rings, control
 * block, cycle-record ring and, for bf16 models, a copy of the draft module's
 * layer matrices in matrix-core tile order: Ls * 2 * ((Hq + 2 Hkv) hd d +
 * Hq hd d + 3 F d) bytes).  Pure host computation.  SPD_EINVAL if the
 * configuration is invalid. */
SPD_API int spd_workspace_bytes(const spd_config *cfg, size_t *bytes);

/* Validate `cfg`, record the weight pointers, carve `workspace` (device
 * memory of at least spd_workspace_bytes, 256-byte aligned) and build the
 * anchor-pattern and RoPE tables on the device.  For bf16 models the draft
 * module's layer matrices (w_qkv, w_o, w_gu, w_down of every pdm layer) are
 * copied into the workspace in matrix-core tile order: the cycles read that
 * copy, so later changes to those caller buffers take effect only through a
 * new spd_init; every other weight is read from the caller's buffers, which
 * must stay valid until spd_destroy.  stage_stream carries the
 * target stage step and verification; pdm_stream the draft module.  The
 * streams must be distinct and of default priority.  On success *out holds
 * the handle.  Errors: SPD_EINVAL (constraints above, null pointers,
 * streams equal), SPD_EHIP. */
SPD_API int spd_init(const spd_config *cfg, const spd_weights *w, void *workspace, size_t ws_bytes,
             void *stage_stream, void *pdm_stream, spd_t **out);

/* Allocation-free variant of spd_init, for callers that cannot allocate
 * device memory around their decode calls (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The engine's
 * per-cycle scratch (activation rows, attention and split-K partials,
 * logits, argmax and sampling partials: everything spd_init carves after the
 * persistent state) lives in a static device array of SPD_STATIC_SCRATCH_MB
 * MiB that the library holds on every GPU it runs on until the process ends;
 * the caller passes only the persistent state (KV caches, control block,
 * rings, tables, in-flight slots) in `state`.
 *   state == NULL: size query -- *state_bytes receives the state size (pure
 *     host computation; the other pointers may be NULL).
 *   state != NULL: *state_bytes is the size of `state` (device memory,
 *     256-byte aligned, at least the queried size); otherwise as spd_init.
 * Calls no hipMalloc / hipFree and allocates nothing on the device.  Every
 * handle made by this call on one GPU shares that GPU's array, which keeps
 * the last user's contents (this call clears it): work of two such handles
 * that overlaps on one GPU races, so the caller must order it (one stream
 * pair at a time).  Handles from spd_init are unaffected.  Errors:
 * SPD_ESCRATCH (the configuration's scratch exceeds the array), SPD_EINVAL
 * (as spd_init, or state_bytes too small), SPD_EHIP. */
#define SPD_STATIC_SCRATCH_MB 64
SPD_API int spd_init_static_scratch(const spd_config *cfg, const spd_weights *w, void *state, size_t *state_bytes,
                                    void *stage_stream, void *pdm_stream, spd_t **out);

/* Select the draft policy.  SPD_DRAFT_FORCED (greedy mode only): when
 * drafting position q < ref_len, if u[q][SPD_U_FORCE] < p_accept the draft is
 * ref_tokens[q], else the PDM's prediction or (ref+1) mod V should that equal
 * ref_tokens[q]; positions >= ref_len use the PDM's prediction.  ref_tokens
 * is a device int32 array the caller keeps alive; the uniform table must be
 * set.  Verification is unchanged, so the output is lossless under any
 * policy.  Errors: SPD_EINVAL. */
SPD_API int spd_set_draft_policy(spd_t *h, int32_t policy, float p_accept, const int32_t *ref_tokens_dev,
                         int32_t ref_len);

/* Forced acceptance for draft trees (test harness device, greedy only; not
 * on the pages): with ref_tokens the target's greedy continuation and the
 * forced leaf (the leaf whose in-flight path matches ref_tokens, else the
 * rank-0 leaf), u = u[q][SPD_U_FORCE] for position q puts the pair (forced
 * leaf, ref[q]) first in the ranking when u < p_first, at rank W-1 when
 * p_first <= u < p_tree (a second-ranked draft only a tree catches), and
 * otherwise replaces it by the next id not already a candidate of that leaf.
 * Positions >= ref_len are drafted naturally.  Needs draft_width >= 2 and the
 * uniform table.  Errors: SPD_EINVAL. */
SPD_API int spd_set_tree_policy(spd_t *h, float p_first, float p_tree, const int32_t *ref_tokens_dev,
                                int32_t ref_len);

/* How spd_cycle submits work.  SPD_LAUNCH_GRAPH (the default): each
 * stream's chain of one cycle is captured once as a HIP graph (on the first
 * spd_cycle after the policy or uniforms changed) and replayed; a cycle then
 * costs one entry launch, two graph launches and four event calls on the
 * host.  SPD_LAUNCH_EAGER: every kernel is launched individually (needed for
 * the per-launch gate/up timing of spd_timing_*).  Either may be or-ed with
 * SPD_LAUNCH_SERIALIZED: the draft module is then enqueued on the stage
 * stream ahead of the stage step instead of running beside it on the draft
 * stream -- the same results (the draft module reads only the state from
 * before the stage step, [RB] method step 4), no overlap; it measures each
 * kernel alone and the draft module's marginal cost.  Waits for both
 * streams.  Errors: SPD_EINVAL. */
#define SPD_LAUNCH_EAGER 0
#define SPD_LAUNCH_GRAPH 1
#define SPD_LAUNCH_SERIALIZED 2
SPD_API int spd_set_launch_mode(spd_t *h, int32_t mode);

/* Per-position uniforms, device fp32 [n_positions][SPD_U_COUNT], values in
 * [0,1); row p is used for the decisions about position p (draft draw,
 * acceptance, residual redraw, prefill draw, forced-acceptance test).
 * Required in sample mode and for the forced policy.  n_positions must
 * cover max_ctx.  Errors: SPD_EINVAL. */
SPD_API int spd_set_uniforms(spd_t *h, const float *uniforms_dev, int32_t n_positions);

/* Prefill.  The pages describe decoding only and say nothing of how the
 * prompt is processed; this library takes the plain reading that a prompt
 * is an ordinary full target pass (the same per-token arithmetic as the
 * pipeline's stages) whose anchor taps also build the draft module's
 * committed state, so that the first cycle starts from the state the method
 * assumes ([RB] method step 1: the pipeline starts from a committed
 * prefix; [PL] section 3.3: the draft module's pre-step inputs).
 *
 * Full target pass over the prompt (host int32 ids in [0,V)),
 * writing every layer's KV and the PDM's committed state for all prompt
 * positions, then the first generated token (argmax, or drawn with
 * u[len][SPD_U_TARGET]).  Leaves the pipeline empty, seeded with that token
 * at position len.  Blocking: returns after the device finished.  Errors:
 * SPD_EINVAL (len < 1, id out of range), SPD_ECTX (len + max_new + n_stages >
 * max_ctx), SPD_EHIP. */
SPD_API int spd_prefill(spd_t *h, const int32_t *prompt_host, int32_t len, int32_t *first_token);

/* One SPD cycle carries out [RB] method steps 1-5: entry of the newest
 * draft with its anchor 0, one stage sub-step of every in-flight token, the
 * draft module on the pre-step anchors, verification of the token leaving
 * the last stage and, on rejection, the three-step rollback; in [PL]'s
 * terms sections 3.1-3.4 (stage-grouped decode, the fused anchor feature,
 * the pre-step draft module, the verify/rollback rule).  With draft_width
 * W >= 2 the in-flight tokens form a draft tree ([RB] prerequisites, draft
 * tree; [PL] appendix B): the entry adds up to W nodes, every node takes
 * the stage sub-step, and verification keeps the exiting node's matching
 * child.  The stage sub-step runs on the stage stream and the draft module
 * on the draft stream, joined by events at the cycle boundary.
 *
 * Enqueue n_cycles SPD cycles on the two streams and return without waiting.
 * Cycles enqueued after max_new tokens have been emitted do nothing (their
 * records carry SPD_FLAG_IDLE).  If log_host is not NULL it must be pinned
 * host memory for n_cycles records; they are valid once spd_sync returned.
 * Errors: SPD_ESTATE (no prefill yet), SPD_EINVAL, SPD_EHIP. */
SPD_API int spd_cycle(spd_t *h, int32_t n_cycles, spd_cycle_rec *log_host);

/* Host-requested form of the rollback ([RB] method step 5): wait for both
 * streams, set every target layer's KV length to keep_len, cut the PDM's
 * committed length to min(committed, keep_len) (position keep_len-1 may stay
 * uncommitted if it is the last verified one), flush the in-flight state and
 * seed reseed_token at position keep_len.  Blocking.  Errors: SPD_ESTATE
 * (keep_len < 1, beyond the verified prefix, or more than one uncommitted
 * position), SPD_EINVAL (token out of range). */
SPD_API int spd_rollback(spd_t *h, int32_t keep_len, int32_t reseed_token);

/* Plain greedy autoregressive decoding of the target from the current
 * seeded state (after prefill or rollback): n_tokens more tokens after the
 * seed token, one whole-model pass each, with the per-row arithmetic of the
 * pipeline's kernels (so its output equals the pipeline's greedy output
 * bit for bit).  The n_tokens new ids go to tokens_host if it is not NULL.
 * Blocking.  Leaves the KV caches extended: call spd_rollback before further
 * cycles.  Errors: SPD_ESTATE (no prefill), SPD_ECTX. */
SPD_API int spd_generate_ar(spd_t *h, int32_t n_tokens, int32_t *tokens_host);

/* Wait for both streams and report the engine status.  Returns SPD_EDEVICE
 * if a device-side check flag is set, SPD_EHIP on a HIP error. */
SPD_API int spd_sync(spd_t *h, spd_status *status);

/* Copy tokens[first .. first+count) of the sequence (prompt, emitted tokens
 * and in-flight drafts) to host memory.  Blocking. */
SPD_API int spd_read_tokens(spd_t *h, int32_t first, int32_t count, int32_t *out_host);

/* Debug copies of device state to host memory (blocking):
 *   SPD_DBG_ANCHORS  anchors of position `index` [m][d] fp32
 *   SPD_DBG_HIDDEN   in-flight hidden state of position `index` [d] fp32
 *   SPD_DBG_LOGITS   target logits of the last verification [V] fp32
 *   SPD_DBG_PDM_LOGITS PDM logits of the last cycle [V] fp32
 *   SPD_DBG_KV_K / SPD_DBG_KV_V  target layer `index` key/value cache
 *                    [max_ctx][Hkv][hd] in config dtype (row-major by position)
 * `bytes` must equal the size of the item. */
#define SPD_DBG_ANCHORS 0
#define SPD_DBG_HIDDEN 1
#define SPD_DBG_LOGITS 2
#define SPD_DBG_PDM_LOGITS 3
#define SPD_DBG_KV_K 4
#define SPD_DBG_KV_V 5
SPD_API int spd_debug_read(spd_t *h, int32_t what, int32_t index, void *out_host, size_t bytes);

/* Timing instrumentation.  spd_timing_enable(h, 1) makes every later cycle
 * record HIP events: at the start of the cycle, after the stage step +
 * verification, after the PDM, and (eager launch mode only) around every
 * launch of the stage-grouped gate/up projection (the largest weight stream).  spd_timing_read waits,
 * returns the number of cycles timed and fills (each may be NULL):
 *   cycle_ms[3*i+0..2]  end of stage work, end of PDM work, cycle end (max of
 *                       both) of cycle i, in ms after that cycle's start;
 *   gu_ms               summed duration of all timed gate/up launches;
 *   gu_launches         their count.
 * cap bounds the cycles written to cycle_ms.  spd_timing_enable(h, 0) stops
 * and discards.  Errors: SPD_EHIP. */
SPD_API int spd_timing_enable(spd_t *h, int32_t enable);
SPD_API int spd_timing_read(spd_t *h, int32_t cap, float *cycle_ms, double *gu_ms, int32_t *gu_launches);

/* Release events and the handle (device memory stays the caller's). */
SPD_API int spd_destroy(spd_t *h);

/* Static text for a return code. */
SPD_API const char *spd_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* SPD_H */
