/*
 * kvev.h -- C ABI of the attention-scored KV-cache eviction library (gfx950).
 *
 * One decode step of the method is kvev_decode_step() followed by
 * kvev_evict(): at each step, given the query, the cached K/V and a fixed
 * budget, the library decides which cached entries are retained.  This is the
 * problem statement of "What Matters for Aggressive Decoding-Time KV
 * Eviction?" (section 1 and section 3: retain or permanently evict under a
 * fixed budget B) and of "MemDecay" (section III-A, objective (1)).
 *
 * Conventions for every entry point:
 *   - Pointers named "device" are HIP device pointers owned by the caller and
 *     read or written in stream order on the context's stream; the caller
 *     keeps them alive until that stream work completes.  Pointers named
 *     "host" are ordinary host memory, read or written before the call
 *     returns (such calls synchronise the stream).
 *   - The library owns all cache memory (allocated by kvev_create); the step
 *     path itself allocates nothing.
 *   - Every call returns a kvev_status.  No exception crosses the ABI.  A HIP
 *     runtime failure returns KVEV_EHIP and makes the context sticky: every
 *     later call except kvev_last_error / kvev_destroy returns KVEV_ESTATE.
 *     kvev_last_error() describes the last failure.
 *   - A context is bound to one HIP stream and is not thread safe.  (With
 *     cfg.prefetch_blocks > 0 it also owns one copy stream of its own, at
 *     default priority, ordered against the context's stream by events.)
 *   - Element dtype of q / k / v inputs is cfg.dtype (fp32 or bf16, dense,
 *     row-major, head_dim innermost); attention outputs are always fp32.
 */
#ifndef KVEV_H
#define KVEV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvev_ctx kvev_ctx;

typedef enum {
  KVEV_OK = 0,
  KVEV_EINVAL = -1, /* bad argument, shape or configuration */
  KVEV_ENOMEM = -2, /* device allocation failed or page pool exhausted */
  KVEV_EHIP = -3,   /* HIP runtime error (context becomes sticky) */
  KVEV_ESTATE = -4, /* call not valid in the current state, or sticky error */
  KVEV_ERANGE = -5  /* host buffer too small / index out of range */
} kvev_status;

typedef enum { KVEV_F32 = 0, KVEV_BF16 = 1 } kvev_dtype;

/* Score aggregation rule.
 *  EMA:        score <- alpha_new*mass + (1-alpha_new)*score, applied once per
 *              layer in ascending layer order ("What Matters ...", section
 *              3.1 Eq.4 and appendix E "Layer scoring").
 *  CUMULATIVE: score <- score + mass per layer (same page, Eq.3).
 *  LRFU_BLOCK: one score per (sequence, 16-token block) over every layer
 *              and head: the block's attention mass summed over layers and
 *              query heads and divided by n_q_heads * n_layers, folded once
 *              per step by the EMA rule; eviction priority
 *              (1 - score)(1 - survival), survival = the block's mean over
 *              its tokens of exp(-(beta + lambda_region) * idle) ("Attention-
 *              Aware Block Eviction" figure page; "MemDecay" section III-C
 *              Eq.3-4 and section IV-B Eq.7 for lambda = ln2 / half-life).
 *              Lower priority is kept.  Selection groups are sequences and
 *              budgets count blocks.                                          */
/*  TIERED_INT2: routing of 32-token windows per layer between a
 *              full-precision tier, a recoverable INT2 tier and permanent
 *              eviction (technical review of "QEvict", section 4).  Every
 *              accessible window's score is the running sum over steps of
 *              the attention probability landing on its tokens, summed over
 *              the layer's query heads and divided by n_q_heads (section
 *              4.2, Eq.1, routing interval one step).  After each step, per
 *              layer, the candidate windows (not evicted, not holding a
 *              sink position, and older than the n_recent newest positions)
 *              are ranked by (score, window index): the best fp_windows are
 *              full precision, the next int2_windows INT2, the rest evicted
 *              for good (section 4.4, Eq.4-6).  A window is quantized once,
 *              at its first demotion (keys: scale and zero point per channel
 *              over the window's tokens; values: per token and 32-channel
 *              group; asymmetric min-max, scale = (max - min) / 3 and zero =
 *              min stored as fp16, codes = clamp(rint((x - zero) / scale),
 *              0, 3) in fp32), and its codes are reused by every later
 *              demotion; a promotion writes the reconstruction code * scale
 *              + zero, rounded to bf16, as the window's full-precision values
 *              (section 4.4, Algorithm 1; no rotary embedding is re-applied).
 *              Attention reads INT2 windows through their reconstruction in
 *              the kernel (section 4.1).  Selection groups are layers.        */
typedef enum {
  KVEV_EMA = 0,
  KVEV_CUMULATIVE = 1,
  KVEV_LRFU_BLOCK = 2,
  KVEV_TIERED_INT2 = 3
} kvev_policy;

#define KVEV_MAX_REGIONS 8

/* Scorer variants of the token policies ("What Matters ...", section 5.1 and
 * appendix E), a bit mask; both act on a layer's observation before the
 * temporal fold.
 *  VNORM:   each head's probability on a token is multiplied by the l2 norm
 *           of that token's value row divided by the mean of those norms over
 *           the tokens the head attends to (at that layer and KV head; all
 *           norms zero: factor 1).
 *  ENTROPY: a layer's observation is multiplied by one scalar, the mean over
 *           the heads pooled into the state of H / ln n, H the Shannon
 *           entropy of the head's attention distribution over its n tokens
 *           (n == 1: factor 1).                                               */
typedef enum { KVEV_SCORE_VNORM = 1, KVEV_SCORE_ENTROPY = 2 } kvev_scorer;

/* What one utility belongs to (token policies).
 *  PER_KV_HEAD:  one utility per (sequence, KV head, token): the sum of the
 *                KV head's query-group probabilities; budgets and retained
 *                sets are per (sequence, KV head).
 *  PER_SEQUENCE: one utility per (sequence, token): the mean over all query
 *                heads of their probabilities ("What Matters ...", section
 *                3.1 Eq.1; appendix E for GQA); one retained set per
 *                sequence, shared by every KV head and layer.                 */
typedef enum { KVEV_PER_KV_HEAD = 0, KVEV_PER_SEQUENCE = 1 } kvev_granularity;

typedef struct {
  int32_t n_layers;         /* L, 1..64 */
  int32_t n_q_heads;        /* Hq: n_kv_heads times 1..8 (times 4 in the block
                               and tiered modes) */
  int32_t n_kv_heads;       /* Hkv */
  int32_t head_dim;         /* d: 64 or 128 */
  int32_t batch;            /* sequences stepped together */
  int32_t dtype;            /* kvev_dtype of q, k, v and the cache */
  int64_t max_tokens;       /* per-sequence slot capacity (>= prefill + steps) */
  int32_t page_tokens;      /* tokens per cache page; must be 16 */
  int32_t policy;           /* kvev_policy */
  float alpha_new;          /* EMA weight on the new observation, (0, 1] */
  int32_t refresh_interval; /* r >= 1: scores observed at t with (t-1) % r == 0
                               ("What Matters ...", section 3.2 Eq.6) */
  int32_t score_free;       /* 1: observe only at t == 1, then freeze
                               (same page, section 3.2 "Score-Free") */
  int32_t n_sink;           /* positions < n_sink are never evicted */
  int32_t n_recent;         /* the n_recent newest positions are never evicted */
  int64_t budget;           /* retained tokens per (sequence, KV head); LRFU_BLOCK:
                               retained blocks per sequence (default for all) */
  /* KVEV_LRFU_BLOCK only (ignored by the token policies).  In this mode
   * max_tokens bounds the positions a sequence reaches (prefill + steps) and
   * may be at most 65536; n_sink, n_recent must be 0, refresh_interval 1,
   * score_free 0 (protection comes from pinned regions). */
  float beta;                                 /* recency rate (>= 0), e.g. 0.001 */
  float region_half_life[KVEV_MAX_REGIONS];   /* steps; <= 0: that region does not decay */
  uint32_t pinned_region_mask;                /* bit r: blocks holding a region-r token are
                                                 never evicted */
  int32_t decode_region;                      /* region of decoded tokens, 0..7, not pinned */
  float access_tau_mult;                      /* a block is accessed when its mass per token
                                                 is >= access_tau_mult / (resident tokens);
                                                 "MemDecay" section IV-A uses 2 */
  /* KVEV_TIERED_INT2 only: dtype bf16, head_dim 128, 4 query heads per KV
   * head, batch 1, max_tokens <= 12288 windows, refresh_interval 1, score_free 0;
   * budget is ignored (the tier capacities replace it).  n_sink positions
   * (their windows) and the n_recent newest positions (their windows) stay
   * full precision and are never routed. */
  int32_t window_tokens;                      /* tokens per window: 32, or 8 ("QEvict" review,
                                                 section 5: the review's default) */
  int32_t fp_windows;                         /* K_f: routed windows kept in full precision */
  int32_t int2_windows;                       /* K_q: routed windows kept in INT2 */
  /* KVEV_EMA and KVEV_CUMULATIVE only (0 in the other modes). */
  int32_t scorer;                             /* kvev_scorer bit mask; 0: attention */
  int32_t granularity;                        /* kvev_granularity */
  /* KVEV_TIERED_INT2 only: the routing interval Omega.  kvev_step runs a
   * routing event after the decode steps t (counted from 1) with
   * t % Omega == 0; the window scores accumulate every step in between
   * ("QEvict" review, section 4.2 Eq.1; the review's default is 8).  0 or 1:
   * every step.  kvev_evict is always one routing event. */
  int32_t route_interval;
  /* Rank-trace diagnostics (KVEV_EMA and KVEV_CUMULATIVE, PER_KV_HEAD,
   * refresh_interval 1, score_free 0; 0 in the other modes).  0: off.
   * k >= 1: every kvev_step also records, per (sequence, KV head) group,
   * the statistics of kvev_diag_group over the top-k sets (k = min(k, the
   * step's token count)); kvev_step is then the only call that changes the
   * state (kvev_decode_step, kvev_evict and kvev_import_group return
   * KVEV_ESTATE).  Appendix I of "What Matters ..." takes k = the budget. */
  int32_t diag_topk;
  /* KVEV_LRFU_BLOCK only: host-offload tier ("MemDecay" section III-E).  0:
   * off.  C >= 1: a pinned host pool of C block slots (each block's K and V
   * pages of every layer and KV head, as stored).  After every selection the
   * evicted blocks are copied into it, ranked by (sequence, block id); when a
   * selection evicts E > C blocks only the last C are kept.  Slots are reused
   * in ring order, so the pool holds the latest C evictions that have not
   * been re-admitted since; kvev_readmit_offloaded recovers them.
   * kvev_import_blocks is then refused (KVEV_ESTATE). */
  int32_t offload_blocks;
  /* KVEV_TIERED_INT2 only: routing diagnostics ("QEvict" review, section 3).
   * 0: off.  g >= 1: every routing event records, per layer, the selection
   * churn of the routed full-precision set and of the routed retained set
   * (full precision or INT2) against the previous event, and Global LIR: a
   * routed window's run of consecutive events outside the full-precision
   * set counts as sustained when it reaches g events, and as revived when
   * the window re-enters the full-precision set after such a run.  Tier
   * imports (kvev_tier_import) are not routing events and record nothing. */
  int32_t revival_gap;
  /* KVEV_LRFU_BLOCK with offload_blocks > 0: device staging slots for
   * kvev_prefetch_offloaded (0: no prefetch). */
  int32_t prefetch_blocks;
  /* KVEV_LRFU_BLOCK with offload_blocks > 0: an evicted block whose
   * persisted score is below this value is dropped instead of offloaded
   * (the graded offload / drop rule of "MemDecay" section III-E; 0: every
   * evicted block is offloaded). */
  float offload_min_score;
  /* Token policies and the block mode, bf16 and head_dim 128: which
   * attention kernel runs (a kvev_attn_path).  AUTO: the whole-cache kernel
   * (one workgroup per (KV head group, layer) over every retained slot; it
   * writes the outputs and each slot's group mass, in the block mode each
   * table entry's, directly) when there are at least 224 (group, layer)
   * pairs, the step's slot count fits its bound (8,192 slots and its LDS)
   * and no scorer variant is set (per-sequence granularity included: the
   * fold then pools each sequence's KV head groups); the split kernel
   * otherwise.  SPLIT: always the split kernel.  WHOLE: the
   * whole-cache kernel whenever it applies, whatever the pair count.
   * Results agree within the tolerances; each path is deterministic. */
  int32_t attn_path;
  /* Token policies: kvev_step selects only after the steps t (counted from
   * 1) with (t - 1) % evict_interval == 0, and in between only appends, so
   * the cache grows to budget + evict_interval - 1 tokens.  This is the
   * literal reading of the batched lazy workload's "recompute scores and
   * evict every 8 steps"; 0 or 1: every step ("What Matters ...", section
   * 3.2 evicts every step).  kvev_evict always selects. */
  int32_t evict_interval;
  /* KVEV_TIERED_INT2 only (0 otherwise): rotary mode ("QEvict" review,
   * section 4.4, "Positional handling for promoted keys").  0: off, keys
   * carry no rotation.  theta > 0: q, k_new and the prefill keys arrive
   * before the rotary embedding; the library rotates channel pair (i, i+64)
   * of a key at position p by p * theta^(-2i/128) (angles and rotation in
   * fp64, rounded to fp32 then bf16) and stores the rotated keys as full
   * precision; keys are quantized from their values before the rotation
   * (kept until the first demotion), and a reconstruction is rotated again
   * at the window's original positions.  The query of a step is rotated at
   * the new token's position.  With rotary mode or 8-token windows, an INT2
   * window is attended through its reconstruction rounded to bf16, which is
   * written into its full-precision storage at its first demotion (so a
   * promotion leaves that storage as it is). */
  float rope_theta;
  /* KVEV_TIERED_INT2 only (0 otherwise): how the INT2 quantizer groups the
   * keys.  0: one scale and zero per channel over the window's tokens (the
   * "QEvict" review, section 4.4 Algorithm 1).  1: one per token and
   * 32-channel group, like the values (the 131k workload's
   * "per-32-channel-group" wording read for keys too).  With 1 an INT2
   * window is attended through its reconstruction rounded to bf16, kept in
   * its full-precision slot (as with rope_theta > 0), and kvev_tier_ledger
   * returns the key parameters as [W][4] (token, group). */
  int32_t int2_key_groups;
  /* Token policies only (0 otherwise): the new token's starting utility on
   * an observation step (a kvev_new_token_init).  ZERO: 0, as the prefill
   * tokens start ("What Matters ...", appendix E), then folded with its
   * own mass.  MEAN: the mean of the other utilities of its group (of its
   * sequence, with per-sequence granularity), the rule appendix E states
   * for the steps without an observation, then folded.  On those steps the
   * new token takes the mean either way. */
  int32_t new_token_init;
} kvev_config;

typedef enum { KVEV_ATTN_AUTO = 0, KVEV_ATTN_SPLIT = 1, KVEV_ATTN_WHOLE = 2 } kvev_attn_path;
typedef enum { KVEV_NEW_TOKEN_ZERO = 0, KVEV_NEW_TOKEN_MEAN = 1 } kvev_new_token_init;

/* Fill *cfg with defaults: page_tokens 16, EMA, alpha_new 0.05,
 * refresh_interval 1, no protection, window_tokens 32, rope_theta 0; shape
 * fields zero. */
void kvev_config_init(kvev_config* cfg);

/* Validate *cfg, allocate the page pool and all per-step state on the
 * current HIP device, bind `hip_stream` (a hipStream_t; NULL = default
 * stream).  On success *out owns everything until kvev_destroy.
 * Errors: KVEV_EINVAL (bad config: d not 64/128, Hq % Hkv != 0 or a group
 * size outside 1..8, budget < 1, n_sink + n_recent > budget, page_tokens !=
 * 16, ...), KVEV_ENOMEM, KVEV_EHIP. */
kvev_status kvev_create(const kvev_config* cfg, void* hip_stream, kvev_ctx** out);

/* Free everything the context owns (synchronises its stream).  NULL is a no-op. */
kvev_status kvev_destroy(kvev_ctx* ctx);

/* Load the prefill cache of sequence `seq` (0 <= seq < batch): device k, v
 * laid out [n_layers][n_kv_heads][n_tokens][head_dim].  Positions are
 * 0..n_tokens-1 and every utility starts at 0 ("What Matters ...", appendix
 * E "Momentum initialization").  region_labels: host, one label (0..7) per
 * token, used by KVEV_LRFU_BLOCK (NULL: every token takes decode_region;
 * ignored by the token policies).  In LRFU_BLOCK mode every block starts
 * resident with score 0 and clock 0; the blocks pinned by the labels plus
 * the last block must fit the budget each selection uses (checked by
 * kvev_set_budget and by every selecting call).  Must be called for every
 * sequence before the first decode step, and not after it.
 * Errors: KVEV_EINVAL (n_tokens < 1 or + decode headroom > max_tokens, a
 * label out of range), KVEV_ESTATE, KVEV_ENOMEM (pool). */
kvev_status kvev_prefill(kvev_ctx* ctx, int32_t seq, const void* k, const void* v,
                         int64_t n_tokens, const uint8_t* region_labels);

/* Decode step t (counted by the context from 1): append k_new/v_new at the
 * next position of every (layer, sequence, KV head); run GQA decode
 * attention of every layer over the group's cached tokens; write the
 * attention output; and, on an observation step, fold each KV head's
 * per-token softmax mass summed over its query group into the utility,
 * layer by layer.  On a non-observation step the new token's utility starts
 * at the mean of the group's existing utilities and nothing else changes
 * ("What Matters ...", appendix E "New token insertion").  On an observation
 * step the new token starts at 0 and is folded with its own mass.
 *   q      device [n_layers][batch][n_q_heads][head_dim]   (cfg.dtype)
 *   k_new  device [n_layers][batch][n_kv_heads][head_dim]  (cfg.dtype)
 *   v_new  device [n_layers][batch][n_kv_heads][head_dim]  (cfg.dtype)
 *   out    device [n_layers][batch][n_q_heads][head_dim]   fp32, written
 * Logits use (q.k)/sqrt(head_dim) in fp32 ("QEvict" review, section 4.1,
 * (Attention)).  Errors: KVEV_ESTATE (a sequence has no prefill, or the
 * slot capacity is exhausted), KVEV_EHIP. */
kvev_status kvev_decode_step(kvev_ctx* ctx, const void* q, const void* k_new,
                             const void* v_new, float* out);

/* Enforce the budget in every (sequence, KV head) group holding more than
 * `budget` tokens (budget <= 0: cfg.budget): keep the protected tokens (sinks
 * and the n_recent newest) and the top (budget - |protected|) of the rest by
 * (utility, position), larger kept; compact the survivors into slots
 * [0, budget) of every layer's K and V (holes below the budget, ascending,
 * take the kept slots at or above it, ascending).  A group within budget is
 * left untouched.  Eviction is irreversible ("What Matters ...", section 3.1;
 * "MemDecay", section III-A (1) with the forced set).
 * Errors: KVEV_EINVAL (budget < n_sink + n_recent), KVEV_EHIP. */
kvev_status kvev_evict(kvev_ctx* ctx, int64_t budget);

/* One whole decode step of the method: kvev_decode_step followed by
 * kvev_evict(budget), fused into two kernel launches (attention with the
 * append; then probability pass, fold, selection and compaction, with
 * moves of more than a few slots in a third launch).  Same arguments,
 * layouts and errors as those two calls; results are identical to calling
 * them in sequence. */
kvev_status kvev_step(kvev_ctx* ctx, const void* q, const void* k_new, const void* v_new,
                      float* out, int64_t budget);

/* Copy the utilities of group (seq, kv_head) in slot order into host `dst`
 * (capacity `cap` floats); *n_written = the group's token count.  In
 * LRFU_BLOCK mode: the scores of every block the sequence has had, by block
 * id (kv_head must be a valid head; scores are shared by all heads).
 * Synchronises.  Errors: KVEV_ERANGE (cap too small / bad indices). */
kvev_status kvev_scores(kvev_ctx* ctx, int32_t seq, int32_t kv_head, float* dst,
                        int64_t cap, int64_t* n_written);

/* Copy the positions of group (seq, kv_head) in slot order into host
 * `positions` (capacity `cap`); *n = count.  Synchronises. */
kvev_status kvev_retained(kvev_ctx* ctx, int32_t seq, int32_t kv_head,
                          int32_t* positions, int64_t cap, int64_t* n);

/* Gather the cached K and V of group (seq, kv_head) in slot order into
 * device buffers k_out / v_out, each [n_layers][n][head_dim] (cfg.dtype),
 * n = the group's count, which is returned in *n.  cap = rows per layer the
 * buffers hold.  Stream-ordered (does not synchronise). */
kvev_status kvev_export_kv(kvev_ctx* ctx, int32_t seq, int32_t kv_head, void* k_out,
                           void* v_out, int64_t cap, int64_t* n);

/* Replace the state of group (seq, kv_head): n tokens with host `positions`
 * and host `scores` (slot order), and device k, v [n_layers][n][head_dim].
 * Used to put both sides of a comparison on the same state.  With
 * granularity KVEV_PER_SEQUENCE every KV head of the sequence holds the same
 * slots: the caller imports each of them with the same positions (and
 * scores), and kvev_decode_step / kvev_step / kvev_evict return KVEV_ESTATE
 * until the sequence's last KV head is imported.
 * Errors: KVEV_EINVAL (different positions for another KV head of a
 * per-sequence context) / KVEV_ERANGE (n > capacity), KVEV_ENOMEM,
 * KVEV_ESTATE (diagnostics on). */
kvev_status kvev_import_group(kvev_ctx* ctx, int32_t seq, int32_t kv_head, int64_t n,
                              const int32_t* positions, const float* scores,
                              const void* k, const void* v);

/* ---- Rank-trace diagnostics (cfg.diag_topk > 0) ------------------------
 * After each kvev_step, for every (sequence, KV head) group, over the n
 * tokens the step attended (the new one included, before the eviction):
 *   raw_t(i)  = the step's observation of token i summed over the layers
 *               (the per-layer group mass, times the scorer factors);
 *   util_t(i) = its utility after the step's fold;
 *   R_t, E_t  = the k tokens with the largest (raw_t, position) and
 *               (util_t, position) keys, k = min(cfg.diag_topk, n);
 *   Ev_t      = the tokens the step evicted; S_t = the tokens kept.
 * Churn of a set is one minus the Jaccard index |X_t & X_t'| / |X_t | X_t'|
 * against the previous step t' ("What Matters ...", appendix I, Table 13:
 * raw and EMA top-k churn, raw / EMA Jaccard overlap, the share of the raw
 * top-k evicted; the "QEvict" review, section 3: selection churn of the
 * retained set between consecutive selections). */
typedef struct {
  /* the last step's counts */
  int32_t n;                /* tokens the step attended */
  int32_t k;                /* |R_t| = |E_t| */
  int32_t raw_overlap;      /* |R_t & R_t-1| */
  int32_t raw_prev;         /* |R_t-1| (0 at the first recorded step) */
  int32_t util_overlap;     /* |E_t & E_t-1| */
  int32_t util_prev;        /* |E_t-1| */
  int32_t raw_util_overlap; /* |R_t & E_t| */
  int32_t raw_top_evicted;  /* |R_t & Ev_t| */
  int32_t evicted;          /* |Ev_t| */
  int32_t retained;         /* |S_t| */
  int32_t retained_overlap; /* |S_t & S_t-1| */
  int32_t retained_prev;    /* |S_t-1| */
  /* sums over the recorded steps (churns over the steps with a previous one) */
  int64_t steps;
  int64_t pairs;
  double sum_raw_churn;     /* 1 - J(R_t, R_t-1) */
  double sum_util_churn;    /* 1 - J(E_t, E_t-1) */
  double sum_raw_util_jaccard;  /* J(R_t, E_t) */
  double sum_raw_top_evicted;   /* |R_t & Ev_t| / k */
  double sum_selection_churn;   /* 1 - J(S_t, S_t-1) */
} kvev_diag_group;

/* Copy the diagnostics of groups 0..n_groups-1 (g = seq * n_kv_heads +
 * kv_head) to host `out`.  Synchronises.  Errors: KVEV_ESTATE (diagnostics
 * off), KVEV_ERANGE (n_groups outside 1..batch * n_kv_heads). */
kvev_status kvev_diag_read(kvev_ctx* ctx, kvev_diag_group* out, int32_t n_groups);

/* Copy the last step's per-token inputs of the diagnostics of group
 * (seq, kv_head), in the step's slot order, to host buffers (any may be
 * NULL): positions, raw_t, util_t; *n = the step's token count (0 before
 * the first step).  Synchronises.  Errors: KVEV_ESTATE (diagnostics off),
 * KVEV_ERANGE (cap too small / bad indices). */
kvev_status kvev_diag_trace(kvev_ctx* ctx, int32_t seq, int32_t kv_head, int32_t* positions,
                            float* raw, float* util, int64_t cap, int64_t* n);

/* Future missed mass ("QEvict" review, section 3): for every group, the
 * share of the full cache's attention at the last step that lands on
 * positions the compressed cache evicted at an earlier step,
 *   fmm[g] = sum_{i evicted before step t} raw_full(i) / sum_i raw_full(i),
 * raw_full = the full context's per-token group mass summed over layers.
 * `full` must never evict (budget >= max_tokens), use the attention scorer
 * and have been stepped with the same prefill and inputs as `compressed`
 * (same shape, same step count, both with diagnostics on).  Waits for
 * `full`'s stream on `compressed`'s stream, then synchronises; fmm: host
 * [batch * n_kv_heads].  Errors: KVEV_EINVAL (mismatched contexts),
 * KVEV_ESTATE (diagnostics off, no step yet). */
kvev_status kvev_diag_fmm(kvev_ctx* full, kvev_ctx* compressed, double* fmm);

/* kvev_diag_fmm for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): same
 * arguments, checks and result, but nothing is allocated.  The per-group
 * results are staged in a fixed device array of 4,096 doubles (32 KiB) that
 * each GPU the library runs on holds until the process ends; instead of an
 * event, the call synchronises `full`'s stream before launching on
 * `compressed`'s.  Every call on a GPU shares that GPU's array, so calls
 * that overlap on one GPU (from several threads) race.  The current device
 * must be the contexts' device.  Errors: as kvev_diag_fmm, and KVEV_ERANGE
 * (more than 4,096 groups), KVEV_EINVAL (another device current). */
kvev_status kvev_diag_fmm_noalloc(kvev_ctx* full, kvev_ctx* compressed, double* fmm);

/* ---- KVEV_LRFU_BLOCK mode ---------------------------------------------- */

/* Set the retained-block budget of sequence `seq` (used by kvev_step and
 * kvev_evict when their budget argument is <= 0).  Errors: KVEV_EINVAL (not
 * block mode, budget below the sequence's pinned blocks + 1). */
kvev_status kvev_set_budget(kvev_ctx* ctx, int32_t seq, int64_t budget);

/* Re-admit n evicted blocks of sequence `seq`: host block_ids (ids are
 * position / 16; each evicted, not the block being filled), device k, v
 * [n_layers][n_kv_heads][16 * n][head_dim] holding the blocks' tokens in
 * the order of block_ids.  Each block returns with the score it had when it
 * was evicted (the "Attention-Aware Block Eviction" figure page: the
 * block's key and score persist and are restored rather than reset) and
 * its clock set to the current step count.  The resident count may then
 * exceed the budget until the next selection.  Synchronises (validation
 * reads the residency flags).  Errors: KVEV_EINVAL (not block mode, a block
 * resident or unknown, duplicates), KVEV_ENOMEM (no free pages). */
kvev_status kvev_readmit(kvev_ctx* ctx, int32_t seq, int64_t n, const int64_t* block_ids,
                         const void* k, const void* v);

/* Re-admit n evicted blocks of sequence `seq` from the host-offload pool
 * (cfg.offload_blocks > 0): as kvev_readmit, with each block's K and V
 * taken from its pool slot (bit-exact copies of its pages at eviction) and
 * the slot released.  Synchronises.  Errors: as kvev_readmit, and
 * KVEV_ESTATE (offload off, or a block no longer in the pool: never
 * offloaded, or its slot reused by a later eviction). */
kvev_status kvev_readmit_offloaded(kvev_ctx* ctx, int32_t seq, int64_t n, const int64_t* block_ids);

/* Background prefetch ("MemDecay" section III-E): start copying n evicted
 * blocks of sequence `seq` from the host pool into device staging slots
 * (cfg.prefetch_blocks, reused in ring order) on a stream of the context's
 * own, so that the copy overlaps later work on the context's stream.  A later
 * kvev_readmit_offloaded of such a block restores it from the device copy.
 * The context's stream waits for the copies before it next writes into the
 * pool or restores from staging; a staging entry is dropped when its pool
 * slot is reused.  Synchronises the context's stream first (to read the
 * blocks' slots).  Errors: KVEV_ESTATE (prefetch off, a block not in the
 * pool), KVEV_EINVAL (bad indices, n > prefetch_blocks). */
kvev_status kvev_prefetch_offloaded(kvev_ctx* ctx, int32_t seq, int64_t n, const int64_t* block_ids);

/* Host-pool slot of every block sequence `seq` has had (ids
 * 0..*n_blocks-1): slot index, or -1 (resident, never evicted, or dropped).
 * Synchronises.  Errors: KVEV_ESTATE (offload off), KVEV_ERANGE. */
kvev_status kvev_offload_state(kvev_ctx* ctx, int32_t seq, int32_t* slot, int64_t cap, int64_t* n_blocks);

/* Copy the state of every block sequence `seq` has had so far (ids
 * 0..*n_blocks-1) to host buffers: score, clock (step of the last access or
 * insertion), resident flag.  Any of the three may be NULL.  Synchronises.
 * Errors: KVEV_EINVAL (not block mode), KVEV_ERANGE (cap too small). */
kvev_status kvev_block_state(kvev_ctx* ctx, int32_t seq, float* score, int32_t* tref,
                             uint8_t* resident, int64_t cap, int64_t* n_blocks);

/* Replace the block state of sequence `seq`: host score, tref, resident for
 * blocks 0..n_blocks-1 (n_blocks must equal the count of blocks seen; the
 * last block must be resident), and device k, v [n_layers][n_kv_heads]
 * [n_tokens][head_dim] with the resident blocks' tokens in ascending block
 * order (n_tokens must equal those blocks' token count).  Used to put both
 * sides of a comparison on the same state.  Errors: KVEV_EINVAL. */
kvev_status kvev_import_blocks(kvev_ctx* ctx, int32_t seq, int64_t n_blocks, const float* score,
                               const int32_t* tref, const uint8_t* resident, int64_t n_tokens,
                               const void* k, const void* v);

/* Tier capacities from a byte budget ("QEvict" review, section 4.3 Eq.3):
 * *k_f = floor((1 - q) * b_hist / m_f) and *k_q = floor(q * b_hist / m_q),
 * evaluated in double precision.  b_hist: the bytes left for routed windows
 * after the sink and local windows (B_total - B_sink - B_local); q: the
 * quantized-tier fraction in [0, 1] (the review uses 0.70); m_f, m_q: the
 * bytes of one window in full precision and as an INT2 record, over the
 * layers and KV heads the budget covers (this library's records: 32 tokens
 * x 512 B and 3,072 B per layer and KV head).  Host arithmetic only: no
 * context and no device work.  Errors: KVEV_EINVAL (null outputs, q outside
 * [0, 1], b_hist < 0, m_f or m_q <= 0, non-finite arguments, a capacity
 * above INT32_MAX). */
kvev_status kvev_tier_capacities(double b_hist, double q, double m_f, double m_q, int32_t* k_f,
                                 int32_t* k_q);

/* ---- KVEV_TIERED_INT2 mode ---------------------------------------------
 * In this mode kvev_prefill takes seq 0; kvev_decode_step appends, attends
 * over the full-precision and INT2 windows of every layer and adds each
 * accessible window's mass to its score; kvev_evict (its budget argument is
 * ignored) runs one routing event in every layer with the tier transitions
 * (quantize on first demotion, dequantize on promotion); kvev_step is the
 * two.  kvev_scores(ctx, 0, layer, ...) returns the layer's window scores
 * by window index.  kvev_retained and kvev_export_kv do not apply (use the
 * calls below). */

/* Copy the window state of `layer` (windows 0..*n_windows-1, window w =
 * positions [W w, W w + W), W = window_tokens) to host buffers: score, tier (0 full precision,
 * 1 INT2, 2 evicted), ledger flag (1 while the window holds an INT2 record:
 * from its first demotion until its eviction).  Any may be NULL.
 * Synchronises.  Errors: KVEV_EINVAL (not tiered mode, bad layer),
 * KVEV_ERANGE (cap too small). */
kvev_status kvev_tier_state(kvev_ctx* ctx, int32_t layer, float* score, uint8_t* tier,
                            uint8_t* ledger, int64_t cap, int64_t* n_windows);

/* Copy the full-precision storage of (layer, kv_head) for windows
 * 0..nw-1 into device k_out, v_out, each [W * nw][128] bf16 by position
 * (keys rotated in rotary mode; a window that holds no full-precision slot,
 * evicted or INT2 without bf16 reconstruction, exports zeros; with bf16
 * reconstruction an INT2 window exports its reconstruction).  cap =
 * rows the buffers hold; *n_rows = W * nw.  Stream-ordered.  Errors: KVEV_EINVAL,
 * KVEV_ERANGE. */
kvev_status kvev_tier_export(kvev_ctx* ctx, int32_t layer, int32_t kv_head, void* k_out,
                             void* v_out, int64_t cap, int64_t* n_rows);

/* Copy and unpack the INT2 record of (layer, kv_head, window) to host
 * buffers: k_codes [W][128] (token, channel; keys before the rotation in
 * rotary mode), k_scale / k_zero [128] fp16 bits (with int2_key_groups:
 * [W][4], token and 32-channel group), v_codes [W][128],
 * v_scale / v_zero [W][4] fp16 bits (token, 32-channel group).  Synchronises.  Errors: KVEV_EINVAL (not tiered mode,
 * bad indices, the window holds no record). */
kvev_status kvev_tier_ledger(kvev_ctx* ctx, int32_t layer, int32_t kv_head, int32_t window,
                             uint8_t* k_codes, uint16_t* k_scale, uint16_t* k_zero,
                             uint8_t* v_codes, uint16_t* v_scale, uint16_t* v_zero);

/* Routing diagnostics of one layer (cfg.revival_gap > 0).  Over the
 * event's candidates (aged windows not evicted before it): F = those routed
 * to full precision, R = those kept (full precision or INT2). */
typedef struct {
  int32_t f_prev, f_new, f_overlap;  /* |F_e-1|, |F_e|, |F_e & F_e-1| of the last event */
  int32_t r_prev, r_new, r_overlap;  /* the same for R */
  int64_t events;                    /* routing events so far */
  int64_t pairs;                     /* events with a previous one */
  int64_t sustained;                 /* runs outside F that reached revival_gap events */
  int64_t revived;                   /* such runs ended by re-entering F */
  double sum_f_churn;                /* 1 - J(F_e, F_e-1) over the pairs */
  double sum_r_churn;                /* 1 - J(R_e, R_e-1) */
} kvev_route_diag;

/* Copy layer `layer`'s routing diagnostics to host *out.  Synchronises.
 * Errors: KVEV_EINVAL (not tiered mode), KVEV_ESTATE (diagnostics off),
 * KVEV_ERANGE (layer). */
kvev_status kvev_tier_diag(kvev_ctx* ctx, int32_t layer, kvev_route_diag* out);

/* Replace the window state of `layer`: host score and tier (as in
 * kvev_tier_state) for windows 0..n_windows-1 (n_windows must equal the
 * windows seen).  The tier change of each window is applied as a routing
 * event would apply it (quantize a window entering INT2 without a record,
 * write the reconstruction of a window promoted from INT2).  The tier
 * counts must equal the context's (pinned and local windows full
 * precision).  An evicted window has released its storage and stays
 * evicted.  Used to put both sides of a comparison on the same state.
 * Synchronises.  Errors: KVEV_EINVAL; KVEV_ESTATE (a tier would keep an
 * evicted window). */
kvev_status kvev_tier_import(kvev_ctx* ctx, int32_t layer, int64_t n_windows, const float* score,
                             const uint8_t* tier);

/* Device memory a tiered context holds for windows ("QEvict" review,
 * section 4.1 (Budget) and section 4.3 Eq.3), in bytes over all layers and
 * KV heads: *fp_pool, the full-precision slot pool (keys and values, and
 * the keys before the rotation in the rotary mode); *record_pool, the INT2
 * record pool; *staging, the prefill staging buffers (the prefill windows
 * until the first routing event places them; released by the next decode
 * step).  Per (layer, KV head) the pool has *fp_slots window slots: the
 * pinned windows, the windows not yet routed (the n_recent newest
 * positions plus route_interval new tokens, plus four windows of slack),
 * K_f routed ones, and with 8-token windows or the rotary mode also K_q
 * (INT2 windows are then read through their bf16 reconstructions); and
 * *record_slots records: K_f + K_q (a promoted window keeps its record for
 * its next demotion).  A window releases its full-precision slot when it
 * leaves full precision (INT2 without reconstruction, or evicted) and its
 * record when it is evicted.  Any output may be null.  Errors: KVEV_EINVAL
 * (not tiered mode). */
kvev_status kvev_tier_footprint(kvev_ctx* ctx, int64_t* fp_pool, int64_t* record_pool, int64_t* staging,
                                int32_t* fp_slots, int32_t* record_slots);

/* Wait for all work queued on the context's stream; report a HIP error. */
kvev_status kvev_sync(kvev_ctx* ctx);

/* Decode steps taken so far (the t of the last kvev_decode_step). */
int64_t kvev_step_index(const kvev_ctx* ctx);

/* Kernel timing, measured with HIP events recorded on the context's stream
 * around every launch of the named kernel while enabled.  `kernel`:
 * "attn" (append + split attention), "attn_whole" (append + whole-cache
 * attention with the probability pass), "post" (split merge, probability
 * pass, fold, and in kvev_step selection + compaction), "select" and "move"
 * (kvev_evict; "move" also in kvev_step when many slots move).  The token
 * policies' "attn", "attn_whole" and "post" launches record their own
 * dispatch start and end (no event packets between the step's kernels);
 * every other name is timed by events recorded around its launches.  LRFU_BLOCK
 * mode: "open" (slot and block of the new token), "attn", "merge" (split
 * merge and output), "mass" (block mass), "policy" (score, clock, priority,
 * selection, table compaction), "readmit".  TIERED_INT2 mode: "append",
 * "attn" (attention over the full-precision and INT2 windows), "merge" (split
 * merge and window mass into the scores), "route" (routing and tier
 * transitions).
 * *total_ms / *launches cover the launches since the last reset. */
kvev_status kvev_profile_enable(kvev_ctx* ctx, int32_t enable);
kvev_status kvev_profile_reset(kvev_ctx* ctx);
kvev_status kvev_profile_read(kvev_ctx* ctx, const char* kernel, double* total_ms,
                              int64_t* launches);

/* Text of the last error on this context ("" if none).  ctx may be NULL
 * (then: the last kvev_create failure). */
const char* kvev_last_error(const kvev_ctx* ctx);

/* ---- Measurement utility (not part of the decode step) --------------------
 * The HBM streaming-read ceiling that the attention kernels' achieved
 * bandwidth is compared with ("What Matters ...", appendix J, and the
 * "QEvict" review, section 4.1: decode attention is bound by reading the
 * cache).  Launches one grid-stride read of `bytes` bytes at device pointer
 * `buf` on HIP stream `stream` (a hipStream_t; NULL: the null stream):
 * `blocks` workgroups of 256 threads, eight independent 16-byte loads per
 * thread and iteration, non-temporal when `nontemporal` != 0.  Each block
 * writes one XOR word of what it read to sink[block] (device, >= `blocks`
 * words), so no load is dead.  Asynchronous: time it with events on
 * `stream`.  Errors: KVEV_EINVAL (null pointer, bytes <= 0 or not a multiple
 * of 16, buf not 16-byte aligned, blocks <= 0), KVEV_EHIP (launch failure).
 * No context and no allocation. */
kvev_status kvev_calibrate_read(const void* buf, int64_t bytes, int32_t nontemporal, int32_t blocks,
                                uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVEV_H */
