/*
 * dflash.h -- C-ABI of one DFlash speculative round at batch 1 on one MI355X (gfx950).
 *
 * The round: the drafter's block forward (encoder.fc + output_norm_enc over the captured
 * target residual streams, then Qwen3-shaped bidirectional sliding-window layers with
 * per-head q/k RMSNorm and a SwiGLU MLP), the target's shared raw embedding table and
 * untied lm_head with a per-row argmax, greedy exact-match verification, and the ring
 * context cache with speculative slack and trim rollback.
 *
 * Sources: lablup/mlxcel #1762 "Muse Glimmer DFlash assistant drafter on the round loop"
 * (What changed; Pre-merge review round), z-lab/dflash #168 "load Meta's
 * Muse-Glimmer-30B-assistant DFlash head" (Why), lablup/mlxcel #1751 "LFM2 / LFM2.5
 * DSpark drafter on the DFlash loop" (Security fixes; Implementation Review Summary).
 *
 * Conventions for every call:
 *  - Device pointers point to device memory owned by the caller (PyTorch or hipMalloc).
 *    The library never allocates device memory: the caller sizes the ring, the workspace
 *    and the packed weights with dflash_query_sizes and keeps them alive while the
 *    context is.
 *  - `stream` is a hipStream_t (NULL = the default stream). Device calls only enqueue
 *    work; outputs are valid once the caller has synchronised the stream.
 *  - Every call returns a status and dflash_last_error() describes a failure. Arguments
 *    and the context's state are checked on the host before anything is enqueued: on
 *    DFLASH_E_ARG, _SHAPE, _RANGE, _NO_CONTEXT, _REWIND or _STATE nothing is enqueued and
 *    the context is unchanged. DFLASH_E_DEVICE means a HIP call failed part way: launches
 *    enqueued before it stay enqueued (for instance the K/V projection of deferred rows,
 *    after which the context no longer counts them as deferred), the committed offsets are
 *    unchanged, and the stream should be treated as failed. Nothing throws or aborts
 *    (lablup/mlxcel #1751, Security fixes: an exception crossing the bridge aborts the
 *    process instead of failing the request).
 *  - A context is used by one host thread and one stream at a time.
 *  - Weight matrices are [out, in] row-major (y = x W^T). bf16 is raw 16-bit storage.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dflash_ctx dflash_ctx; /* opaque */

typedef enum {
  DFLASH_OK = 0,
  DFLASH_E_ARG = 1,        /* null pointer or malformed argument */
  DFLASH_E_SHAPE = 2,      /* a dimension out of range, inconsistent, or a size overflow */
  DFLASH_E_RANGE = 3,      /* a token id or a block width out of range */
  DFLASH_E_NO_CONTEXT = 4, /* a draft before any committed context row */
  DFLASH_E_REWIND = 5,     /* a trim deeper than the pending rows or than the slack */
  DFLASH_E_STATE = 6,      /* a draft while appended rows are still uncommitted */
  DFLASH_E_DEVICE = 7      /* a HIP call failed */
} dflash_status;

typedef enum {
  DFLASH_F32 = 0,  /* float32 */
  DFLASH_BF16 = 1, /* bfloat16 */
  DFLASH_Q4G64 = 2 /* 4-bit affine, group 64 along the input dim (weights only, see below) */
} dflash_dtype;

/*
 * Drafter shape. All dimensions are positive and bounded so that every extent and
 * every element count fits an int32 (lablup/mlxcel #1762, Pre-merge review round, third
 * finding: dimensions that would wrap an i32 are refused).
 *   hidden, intermediate, q_heads*head_dim, target_streams*target_width: multiples of
 *     256 for bf16 weights (128 for f32) with a launch plan (every C1-style shape has
 *     one); hidden, intermediate, q/kv_heads*head_dim and vocab multiples of 16.
 *   head_dim: a multiple of 16, at most 128. q_heads a multiple of kv_heads.
 *   window W, 1..4096: keys at absolute position p are visible to a query at q iff
 *     |q - p| <= W (lablup/mlxcel #1762, What changed).
 *   max_block: largest block a draft may use, 1..256. The ring's slack is
 *     S = max(clamp(8*max_block, 32, 128), max_block) rows and its capacity C = W + S
 *     (lablup/mlxcel #1762, What changed; Pre-merge review round, second finding). The
 *     ring stores Cs = max(C, W + max_block + 1, 64) rounded up to a multiple of 8 slots
 *     per layer and kv head, so that the draft's own block rows have slots of their own
 *     past the window and attention reads 8-aligned runs of slots.
 *   mask_token_id: the token of the block's mask rows, in [0, vocab) (lablup/mlxcel
 *     #1751, Review fixes: the mask id indexes the target's embedding table).
 *   ring_phase: slot of absolute position p is (p + phi) mod Cs, with phi = ring_phase
 *     mod Cs rounded down to a multiple of 8. Nothing the calls return depends on it; it
 *     places the ring's wrap point (tests force wraps with it).
 *   weight_dtype: dtype of fc, every layer linear and the lm_head. With DFLASH_Q4G64
 *     the embedding table and the norm gains are bf16; otherwise they use weight_dtype.
 *   act_dtype: DFLASH_F32 with f32 weights, DFLASH_BF16 otherwise. It is the dtype of
 *     the residual slab, of every GEMM operand, of the ring and of lm_head input rows.
 *   variant: DFLASH_VARIANT_DFLASH (0) or DFLASH_VARIANT_DSPARK, the DSpark form of the
 *     drafter (lablup/mlxcel #1751, opening paragraph; Implementation Review Summary,
 *     Verified against the issue): a block of gamma rows [anchor, mask x (gamma-1)] whose
 *     every row proposes a token through a low-rank Markov token-transition head chained
 *     from the anchor (dflash_draft_block). A DSpark context takes max_block + 1 <= 32
 *     (the verify width clamp of the same page, Security fixes) and markov_rank in {64,
 *     128, 256} (also 512 with bf16 activations); a DFlash one takes markov_rank 0.
 *   rope_traditional: 0 pairs each head's elements (i, i + head_dim/2) in RoPE (the
 *     rotate-half form); 1 pairs neighbours (2i, 2i + 1), the DSpark checkpoints' form
 *     (same page, opening paragraph). Pair i turns by p * theta^(-2i/head_dim) either way.
 */
typedef struct {
  int32_t hidden, layers, q_heads, kv_heads, head_dim, intermediate, vocab;
  int32_t target_streams, target_width;
  int32_t window, max_block, mask_token_id, ring_phase;
  float rms_eps, rope_theta;
  int32_t weight_dtype; /* dflash_dtype */
  int32_t act_dtype;    /* dflash_dtype */
  int32_t variant;      /* dflash_variant */
  int32_t rope_traditional;
  int32_t markov_rank;
} dflash_config;

typedef enum { DFLASH_VARIANT_DFLASH = 0, DFLASH_VARIANT_DSPARK = 1 } dflash_variant;

/* A linear layer [out, in]. For DFLASH_Q4G64: w is uint32 [out, in/8] holding eight
 * 4-bit codes per word along the input dim, lowest nibble first; scales and biases are
 * bf16 [out, in/64]; the weight is scale*code + bias. Otherwise scales/biases are NULL. */
typedef struct {
  const void *w, *scales, *biases;
} dflash_linear;

typedef struct {
  dflash_linear q, k, v, o, gate, up, down;
  const void *in_norm, *post_norm; /* [hidden] */
  const void *q_norm, *k_norm;     /* [head_dim] */
} dflash_layer;

/* embed and lm_head are the target's raw embedding table [vocab, hidden] and untied
 * lm_head, shared with the drafter (lablup/mlxcel #1762, What changed). fc is
 * encoder.fc [hidden, target_streams*target_width]; enc_norm is encoder.output_norm_enc.
 * `layers` is a host array of cfg.layers entries; it is copied at create.
 * markov_w1 and markov_w2 (DSpark only, else NULL) are the Markov head's factors, both
 * [vocab, markov_rank] row-major in the embedding table's dtype: w1 is gathered at the
 * previous token and w2 maps that rank-r row to one logit per vocabulary entry
 * (lablup/mlxcel #1751, Security fixes). They are read in place (16-byte aligned, alive
 * while the context is). */
typedef struct {
  const void *embed;
  dflash_linear lm_head, fc;
  const void *enc_norm, *final_norm;
  const dflash_layer *layers;
  const void *markov_w1, *markov_w2;
} dflash_weights;

/* Bytes of ring (layers * 2 * kv_heads * Cs * head_dim * act element size), of workspace
 * and of packed weights a context with this config needs. Host only. */
dflash_status dflash_query_sizes(const dflash_config *cfg, size_t *ring_bytes, size_t *workspace_bytes,
                                 size_t *packed_bytes);

/* Validate cfg and the weight pointers, bind the caller's buffers and initialise the
 * workspace on `stream`. The drafter shares the target's raw embedding table and untied
 * lm_head by pointer (lablup/mlxcel #1762, What changed: the Drafter adapter binds the
 * target's raw embedding table and untied lm_head); config dimensions are bounded before
 * any device call (same page, Pre-merge review round, third finding). ring, workspace and packed must be at least the queried sizes and
 * 256-byte aligned. Every linear (fc, lm_head and the layer linears) is copied once into
 * `packed` in a fragment-major order: each 16-row x 16-byte-per-lane block of the matrix
 * becomes one contiguous kilobyte in the lane order of the MFMA operand, so that the
 * weight streams of every later call read whole contiguous kilobytes. The call
 * synchronises `stream`; afterwards the caller may free those row-major linears. The
 * embedding table and the norm gains are read in place and must stay alive; the linears
 * and the norm gains must be 16-byte aligned (DFLASH_E_ARG otherwise). The ring is
 * zero-filled and starts empty: e = 0, no pending rows. With rope_traditional the packed
 * q and k projections, and copies of q_norm and k_norm in `packed`, hold each head's
 * elements in the order (0, 2, 4, ..., 1, 3, 5, ...): the rotate-half rotation of that
 * order is the adjacent-pair rotation of the original one, and attention scores are
 * unchanged by a permutation shared by queries and keys, so every kernel runs one RoPE
 * form; the ring keeps keys in that order and dflash_cache_read restores the original. */
dflash_status dflash_create(const dflash_config *cfg, const dflash_weights *weights, void *ring,
                            size_t ring_bytes, void *workspace, size_t workspace_bytes, void *packed,
                            size_t packed_bytes, void *stream, dflash_ctx **out);

void dflash_destroy(dflash_ctx *ctx);

/*
 * Append n captured target residual rows (device, act_dtype, [n, target_streams *
 * target_width] row-major) at the next absolute positions. Each row goes through
 * encoder.fc and output_norm_enc, then every layer's k/v projection, k_norm and RoPE at
 * its position, and is written to its ring slot. commit = 0: the rows are pending until
 * dflash_cache_trim. commit != 0: all pending rows and these are committed now, and rows
 * that the committed window can no longer see are dropped before the encoder
 * (lablup/mlxcel #1762, Pre-merge review round, third finding). A pending append of a few
 * rows (bf16 shapes with head_dim 64 or 128, at most 14 rows) runs only encoder.fc here and
 * leaves the rest of the projection to the next call that needs the ring: the next
 * dflash_draft_block does it inside its own launches when its rows and the committed ones
 * fit, else that call, dflash_cache_read or the next append does it first, on its own
 * stream. The ring then holds the same values either way. Errors: n <= 0 or a NULL
 * slab ("no residual stream captured", lablup/mlxcel #1762, Pre-merge review round,
 * second finding).
 */
dflash_status dflash_cache_append(dflash_ctx *ctx, const void *resid, int32_t n, int32_t commit, void *stream);

/*
 * Commit the pending rows except the last m: e += pending - m, pending = 0. Host
 * bookkeeping only: the offsets rewind, no slot is restored (lablup/mlxcel #1762,
 * Pre-merge review round: RotatingKVCache::trim). After a round of block B with k
 * accepted, m = B - k (lablup/mlxcel #1751, Short-conv rollback: trim(block_size - n)
 * with n = accepted + 1). DFLASH_E_REWIND unless 0 <= m <= min(pending, slack).
 */
dflash_status dflash_cache_trim(dflash_ctx *ctx, int32_t m);

/*
 * Draft one block: rows [anchor, mask x block] at absolute positions e..e+block are
 * embedded with the raw table, run through every layer over the ring's committed context
 * and the block's own keys, and rows 1..block go through final_norm and the lm_head. The
 * layers are Qwen3-shaped and bidirectional (z-lab/dflash #168, Why: is_causal False);
 * each attends under |q - k| <= W over absolute positions, with per-head q/k norms, and the
 * embedding table and lm_head are the target's (lablup/mlxcel #1762, What changed); the
 * context K/V come from the cache with the block's own K/V after them (lablup/mlxcel
 * #1751, Implementation Review Summary).
 * The ring slots of positions e..e+block lie past the committed window: a layer may store
 * the block's own k/v there (f32 shapes do; dflash_cache_read never returns those slots and
 * the next append overwrites them), and of the committed window only rows whose projection
 * an append left to this call are written (their ring slots, once). d_tokens (device int32
 * [block]) receives the first index of each row's maximum f32 logit. d_hidden (device f32
 * [block+1, hidden], or NULL) receives the residual stream after the last layer. Errors:
 * block outside 1..max_block or anchor outside [0, vocab) (DFLASH_E_RANGE); NULL d_tokens
 * (DFLASH_E_ARG); e == 0 (DFLASH_E_NO_CONTEXT); pending rows (DFLASH_E_STATE).
 *
 * DSpark contexts (lablup/mlxcel #1751, Implementation Review Summary, Verified against the
 * issue): block = gamma proposals from gamma rows [anchor, mask x (gamma-1)] at positions
 * e..e+gamma-1, every row through final_norm and the lm_head (row 0 included), then the
 * Markov chain on the device: step i adds markov_w2 . markov_w1[t_i] to row i's logits
 * (t_0 = anchor, t_{i+1} = the step's token) and d_tokens[i] receives the first index of
 * the maximum, which the next step gathers; no host round trip inside the chain. The
 * DSpark backbone attends to every context row (no mask), which the window rule matches
 * while e + gamma - 1 <= window: a longer context is refused (DFLASH_E_RANGE) rather than
 * cut. d_hidden then has gamma rows.
 */
dflash_status dflash_draft_block(dflash_ctx *ctx, int32_t anchor, int32_t block, int32_t *d_tokens,
                                 float *d_hidden, void *stream);

/* argmax over the vocabulary of rows (device, act_dtype [n, hidden]) times the shared
 * lm_head, first index of the maximum f32 logit, into d_idx (device int32 [n]); the
 * target's verify rows use this (lablup/mlxcel #1762, What changed: lm_head_module, no
 * softcap). 1 <= n <= 4096. */
dflash_status dflash_lm_head_argmax(dflash_ctx *ctx, const void *rows, int32_t n, int32_t *d_idx, void *stream);

/* dflash_lm_head_argmax without any device allocation, for callers that cannot allocate
 * device memory at the call (code under HIP graph capture, tight serving loops, harnesses
 * that forbid it). Same rows, output and result as dflash_lm_head_argmax; its per-work-group
 * argmax keys go to a fixed 4 MiB device array of the library (one copy per GPU, held until
 * the process ends) instead of the context's workspace, so nothing is allocated or freed.
 * Every call on one GPU shares that array: calls that overlap on one GPU (several streams or
 * host threads) race on it. Call with the context's device current. Errors: as
 * dflash_lm_head_argmax; DFLASH_E_SHAPE (nothing enqueued) if the vocabulary needs more keys
 * than the array holds (above 524288 rows); DFLASH_E_ARG if another device is current. */
dflash_status dflash_lm_head_argmax_noalloc(dflash_ctx *ctx, const void *rows, int32_t n, int32_t *d_idx,
                                            void *stream);

/* Kernel timing of the vocabulary argmax (profiling; no counterpart on the pages). The next
 * dflash_lm_head_argmax call on ctx records `start` on its stream right before its first
 * argmax GEMM launch (rows 0..31) and `end` right after it, before the per-row reduction
 * of the work-group maxima, so the elapsed time between the two is that one kernel's
 * duration; the call then forgets both. start and end are hipEvent_t handles created by
 * the caller with timing enabled and owned by it. Passing two NULLs cancels a pending
 * request. Errors: NULL ctx, or exactly one NULL event (DFLASH_E_ARG). */
dflash_status dflash_time_next_argmax(dflash_ctx *ctx, void *start, void *end);

/* Kernel timing of the DSpark Markov chain (profiling; no counterpart on the pages). The
 * next dflash_draft_block call on a DSpark context records `start` on its stream right
 * before the first chain step and `end` right after the last, so the elapsed time is the
 * gamma step launches back to back; the call then forgets both. Events as for
 * dflash_time_next_argmax. Errors: NULL ctx, exactly one NULL event, or a DFlash context
 * (DFLASH_E_ARG). */
dflash_status dflash_time_next_chain(dflash_ctx *ctx, void *start, void *end);

/* HBM streaming-read probe (measurement; no counterpart on the pages): `groups` work-groups
 * each read a contiguous share of `bytes` from src (device, 16-byte aligned, bytes a multiple
 * of 16 and at least groups * 4096) with 16-byte non-temporal loads and write the XOR of what
 * they read to sink (device uint32 [groups]). Timed by the caller, it gives the practical read
 * bandwidth the weight streams are compared with. Context-free; errors go to
 * dflash_last_error(NULL): DFLASH_E_ARG for the conditions above, DFLASH_E_DEVICE. */
dflash_status dflash_hbm_read_probe(const void *src, size_t bytes, uint32_t *sink, int32_t groups, void *stream);

/*
 * Greedy exact-match verify of one block (lablup/mlxcel #1751, Implementation Review
 * Summary: greedy exact-match verify rule, verify width = block + 1). d_draft: device
 * int32 [block] = d_1..d_block; d_target: device int32 [block+1] = the target's argmax
 * at verify rows e..e+block. d_out (int32 [3]: device memory, or pinned host memory from
 * hipHostMalloc, which the kernel then writes directly) receives k = the number of leading
 * rows with d_{i+1} == a_i (0..block), the bonus token a_k, and a status word: 0, or 1
 * if any target id lies outside [0, vocab) (then k = 0 and bonus = -1).
 */
dflash_status dflash_verify_greedy(dflash_ctx *ctx, const int32_t *d_draft, const int32_t *d_target,
                                   int32_t block, int32_t *d_out, void *stream);

/*
 * Adaptive verify width (host only). A drafter whose declared depth lies below the requested
 * width runs the round loop under a throughput controller between the two: it warms up at the
 * depth and widens to the ceiling only when a measured window pays for it; the widths a run
 * can settle on are the depth and the ceiling (lablup/mlxcel #1762, What changed, "Round
 * loop"; Pre-merge review round, first finding). The measure is committed tokens per
 * millisecond over a window of rounds (same page, Real-checkpoint validation, item 5).
 * Schedule: windows of `window` rounds at the incumbent width (first the depth); after every
 * `challenge_every` of them one window at the other width, adopted (the two swap roles) only
 * if its rate is strictly above the incumbent's rate over its whole measurement period since
 * the last challenge; a new period then starts from the adopted window, or empty. A drafter context
 * serving these widths needs max_block >= ceiling (its slack is sized for the ceiling).
 *   create: 1 <= depth <= ceiling, window >= 1, challenge_every >= 1 (DFLASH_E_RANGE).
 *   width: the block of the next round (0 for a NULL controller).
 *   record: one finished round at `block` (must equal width(), else DFLASH_E_STATE) that
 *     committed `committed` >= 1 tokens (accepted + bonus) in `ms` > 0 milliseconds
 *     (DFLASH_E_RANGE otherwise); on error the controller is unchanged.
 *   state: the incumbent and challenger widths, whether the next round is a challenge, the
 *     incumbent's period rate and the latest challenge rate (-1 before the first), and
 *     how many challenges ran and were adopted. Any output may be NULL.
 */
typedef struct dflash_width_ctl dflash_width_ctl;
dflash_status dflash_width_ctl_create(int32_t depth, int32_t ceiling, int32_t window, int32_t challenge_every,
                                      dflash_width_ctl **out);
int32_t dflash_width_ctl_width(const dflash_width_ctl *ctl);
dflash_status dflash_width_ctl_record(dflash_width_ctl *ctl, int32_t block, int32_t committed, double ms);
dflash_status dflash_width_ctl_state(const dflash_width_ctl *ctl, int32_t *incumbent, int32_t *challenger,
                                     int32_t *challenging, double *incumbent_rate, double *challenge_rate,
                                     int64_t *challenges, int64_t *adoptions);
void dflash_width_ctl_destroy(dflash_width_ctl *ctl);

/*
 * The target side of the round: the verify forward of a causal target that shares its raw
 * embedding table and untied lm_head with the drafter and hands the drafter its residual
 * streams (lablup/mlxcel #1762, What changed, "Muse target": residual-stream capture before
 * the final norm, trim rollback over the mixed caches, sliding caches armed with the
 * drafter's slack rule; lablup/mlxcel #1751, opening paragraph: the verify forward with
 * residual-stream capture, a drafter fed five of the target's residual streams).
 *
 * Layers are Qwen3-shaped (RMSNorm, q/k/v, per-head q/k RMSNorm, neox RoPE, attention, o +
 * residual, RMSNorm, SwiGLU, down + residual); a final RMSNorm and the lm_head follow. A
 * query at absolute position q sees the keys p <= q, and on a sliding layer only q - window <
 * p (the last `window` positions, itself included). Sliding caches hold window + S slots with
 * S = max(clamp(8*max_block, 32, 128), max_block); full-attention caches hold max_context.
 *   hidden, intermediate, q_heads*head_dim, vocab, head_dim, dtypes: as dflash_config.
 *   full_mask: bit l set = layer l attends to every earlier position (layers <= 64).
 *   capture_layers[0..n_capture-1]: strictly increasing layer ids (1..8 of them) whose
 *     residual stream, after the layer and before the final norm, is captured; the captured
 *     row is the concatenation in this order, [n_capture * hidden], in act_dtype.
 *   window 1..4096; max_context 64..4096 (positions a full layer can hold; every forward
 *     must end at or before it when a full layer exists); max_block 1..64 (forwards take at
 *     most max(max_block + 1, 32) rows).
 */
typedef struct {
  int32_t hidden, layers, q_heads, kv_heads, head_dim, intermediate, vocab;
  int32_t window, max_context, max_block;
  uint64_t full_mask;
  int32_t n_capture, capture_layers[8];
  float rms_eps, rope_theta;
  int32_t weight_dtype, act_dtype;
} dflash_target_config;

/* embed and lm_head: the table and lm_head the drafter binds (the same device buffers may
 * serve both); layers: a host array of cfg.layers entries (copied at create). */
typedef struct {
  const void *embed;
  dflash_linear lm_head;
  const void *final_norm;
  const dflash_layer *layers;
} dflash_target_weights;

typedef struct dflash_target dflash_target; /* opaque */

/* Bytes of caches, workspace and packed weights a target with this config needs. */
dflash_status dflash_target_query_sizes(const dflash_target_config *cfg, size_t *cache_bytes,
                                        size_t *workspace_bytes, size_t *packed_bytes);

/* As dflash_create: validate, bind the caller's buffers (256-byte aligned, at least the
 * queried sizes), repack the lm_head and layer linears into `packed`, zero the caches, and
 * synchronise `stream`. The target starts empty: e = 0, no pending rows. */
dflash_status dflash_target_create(const dflash_target_config *cfg, const dflash_target_weights *weights,
                                   void *cache, size_t cache_bytes, void *workspace, size_t workspace_bytes,
                                   void *packed, size_t packed_bytes, void *stream, dflash_target **out);
void dflash_target_destroy(dflash_target *t);

/*
 * One forward over n rows [anchor, d_tokens[0], .., d_tokens[n-2]] at absolute positions
 * e..e+n-1: the verify rows of a round (anchor and the drafted tokens), or a chunk of a prompt.
 * Their keys and values are appended to every layer's cache as pending rows. d_tokens:
 * device int32 [n-1] (ids are clamped into [0, vocab)); d_argmax (device int32 [n]) receives
 * the first index of each row's maximum f32 logit through final_norm and the lm_head;
 * d_capture (device act_dtype [n, n_capture * hidden], or NULL) the captured residual
 * streams, which dflash_cache_append takes as the drafter's input rows. Errors: n outside
 * 1..max rows or anchor outside [0, vocab) (DFLASH_E_RANGE), a full layer that would pass
 * max_context (DFLASH_E_RANGE), pending rows (DFLASH_E_STATE), NULL d_argmax or a NULL
 * d_tokens with n > 1 (DFLASH_E_ARG).
 */
dflash_status dflash_target_forward(dflash_target *t, int32_t anchor, const int32_t *d_tokens, int32_t n,
                                    int32_t *d_argmax, void *d_capture, void *stream);

/* Commit the pending rows except the last m (attention caches trim by block - n with n =
 * accepted + 1: lablup/mlxcel #1751, Implementation Review Summary). Host bookkeeping;
 * DFLASH_E_REWIND unless 0 <= m <= min(pending, S). */
dflash_status dflash_target_trim(dflash_target *t, int32_t m);

/* Committed end e, pending rows and slack S. Host only. */
dflash_status dflash_target_state(const dflash_target *t, int64_t *e, int32_t *pending, int32_t *slack);

/* The committed keys and values the next query (at e) sees on one layer, in position order:
 * positions max(0, e - window + 1)..e-1 on a sliding layer, 0..e-1 on a full one, into k_out
 * and v_out (device act_dtype [kv_heads, n, head_dim]); *n_out = n. */
dflash_status dflash_target_cache_read(dflash_target *t, int32_t layer, void *k_out, void *v_out, int32_t *n_out,
                                       void *stream);

const char *dflash_target_last_error(const dflash_target *t);

/* Committed end e, pending rows, slack S and capacity C. Host only. */
dflash_status dflash_cache_state(const dflash_ctx *ctx, int64_t *e, int32_t *pending, int32_t *slack,
                                 int32_t *capacity);

/* Copy one layer's live window, positions max(0, e-W)..e-1 in position order, into
 * k_out and v_out (device, act_dtype [kv_heads, n, head_dim], at least kv_heads * min(e, W)
 * * head_dim elements each); *n_out = n (host). Keys come out in the original element
 * order whatever the RoPE form. Rows whose K/V an append deferred are projected into the
 * ring first. Errors: NULL n_out, k_out or v_out, or a layer outside 0..layers-1 (nothing
 * enqueued). */
dflash_status dflash_cache_read(dflash_ctx *ctx, int32_t layer, void *k_out, void *v_out, int32_t *n_out,
                                void *stream);

/*
 * Independent sequences drafted together (B > 1 requests; the pages' Muse pairing declines
 * them, lablup/mlxcel #1762, Not in this PR, and the LFM2 pairing is batch 1 as well,
 * lablup/mlxcel #1751, Review fixes). A batch holds n_seq sequences of one drafter config,
 * each with its own ring, committed end e_s and pending rows; nothing couples two
 * sequences, so sequence s computes exactly what a dflash_ctx fed the same calls computes.
 * One round drafts every sequence at the same block width; accept lengths, and so trims
 * and contexts, differ per sequence. Every GEMM of a round runs once over the rows of all
 * sequences (each weight byte is read once per round for the batch); the rest runs per
 * sequence. The DFlash form only (variant 0); 1 <= n_seq <= 64 and n_seq * (max_block + 1)
 * <= 512 (DFLASH_E_RANGE otherwise). Conventions as for dflash_ctx; per-sequence host
 * arrays have n_seq entries.
 */
typedef struct dflash_batch dflash_batch; /* opaque */

/* Ring bytes for all sequences (n_seq rings of the single-sequence size, back to back),
 * workspace and packed bytes. Host only. */
dflash_status dflash_batch_query_sizes(const dflash_config *cfg, int32_t n_seq, size_t *ring_bytes,
                                       size_t *workspace_bytes, size_t *packed_bytes);

/* As dflash_create, for n_seq sequences (every ring empty). */
dflash_status dflash_batch_create(const dflash_config *cfg, int32_t n_seq, const dflash_weights *weights,
                                  void *ring, size_t ring_bytes, void *workspace, size_t workspace_bytes, void *packed,
                                  size_t packed_bytes, void *stream, dflash_batch **out);
void dflash_batch_destroy(dflash_batch *b);

/* Append captured residual rows: resid (device, act_dtype [sum(counts), F]) holds sequence
 * 0's counts[0] rows, then sequence 1's, ...; counts (host) may hold zeros. Per sequence as
 * dflash_cache_append (commit, drop before the encoder); pending appends of at most C rows
 * per sequence run the encoder and K/V projections once over all rows. Errors: NULL resid
 * or counts, a negative count, or no rows at all (DFLASH_E_ARG). */
dflash_status dflash_batch_append(dflash_batch *b, const void *resid, const int32_t *counts, int32_t commit,
                                  void *stream);

/* Per sequence: commit the pending rows except the last m[s] (host array). All legal or
 * nothing changes (DFLASH_E_REWIND). */
dflash_status dflash_batch_trim(dflash_batch *b, const int32_t *m);

/* One block of `block` drafted tokens for every sequence: sequence s runs rows [anchors[s],
 * mask x block] at its positions e_s..e_s+block over its own ring (dflash_draft_block).
 * anchors: host int32 [n_seq]; d_tokens: device int32 [n_seq][block]; d_hidden: device f32
 * [n_seq][block+1][hidden] or NULL. Errors as dflash_draft_block, for any sequence. */
dflash_status dflash_batch_draft(dflash_batch *b, const int32_t *anchors, int32_t block, int32_t *d_tokens,
                                 float *d_hidden, void *stream);

/* dflash_lm_head_argmax on the batch's lm_head (rows of any sequences, 1 <= n <= 4096). */
dflash_status dflash_batch_lm_head_argmax(dflash_batch *b, const void *rows, int32_t n, int32_t *d_idx, void *stream);

/* dflash_verify_greedy of every sequence in one launch: d_draft [n_seq][block], d_target
 * [n_seq][block+1], d_out [n_seq][3] (device or pinned host memory). */
dflash_status dflash_batch_verify_greedy(dflash_batch *b, const int32_t *d_draft, const int32_t *d_target,
                                         int32_t block, int32_t *d_out, void *stream);

/* Sequence seq's committed end and pending rows (host only; DFLASH_E_RANGE for a bad seq). */
dflash_status dflash_batch_state(const dflash_batch *b, int32_t seq, int64_t *e, int32_t *pending);

/* dflash_cache_read of sequence seq's ring. */
dflash_status dflash_batch_cache_read(dflash_batch *b, int32_t seq, int32_t layer, void *k_out, void *v_out,
                                      int32_t *n_out, void *stream);

const char *dflash_batch_last_error(const dflash_batch *b);

/* Description of the last error on ctx (never NULL), and of a status code. */
const char *dflash_last_error(const dflash_ctx *ctx);
const char *dflash_status_string(dflash_status s);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
