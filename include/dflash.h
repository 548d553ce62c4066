/*
 * dflash.h -- C ABI of the MI355X (gfx950) DFlash drafter library.
 *
 * One parallel forward pass of the DFlash block-diffusion drafter, as the
 * pages describe it:
 *   [W] "DFlash: Block Diffusion for Flash Speculative Decoding" (wikillm
 *       summary: "Method" > Inference, "Paper vs code", and its decoding-loop
 *       and draft-layer pseudocode);
 *   [R] "DFlash: Why a Diffusion Drafter Can Accelerate an Autoregressive
 *       Model" (technical review: sec. 4.1, sec. 5.1 eqs. 9-10, sec. 5.3).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every tensor argument is CALLER-OWNED DEVICE MEMORY on the current HIP
 *    device. The library never allocates or frees device memory; it reads
 *    and writes the buffers it is given, and a handle keeps the weight
 *    pointers of dflash_create. Scratch space comes from the caller's
 *    workspace.
 *  - Every compute call takes the caller's stream (a hipStream_t passed as
 *    void*) and is asynchronous on it: it enqueues kernels and returns; it
 *    never synchronises the device. Results are valid once the stream reaches
 *    that point.
 *  - Weights are given row-major [out, in] (the Linear layout), all in the
 *    model dtype (DFLASH_BF16 or DFLASH_FP32), norm gains included; the
 *    projections are read from a tiled copy the caller has
 *    dflash_pack_weights write once (see there).
 *  - Every device pointer must be 16-byte aligned.
 *  - Return value: DFLASH_OK (0) or a negative dflash_status. Arguments are
 *    validated on the host before anything is enqueued; a call that returns an
 *    error has enqueued nothing (except DFLASH_ERR_HIP, which reports a launch
 *    failure after earlier launches of the same call may have been enqueued).
 *  - Conditions only the device can see (a context longer than the cache
 *    capacity, a token id outside the vocabulary, inconsistent prefix offsets)
 *    are clamped so that nothing is written out of bounds, and the matching
 *    DFLASH_DEV_* bit is OR-ed into *dev_status when dev_status is non-NULL.
 *  - A handle is immutable after dflash_create; concurrent calls with one
 *    handle on different streams are safe when their workspaces and output
 *    buffers differ.
 *
 * Departures from a plain row-major interface (both for the matrix cores'
 * operand order; see dflash_kv_cache and dflash_pack_weights)
 * ---------------------------------------------------------------------
 *  - The V cache is not [capacity][head_dim] per (layer, sequence, KV head)
 *    but [capacity/32][head_dim][32]: positions in blocks of 32, channel-major
 *    inside a block. The K cache is plain [capacity][head_dim].
 *  - The projections are not read from the caller's row-major matrices in
 *    place: dflash_pack_weights writes a tiled copy once (3.42 GB for a
 *    Qwen3-8B-shaped drafter) into a caller buffer, and every call reads that.
 *    The embedding table and the norm gains are read in place.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dflash_status {
  DFLASH_OK = 0,
  DFLASH_ERR_NULL = -1,          /* a required pointer is NULL */
  DFLASH_ERR_SHAPE = -2,         /* a size is out of range or inconsistent */
  DFLASH_ERR_DTYPE = -3,         /* unknown dtype */
  DFLASH_ERR_ALIGN = -4,         /* a pointer or stride breaks 16-byte alignment */
  DFLASH_ERR_WORKSPACE = -5,     /* workspace or packed buffer smaller than its size query */
  DFLASH_ERR_UNSUPPORTED = -6,   /* a configuration the kernels do not cover */
  DFLASH_ERR_HIP = -7,           /* a HIP launch reported an error */
  DFLASH_ERR_STATE = -8,         /* profiler misuse, or graph capture while it records */
  DFLASH_ERR_SCRATCH = -9        /* request larger than the library's static scratch */
} dflash_status;

typedef enum dflash_dtype { DFLASH_FP32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

/* Bits OR-ed into *dev_status by kernels that detect bad device-side data. */
#define DFLASH_DEV_CAPACITY 1   /* ctx_len + new rows (or + block) exceeds capacity: rows dropped */
#define DFLASH_DEV_TOKEN 2      /* a token id outside [0, vocab): clamped */
#define DFLASH_DEV_OFFSETS 4    /* cu_new not monotone or not ending at n_tok: rows dropped */

/* Drafter shape. Supported: head_dim 64 or 128; n_heads a multiple of
 * n_kv_heads with n_heads/n_kv_heads <= 8; 1 <= block_size <= 16;
 * 1 <= n_layers <= 16; hidden, intermediate, n_heads*head_dim and
 * target_hidden multiples of 32 (bf16) / 16 (fp32); vocab >= 2.
 * rope_theta <= 0 disables the rotary embedding. */
typedef struct dflash_config {
  int32_t hidden;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t n_layers;
  int32_t intermediate;
  int32_t n_target_feats;   /* number of target layers whose features are fused */
  int32_t target_hidden;    /* width of each target feature */
  int32_t vocab;
  int32_t block_size;       /* B: anchor + B-1 mask slots */
  int32_t mask_token_id;
  int32_t dtype;            /* dflash_dtype */
  float rms_eps;
  float rope_theta;
  /* Sliding-window layers [W "Paper vs code", attention-pattern bullet: the
   * reference code supports per-layer sliding-window attention]: layer l
   * with bit l of sliding_layer_mask set lets block query i (position
   * ctx_len + i) see key position p only when ctx_len + i - p < sliding_window;
   * other layers attend to every position. mask 0: no sliding layer (window
   * ignored); otherwise window >= 1 and no bit at or above n_layers. */
  int32_t sliding_window;
  uint32_t sliding_layer_mask;
} dflash_config;

/* One draft layer. Shapes (d = hidden, hd = head_dim, I = intermediate):
 * in_norm/post_norm [d]; wq [n_heads*hd, d]; wk, wv [n_kv_heads*hd, d];
 * q_norm, k_norm [hd]; wo [d, n_heads*hd]; w_gate, w_up [I, d]; w_down [d, I]. */
typedef struct dflash_layer_weights {
  const void *in_norm, *wq, *wk, *wv, *q_norm, *k_norm, *wo, *post_norm;
  const void *w_gate, *w_up, *w_down;
} dflash_layer_weights;

/* embed, lm_head [vocab, d] (may alias); fc [d, n_target_feats*target_hidden];
 * fc_norm, final_norm [d]; layers: host array of n_layers entries (copied by
 * dflash_create).
 * packed: the tiled copy of the projection weights that dflash_pack_weights
 * wrote for this configuration and these weights (packed_bytes: its size,
 * at least dflash_packed_weight_bytes). Every projection (wq, wk, wv, wo,
 * w_gate, w_up, w_down, fc, lm_head) is read from it, never from the row-major
 * matrices; embed, the norm gains and packed are read by every call and must
 * outlive the handle. dflash_create checks packed's size and alignment, not
 * its content. */
typedef struct dflash_weights {
  const void *embed, *lm_head, *fc, *fc_norm, *final_norm;
  const dflash_layer_weights *layers;
  const void *packed;
  int64_t packed_bytes;
} dflash_weights;

/* Per-layer context K/V cache, caller-owned, model dtype.
 *   k: [n_layers][batch][n_kv_heads][capacity][head_dim]   (row per position)
 *   v: [n_layers][batch][n_kv_heads][capacity/32][head_dim][32]
 *      (positions grouped in blocks of 32; inside a block the 32 positions of
 *      one channel are contiguous, so attention reads V channel-major)
 *   ctx_len: device int32 [batch], number of valid positions per sequence.
 * capacity must be a multiple of 32. Positions [ctx_len, ctx_len+block_size)
 * are scratch for the draft forward, so a forward needs
 * ctx_len + block_size <= capacity. */
typedef struct dflash_kv_cache {
  void *k;
  void *v;
  int32_t *ctx_len;
  int32_t batch;
  int32_t capacity;
} dflash_kv_cache;

typedef struct dflash_handle dflash_handle;

/* Tiled weight copy. The projections stream their weights from one copy in
 * the order the matrix-core loop consumes them: rows in tiles of 16, the
 * input dimension in chunks of 256 bytes, and inside each (row tile, chunk)
 * four 1 KB fragments, fragment f holding for lane l = r + 16 g the 16 bytes
 * of row r at element 16*EPF*c + 4*EPF*f + EPF*g (EPF = 8 for bf16, 4 for
 * fp32), zero-padded to whole tiles and chunks. Every load of a wave then
 * reads one contiguous kilobyte. The copy holds, per layer, [wq; wk; wv]
 * stacked, wo, w_gate, w_up, w_down; then fc; then every layer's [wk; wv]
 * stacked (the context K/V projection); then lm_head.
 *
 * dflash_packed_weight_bytes: bytes of the copy for cfg (negative
 * dflash_status on a bad cfg).
 * dflash_pack_weights: enqueue on stream the kernels that write the copy of
 * w's projections into packed (caller-owned device memory of packed_bytes
 * bytes). Reads lm_head, fc and each layer's wq, wk, wv, wo, w_gate, w_up,
 * w_down; once stream has passed the call, those row-major matrices are no
 * longer needed by the library. Errors: DFLASH_ERR_NULL / _ALIGN for a
 * missing or misaligned matrix or packed, DFLASH_ERR_WORKSPACE when
 * packed_bytes is too small, config errors as dflash_create. */
int64_t dflash_packed_weight_bytes(const dflash_config *cfg);
int32_t dflash_pack_weights(const dflash_config *cfg, const dflash_weights *w, void *packed,
                            int64_t packed_bytes, void *stream);

/* Validate the shape and keep a copy of the weight pointers (no device work:
 * packed must already hold dflash_pack_weights' output before the first call
 * that uses the handle runs). Needs embed, fc_norm, final_norm, packed and
 * each layer's in_norm, q_norm, k_norm, post_norm; the row-major projection
 * pointers may be NULL. DFLASH_ERR_WORKSPACE when packed_bytes is too small.
 * Returns DFLASH_OK and *out, or an error with *out = NULL. */
int32_t dflash_create(const dflash_config *cfg, const dflash_weights *w, dflash_handle **out);
void dflash_destroy(dflash_handle *h);

/* Bytes of workspace that every call below needs when batch <= max_batch,
 * capacity <= the given capacity and n_tok <= max_tokens (ctx_project and
 * ctx_kv_append). Returns a negative dflash_status on bad arguments. */
int64_t dflash_workspace_bytes(const dflash_handle *h, int32_t max_batch, int32_t capacity,
                               int32_t max_tokens);

/* Target-context-feature fusion [R eq. 9; W "Method" step 1]:
 *   ctx = RMSNorm(fc · concat(feats[0..n_target_feats-1]); fc_norm).
 * feats: HOST array of n_target_feats device pointers, each [n_tok, target_hidden]
 *        with a row stride of feat_row_stride ELEMENTS (multiple of 8).
 * ctx_out: [n_tok, hidden], model dtype. n_tok >= 0 (0 is a no-op). */
int32_t dflash_ctx_project(const dflash_handle *h, const void *const *feats,
                           int64_t feat_row_stride, int32_t n_tok, void *ctx_out, void *ws,
                           int64_t ws_bytes, void *stream);

/* Context K/V injection [R eq. 10; W "Paper vs code" KV-injection bullet]:
 * for every layer l and every new context row r of sequence s,
 *   K = RoPE(headRMS(ctx_r · wk_l^T; k_norm_l), pos),  V = ctx_r · wv_l^T,
 * stored at pos = ctx_len[s] + (r - cu_new[s]); afterwards
 * ctx_len[s] += cu_new[s+1] - cu_new[s].
 * ctx: [n_tok, hidden] model dtype (rows of all sequences, packed in order);
 * cu_new: DEVICE int32 [cache->batch + 1] prefix offsets, cu_new[0] = 0,
 *         cu_new[batch] = n_tok. */
int32_t dflash_ctx_kv_append(const dflash_handle *h, const dflash_kv_cache *cache,
                             const void *ctx, const int32_t *cu_new, int32_t n_tok,
                             int32_t *dev_status, void *ws, int64_t ws_bytes, void *stream);

/* The same injection for the rows of a verified block, with the row count
 * taken on the device [W decoding-loop pseudocode: the accepted tokens' target
 * features join the context before the next round; R sec. 4.1]: for every
 * sequence s < cache->batch, rows s*B + i of ctx with i <= accept_len[s] (the
 * anchor and the accepted candidates) are stored at pos = ctx_len[s] + i, then
 * ctx_len[s] += accept_len[s] + 1. No host-side count, so a round built on it
 * has fixed shapes (it can be captured in a HIP graph).
 * ctx: [cache->batch * B, hidden] model dtype: the block positions of every
 *      sequence (dflash_ctx_project over cache->batch * B rows);
 * accept_len: DEVICE int32 [cache->batch], values in [0, B-1] (dflash_accept's
 *      output); a value outside is clamped and flags DFLASH_DEV_OFFSETS. */
int32_t dflash_ctx_kv_append_accepted(const dflash_handle *h, const dflash_kv_cache *cache,
                                      const void *ctx, const int32_t *accept_len,
                                      int32_t *dev_status, void *ws, int64_t ws_bytes,
                                      void *stream);

/* One parallel drafter pass over batch sequences [W decoding-loop and
 * draft-layer pseudocode; "Method" steps 2-3]:
 *   block = [anchor[s], MASK x (B-1)] embedded with `embed`;
 *   n_layers x { pre-norm, QKV, per-head q/k RMSNorm + RoPE at ctx_len[s]+i,
 *                non-causal attention over [cached context ; block] K/V,
 *                O + residual, post-norm, SwiGLU MLP + residual };
 *   final RMSNorm of slots 1..B-1, LM head, greedy argmax (lowest id on ties).
 * The cache is read; its scratch positions [ctx_len, ctx_len+B) are
 * overwritten; ctx_len is not changed.
 * anchor: device int32 [batch]; batch <= cache->batch.
 * draft_tokens: device int32 [batch, B-1] (required).
 * logits: optional fp32 [batch, B-1, vocab].
 * hidden_out: optional fp32 [batch, n_layers, B, hidden]: residual stream
 *             after each layer.
 * target_tokens: optional device int32 [batch, B]; when given, accept_len and
 *             bonus (device int32 [batch]) receive dflash_accept's result.
 *             bonus may alias anchor: the anchor is read before the bonus is
 *             written, so the bonus becomes the next round's anchor in place. */
int32_t dflash_draft_forward(const dflash_handle *h, const dflash_kv_cache *cache,
                             const int32_t *anchor, int32_t batch, int32_t *draft_tokens,
                             float *logits, float *hidden_out, const int32_t *target_tokens,
                             int32_t *accept_len, int32_t *bonus, int32_t *dev_status,
                             void *ws, int64_t ws_bytes, void *stream);

/* Training-pattern attention of packed blocks [W "Training" step 4 and the
 * training-loss pseudocode; R sec. 6.1]: the blocks drawn from one sequence
 * are trained together; a block anchored at position a (its B positions at
 * a .. a+B-1) attends, in both directions, to its own B keys and to the
 * target's context features at positions 0 .. a-1 (the anchor's own feature
 * is not used, as when drafting, where the context ends right before the
 * anchor), never to another block. One call covers one layer.
 *   cache, layer: the context K/V of every sequence in the drafting cache
 *        layout (dflash_kv_cache), e.g. written by dflash_ctx_kv_append over
 *        the sequence's fused features; sequence s reads cache row s, whose
 *        ctx_len[s] must cover its anchors.
 *   n_seq <= cache->batch sequences of blocks_per_seq blocks each; block
 *        b = s * blocks_per_seq + j.
 *   anchors: device int32 [n_seq * blocks_per_seq]; an anchor outside
 *        [0, min(ctx_len[s], capacity)] is clamped and flags DFLASH_DEV_CAPACITY.
 *   q: [n_blk][B][n_heads][head_dim], the blocks' queries after q-norm and
 *        rotation at their positions; k_blk, v_blk: [n_blk][B][n_kv_heads]
 *        [head_dim] likewise (keys rotated); out: [n_blk][B][n_heads][head_dim].
 *        All in the config's dtype, 16-byte aligned, caller-owned device memory.
 * Scale 1/sqrt(head_dim); query head j reads KV head j / (n_heads / n_kv_heads).
 * Errors (nothing enqueued): DFLASH_ERR_NULL, _ALIGN, _SHAPE (layer or counts
 * out of range, n_seq > cache->batch), as for the cache in
 * dflash_draft_forward; DFLASH_ERR_HIP on a launch failure. */
int32_t dflash_packed_block_attention(const dflash_handle *h, const dflash_kv_cache *cache,
                                      int32_t layer, int32_t n_seq, int32_t blocks_per_seq,
                                      const int32_t *anchors, const void *q, const void *k_blk,
                                      const void *v_blk, void *out, int32_t *dev_status,
                                      void *stream);

/* Greedy accept-prefix [W decoding-loop pseudocode; R sec. 4.1]:
 *   accept_len[s] = number of leading i < B-1 with draft[s][i] == target[s][i],
 *   bonus[s] = target[s][accept_len[s]]; anchor_out (optional) = bonus.
 * draft_tokens [batch, B-1], target_tokens [batch, B], all device int32. */
int32_t dflash_accept(const int32_t *draft_tokens, const int32_t *target_tokens, int32_t batch,
                      int32_t block_size, int32_t *accept_len, int32_t *bonus,
                      int32_t *anchor_out, void *stream);

/* Temperature > 0: drafting by sampling and speculative verification with
 * residual resampling [R sec. 4.2 eqs. 6-8 and its Algorithm 1; W "Paper vs
 * code": above temperature 0 the reference code verifies by rejection
 * sampling with residual resampling]. p and q are softmax(logits / T) of the
 * target's and the draft's logits at the same temperature T > 0 (no top-p /
 * top-k filtering).
 *
 * Random numbers: Philox4x32-10 (Salmon et al., "Parallel random numbers: as
 * easy as 1, 2, 3", SC 2011) with key (low, high 32 bits of seed). Element i
 * of a (row, round, stream) triple is word i % 4 of the block at counter
 * (i / 4, row, round, stream) (each word 32 bits, so round is taken modulo
 * 2^32); a uniform is ((w >> 9) + 0.5) * 2^-23. Streams: 0 drafting (row =
 * the logits row), 1 acceptance tests (row = sequence, element = position),
 * 2 correction / bonus draws (row = sequence * block_size + position).
 * A categorical draw is the Gumbel-max argmax of log-probability +
 * (-log(-log u)) over the support, lowest index on ties.
 *
 * dflash_sampling_workspace_bytes: workspace bytes that both calls below need
 * for up to `batch` sequences of `block_size` (dflash_sample_drafts with
 * rows <= batch * (block_size - 1)). Negative dflash_status on bad sizes.
 *
 * dflash_sample_drafts: tokens[r] ~ softmax(logits[r] / T) for r < rows
 * (stream 0, row r); logq[r] (optional) = log q(tokens[r]).
 * logits: fp32 device [rows, row_stride >= vocab] -- for the drafter's
 * candidates, dflash_draft_forward's logits output ([batch * (B-1), vocab]).
 *
 * dflash_verify_sampled: per sequence s, candidates drafts[s][0..B-2] are
 * scanned left to right; candidate i is accepted when u_i < min(1,
 * p_i(y) / q_i(y)) (eq. 6). accept_len[s] = the number accepted before the
 * first rejection; out_token[s] = a draw from the residual [p - q]_+ at the
 * first rejected position (eq. 7; from p if that support is empty), or, when
 * all B-1 are accepted, the bonus token drawn from the target's law at
 * position B-1. anchor_out (optional) receives out_token (the next anchor).
 * drafts: int32 [batch, B-1]; draft_logits: fp32 [batch, B-1, vocab] (the
 * logits the candidates were drawn from); draft_logq (optional, may be null):
 * fp32 [batch, B-1], log q_i(drafts[s][i]) as dflash_sample_drafts returned
 * it for these rows at this temperature -- when given, each draft row's
 * normaliser is recovered from it (logit / T - log q of the drawn token)
 * instead of by a pass over the draft rows, which halves the bytes read;
 * target_logits: fp32
 * [batch, B, vocab] (the target's logits at the B-1 candidate positions and
 * the position after them). round separates the random numbers of
 * successive rounds. Candidate ids outside [0, vocab) are clamped.
 * Errors (before anything is enqueued): DFLASH_ERR_NULL, DFLASH_ERR_ALIGN,
 * DFLASH_ERR_SHAPE (T not finite and > 0, vocab < 2, block_size outside
 * 2..17, negative sizes, row_stride < vocab), DFLASH_ERR_WORKSPACE. */
int64_t dflash_sampling_workspace_bytes(int32_t batch, int32_t block_size, int32_t vocab);
int32_t dflash_sample_drafts(const float *logits, int64_t row_stride, int32_t rows, int32_t vocab,
                             float temperature, uint64_t seed, int32_t round, int32_t *tokens,
                             float *logq, void *ws, int64_t ws_bytes, void *stream);
/* dflash_sample_drafts without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments, kernels, random numbers and results
 * as dflash_sample_drafts; the per-(row, 8192-logit split) statistics that the
 * workspace would hold (16 bytes each) live instead in a file-scope device
 * array of 256 KiB inside the library, which every GPU the library runs on
 * holds until the process ends. So rows * ceil(vocab / 8192) <= 16384 (e.g.
 * 480 rows at vocab 151936, 512 at 262144); a larger request returns
 * DFLASH_ERR_SCRATCH before anything is enqueued. Nothing is allocated: the
 * array's device address is looked up once per device on the first call there
 * (DFLASH_ERR_HIP if that fails). Every entry of the scratch that a call reads
 * is written by the same call first, so no clearing is needed between calls.
 * All calls on one GPU share that GPU's array: calls that may overlap on one
 * device (different streams, or several host threads) race on it and must be
 * serialised by the caller. Other errors as dflash_sample_drafts. */
int32_t dflash_sample_drafts_static(const float *logits, int64_t row_stride, int32_t rows,
                                    int32_t vocab, float temperature, uint64_t seed,
                                    int32_t round, int32_t *tokens, float *logq, void *stream);
int32_t dflash_verify_sampled(const int32_t *drafts, const float *draft_logits,
                              const float *draft_logq, const float *target_logits,
                              int32_t batch, int32_t block_size,
                              int32_t vocab, float temperature, uint64_t seed, int32_t round,
                              int32_t *accept_len, int32_t *out_token, int32_t *anchor_out,
                              void *ws, int64_t ws_bytes, void *stream);

/* A whole decoding round with device-resident state, captured once as a HIP
 * graph and replayed [W decoding-loop pseudocode; R sec. 3.1 eq. 4, whose
 * T_o term is the per-round orchestration and cache overhead this removes]. Between two replays the caller's target pass writes
 * its tokens and features for the block the previous replay drafted; one
 * replay then runs, on the stream it is launched on:
 *   1. dflash_accept(draft_tokens, target_tokens) -> accept_len, and the
 *      bonus written over anchor;
 *   2. dflash_ctx_project(feats, batch * B rows) -> ctx;
 *   3. dflash_ctx_kv_append_accepted(ctx, accept_len): the anchor and the
 *      accepted candidates join the context, ctx_len advances on the device;
 *   4. dflash_draft_forward(anchor) -> draft_tokens (and logits when given)
 *      for the next block.
 * Every pointer in io and *cache, and the values of the sizes, are fixed at
 * creation; the buffers' contents may change between replays. The first
 * block's drafts come from an ordinary dflash_draft_forward call.
 * The workspace and ctx belong to the graph while replays may run; replays
 * of one graph, and other calls on the same buffers, must not overlap.
 *
 * dflash_round_graph_create: captures the four steps on `stream`, which must
 * be a stream that can be captured (not the legacy NULL stream), and
 * instantiates the graph. Arguments are validated as by the four calls;
 * DFLASH_ERR_STATE while the profiler records, DFLASH_ERR_HIP when capture or
 * instantiation fails. Nothing is enqueued on `stream`.
 * dflash_round_graph_launch: enqueues one replay on `stream` (any stream).
 * dflash_round_graph_destroy: frees the graph (host and driver objects only). */
typedef struct dflash_round_io {
  int32_t batch;                /* sequences; must equal cache->batch */
  const void *const *feats;     /* HOST array of n_target_feats device pointers, each
                                   [batch * B, target_hidden]: the target's features at
                                   every block position (row s*B + i) */
  int64_t feat_row_stride;      /* elements */
  const int32_t *target_tokens; /* device [batch, B]: the target's tokens for the block */
  int32_t *draft_tokens;        /* device [batch, B-1]: read (the verified block), then
                                   overwritten with the next block's drafts */
  int32_t *accept_len;          /* device [batch], written */
  int32_t *anchor;              /* device [batch]: set to the bonus token, then drafted from */
  void *ctx;                    /* device [batch * B, hidden], model dtype (scratch) */
  float *logits;                /* optional fp32 [batch, B-1, vocab] */
  int32_t *dev_status;          /* optional */
  void *ws;                     /* workspace of dflash_workspace_bytes(h, batch,
                                   cache->capacity, batch * B) bytes */
  int64_t ws_bytes;
} dflash_round_io;
typedef struct dflash_round_graph dflash_round_graph;
int32_t dflash_round_graph_create(const dflash_handle *h, const dflash_kv_cache *cache,
                                  const dflash_round_io *io, void *stream,
                                  dflash_round_graph **out);
int32_t dflash_round_graph_launch(dflash_round_graph *g, void *stream);
void dflash_round_graph_destroy(dflash_round_graph *g);

/* Static text for a dflash_status code. */
const char *dflash_status_string(int32_t code);

/* Kernel timing (benchmarking aid, process-wide, not thread-safe).
 * dflash_profiler_start(n, mask): from now on every library kernel launch of a
 * class whose bit (1 << class) is set in mask (0 = every class) is bracketed
 * by HIP events on its own stream, up to n launches.
 * dflash_profiler_stop(): stop recording (events are kept).
 * dflash_profiler_read(kind, ...): waits for the recorded events and returns,
 * for kernel class `kind` (see dflash_kernel_class), the number of launches,
 * their summed duration in ms, and their summed algorithmic HBM bytes and
 * flops (from the launch shapes). dflash_profiler_reset() frees the events. */
typedef enum dflash_kernel_class {
  DFLASH_K_GEMM_F32OUT = 0,  /* projections with an fp32 output: QKV, fusion, context K/V */
  DFLASH_K_GEMM_RESID = 1,   /* projections added into the residual stream: O, down */
  DFLASH_K_GEMM_SWIGLU = 2,  /* gate/up projection with the SwiGLU product */
  DFLASH_K_LMHEAD = 3,       /* LM head with fused argmax */
  DFLASH_K_ATTN = 4,         /* KV-injected attention partials */
  DFLASH_K_ATTN_COMBINE = 5,
  DFLASH_K_NORM_ROPE = 6,    /* per-head q/k RMSNorm + RoPE + cache scatter */
  DFLASH_K_RMSNORM = 7,
  DFLASH_K_SMALL = 8,        /* embedding, argmax reduce, accept, ctx_len update */
  DFLASH_K_SAMPLING = 9,     /* temperature > 0 drafting and verification */
  DFLASH_K_ATTN_PACKED = 10, /* training-pattern attention of packed blocks */
  DFLASH_K_NCLASSES = 11
} dflash_kernel_class;

int32_t dflash_profiler_start(int32_t max_launches, uint32_t class_mask);
int32_t dflash_profiler_stop(void);
int32_t dflash_profiler_read(int32_t kind, int64_t *launches, double *total_ms,
                             double *total_bytes, double *total_flops);
int32_t dflash_profiler_reset(void);

/* Measurement aid: a calibration loop for the MFMA roofline. Enqueues on
 * stream n_workgroups workgroups of 8 waves (two per SIMD of a CU); every
 * wave issues iters x 8 independent bf16 16x16x32 matrix multiply-accumulates
 * on register operands with random bits and nothing else, so the time the
 * caller measures around the launch gives the MFMA rate this chip sustains
 * with every matrix core busy (its clock under that load, not the nominal
 * one). *flops (optional host pointer) receives the launch's flop count,
 * n_workgroups * 8 * iters * 8 * 2*16*16*32. sink: device fp32 buffer of at
 * least n_workgroups * 8 entries (one value per wave; written so the loop
 * cannot be optimised away). Errors: DFLASH_ERR_SHAPE (a count < 1),
 * DFLASH_ERR_NULL (sink), DFLASH_ERR_HIP (launch). */
int32_t dflash_probe_mfma_bf16(int32_t n_workgroups, int32_t iters, float *sink, double *flops,
                               void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
