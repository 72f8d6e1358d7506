/*
 * pe.h -- C ABI of libpe, the MI355X (gfx950) P-EAGLE parallel-draft step.
 *
 * One draft step is four calls, in this order, on one stream:
 *   pe_prepare        batch metadata for the draft batch
 *   pe_gather_hidden  target hidden states into their slots, h_shared into MASK slots
 *   pe_draft_forward  one drafter pass over every slot, LM head + argmax -> t_1..t_K
 *   pe_verify         greedy verification -> accepted length and bonus token
 * pe_step_graph captures the four into one hipGraph and replays it.
 * pe_ar_draft runs the same kernels as K sequential drafting passes, the
 * autoregressive baseline, in place of pe_draft_forward.
 * pe_prefill_prepare / pe_prefill_gather / pe_prefill_forward draft the first
 * round after a prompt: prompt positions, the NTP position and K-1 MASK
 * positions in one pass.
 * pe_draft_forward_sampled / pe_verify_sampled draw the drafts and verify them
 * by rejection sampling instead of greedily.
 * pe_dflash_prepare / pe_dflash_inject / pe_dflash_forward run a DFlash-style
 * round: verifier hidden states projected into the KV cache, then one block of
 * MASK slots drafted in a single pass.
 *
 * Sources (page titles as published):
 *   [P1] "P-EAGLE: parallel speculative decoding in vLLM" -- sections
 *        "Architecture and mechanism" (Step 1, Prefilling; Step 2, Parallel
 *        Drafting), "vLLM
 *        implementation details" (Fused Triton kernel; Hidden-state
 *        management; KV cache and CUDA Graphs), "Benchmarks" (Acceptance length).
 *   [P2] "vLLM Speculators: parallel drafting for speculative decoding" --
 *        "Production integration" (verification by rejection sampling).
 *   [P3] "AWS and vLLM ship P-EAGLE" -- "How it works", "Integration and numbers".
 *
 * Conventions for every entry point
 *   - Pointers named as device pointers must point to device memory (any
 *     allocator; the library never frees caller memory).  Float/bf16 tensors
 *     and the KV caches must be 16-byte aligned; int32 arrays 4-byte aligned;
 *     int64 arrays 8-byte aligned.
 *   - Storage type of weights, hidden states and KV caches is cfg.dtype:
 *     PE_F32 (IEEE float32) or PE_BF16 (bfloat16 bit patterns).  Row-major.
 *   - Every call is asynchronous on the context's stream; nothing
 *     synchronizes except pe_get_device_error.
 *   - Host-detectable argument errors (null pointers, sizes out of range,
 *     misalignment) return PE_ERR_INVALID_ARG and launch nothing.
 *   - Data-dependent errors found on the device (see PE_DEVERR_*) never fault:
 *     the offending request turns into padding (all slots rejected, KV slot
 *     -1, seq_len 0, draft tokens -1) and a sticky device error word records
 *     the kinds and the lowest failing request; pe_get_device_error reads it.
 *   - One context per stream; calls on one context must not overlap.
 *   - B == 0 is valid and launches nothing.
 */
#ifndef PE_H
#define PE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pe_status {
  PE_OK = 0,
  PE_ERR_INVALID_ARG = 1,
  PE_ERR_NOMEM = 2,
  PE_ERR_HIP = 3,          /* a HIP runtime call failed; pe_last_error() has text */
  PE_ERR_UNSUPPORTED = 4   /* a shape the kernels do not implement */
} pe_status;

typedef enum pe_dtype { PE_F32 = 0, PE_BF16 = 1 } pe_dtype;

/* Device error kinds (bitmask), see pe_get_device_error. */
#define PE_DEVERR_ACCEPTED 1u  /* num_accepted outside [0, K] */
#define PE_DEVERR_TOKEN    2u  /* an accepted draft or the bonus token outside [0, vocab) */
#define PE_DEVERR_BLOCK    4u  /* p0 < 0, block table too short, or a block id outside [0, num_kv_blocks) */
#define PE_DEVERR_LAYOUT   8u  /* verify positions are not p0, p0+1, ..., p0+K */

#define PE_PADDING_SLOT_ID (-1) /* KV slot of a slot that must not write the cache [P1, KV cache] */
#define PE_PAD_TOKEN 0          /* token id written into rejected slots */

/* Drafter shape and step parameters, fixed for the life of a context. */
typedef struct pe_config {
  int32_t K;            /* draft depth (num_speculative_tokens), 1..32 */
  int32_t max_num_seqs; /* largest B any call may pass, >= 1 */
  int32_t d;            /* hidden size, multiple of 64 */
  int32_t n_q_heads;    /* query heads */
  int32_t n_kv_heads;   /* KV heads; n_q_heads % n_kv_heads == 0 */
  int32_t head_dim;     /* 64 for PE_BF16; even and <= 128 for PE_F32 */
  int32_t mlp;          /* MLP size I, multiple of 32 */
  int32_t layers;       /* decoder layers N >= 1 */
  int32_t vocab;        /* V, multiple of 16 */
  int32_t block_size;   /* KV page size in tokens, a power of two >= 16 */
  int32_t mask_id;      /* token id of MASK; its embedding row is emb(mask) [P1, Step 2] */
  int32_t dtype;        /* pe_dtype */
  float rms_eps;        /* RMSNorm epsilon */
  float rope_theta;     /* RoPE base */
  int32_t max_prefill_slots; /* largest B*S of a drafting round after a prompt
                                (pe_prefill_*); 0 = none */
} pe_config;

/* Device pointers of one decoder layer.  Linear weights are [out, in]. */
typedef struct pe_layer_weights {
  const void* attn_norm; /* [d] */
  const void* wq;        /* [n_q_heads*head_dim, d] */
  const void* wk;        /* [n_kv_heads*head_dim, d] */
  const void* wv;        /* [n_kv_heads*head_dim, d] */
  const void* wo;        /* [d, n_q_heads*head_dim] */
  const void* mlp_norm;  /* [d] */
  const void* w_gate;    /* [mlp, d] */
  const void* w_up;      /* [mlp, d] */
  const void* w_down;    /* [d, mlp] */
} pe_layer_weights;

/* Drafter weights.  Device pointers, borrowed for the context's life;
 * `layers` is a host array of cfg.layers entries, copied by pe_create.
 * For PE_BF16, pe_create also makes a context-owned copy of lm_head in MFMA
 * fragment order (V*d*2 bytes), read by the draft step at small batch: the
 * weights must not change after pe_create. */
typedef struct pe_weights {
  const void* embed;      /* [vocab, d] token embeddings; row mask_id is emb(mask) */
  const void* w_fc;       /* [d, 2d] fc over concat(emb, hidden), embedding first */
  const pe_layer_weights* layers;
  const void* final_norm; /* [d] */
  const void* lm_head;    /* [vocab, d] */
} pe_weights;

/* The draft batch: caller-allocated device buffers that pe_prepare fills and
 * the later calls read.  S = 2K slots per request, request r at base r*S:
 * slots 0..K are the copied region (slot j at the previous verify position
 * p0+j), slots K+1..2K-1 are the K-1 MASK slots [P1, Fused Triton kernel]. */
typedef struct pe_batch {
  int32_t* input_ids;    /* [B*S]  token per slot */
  int32_t* positions;    /* [B*S]  sequence position per slot */
  int32_t* hidden_src;   /* [B*S]  row of target_hidden, -1 = h_shared (hidden-state map) */
  uint8_t* is_rejected;  /* [B*S]  1 for copied slots beyond the accepted prefix + 1 */
  uint8_t* is_masked;    /* [B*S]  1 for MASK slots (by role, not by token) */
  int64_t* slot_mapping; /* [B*S]  paged KV slot, PE_PADDING_SLOT_ID if rejected */
  int32_t* draft_rows;   /* [B*K]  slots whose outputs are t_1..t_K: NTP slot, then MASK slots */
  int32_t* seq_lens;     /* [B]    p0 + a + K (0 for a request turned into padding) */
} pe_batch;

typedef struct pe_ctx pe_ctx;

/* Creates a context on the current HIP device.  Validates the shape (returns
 * PE_ERR_UNSUPPORTED for shapes the kernels do not cover), copies cfg and the
 * weight pointers, and allocates the workspace for max_num_seqs requests
 * (activations, attention partials, argmax keys, the device error word).
 * stream: a hipStream_t (NULL = the default stream). */
pe_status pe_create(const pe_config* cfg, const pe_weights* w, void* stream, pe_ctx** out);
pe_status pe_destroy(pe_ctx* ctx);
pe_status pe_set_stream(pe_ctx* ctx, void* stream);

/* Batch preparation, one fused pass [P1, Fused Triton kernel; KV cache].
 * Per request r (a = num_accepted[r], p0 = verify_positions[r*(K+1)]):
 *   copied slot j=0..K: position verify_positions[r][j], hidden_src r(K+1)+j,
 *     token verify_tokens[r][j+1] if j<a, bonus_tokens[r] if j==a (the NTP
 *     slot), else PE_PAD_TOKEN and rejected;
 *   MASK slot K+m, m=1..K-1: token mask_id, position p0+a+m, hidden_src -1;
 *   slot_mapping = block_table[r][pos/bs]*bs + pos%bs, or -1 when rejected;
 *   draft_rows[r] = {r*S+a, r*S+K+1, ..., r*S+2K-1}; seq_lens[r] = p0+a+K.
 * Inputs (device): verify_tokens, verify_positions [B, K+1] int32 -- the
 * previous verify batch x0, d_1..d_K and its positions; num_accepted,
 * bonus_tokens [B]; block_table [B, max_blocks] int32.  num_kv_blocks is the
 * size of the KV pool in blocks (for validation).  out: filled. */
pe_status pe_prepare(pe_ctx* ctx, int32_t B,
                     const int32_t* verify_tokens, const int32_t* verify_positions,
                     const int32_t* num_accepted, const int32_t* bonus_tokens,
                     const int32_t* block_table, int32_t max_blocks, int32_t num_kv_blocks,
                     const pe_batch* out);

/* Hidden-state copy [P1, Hidden-state management]: draft_hidden[s] =
 * target_hidden[hidden_src[s]] when hidden_src[s] >= 0, else h_shared; a bit
 * copy.  target_hidden [B*(K+1), d], h_shared [d], draft_hidden [B*S, d],
 * all cfg.dtype, device.  batch must come from pe_prepare. */
pe_status pe_gather_hidden(pe_ctx* ctx, int32_t B, const pe_batch* batch,
                           const void* target_hidden, const void* h_shared, void* draft_hidden);

/* One drafter forward over all B*S slots [P1, Step 2: every position goes
 * through the N-layer Transformer and the LM head, predicting t_1..t_K at
 * once].  x = W_fc[emb(token); hidden]; per layer pre-norm attention (RoPE,
 * KV written at slot_mapping, skipped for -1 [P1, KV cache], causal over the
 * request's positions [0, position] through block_table) and SwiGLU MLP;
 * final RMSNorm on the draft rows; argmax of W_lm z (lowest index on ties).
 * k_cache, v_cache: host arrays of cfg.layers device pointers.
 *   K cache layer l: [num_kv_blocks*block_size, n_kv_heads, head_dim]
 *   V cache layer l: [num_kv_blocks, n_kv_heads, head_dim, block_size]
 *                    (d-major inside a block)
 * draft_tokens [B*K] int32 out (t_1..t_K per request, -1 for padding).
 * logits: NULL, or [B*K, vocab] float32 out (debug/parity; costs bandwidth);
 * the rows of a padded request are unspecified.
 * batch must come from pe_prepare and draft_hidden from pe_gather_hidden:
 * the K-1 MASK slots of a request then carry the same input (emb(mask),
 * h_shared), and in bf16 with K >= 3 and B*(K+2) > 64 the first layer's fc
 * and QKV products compute it once per request (RoPE and the KV write still
 * run per slot). */
pe_status pe_draft_forward(pe_ctx* ctx, int32_t B, const pe_batch* batch,
                           const void* draft_hidden,
                           const int32_t* block_table, int32_t max_blocks, int32_t num_kv_blocks,
                           void* const* k_cache, void* const* v_cache,
                           int32_t* draft_tokens, float* logits);

/* Autoregressive drafting with the same kernels, the sequential baseline
 * the parallel pass replaces [P1, Solving the autoregressive drafting
 * bottleneck: an EAGLE drafter runs one forward pass per draft token].
 * Same arguments and outputs as pe_draft_forward; batch and draft_hidden come
 * from pe_prepare and pe_gather_hidden.
 *   pass 1: the K+1 copied slots of every request (rejected slots attend to
 *     nothing and write no KV); t_1 is drafted at the NTP slot;
 *   pass k = 2..K: one slot per request holding t_{k-1} at position
 *     p0+a+k-1, paired with the drafter's own output hidden state (the
 *     residual stream after the last layer) of the previous pass's draft row;
 *     it drafts t_k.
 * Feeding back the drafter's hidden state is EAGLE's drafting loop; the pages
 * describe only its cost, so this is a reading of it.  KV is written at
 * positions p0..p0+a+K-1, the positions the parallel pass writes (with
 * different values at the MASK positions).  The MASK slots of batch and rows
 * K+1..2K-1 of draft_hidden are not read.  logits, when not NULL, is
 * [B*K, vocab] as for pe_draft_forward. */
pe_status pe_ar_draft(pe_ctx* ctx, int32_t B, const pe_batch* batch,
                      const void* draft_hidden,
                      const int32_t* block_table, int32_t max_blocks, int32_t num_kv_blocks,
                      void* const* k_cache, void* const* v_cache,
                      int32_t* draft_tokens, float* logits);

/* Greedy verification [P1, Benchmarks, Acceptance length; P3, Integration
 * and numbers]: num_accepted[r] = first j in 0..K-1 with draft_tokens[r][j]
 * != target_tokens[r][j], or K; bonus_tokens[r] = target_tokens[r][that j].
 * draft_tokens [B, K], target_tokens [B, K+1] int32 in; outputs [B] int32. */
pe_status pe_verify(pe_ctx* ctx, int32_t B, const int32_t* draft_tokens,
                    const int32_t* target_tokens, int32_t* num_accepted, int32_t* bonus_tokens);

/* ---- Drafting round after a prompt ------------------------------------------
 * [P1, Architecture and mechanism: Step 1, Prefilling -- the target runs the
 * prompt and returns a hidden state per position and one new token; Step 2,
 * Parallel Drafting -- a prompt position pairs the embedding of the token one
 * position later with the target's hidden state there, the NTP position pairs
 * the new token with the last hidden state, positions 2..K take emb(mask) and
 * h_shared; all go through the drafter in one pass.]
 * A prefill batch has a fixed stride of S slots per request (K <= S), and
 * L = S-K+1 rows per request in chunk_tokens and target_hidden.  Request r
 * covers prompt positions c0..c0+n-1 (c0 = start_pos[r], n = chunk_lens[r] in
 * [1, L]); positions below c0 were drafted by earlier calls and are in the KV
 * cache:
 *   copied slot j = 0..n-1: position c0+j, hidden_src r*L+j, token
 *     chunk_tokens[r][j+1] (j < n-1) or new_tokens[r] (j = n-1: the NTP slot);
 *   MASK slot j = n..n+K-2: token mask_id, position c0+j, hidden_src -1;
 *   slot j >= n+K-1: rejected padding (PE_PAD_TOKEN, position 0, hidden_src
 *     -1, KV slot -1);
 *   draft_rows[r] = {r*S+n-1, ..., r*S+n+K-2}; seq_lens[r] = c0+n+K-1.
 * A chunk that does not end the prompt is the same call with new_tokens[r] =
 * the next prompt token: its drafts are ignored, and the next chunk
 * overwrites the KV its MASK slots wrote.  Device errors: n outside [1, L]
 * (PE_DEVERR_ACCEPTED), a token the request reads outside [0, vocab)
 * (PE_DEVERR_TOKEN), c0 < 0 or a block of [0, seq_len) missing
 * (PE_DEVERR_BLOCK); the request becomes padding as in pe_prepare.
 * Sizes: B <= max_num_seqs, B*S <= cfg.max_prefill_slots; pe_batch buffers
 * hold B*S slots (draft_rows B*K, seq_lens B). */

/* Batch preparation of a prefill batch.  chunk_tokens [B, L] int32: column j
 * is the prompt token at position c0+j; chunk_lens, start_pos, new_tokens
 * [B] int32; block_table [B, max_blocks] int32; all device. */
pe_status pe_prefill_prepare(pe_ctx* ctx, int32_t B, int32_t S, const int32_t* chunk_tokens,
                             const int32_t* chunk_lens, const int32_t* start_pos,
                             const int32_t* new_tokens, const int32_t* block_table,
                             int32_t max_blocks, int32_t num_kv_blocks, const pe_batch* out);

/* Hidden-state copy of a prefill batch, as pe_gather_hidden:
 * target_hidden [B*L, d], draft_hidden [B*S, d]. */
pe_status pe_prefill_gather(pe_ctx* ctx, int32_t B, int32_t S, const pe_batch* batch,
                            const void* target_hidden, const void* h_shared, void* draft_hidden);

/* One drafter forward over the B*S slots of a prefill batch, as
 * pe_draft_forward: draft_tokens [B*K] (t_1..t_K per request), logits NULL or
 * [B*K, vocab].  PE_BF16 attention takes a request's slots in groups of
 * 512/(n_q_heads/n_kv_heads) rounded down to a power of two: S must be at most
 * one group or a multiple of it, and B*S/group <= 1024
 * (PE_ERR_UNSUPPORTED otherwise). */
pe_status pe_prefill_forward(pe_ctx* ctx, int32_t B, int32_t S, const pe_batch* batch,
                             const void* draft_hidden,
                             const int32_t* block_table, int32_t max_blocks, int32_t num_kv_blocks,
                             void* const* k_cache, void* const* v_cache,
                             int32_t* draft_tokens, float* logits);

/* ---- DFlash-style round: KV injection + one bidirectional block -------------
 * [P2, comparison of P-EAGLE, DFlash and DSpark: DFlash projects the
 * verifier's hidden states into the drafter's KV cache, so that the drafter's
 * attention is conditioned on them without a longer input, and drafts the
 * candidate tokens by block diffusion.]  The page gives no more; this library
 * takes the following reading.  After a verify batch as for pe_prepare (K+1
 * tokens at p0..p0+K, a accepted, the bonus token):
 *   injection  per layer l, the verifier hidden state h_j of each kept
 *              position p0+j (j <= a) is written to the layer's KV cache as
 *              k = RoPE(Wk_inj[l] h_j) at p0+j and v = Wv_inj[l] h_j;
 *   block      K+1 slots [bonus, MASK x K] at positions p0+a+1 .. p0+a+K+1,
 *              input emb(token) alone, through the drafter's layers (fc and
 *              h_shared are not used); every slot attends to positions
 *              [0, p0+a+K+1] (the whole block: one denoising step);
 *   drafts     the argmax of the LM head at MASK slot i is the draft for that
 *              slot's own position (K drafts per request).
 * One round is pe_dflash_prepare, pe_dflash_inject, pe_dflash_forward, in
 * stream order. */

/* Batch preparation of the block.  verify_positions [B, K+1], num_accepted,
 * bonus_tokens [B], block_table [B, max_blocks]: as pe_prepare (device int32).
 * out: a pe_batch with S = K+1 slots per request (input_ids, positions,
 * hidden_src (all -1), is_rejected, is_masked, slot_mapping, draft_rows
 * [B*K] = the MASK slots, seq_lens = p0+a+K+2); attn_positions [B*(K+1)]
 * int32: the last position each slot attends to (p0+a+K+1); inject_slots
 * [B*(K+1)] int64: the KV slot of verify position j of request r at
 * r*(K+1)+j when j <= a, else -1.  The block table must cover
 * [0, p0+a+K+2).  Checks and padding as pe_prepare (the accepted drafts'
 * token ids are not read).  K <= 63. */
pe_status pe_dflash_prepare(pe_ctx* ctx, int32_t B, const int32_t* verify_positions,
                            const int32_t* num_accepted, const int32_t* bonus_tokens,
                            const int32_t* block_table, int32_t max_blocks, int32_t num_kv_blocks,
                            const pe_batch* out, int32_t* attn_positions, int64_t* inject_slots);

/* KV injection: for every layer, the target_hidden rows [B*(K+1), d]
 * (cfg.dtype) projected by wk_inject[l], wv_inject[l] ([n_kv_heads*head_dim,
 * d] row-major, cfg.dtype, borrowed for the call) into k_cache[l], v_cache[l]
 * at inject_slots (from pe_dflash_prepare; rows with -1 write nothing).  K
 * takes RoPE at verify_positions; storage and layouts as pe_draft_forward. */
pe_status pe_dflash_inject(pe_ctx* ctx, int32_t B, const int32_t* verify_positions,
                           const int64_t* inject_slots, const void* target_hidden,
                           const void* const* wk_inject, const void* const* wv_inject,
                           int32_t num_kv_blocks, void* const* k_cache, void* const* v_cache);

/* One drafter pass over the block (B*(K+1) slots), as pe_draft_forward with
 * the batch and attn_positions of pe_dflash_prepare: draft_tokens [B*K] (-1
 * for a padded request), logits NULL or [B*K, vocab] fp32. */
pe_status pe_dflash_forward(pe_ctx* ctx, int32_t B, const pe_batch* batch, const int32_t* attn_positions,
                            const int32_t* block_table, int32_t max_blocks, int32_t num_kv_blocks,
                            void* const* k_cache, void* const* v_cache, int32_t* draft_tokens,
                            float* logits);

/* ---- Stochastic drafting and verification by rejection sampling -------------
 * [P2, Production integration: speculative decoding verifies by rejection
 * sampling, so the output keeps the verifier's distribution.]  With
 * temperature T, q_j = softmax(z_j / T) is the drafter's distribution at draft
 * row j of a request and p_j = softmax(y_j / T) the verifier's at the same
 * position:
 *   drafts    t_j is a draw from q_j;
 *   accept    t_j is kept while U_j < min(1, p_j(t_j) / q_j(t_j));
 *   emit      at the first rejection j: a draw from max(0, p_j - q_j),
 *             normalised (num_accepted = j); after K kept drafts: a draw from
 *             p_K (num_accepted = K).
 * Random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC 2011), key = *seed (64 bits, low word
 * first), counter (c0, c1, 0, stream); U = ((x >> 9) + 1/2) / 2^23 from the
 * first output word x.  A draw from w is argmax_v(log w(v) - log(-log U_v))
 * (Gumbel-max; lowest index on ties) with
 *   drafting: stream 0, counter (v, draft row r*K+j);
 *   acceptance: stream 1, counter (j, r);
 *   emitted token: stream 2, counter (v, r).
 * seed is a device pointer (8-byte aligned), read by the kernels, so a caller
 * can change it between graph replays. */

/* As pe_draft_forward, with each draft token drawn from softmax(logits / T)
 * instead of the argmax.  logits ([B*K, vocab] float32, required, 16-byte
 * aligned) receives the
 * raw logits the draws are made from; pe_verify_sampled takes them as
 * draft_logits. */
pe_status pe_draft_forward_sampled(pe_ctx* ctx, int32_t B, const pe_batch* batch,
                                   const void* draft_hidden,
                                   const int32_t* block_table, int32_t max_blocks, int32_t num_kv_blocks,
                                   void* const* k_cache, void* const* v_cache, float temperature,
                                   const uint64_t* seed, int32_t* draft_tokens, float* logits);

/* Verification by rejection sampling.  draft_tokens [B, K] int32 (a token
 * outside [0, vocab), e.g. -1 of a padded request, is rejected);
 * draft_logits [B*K, vocab] float32 (the drafter's rows); target_logits
 * [B*(K+1), vocab] float32 (the verifier's rows at the K+1 positions);
 * num_accepted [B] and next_tokens [B] int32 out (the emitted token: the
 * residual draw or the bonus draw).  All device; logit rows 16-byte aligned. */
pe_status pe_verify_sampled(pe_ctx* ctx, int32_t B, const int32_t* draft_tokens,
                            const float* draft_logits, const float* target_logits, float temperature,
                            const uint64_t* seed, int32_t* num_accepted, int32_t* next_tokens);

/* Verification by rejection sampling that allocates nothing, for callers that
 * cannot allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same inputs, outputs and results as
 * pe_verify_sampled, but no context: K (1..32) and vocab (a multiple of 4) are
 * arguments, and the work runs on `stream` (a hipStream_t, NULL = the default
 * stream).  Its workspace (per-row log-sum-exp, per-slice partials, draw keys)
 * is a fixed device array of the library, about 2.1 MB per GPU, held until
 * the process ends: B <= 2048 and B*(2K+1) <= 8192, else PE_ERR_UNSUPPORTED
 * and nothing is launched.  Every call on one GPU uses that GPU's one
 * workspace: calls that overlap on a GPU (other streams, other threads) race
 * and must be serialized by the caller.  Argument errors as pe_verify_sampled;
 * no implicit synchronization. */
pe_status pe_verify_sampled_noalloc(int32_t B, int32_t K, int32_t vocab, const int32_t* draft_tokens,
                                    const float* draft_logits, const float* target_logits, float temperature,
                                    const uint64_t* seed, int32_t* num_accepted, int32_t* next_tokens,
                                    void* stream);

/* Draft depth selection [P1, Speculative depth efficiency: throughput peaks
 * at the depth where more accepted drafts stop paying for a deeper draft; P2,
 * Limits of autoregressive drafting: the speculation length is tuned to the
 * drafting cost].  Reading (the pages give no acceptance model): each draft is
 * kept with probability alpha while every earlier one was, so a round at
 * depth K emits E(K) = sum_{i=0..K} alpha^i tokens; it costs draft_us[i] (a
 * measured step time, e.g. from pe_step_graph) + verify_fixed_us +
 * verify_per_token_us * (K + 1).  Returns the K of Ks[0..n) with the largest
 * E(K) / cost (the smaller K on ties) and that rate in tokens per
 * microsecond.  Host arrays; host-only, nothing is launched.  Errors: n < 1,
 * alpha outside [0, 1], a cost that is not positive, a K outside [1, 32]. */
pe_status pe_choose_depth(const int32_t* Ks, const double* draft_us, int32_t n, double alpha,
                          double verify_fixed_us, double verify_per_token_us,
                          int32_t* best_K, double* tokens_per_us);

/* Drafting pass of a step graph: pe_draft_forward or pe_ar_draft. */
typedef enum pe_step_mode { PE_STEP_PARALLEL = 0, PE_STEP_AUTOREGRESSIVE = 1, PE_STEP_DFLASH = 2 } pe_step_mode;

/* All buffers of one step, for pe_step_graph. */
typedef struct pe_step_args {
  const int32_t* verify_tokens;
  const int32_t* verify_positions;
  const int32_t* num_accepted;
  const int32_t* bonus_tokens;
  const int32_t* block_table;
  int32_t max_blocks;
  int32_t num_kv_blocks;
  pe_batch batch;
  const void* target_hidden;
  const void* h_shared;
  void* draft_hidden;
  void* const* k_cache;      /* host array, cfg.layers entries */
  void* const* v_cache;
  int32_t* draft_tokens;
  float* logits;             /* NULL unless wanted */
  const int32_t* target_tokens;
  int32_t* accepted_out;     /* pe_verify outputs; may alias nothing above */
  int32_t* bonus_out;
  int32_t mode;              /* pe_step_mode */
  /* PE_STEP_DFLASH only (NULL otherwise): the round is pe_dflash_prepare ->
   * pe_dflash_inject -> pe_dflash_forward -> pe_verify; batch has S = K+1
   * slots per request; verify_tokens, h_shared and draft_hidden are not read */
  const void* const* wk_inject;  /* host arrays, cfg.layers entries */
  const void* const* wv_inject;
  int32_t* attn_positions;       /* [B*(K+1)] */
  int64_t* inject_slots;         /* [B*(K+1)] */
  /* Occupancy: NULL (all B requests active), or a device int32 holding the
   * number n of active requests; requests n..B-1 are inactive slots of the
   * batch.  Read on the device at every replay, so one captured graph serves
   * any occupancy 0..B [P1, KV cache and CUDA Graphs: the graph is captured
   * for the K x max_num_seqs draft rows of the largest batch].  An inactive
   * request is not validated and sets nothing in the device error word; its
   * slots become padding (rejected, KV slot -1, seq_len 0, no KV write), its
   * draft tokens are -1, accepted_out 0 and bonus_out PE_PAD_TOKEN, and the
   * dense products, attention and LM head skip its rows where they can.
   * n is clamped to [0, B]. */
  const int32_t* num_active;
} pe_step_args;

/* Captures prepare -> gather -> forward (args->mode picks the parallel pass,
 * the sequential passes or a DFlash-style round) -> verify for (B, *args)
 * into a hipGraph on the first call and replays it on later calls with the
 * same B and the same pointers.  Values inside the buffers may change between
 * replays -- a, p0, tokens, block tables and the occupancy *num_active are
 * read on the device -- so a graph captured at B = max_num_seqs serves every
 * batch of up to max_num_seqs requests [P1, KV cache and CUDA Graphs: one
 * graph covers the K x max_num_seqs draft rows].  A call with other pointers
 * or another B recaptures; capture runs on a private non-blocking stream of
 * the context (the legacy default stream cannot be captured), and only a
 * recapture that replaces an earlier graph first waits for the context's
 * stream (the old graph may still run).  Every launch of the graph is
 * enqueued on the context's stream.  The graph holds no memset node. */
pe_status pe_step_graph(pe_ctx* ctx, int32_t B, const pe_step_args* args);

/* Number of captures and of replays pe_step_graph has made on this context. */
pe_status pe_step_graph_stats(pe_ctx* ctx, int64_t* captures, int64_t* replays);

/* Synchronizes the context's stream, reads and clears the sticky device error
 * word.  kinds: OR of PE_DEVERR_*; first_request: lowest failing request
 * index, or -1 when kinds == 0. */
pe_status pe_get_device_error(pe_ctx* ctx, uint32_t* kinds, int32_t* first_request);

/* Per-phase kernel timing.  With profiling on, every eager launch of a phase
 * is bracketed by a pair of HIP events on the context's stream; nothing is
 * recorded while a step graph is being captured.  pe_profile_read
 * synchronizes the stream and returns, per phase, the summed event time in ms
 * and the number of launches since the last reset. */
typedef enum pe_phase {
  PE_PH_PREPARE = 0, PE_PH_GATHER, PE_PH_FC, PE_PH_NORM, PE_PH_QKV, PE_PH_ATTN,
  PE_PH_O, PE_PH_GATEUP, PE_PH_DOWN, PE_PH_LMHEAD, PE_PH_VERIFY, PE_PH_ARGMAX,
  PE_PH_AR, /* batch of a sequential pass (pe_ar_draft) */
  PE_PH_COUNT
} pe_phase;
pe_status pe_profile_enable(pe_ctx* ctx, int on);
pe_status pe_profile_read(pe_ctx* ctx, double* ms /* [PE_PH_COUNT] */,
                          int64_t* launches /* [PE_PH_COUNT] */, int reset);

/* Text of the last error on this thread ("" if none). */
const char* pe_last_error(void);
const char* pe_status_string(pe_status s);

#ifdef __cplusplus
}
#endif
#endif /* PE_H */
