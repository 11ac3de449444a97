/*
 * qtalk.h - C ABI of the KV-cached Talker forward on MI355X (gfx950).
 *
 * The library computes the Qwen3-lineage Talker decoder stack used by
 * Qwen3-TTS: per layer a pre-norm RMSNorm, bias-free Q/K/V projections,
 * per-head QK-RMSNorm, 1-D NEOX rotary embedding, a write of K and V into a
 * per-sequence KV cache, causal grouped-query attention that reads the cache
 * back, o_proj plus residual, a post-attention RMSNorm and a SwiGLU MLP plus
 * residual; then a final RMSNorm and the codec_head projection to codebook-0
 * logits.  Sources: "qwentts.cpp src/talker-forward.h" (file header,
 * talker_layer_forward, talker_forward_core, talker_forward_prefill,
 * talker_forward_decode), "transcribe.cpp src/causal_lm/causal_lm.cpp"
 * (block_prefill, block_step, mul_mat_f32acc) and "rightkit-qts 0.2.3
 * src/pipeline/tts_transformer.rs" (TtsTransformerConfig defaults,
 * forward_prefill_cached, forward_step_cached).
 *
 * General conventions
 *  - All compute runs as HIP kernels on the stream given to qtalk_create.
 *    Every call validates its arguments on the host first; on any error it
 *    launches nothing, leaves every cache length unchanged, records a message
 *    (qtalk_last_error) and returns a negative qtalk_status.
 *  - Calls that take activations (emb, logits, hidden_out, kv_read dst) take
 *    DEVICE pointers owned by the caller, in float32, row-major.  They return
 *    once the work is enqueued; results are ready when the stream reaches
 *    that point (synchronise the stream, or order later work on it).
 *  - Accumulation is float32 everywhere (dot products, sums of squares,
 *    softmax), as the pages require to keep large residual channels from
 *    overflowing ("transcribe.cpp src/causal_lm/causal_lm.cpp",
 *    mul_mat_f32acc).
 *  - A context is not thread-safe; use one per host thread, or serialise.
 */
#ifndef QTALK_H
#define QTALK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QTALK_OK = 0,
  QTALK_E_INVAL = -1,    /* bad argument: null pointer, bad id, T < 1, shape */
  QTALK_E_OVERFLOW = -2, /* the write would pass the KV capacity            */
  QTALK_E_NOMEM = -3,    /* device allocation failed                         */
  QTALK_E_DEVICE = -4    /* a HIP call or kernel launch failed               */
} qtalk_status;

/* QTALK_Q8 (KV cache only): Q8_0 blocks of 32 values along head_dim, int8
 * codes with one float16 scale per block ("rightkit-qts 0.2.3
 * src/pipeline/tts_transformer.rs", TalkerKvStorage::TurboQuantQ8_0). */
typedef enum { QTALK_F32 = 0, QTALK_BF16 = 1, QTALK_F16 = 2, QTALK_Q8 = 3 } qtalk_dtype;

/* Model geometry and cache sizes.  The Talker defaults are hidden 1024,
 * 28 layers, 16 query heads, 8 KV heads, head_dim 128, intermediate 3072,
 * vocab 3072, eps 1e-6, theta 1e6 ("rightkit-qts 0.2.3
 * src/pipeline/tts_transformer.rs", TtsTransformerConfig::default).
 * Requirements (else QTALK_E_INVAL): every size >= 1; head_dim is 64 or 128;
 * n_heads % n_kv_heads == 0; hidden, intermediate and n_heads*head_dim are
 * multiples of 64 and at most 8192; intermediate is a multiple of 16;
 * weight_dtype is F32 or BF16; kv_dtype is F32, F16 or Q8.  q_dim = n_heads*head_dim need not equal
 * hidden (it does not for the Talker: 2048 vs 1024). */
typedef struct {
  int32_t n_layers;
  int32_t hidden;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t intermediate;
  int32_t vocab;
  float rms_eps;
  float rope_theta;
  int32_t max_seq_len;  /* KV capacity per sequence                    */
  int32_t max_seqs;     /* number of independent sequences (KV sets)   */
  int32_t weight_dtype; /* qtalk_dtype: F32 or BF16 (projections, head) */
  int32_t kv_dtype;     /* qtalk_dtype: F32, F16 or Q8 (cache storage)  */
  int32_t n_output_heads; /* output projections stacked in codec_head
                             (0 or 1: one; the code predictor has 15),
                             at most 64; see qtalk_select_head           */
} qtalk_config;

/* One layer's weights.  Projections are row-major [out][in] in weight_dtype,
 * as ggml's mul_mat(W, x) stores them ("qwentts.cpp
 * src/talker-forward.h", talker_layer_forward):
 *   q_proj [n_heads*head_dim][hidden], k_proj and v_proj
 *   [n_kv_heads*head_dim][hidden], o_proj [hidden][n_heads*head_dim],
 *   gate_proj and up_proj [intermediate][hidden], down_proj
 *   [hidden][intermediate].
 * Norm gains are float32: input_norm and post_attn_norm [hidden], q_norm and
 * k_norm [head_dim] (one gain shared by every head).
 * Pointers may be host or device memory; qtalk_create copies (and repacks)
 * them into library-owned device memory, so the caller may free them
 * afterwards. */
typedef struct {
  const void *q_proj, *k_proj, *v_proj, *o_proj;
  const void *gate_proj, *up_proj, *down_proj;
  const float *input_norm, *post_attn_norm, *q_norm, *k_norm;
} qtalk_layer_weights;

typedef struct {
  const qtalk_layer_weights *layers; /* host array [n_layers]              */
  const float *final_norm;           /* [hidden] float32                    */
  const void *codec_head;            /* [n_output_heads][vocab][hidden] in
                                        weight_dtype                        */
} qtalk_weights;

typedef struct qtalk_ctx qtalk_ctx;

/* Create a context on the current HIP device: copy the weights, allocate the
 * zero-initialised KV cache ([n_layers][max_seqs][n_kv_heads][max_seq_len]
 * [head_dim] for K and for V) and scratch buffers.  `hip_stream` is a
 * hipStream_t (NULL: the default stream).  On success *out owns everything
 * until qtalk_destroy.  Errors: QTALK_E_INVAL (config, null pointer),
 * QTALK_E_NOMEM, QTALK_E_DEVICE; *out is then NULL. */
qtalk_status qtalk_create(const qtalk_config *config,
                          const qtalk_weights *weights, void *hip_stream,
                          qtalk_ctx **out);

/* Wait for the context's stream, then free everything it owns.  NULL is a
 * no-op. */
void qtalk_destroy(qtalk_ctx *ctx);

/* Prefill: rewind sequence `seq` to 0 and write T positions from
 * emb [T][hidden]; logits [vocab] receive the codebook-0 logits of the last
 * row; hidden_out [hidden] (nullable) receives that row's hidden state after
 * the final RMSNorm.  ("qwentts.cpp src/talker-forward.h",
 * talker_forward_prefill.)  Errors: QTALK_E_INVAL (seq out of range, T < 1,
 * null emb/logits), QTALK_E_OVERFLOW (T > max_seq_len). */
qtalk_status qtalk_prefill(qtalk_ctx *ctx, int32_t seq, const float *emb,
                           int32_t T, float *logits, float *hidden_out);

/* Extend: append T positions at cur_len(seq) (chunked prefill: the rows
 * attend to everything before them), same outputs as qtalk_prefill.
 * ("qwentts.cpp src/talker-forward.h", talker_forward_core with n_past.)
 * Errors as qtalk_prefill; QTALK_E_OVERFLOW when cur_len + T > max_seq_len. */
qtalk_status qtalk_extend(qtalk_ctx *ctx, int32_t seq, const float *emb,
                          int32_t T, float *logits, float *hidden_out);

/* Decode: one position at cur_len(seq) from emb [hidden]; attends to
 * [0, cur_len + 1); cur_len advances by one.  ("qwentts.cpp
 * src/talker-forward.h", talker_forward_decode.)  Errors: QTALK_E_INVAL,
 * QTALK_E_OVERFLOW when cur_len + 1 > max_seq_len. */
qtalk_status qtalk_decode(qtalk_ctx *ctx, int32_t seq, const float *emb,
                          float *logits, float *hidden_out);

/* The step input gathered on the device (see qtalk_embed_sum): row
 * ids[g] of each tables[g], summed in float32 in table order, plus the
 * overlay row. */
#define QTALK_MAX_GATHER 16
typedef struct {
  int32_t n_tables;                       /* 1 .. QTALK_MAX_GATHER           */
  const float *tables[QTALK_MAX_GATHER];  /* DEVICE float32 [table_rows[g]][hidden] */
  int32_t table_rows[QTALK_MAX_GATHER];
  const int32_t *ids;                     /* DEVICE int32 [n_tables]          */
  const float *overlay;                   /* DEVICE float32 [hidden], or NULL */
} qtalk_gather;

/* One step of a codec frame: qtalk_decode of one position of
 * `seq` whose input row is either emb [hidden] or the gather above (the
 * Talker's 16-table step embedding plus the text overlay, or the code
 * predictor's previous code looked up in its table), and, when out_id is
 * set, the suppressed greedy pick of its logits written to *out_id (device
 * int32; same rule as qtalk_argmax).  ("qwentts.cpp src/talker-forward.h",
 * the batched step graph's input_embed; "rightkit-qts 0.2.3
 * src/pipeline/tts_transformer.rs", build_talker_step_embedding and the
 * suppression loop before select_token.)  The results equal
 * qtalk_embed_sum + qtalk_decode + qtalk_argmax bit for bit.  Where the
 * persistent decode runs, a one-table lookup and the pick happen inside its
 * launch, and a sum of several tables is one gather kernel before it;
 * elsewhere it runs as those three calls.  An id outside its table cannot
 * be seen on the host: the step then computes on a NaN row, and the next
 * qtalk_sync reports it and rolls the sequence back to before that step.
 * Errors: QTALK_E_INVAL (bad seq, null logits, both or neither of emb and
 * gather, a bad gather), QTALK_E_OVERFLOW as qtalk_decode. */
qtalk_status qtalk_decode_step(qtalk_ctx *ctx, int32_t seq, const float *emb,
                               const qtalk_gather *gather, float *logits,
                               float *hidden_out, int32_t suppress_begin,
                               int32_t keep_id, int32_t *out_id);

/* qtalk_decode without the context's exchange buffers, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same persistent kernel and
 * arithmetic as qtalk_decode (same results bit for bit), whose blocks pass
 * their words and attention partials through one static device array per GPU
 * (2 MiB, held until the process ends) instead of buffers of the context.
 * It allocates and frees nothing and enqueues no memset.  Calls on one GPU
 * share that array: they are ordered per device like every batch-1 decode,
 * and calls from several host threads on one GPU at once race.  Same
 * arguments, outputs and errors as qtalk_decode, plus QTALK_E_INVAL when the
 * context has no persistent decode (it needs the Talker geometry and bf16
 * weights) or would need more than the array holds, and QTALK_E_DEVICE when
 * the array has no address on this device. */
qtalk_status qtalk_decode_noalloc(qtalk_ctx *ctx, int32_t seq, const float *emb,
                                  float *logits, float *hidden_out);

/* Batched decode: one position for each of n distinct sequences seqs[0..n)
 * (a HOST array), emb [n][hidden], logits [n][vocab], hidden_out [n][hidden]
 * (nullable).  Row i is the single-sequence decode of seqs[i]; the sequences
 * may have different lengths.  Below 8 rows the rows go through the
 * per-step decode kernels (float32 activations, the same results as
 * single-sequence decodes on those kernels); from 8 rows the projections
 * (the codec head included) run on the matrix cores with activations
 * rounded to bf16, so results differ from single decodes at that rounding.
 * ("qwentts.cpp
 * src/talker-forward.h", talker_forward_decode and
 * talker_layer_forward_batch.)  Errors: QTALK_E_INVAL (n < 1, n > max_seqs,
 * repeated or out-of-range id), QTALK_E_OVERFLOW if any sequence is full;
 * then no sequence advances. */
qtalk_status qtalk_decode_batch(qtalk_ctx *ctx, int32_t n, const int32_t *seqs,
                                const float *emb, float *logits,
                                float *hidden_out);

/* Truncate sequence `seq` to its first n_keep positions (0 <= n_keep <=
 * cur_len); slots at and above n_keep are never read again.  Rewind to 0 is
 * the pages' kv_cache_reset.  Errors: QTALK_E_INVAL. */
qtalk_status qtalk_kv_rewind(qtalk_ctx *ctx, int32_t seq, int32_t n_keep);

/* Current length of sequence `seq`, or -1 for a bad context or id. */
int32_t qtalk_kv_len(const qtalk_ctx *ctx, int32_t seq);

/* Test hook: copy the cached K (kv = 0) or V (kv = 1) of (seq, layer),
 * converted to float32, into the device buffer dst
 * [n_kv_heads][cur_len][head_dim].  Errors: QTALK_E_INVAL. */
qtalk_status qtalk_kv_read(qtalk_ctx *ctx, int32_t seq, int32_t layer,
                           int32_t kv, float *dst);

/* Batched prefill: rewind each of the n distinct sequences seqs[b] (host
 * array) to 0 and write T positions from emb[b] (emb is [n][T][hidden]);
 * logits [n][vocab] receive each sequence's last-row logits and hidden_out
 * [n][hidden] (nullable) its last row after the final RMSNorm.  The pages'
 * batched prefill: B utterances of T tokens each, every one into positions
 * [0, T) of its own KV slab, projections over all B*T rows at once
 * ("transcribe.cpp src/causal_lm/causal_lm.cpp", block_prefill_batched).
 * Results equal n separate qtalk_prefill calls up to summation order.
 * Errors: QTALK_E_INVAL (n < 1, T < 1, null pointer, a sequence id out of
 * range or listed twice), QTALK_E_OVERFLOW (T > max_seq_len); nothing is
 * launched and no cache length changes. */
qtalk_status qtalk_prefill_batch(qtalk_ctx *ctx, int32_t n, const int32_t *seqs,
                                 const float *emb, int32_t T, float *logits,
                                 float *hidden_out);

/* Step embeddings of n frame slots, on the device: for slot s,
 *   out[s] = tables[0][ids[0*n + s]] + tables[1][ids[1*n + s]] + ...
 *          + tables[n_groups-1][ids[(n_groups-1)*n + s]] + overlay[s]
 * summed in float32 in that order.  With the codec embedding as table 0 and
 * the 15 acoustic tables after it, this is the Talker's step input: the
 * codebook-0 token's codec row, each further codebook's acoustic row and the
 * trailing text row ("qwentts.cpp src/talker-forward.h", the batched step
 * graph's input_embed; "rightkit-qts 0.2.3 src/pipeline/tts_transformer.rs",
 * build_talker_step_embedding); with one table it is a plain row gather (the
 * code predictor's step input).
 *   tables     host array [n_groups] of DEVICE pointers, each a float32
 *              [table_rows[g]][hidden] table owned by the caller
 *   table_rows host array [n_groups]
 *   ids        DEVICE int32 [n_groups][n], group-major
 *   overlay    DEVICE float32 [n][hidden], or NULL for none
 *   out        DEVICE float32 [n][hidden]
 * Errors: QTALK_E_INVAL (n_groups outside 1..32, n < 1, a null pointer, an
 * empty table, hidden not a multiple of 4 or above 4096).  An id outside its
 * table cannot be seen on the host: that slot's row becomes NaN and the next
 * qtalk_sync returns QTALK_E_DEVICE. */
qtalk_status qtalk_embed_sum(qtalk_ctx *ctx, int32_t n_groups,
                             const float *const *tables,
                             const int32_t *table_rows, const int32_t *ids,
                             int32_t n, const float *overlay, float *out);

/* Greedy pick of each of n logits rows [n][vocab] (DEVICE float32) into
 * out_ids[n] (DEVICE int32): ids from suppress_begin up are excluded except
 * keep_id, then the maximum, the lowest id among equal maxima; NaN counts as
 * -inf.  For codebook 0 the pages suppress [vocab - 1024, vocab) except the
 * end-of-speech id ("rightkit-qts 0.2.3 src/pipeline/tts_transformer.rs",
 * the suppression loop before select_token); pass suppress_begin >= vocab
 * for none.  A row with no candidate gets -1.  Errors: QTALK_E_INVAL (null
 * pointer, n or vocab < 1). */
qtalk_status qtalk_argmax(qtalk_ctx *ctx, const float *logits, int32_t n,
                          int32_t vocab, int32_t suppress_begin,
                          int32_t keep_id, int32_t *out_ids);

/* qtalk_argmax and the row lookup that feeds the next code predictor step,
 * in one kernel: for each of the n logits rows, the pick (same suppression,
 * tie and NaN rules as qtalk_argmax) goes to out_ids[i], and row out_ids[i]
 * of table ([table_rows][hidden] DEVICE float32, hidden of the context) to
 * out_rows[i] ([n][hidden] DEVICE float32): step j's input is the embedding
 * of code j - 1 ("rightkit-qts 0.2.3 src/pipeline/tts_transformer.rs",
 * forward_code_pred_step_cached).  A row whose pick is -1 or not below
 * table_rows gets a NaN row, and the next qtalk_sync returns QTALK_E_DEVICE.
 * Errors: QTALK_E_INVAL (null pointer; n, vocab or table_rows < 1). */
qtalk_status qtalk_argmax_embed(qtalk_ctx *ctx, const float *logits,
                                int32_t n, int32_t vocab,
                                int32_t suppress_begin, int32_t keep_id,
                                const float *table, int32_t table_rows,
                                int32_t *out_ids, float *out_rows);

/* Choose which of the n_output_heads stacked output projections produces
 * the logits of the calls enqueued after this one (initially head 0).  The
 * code predictor, a second decoder of the same block structure, reads step
 * j's logits through its own head j: head 0 after its two-row prefill
 * (the Talker's last hidden state, then the codebook-0 embedding) and head j
 * at generation step j ("rightkit-qts 0.2.3 src/pipeline/tts_transformer.rs",
 * forward_code_pred_prefill_cached, forward_code_pred_step_cached).  Host
 * state only; nothing is enqueued.  Errors: QTALK_E_INVAL (head outside
 * 0 .. n_output_heads-1); the selection is then unchanged. */
qtalk_status qtalk_select_head(qtalk_ctx *ctx, int32_t head);

/* Block until the context's stream has finished all enqueued work.
 * Errors: QTALK_E_DEVICE if a kernel failed, or if a kernel reported a
 * failure of its own since the previous qtalk_sync:
 *  - a batch-1 decode (qtalk_decode, qtalk_decode_step, or a one- or
 *    two-row prefill/extend, which run on the same persistent kernel) gave
 *    up waiting for its other blocks, or its blocks were placed differently
 *    than set-up found (then later decodes use the slower
 *    placement-independent exchange), or a qtalk_decode_step's gathered
 *    input had an id outside its table.  Its
 *    outputs, and those of every later call, are not valid: each sequence
 *    such a decode wrote since the previous qtalk_sync is rolled back to
 *    the first position it wrote there (qtalk_kv_len shows the result, the
 *    message lists the sequences), and later calls work normally;
 *  - an id given to qtalk_embed_sum or picked by qtalk_argmax_embed was
 *    outside its table (those output rows hold NaN).
 * The status words are cleared either way. */
qtalk_status qtalk_sync(qtalk_ctx *ctx);

/* Test hook for the failure path above: a batch-1 decode enqueued after this
 * call gives up a wait after `polls` re-polls (0 restores the default, about
 * 1-2 s of polling).  Every block of a launch that gives up leaves the
 * kernel; nothing waits without bound.  Errors: QTALK_E_INVAL (polls < 0). */
qtalk_status qtalk_set_wait_limit(qtalk_ctx *ctx, int64_t polls);

/* Message of the last error on this context ("" if none).  The string lives
 * until the next call on the context. */
const char *qtalk_last_error(const qtalk_ctx *ctx);

#ifdef __cplusplus
}
#endif

#endif /* QTALK_H */
