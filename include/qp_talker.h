/* Talker decode step: the long-context transformer step that yields, per
 * request and audio frame, the frame hidden state H and the first codebook
 * token q0 that the Code Predictor (qp.h) consumes.
 *
 * Sources: the Talker attends over the request's whole history kept in a
 * paged KV cache and produces H and q0 for every frame (mixtureofinsights
 * OpenVINO port, section 1 diagram and sections 2.1-2.2; hackernews.jp
 * translation of the Nari Labs post, "Qwen3-TTSの最適化方法"); the history
 * is a per-request store of fixed capacity (forpes.ru RustTTS article,
 * "KV-Cache с блочным хранением"); 1.7B geometry: width 2048, 28 blocks,
 * 16 query / 8 kv heads of 128, FFN 6144, the predictor's block tensors, and
 * a 3072-row codec table (rightkit-qts exporter README, "Loader contract").
 *
 * Readings where the pages are silent:
 *   - the step's input row is the caller's (its composition, e.g. the
 *     previous frame's summed codebook embeddings plus text conditioning, is
 *     not part of this step);
 *   - the multimodal RoPE's three position streams coincide for codec
 *     frames, so keys and queries turn by rotate-half RoPE at the absolute
 *     position;
 *   - H is the final-norm output the codec head reads; q0 is the argmax over
 *     all head rows (lowest index on exact ties);
 *   - the cache holds keys (after per-head norm and RoPE) and values in bf16.
 *
 * Conventions as in qp.h: every call returns a qp_status; pointers to
 * per-step data are DEVICE pointers; calls are asynchronous on `stream`;
 * nothing aborts, and nothing is printed unless QP_LOG is set; calls on one
 * handle must not overlap (its staging buffers, graphs and split counters are
 * shared).  The library owns the KV cache; its slots are addressed by the
 * caller, so any request may use any slot in any batch. */
#ifndef QP_TALKER_H
#define QP_TALKER_H

#include "qp.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t d_model;      /* width (talker.embedding_length), multiple of 256  */
    int32_t n_layers;     /* block_count, >= 0                                 */
    int32_t n_q_heads;    /* attention.head_count                              */
    int32_t n_kv_heads;   /* attention.head_count_kv; n_q_heads = n_kv_heads
                             or 2 * n_kv_heads                                 */
    int32_t head_dim;     /* attention.key_length: 64 or 128; n_q_heads *
                             head_dim a multiple of 256                        */
    int32_t d_ffn;        /* feed_forward_length, multiple of 256              */
    int32_t vocab;        /* codec head rows (codec_vocab_size), multiple of 32 */
    float rms_eps;        /* attention.layer_norm_rms_epsilon, > 0             */
    float rope_base;      /* rope.freq_base, > 1                               */
    int32_t weight_dtype; /* QP_WEIGHT_BF16, QP_WEIGHT_Q8_0 or QP_WEIGHT_Q4_0  */
    int32_t max_batch;    /* largest B of a step, >= 1                         */
    int32_t n_slots;      /* KV cache slots (requests held at once), >= 1      */
    int32_t max_ctx;      /* positions per slot, >= 1                          */
} qp_talker_geometry;

/* Host pointers, copied by qp_talker_create (the caller may free them after
 * it returns).  Matrices row-major [out, in] in geometry.weight_dtype, norm
 * gains fp32. */
typedef struct {
    const qp_layer_weights* layers;  /* n_layers blocks (talker.blk.*)       */
    const float* output_norm;        /* talker.output_norm [d_model]         */
    const void* codec_head;          /* talker.codec_head [vocab, d_model]   */
} qp_talker_weights;

typedef struct qp_talker qp_talker;

/* Validate, allocate everything later calls need (the KV cache: 2 x n_slots x
 * n_layers x n_kv_heads x max_ctx x head_dim bf16), repack the weights, and
 * capture and instantiate the step graphs, one per batch bucket, kept until
 * qp_talker_destroy.  On failure *out is NULL and nothing is leaked. */
qp_status qp_talker_create(const qp_talker_weights* w, const qp_talker_geometry* g,
                           int32_t device, qp_talker** out);

/* Write a history of n positions into a slot: k, v are device bf16 bit
 * patterns [n_layers, n, n_kv_heads, head_dim] holding the keys (after the
 * per-head norm and RoPE) and values of positions 0..n-1.  0 <= slot <
 * n_slots, 0 <= n <= max_ctx, else QP_ERR_INVALID_ARG. */
qp_status qp_talker_load_history(qp_talker* t, int32_t slot, int32_t n,
                                 const uint16_t* k, const uint16_t* v, void* stream);

/* One decode step for B requests (0 <= B <= max_batch):
 *   x        float [B, d_model]  input rows
 *   slots    int32 [B]           KV slot of each request
 *   pos      int32 [B]           position of this step = history length; the
 *                                step attends over positions 0..pos and
 *                                writes its key and value at pos
 *   max_len  host int: an upper bound of pos[b] + 1 over the batch, in
 *            [1, max_ctx] (it sizes the attention grid)
 *   H_out    float [B, d_model]  frame hidden state
 *   q0_out   int32 [B]           argmax of the codec head
 *   logits_out float [B, vocab] or NULL
 * A row whose pos is negative, at or past max_ctx, or past the attention
 * grid that max_len sizes (pos >= max_len is only guaranteed to be caught
 * when it lies beyond that grid), or whose slot is outside [0, n_slots),
 * raises the sticky device flag (qp_talker_get_error), writes nothing into
 * the cache and returns unspecified values.
 * Without logits_out the step replays a graph that qp_talker_create
 * prepared for the smallest batch bucket holding B rows (buckets as for
 * qp_run_frames); its attention grid covers max_ctx, and the call's B and
 * max_len (the split limit above) are written to device memory before the
 * replay.  With logits_out the same kernels are launched directly with a grid
 * sized by max_len.  No step captures, instantiates or frees a graph. */
qp_status qp_talker_step(qp_talker* t, int32_t B, const float* x, const int32_t* slots,
                         const int32_t* pos, int32_t max_len, float* H_out, int32_t* q0_out,
                         float* logits_out, void* stream);

/* Synchronise, then return and clear the sticky flag: QP_OK, or
 * QP_ERR_DEVICE_FLAG (bits from qp_talker_last_device_flags: 1 = position
 * out of range, 2 = slot out of range). */
qp_status qp_talker_get_error(qp_talker* t);
uint32_t qp_talker_last_device_flags(qp_talker* t);

/* Free everything; NULL is allowed. */
void qp_talker_destroy(qp_talker* t);

#ifdef __cplusplus
}
#endif

#endif /* QP_TALKER_H */
