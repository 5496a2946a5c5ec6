/*
 * qp.h — C ABI of the MI355X (gfx950) Code Predictor library.
 *
 * The library runs the Qwen3-TTS Code Predictor ("Subcode") loop: per audio
 * frame and per request it takes the Talker's frame hidden state H and the
 * first codebook token q0, greedily emits the remaining 15 RVQ codebook
 * tokens through a small Qwen3-style transformer, and returns the sum of the
 * frame's 16 codebook embeddings.
 *
 *   - Three modules, the predictor emitting the 15 tokens after the Talker's
 *     first one, in a fixed 15-step loop per frame: hackernews.jp story
 *     49389952 (translation of the Nari Labs post), section
 *     "Qwen3-TTSの最適化方法", subsections 1 and 3; agentlenshq.com summary,
 *     "Qwen3-TTS 的架构优化" / "Code Predictor 与 Codec 增强".
 *   - Stateless, greedy, batched, KV-cached, fed by H: mixtureofinsights.com
 *     "拆解 Qwen3-TTS", section 2.2.
 *   - Geometry keys, tensor names, projection and shapes: docs.rs
 *     rightkit-qts 0.2.3 scripts/README.md ("Qwen3-TTS 1.7B → QTS GGUF"),
 *     "Loader contract" and "Expected verification shapes".
 *   - EMA codebooks (embedding_sum / (cluster_usage + 1e-7)): forpes.ru post
 *     217414 (Qwen3-TTS in Rust), "Проблема 1: Формат codebook'ов".
 *   - 16 RVQ codebooks: same post, "Компоненты".
 *
 * Conventions
 *   - Every function returns a qp_status (0 = success, negative = error) and
 *     never aborts.  qp_last_error() returns a text for the last failing call
 *     on the calling thread.  Nothing is printed unless the environment
 *     variable QP_LOG is set; then each failure also writes that text and the
 *     status name to stderr, one line per failure.
 *   - For tests only: QP_TEST_EPOCH0, if set when qp_create runs, is the first
 *     32-bit record tag of the new handle's dataflow frames (small and
 *     moderate batches; the tags restart, after every record is cleared,
 *     before they would wrap; a test sets it near that point).  Results do
 *     not depend on it.
 *   - Weight pointers given to qp_create are HOST pointers; the library copies
 *     and repacks everything before returning, so the caller keeps ownership
 *     and may free them afterwards.
 *   - Pointers given to qp_run_frames / qp_run_frames_ex are DEVICE pointers
 *     on the handle's device, owned by the caller.  The calls only enqueue
 *     work on `stream` (a hipStream_t, NULL = the null stream) and do not
 *     synchronise; argument checks happen on the host before anything is
 *     enqueued.
 *   - A handle owns its device scratch (KV cache, activations, barrier words);
 *     calls on one handle must not overlap (one in flight at a time, e.g. all
 *     on one stream).  Different handles are independent.
 *   - Matrices are HF row-major [out, in].
 */
#ifndef QP_H
#define QP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QP_N_CODEBOOKS 16            /* q0 from the Talker + 15 predicted  */
#define QP_N_STEPS (QP_N_CODEBOOKS - 1)

typedef enum {
    QP_OK = 0,
    QP_ERR_INVALID_ARG = -1,   /* NULL pointer, negative size, bad flag       */
    QP_ERR_GEOMETRY = -2,      /* inconsistent or unsupported geometry        */
    QP_ERR_SHAPE = -3,         /* a size that does not fit the weight format  */
    QP_ERR_DTYPE = -4,         /* unknown weight dtype or embedding format    */
    QP_ERR_OOM = -5,           /* device allocation failed                    */
    QP_ERR_HIP = -6,           /* a HIP runtime call failed                   */
    QP_ERR_BATCH = -7,         /* B outside [0, max_batch]                    */
    QP_ERR_DEVICE_FLAG = -8    /* a kernel flagged bad data (see qp_get_error)*/
} qp_status;

/* Storage type of every linear: projection, q/k/v/o, gate/up/down, heads. */
typedef enum {
    QP_WEIGHT_F32 = 0,
    QP_WEIGHT_BF16 = 1,   /* uint16 bfloat16 bit patterns                     */
    QP_WEIGHT_Q8_0 = 2,   /* GGUF Q8_0: per row, in/32 blocks of 34 bytes =
                             little-endian f16 scale d, then 32 int8 codes q;
                             value = q * d (rightkit-qts README: Q8_0 through
                             gguf's quantizer)                                 */
    QP_WEIGHT_Q4_0 = 3    /* GGUF Q4_0: per row, in/32 blocks of 18 bytes =
                             little-endian f16 scale d, then 16 bytes, byte j
                             holding the 4-bit code c of element j (low
                             nibble) and of element j + 16 (high nibble);
                             value = (c - 8) * d (forpes.ru RustTTS article,
                             "Поддержка GGUF-квантизации": q4_0 GGUF files)  */
} qp_weight_dtype;

/* Storage of the 16 codebook tables [V, d_talker]. */
typedef enum {
    QP_EMB_F32 = 0,
    QP_EMB_BF16 = 1,
    QP_EMB_EMA = 2        /* fp32 embedding_sum [V, d_talker] + cluster_usage
                             [V]; the table is sum / (usage + 1e-7) row-wise,
                             computed once on the device by qp_create          */
} qp_emb_format;

/* Predictor geometry; mirrors the exporter's qwen3-tts.code_pred.* keys. */
typedef struct {
    int32_t d_talker;     /* dT: width of H and of the codebook tables        */
    int32_t d_model;      /* dP: predictor hidden width (embedding_length)    */
    int32_t n_layers;     /* L  (layer_count)                                 */
    int32_t n_q_heads;    /* nq (attention.head_count)                        */
    int32_t n_kv_heads;   /* nkv (attention.head_count_kv), nq % nkv == 0     */
    int32_t head_dim;     /* hd (attention.key_length), even                  */
    int32_t d_ffn;        /* F  (feed_forward_length)                         */
    int32_t vocab;        /* V  per codebook (vocab_size)                     */
    int32_t n_codebooks;  /* must be QP_N_CODEBOOKS                           */
    float rms_eps;        /* attention.layer_norm_rms_epsilon, > 0            */
    float rope_base;      /* rope.freq_base, > 1                              */
    int32_t weight_dtype; /* qp_weight_dtype (Q8_0, Q4_0: every input width a
                             multiple of 32)                                 */
    int32_t emb_format;   /* qp_emb_format                                    */
    int32_t max_batch;    /* largest B a later qp_run_frames may pass, >= 1   */
} qp_geometry;

/* One decoder block (suffixes attn_norm, attn_q, attn_k, attn_v, attn_output,
 * attn_q_norm, attn_k_norm, ffn_norm, ffn_gate, ffn_up, ffn_down).  Matrices
 * are in geometry.weight_dtype; norm gains are fp32. */
typedef struct {
    const float* attn_norm;  /* [dP]                                          */
    const void* wq;          /* [nq*hd, dP]                                   */
    const void* wk;          /* [nkv*hd, dP]                                  */
    const void* wv;          /* [nkv*hd, dP]                                  */
    const void* wo;          /* [dP, nq*hd]                                   */
    const float* q_norm;     /* [hd] per-head RMSNorm gain on q               */
    const float* k_norm;     /* [hd] per-head RMSNorm gain on k               */
    const float* ffn_norm;   /* [dP]                                          */
    const void* w_gate;      /* [F, dP]                                       */
    const void* w_up;        /* [F, dP]                                       */
    const void* w_down;      /* [dP, F]                                       */
} qp_layer_weights;

typedef struct {
    const void* proj_w;      /* small_to_mtp_projection.weight [dP, dT]       */
    const float* proj_b;     /* small_to_mtp_projection.bias [dP]             */
    /* Codebook tables, index j embeds token q_j: emb[0] is the Talker's
     * codebook-0 table, emb[j] = codec_embd.{j-1} for j = 1..15.
     * QP_EMB_F32 / QP_EMB_BF16: emb[j] -> [V, dT] (float / uint16 bf16).
     * QP_EMB_EMA: ema_sum[j] -> float [V, dT], ema_usage[j] -> float [V].   */
    const void* emb[QP_N_CODEBOOKS];
    const float* ema_sum[QP_N_CODEBOOKS];
    const float* ema_usage[QP_N_CODEBOOKS];
    const qp_layer_weights* layers;   /* n_layers entries                    */
    const float* out_norm;   /* output_norm [dP]                              */
    /* lm_head.{k-1} [V, dP] predicts q_k, k = 1..15                          */
    const void* lm_head[QP_N_STEPS];
} qp_weights;

typedef struct qp_handle qp_handle;

/* Build a predictor on HIP device `device`: validates the geometry (first
 * failure returned as status), allocates every device buffer the later calls
 * need for up to max_batch requests (later calls never allocate), copies and
 * repacks the weights, computes EMA tables and the per-codebook projected
 * tables W_p . E_j + b_p.  Where the batched matrix-core path applies, it
 * also captures and instantiates that path's frame graphs, one per batch
 * bucket (greedy, and sampled for V <= 4096), kept until qp_destroy.  For the 1.7B geometry with bf16, Q8_0 or Q4_0
 * weights (the small-batch dataflow driver) it also computes layer 0's q/k/v
 * rows of every projected-table row of codebooks 1..14 (fp32, 14 x V x
 * (nq + 2 nkv) hd values, 470 MB), which that driver reads from step 2 on.
 * On failure *out is NULL and nothing is leaked. */
qp_status qp_create(const qp_weights* w, const qp_geometry* g, int32_t device,
                    qp_handle** out);

/* One audio frame for B independent requests (0 <= B <= max_batch; B = 0 is
 * a no-op).  Device pointers:
 *   H          float [B, dT]   Talker frame hidden states
 *   q0         int32 [B]       codebook-0 tokens in [0, V)
 *   tokens_out int32 [B, 15]   q1..q15 (greedy; lowest index on exact ties)
 *   embsum_out float [B, dT]   E_0[q0] + E_1[q1] + ... + E_15[q15], fp32,
 *                              summed in that order
 * Row b of the outputs depends only on (H[b], q0[b]).  An out-of-range q0 is
 * replaced by 0 and raises the sticky device flag (qp_get_error).
 * On the batched matrix-core path the frame replays a graph that qp_create
 * prepared for the smallest batch bucket holding B rows (buckets 1, 2, 4, 8,
 * 16, 32, 48, 64, 96, 128, 192, ... below max_batch, and max_batch); the
 * bucket's extra rows are computed on zero inputs and not returned.  No call
 * captures, instantiates or frees a graph, and none allocates. */
qp_status qp_run_frames(qp_handle* h, int32_t B, const float* H,
                        const int32_t* q0, int32_t* tokens_out,
                        float* embsum_out, void* stream);

/* qp_run_frames for callers that cannot allocate device memory or must not
 * touch a handle's scratch between calls (code under stream capture, tight
 * serving loops, harnesses that forbid allocation): the same frame, on the
 * small-batch dataflow driver, with that driver's scratch (its exchange
 * records and a two-request KV cache, 1,646,592 bytes) in a static device
 * array that each GPU holds until the process ends, set up by the first
 * qp_create of a dataflow-capable handle on that GPU.  The call allocates
 * nothing and frees nothing.
 *   - Only handles of the 1.7B predictor geometry with bf16, Q8_0 or Q4_0
 *     weights (the dataflow driver), else QP_ERR_INVALID_ARG.
 *   - 0 <= B <= min(2, max_batch), else QP_ERR_BATCH (the static array holds
 *     two requests); B = 0 is a no-op.
 *   - Arguments, outputs, results and the sticky device flag are those of
 *     qp_run_frames; results equal qp_run_frames' bit for bit.
 *   - Every call on one GPU, from any handle, shares that GPU's array: calls
 *     that overlap on one GPU (on different streams, or from different
 *     threads without ordering) race and give wrong results.  Calls ordered
 *     on one stream are safe. */
qp_status qp_run_frames_noalloc(qp_handle* h, int32_t B, const float* H,
                                const int32_t* q0, int32_t* tokens_out,
                                float* embsum_out, void* stream);

/* Execution strategy hints for qp_run_frames_ex `flags`. */
#define QP_FLAG_STEPWISE 0x1u   /* one kernel per phase (no persistent kernel) */
#define QP_FLAG_GENERIC 0x2u    /* the generic persistent kernel even where a
                                   specialised one exists                      */
#define QP_FLAG_TILED 0x4u      /* the batched matrix-core path (one kernel per
                                   phase, projections on MFMA) for any B; only
                                   for bf16, Q8_0 or Q4_0 weights with dT, dP, nq*hd
                                   and F multiples of 256, dP and dT <= 4096, nqkv and V multiples
                                   of 32 (else QP_ERR_INVALID_ARG); excludes
                                   the other flags                            */
#define QP_FLAG_FLOW 0x8u       /* the moderate-batch dataflow kernel (1.7B
                                   predictor geometry with bf16 weights,
                                   B <= 16, else QP_ERR_INVALID_ARG); excludes
                                   the other flags.
   Without flags the library picks: B <= 2 with bf16, Q8_0 or Q4_0 weights
   and the 1.7B predictor geometry -> the small-batch dataflow kernel;
   3 <= B <= 16 with bf16 weights and that geometry -> the moderate-batch
   dataflow kernel (matrix-core products); otherwise, where the batched path
   applies -> it; otherwise the generic persistent kernel. */

/* Same computation with test hooks (any hook may be NULL):
 *   force_tokens int32 [B, 15]  teacher forcing: the token fed back at step
 *                               k and summed into embsum is force[b, k-1];
 *                               tokens_out still receives the model's argmax
 *   logits_out   float [B, 15, V]   the fp32 logits of every step
 *   taps_out     float [16, L, B, dP]  residual stream after every layer at
 *                               every position (position 0 = H's row)
 *   flags        QP_FLAG_* */
qp_status qp_run_frames_ex(qp_handle* h, int32_t B, const float* H,
                           const int32_t* q0, int32_t* tokens_out,
                           float* embsum_out, void* stream,
                           const int32_t* force_tokens, float* logits_out,
                           float* taps_out, uint32_t flags);

/* Caller-controlled sampling.  The pages leave sampling to the caller (the
 * GGUF loaders do not read the generation config: rightkit-qts exporter
 * README, "Qwen3-TTS 1.7B -> QTS GGUF", section "Usage") and describe the
 * exported predictor loop as greedy.  A sampled step replaces the argmax by
 * this draw from the step's fp32 logits z:
 *   1. rank order: descending logit, lower vocabulary index first on ties;
 *   2. weights w_r = exp((z_r - z_0) / temperature), z_0 the largest logit;
 *   3. top-k: the first top_k ranks stay (0 = all);
 *   4. top-p: of those, the shortest rank-order prefix whose weight reaches
 *      top_p times their total stays (at least one token; 1 = all);
 *   5. the token is the first kept rank whose inclusive cumulative weight
 *      exceeds u times the kept total, u being the caller's uniform for that
 *      request and step (clamped to [0, 1], NaN as 0), else the last kept rank.
 * The weights are summed in fp32; only draws whose threshold lies within
 * about 2e-6 of the total from a cumulative boundary can differ from exact
 * arithmetic.
 * top_k = 1 reproduces the argmax. */
typedef struct {
    float temperature;  /* finite, > 0                                  */
    int32_t top_k;      /* >= 0; 0 keeps every token                    */
    float top_p;        /* in (0, 1]; 1 keeps every token top-k kept     */
} qp_sampling;

/* One frame with every step's token drawn as above instead of the argmax.
 * Same arguments as qp_run_frames_ex, plus:
 *   sampling     host pointer, read before return (one setting for all rows)
 *   uniforms     float [B, 15] device: the draw of step k for request b is
 *                uniforms[b, k-1]
 * tokens_out receives the drawn tokens; force_tokens (may be NULL) overrides
 * the fed-back token as in qp_run_frames_ex, logits_out (may be NULL) receives
 * the logits.  Runs on the batched matrix-core path (its weight and geometry
 * conditions under QP_FLAG_TILED, and V <= 4096), else QP_ERR_INVALID_ARG;
 * invalid parameters give QP_ERR_INVALID_ARG.  Without hooks the frame
 * replays the bucket's prepared graph, as qp_run_frames does. */
qp_status qp_run_frames_sampled(qp_handle* h, int32_t B, const float* H,
                                const int32_t* q0, const qp_sampling* sampling,
                                const float* uniforms, int32_t* tokens_out,
                                float* embsum_out, void* stream,
                                const int32_t* force_tokens, float* logits_out);

/* The draw alone, on caller-provided logits (no handle needed).  Device
 * pointers: logits float [rows, row_stride] (the first V of each row are
 * read), uniforms float with row r's uniform at uniforms[r * uniform_stride],
 * tokens_out int32 [rows].  1 <= V <= 4096, row_stride >= V,
 * uniform_stride >= 1, else QP_ERR_INVALID_ARG; rows = 0 is a no-op.
 * Asynchronous on `stream` (a hipStream_t). */
qp_status qp_sample_logits(const float* logits, int32_t rows, int32_t V,
                           int64_t row_stride, const qp_sampling* sampling,
                           const float* uniforms, int32_t uniform_stride,
                           int32_t* tokens_out, void* stream);

/* Synchronise the handle's device, then return and clear the sticky device
 * flag: QP_OK, or QP_ERR_DEVICE_FLAG when a kernel saw an out-of-range token
 * (q0 or a forced token) or a grid barrier timed out since the last call. */
qp_status qp_get_error(qp_handle* h);

/* Raw flag bits behind the last QP_ERR_DEVICE_FLAG (1 = bad q0, 2 = bad
 * forced token, 4 = barrier timeout); 0 when none. */
uint32_t qp_last_device_flags(qp_handle* h);

/* Free everything; NULL is allowed. */
void qp_destroy(qp_handle* h);

const char* qp_status_string(int32_t status);

/* Text describing the last failing call on this thread ("" if none). */
const char* qp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QP_H */
