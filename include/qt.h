/*
 * qt.h - C ABI of the Qwen3-TTS 12 Hz per-frame generation step on MI355X.
 *
 * What one frame computes (Mizuoto engine page, "How it works"; ncnn port
 * discussion 6798, section 1 "structure"):
 *   - the code predictor, a 5-layer Qwen3-style decoder with 15 embedding
 *     tables and 15 heads, runs a 2-token prefill [previous talker hidden ;
 *     talker codec embedding of code 0] and applies head 0 to get code 1, then
 *     14 autoregressive steps where step s embeds code s with table s-1 and
 *     applies head s to get code s+1;
 *   - the 16 codes form one 80 ms frame; the sum of their embeddings plus the
 *     next trailing text embedding (tts_pad once the text is used up) is the
 *     next talker input;
 *   - the 28-layer talker decoder runs one step on that input and its codec
 *     head picks the next code 0 through the logits processors (repetition
 *     penalty -> min-new-tokens EOS mask -> suppress [suppress_begin,
 *     suppress_end) except EOS -> greedy argmax, or temperature -> top-k ->
 *     top-p -> one exponential-race draw argmax(p / Exp(1))).
 * N frames therefore take N+1 talker selections and 15 N predictor passes
 * (ncnn CustomVoice port discussion 6832, section 3.1).
 *
 * Conventions for every entry point:
 *   - All device pointers point to memory the caller owns, allocated on the
 *     device the context was created on; all work is enqueued on the stream
 *     given to qt_create. Host pointers are plain host memory.
 *   - Weight matrices are row-major [out, in] (nn.Linear layout); every
 *     weight tensor (matrices, norm gains, tables, heads) has element type
 *     qt_config.weight_dtype (QT_DTYPE_F32: float, QT_DTYPE_BF16: the upper 16
 *     bits of a float). Activations, prompts and logits are float32.
 *   - Arguments are validated before any device work (dimensions, sizes,
 *     capacity, id ranges - ncnn CustomVoice port section 3.6: every length
 *     and id is checked before an embedding access or copy). On error nothing
 *     is written, the status code is returned and qt_last_error() describes
 *     it. No C++ exception crosses this boundary.
 *   - Non-finite logits (NaN or +inf) seen on the device are reported at the
 *     once-per-frame synchronisation as QT_E_NAN (Mizuoto "Speed": a NaN
 *     probability is still an error, read at the one wait per frame); the
 *     context then needs a new qt_prefill.
 */
#ifndef QT_H
#define QT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t qt_status;
#define QT_OK 0
#define QT_E_INVALID 1  /* bad argument or dimension                           */
#define QT_E_RANGE 2    /* id or length out of range                            */
#define QT_E_CAPACITY 3 /* B > max_batch or P_r + max_frames > max_positions    */
#define QT_E_NOMEM 4    /* workspace too small / allocation failed              */
#define QT_E_HIP 5      /* HIP runtime error                                    */
#define QT_E_NAN 6      /* non-finite logit seen on the device                  */
#define QT_E_STATE 7    /* call out of order                                    */

#define QT_DTYPE_F32 0
#define QT_DTYPE_BF16 1
#define QT_DTYPE_F16 2   /* IEEE half: KV caches only */

/* Dimensions of one Qwen3-style decoder (talker or code predictor). */
typedef struct qt_decoder_dims {
  int32_t layers;
  int32_t hidden;       /* multiple of 64                                       */
  int32_t n_heads;      /* q heads; n_heads / n_kv_heads is 1, 2, 4 or 8         */
  int32_t n_kv_heads;
  int32_t head_dim;     /* even, 16..256; n_heads*head_dim multiple of 64       */
  int32_t intermediate; /* SwiGLU width, multiple of 64                         */
  float rope_theta;
  float rms_eps;
} qt_decoder_dims;

typedef struct qt_config {
  qt_decoder_dims talker;
  qt_decoder_dims predictor;
  int32_t talker_vocab;   /* codec vocabulary of the talker head (3072), <= 6144 */
  int32_t n_groups;       /* codes per frame; must be 16                        */
  int32_t codebook;       /* predictor vocabulary (2048), <= 6144               */
  int32_t eos_id;         /* 2150                                               */
  int32_t suppress_begin; /* 2048: talker ids in [begin, end) except EOS are    */
  int32_t suppress_end;   /* 3072: never chosen                                 */
  int32_t pred_in_proj;   /* 1: predictor inputs pass a [Hp, H] projection;     */
                          /* 0: requires predictor.hidden == talker.hidden      */
  int32_t weight_dtype;   /* QT_DTYPE_F32 | QT_DTYPE_BF16                       */
  int32_t kv_dtype;       /* element type of both KV caches: F32 | BF16 | F16   */
  int32_t max_batch;      /* rows per prefill                                   */
  int32_t max_positions;  /* talker cache length per row                        */
} qt_config;

/* Device pointers of one decoder layer (element type weight_dtype). */
typedef struct qt_layer_weights {
  const void* attn_norm; /* [H]               */
  const void* wq;        /* [n_heads*d, H]    */
  const void* wk;        /* [n_kv*d, H]       */
  const void* wv;        /* [n_kv*d, H]       */
  const void* q_norm;    /* [d]               */
  const void* k_norm;    /* [d]               */
  const void* wo;        /* [H, n_heads*d]    */
  const void* mlp_norm;  /* [H]               */
  const void* w_gate;    /* [I, H]            */
  const void* w_up;      /* [I, H]            */
  const void* w_down;    /* [H, I]            */
} qt_layer_weights;

typedef struct qt_weights {
  const qt_layer_weights* talker_layers; /* host array [talker.layers]                  */
  const void* talker_norm;               /* [H] final norm of the talker                */
  const void* talker_codec_embed;        /* [talker_vocab, H]                           */
  const void* talker_codec_head;         /* [talker_vocab, H]                           */
  const qt_layer_weights* pred_layers;   /* host array [predictor.layers]               */
  const void* pred_norm;                 /* [Hp]                                        */
  const void* pred_embeds;               /* [15*codebook, H]: table j at rows j*codebook */
  const void* pred_heads;                /* [15*codebook, Hp]: head s at rows s*codebook */
  const void* pred_in_proj;              /* [Hp, H] or NULL when pred_in_proj == 0      */
} qt_weights;

/* Logits processing of one selector (talker or predictor). */
typedef struct qt_sampling {
  int32_t do_sample;        /* 0: greedy argmax, lowest index on ties              */
  float temperature;        /* > 0                                                 */
  int32_t top_k;            /* 0 disables                                          */
  float top_p;              /* (0, 1]; 1 disables                                  */
  float repetition_penalty; /* talker only: >= 1 (1 disables)                      */
  int32_t min_new_tokens;   /* talker only: EOS masked while selections < this     */
} qt_sampling;

typedef struct qt_ctx qt_ctx;

/* Device bytes qt_create needs for this configuration (packed weights, the
 * code predictor's code-indexed first-layer tables, KV caches, activations,
 * row state). Host-only arithmetic; overflow-checked. */
qt_status qt_workspace_bytes(const qt_config* cfg, size_t* bytes);

/* Validate a configuration without touching any device. */
qt_status qt_config_check(const qt_config* cfg);

/* Create a context on the current HIP device. Copies and repacks the weights
 * (fused q/k/v and gate/up matrices) into `workspace` (device memory of at
 * least qt_workspace_bytes bytes, owned by the caller and kept alive until
 * qt_destroy), so the caller may free its weight buffers afterwards. It also
 * tabulates, for each of the 14 single-token code predictor steps and every
 * code of that step's input table, the first layer's q/k/v of the code's
 * embedding row (the step's input depends on the code alone), so the frame
 * reads one table row where it would stream the q/k/v weights. With
 * workspace == NULL the library allocates the workspace itself and frees it
 * in qt_destroy. hip_stream: a hipStream_t (NULL = the default stream). */
qt_status qt_create(const qt_config* cfg, const qt_weights* w, void* workspace, size_t ws_bytes,
                    void* hip_stream, qt_ctx** out);

/* Start generation for B rows (the prompt prefill; ncnn port section 5).
 *   prompt      device float [sum(prompt_lens), H]: row r's prompt embeddings
 *               packed after row r-1's, positions 0..P_r-1
 *   prompt_lens host int32 [B], each >= 1
 *   text        device float [sum(text_lens), H] or NULL: trailing text
 *               embeddings; frame k of row r adds text row k while k < n_r
 *   text_lens   host int32 [B] or NULL (NULL: no trailing text)
 *   tts_pad     device float [H]: added once the text is used up
 *   talker, predictor: processor / warper settings
 *   seed        key of the sampling noise (Philox4x64-10, counter = (vocab
 *               id, stream, selection index, row))
 *   max_frames  >= 1; P_r + max_frames <= max_positions
 * Runs the talker over the prompts, applies the codec head at each row's last
 * position and performs talker selection 0 (ncnn CustomVoice port section
 * 3.1: step 0 only selects the first code 0). Synchronises the stream. */
qt_status qt_prefill(qt_ctx* ctx, int32_t B, const float* prompt, const int32_t* prompt_lens,
                     const float* text, const int32_t* text_lens, const float* tts_pad,
                     const qt_sampling* talker, const qt_sampling* predictor, uint64_t seed,
                     int32_t max_frames);

/* One frame for every row: predictor codes 1..15 for the current code 0, the
 * feedback sum, one talker step and the next talker selection (the
 * lookahead). One host synchronisation.
 *   codes  host int32 [B, 16]: the frame (code 0, codes 1..15)
 *   state  host uint8 [B]: 0 active; 1 finished with this frame (the
 *          lookahead is EOS: reason stop); 2 finished with this frame
 *          (max_frames reached: reason length, lookahead discarded); 3 row
 *          had already finished (codes undefined; the row is fed EOS).
 * Each row ends on its own frame cap (max_frames of qt_prefill or
 * qt_admit). Returns QT_E_STATE when every row has finished or no prefill
 * was done. */
qt_status qt_step_frame(qt_ctx* ctx, int32_t* codes, uint8_t* state);

/* Continuous batching (Mizuoto engine page, "Matching upstream", sampler
 * bullet: finished rows of a batch are fed EOS; the SGLang-Omni case runs
 * the talker as a serving stage with requests joining a running batch): start
 * a new request in a slot whose request has finished, between two frames,
 * while the other rows keep generating. The slot's talker prefill over its
 * prompt (its K/V rows), selection 0 and its row state (position, frame
 * counter, seen ids, noise key) are reset; the other rows are untouched and
 * the next qt_step_frame carries the slot with them.
 *   slot        0..B-1 of the running batch; its request must have finished
 *               (state 1 or 2 reported earlier), else QT_E_STATE
 *   prompt      device float [prompt_len, H]; prompt_len >= 1
 *   text        device float [text_len, H] trailing text rows, or NULL
 *               (text_len 0); kept by the caller until the request ends
 *   seed, noise_row  the sampling noise of this request: key (seed, 0),
 *               counter row noise_row (a request reproduces row noise_row of
 *               a batch started with this seed)
 *   max_frames  this request's frame cap; prompt_len + max_frames <= max_positions
 * The sampling settings and tts_pad are those of qt_prefill. Synchronises.
 * The slot's first frame comes with the next qt_step_frame; a slot whose
 * selection 0 is already EOS is reported finished (state 3) there. */
qt_status qt_admit(qt_ctx* ctx, int32_t slot, const float* prompt, int32_t prompt_len, const float* text,
                   int32_t text_len, uint64_t seed, int32_t noise_row, int32_t max_frames);

/* qt_prefill + qt_step_frame until every row finished.
 *   codes    host int32 [B, max_frames, 16]; frames past n_frames[r] untouched
 *   n_frames host int32 [B]
 *   finish   host uint8 [B]: 1 stop (EOS), 2 length (max_frames) */
qt_status qt_generate(qt_ctx* ctx, int32_t B, const float* prompt, const int32_t* prompt_lens,
                      const float* text, const int32_t* text_lens, const float* tts_pad,
                      const qt_sampling* talker, const qt_sampling* predictor, uint64_t seed,
                      int32_t max_frames, int32_t* codes, int32_t* n_frames, uint8_t* finish);

/* Release the context and everything it allocated. NULL is a no-op. */
void qt_destroy(qt_ctx* ctx);

/* Text of the last error of `ctx` (or of the calling thread when ctx is NULL:
 * errors of qt_create / qt_config_check). Never NULL. */
const char* qt_last_error(const qt_ctx* ctx);

/* ---- token-id frontend (ncnn port discussion 6798, section 1 "structure",
 * Talker and generation-loop bullets; section 8 on built-in voices) ----
 * Text ids index a text embedding table whose rows a ResizeMLP maps to the
 * talker's width: row = W2 · silu(W1 · text_embed[id] + b1) + b2 (the text
 * track). A prompt row adds, position by position, the text track of a text
 * id and the codec track of a codec id, talker_codec_embed[id] (role,
 * language and think prefixes, codec_bos / codec_pad; a built-in voice's
 * speaker row is the codec row of its speaker id). Id -1 leaves a track
 * empty (a zero row). The tokenizer that makes the ids is not part of this
 * library. */
typedef struct qt_frontend_config {
  int32_t text_vocab;   /* rows of the text embedding (151936 for the Qwen2 vocabulary)   */
  int32_t text_hidden;  /* width of a text embedding row (2048), multiple of 8, <= 24576   */
  int32_t mlp_hidden;   /* inner width of the ResizeMLP (2048), multiple of 8, <= 24576    */
  int32_t max_rows;     /* most rows one qt_embed_ids / qt_prefill_ids call embeds          */
} qt_frontend_config;

/* Device pointers, element type qt_config.weight_dtype, row-major [out, in]. */
typedef struct qt_frontend_weights {
  const void* text_embed; /* [text_vocab, text_hidden]                        */
  const void* fc1_w;      /* [mlp_hidden, text_hidden]                        */
  const void* fc1_b;      /* [mlp_hidden] or NULL (zero bias)                 */
  const void* fc2_w;      /* [talker.hidden, mlp_hidden]                      */
  const void* fc2_b;      /* [talker.hidden] or NULL (zero bias)              */
} qt_frontend_weights;

/* Device bytes qt_attach_frontend needs (packed weights, id arrays, the MLP's
 * row buffers and scratch, the assembled rows of qt_prefill_ids). */
qt_status qt_frontend_bytes(const qt_config* cfg, const qt_frontend_config* fc, size_t* bytes);

/* Copy / repack the frontend weights into `workspace` (device, at least
 * qt_frontend_bytes, caller-owned until qt_destroy; NULL: the library
 * allocates and frees it). Replaces an earlier frontend. Synchronises the
 * context's stream. */
qt_status qt_attach_frontend(qt_ctx* ctx, const qt_frontend_config* fc, const qt_frontend_weights* fw,
                             void* workspace, size_t ws_bytes);

/* Dual-track rows for n positions: out[i] = text track(text_ids[i]) + codec
 * track(codec_ids[i]) (+ extra[i]).
 *   text_ids   host int32 [n], each -1 or in 0..text_vocab-1
 *   codec_ids  host int32 [n], each -1 or in 0..talker_vocab-1
 *   extra      device float [n, talker.hidden] or NULL (e.g. x-vector rows)
 *   out        device float [n, talker.hidden]
 * out and extra 16-byte aligned; 1 <= n <= max_rows. Ids are checked on the
 * host before any device work (QT_E_RANGE). Enqueued on the context's stream
 * (the host id arrays are free to reuse on return). QT_E_STATE without a
 * frontend. */
qt_status qt_embed_ids(qt_ctx* ctx, int32_t n, const int32_t* text_ids, const int32_t* codec_ids,
                       const float* extra, float* out);

/* qt_prefill from ids: the prompt rows of every row (prompt_lens[r] positions
 * each, packed row after row in text_ids / codec_ids), the trailing text rows
 * (trailing_ids packed the same way, trailing_lens[r] each, text track only;
 * trailing_lens NULL: none) and tts_pad's row (the text track of
 * tts_pad_id) are embedded by the frontend into its own workspace, where
 * they stay for the frames of this request; then exactly qt_prefill. Rows
 * embedded: sum(prompt_lens) + sum(trailing_lens) + 1 <= max_rows. */
qt_status qt_prefill_ids(qt_ctx* ctx, int32_t B, const int32_t* text_ids, const int32_t* codec_ids,
                         const int32_t* prompt_lens, const int32_t* trailing_ids, const int32_t* trailing_lens,
                         int32_t tts_pad_id, const qt_sampling* talker, const qt_sampling* predictor, uint64_t seed,
                         int32_t max_frames);

/* ---- the 12 Hz codec decoder: codes -> 24 kHz audio (ncnn port discussion
 * 6798, section 1 "structure", Codec Decoder bullet; Mizuoto engine page,
 * "Matching upstream" codec bullet and "Speed" frame-streaming bullet) ----
 * Per frame of 16 codes: SplitRVQ dequantisation (code 0 from the semantic
 * codebook, codes 1..15 from the acoustic ones; each group's sum projected
 * codebook_dim -> hidden and the two added), a transformer whose attention
 * sees `window` frames (pre-norm LayerNorm blocks, rope at positions from 0,
 * GELU MLP, LayerScale), a final LayerNorm, two upsampling stages (causal
 * transposed convolution kernel 2 stride 2, then a ConvNeXt block: causal
 * depthwise convolution kernel 7, LayerNorm, GELU MLP, LayerScale, residual),
 * and a DAC-style vocoder (causal convolution kernel 7 to channels[0]; per
 * block b: SnakeBeta, causal transposed convolution kernel 2 strides[b] to
 * channels[b+1], residual units with the given dilations: SnakeBeta, causal
 * dilated convolution kernel 7, SnakeBeta, convolution kernel 1, add; then
 * SnakeBeta, causal convolution kernel 7 to one channel, tanh). The decoder
 * is causal: samples of frames 0..t depend on codes of frames 0..t only.
 * hop = 4 * prod(strides) samples per frame (1920 at 24 kHz for 8, 5, 4, 3).
 * Weight element type weight_dtype; matrices [out, in]; convolution weights
 * tap-major [k][out][in]; depthwise weights [7][channels]. */
#define QT_CODEC_MAX_BLOCKS 6
#define QT_CODEC_UNITS 3
typedef struct qt_codec_config {
  int32_t n_q;            /* codebooks per frame: 16                                   */
  int32_t codebook;       /* entries per codebook: 2048                                */
  int32_t codebook_dim;   /* 256, multiple of 8                                        */
  int32_t hidden;         /* transformer / upsampling width: 512, multiple of 64       */
  int32_t layers;         /* transformer layers: 8                                     */
  int32_t heads;          /* 8                                                         */
  int32_t head_dim;       /* 64 (even, <= 128)                                         */
  int32_t ffn;            /* transformer MLP width: 2048, multiple of 8                */
  int32_t window;         /* attention window in frames: 72                            */
  float rope_theta;       /* 1e4                                                       */
  int32_t up_ffn;         /* ConvNeXt MLP width: 2048, multiple of 8                   */
  int32_t n_blocks;       /* vocoder blocks: 4 (<= QT_CODEC_MAX_BLOCKS)                */
  int32_t channels[QT_CODEC_MAX_BLOCKS + 1]; /* 1536, 768, 384, 192, 96; multiples of 8 */
  int32_t strides[QT_CODEC_MAX_BLOCKS];      /* 8, 5, 4, 3                              */
  int32_t dilations[QT_CODEC_UNITS];         /* 1, 3, 9                                 */
  int32_t chunk;          /* frames per chunk of the chunk grid: 300                   */
  int32_t context;        /* left-context frames per chunk: 25                         */
  int32_t weight_dtype;   /* QT_DTYPE_F32 | QT_DTYPE_BF16                              */
} qt_codec_config;

typedef struct qt_codec_layer_weights {
  const void *ln1_g, *ln1_b, *wqkv /* [3 heads head_dim, hidden] */, *wo /* [hidden, heads head_dim] */, *ls1;
  const void *ln2_g, *ln2_b, *fc1 /* [ffn, hidden] */, *fc2 /* [hidden, ffn] */, *ls2;
} qt_codec_layer_weights;

typedef struct qt_codec_up_weights {
  const void *up /* [2][hidden][hidden] */, *dw /* [7][hidden] */, *ln_g, *ln_b;
  const void *fc1 /* [up_ffn, hidden] */, *fc2 /* [hidden, up_ffn] */, *gamma;
} qt_codec_up_weights;

typedef struct qt_codec_unit_weights {
  const void *a1, *b1, *conv7 /* [7][c][c] */, *a2, *b2, *conv1 /* [1][c][c] */;  /* SnakeBeta logs a, b */
} qt_codec_unit_weights;

typedef struct qt_codec_block_weights {
  const void *snake_a, *snake_b;  /* [channels[b]]                                          */
  const void *up;                 /* [2 strides[b]][channels[b+1]][channels[b]]             */
  qt_codec_unit_weights units[QT_CODEC_UNITS];
} qt_codec_block_weights;

typedef struct qt_codec_weights {
  const void* codebooks;                 /* [n_q][codebook][codebook_dim]               */
  const void *proj_sem, *proj_ac;        /* [hidden, codebook_dim] each                 */
  const qt_codec_layer_weights* layers;  /* host array [layers]                         */
  const void *ln_f_g, *ln_f_b;           /* [hidden]                                    */
  qt_codec_up_weights up[2];
  const void* voc_in;                    /* [7][channels[0]][hidden]                    */
  qt_codec_block_weights blocks[QT_CODEC_MAX_BLOCKS];
  const void *voc_out_a, *voc_out_b;     /* [channels[n_blocks]]                        */
  const void* voc_out;                   /* [7][1][channels[n_blocks]]                  */
} qt_codec_weights;

typedef struct qt_codec qt_codec;

/* Device bytes qt_codec_create needs for decodes of up to chunk + context
 * frames (packed weights, activations, GEMM scratch). Host arithmetic only. */
qt_status qt_codec_workspace_bytes(const qt_codec_config* cfg, size_t* bytes);

/* Create a decoder on the current device; weights are copied / repacked into
 * `workspace` (or a library allocation when NULL). hip_stream as qt_create. */
qt_status qt_codec_create(const qt_codec_config* cfg, const qt_codec_weights* w, void* workspace, size_t ws_bytes,
                          void* hip_stream, qt_codec** out);
void qt_codec_destroy(qt_codec* c);
const char* qt_codec_last_error(const qt_codec* c);

/* One causal pass over frames 0..T-1 (positions from 0):
 *   codes  host int32 [T, n_q], each in 0..codebook-1 (checked first)
 *   audio  device float [T * hop]
 * 1 <= T <= chunk + context. Enqueued on the decoder's stream. */
qt_status qt_codec_decode(qt_codec* c, const int32_t* codes, int32_t T, float* audio);

/* The chunk grid over any number of frames: chunk k covers frames
 * [k chunk, (k+1) chunk) and is decoded from frame max(0, k chunk - context),
 * the context's samples dropped. audio device float [T * hop]. */
qt_status qt_codec_decode_chunked(qt_codec* c, const int32_t* codes, int32_t T, float* audio);

/* Streaming step (the DecodeStream rule): given all T frames so far and the
 * number of samples already emitted (`sent`, a multiple of hop, < T * hop),
 * decode from the chunk grid's regular start of the chunk that holds sample
 * `sent` up to frame T (one decode per chunk touched) and write the new
 * samples sent .. T * hop - 1 to out (device float, at least T * hop - sent).
 * The caller chooses when to call (the pages: after 4 frames, then every
 * 12). The samples equal those of qt_codec_decode_chunked up to rounding. */
qt_status qt_codec_stream(qt_codec* c, const int32_t* codes, int32_t T, int64_t sent, float* out);

/* ---- test and measurement entry points (same kernels as the frame) ---- */

/* Teacher-forced frame: like qt_step_frame, but code 0 of this frame is
 * forced[r][0] and the predictor chain and feedback use forced[r][1..15];
 * rows never finish. Outputs (host, each may be NULL):
 *   talker_logits [B, talker_vocab]  raw logits of the lookahead selection
 *   pred_logits   [B, 15, codebook]  raw logits of predictor heads 0..14
 *   chosen        [B, 16]            the kernels' own choices: [1..15] the
 *                                     predictor's, [0] the lookahead code 0
 * forced ids are range-checked on the host first. */
qt_status qt_debug_step_forced(qt_ctx* ctx, const int32_t* forced, float* talker_logits,
                               float* pred_logits, int32_t* chosen);

/* Raw talker logits of the latest talker selection, host float [B, vocab]
 * (after qt_prefill: selection 0). */
qt_status qt_debug_talker_logits(qt_ctx* ctx, float* logits);

/* Run the selection kernel once on caller data (no context needed).
 *   logits    device float [B, V]
 *   seen      device uint32 [B, ceil(V/32)] or NULL (penalty set)
 *   noise     device float [B, V] explicit Exp(1) noise, or NULL (Philox)
 *   probs     device float [B, V] explicit probabilities (skips temperature,
 *             top-k and softmax; top-p and the race still run), or NULL
 *   processors 1: apply penalty / min-new / suppress (talker), 0: none
 *   sel_index selection index (min-new test and noise counter)
 *   out_code  device int32 [B]; processed device float [B, V] or NULL
 *   status    device int32 [1], OR-ed with 1 on a non-finite logit */
qt_status qt_debug_select(void* hip_stream, int32_t B, int32_t V, const float* logits,
                          const uint32_t* seen, const float* noise, const float* probs,
                          int32_t processors, int32_t eos, int32_t suppress_begin, int32_t suppress_end,
                          const qt_sampling* samp, uint64_t seed, int32_t stream, int32_t sel_index,
                          int32_t* out_code, float* processed, int32_t* status);

/* The Exp(1) noise of the selection kernel's single-sample race, for
 * comparing it bit for bit with an independent implementation (Mizuoto
 * engine page, "Speed": one multinomial draw computed as argmax(p / E) with
 * E ~ Exp(1)). Same device function as the selection kernel.
 *   mode 0: in = device uint64 [n][4] counters (vocab id, stream, selection
 *           index, row), each in 0..2^31-1; the noise is that of Philox4x64-10
 *           with key (seed, 0), first output word x;
 *   mode 1: in = device uint64 [n] words x.
 *   out     device float [n]: E = -ln u, u = ((x >> 12) + 1/2) 2^-52, the
 *           logarithm in double, rounded once to float.
 * Enqueued on hip_stream; QT_E_INVALID for a bad mode, n or NULL pointer. */
qt_status qt_debug_exp_noise(void* hip_stream, int32_t mode, const uint64_t* in, int64_t n, uint64_t seed,
                             float* out);

/* Y = op(W · norm(X)) with the projection kernels of the frame (no context).
 *   W [N, K] device, element type wdtype; X device float [M, K];
 *   gain device float [K] or NULL (RMSNorm prologue with eps);
 *   epilogue 0: Y = W x, 1: Y += W x, 2: SwiGLU over (gate, up) row pairs,
 *   Y [M, N] (or [M, N/2] for SwiGLU) device float.
 *   scratch device float [scratch_floats] or NULL: with bf16 weights it lets
 *   the frame's matrix-core kernels run: at least M floats (row RMS
 *   denominators) enable the tiled MFMA GEMM; beyond the first M rounded up
 *   to 64 floats, space for K-range partial sums (up to (K / 256) * M * (N + 1)
 *   floats) lets the row-block MFMA GEMM for 17..128 rows split K, and
 *   M * K floats there let more than 128 rows take the split-activation GEMM
 *   (the rows normalised once and held as bf16 hi + lo planes).
 *   reps >= 1 launches (for timing); launch i uses the weight copy
 *   W + (i % w_copies) * w_copy_stride bytes (w_copies >= 1; copies of at
 *   least N * K elements each, so timed launches can stream from HBM rather
 *   than from a cache that holds one copy). */
qt_status qt_debug_linear(void* hip_stream, int32_t wdtype, const void* W, int32_t N, int32_t K,
                          const float* X, int32_t M, const float* gain, float eps, int32_t epilogue,
                          float* Y, float* scratch, int64_t scratch_floats, int32_t reps,
                          int32_t w_copies, int64_t w_copy_stride);

/* Y = op(W · norm(X)) exactly as qt_debug_linear computes it with full
 * matrix-core scratch, but allocating nothing: for callers that cannot call
 * hipMalloc (code under graph capture, tight serving loops, harnesses that
 * forbid allocation). The scratch (row RMS denominators, K-range partial
 * sums, hi/lo split planes) is a static device array of 8 Mi floats (32 MiB)
 * per GPU, held until the process ends; its address is looked up once per
 * device on the first call there. Arguments as qt_debug_linear (one launch,
 * one weight copy). A projection whose scratch need, (M rounded up to 64) +
 * (K / 256) * M * (N + 1) floats for M <= 128 or + M * K floats above, exceeds
 * the static array returns QT_E_CAPACITY before any device work. Every call
 * on one GPU shares that array: calls that overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller. Enqueued on
 * hip_stream; nothing is synchronised. */
qt_status qt_linear_noalloc(void* hip_stream, int32_t wdtype, const void* W, int32_t N, int32_t K, const float* X,
                            int32_t M, const float* gain, float eps, int32_t epilogue, float* Y);

/* The prompt prefill's attention of one decoder layer with the frame's
 * kernels (no context): per-head RMSNorm of q and k with their gains, rope of
 * both, the K/V rows written to the cache, then causal GQA attention of every
 * prompt token over the positions up to its own, scaled by 1/sqrt(head_dim)
 * (ncnn port discussion 6798, section 1 "structure": Qwen3 decoders with
 * GQA 16/8, head_dim 128 and QK-Norm; ncnn port section 5: the prompt
 * prefill).
 *   kv_dtype QT_DTYPE_F32, QT_DTYPE_BF16 or QT_DTYPE_F16; head_dim 16, 32, 64,
 *   128 or 256; nq a multiple of nkv with nq / nkv in {1, 2, 4, 8}.
 *   B rows; lens host int32 [B], 1 .. max_pos tokens each; the tokens sit in
 *   activation rows row after row, T = sum of lens.
 *   qkv device float [T, (nq + 2 nkv) head_dim]: q heads, then k, then v.
 *   q_gain, k_gain device float [head_dim]; eps > 0.
 *   cos, sin device float [max_pos, head_dim / 2] (angle of pair (i, i + d/2)).
 *   kc, vc device [B, nkv, max_pos, head_dim] of kv_dtype: rows 0 .. lens[r] - 1
 *   of row r are written, others untouched.
 *   out device float [T, nq head_dim].
 *   tiled 1: the attend pass takes runs of up to 32 tokens of one row on the
 *   matrix cores (head_dim 128, nq = 2 nkv, 16-bit cache; other shapes
 *   return QT_E_INVALID); 0: one run per token.
 *   runs device int32 [runs_ints] scratch for the run tables, at least
 *   4 (T + T / 32 + B) ints.
 * Returns after the stream has finished. QT_E_INVALID on a bad argument,
 * QT_E_HIP on a launch failure. */
qt_status qt_debug_prefill_attention(void* hip_stream, int32_t kv_dtype, int32_t head_dim, int32_t nq, int32_t nkv,
                                     int32_t B, const int32_t* lens, int32_t max_pos, const float* qkv,
                                     const float* q_gain, const float* k_gain, float eps, const float* cos,
                                     const float* sin, void* kc, void* vc, float* out, int32_t tiled,
                                     int32_t* runs, int64_t runs_ints);

/* One decode step of one decoder layer's attention with the frame's kernels
 * (no context), for ntok new tokens per row: token t of row r (row
 * r ntok + t of qkv) goes through per-head RMSNorm (q, k) and rope at
 * position pos[r] + t, its K and V are written to cache position pos[r] + t,
 * and its q heads attend over positions 0 .. pos[r] + t (GQA, scale
 * 1/sqrt(head_dim); ntok 2 is the code predictor's two-token pass) (ncnn port discussion
 * 6798, section 1 "structure": Qwen3 decoders with GQA 16/8, head_dim 128 and
 * QK-Norm; Mizuoto "Qwen3-TTS" page, "速度": decoding over a KV cache).
 *   kv_dtype, head_dim, nq, nkv as qt_debug_prefill_attention; B 1 .. 4096;
 *   ntok 1, or 2 with kv_split 1 and head_dim <= 128.
 *   pos host int32 [B], 0 .. max_pos - ntok each; pos_dev device int32 [B]
 *   scratch (receives a copy).
 *   qkv device float [B ntok, (nq + 2 nkv) head_dim]: q heads, then k, then v.
 *   q_gain, k_gain device float [head_dim]; eps > 0.
 *   cos, sin device float [max_pos, head_dim / 2].
 *   kc, vc device [B, nkv, max_pos, head_dim] of kv_dtype: positions
 *   0 .. pos[r] - 1 of row r hold the cached keys and values as stored;
 *   positions pos[r] .. pos[r] + ntok - 1 are written, others untouched.
 *   out device float [B ntok, nq head_dim].
 *   kv_split 1: one block per (row, kv head); 2, 4, 8 or 16 (head_dim 128,
 *   nq / nkv <= 4): that many key ranges per row, combined in range order,
 *   with split_buf device float [B, nkv, kv_split, nq / nkv, head_dim + 2]
 *   scratch (NULL allowed with kv_split 1).
 * Returns after the stream has finished. QT_E_INVALID on a bad argument,
 * QT_E_HIP on a launch failure. */
qt_status qt_debug_decode_attention(void* hip_stream, int32_t kv_dtype, int32_t head_dim, int32_t nq, int32_t nkv,
                                    int32_t B, int32_t ntok, const int32_t* pos, int32_t* pos_dev, int32_t max_pos,
                                    const float* qkv, const float* q_gain, const float* k_gain, float eps,
                                    const float* cos, const float* sin, void* kc, void* vc, float* out,
                                    int32_t kv_split, float* split_buf);

#ifdef __cplusplus
}
#endif

#endif /* QT_H */
