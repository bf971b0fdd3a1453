/*
 * moshi_mi355x.h -- C ABI of the MI355X (gfx950) Moshi RQ-Transformer frame step.
 *
 * One call of moshi_frame_step runs one 80 ms frame of Moshi's RQ-Transformer LM on the GPU:
 * the delay-aligned token ring, the summed 17-stream embedding, the temporal decoder at one
 * position against its KV cache, the text head with greedy argmax, and the 8 sequential
 * depformer codebook steps, each ending in a greedy argmax.  The operation is the one the
 * docs.rs page "inferencelayer 0.2.4 src/moshi_lm.rs" defines (module doc, MoshiLm::step_ext and
 * the items it calls); that page is cited below as [LM].
 *
 * Conventions shared by every entry point:
 *   - Pointers named host_* or documented as host memory are plain CPU memory owned by the
 *     caller; the library copies what it needs before returning and keeps no reference.
 *   - All device memory (weights, KV caches, ring, activations) is owned by the moshi_state and
 *     released by moshi_destroy.  Nothing here takes torch or HIP types other than an optional
 *     hipStream_t passed as void*.
 *   - Calls on one moshi_state are not reentrant: use one state per thread.
 *   - Every call returns a moshi_status; on failure moshi_last_error(state) holds a message.
 *     A device (HIP) error returns MOSHI_EDEVICE and leaves the session contents undefined
 *     until moshi_reset.
 */
#ifndef MOSHI_MI355X_H
#define MOSHI_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOSHI_OK = 0,
  MOSHI_NONE = 1,      /* the step ran, but no conversation has output yet ([LM] step: none
                          until offset > max_delay) */
  MOSHI_EINVAL = -1,   /* bad argument (state unchanged) */
  MOSHI_ESTATE = -2,   /* call out of order, e.g. a step before all weights are loaded */
  MOSHI_ESHAPE = -3,   /* unknown tensor name, wrong shape or dtype at load */
  MOSHI_ENOMEM = -4,   /* device or pinned host allocation failed */
  MOSHI_EDEVICE = -5,  /* HIP error; session contents undefined until moshi_reset */
  MOSHI_ERANGE = -6    /* the step would write past kv_capacity (state unchanged) */
} moshi_status;

/* Weight band: the storage type of every linear weight on the device. */
typedef enum {
  MOSHI_BAND_F32 = 0,  /* float32 linears and embeddings ([LM] Band::F32, the parity band) */
  MOSHI_BAND_BF16 = 1, /* bfloat16 linears and embeddings, float32 arithmetic */
  MOSHI_BAND_I8 = 2,   /* int8 linears with one float32 scale per output row ([LM] Band::I8);
                          embeddings bfloat16.  Quantised at load, see moshi_load_weights. */
  MOSHI_BAND_Q4 = 3,   /* Q4_0 linears ([LM] q4_roundtrip, load_q4sim): per row and 32-column block
                          one float32 scale and 16 bytes of 4-bit codes; embeddings bfloat16.
                          Quantised at load.  Batch 1 only (graph, stream, persistent executors). */
  MOSHI_BAND_Q8 = 4    /* q8_0 linears ([LM] qn_roundtrip at 8 bits, group 32): per row and 32-column
                          block one float32 scale and 32 int8 codes; embeddings bfloat16.
                          Quantised at load.  Batch 1 only. */
} moshi_band;

/* Storage type of the temporal KV cache. */
typedef enum {
  MOSHI_KV_F32 = 0,  /* float32 (the default, every band): no storage loss, so long contexts keep
                        the greedy tokens of the float32 definition */
  MOSHI_KV_BF16 = 1  /* bfloat16 (bf16 and int8 bands only): half the KV bytes, at a storage loss
                        that grows with the context length */
} moshi_kv;

typedef enum { MOSHI_DTYPE_F32 = 0, MOSHI_DTYPE_BF16 = 1 } moshi_dtype;

/* How a frame is issued to the GPU. */
typedef enum {
  MOSHI_EXEC_GRAPH = 0,      /* the whole frame is captured once into a hipGraph and replayed */
  MOSHI_EXEC_STREAM = 1,     /* kernels are launched one by one on the stream each frame */
  MOSHI_EXEC_PERSISTENT = 2  /* one cooperative kernel per frame, one block per CU, phases chained
                                by device-side completion counters (batch 1; shapes with a compiled
                                variant, else moshi_create returns MOSHI_EINVAL).  Teacher-forced
                                prefill still runs as stream launches. */
} moshi_exec;

/*
 * Model shape and session layout (plain C struct).  The Moshi-7B shape ([LM] constants) is
 * n_layers 32, d_model 4096, n_heads 32, ffn_hidden 11264, context 3000, text_card 32000,
 * audio_card 2048, dep_layers 6, dep_d_model 1024, dep_heads 16, dep_ffn_hidden 2816, dep_q 8,
 * rope_theta 10000, rms_eps 1e-8.
 *   text_card / audio_card : head widths; the INITIAL tokens are text_card and audio_card and
 *                            the embedding tables have card + 1 rows ([LM] module doc).
 *   batch                  : independent conversations stepped together (each with its own
 *                            ring, offset and KV cache).
 *   kv_capacity            : positions of temporal KV held per conversation; 0 means context.
 *                            Must be <= context.  When equal to context the cache is a ring and
 *                            the offset may grow without bound (sliding window of the last
 *                            `context` positions, absolute rope positions); when smaller, a step
 *                            at offset >= kv_capacity returns MOSHI_ERANGE.
 *   exec                   : a moshi_exec value.
 *   kv_dtype               : a moshi_kv value (0 = float32).
 * Constraints (else MOSHI_EINVAL): d_model % n_heads == 0 with head_dim 64 or 128; the Q4 and Q8
 * bands need batch 1 and d_model, ffn_hidden, dep_d_model and dep_ffn_hidden multiples of 32;
 * dep_d_model % dep_heads == 0; 1 <= dep_q <= 16 (Moshi uses 8); d_model, ffn_hidden,
 * dep_d_model and dep_ffn_hidden multiples of 16 and at most 16384; batch >= 1; kv_dtype
 * MOSHI_KV_BF16 only with the bf16 and int8 bands.
 */
typedef struct moshi_config {
  int32_t n_layers, d_model, n_heads, ffn_hidden, context;
  int32_t text_card, audio_card;
  int32_t dep_layers, dep_d_model, dep_heads, dep_ffn_hidden, dep_q;
  float rope_theta, rms_eps;
  int32_t band, batch, kv_capacity, exec;
  int32_t kv_dtype;
} moshi_config;

/*
 * One tensor handed to moshi_load_weights.  `name` and `shape` follow the checkpoint layout
 * that [LM] MoshiLm::load_band reads:
 *   emb.{0..15}.weight [audio_card+1, d_model]           text_emb.weight [text_card+1, d_model]
 *   transformer.layers.{l}.norm1.alpha / norm2.alpha [d_model]
 *   transformer.layers.{l}.self_attn.in_projs.0.weight [3 d_model, d_model]   (rows q | k | v)
 *   transformer.layers.{l}.self_attn.out_projs.0.weight [d_model, d_model]
 *   transformer.layers.{l}.gating.linear_in.weight [2 ffn_hidden, d_model]    (rows gate | mult)
 *   transformer.layers.{l}.gating.linear_out.weight [d_model, ffn_hidden]
 *   out_norm.alpha [d_model]                              text_linear.weight [text_card, d_model]
 *   depformer_in.{s}.weight [dep_d_model, d_model]        linears.{s}.weight [audio_card, dep_d_model]
 *   depformer_text_emb.weight [text_card+1, dep_d_model]  depformer_emb.{0..6}.weight [audio_card+1, dep_d_model]
 *   depformer.layers.{j}.norm1.alpha / norm2.alpha [dep_d_model]   (shared by the 8 steps)
 *   depformer.layers.{j}.self_attn.in_projs.{s}.weight [3 dep_d_model, dep_d_model]
 *   depformer.layers.{j}.self_attn.out_projs.{s}.weight [dep_d_model, dep_d_model]
 *   depformer.layers.{j}.gating.{s}.linear_in.weight [2 dep_ffn_hidden, dep_d_model]
 *   depformer.layers.{j}.gating.{s}.linear_out.weight [dep_d_model, dep_ffn_hidden]
 * Matrices are row-major [rows, cols] (output row r is contiguous).  `data` is host memory
 * holding float32 or bfloat16 (raw uint16 bits) as `dtype` says; ndim is 1 or 2.
 */
typedef struct moshi_tensor {
  const char *name;
  int32_t dtype; /* moshi_dtype */
  int32_t ndim;
  int64_t shape[2];
  const void *data;
} moshi_tensor;

/*
 * Where moshi_read_trace copies the last step's stages ([LM] StepTrace).  Every pointer is
 * caller-owned host memory or NULL (skipped).
 */
typedef struct moshi_trace {
  int32_t *input_tokens;    /* [2 dep_q + 1] gathered model input tokens */
  float *emb_sum;           /* [d_model] summed embedding */
  float *transformer_out;   /* [d_model] post-out_norm hidden */
  float *text_logits;       /* [text_card] */
  float *audio_logits;      /* [dep_q][audio_card] */
  int32_t *tokens;          /* [1 + dep_q] text token, then the dep_q audio tokens */
} moshi_trace;

typedef struct moshi_state moshi_state;

/*
 * Create a session on the current HIP device.  `hip_stream` is a hipStream_t to run on, or NULL
 * for a stream the library creates.  Allocates all device memory up front (weights, KV caches
 * of batch x n_layers x kv_capacity positions, ring, activations).  The session starts reset
 * ([LM] state(): ring all -2, offset 0, no KV).  Errors: MOSHI_EINVAL (bad config),
 * MOSHI_ENOMEM, MOSHI_EDEVICE (no usable GPU).  On error *out is NULL.
 */
moshi_status moshi_create(const moshi_config *cfg, void *hip_stream, moshi_state **out);

/*
 * Copy `n` tensors to the device (may be called several times; a later tensor of the same name
 * replaces the earlier one).  Storage follows the band: MOSHI_BAND_F32 widens bfloat16 input to
 * float32; MOSHI_BAND_BF16 rounds float32 input to bfloat16 (nearest-even); MOSHI_BAND_I8
 * quantises every linear per output row r: s_r = max_k |w_rk| / 127 (float32), q_rk =
 * round-half-away-from-zero(w_rk / s_r) clamped to [-127, 127], q = 0 when s_r = 0, and the
 * product is s_r * sum_k q_rk x_k.  MOSHI_BAND_Q4 and MOSHI_BAND_Q8 quantise every linear per row
 * and 32-column block with [LM] qn_roundtrip's rule: d = (the block's value of largest magnitude,
 * the first on ties) / -2^(b-1) with b = 4 or 8, q = clamp(round-half-away(w * (1 / d)),
 * -2^(b-1), 2^(b-1) - 1), q = 0 where d = 0; the weight is q * d (float32 operations, IEEE
 * round to nearest).  Norm gains are always float32.  Errors: MOSHI_ESHAPE (unknown name, wrong
 * shape, bad dtype), MOSHI_EDEVICE.
 */
moshi_status moshi_load_weights(moshi_state *s, const moshi_tensor *tensors, int32_t n);

/*
 * One frame for every conversation ([LM] step_ext, greedy).  user_tokens [batch][dep_q] host
 * int32: each in [0, audio_card) or -1 (embeds to exact zero).  Any other value gives
 * MOSHI_EINVAL before device work, leaving the state unchanged.  On success out [batch][1+dep_q]
 * (host) receives the delay-realigned [text, audio x dep_q] of each conversation that has one
 * (offset > 1 after the step), and has_out [batch] (host; may be NULL when batch == 1) says
 * which.  Returns MOSHI_OK if any conversation produced output, MOSHI_NONE if none did.
 * Errors: MOSHI_ESTATE (weights incomplete), MOSHI_ERANGE, MOSHI_EDEVICE.
 */
moshi_status moshi_frame_step(moshi_state *s, const int32_t *user_tokens, int32_t *out,
                              uint8_t *has_out);

/* Reset conversation `conv` (or all when conv == -1) to [LM] state(): ring -2, offset 0, empty
 * KV.  Weights are kept.  Errors: MOSHI_EINVAL (conv out of range), MOSHI_EDEVICE. */
moshi_status moshi_reset(moshi_state *s, int32_t conv);

/* Free every device and host allocation of the session.  NULL is ignored. */
void moshi_destroy(moshi_state *s);

/* Message of the last failed call on `s` (empty string if none; static text when s is NULL). */
const char *moshi_last_error(const moshi_state *s);

/* Name of a moshi_status value. */
const char *moshi_status_string(int32_t status);

/* ---- session hooks (tests, teacher forcing, measurement) ------------------------------------ */

/* Absolute offset of conversation `conv`, i.e. the temporal position of its next step ([LM]
 * MoshiState::clock). */
moshi_status moshi_get_offset(const moshi_state *s, int32_t conv, int64_t *offset);

/* [LM] MoshiState::force_generated: overwrite the tokens written by the last step of `conv`
 * (ring slot offset % 3) with text and audio[dep_q] (host).  Used to judge a non-parity band
 * step by step on a reference trajectory.  text in [0, text_card), audio in [0, audio_card). */
moshi_status moshi_force_generated(moshi_state *s, int32_t conv, int32_t text, const int32_t *audio);

/* Copy the last step's stages of `conv` to host memory (see moshi_trace). */
moshi_status moshi_read_trace(moshi_state *s, int32_t conv, const moshi_trace *trace);

/* [LM] step_forced, T times: teacher-forced steps of conversation `conv` that advance the
 * temporal KV cache on the gathered inputs, skip the heads and the depformer, and record the
 * forced text [T] and agent [T][dep_q] tokens in the ring; user [T][dep_q] as in
 * moshi_frame_step.  All arrays are host int32. */
moshi_status moshi_prefill_forced(moshi_state *s, int32_t conv, int32_t T, const int32_t *text,
                                  const int32_t *agent, const int32_t *user);

/* ---- sampled decoding ([LM] Sampling, MoshiLm::pick) ------------------------------------------ */

typedef enum {
  MOSHI_PICK_GREEDY = 0,  /* first-wins argmax ([LM] argmax), the default */
  MOSHI_PICK_TOPK = 1,    /* [LM] topk_sample: the k largest logits, exp(double((l - max) / T)) weights
                             summed in order of decreasing logit (equal logits by increasing index),
                             normalised, one uniform, inverse-CDF walk */
  MOSHI_PICK_GUMBEL = 2   /* [LM] gumbel_full_pick: argmax over the whole head of float32(l / T) +
                             float32(-ln(-ln(max(u, 1e-300)))), one uniform per logit in index order */
} moshi_pick;

/* How a conversation picks its tokens.  The text head uses temp_text / top_k_text, the codebook
 * heads temp / top_k ([LM] Sampling; LMGen defaults 0.8, 0.7, 250, 25).  Uniforms come from one
 * 64-bit xorshift stream per conversation ([LM] xorshift_u01: shifts 13, 7, 17; u = top 53 bits /
 * 2^53), drawn in pick order (text, then codebooks 0..dep_q-1), started at max(seed, 1). */
typedef struct moshi_sampling {
  int32_t mode;        /* moshi_pick */
  float temp;          /* codebook temperature, > 0 */
  float temp_text;     /* text temperature, > 0 */
  int32_t top_k;       /* codebook k, in [1, 1024] (top-k mode) */
  int32_t top_k_text;  /* text k, in [1, 1024] (top-k mode) */
  uint64_t seed;       /* xorshift state; 0 means 1 */
} moshi_sampling;

/* Set conversation `conv`'s (or with conv == -1 every conversation's) token pick and restart its
 * xorshift stream at max(seed, 1).  Later frames use it; moshi_reset and snapshots leave it alone
 * (on the page the sampler belongs to the model, not to the session state).  The persistent
 * executor samples with MOSHI_PICK_GUMBEL (folded into its heads' argmax) or greedy; top-k needs the
 * graph or stream executor and heads of at most 36864 logits.  Errors: MOSHI_EINVAL (bad mode,
 * temperature or k, or top-k on the persistent executor), MOSHI_EDEVICE. */
moshi_status moshi_set_sampling(moshi_state *s, int32_t conv, const moshi_sampling *smp);

/* The current xorshift state of conversation `conv`'s sampler (after the frames run so far). */
moshi_status moshi_sampler_state(moshi_state *s, int32_t conv, uint64_t *state);

/* ---- session snapshot ([LM] MoshiState::snapshot) --------------------------------------------- */

/* A copy of one conversation's session state: the ring, the offset and the cached temporal KV
 * positions (the last min(offset, context) positions, kept on the device in position order).  The
 * depformer keeps no state across frames, and a sampler's random state (moshi_set_sampling) is
 * not part of it, as on the page.  Opaque; owned by the caller until moshi_snapshot_free. */
typedef struct moshi_snapshot moshi_snapshot;

/* Copy conversation `conv` of `s` into a new snapshot (*out).  Allocates device memory of
 * 2 x n_layers x positions x d_model KV elements on the session's device.  The session is not
 * changed.  Errors: MOSHI_EINVAL, MOSHI_ESTATE (after a device error, before moshi_reset),
 * MOSHI_ENOMEM, MOSHI_EDEVICE; *out is NULL on error. */
moshi_status moshi_snapshot_take(moshi_state *s, int32_t conv, moshi_snapshot **out);

/* Make conversation `conv` of `s` continue from the snapshot: its ring, offset and cached KV
 * positions become the snapshot's (the cache slots are position % kv_capacity, so the destination
 * may hold its conversations at another kv_capacity or batch).  The snapshot is unchanged and can
 * be restored again, into any conversation of any session of the same model shape, band and KV
 * storage on the same device.  Like moshi_reset it also clears a device-error state.  Errors:
 * MOSHI_EINVAL (another shape, band, KV storage or device), MOSHI_ERANGE (kv_capacity below context
 * and below the snapshot's offset), MOSHI_EDEVICE. */
moshi_status moshi_snapshot_restore(moshi_state *s, int32_t conv, const moshi_snapshot *snap);

/* The snapshot's offset, cached positions and device bytes (each optional). */
moshi_status moshi_snapshot_info(const moshi_snapshot *snap, int64_t *offset, int64_t *positions, int64_t *bytes);

/* Free a snapshot and its device memory.  NULL is ignored. */
void moshi_snapshot_free(moshi_snapshot *snap);

/* GPU time of frames: with enable >= 0 the per-frame HIP event pair around the frame's device
 * work (graph replay or persistent kernel, recorded on the session stream) is switched on (1)
 * or off (0) and the totals are cleared; with enable < 0 nothing changes.  *total_us and *frames
 * (optional) receive the totals since the last clear. */
moshi_status moshi_gpu_time(moshi_state *s, int32_t enable, double *total_us, int64_t *frames);

/* Measurement (persistent executor): with enable = 1 the following frames record, per phase, the
 * device wall-clock time at which block 0 finished its share and at which the phase completed;
 * ts [max_phases][2] (host, optional) receives the last frame's record in microseconds from the
 * frame's first arrival, *n_phases the phase count.  enable = 0 switches it off. */
moshi_status moshi_phase_times(moshi_state *s, int32_t enable, double *ts, int32_t max_phases, int32_t *n_phases);

/* Measurement (persistent executor): after moshi_phase_times(s, 2, ...) the frames also record
 * every block's arrival at every phase; ts [n_phases][n_blocks] (host, up to max_values values)
 * receives the last frame's record in microseconds from its first arrival, *n_blocks the grid
 * size.  MOSHI_ESTATE if the record was never switched on. */
moshi_status moshi_block_times(moshi_state *s, double *ts, int32_t max_values, int32_t *n_blocks);

/* Test hook (persistent executor): every wait of the frame kernel (a phase flag or a polled
 * exchange value) gives up after `spins` polls (default 2^20, about a second); the kernel then
 * raises its error flag, every block leaves, and moshi_frame_step returns MOSHI_EDEVICE (the
 * session needs moshi_reset before the next frame).  It lets a test force that exit path from the
 * host.  MOSHI_EINVAL for spins < 0, MOSHI_ESTATE for a session of another executor. */
moshi_status moshi_set_spin_limit(moshi_state *s, int32_t spins);

/* Bytes of linear weights (what one frame must stream) and of all device weights. */
moshi_status moshi_weight_bytes(const moshi_state *s, int64_t *linear_bytes, int64_t *all_bytes);

/* The HIP stream the session runs on (a hipStream_t). */
void *moshi_stream(const moshi_state *s);

/* Stages of one frame, in launch order (each is one kernel per launch). */
typedef enum {
  MOSHI_STAGE_EMBED = 0,     /* user write, gather, 17-row embedding sum */
  MOSHI_STAGE_QKV,           /* temporal norm1 + q|k|v + rope + KV append   (x n_layers) */
  MOSHI_STAGE_ATTN,          /* temporal decode attention                   (x n_layers) */
  MOSHI_STAGE_OUT_PROJ,      /* temporal out_proj + residual                (x n_layers) */
  MOSHI_STAGE_GATE_IN,       /* temporal norm2 + linear_in + silu * mult    (x n_layers) */
  MOSHI_STAGE_GATE_OUT,      /* temporal linear_out + residual              (x n_layers) */
  MOSHI_STAGE_TEXT_HEAD,     /* out_norm + text head + greedy argmax */
  MOSHI_STAGE_DEP_IN,        /* depformer_in for all codebooks */
  MOSHI_STAGE_DEP_QKV,       /* depformer (entry) norm1 + q|k|v   (x dep_q x dep_layers) */
  MOSHI_STAGE_DEP_OUT,       /* depformer attention + out_proj    (x dep_q x dep_layers) */
  MOSHI_STAGE_DEP_GATE_IN,   /* depformer norm2 + linear_in       (x dep_q x dep_layers) */
  MOSHI_STAGE_DEP_GATE_OUT,  /* depformer linear_out + residual   (x dep_q x dep_layers) */
  MOSHI_STAGE_DEP_HEAD,      /* codebook head + greedy argmax     (x dep_q) */
  MOSHI_STAGE_FRAME_END,     /* offset, ring write, realigned output */
  MOSHI_N_STAGES
} moshi_stage;

/*
 * Measurement: run `n_frames` real frames (state advances as with moshi_frame_step) with the
 * kernels launched one by one and every launch bracketed by a HIP event pair on the session
 * stream.  user_tokens [n_frames][batch][dep_q] host.  stage_us[MOSHI_N_STAGES] receives the
 * summed event time per stage (microseconds) and stage_launches[MOSHI_N_STAGES] the launch
 * counts.  Errors as moshi_frame_step.
 */
moshi_status moshi_profile_frames(moshi_state *s, int32_t n_frames, const int32_t *user_tokens,
                                  double *stage_us, int64_t *stage_launches);

/* ---- kernel-level hooks (tests and micro-benchmarks) ---------------------------------------- */

/*
 * y[N] = W[N][K] . x[K] with the library's weight-streaming GEMV, on fresh device copies of the
 * host arrays.  band picks the weight storage (W is given as float32 host data and converted as
 * moshi_load_weights would).  If iters > 0 the kernel is also launched `iters` more times between
 * HIP events and *avg_us receives the mean duration.  Errors: MOSHI_EINVAL, MOSHI_ENOMEM,
 * MOSHI_EDEVICE.
 */
moshi_status moshi_debug_gemv(int32_t band, int32_t N, int32_t K, const float *W, const float *x,
                              float *y, int32_t iters, float *avg_us);

/*
 * Y[M][N] = X[M][K] . W[N][K]^T with the library's matrix-core projection (the batched-frame and
 * prefill path), on fresh device copies of the host arrays.  W is given as float32 and stored per
 * band as moshi_load_weights would (f32, bf16, or int8 with per-row scales); X is float32 and is
 * rounded to bf16 for the bf16 and int8 bands, as the batched path rounds its activations.  Y is
 * float32 [M][N], written on success.  iters / avg_us as for moshi_debug_gemv.  Requires M >= 1,
 * N >= 1, K >= 16 and K % 16 == 0.  Errors: MOSHI_EINVAL, MOSHI_ENOMEM, MOSHI_EDEVICE.
 */
moshi_status moshi_debug_gemm(int32_t band, int32_t M, int32_t N, int32_t K, const float *W, const float *X,
                              float *Y, int32_t iters, float *avg_us);

/*
 * Measurement: the device's streaming-read rate, the ceiling the frame's weight streaming is
 * compared with.  A kernel reads `bytes` of a fresh device allocation with 16-byte nontemporal
 * loads (8 per lane in flight, each block a contiguous share), once untimed and then `iters`
 * times between HIP events, for each of a few launch shapes (1 to 8 blocks of 256 to 1024
 * threads per compute unit); *gbs receives the best bytes x iters / elapsed time in GB/s (10^9
 * bytes per second).  Errors: MOSHI_EINVAL (bytes outside
 * [2^20, 2^31 - 16], iters < 1, gbs NULL), MOSHI_ENOMEM, MOSHI_EDEVICE.
 */
moshi_status moshi_debug_read_bw(int64_t bytes, int32_t iters, double *gbs);

/*
 * Y[M][N] = X[M][K] . W[N][K]^T (times the int8 row scales) with the matrix-core projection of
 * moshi_debug_gemm, for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): it allocates nothing and only enqueues
 * kernels on `hip_stream` (a hipStream_t, NULL for the null stream); the caller synchronises.
 * All pointers are device memory owned by the caller: W row-major in the band's storage (float32,
 * bfloat16 bits, or int8 with `scale` [N] float32 per-row scales; scale is ignored otherwise),
 * X float32 [M][K], Y float32 [M][N] (written).  The bf16 and int8 bands round X to bf16 hi / lo
 * parts as the batched frame does.  Its scratch (those activation planes and the split-K partial
 * tiles) is a 32 MiB device array inside the library, one per device, held until the process
 * ends and shared by every call on that device: calls that overlap on one device race, and each
 * call overwrites what the previous one left there.  Limits: 1 <= M <= 256, K a multiple of 16 in
 * [16, 16384], 4 M K <= 16 MiB for the bf16 and int8 bands.  Errors: MOSHI_EINVAL (bad argument),
 * MOSHI_ERANGE (beyond the scratch), MOSHI_EDEVICE (HIP error at launch).
 */
moshi_status moshi_gemm_noalloc(int32_t band, int32_t M, int32_t N, int32_t K, const void *W, const float *scale,
                                const float *X, float *Y, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* MOSHI_MI355X_H */
