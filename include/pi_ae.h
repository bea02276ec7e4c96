/*
 * pi_ae.h -- C ABI of libpi_ae.so, the MI355X (gfx950) action-expert
 * flow-matching denoise loop of pi0.5-style vision-language-action policies.
 *
 * What the library computes (Realtime-VLA technical blog, blog.w4k4.me,
 * section "pi0.5 inference flow"): the VLM runs once and leaves a per-layer
 * key/value cache of the prefix (images + prompt); the action expert then runs
 * the flow-matching denoise loop against that cache.  Every denoise step
 * projects the noisy action chunk (action_in_proj, 32 -> 1024), runs the
 * 18-layer expert (AdaRMS-modulated attention over prefix + suffix keys and a
 * GELU-gated MLP, both with gated residuals), projects back (action_out_proj,
 * 1024 -> 32) to a velocity v_t and takes the Euler step x <- x + dt * v_t.
 *
 * The split into a one-time preparation call and a cheap per-call sample
 * follows the blog's sections "precompute (__init__)" and "CUDA Graph"
 * (all tables and buffers are built at initialisation; the per-call forward is
 * "copy inputs, replay the graph").
 *
 * Conventions for every entry point:
 *   - No C++ exception crosses this ABI.  Every call returns a pi_ae_status;
 *     on failure pi_ae_last_error() gives a message for the calling thread.
 *   - All arguments are validated before any GPU work is enqueued: a call
 *     that returns an error has enqueued nothing.
 *   - bf16 values are passed as their 16-bit patterns (uint16_t).
 *   - Streams are HIP streams (hipStream_t) passed as void*; NULL is the
 *     default stream of the current device.
 */
#ifndef PI_AE_H
#define PI_AE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pi_ae_status {
  PI_AE_OK = 0,
  PI_AE_EINVAL = 1,        /* a NULL pointer, a size out of range, a misaligned pointer */
  PI_AE_EUNSUPPORTED = 2,  /* a shape the kernels do not implement (see pi_ae_config) */
  PI_AE_ENOMEM = 3,        /* device or host allocation failed */
  PI_AE_EHIP = 4,          /* a HIP runtime call failed */
  PI_AE_ESTATE = 5         /* the context cannot take this call (e.g. destroyed or failed) */
} pi_ae_status;

/*
 * Model and call limits.  Shapes are those of the blog's section "LeRobot
 * implementation" (Gemma-300M-shaped expert): the kernels implement exactly
 *   width 1024, mlp_dim 4096, num_heads 8, num_kv_heads 1, head_dim 256,
 *   action_dim 32, 1 <= chunk_len <= 256,
 * and return PI_AE_EUNSUPPORTED for anything else.  num_layers >= 1,
 * num_steps >= 1 (at most 64).  t0 and dt give the timestep schedule
 * t_k = fp32(t0 + k * dt), k = 0 .. num_steps-1 (dt = -1/num_steps in the
 * pages; it is a separate field so that a shortened schedule can keep dt).
 * max_batch and max_prefix_len size the workspaces: a sample call may use any
 * batch <= max_batch and prefix_len <= max_prefix_len.  rope_base is the RoPE
 * base (10000), rms_eps the RMS-norm epsilon (1e-6).  final_norm = 1 adds an
 * AdaRMS norm with its own modulation dense before action_out_proj.
 * variant selects the expert:
 *   0 = pi0.5 (Realtime-VLA blog, "pi0.5 inference flow"): AdaRMS norms
 *       conditioned on the time MLP, gated residuals;
 *   1 = pi0 ("Running VLAs at Real-time Speed" notes, section How; blog
 *       section 3.2): RMS norms with a learnable scale gamma, plain residuals,
 *       and as step input the action-time encoder
 *       h = W_to SiLU(W_ti [action_in_proj(x) | emb(t)] + b_ti) + b_to;
 *       final_norm = 1 adds an RMS norm with scale gamma before action_out_proj.
 */
typedef struct pi_ae_config {
  int32_t num_layers;
  int32_t width;
  int32_t mlp_dim;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t action_dim;
  int32_t chunk_len;
  int32_t num_steps;
  float t0;
  float dt;
  int32_t max_batch;
  int32_t max_prefix_len;
  float rope_base;
  float rms_eps;
  int32_t final_norm;
  int32_t variant;
} pi_ae_config;

/* One nn.Linear: weight [out][in] row-major, bias [out] (NULL where the layer
 * has no bias).  Host pointers to bf16 bit patterns. */
typedef struct pi_ae_linear {
  const uint16_t* w;
  const uint16_t* b;
} pi_ae_linear;

/* One expert layer.  attn_mod / ffn_mod: the AdaRMS modulation denses
 * (width -> 3*width, with bias; output split in thirds: scale, shift, gate).
 * q [heads*head_dim][width], k and v [head_dim][width], o [width][heads*head_dim],
 * gate and up [mlp_dim][width], down [width][mlp_dim]; these have no bias. */
typedef struct pi_ae_layer_weights {
  pi_ae_linear attn_mod, q, k, v, o, ffn_mod, gate, up, down;
  /* variant 1 only: the two RMS norms' scales gamma [width] (bf16); attn_mod
   * and ffn_mod are then not read. */
  const uint16_t* attn_norm;
  const uint16_t* ffn_norm;
} pi_ae_layer_weights;

/* The unfolded expert.  action_in [width][action_dim] + b; time_in and
 * time_out [width][width] + b (the time MLP: cond = SiLU(time_out(SiLU(
 * time_in(emb(t)))))); final_mod [3*width][width] + b (read only when
 * final_norm = 1); action_out [action_dim][width] + b; layers[num_layers].
 * Variant 1 reads action_in, action_out and the layers' q..down as above and,
 * instead of time_in / time_out / final_mod / the modulation denses:
 * action_time_in [width][2*width] + b (input: [action_in_proj(x) | emb(t)]),
 * action_time_out [width][width] + b, final_norm (gamma [width], read when
 * final_norm = 1) and the layers' attn_norm / ffn_norm. */
typedef struct pi_ae_weights {
  pi_ae_linear action_in, time_in, time_out, final_mod, action_out;
  const pi_ae_layer_weights* layers;
  pi_ae_linear action_time_in, action_time_out;
  const uint16_t* final_norm;
} pi_ae_weights;

/* The VLM prefix cache for one call (device memory, read only).
 *   k, v:     bf16 [num_layers][batch][prefix_len][head_dim], contiguous,
 *             16-byte aligned; keys already rotated by the producer's RoPE.
 *   pad_mask: u8 [batch][prefix_len], nonzero = valid key; NULL = all valid.
 *   prefix_len: P, 0 <= P <= max_prefix_len. */
typedef struct pi_ae_prefix_kv {
  const void* k;
  const void* v;
  const uint8_t* pad_mask;
  int32_t prefix_len;
} pi_ae_prefix_kv;

typedef struct pi_ae_ctx pi_ae_ctx;

/*
 * One-time weight preparation (blog sections 3.2 "simplifying the
 * computational graph" and "precompute (__init__)"):
 *   - the time embedding and time MLP for the num_steps timesteps, and every
 *     layer's AdaRMS scale/shift/gate (and the final norm's) are tabulated;
 *   - each AdaRMS shift is folded into a bias of the following linear
 *     (c = shift @ W^T), the scale stays a per-channel factor;
 *   - Q, K and V are fused into one [(heads+2)*head_dim][width] matrix whose
 *     RoPE is applied in the GEMM epilogue; gate and up are fused likewise;
 *   - dt is applied to action_out_proj's output in the fp32 epilogue;
 *   - the RoPE inverse frequencies base^(-2i/head_dim) in fp64 (each call
 *     turns them into the cos/sin rows of its own suffix positions).
 * Host arithmetic is fp64; tables are stored fp32, weights stay bf16.
 * Synchronous on the current HIP device; reads the host arrays only during the
 * call.  The library owns everything it allocates; *out is written only on
 * success.  Errors: EINVAL (NULL cfg/w/out/weight pointer, bad sizes),
 * EUNSUPPORTED (shapes other than the ones above), ENOMEM, EHIP.
 */
pi_ae_status pi_ae_prepare_weights(const pi_ae_config* cfg, const pi_ae_weights* w, pi_ae_ctx** out);

/*
 * Run the denoise loop for `batch` episodes (the blog's "sample_actions"):
 * x <- noise; for k in 0..num_steps-1: x <- x + dt * v(x, t_k); actions <- x.
 *   kv:      the prefix cache (see pi_ae_prefix_kv).
 *   noise:   device fp32 [batch][chunk_len][action_dim], 16-byte aligned.
 *   actions: device fp32 [batch][chunk_len][action_dim], 16-byte aligned;
 *            may equal noise (in place).
 *   batch:   0 <= batch <= max_batch (0 does nothing).
 *   stream:  hipStream_t (void*); the call is asynchronous and stream-ordered.
 * Suffix token j of episode b sits at RoPE position n_valid[b] + j, where
 * n_valid[b] is the number of valid prefix keys of that episode.
 * All inputs must stay alive and unmodified until the stream has passed the
 * call.  One call in flight per context: concurrent calls on one context (on
 * any streams) race on its workspaces; use one context per concurrent stream.
 * The step sequence is captured as a hipGraph per (batch, prefix_len) on first
 * use and replayed afterwards; a context keeps at most 8 such graphs (the
 * least recently used is dropped, after its last launch has finished), so
 * callers with many prefix lengths should pad them to a few fixed ones.
 * Errors: EINVAL (NULL ctx/kv/noise/actions,
 * batch or prefix_len out of range, misaligned pointers), ESTATE (ctx
 * unusable), EHIP (a launch failed).  Device faults surface at the caller's
 * next synchronisation.
 */
pi_ae_status pi_ae_sample(pi_ae_ctx* ctx, const pi_ae_prefix_kv* kv, const float* noise, float* actions,
                          int32_t batch, void* stream);

/* Allocation-free variant of pi_ae_sample, for callers that cannot allocate
 * device memory: code under stream capture (its launches are plain kernel
 * launches on `stream`, no graph of the library's own), tight serving loops,
 * harnesses that forbid it.  Same arguments, validation, results and stream
 * semantics as pi_ae_sample (the same kernels in the same order), but the
 * call's working memory (residual stream, GEMM operands, packed K/V, key
 * bias, RoPE rows) is a fixed device array of the library (24 MiB, one copy
 * per GPU, held until the process ends) instead of the context's workspace,
 * and no graph is captured or instantiated.  Limits: batch * chunk_len <= 64
 * and 2 * num_layers * batch * ceil((prefix_len + chunk_len) / 32) * 16 KiB
 * of packed K/V plus about 2.1 MiB of activations within the 24 MiB (an
 * 18-layer expert: prefix_len + chunk_len <= 1088 at batch 1); larger calls
 * return PI_AE_EINVAL before anything is enqueued.  It calls no hipMalloc or
 * hipFree.  Every call on one GPU uses that GPU's array and leaves its last
 * contents there (every part a call reads is written earlier in the same
 * call): calls that overlap on one GPU, on any streams or contexts, race and
 * must be serialised by the caller. */
pi_ae_status pi_ae_sample_noalloc(pi_ae_ctx* ctx, const pi_ae_prefix_kv* kv, const float* noise, float* actions,
                                  int32_t batch, void* stream);

/* Wait for the work this context has enqueued (the graphs it launched, on
 * whatever streams), then free everything it owns.  Other work on the device
 * is not waited for.  NULL is a no-op. */
void pi_ae_destroy(pi_ae_ctx* ctx);

/* Static string for a status code: any integer (a pi_ae_status value, or
 * anything else, which gives "unknown status"). */
const char* pi_ae_status_string(int32_t status);

/* Message of the last failed call on this thread ("" if none). */
const char* pi_ae_last_error(void);

/* ------------------------------------------------------------------------
 * The VLM prefix prefill: the step before the denoise loop, which fills the
 * prefix cache that pi_ae_sample reads (Realtime-VLA technical blog, section
 * "pi0.5 inference flow", Encoder (prefix) phase, run once per inference: the
 * image tokens and the prompt tokens, each scaled by sqrt(2048), form the
 * prefix sequence, which passes through the 18 layers of the Gemma-2B VLM;
 * every layer's key and value are kept as the cache).  Layer l is
 *   u = rms_norm(h) * gamma_attn;  q, k, v = u W_q^T, u W_k^T, u W_v^T;
 *   RoPE on q and k at position j (token j of its episode);
 *   cache[l] = (k, v);  h += attention(q, k, v) W_o^T  (every token attends to
 *   every valid token of its episode: bidirectional, pad-masked keys excluded);
 *   u = rms_norm(h) * gamma_ffn;  h += (GELU_tanh(u W_g^T) * (u W_u^T)) W_d^T
 * (section 4 kernel list, Encoder layers).  The last layer stops after its
 * keys and values, which are all the expert reads of it (section 4.1: 17
 * layers run in full).  bf16 weights and activations, fp32 accumulation and
 * residual stream.
 * ------------------------------------------------------------------------ */

/* VLM shape and call limits.  The kernels implement exactly width 2048,
 * mlp_dim 16384, num_heads 8, num_kv_heads 1, head_dim 256 (the section 4
 * kernel list's 2048 -> 2560 fused QKV and 2048 -> 16384 gated MLP, with the
 * expert's 256-wide KV head) and return PI_AE_EUNSUPPORTED otherwise;
 * 1 <= num_layers <= 64.  max_batch >= 1 and 1 <= max_prefix_len <= 4096 size
 * the workspaces and the cache; rope_base is the RoPE base (10000), rms_eps
 * the RMS-norm epsilon (1e-6). */
typedef struct pi_ae_vlm_config {
  int32_t num_layers;
  int32_t width;
  int32_t mlp_dim;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_batch;
  int32_t max_prefix_len;
  float rope_base;
  float rms_eps;
} pi_ae_vlm_config;

/* One VLM layer, host pointers to bf16 bit patterns, nn.Linear layout
 * [out][in], no biases: attn_norm and ffn_norm the norms' scales gamma
 * [width]; q [heads*head_dim][width], k and v [head_dim][width],
 * o [width][heads*head_dim], gate and up [mlp_dim][width], down
 * [width][mlp_dim].  The last layer's o, ffn_norm, gate, up and down are not
 * read (they may be NULL). */
typedef struct pi_ae_vlm_layer_weights {
  const uint16_t* attn_norm;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* ffn_norm;
  const uint16_t* gate;
  const uint16_t* up;
  const uint16_t* down;
} pi_ae_vlm_layer_weights;

typedef struct pi_ae_vlm pi_ae_vlm;

/* One-time preparation of the VLM (blog section 3.2: Q, K and V fused into
 * one 2560-row matrix with RoPE in the GEMM epilogue, gate and up fused; the
 * norms' scales kept as per-channel factors of the normalised operand).
 * layers: num_layers entries.  Synchronous on the current HIP device; reads
 * the host arrays only during the call; the library owns what it allocates,
 * the prefix cache included.  *out is written only on success.  Errors:
 * EINVAL (NULL pointers, sizes out of range), EUNSUPPORTED, ENOMEM, EHIP. */
pi_ae_status pi_ae_vlm_prepare(const pi_ae_vlm_config* cfg, const pi_ae_vlm_layer_weights* layers,
                               pi_ae_vlm** out);

/* Run the prefill for `batch` episodes of `prefix_len` tokens.
 *   prefix_emb: device bf16 [batch][prefix_len][width], 16-byte aligned: the
 *               prefix sequence after the sqrt(2048) scaling.
 *   pad_mask:   device u8 [batch][prefix_len], nonzero = valid token; NULL =
 *               all valid.  Pad tokens are computed like the others but no
 *               token attends to them; an episode without a valid token gets
 *               a zero attention output.
 *   batch:      1 <= batch <= max_batch; 1 <= prefix_len <= max_prefix_len.
 *   kv_out:     host struct, filled on success: k and v point to the
 *               context's cache, bf16 [num_layers][batch][prefix_len][256]
 *               (k rotated), pad_mask = the argument, prefix_len: exactly
 *               the pi_ae_prefix_kv that pi_ae_sample takes.  The cache stays
 *               valid until the next prefill on this context or its
 *               destruction.
 *   stream:     hipStream_t (void*); asynchronous and stream-ordered; inputs
 *               must stay alive until the stream has passed the call.
 * One call in flight per context.  The layer sequence is captured as a
 * hipGraph per (batch, prefix_len) on first use.  Errors: EINVAL (NULL
 * ctx / prefix_emb / kv_out, sizes out of range, misaligned prefix_emb),
 * ESTATE, EHIP. */
pi_ae_status pi_ae_vlm_prefill(pi_ae_vlm* ctx, const uint16_t* prefix_emb, const uint8_t* pad_mask, int32_t batch,
                               int32_t prefix_len, pi_ae_prefix_kv* kv_out, void* stream);

/* Wait for the work this context has enqueued, then free everything it owns
 * (the cache included).  A pipeline or inference object that joins this
 * context must be destroyed first.  NULL is a no-op. */
void pi_ae_vlm_destroy(pi_ae_vlm* ctx);

/* The VLM prefill and the denoise loop as one pipeline (RV-blog sections
 * "CUDA Graph" and "static buffers": the whole inference is one captured
 * graph over static buffers).  A pipeline pairs a prepared VLM with a
 * prepared expert of the same depth (the expert's layer l reads the VLM
 * layer l's keys and values); both must outlive it.  Errors: EINVAL (NULL
 * pointers, different layer counts). */
typedef struct pi_ae_pipeline pi_ae_pipeline;
pi_ae_status pi_ae_pipeline_create(pi_ae_vlm* vlm, pi_ae_ctx* expert, pi_ae_pipeline** out);

/* One inference: the prefill of prefix_emb (as pi_ae_vlm_prefill) and then
 * the denoise loop of noise into actions (as pi_ae_sample) on the cache it
 * leaves.  Per call, a staging kernel for each model; the layer sequences of
 * both are captured once per (batch, prefix_len) as a single hipGraph.  Same
 * argument rules as the two calls (batch and prefix_len within both
 * contexts' limits); asynchronous and stream-ordered; one call in flight per
 * pipeline and its two contexts.  The cache stays in the VLM context as
 * after pi_ae_vlm_prefill. */
pi_ae_status pi_ae_pipeline_run(pi_ae_pipeline* pipe, const uint16_t* prefix_emb, const uint8_t* pad_mask,
                                const float* noise, float* actions, int32_t batch, int32_t prefix_len, void* stream);

/* Wait for the pipeline's own launched graphs, then free them (not the two
 * contexts, which must outlive it).  NULL is a no-op. */
void pi_ae_pipeline_destroy(pi_ae_pipeline* pipe);

/* Test-only: time one kernel of the prefill in its real sequence, as
 * pi_ae_debug_time_phase does for the loop: the whole prefill is run `reps`
 * times on `stream`, kernel by kernel, with a HIP event pair bound to each
 * launch of `phase` (1 = QKV + RoPE, 2 = attention, 3 = O + residual,
 * 4 = gate/up, 5 = down + residual); *avg_us = mean duration.  Same argument
 * rules as pi_ae_vlm_prefill, plus 1 <= reps <= 1000.  Synchronises `stream`. */
pi_ae_status pi_ae_vlm_debug_time_phase(pi_ae_vlm* ctx, const uint16_t* prefix_emb, const uint8_t* pad_mask,
                                        int32_t batch, int32_t prefix_len, int32_t phase, int32_t reps,
                                        void* stream, float* avg_us);

/* ------------------------------------------------------------------------
 * The vision encoder: each camera view becomes the 256 image tokens of the
 * VLM prefix (Realtime-VLA technical blog, "pi0.5 inference flow": SigLIP
 * turns a 224x224 view into 256 tokens, scaled by sqrt(2048); "LeRobot
 * implementation": a 27-layer vision tower and the multi-modal projector,
 * Linear 1152 -> 2048).  Per view: the 14x14 patches (row by row, each in
 * (channel, y, x) order) embedded by a strided convolution with bias, plus a
 * learned position embedding; 27 pre-norm layers h += attn(LN1(h)) (16
 * heads x 72, bidirectional over the 256 patches, biases on q, k, v, o),
 * h += fc2(GELU_tanh(fc1(LN2(h)))) (MLP 4304, biases); a final LayerNorm and
 * the projector, whose output is multiplied by sqrt(2048).  LayerNorms have a
 * scale and a bias, eps as configured.  bf16 weights and activations, fp32
 * accumulation and residual stream.
 * ------------------------------------------------------------------------ */

/* The kernels implement exactly width 1152, mlp_dim 4304, 16 heads x 72,
 * patch 14, image 224, out_width 2048 (EUNSUPPORTED otherwise);
 * 1 <= num_layers <= 64; 1 <= max_views <= 64 sizes the workspaces. */
typedef struct pi_ae_vision_config {
  int32_t num_layers;
  int32_t width;
  int32_t mlp_dim;
  int32_t num_heads;
  int32_t head_dim;
  int32_t patch;
  int32_t image;
  int32_t out_width;
  int32_t max_views;
  float ln_eps;
} pi_ae_vision_config;

/* One vision layer, host bf16 bit patterns, nn.Linear layout [out][in]:
 * LayerNorm scales / biases [width]; q, k, v, o [width][width] with biases
 * [width]; fc1 [mlp_dim][width] + [mlp_dim]; fc2 [width][mlp_dim] + [width]. */
typedef struct pi_ae_vision_layer_weights {
  const uint16_t *ln1_w, *ln1_b, *q_w, *q_b, *k_w, *k_b, *v_w, *v_b, *o_w, *o_b;
  const uint16_t *ln2_w, *ln2_b, *fc1_w, *fc1_b, *fc2_w, *fc2_b;
} pi_ae_vision_layer_weights;

/* patch_w [width][3][patch][patch] (convolution layout) + patch_b [width];
 * pos [256][width]; layers[num_layers]; post_ln_w / post_ln_b [width];
 * proj_w [out_width][width] + proj_b [out_width]. */
typedef struct pi_ae_vision_weights {
  const uint16_t *patch_w, *patch_b, *pos;
  const pi_ae_vision_layer_weights* layers;
  const uint16_t *post_ln_w, *post_ln_b, *proj_w, *proj_b;
} pi_ae_vision_weights;

typedef struct pi_ae_vision pi_ae_vision;

/* One-time preparation (fused q|k|v, operands padded with zero columns to
 * whole k-blocks, weights swizzled into MFMA fragments).  Synchronous on the
 * current device; reads the host arrays only during the call.  Errors:
 * EINVAL, EUNSUPPORTED, ENOMEM, EHIP. */
pi_ae_status pi_ae_vision_prepare(const pi_ae_vision_config* cfg, const pi_ae_vision_weights* w,
                                  pi_ae_vision** out);

/* Encode `views` images into their tokens.
 *   images: device bf16 [views][224][224][3] (rows, columns, RGB), resized
 *           and normalised, 16-byte aligned.
 *   tokens: device bf16 [views * 256][2048], 16-byte aligned: view v's token
 *           t at row 256 v + t, scaled by sqrt(2048) -- the image part of the
 *           prefix sequence that pi_ae_vlm_prefill takes (an episode's prompt
 *           tokens follow its views).
 *   1 <= views <= max_views.  Asynchronous and stream-ordered; the layer
 *   sequence is captured as a hipGraph per view count on first use; one call
 *   in flight per context.  Errors: EINVAL, ESTATE, EHIP. */
pi_ae_status pi_ae_vision_encode(pi_ae_vision* ctx, const uint16_t* images, int32_t views, uint16_t* tokens,
                                 void* stream);

/* Wait for the work this context has enqueued, then free everything it owns.
 * An inference object that joins it must be destroyed first.  NULL is a no-op. */
void pi_ae_vision_destroy(pi_ae_vision* ctx);

/* The whole inference as one graph (RV-blog sections "CUDA Graph" and
 * "static buffers"): the vision encoder, the VLM prefill and the denoise loop
 * of one episode.  The three contexts must outlive the object; the VLM and
 * the expert must have the same depth.  The prefix sequence (the views' tokens
 * then the prompt's) and the pad mask live in static buffers of the object,
 * sized by the VLM's max_prefix_len.  Errors: EINVAL, ENOMEM, EHIP. */
typedef struct pi_ae_inference pi_ae_inference;
pi_ae_status pi_ae_inference_create(pi_ae_vision* vision, pi_ae_vlm* vlm, pi_ae_ctx* expert, pi_ae_inference** out);

/* Images to actions for one episode:
 *   images:     device bf16 [views][224][224][3], 16-byte aligned;
 *   prompt_emb: device bf16 [prompt_len][2048] (the prompt's embedded tokens,
 *               after their sqrt(2048) scaling), or NULL with prompt_len 0;
 *   pad_mask:   device u8 [views * 256 + prompt_len], or NULL (all valid);
 *   noise, actions: device fp32 [chunk_len][action_dim] (may alias).
 * Per call: the prompt and the mask are copied into the static buffers, the
 * images staged and the loop's arguments published; then one hipGraph per
 * (views, prompt_len) runs every layer of the three models.  Asynchronous and
 * stream-ordered; one call in flight per object and its contexts. */
pi_ae_status pi_ae_inference_run(pi_ae_inference* inf, const uint16_t* images, int32_t views,
                                 const uint16_t* prompt_emb, int32_t prompt_len, const uint8_t* pad_mask,
                                 const float* noise, float* actions, void* stream);

/* Wait for the object's own launched graphs, then free them and its static
 * buffers (not the contexts, which must outlive it).  NULL is a no-op. */
void pi_ae_inference_destroy(pi_ae_inference* inf);

/* Test-only: time one kernel of the encoder in its real sequence (as
 * pi_ae_vlm_debug_time_phase): phase 0 = patch embedding, 1 = layer 0's
 * first LayerNorm (every later LayerNorm is part of phase 4 or 6), 2 = QKV,
 * 3 = attention, 4 = O + residual + the layer's second LayerNorm, 5 = fc1 +
 * GELU, 6 = fc2 + residual + the next layer's first (or the final)
 * LayerNorm, 7 = projector; phases 4 and 6 are two kernels each, timed from
 * the start of the first to the end of the second; `reps` whole encodes on
 * `stream`; *avg_us = mean duration of one instance of that phase. */
pi_ae_status pi_ae_vision_debug_time_phase(pi_ae_vision* ctx, const uint16_t* images, int32_t views,
                                           uint16_t* tokens, int32_t phase, int32_t reps, void* stream,
                                           float* avg_us);

/* ------------------------------------------------------------------------
 * Test-only exports (unstable; used by the parity tests).
 * ------------------------------------------------------------------------ */

/* Copy one prepared fp32 table to host memory.  which: 0 = attn (1+scale)
 * [S][L][width], 1 = attn gate [S][L][width], 2 = ffn (1+scale), 3 = ffn gate,
 * 4 = final (1+scale) [S][width], 5 = c_out [S][action_dim] (shift @ W_out^T +
 * b_out), 6 = c_qkv [S][L][(heads+2)*head_dim] (natural q|k|v column order),
 * 7 = c_gu [S][L][2*mlp_dim] (natural gate|up order), 8 = timesteps [S],
 * 9 = cond [S][width] (variant 1: the action-time encoder's per-step bias
 * before its SiLU, W_ti[:, :width] b_in + W_ti[:, width:] emb(t_k) + b_ti; its
 * norm scales fill tables 0/2/4 as (1 + scale) = gamma, gates 1, shifts 0).  n_floats must equal the table's size.  Synchronous. */
pi_ae_status pi_ae_debug_table(pi_ae_ctx* ctx, int32_t which, float* host_out, size_t n_floats);

/* The same tables computed by the host half of pi_ae_prepare_weights alone
 * (fp64 arithmetic, no GPU work, no allocation on the device): lets the
 * preparation be checked on a machine without a GPU.  Same `which` codes. */
pi_ae_status pi_ae_debug_host_table(const pi_ae_config* cfg, const pi_ae_weights* w, int32_t which,
                                    float* host_out, size_t n_floats);

/* Run the loop only up to a point and copy an intermediate to host memory.
 * Runs steps 0..step-1 fully, then in step `step` the layers before `layer`
 * and, in layer `layer`, the phases up to and including `phase`
 * (0 = step input: action_in, or for variant 1 the whole action-time encoder,
 * 1 = QKV+RoPE, 2 = attention, 3 = O + gated
 * residual, 4 = gate/up, 5 = down + gated residual).  which: 0 = h fp32
 * [M][width], 1 = Q bf16 [M][heads][head_dim], 2 = K_s bf16 [M][head_dim],
 * 3 = V_s bf16 [M][head_dim], 4 = O bf16 [M][heads*head_dim], 5 = m bf16
 * [M][mlp_dim], 6 = x fp32 [M][action_dim], 7 = second partial O bf16
 * [M][heads*head_dim], 8 = attention row statistics fp32 [M][heads][4];
 * M = batch*chunk_len, rows in natural order.  At M < 129 with at least 16
 * key blocks of 32 (nkb = ceil((prefix_len + chunk_len) / 32) >= 16) the
 * attention splits each query's keys into two ranges (blocks [0, nkb/2) and
 * [nkb/2, nkb)): 4 and 7 are then the two ranges' normalised outputs and 8
 * holds (max_0, sum_0, max_1, sum_1) per query, max in units of log2 after
 * the 1/sqrt(head_dim) scaling; the attention output is
 * (a_0 sum_0 O_0 + a_1 sum_1 O_1) / (a_0 sum_0 + a_1 sum_1), a_s =
 * 2^(max_s - max(max_0, max_1)) (a_s = 0 where max_s = -inf).  Otherwise 4
 * is the attention output and 7 / 8 are unused.  Synchronous; uses the null
 * stream. */
pi_ae_status pi_ae_debug_probe(pi_ae_ctx* ctx, const pi_ae_prefix_kv* kv, const float* noise, int32_t batch,
                               int32_t step, int32_t layer, int32_t phase, int32_t which, void* host_out,
                               size_t n_bytes);

/* Time one phase's kernel inside the real loop: run the whole loop `chunks`
 * times on `stream`, launched kernel by kernel (the same kernels, order and
 * arguments as the captured graph), with a pair of HIP events bound to each
 * launch of the kernel of `phase` (numbering as in pi_ae_debug_probe): the
 * events are taken at that kernel's own start and end, so each pair's
 * elapsed time is one launch's duration in the loop's context.  *avg_us =
 * mean over all timed launches.  The result of the last pass lands in
 * `actions`.  Synchronises `stream`.  Same argument rules as pi_ae_sample,
 * plus batch >= 1 and 1 <= chunks <= 1000. */
pi_ae_status pi_ae_debug_time_phase(pi_ae_ctx* ctx, const pi_ae_prefix_kv* kv, const float* noise, float* actions,
                                    int32_t batch, int32_t phase, int32_t chunks, void* stream, float* avg_us);

/* Check the guard bytes around every device allocation of a prepared object
 * (kind 0: pi_ae_ctx, 1: pi_ae_vlm, 2: pi_ae_vision): each allocation is
 * flanked by 256 bytes of a fixed pattern, and a kernel that wrote past either
 * end of a buffer leaves a changed guard.  Synchronises the device first.
 * corrupt >= 0 first overwrites one guard byte of allocation `corrupt` from
 * the host (a test of the check itself; the object stays usable).  Returns
 * PI_AE_OK with *first_bad = -1, or PI_AE_ESTATE with *first_bad = the first
 * allocation whose guard changed.  (Test-only.  A prepared object's device
 * allocations also honour PI_AE_FAIL_ALLOC=N in the environment, read when it
 * is prepared: its N-th allocation then fails as out of memory.) */
pi_ae_status pi_ae_debug_check_guards(const void* object, int32_t kind, int32_t corrupt, int32_t* first_bad);

/* Device bytes held by every prepared object of the process (expert, VLM and
 * vision contexts; guards included): what a failed preparation must leave
 * unchanged.  (Test-only.) */
int64_t pi_ae_debug_live_device_bytes(void);

/* ---------------------------------------------------------------------------
 * Measurement diagnostics (test-only; no context needed).  They measure the
 * floors under the loop's design on the current device (Realtime-VLA
 * technical blog, section 5: the roofline lower bound is the weights streamed
 * once per step; sections "CUDA Graph" and 4: the loop is a replayed graph of
 * about 900 decoder kernels).  Each allocates and frees its own device
 * buffers, runs on `stream` (NULL: the null stream) and synchronises it.
 * ------------------------------------------------------------------------- */

/* Plain streaming read of a `bytes` buffer (1 MiB .. 16 GiB), `reps` timed
 * passes (1 .. 1000) after one warm-up; *gbps = the best pass's rate in GB/s
 * (1e9 bytes per second). */
pi_ae_status pi_ae_debug_stream_read(size_t bytes, int32_t reps, void* stream, float* gbps);

/* A graph of `kernels` (1 .. 4096) dependent empty kernels of `grid`
 * (1 .. 65536) workgroups of 256 threads, replayed 10 times after 2 warm-up
 * replays; *us_per_kernel = elapsed time / (10 * kernels): what each kernel
 * boundary of a replayed graph costs with no work in it. */
pi_ae_status pi_ae_debug_graph_floor(int32_t kernels, int32_t grid, void* stream, float* us_per_kernel);

/* `rounds` (1 .. 100000) grid-wide barriers inside one kernel of one
 * workgroup per CU.  mode 0: per-workgroup flags, each on its own 128-byte
 * line, stored with agent scope and polled by every workgroup; mode 1:
 * counters per XCD residue (workgroup index mod 8) whose last arriver bumps
 * one global counter.  *us_per_round = elapsed time / rounds.  Every wait is
 * bounded: PI_AE_ESTATE if one passed its spin limit (the kernel still ends),
 * PI_AE_EUNSUPPORTED if one workgroup per CU cannot be resident. */
pi_ae_status pi_ae_debug_grid_sync(int32_t rounds, int32_t mode, void* stream, float* us_per_round);

#ifdef __cplusplus
}
#endif
#endif /* PI_AE_H */
