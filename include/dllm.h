/*
 * dllm.h - C ABI of the block-diffusion denoising library (libdllm.so).
 *
 * The library runs the hot path of a masked block-diffusion MoE language
 * model (LLaDA2.0-Uni backbone, arXiv 2604.20796) on one AMD Instinct
 * MI355X (gfx950): block-wise attention with 1D RoPE over a KV-cached prefix,
 * sigmoid-plus-bias top-k MoE with a shared expert, the LM head with optional
 * classifier-free guidance, confidence-based unmasking, and SPRINT-style
 * prefix-KV retention.
 *
 * Problem statement followed (the model card's understand_image /
 * generate_image calls): given a token prefix, generate tokens in blocks of
 * `block_length`; each block starts as [MASK] (or with some fixed ids) and
 * gets up to `steps` denoising steps; every step commits a quota of masked
 * positions, the most confident first.  Finished blocks are appended to the
 * cache clean (paper review, "BDLM": earlier blocks are always clean context).
 *
 * Conventions for every call:
 *  - All device memory (weights, KV cache, workspace, token ids) belongs to
 *    the caller.  The library stores raw pointers, never allocates, frees or
 *    copies device memory it was not given, and never reads the pointers
 *    after dllm_destroy.
 *  - Argument checks are synchronous on the host and happen before any
 *    launch; failures return a negative status and dllm_last_error() holds
 *    the reason.  Kernels are enqueued asynchronously on the context's
 *    stream; a launch failure returns DLLM_ERR_HIP.
 *  - A context is not thread-safe.  Separate contexts may run concurrently on
 *    separate streams.
 *  - Token ids are int32: text ids [0, vocab_text), visual ids
 *    [vocab_text, vocab_text + vocab_image) (model card: visual id = VQ code
 *    + image_token_offset), and [MASK] = vocab_text + vocab_image.  Ids
 *    outside [0, mask] are read as [MASK] by the embedding gather.
 */
#ifndef DLLM_H
#define DLLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dllm_ctx dllm_ctx;

/* status codes */
#define DLLM_OK                 0
#define DLLM_ERR_INVALID_ARG   -1  /* bad shape, pointer or parameter */
#define DLLM_ERR_OUT_OF_MEMORY -2  /* workspace or KV capacity too small */
#define DLLM_ERR_HIP           -3  /* HIP runtime or launch error */
#define DLLM_ERR_BAD_STATE     -4  /* call out of order (e.g. no open block) */
#define DLLM_ERR_UNSUPPORTED   -5  /* valid but not implemented combination */

/* storage / arithmetic types */
#define DLLM_F32      0
#define DLLM_BF16     1
#define DLLM_FP8_E4M3 2   /* OCP E4M3FN codes with float32 per-output-row scales */

/* confidence strategies (model card, SPRINT: low_confidence, top_k_margin,
 * neg_entropy) */
#define DLLM_CONF_LOW_CONFIDENCE 0  /* max softmax probability */
#define DLLM_CONF_TOP_K_MARGIN   1  /* p1 - p2 */
#define DLLM_CONF_NEG_ENTROPY    2  /* sum p log p */

/* prefix retention scores (paper review, SPRINT "sparse prefix retention";
 * model card, SPRINT "KV cache reuse and pruning") */
#define DLLM_RETAIN_MASS          0  /* attention mass of the block's queries on
                                        each prefix key, summed over layers
                                        and heads, at the warm-up step */
#define DLLM_RETAIN_KEYNORM_CONF  1  /* alpha * l~_i + (1 - alpha) * c_i: l~ the
                                        key norm averaged over layers and heads
                                        divided by its prefix mean, c the top-1
                                        probability at prefix position i */

/* Model shape (paper review, "MoE backbone and block-wise attention":
 * 16B-parameter MoE backbone; shapes are caller-chosen). */
typedef struct dllm_model_config {
  int32_t n_layers;
  int32_t hidden;        /* D: a multiple of 256, at most 8192 */
  int32_t n_heads;       /* H (key/value heads = query heads) */
  int32_t head_dim;      /* dh: 32, 64 or 128 */
  int32_t n_experts;     /* E routed experts */
  int32_t top_k;         /* experts per token */
  int32_t n_shared;      /* 0 or 1 shared expert (gate weight 1) */
  int32_t expert_ffn;    /* F, SwiGLU width of a routed expert */
  int32_t shared_ffn;    /* Fs, SwiGLU width of the shared expert */
  int32_t vocab_text;
  int32_t vocab_image;
  float rope_base;       /* 1D RoPE, rotate-half pairs (i, i + dh/2) */
  float rms_eps;
  int32_t act_dtype;     /* DLLM_F32 or DLLM_BF16: dense weights, embeddings,
                            KV cache and GEMM inputs */
  int32_t expert_dtype;  /* DLLM_F32 (requires act F32), DLLM_BF16 or
                            DLLM_FP8_E4M3 (both require act BF16; fp8 also
                            needs hidden % 512 == 0, expert_ffn % 64 == 0) */
} dllm_model_config;

/* Generation knobs (model card: block_length, steps, cfg_scale, threshold,
 * keep_ratio, cache_warmup_steps; paper review, SPRINT). */
typedef struct dllm_gen_params {
  int32_t block_length;     /* L_B, 1..64 */
  int32_t steps;            /* T denoising steps per block */
  int32_t n_seq;            /* sequences denoised together */
  float cfg_scale;          /* <= 0: off.  > 0: model rows are (cond, uncond)
                               pairs, logits l_u + w (l_c - l_u) */
  int32_t vocab_lo;         /* sub-vocabulary [vocab_lo, vocab_hi) for the  */
  int32_t vocab_hi;         /* LM head; vocab_hi = 0 means the full vocabulary */
  int32_t confidence;       /* DLLM_CONF_* */
  int32_t use_threshold;    /* also accept every masked position with c > threshold */
  float threshold;
  int32_t use_sprint;       /* prefix-KV retention: the last warm-up step
                               scores the prefix and picks the kept positions
                               that later steps of the block attend to */
  float keep_ratio;         /* retained prefix = ceil(keep_ratio * P) positions */
  int32_t cache_warmup_steps; /* steps t < this attend to the whole prefix */
  int32_t max_prefix;       /* KV capacity per model row, tokens */
  int32_t max_clean_tokens; /* largest n_clean accepted by dllm_block_init */
  int32_t retention_score;  /* DLLM_RETAIN_* (KEYNORM_CONF makes dllm_block_init
                               also run the LM head over appended positions) */
  float retention_alpha;    /* weight of the key-norm term, 0..1 */
  float image_keep_ratio;   /* > 0 (either ratio): modality pools.  Visual prefix */
  float text_keep_ratio;    /* ids keep ceil(image r * P_img), all other ids
                               ceil(text r * P_text); an unset (<= 0) pool
                               ratio takes keep_ratio.  Ratios <= 1. */
  float cfg_text_scale;     /* > 0: three-way editing guidance (model card
                               edit_image).  Model rows come in triples (full
                               prompt, image-only prompt, unconditional) and the
                               logits are l_u + s_img (l_img - l_u)
                               + s_txt (l_full - l_img).  Needs cfg_scale <= 0;
                               prefix retention is then off (SPRINT falls back
                               to the baseline, as the model card notes). */
  float cfg_image_scale;    /* s_img, >= 0 (three-way guidance only) */
} dllm_gen_params;

/* Weights: device pointers, row-major, output dimension first and the
 * reduction dimension contiguous.  L = n_layers, V = vocab_text + vocab_image,
 * HD = n_heads * head_dim.  "act" = act_dtype, "exp" = expert_dtype. */
typedef struct dllm_weights {
  const void* embed;        /* act [V + 1][D]   (row V is [MASK]) */
  const float* attn_norm;   /* f32 [L][D]       RMSNorm gains before attention */
  const void* w_qkv;        /* act [L][3*HD][D] rows: q heads, k heads, v heads */
  const void* w_o;          /* act [L][D][HD] */
  const float* moe_norm;    /* f32 [L][D] */
  const void* w_router;     /* act [L][E][D] */
  const float* router_bias; /* f32 [L][E]       selection-only bias */
  const void* w_gate;       /* exp [L][E][F][D] */
  const void* w_up;         /* exp [L][E][F][D] */
  const void* w_down;       /* exp [L][E][D][F] */
  const float* s_gate;      /* f32 [L][E][F]    fp8 experts only, else NULL */
  const float* s_up;        /* f32 [L][E][F] */
  const float* s_down;      /* f32 [L][E][D] */
  const void* ws_gate;      /* act [L][Fs][D]   n_shared = 1 only */
  const void* ws_up;        /* act [L][Fs][D] */
  const void* ws_down;      /* act [L][D][Fs] */
  const float* final_norm;  /* f32 [D] */
  const void* lm_head;      /* act [V][D] */
  int32_t gate_up_packed;   /* 0: w_gate / w_up row-major as above.  1: both in
                               the packed fragment layout written by
                               dllm_pack_gate_up (same size; streams faster) */
} dllm_weights;

/* KV cache: act [L][rows][H][max_prefix][dh] for K and for V, post-RoPE.
 * rows = n_seq, 2 * n_seq with CFG (row 2s cond, 2s+1 uncond), or 3 * n_seq
 * with three-way guidance (3s full, 3s+1 image-only, 3s+2 uncond). */
typedef struct dllm_kv_cache {
  void* k;
  void* v;
} dllm_kv_cache;

/* Bytes of device workspace dllm_create needs for this shape.  0 on invalid
 * arguments. */
size_t dllm_workspace_bytes(const dllm_model_config* cfg, const dllm_gen_params* gp);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): dllm_create
 * with the workspace taken from a static device array of the library (64 MiB,
 * one per GPU, held until the process ends) instead of caller memory.  The
 * call allocates nothing (no hipMalloc / hipFree); it looks the array up on
 * the current device once, and enqueues a fill kernel on `stream` that clears
 * the bytes this shape uses.  Shapes whose dllm_workspace_bytes exceed 64 MiB
 * return DLLM_ERR_OUT_OF_MEMORY (checked on the host before any HIP call;
 * e.g. the small test models fit, a 4096-token append pass at hidden 2048
 * does not).  Every context created this way on one GPU shares that array:
 * use one at a time per device.  Calls of two such contexts that overlap
 * race, and a second context's calls overwrite the first's per-block state
 * (kept prefix positions, retention state).  Weights, KV cache and ids stay
 * caller memory; dllm_destroy as usual. */
int dllm_create_static(dllm_ctx** out, const dllm_model_config* cfg, const dllm_gen_params* gp,
                       const dllm_weights* w, const dllm_kv_cache* kv, void* stream);

/* Repack one routed-expert gate or up weight tensor, exp [L][E][F][D]
 * row-major at d_src, into the packed fragment layout at d_dst (same byte
 * size, caller-allocated, must not overlap d_src).  With KL = 16 for fp8 and
 * 8 for bf16 / f32, and KC = 4 KL: for each [F][D] matrix, fragment (t, c) of
 * rows 16t..16t+15 and reduction columns KC c .. KC c + KC - 1 is 64 x KL
 * contiguous elements, element KL l + j holding W[16t + l%16][KC c +
 * KL (l/16) + j]; fragments ordered by (layer, expert, t, c).  This is the
 * order in which the matrix-core kernels read the weights, so each read is
 * one contiguous 64-lane access.  The fp8 per-row scales are unchanged.
 * Asynchronous on `stream`; DLLM_ERR_INVALID_ARG on a bad shape (F % 16, or
 * D % KC) or pointer. */
int dllm_pack_gate_up(const dllm_model_config* cfg, const void* d_src, void* d_dst, void* stream);

/* Bytes of one of the two KV cache buffers (K or V). */
size_t dllm_kv_bytes(const dllm_model_config* cfg, const dllm_gen_params* gp);

/* Tokens per sequence of each append pass dllm_block_init makes for this
 * shape: the most whole blocks whose model-row tokens (model rows x tokens)
 * fit in 4096, at least one block; lowered to gp->max_clean_tokens when that
 * is set and smaller, but never below block_length.  A call with n_clean
 * tokens runs ceil(n_clean / this) passes, the last one shorter.  Host only;
 * 0 on invalid arguments. */
int dllm_append_tokens(const dllm_model_config* cfg, const dllm_gen_params* gp);

/* Create a context.  `d_workspace` must hold dllm_workspace_bytes() bytes,
 * 256-byte aligned (DLLM_ERR_OUT_OF_MEMORY if smaller).  `stream` is a
 * hipStream_t (NULL: the default stream).  The cache starts empty (P = 0). */
int dllm_create(dllm_ctx** out, const dllm_model_config* cfg, const dllm_gen_params* gp,
                const dllm_weights* w, const dllm_kv_cache* kv,
                void* d_workspace, size_t ws_bytes, void* stream);

/* Append `n_clean` committed tokens per row to the cache and open a new block
 * (paper review, "BDLM": a finished block is later seen as clean context).
 * d_clean_ids: device int32 [rows][n_clean].  n_clean must be a multiple of
 * block_length (blocks are aligned from position 0; a prompt tail that is not
 * aligned goes into the first block as fixed ids) and at most
 * max_clean_tokens; P + n_clean <= max_prefix (else DLLM_ERR_OUT_OF_MEMORY).
 * n_clean = 0 only opens a new block. */
int dllm_block_init(dllm_ctx* ctx, const int32_t* d_clean_ids, int32_t n_clean);

/* One denoising step t (0 <= t < steps) of the open block (paper review,
 * SPRINT: non-uniform unmasking; model card: k = ceil(remaining/steps_left),
 * threshold batch acceptance).  d_ids_in / d_ids_out: device int32
 * [n_seq][block_length] (may alias); non-[MASK] ids are fixed.
 * d_remaining: device int32 [n_seq], [MASK] count after the step.
 * With use_sprint, steps t >= cache_warmup_steps need the warm-up step
 * (t = cache_warmup_steps - 1) of this block to have run
 * (DLLM_ERR_BAD_STATE otherwise). */
int dllm_denoise_step(dllm_ctx* ctx, int32_t t, const int32_t* d_ids_in, int32_t* d_ids_out,
                      int32_t* d_remaining);

/* The block loop of one block (paper review, "SPRINT": block diffusion costs
 * B x T forward passes, and with non-uniform unmasking a block can finish in
 * fewer than T steps; model card, "SPRINT" acceleration: steps per block,
 * threshold batch acceptance).  Runs dllm_denoise_step for t = 0, 1, ... on
 * d_ids (device int32 [n_seq][block_length], in place) until no [MASK]
 * remains in any sequence or the `steps` budget is spent; *h_steps_taken
 * (host) receives the number of steps run (0 if the first call failed).
 * Synchronises the stream once per step to read the remaining counts.  The
 * block stays open: append it with dllm_block_init(ctx, d_ids, block_length)
 * before generating the next one.  Errors: those of dllm_denoise_step
 * (DLLM_ERR_BAD_STATE without an open block), DLLM_ERR_HIP on a failed copy
 * or synchronisation. */
int dllm_generate_block(dllm_ctx* ctx, int32_t* d_ids, int32_t* h_steps_taken);

/* Current cached prefix length P (tokens per row). */
int32_t dllm_prefix_length(const dllm_ctx* ctx);

void dllm_destroy(dllm_ctx* ctx);
const char* dllm_last_error(const dllm_ctx* ctx);
const char* dllm_status_string(int status);

/* ---- inspection and decision checks (test support) ---------------------
 * dllm_debug_buffer returns a device pointer into the workspace and its size
 * for one internal result of the last step or forward:
 *   0 routing indices int32 [M][top_k] of layer `layer` (M = model rows x
 *     tokens of the last forward), 1 router gates f32 [M][top_k] (last layer),
 *   2 confidences f32 [n_seq][L_B] (-inf where not masked), 3 argmax ids
 *     int32 [n_seq][L_B], 4 attention mass f32 [rows][max_prefix],
 *   5 kept prefix positions int32 [rows][max_prefix], 6 kept counts int32
 *     [rows], 7 final hidden state f32 [M][D], 9 prefix key norms
 *     f32 [rows][max_prefix] (sum over layers and heads), 10 prefix top-1
 *     probabilities f32 [rows][max_prefix], 11 prefix ids int32
 *     [rows][max_prefix] (9-11 filled only when the knobs need them; buffer 4
 *     holds the retention score of the last selection), 13 the final-normed
 *     rows (LM-head input) of the last forward pass, act [M][D] (after
 *     dllm_block_init: the last append chunk's tokens, row-major by model row).
 * With an inspection buffer attached (dllm_debug_attach):
 *   8 masked-position logits f32 [n_masked x (2 with CFG, 4 with three-way
 *     guidance: full, image-only, uncond, uncond again)][V_sub] of the last
 *     step, recomputed on the call (synchronous) by the plain GEMM kernel from
 *     the step's final normed rows (the step itself keeps them on-chip),
 *   12 router logits f32 [M][E] of layer `layer`: the sums the top-k keys of
 *     the last forward pass were formed from.
 * Without one, 8 and 12 return DLLM_ERR_BAD_STATE. */
int dllm_debug_buffer(dllm_ctx* ctx, int32_t which, int32_t layer, void** d_ptr, size_t* bytes);

/* Bytes of the inspection buffer for this shape (0 on invalid arguments). */
size_t dllm_debug_bytes(const dllm_model_config* cfg, const dllm_gen_params* gp);

/* Attach caller device memory (>= dllm_debug_bytes, 256-byte aligned) as the
 * inspection buffer: later forward passes also write each layer's router
 * logits there, and dllm_debug_buffer 8 recomputes the head logits into it.
 * d_buf = NULL detaches (the step then writes nothing extra).  The buffer
 * stays the caller's; DLLM_ERR_OUT_OF_MEMORY if too small,
 * DLLM_ERR_INVALID_ARG if misaligned. */
int dllm_debug_attach(dllm_ctx* ctx, void* d_buf, size_t bytes);

/* Attention launch plan of the last forward pass (host ints): h_plan[0]
 * kernel (0 float32 partials, 1 128-key matrix-core partials, 2 streaming,
 * 3 append pass with 4 query blocks sharing each key tile), h_plan[1] keys
 * per workgroup, h_plan[2] workgroups per (row, head, query block). */
int dllm_debug_attn_plan(const dllm_ctx* ctx, int32_t* h_plan);

/* Block-wise attention alone, with the step's kernels and launch plan (paper
 * review, "BDLM" and "MoE backbone and block-wise attention": a block's
 * queries see every cached prefix key, or the retained subset, and the keys of
 * their own block bidirectionally; scale 1/sqrt(head_dim)).  One query block
 * of block_length positions per (row, head); elements in act_dtype
 * (DLLM_F32 or DLLM_BF16), RoPE already applied:
 *   d_q        [rows][n_heads][block_length][head_dim]
 *   d_kc, d_vc [rows][n_heads][cap][head_dim], prefix positions 0 .. P-1 read
 *              (may be NULL when P = 0)
 *   d_bk, d_bv [rows][n_heads][block_length][head_dim], the block's own keys
 *   d_kept     NULL (every prefix key), or int32 [rows][cap] retained prefix
 *              positions (ascending), d_n_kept int32 [rows] their counts
 *   d_out      [rows][block_length][n_heads * head_dim] (act_dtype)
 *   d_lse      NULL or f32 [rows][n_heads][block_length]: log-sum-exp of each
 *              query's scaled scores
 *   h_plan     NULL or host int32[3]: the plan (as dllm_debug_attn_plan).
 * head_dim 32, 64 or 128; 1 <= block_length <= 64; 0 <= P <= cap, P a
 * multiple of block_length (blocks are aligned from position 0).  Allocates
 * its key-split partials for the call and synchronises the stream.  Errors:
 * DLLM_ERR_INVALID_ARG on shapes or missing pointers, DLLM_ERR_HIP. */
int dllm_debug_block_attention(int32_t act_dtype, const void* d_q, const void* d_kc, const void* d_vc,
                               int32_t cap, const void* d_bk, const void* d_bv, const int32_t* d_kept,
                               const int32_t* d_n_kept, int32_t rows, int32_t n_heads, int32_t head_dim,
                               int32_t block_length, int32_t P, void* d_out, float* d_lse,
                               int32_t* h_plan, void* stream);

/* Router decision on given logits (same kernel as the step): d_logits f32
 * [n][E], d_bias f32 [E] -> d_idx int32 [n][k], d_gates f32 [n][k].
 * Runs on `stream`, synchronously. */
int dllm_debug_route(const float* d_logits, const float* d_bias, int32_t n, int32_t n_experts,
                     int32_t top_k, int32_t* d_idx, float* d_gates, void* stream);

/* Confidence + commit decision on given logits (same kernels as the step):
 * d_ids_in int32 [n_seq][L_B]; d_logits f32 [n_seq][L_B][V_sub] (rows of
 * non-masked positions are ignored); writes d_ids_out, d_remaining [n_seq],
 * d_conf f32 [n_seq][L_B] and d_xhat int32 [n_seq][L_B].  Synchronous. */
int dllm_debug_unmask(const int32_t* d_ids_in, const float* d_logits, int32_t n_seq,
                      int32_t block_length, int32_t v_sub, int32_t vocab_lo, int32_t mask_id,
                      int32_t steps, int32_t t, int32_t confidence, int32_t use_threshold,
                      float threshold, int32_t* d_ids_out, int32_t* d_remaining,
                      float* d_conf, int32_t* d_xhat, void* stream);

/* Retention decision on given scores (same kernel as the step): d_score f32
 * [rows][P] (>= 0) -> d_kept int32 [rows][P] (first d_count[r] entries valid,
 * ascending) and d_count int32 [rows].  d_ids int32 [rows][P] or NULL: with
 * ids, positions whose id is in [vis_lo, vis_hi) form the image pool and keep
 * ceil(image_keep_ratio P_img), the others ceil(text_keep_ratio P_text)
 * (ratios in (0, 1]); without, one pool keeps ceil(keep_ratio P).
 * Synchronous. */
int dllm_debug_retention(const float* d_score, int32_t rows, int32_t P, float keep_ratio,
                         const int32_t* d_ids, int32_t vis_lo, int32_t vis_hi,
                         float image_keep_ratio, float text_keep_ratio,
                         int32_t* d_kept, int32_t* d_count, void* stream);

/* E4M3FN -> float32 decode of n codes with the expert kernels' converter.
 * Synchronous. */
int dllm_debug_decode_fp8(const uint8_t* d_codes, int32_t n, float* d_out, void* stream);

/* ---- launch timing ------------------------------------------------------
 * dllm_profile_enable(ctx, groups): for each group g with bit (1 << g) set,
 * the context records a HIP event pair on its stream around every later
 * launch of that kernel group; groups = 0 stops recording (pairs already
 * recorded stay pending, no wait).  Each pair adds a marker to the stream, so
 * time only what is needed.  dllm_profile_read returns (and resets) the summed
 * milliseconds and launch counts per group, waiting for the recorded events.
 * Host arrays hold DLLM_PROF_GROUPS entries.  Unknown bits:
 * DLLM_ERR_INVALID_ARG. */
#define DLLM_PROF_EXPERT_GATEUP 0  /* grouped expert gate/up + SwiGLU */
#define DLLM_PROF_EXPERT_DOWN   1  /* grouped expert down projection */
#define DLLM_PROF_ATTN          2  /* block-wise attention: all its launches (partials and
                                        merge, or one streaming pass) */
#define DLLM_PROF_QKV           3  /* QKV projection */
#define DLLM_PROF_HEAD          4  /* LM head over masked rows */
#define DLLM_PROF_GROUPS        5
#define DLLM_PROF_ALL           ((1 << DLLM_PROF_GROUPS) - 1)
int dllm_profile_enable(dllm_ctx* ctx, int32_t groups);
int dllm_profile_read(dllm_ctx* ctx, double* h_ms, long long* h_count);

#ifdef __cplusplus
}
#endif
#endif /* DLLM_H */
