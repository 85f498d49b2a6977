/*
 * dg.h — C ABI of the MI355X (gfx950) canvas denoise-step library, libdg.so.
 *
 * The library runs the data-parallel hot path of DiffusionGemma-style discrete text diffusion:
 * one denoising step over a block of 256-token canvases.  Sources for what is computed:
 *   [TR]  "DiffusionGemma Technical Report 정리" (juhoplayground.github.io):
 *         §Forward Process, §Backward Denoising Process, §아키텍처와 블록 자기회귀 생성 (block-AR
 *         generation: causal context encoding into a KV cache, bidirectional canvas decoder,
 *         append-after-encode), §디노이징 반복과 self-conditioning (T steps of size h = 1/T,
 *         p_hat = softmax(logits / tau)), §CPU-GPU 동기화 제거 (no host synchronisation).
 *   [PBD] the "parallel block decoding" explainer (molayo1419.me), glossary "Iterative
 *         denoising": each pass locks in high-confidence tokens and re-evaluates the rest.
 *   [CA]  "DiffusionGemma 완전분석" (cell-devlog), §스펙 정리: 30 layers, sliding window 1024,
 *         128 experts with 8 active plus one always-on shared expert, 262K vocabulary,
 *         256-token canvas.
 *
 * Conventions for every call:
 *   - Pointers named as device pointers must point to device memory allocated by the caller;
 *     descriptors, parameter structs, pointer tables and `cap` are host memory.
 *     Weight pointers must be 16-byte aligned (dg_create checks), as every allocator's are.
 *   - The library never allocates device memory.  All scratch lives in the caller's workspace
 *     (`ws`, at least dg_workspace_bytes() bytes, 256-byte aligned).  One workspace must not be
 *     used by two streams at once.
 *   - Arguments are validated on the host before anything is enqueued.  On failure the call
 *     returns a negative dg_status, dg_last_error() describes it, and nothing is enqueued.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream); no call synchronises
 *     the host except dg_query_status().  Buffers must stay alive until the work completes.
 *   - Row-major layouts throughout.  "act" = the model's activation dtype (F32 or BF16);
 *     BF16 tensors are raw 16-bit bf16 words.
 */
#ifndef DG_H_
#define DG_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DG_OK = 0,
  DG_EINVAL = -1,        /* null pointer, bad size, bad parameter value */
  DG_EUNSUPPORTED = -2,  /* shape outside what the kernels tile (see dg_create) */
  DG_EWORKSPACE = -3,    /* workspace smaller than dg_workspace_bytes() or misaligned */
  DG_EHIP = -4,          /* a HIP launch or runtime call failed */
  DG_ENONFINITE = -5     /* a non-finite hidden state or logit was seen (dg_query_status) */
} dg_status;

/* MXFP4 is the OCP microscaling format: e2m1 elements (1 sign, 2 exponent bits with bias 1, 1
 * mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) in blocks of 32 consecutive K-elements
 * sharing one e8m0 scale byte s (value 2^(s - 127); 255 is NaN). */
typedef enum { DG_F32 = 0, DG_BF16 = 1, DG_FP8E4M3 = 2, DG_MXFP4 = 3 } dg_dtype;

/* Noise schedule kappa_t: decreasing from kappa_0 = 1 to kappa_1 = 0 [TR §Forward Process]. */
typedef enum {
  DG_KAPPA_LINEAR = 0,     /* 1 - t          */
  DG_KAPPA_QUADRATIC = 1,  /* 1 - t^2        */
  DG_KAPPA_COSINE = 2      /* cos(pi t / 2)  */
} dg_schedule;

/* Model shape.  Layer l (0-based) is global iff window <= 0, global_every <= 0 or
 * (l + 1) % global_every == 0; other layers are local (sliding window `window`).
 * Supported: head_dim in {64, 128, 256}; n_q_heads % n_kv_heads == 0; d_model, expert_hidden
 * and shared_hidden multiples of 64; vocab % 16 == 0; top_k <= n_experts <= 256, n_experts % 4 == 0, top_k <= 16;
 * act_dtype F32 or BF16;
 * expert_dtype = act_dtype, or FP8E4M3 / MXFP4 when act_dtype is BF16 (weights-only: the codes are
 * widened exactly to bf16 and the math is bf16 MFMA; with expert_act_fp8 = 1 and FP8E4M3 weights the
 * expert inputs are quantised too, W8A8, and the products run on the fp8 MFMA). */
typedef struct {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim;
  int32_t n_experts, top_k, expert_hidden, shared_hidden, vocab;
  int32_t window, global_every;
  float rope_theta; /* RoPE base (rotate-half pairs j, j + head_dim/2) */
  float norm_eps;   /* RMSNorm epsilon */
  dg_dtype act_dtype, expert_dtype;
  int32_t sc_hidden; /* hidden width of the self-conditioning block (multiple of 64; vocab % 64 == 0),
                        0: the model has none [TR §디노이징 반복과 self-conditioning] */
  int32_t expert_act_fp8; /* 1: W8A8 experts (needs expert_dtype FP8E4M3, act_dtype BF16; the pages
                        measure fp8 builds [TR §배치 크기 1 처리량] and fix no activation scheme): each
                        row of an expert GEMM's input, the FFN-normalised rows and the SwiGLU products
                        (stored bf16 first), is coded to e4m3 with the float32 scale max|row| / 448 (1 for a
                        zero row; codes by round-to-nearest-even of the float32 quotient, saturating);
                        a product is (codes . codes) * row scale * weight scale; needs expert_hidden
                        and shared_hidden <= 4096.  0: the expert inputs stay in act_dtype */
} dg_model_desc;

/* One layer's weights: device pointers, borrowed until dg_destroy().  Every matrix is stored
 * [out][in] (both GEMM operands K-contiguous).  Expert matrices use expert_dtype; with
 * FP8E4M3 each has a bf16 scale per output row (s_*), and the weight is code * scale.  With
 * MXFP4 an expert matrix [N][K] is stored as N rows of K/2 bytes (element 2j in the low nibble of
 * byte j) and its s_* array holds N rows of K/32 e8m0 bytes (one per 32 consecutive elements):
 * weight = e2m1(code) * 2^(s - 127).  Matrix pointers must be 16-byte aligned; scale arrays have
 * no alignment requirement. */
typedef struct {
  const void *attn_norm;   /* [d] act, RMSNorm gain before attention                       */
  const void *w_qkv;       /* [(Hq + 2 Hkv) dh][d] act: q heads, then k heads, then v heads */
  const void *w_o;         /* [d][Hq dh] act                                                */
  const void *ffn_norm;    /* [d] act                                                       */
  const void *w_router;    /* [E][d] act                                                    */
  const float *router_bias;/* [E] fp32 added to the router logits, or NULL                  */
  const void *w_gate, *w_up;      /* [E][f][d] expert dtype                                 */
  const void *w_down;             /* [E][d][f]                                              */
  const void *s_gate, *s_up;      /* [E][f] bf16 (FP8), [E][f][d/32] e8m0 (MXFP4), else NULL */
  const void *s_down;             /* [E][d] bf16 (FP8), [E][d][f/32] e8m0 (MXFP4)            */
  const void *sh_gate, *sh_up;    /* [fs][d] shared expert                                  */
  const void *sh_down;            /* [d][fs]                                                */
  const void *sh_s_gate, *sh_s_up, *sh_s_down; /* [fs], [fs], [d] bf16 scales (FP8) or
                                  [fs][d/32], [fs][d/32], [d][fs/32] e8m0 (MXFP4)          */
} dg_layer_weights;

typedef struct {
  const void *embed;        /* [V][d] act: tied input embedding and LM head; NULL allowed
                               only for calls that take resid_in and produce no logits        */
  const void *final_norm;   /* [d] act                                                        */
  const dg_layer_weights *layers; /* host array [n_layers]                                    */
  /* self-conditioning (sc_hidden > 0, else NULL): s = FFW(p_hat_0 . E) with the gated block
   * A = silu(x sc_gate^T) * (x sc_up^T), s = A sc_down^T, x = p_hat_0 . E stored in act.      */
  const void *embed_t;      /* [d][V] act: E transposed, so the product over the vocabulary
                               streams K-contiguous rows (same values as embed)                */
  const void *sc_gate, *sc_up; /* [sc_hidden][d] act                                          */
  const void *sc_down;      /* [d][sc_hidden] act                                              */
} dg_weights;

/* Prefix KV cache, filled by the causal encoder (dg_prefill_kv) or by the caller.  The prefix
 * lengths live on the device, so a loop on the device can advance them without a host read
 * ([TR §CPU-GPU 동기화 제거]); the host passes only an upper bound, used to size the grids and to
 * check the caches' capacity before anything is enqueued.
 * k[l]: device [batch][Hkv][cap[l]][dh] act, keys stored after RoPE (slot-major rows).
 * v[l]: device [batch][Hkv][dh][cap[l]] act, values stored head-dim-major (one row of cap[l]
 * slots per head-dim index), so value tiles stream into the attention kernel's LDS as stored.
 * Global layers keep position p in slot p (cap[l] >= every prefix length).  Local layers keep
 * a ring of cap[l] == window slots, position p in slot p % window.  cap[l] must be a multiple
 * of 8 (DG_EUNSUPPORTED otherwise). */
typedef struct {
  void *const *k;            /* host array [n_layers] of device pointers */
  void *const *v;
  const int32_t *cap;        /* host [n_layers] */
  int32_t *prefix_len;       /* device [batch], in/out: tokens already encoded for each canvas.
                                dg_prefill_kv and the append canvases of dg_mixed_forward add the
                                tokens they encode; every other call only reads it. */
  int32_t max_prefix;        /* host: an upper bound on every prefix_len[b] when the call starts.
                                A device value outside [0, max_prefix] is clamped into it and
                                flagged: dg_query_status then returns DG_EINVAL. */
  int32_t batch;
} dg_kv;

/* One Step [TR §Backward Denoising Process; PBD "Iterative denoising"].
 * Unlocked position: c = max_v p(v) >= lock_threshold -> take the argmax and lock; otherwise
 * with probability lambda = min(1, h |kappa'(t)| / (1 - kappa(t))) jump to a token drawn from
 * p = softmax(logits / tau) (Gumbel-max with Philox4x32-10 noise), else keep the token. */
typedef struct {
  dg_schedule schedule;
  float t, h, tau, lock_threshold; /* lock_threshold > 1 disables lock-in */
  uint64_t seed;
  uint32_t step;                   /* step index s: part of every random-draw counter */
} dg_step_params;

/* The pages' default sampler, one entropy-bounded step [TR §DiffusionGemma 샘플러].  With
 * p = softmax(logits / tau_t), tau_t = tau_end + (tau_start - tau_end) t (0.8 -> 0.4 on the pages),
 * each position has entropy H (nats), argmax a and a Gumbel-max draw y from p.  Positions are
 * taken in ascending (H, position) order while the float32 running sum of their entropies stays
 * <= gamma (0.1): those take y, every other position a uniform re-noise token (Philox stream tag 5).
 * A canvas stops (adaptive) when has_prev is set, its argmax sequence equals the previous step's
 * and its mean entropy (float32 sum in the same order / L) is below stop_entropy (0.005); a
 * stopped canvas, and every canvas at final_step, takes its argmax sequence and is marked done. */
typedef struct {
  float t;                         /* denoising time of this step, 0 < t <= 1 */
  float tau_start, tau_end;        /* temperature at t = 1 and at t = 0 */
  float gamma, stop_entropy;
  uint64_t seed;
  uint32_t step;                   /* step index s: part of every random-draw counter */
  int32_t has_prev;                /* prev_argmax holds the previous step's argmax sequence */
  int32_t final_step;              /* last step of the loop */
  int32_t adaptive;                /* 0: never stop before final_step */
} dg_eb_params;

typedef enum {
  DG_SAMPLER_EULER = 0,            /* dg_step_sample: Euler jump + confidence lock-in */
  DG_SAMPLER_ENTROPY_BOUNDED = 1   /* dg_step_entropy_bounded (lock is not used) */
} dg_sampler;

typedef struct {
  dg_schedule schedule;
  int32_t max_steps;            /* T: steps at t_s = 1 - s/T, s = 0..T-1, h = 1/T */
  float tau, lock_threshold;    /* entropy-bounded: tau is tau_start */
  uint64_t seed;
  int32_t adaptive;             /* 1: a canvas stops early (all locked / the entropy stop rule) */
  int32_t init_canvas;          /* 1: draw the canvas uniformly at t = 1 (and clear the lock) */
  dg_sampler sampler;           /* DG_SAMPLER_EULER (0) or DG_SAMPLER_ENTROPY_BOUNDED */
  float gamma, stop_entropy, tau_end;   /* entropy-bounded sampler only */
  int32_t self_condition;       /* 1: feed s = FFW(p_hat_0 . E) of each step into the next step's
                                   decoder (s = 0 at a canvas's first step); needs sc_hidden > 0 */
} dg_run_params;

typedef struct dg_ctx dg_ctx;   /* opaque, host-side; holds the descriptor and borrowed weights */

/* Validates the descriptor (DG_EUNSUPPORTED outside the supported shapes) and the weight
 * table (DG_EINVAL on a NULL matrix), then copies both.  *out is owned by the caller. */
dg_status dg_create(const dg_model_desc *desc, const dg_weights *weights, dg_ctx **out);
void dg_destroy(dg_ctx *ctx);

/* Workspace needed by any call with up to `batch` canvases of `rows_per_canvas` rows (canvas
 * length, or tokens per prefill call) and prefixes up to `max_prefix` tokens. */
size_t dg_workspace_bytes(const dg_ctx *ctx, int32_t batch, int32_t rows_per_canvas,
                          int32_t max_prefix);

/* Thread-local description of the last failure; valid until the next dg_* call. */
const char *dg_last_error(void);

/* Waits for `stream`, then reads the workspace status word: DG_ENONFINITE if a non-finite
 * hidden state or logit was seen since the workspace was last cleared (dg_clear_status). */
dg_status dg_query_status(const dg_ctx *ctx, const void *ws, hipStream_t stream);
dg_status dg_clear_status(const dg_ctx *ctx, void *ws, hipStream_t stream);

/* Causal encoder pass ("context encoding" and "append after encode", [TR §아키텍처와 블록
 * 자기회귀 생성]): tokens [batch][n] (device int32) at positions prefix_len[b] .. + n - 1 attend
 * causally (window on local layers) to the cache and to each other; their post-RoPE keys and
 * values are written into every layer's cache, and n is added to prefix_len[b] on the device.
 * Global-layer caches need cap >= max_prefix + n. */
dg_status dg_prefill_kv(dg_ctx *ctx, const dg_kv *kv, const int32_t *tokens, int32_t n,
                        void *ws, size_t ws_bytes, hipStream_t stream);

/* Decoder pass over the canvases ([TR §아키텍처와 블록 자기회귀 생성]: the decoder refines the
 * canvas with bidirectional attention over the encoder's KV cache, no causal mask inside the canvas;
 * [CA §스펙 정리]: sliding window 1024 on local layers, 8 of 128 routed experts plus one always-on
 * shared expert): bidirectional attention of every canvas position over the
 * visible prefix (all of it on global layers, the last `window` positions on local layers)
 * plus the whole canvas, then the MoE FFN with the shared expert; layers
 * [layer_begin, layer_end).  Input: canvas tokens (device int32 [batch][L], embedded by row
 * lookup of `embed`) or, when resid_in is non-NULL, the fp32 residual stream [batch*L][d].
 * Output: hidden_out [batch*L][d] act = RMSNorm(residual) * final_norm (may be NULL), and
 * resid_out [batch*L][d] fp32 = the residual after layer_end - 1 (may be NULL).
 * sc_in (nullable, device [batch*L][d] fp32): the self-conditioning signal s_t, added to the
 * embedded canvas ([TR §디노이징 반복과 self-conditioning]: the decoder takes x_t, the cache and s_t);
 * only with canvas tokens and layer_begin 0.
 * Canvas position i of canvas b has RoPE position prefix_len[b] + i. */
dg_status dg_denoise_step(dg_ctx *ctx, const dg_kv *kv, const int32_t *canvas,
                          const float *resid_in, const float *sc_in, int32_t L, int32_t layer_begin,
                          int32_t layer_end, void *hidden_out, float *resid_out,
                          void *ws, size_t ws_bytes, hipStream_t stream);

/* One pass over a batch that mixes the two kinds of forward pass ([TR §CPU-GPU 동기화 제거]:
 * denoising steps and cache updates share a batch, told apart by a per-sequence causal flag, with
 * no host synchronisation).  tokens: device int32 [batch][L]; append: device int32 [batch], read
 * only by the kernels.  Canvas b with append[b] != 0 takes the dg_prefill_kv pass: causal
 * attention to the cache and to itself, its keys and values written at positions prefix_len[b]
 * .. + L - 1 of every layer's cache, and L added to prefix_len[b] on the device.  Canvas b with
 * append[b] == 0 takes the dg_denoise_step pass: bidirectional attention over its prefix and
 * canvas, its cache untouched.  Every row then runs the MoE FFN of every layer; hidden_out
 * [batch*L][d] act = RMSNorm(residual) * final_norm for all rows (for an append canvas, the causal
 * encoder's output).  Pass `append` as dg_step_sample's `done` to step only the denoising
 * canvases.  resid_out (nullable, [batch*L][d] fp32) receives the residual before the final norm.
 * The global-layer caches need cap >= max_prefix + L. */
dg_status dg_mixed_forward(dg_ctx *ctx, const dg_kv *kv, const int32_t *tokens,
                           const int32_t *append, int32_t L, void *hidden_out, float *resid_out,
                           void *ws, size_t ws_bytes, hipStream_t stream);

/* Fused LM head + Step: logits = hidden [batch*L][d] . embed^T are streamed through an online
 * max / sum-exp / Philox-Gumbel argmax and never stored; then every position of canvas
 * (device int32 [batch][L], in/out) and lock (device uint8 [batch][L], in/out) is updated as
 * described at dg_step_params.  n_locked (device int32 [batch], out, may be NULL) receives the
 * locked count per canvas, or -1 if a non-finite value was seen in that canvas.
 * `done` (device int32 [batch], may be NULL): canvases with done[b] != 0 are left unchanged.
 * sc_out (nullable, device [batch*L][d] fp32; needs sc_hidden > 0): the self-conditioning signal
 * for the next step, s = FFW(p_hat_0 . E) with p_hat_0 the Step's softmax(logits / tau), formed
 * from the same vocabulary pass (its probabilities kept for a second product with E). */
dg_status dg_step_sample(dg_ctx *ctx, const void *hidden, int32_t *canvas, uint8_t *lock,
                         int32_t *n_locked, const int32_t *done, float *sc_out, int32_t batch,
                         int32_t L, const dg_step_params *params, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/* dg_step_sample for callers that cannot allocate device memory or hand over a workspace (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the same kernels and
 * outputs, with the scratch (status word, per-row statistics, vocabulary-slice partials, about 1.6 MB
 * for up to 16,384 rows) in a static array of 2 MiB that the library holds on every GPU it runs on
 * until the process ends.  Nothing is allocated.  Shapes whose scratch exceeds 2 MiB are rejected with
 * DG_EUNSUPPORTED before anything is enqueued.  Every call on one GPU shares that GPU's array, so calls
 * that overlap on one GPU (two streams, two threads) race; calls in order on one stream do not.
 * A non-finite statistic shows as n_locked[b] = -1 (there is no workspace status word to query). */
dg_status dg_step_sample_noalloc(dg_ctx *ctx, const void *hidden, int32_t *canvas, uint8_t *lock,
                                 int32_t *n_locked, const int32_t *done, int32_t batch, int32_t L,
                                 const dg_step_params *params, hipStream_t stream);

/* One entropy-bounded step (see dg_eb_params) from final-normed hidden states [batch*L][d]:
 * the fused LM head accumulates argmax, Gumbel-max draw and entropy in one pass over the
 * vocabulary, then one block per canvas selects.  canvas device int32 [batch][L] (out for
 * canvases not done); prev_argmax device int32 [batch][L] (in when has_prev, out: this step's
 * argmax); done device int32 [batch] (inout: done canvases are skipped); n_accepted (int32
 * [batch]) and mean_entropy (float [batch]) are optional outputs.  L <= 1024. */
dg_status dg_step_entropy_bounded(dg_ctx *ctx, const void *hidden, int32_t *canvas, int32_t *prev_argmax,
                                  int32_t *done, int32_t *n_accepted, float *mean_entropy, int32_t batch,
                                  int32_t L, const dg_eb_params *params, void *ws, size_t ws_bytes,
                                  hipStream_t stream);

/* The denoising loop for one block [TR §디노이징 반복과 self-conditioning]: optional uniform
 * canvas at t = 1, then up to max_steps of dg_denoise_step + the sampler's step at t_s = 1 - s/T.
 * All max_steps passes are enqueued at once with no host synchronisation ([TR §CPU-GPU 동기화
 * 제거]); with `adaptive`, once every canvas has stopped ([TR §DiffusionGemma 샘플러, adaptive
 * stopping]) each kernel of the remaining passes returns at entry, so a batch that stops early
 * costs only the launches of the passes it skips.
 * DG_SAMPLER_EULER: dg_step_sample; with `adaptive`, a canvas whose positions are all locked is
 * left unchanged by later steps.  DG_SAMPLER_ENTROPY_BOUNDED: dg_step_entropy_bounded with
 * tau_start = tau and the given tau_end, gamma, stop_entropy; `lock` may be NULL.
 * steps_taken (device int32 [batch], out, may be NULL) counts the steps each canvas took. */
dg_status dg_canvas_run(dg_ctx *ctx, const dg_kv *kv, int32_t *canvas, uint8_t *lock,
                        int32_t *steps_taken, int32_t L, const dg_run_params *params,
                        void *ws, size_t ws_bytes, hipStream_t stream);

/* Block-AR generation [TR §아키텍처와 블록 자기회귀 생성; §추론 효율 지표] after the caller has
 * encoded the prompt with dg_prefill_kv (kv->prefix_len = prompt lengths): K canvases of L tokens;
 * canvas k is denoised by dg_canvas_run with `params` (random streams of seed + k, canvas drawn
 * uniform at t = 1) and, except the last, appended to the KV cache by the causal encoder at
 * positions prefix_len[b] .. (which then advance by L on the device).  Global-layer caches need
 * cap >= max_prefix + (K - 1) L.  out: device int32 [K][batch][L]; steps: device int32 [K][batch]
 * (denoising steps of each canvas, may be NULL); valid: device int32 [K][batch] (tokens before the
 * sequence's first eos_id, L for a canvas without one, 0 after it; may be NULL); eos_seen: device
 * int32 [K][batch] (canvas holds an eos_id; may be NULL).  On return kv->prefix_len has grown by
 * (K - 1) L.  No host synchronisation; eos only decides which tokens count. */
dg_status dg_generate(dg_ctx *ctx, const dg_kv *kv, int32_t *out, int32_t *steps, int32_t *valid,
                      int32_t *eos_seen, int32_t K, int32_t L, int32_t eos_id, const dg_run_params *params,
                      void *ws, size_t ws_bytes, hipStream_t stream);

/* Block-AR generation with every sequence on its own schedule ([TR §CPU-GPU 동기화 제거]: denoising
 * canvases and cache updates share a batch, told apart by a per-sequence flag; [TR §DiffusionGemma
 * 샘플러]: a canvas stops refining once settled).  Same results per sequence as dg_generate with the
 * Euler sampler: canvas k of sequence b is denoised from a uniform canvas with the random streams of
 * seed + k and, except the last, appended to the cache at positions prefix_len[b] ..  But each pass
 * is one dg_mixed_forward over all sequences: a sequence whose canvas has stopped (every position
 * locked with `adaptive`, or max_steps steps taken) appends it in the next pass while the others keep
 * denoising, then starts its next canvas — all decided on the device.  Sequence b thus uses
 * sum_k steps[k][b] + K - 1 passes (the denominator of tokens per forward pass, [TR §추론 효율
 * 지표]); the batch runs until its longest sequence finishes.  All K max_steps + K - 1 passes are
 * enqueued at once; those after the last sequence finishes return at kernel entry.
 * Arguments as for dg_generate (params->sampler must be DG_SAMPLER_EULER, max_steps <= 256); passes
 * (device int32 [1], may be NULL) receives the number of passes that ran.  Global-layer caches need
 * cap >= max_prefix + (K - 1) L; on return kv->prefix_len has grown by (K - 1) L. */
dg_status dg_generate_continuous(dg_ctx *ctx, const dg_kv *kv, int32_t *out, int32_t *steps, int32_t *valid,
                                 int32_t *eos_seen, int32_t *passes, int32_t K, int32_t L, int32_t eos_id,
                                 const dg_run_params *params, void *ws, size_t ws_bytes, hipStream_t stream);

/* lambda of one Step as the library computes it (host function, float32 result). */
float dg_jump_prob(dg_schedule schedule, float t, float h);

/* The canvas at t = 1 [TR §Forward Process: the uniform prior]: every position an independent
 * uniform token from the Philox canvas-init stream of `seed`.  canvas device int32 [batch][L];
 * lock (device uint8 [batch][L], may be NULL) is cleared. */
dg_status dg_init_canvas(int32_t *canvas, uint8_t *lock, int32_t batch, int32_t L, int32_t vocab,
                         uint64_t seed, hipStream_t stream);

/* ---- kernel timing (HIP events recorded around the library's own launches) -------------- */
typedef enum {
  DG_PROF_MOE_GATE_UP = 0, DG_PROF_MOE_DOWN = 1, DG_PROF_ATTENTION = 2, DG_PROF_SAMPLER = 3,
  DG_PROF_QKV = 4, DG_PROF_O_PROJ = 5,
  DG_PROF_SHARED = 6,   /* records nothing: the shared expert runs inside the two MoE launches */
  DG_PROF_ROUTING = 7,
  DG_PROF_SELF_COND = 8,   /* the self-conditioning product with E and its feed-forward block */
  DG_PROF_NORM_COMBINE = 9,/* residual adds fused with RMSNorm, and the MoE combine (with the next norm) */
  DG_PROF_STEP = 10,       /* the merge of the sampler's partials and the Step */
  DG_PROF_EMBED = 11,      /* canvas embedding and the RoPE angle table */
  DG_PROF_N = 12
} dg_prof_class;

/* Starts recording a pair of events around every launch of the classes in `mask` (bit i =
 * class i; 0 stops).  Recording adds a timestamp write before and after each such launch (timing
 * events without a system-scope fence, so they do not stall the following launch). */
dg_status dg_profile_enable(dg_ctx *ctx, uint32_t mask);
/* Waits for the recorded launches of class `cls`, returns their summed duration (ms) and
 * count, and forgets them. */
dg_status dg_profile_read(dg_ctx *ctx, int32_t cls, double *total_ms, int32_t *launches);

/* ---- hooks for parity tests (same kernels as the calls above, exposed piecewise) ---------- */

/* Step from given fp32 logits z [batch*L][vocab] (device; divided by tau like the fused path).
 * Uses the merge/Step kernel of dg_step_sample; the statistics are readable afterwards. */
dg_status dg_test_step_from_logits(dg_ctx *ctx, const float *logits, int32_t *canvas,
                                   uint8_t *lock, int32_t *n_locked, int32_t batch, int32_t L,
                                   const dg_step_params *params, void *ws, size_t ws_bytes,
                                   hipStream_t stream);

/* Entropy-bounded step from given fp32 logits z [batch*L][vocab] (device; divided by tau_t like
 * the fused path); same outputs as dg_step_entropy_bounded, statistics readable afterwards. */
dg_status dg_test_eb_from_logits(dg_ctx *ctx, const float *logits, int32_t *canvas, int32_t *prev_argmax,
                                 int32_t *done, int32_t *n_accepted, float *mean_entropy, int32_t batch,
                                 int32_t L, const dg_eb_params *params, void *ws, size_t ws_bytes,
                                 hipStream_t stream);

/* The selection of the entropy-bounded step alone, from given per-position float32 entropies,
 * argmax and Gumbel-max draws (device, [batch*L] each); same outputs as dg_step_entropy_bounded. */
dg_status dg_test_eb_select(dg_ctx *ctx, const float *entropy, const int32_t *argmax, const int32_t *draw,
                            int32_t *canvas, int32_t *prev_argmax, int32_t *done, int32_t *n_accepted,
                            float *mean_entropy, int32_t batch, int32_t L, const dg_eb_params *params, void *ws,
                            size_t ws_bytes, hipStream_t stream);

/* Copies the per-row sampler statistics of the last Step out of the workspace (device outputs,
 * [rows] each, any may be NULL): max logit/tau, its argmax, confidence c, Gumbel argmax y, its
 * key (logit/tau + Gumbel) and the entropy of softmax(logit/tau) in nats. */
dg_status dg_test_read_stats(const dg_ctx *ctx, const void *ws, int32_t rows, float *m,
                             int32_t *a, float *c, int32_t *y, float *best, float *entropy,
                             hipStream_t stream);

/* Top-k routing of given fp32 scores [T][E] (device): idx/gates [T][k]; counts/offsets [E];
 * perm [T*k] = assignment id t*k+s at each expert-grouped position.  Any output may be NULL. */
dg_status dg_test_router_topk(const float *scores, int32_t T, int32_t E, int32_t k,
                              int32_t *idx, float *gates, int32_t *counts, int32_t *offsets,
                              int32_t *perm, void *ws, size_t ws_bytes, hipStream_t stream);

/* Routing of the last layer run by dg_denoise_step, read from the workspace: router logits
 * [rows][E] fp32 (bias included), idx/gates [rows][k]. */
dg_status dg_test_read_routing(const dg_ctx *ctx, const void *ws, int32_t rows, float *logits,
                               int32_t *idx, float *gates, hipStream_t stream);

/* Forward noising x_t ~ p_t(. | x0) [TR §Forward Process] with the library's random streams:
 * x0, xt device int32 [batch][L]. */
dg_status dg_test_noise(const int32_t *x0, int32_t *xt, int32_t batch, int32_t L, int32_t vocab,
                        dg_schedule schedule, float t, uint64_t seed, uint32_t step,
                        hipStream_t stream);

/* The expert inputs of the last layer run by dg_denoise_step over batch x L rows (R = batch*L),
 * read from the workspace (device outputs, any may be NULL): xhat [R][d] act (the FFN-normalised
 * rows), a_grp [R*top_k][expert_hidden] act (the routed SwiGLU products in expert-grouped order:
 * experts ascending, each expert's assignments t*top_k+s ascending), sh_a [R][shared_hidden] act;
 * with expert_act_fp8 = 1 also their e4m3 codes and float32 row scales (xq/xs, aq/as, shq/shs;
 * asking for them otherwise is DG_EINVAL). */
dg_status dg_test_read_expert_inputs(const dg_ctx *ctx, const void *ws, int32_t batch, int32_t L,
                                     void *xhat, uint8_t *xq, float *xs, void *a_grp, uint8_t *aq,
                                     float *as, void *sh_a, uint8_t *shq, float *shs,
                                     hipStream_t stream);

/* W8A8 activation coding of bf16 rows x [rows][K] (device, row stride K, K % 8 == 0, K <= 4096), as the
 * experts take their inputs when expert_act_fp8 = 1: s [rows] float32 = max|row| / 448 (1 for a
 * zero row), q [rows][K] e4m3 codes of x / s (round to nearest even, saturating at 448). */
dg_status dg_test_quant_rows(const void *x, int32_t rows, int32_t K, uint8_t *q, float *s,
                             hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DG_H_ */
