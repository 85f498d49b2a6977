// Kernel launch interface between the host runtime (runtime.cpp) and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

// Launch gate: a device int32 that, when nonzero as a kernel starts, makes every block of that
// kernel return at once.  The canvas loops point it at a flag their Step sets once every canvas is
// done, so the passes enqueued up front for the remaining steps cost only their launches, with no
// host read.  The current gate belongs to the calling host thread while a GateScope lives; every
// launcher below passes it to its kernel (null: always open).
const int32_t* launch_gate();
struct GateScope {
  const int32_t* prev;
  explicit GateScope(const int32_t* gate);
  ~GateScope();
};

constexpr int MAX_BATCH = 64;     // canvases per call
constexpr int GROUP_BM = 32;       // rows per expert tile of the grouped GEMMs
constexpr int GROUP_BM_WIDE = 128; // ... once experts average 64 rows or more (batched canvases)
constexpr int GROUP_BM_Q8 = 64;    // rows per routed tile below that with W8A8 experts
// rows per routed expert tile for `picks` = rows x top_k routed rows over E experts
inline int group_bm(int64_t picks, int E) { return picks >= (int64_t)64 * E ? GROUP_BM_WIDE : GROUP_BM; }

enum WKind { W_F32 = 0, W_BF16 = 1, W_FP8 = 2, W_MXFP4 = 3, W_FP8A8 = 4 };  // W_FP8A8: fp8 weights, e4m3 activations
enum Epi { EPI_STORE_F32 = 0, EPI_ADD_F32 = 1, EPI_STORE_ACT = 2, EPI_SWIGLU = 3, EPI_QKV = 4 };

struct DenseArgs {
  int epi;
  const void* A; int64_t lda;            // activations [M][K]
  const void* B; const void* B2;         // weights [N][K]; B2 = up matrix for SwiGLU
  int64_t ldb;
  const uint16_t* sB; const uint16_t* sB2;  // fp8 per-row scales (bf16)
  int M, N, K;                           // N: output columns (SwiGLU: hidden width)
  void* C; int64_t ldc;
  const float* bias;                     // per-column fp32 bias or null
  int ksplit;                            // split-K parts (EPI_STORE_F32 only; part s -> C + s*c_split)
  int64_t c_split;
  int n_mt, n_nt;                        // filled by the launcher
  // QKV + RoPE
  void* q_out; void* k_out; void* v_out; // q [M][Hq][dh]; k [B][Hkv][rows_per_canvas][dh];
                                         // v d-major [B][Hkv][dh][v_ld]
  int Hq, Hkv, dh, rows_per_canvas, v_ld;
  const float2* rope;                    // (cos, sin) [M][dh/2] from launch_rope_table
  const int32_t* gate;                   // launch gate (set by the launcher)
};

// (cos, sin) table [rows][head_dim/2] for the RoPE positions plen[b] + i of canvas rows; plen is
// device [B], each value clamped to [0, max_prefix] (a value outside sets bit 4 of *status)
hipError_t launch_rope_table(float2* tab, int rows, int rows_per_canvas, int head_dim, double log2_theta,
                             const int32_t* plen, int max_prefix, int* status, hipStream_t s);

struct GroupedArgs {
  int epi;
  const void* A; int64_t lda; const int32_t* a_tok;  // A row of grouped position p: a_tok[p] (or p)
  const void* B; const void* B2; int64_t ldb; int64_t b_estride;  // ldb, b_estride in storage units
  // quantised weights: fp8 per-row bf16 scales [E][N], or MXFP4 e8m0 block scales [E][N][K/32];
  // s_estride = bytes per expert, s_ld = bytes per weight row (MXFP4)
  const void* sB; const void* sB2; int64_t s_estride; int64_t s_ld;
  int N, K;
  const int32_t* work; const int32_t* n_items;       // (expert, first row) per tile
  const int32_t* offsets; const int32_t* counts;
  void* C; int64_t ldc;                               // output row = grouped position
  // shared expert (every row, in row order), tiles of GROUP_BM rows before the routed tiles
  const void* shA; int64_t sh_lda;
  const void* shB; const void* shB2; int64_t sh_ldb;
  const void* sh_sB; const void* sh_sB2; int64_t sh_s_ld;
  int shN, shK, sh_rows;
  void* shC; int64_t sh_ldc;
  int bm;                                             // rows per routed tile: GROUP_BM, GROUP_BM_Q8 or GROUP_BM_WIDE
  const float* sA; const float* sh_sA;                // W8A8: fp32 scale per A row (source row or grouped position)
  int nt_r, nt_s, sh_blocks, n_sh_items;              // filled by the launcher
  const int32_t* gate;                                // launch gate (set by the launcher)
};

hipError_t launch_dense(const DenseArgs& a, int act_bf16, int w_kind, hipStream_t s);
hipError_t launch_grouped(const GroupedArgs& a, int act_bf16, int w_kind, int max_items, hipStream_t s);

// ---- attention -------------------------------------------------------------------------------
struct AttnArgs {
  const void* q;          // [B*n][Hq][dh]
  const void* kn; const void* vn;   // new/canvas keys [B][Hkv][n][dh], values d-major [B][Hkv][dh][vn_ld]
  const void* kc; const void* vc;   // cache keys [B][Hkv][cap][dh], values d-major [B][Hkv][dh][cap]
  int B, n, Hq, Hkv, dh, cap, vn_ld;  // vn_ld: n rounded up to a multiple of 8
  int causal, window, is_global;
  const int32_t* seq_causal;        // device [B] or null: canvas b is causal iff seq_causal[b] != 0
                                    // (a mixed batch); null: `causal` holds for every canvas
  float scale_log2;       // log2(e) / sqrt(dh)
  int splits, keys_per_split;       // key-range split (multiple of 64 keys; fp32 kernel)
  int tiles_per_split;              // split of the 64-key tile list (bf16 kernel)
  float* part_o; float* part_ml;    // [splits][B*n][Hq][dh], [splits][B*n][Hq][2] (splits > 1);
                                    // part_o holds fp32 sums (fp32 kernel) or IEEE-half O_s / l_s (bf16)
  void* out;              // [B*n][Hq*dh] act (splits == 1)
  const int32_t* plen;    // device [B]: prefix length per canvas, clamped to [0, max_prefix]
  int max_prefix;
  const int32_t* gate;    // launch gate (set by the launcher)
};
hipError_t launch_attention(const AttnArgs& a, int act_bf16, hipStream_t s);
hipError_t launch_flash(const AttnArgs& a, hipStream_t s);
// bf16 attention blocks: FLASH_WAVES waves of FLASH_QPW 16-row query blocks each
constexpr int FLASH_QPW = 1, FLASH_WAVES = 8;
constexpr int FLASH_QROWS = 16 * FLASH_QPW * FLASH_WAVES;
hipError_t launch_attn_merge(const AttnArgs& a, int act_bf16, hipStream_t s);

// ---- elementwise / small kernels -------------------------------------------------------------
// resid[r] = embed[tokens[r]] (+ add[r] when add is non-null: the self-conditioning signal)
hipError_t launch_embed(const int32_t* tokens, const void* embed, float* resid, int rows, int d,
                        int vocab, int act_bf16, hipStream_t s, const float* add = nullptr);
// per-row dynamic e4m3 quantisation of bf16 rows x [rows][K] (row stride ldx): s[r] = max|x| / 448
// (fp32; 1 for an all-zero row), q[r][k] = nearest e4m3 code of x / s (ties to even, saturating)
hipError_t launch_quant_rows(const void* x, int64_t ldx, int rows, int K, uint8_t* q, float* s, hipStream_t st);
// out[i] = act(sum over nparts of parts[p * pstride + i]), parts summed in order
hipError_t launch_sum_parts_cast(const float* parts, int nparts, int64_t pstride, void* out, int64_t n, int act_bf16,
                                 hipStream_t s);
hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s);
hipError_t launch_rmsnorm(const float* x, const void* g, void* y, int rows, int d, float eps,
                          int act_bf16, int* status, hipStream_t s);
// seq_mask: device [B] or null; with it only canvases b with seq_mask[b] != 0 are appended at
// positions plen[b] .. (device [B], clamped to [0, max_prefix])
hipError_t launch_kv_append(const void* kn, const void* vn, int vn_ld, void* kc, void* vc, int B, int n,
                            int Hkv, int dh, int cap, int window, int is_global,
                            const int32_t* plen, int max_prefix, const int32_t* seq_mask, int act_bf16,
                            hipStream_t s);
// plen[b] += n for every canvas (seq_mask null) or those with seq_mask[b] != 0 (gated like the passes)
hipError_t launch_advance_prefix(int32_t* plen, int B, int n, const int32_t* seq_mask, hipStream_t s);
// *flag = 1 if every v[0..n) is nonzero, else 0 (never gated, nor is launch_fill_i32)
hipError_t launch_all_set(const int32_t* v, int n, int32_t* flag, hipStream_t s);
// resid += MoE output (gated expert rows + shared row; y and shared in the activation type, bf
// selecting bf16); with g, out = RMSNorm(resid) * g
hipError_t launch_moe_combine_norm(float* resid, const void* y, const void* shared, const float* gates,
                                   const int32_t* inv_perm, int rows, int d, int k, const void* g, void* out,
                                   float eps, int bf, int* status, hipStream_t s);
// resid += sum of nparts split-K partials; y = RMSNorm(resid) * g (d <= 4096)
hipError_t launch_resid_add_rmsnorm(float* resid, const float* parts, int nparts, int64_t pstride,
                                    const void* g, void* y, int rows, int d, float eps, int act_bf16,
                                    int* status, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s);
// block-AR: tokens before each sequence's first eos per canvas of out [K][B][L]
hipError_t launch_valid_tokens(const int32_t* out, int K, int B, int L, int32_t eos, int32_t* valid, int32_t* seen,
                               hipStream_t s);

// ---- routing ---------------------------------------------------------------------------------
// router logits = sum of `nparts` split-K partials (part p at parts + p*part_stride) + bias
hipError_t launch_router_topk(const float* parts, int nparts, int64_t part_stride, const float* bias,
                              int T, int E, int k, float* logits_out, int32_t* idx, float* gates,
                              hipStream_t s);
// counts/offsets [E], perm [T*k], inv_perm [T*k], tok [T*k] (token of grouped position),
// work [2*max_items] + n_items for BM-row tiles
hipError_t launch_route_tables(const int32_t* idx, int T, int E, int k, int32_t* counts,
                               int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* tok,
                               int32_t* work, int32_t* n_items, int bm, hipStream_t s);

// ---- sampler / Step --------------------------------------------------------------------------
struct SampArgs {
  const void* H; const void* E;   // [rows][d], [V][d] act
  int rows, d, V, L;
  float zscale_log2;              // log2(e) / tau
  uint32_t k0, k1, step;          // Philox key (seed) and step index
  int slices, v_per_slice;        // vocabulary split
  float* part;                    // [slices][rows][6] partial (m2, s, a, g2, y, w) as floats/ints
  const uint32_t* canvas_rng;     // device [B][4] (k0, k1, step, -) per canvas, or null: k0, k1, step
  void* pmat;                     // or null: [rows][V] act, 2^(z2 - the row's max over its vocabulary tile)
  float* ptile;                   // with pmat: [rows][n_vtiles] those tile maxima (log2 units)
  int n_vtiles;                   // vocabulary tiles of the sampler (V / its tile width, rounded up)
  const int32_t* gate;            // launch gate (set by the launcher)
};
hipError_t launch_lmhead_sampler(const SampArgs& a, int act_bf16, hipStream_t s);
// vocabulary tile width of the fused sampler for the activation dtype
inline int sampler_bn(int act_bf16) { return act_bf16 ? 256 : 128; }
// p_hat_0 in place: P[r][v] *= 2^(ptile[r][v / bn] - lse2[r]), lse2 = log2 of the row's partition sum
// (from the merged statistics: m * log2(e) - log2(c))
hipError_t launch_p_rescale(void* P, const float* ptile, const float* stats, int rows, int V, int bn, int n_vtiles,
                            int act_bf16, hipStream_t s);
// fused LM head tiles: rows x vocabulary entries per block step (bf16: 256 x 256 on 8 waves of 32
// rows, so a 256-row canvas is one row tile and every embedding tile streams once)
constexpr int SAMPLER_BM_BF16 = 256, SAMPLER_BN_BF16 = 256, SAMPLER_BM_F32 = 128, SAMPLER_BN_F32 = 128;
static_assert(SAMPLER_BN_BF16 == 256 && SAMPLER_BN_F32 == 128, "sampler_bn");
constexpr int SAMPLER_PART = 6;   // floats per (row, slice) partial: m2, s, a, g2, y, w
hipError_t launch_logits_partials(const float* z, int rows, int V, int L, float zscale_log2,
                                  uint32_t k0, uint32_t k1, uint32_t step, int slices,
                                  int v_per_slice, float* part, hipStream_t s);

struct StepArgs {
  const float* part; int slices;  // partials from the sampler
  int B, L;
  int32_t* canvas; uint8_t* lock; int32_t* n_locked; const int32_t* done;
  float lam, theta;
  uint32_t k0, k1, step;
  float* stats;                   // [rows][STAT_FIELDS]: m, a, c, y, best, H (a, y stored as int bits)
  int* status;
  int32_t* steps_taken;           // incremented for canvases that stepped (or null)
  int32_t* done_out;              // set when all positions locked (adaptive), or null
  int stats_only;                 // merge and write stats; leave canvas / lock / counts alone
  const uint32_t* canvas_rng;     // device [B][4] (k0, k1, step, -) per canvas, or null: k0, k1, step
  const float* lam_table;         // with canvas_rng: device [steps], lambda of canvas b = lam_table[step_b]
  const int32_t* gate;            // launch gate (set by the launcher)
};
constexpr int STAT_FIELDS = 6;
hipError_t launch_step_merge(StepArgs a, hipStream_t s);

// entropy-bounded step over merged stats: one block per canvas (L <= 1024)
struct EbArgs {
  const float* stats;             // [B*L][STAT_FIELDS]
  int B, L;
  int32_t* canvas;                // [B][L] out (canvases not done)
  int32_t* prev;                  // [B][L] argmax of the previous step (read if has_prev), then this step's
  int32_t* done;                  // [B] inout
  int32_t* n_accepted;            // [B] out, or null
  float* mean_entropy;            // [B] out, or null
  int32_t* steps_taken;           // [B] incremented for canvases that stepped, or null
  float gamma, stop_entropy;
  int has_prev, final_step, adaptive, vocab, vocab_log2;
  uint32_t k0, k1, step;
  const int32_t* gate;            // launch gate (set by the launcher)
};
hipError_t launch_eb_select(EbArgs a, hipStream_t s);

hipError_t launch_init_canvas(int32_t* canvas, uint8_t* lock, int B, int L, int V, uint32_t k0,
                              uint32_t k1, hipStream_t s);

// Static device scratch of dg_step_sample_noalloc: STATIC_SCRATCH_BYTES per device, 256-byte aligned.
// static_scratch returns the current device's copy (its address is looked up once per device).
constexpr size_t STATIC_SCRATCH_BYTES = size_t(2) << 20;
hipError_t static_scratch(void** out);

// Continuous block-AR scheduling: one sequence per block, after each pass (or, with init, before the
// first).  A sequence is denoising canvas k at step s, appending its finished canvas, or finished.
enum SeqPhase : int32_t { SEQ_DENOISE = 0, SEQ_APPEND = 1, SEQ_FINISHED = 2 };
struct SeqArgs {
  int B, L, K, T, V, adaptive, init;
  uint64_t seed;                  // canvas k draws from seed + k
  int32_t* state;                 // [B][4]: phase, k, s, steps taken on canvas k
  uint32_t* rng;                  // [B][4] out: key of seed + k, step s (the next pass's draws)
  int32_t* cur; uint8_t* lock;    // [B][L] working canvas and its locks
  const int32_t* n_locked;        // [B] from the Step of this pass
  int32_t* out; int32_t* steps;   // [K][B][L] finished canvases, [K][B] their steps (or null)
  int32_t* append; int32_t* skip; int32_t* finished;  // [B] flags for the next pass
  int32_t* passes;                // [1] passes that ran (or null)
  float* sc; int d;               // [B*L][d] self-conditioning signal (or null): cleared for canvases whose
                                  // next pass appends or starts a canvas
  const int32_t* gate;            // set by the launcher
};
hipError_t launch_seq_schedule(SeqArgs a, hipStream_t s);
// dst[0..n) = vals[0..n), n <= 256 (never gated)
hipError_t launch_write_f32(float* dst, const float* vals, int n, hipStream_t s);
hipError_t launch_noise(const int32_t* x0, int32_t* xt, int B, int L, int V, float kappa,
                        uint32_t k0, uint32_t k1, uint32_t step, hipStream_t s);

}  // namespace dg

namespace dg {
// Kernels needing more than 64 KB of dynamic LDS must say so once before their first launch.
template <class F>
inline hipError_t allow_lds(F* f, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(f), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}
}  // namespace dg
