// Host side of libdg: argument validation, workspace carving and the launch sequence of each
// C-ABI call.  Nothing here allocates device memory or synchronises the host (except
// dg_query_status); every launch goes onto the caller's stream.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/dg.h"
#include "internal.h"

using namespace dg;

// Event pairs recorded around the launches of the profiled kernel classes.
struct Prof {
  uint32_t mask = 0;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> recs[DG_PROF_N];
  std::vector<hipEvent_t> pool;
  ~Prof() {
    for (auto& v : recs)
      for (auto& p : v) { (void)hipEventDestroy(p.first); (void)hipEventDestroy(p.second); }
    for (auto e : pool) (void)hipEventDestroy(e);
  }
  hipEvent_t get() {
    if (!pool.empty()) { hipEvent_t e = pool.back(); pool.pop_back(); return e; }
    // timing-only events: no system-scope fence on record (a fence writes back and invalidates
    // the caches, a ~5 us stall of the next launch; elapsed times are read after the event syncs)
    hipEvent_t e = nullptr;
    (void)hipEventCreateWithFlags(&e, hipEventDisableSystemFence);
    return e;
  }
};

struct dg_ctx {
  dg_model_desc d;
  std::vector<dg_layer_weights> layers;
  const void* embed;
  const void* final_norm;
  const void* embed_t;                       // self-conditioning: E transposed, [d][V]
  const void* sc_gate; const void* sc_up; const void* sc_down;
  Prof* prof;
};

namespace {

thread_local std::string g_err;

dg_status fail(dg_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

#define HIPCHK(expr)                                                                            \
  do {                                                                                          \
    hipError_t e_ = (expr);                                                                     \
    if (e_ != hipSuccess) return fail(DG_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

constexpr size_t ALIGN = 256;
constexpr int MAX_SPLITS = 16;
constexpr int MAX_RSPLIT = 16;   // split-K parts of the router GEMM
constexpr int MAX_KSPLIT = 8;    // split-K parts of the O projection and the shared-expert down GEMM

inline size_t up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }
inline int up8(int x) { return (x + 7) / 8 * 8; }
inline int act_bytes(const dg_model_desc& d) { return d.act_dtype == DG_BF16 ? 2 : 4; }
inline int w_kind(const dg_model_desc& d) {
  if (d.expert_act_fp8) return W_FP8A8;
  return d.expert_dtype == DG_FP8E4M3 ? W_FP8 : d.expert_dtype == DG_MXFP4 ? W_MXFP4
                                      : d.expert_dtype == DG_BF16 ? W_BF16 : W_F32;
}
inline bool is_global(const dg_model_desc& d, int l) {
  return d.window <= 0 || d.global_every <= 0 || (l + 1) % d.global_every == 0;
}

int sampler_slices(const dg_model_desc& d, int rows, int* v_per_slice) {
  // one block per (slice, row tile), about one block per CU: each block streams its slice's
  // vocabulary tiles through one continuous ring
  const int bn = d.act_dtype == DG_BF16 ? SAMPLER_BN_BF16 : SAMPLER_BN_F32;
  const int bm = d.act_dtype == DG_BF16 ? SAMPLER_BM_BF16 : SAMPLER_BM_F32;
  const int n_mt = (rows + bm - 1) / bm;
  const int tiles = (d.vocab + bn - 1) / bn;
  int want = (256 + n_mt - 1) / n_mt;
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  const int tiles_per = (tiles + want - 1) / want;
  *v_per_slice = tiles_per * bn;
  return (d.vocab + *v_per_slice - 1) / *v_per_slice;
}

// split-K parts of the self-conditioning product p_hat_0 . E (K = the vocabulary): a power of two
// up to 32 that divides the K tiles and keeps the block count near 512
int sc_splits(const dg_model_desc& d, int R) {
  const int kt = d.act_dtype == DG_BF16 ? 64 : 32;
  const int ktiles = d.vocab / kt;
  const int blocks = ((R + 255) / 256) * ((d.d_model + 255) / 256);
  int s = 1;
  while (s < 32 && ktiles % (2 * s) == 0 && blocks * 2 * s <= 512) s *= 2;
  return s;
}

// Workspace layout.  The inspectable regions (status, stats, routing) come first and depend only
// on the row count, so the test hooks can find them from `rows` alone.
struct Layout {
  size_t status, stats, rlogits, idx, gates;
  size_t resid, xhat, rope, q, kn, vn, attn_o, part_o, part_ml, rparts, o_parts, sh_parts;
  size_t counts, offsets, perm, inv_perm, tok, work, n_items;
  size_t a_grp, y, sh_a, samp_part, hidden, done, n_locked, prev, lockbuf, all_done;
  size_t seq_state, seq_rng, seq_flags, lam_table;
  size_t sc_p, sc_ptile, sc_parts, sc_x, sc_a, sc_state;   // self-conditioning (sc_hidden > 0)
  size_t q_x, q_xs, q_a, q_as, q_sh, q_shs;                // W8A8: e4m3 codes and row scales of the expert inputs
  size_t total;
  int max_items;
};

Layout layout(const dg_model_desc& d, int B, int n, int max_prefix) {
  Layout w{};
  const size_t R = (size_t)B * n, ab = act_bytes(d);
  const size_t Rk = R * d.top_k;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o += up(bytes); return at; };
  w.status = take(256);
  w.stats = take(R * STAT_FIELDS * 4);
  w.rlogits = take(R * d.n_experts * 4);
  w.idx = take(Rk * 4);
  w.gates = take(Rk * 4);
  w.resid = take(R * d.d_model * 4);
  w.xhat = take(R * d.d_model * ab);
  w.rope = take(R * (d.head_dim / 2) * 8);
  w.q = take(R * d.n_q_heads * d.head_dim * ab);
  w.kn = take(R * d.n_kv_heads * d.head_dim * ab);
  w.vn = take((size_t)B * up8(n) * d.n_kv_heads * d.head_dim * ab);
  w.attn_o = take(R * d.n_q_heads * d.head_dim * ab);
  (void)max_prefix;
  w.part_o = take((size_t)MAX_SPLITS * R * d.n_q_heads * d.head_dim * 4);
  w.part_ml = take((size_t)MAX_SPLITS * R * d.n_q_heads * 2 * 4);
  w.rparts = take((size_t)MAX_RSPLIT * R * d.n_experts * 4);
  w.o_parts = take((size_t)MAX_KSPLIT * R * d.d_model * 4);
  w.sh_parts = take(R * d.d_model * ab);     // shared-expert output rows (activation type)
  w.counts = take(d.n_experts * 4);
  w.offsets = take(d.n_experts * 4);
  w.perm = take(Rk * 4);
  w.inv_perm = take(Rk * 4);
  w.tok = take(Rk * 4);
  w.max_items = (int)((Rk + GROUP_BM - 1) / GROUP_BM) + d.n_experts;
  w.work = take((size_t)w.max_items * 2 * 4);
  w.n_items = take(4);
  w.a_grp = take(Rk * d.expert_hidden * ab);
  w.y = take(Rk * d.d_model * ab);           // routed expert output rows (activation type)
  w.sh_a = take(R * d.shared_hidden * ab);
  int vps;
  const int slices = sampler_slices(d, (int)R, &vps);
  w.samp_part = take((size_t)((slices + 7) / 8 * 8) * R * SAMPLER_PART * 4);
  w.hidden = take(R * d.d_model * ab);
  w.done = take(B * 4);
  w.n_locked = take(B * 4);
  w.prev = take(R * 4);
  w.lockbuf = take(R);
  w.all_done = take(4);
  w.seq_state = take((size_t)B * 16);
  w.seq_rng = take((size_t)B * 16);
  w.seq_flags = take((size_t)B * 12);     // append, skip, finished
  w.lam_table = take(256 * 4);
  if (d.sc_hidden > 0) {
    const int bn = sampler_bn(d.act_dtype == DG_BF16);
    w.sc_p = take(R * d.vocab * ab);
    w.sc_ptile = take(R * ((d.vocab + bn - 1) / bn) * 4);
    w.sc_parts = take((size_t)sc_splits(d, (int)R) * R * d.d_model * 4);
    w.sc_x = take(R * d.d_model * ab);
    w.sc_a = take(R * d.sc_hidden * ab);
    w.sc_state = take(R * d.d_model * 4);
  }
  if (d.expert_act_fp8) {
    w.q_x = take(R * d.d_model);
    w.q_xs = take(R * 4);
    w.q_a = take(Rk * d.expert_hidden);
    w.q_as = take(Rk * 4);
    w.q_sh = take(R * d.shared_hidden);
    w.q_shs = take(R * 4);
  }
  w.total = o;
  return w;
}

template <class T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

dg_status check_ws(const dg_ctx* c, void* ws, size_t ws_bytes, int B, int n, int max_prefix) {
  if (!ws) return fail(DG_EINVAL, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % ALIGN) return fail(DG_EWORKSPACE, "workspace not 256-byte aligned");
  const size_t need = layout(c->d, B, n, max_prefix).total;
  if (ws_bytes < need) return fail(DG_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  return DG_OK;
}

dg_status check_kv(const dg_ctx* c, const dg_kv* kv, int extra_tokens, int* max_prefix) {
  const dg_model_desc& d = c->d;
  if (!kv || !kv->k || !kv->v || !kv->cap || !kv->prefix_len) return fail(DG_EINVAL, "kv: NULL field");
  if (kv->batch < 1 || kv->batch > MAX_BATCH) return fail(DG_EUNSUPPORTED, "batch %d not in [1, %d]", kv->batch, MAX_BATCH);
  // the prefix lengths themselves live on the device: caches are validated against their host bound
  const int mp = kv->max_prefix;
  if (mp < 0) return fail(DG_EINVAL, "max_prefix %d < 0", mp);
  for (int l = 0; l < d.n_layers; ++l) {
    if (!kv->k[l] || !kv->v[l]) return fail(DG_EINVAL, "kv layer %d: NULL cache", l);
    if (kv->cap[l] % 8) return fail(DG_EUNSUPPORTED, "kv layer %d: cap %d not a multiple of 8", l, kv->cap[l]);
    if (is_global(d, l)) {
      if (kv->cap[l] < mp + extra_tokens)
        return fail(DG_EINVAL, "kv layer %d: cap %d < prefix %d + %d", l, kv->cap[l], mp, extra_tokens);
    } else if (kv->cap[l] != d.window) {
      return fail(DG_EINVAL, "kv layer %d (local): cap %d != window %d", l, kv->cap[l], d.window);
    }
  }
  *max_prefix = mp;
  return DG_OK;
}

uint32_t key0(uint64_t s) { return (uint32_t)(s & 0xffffffffu); }
uint32_t key1(uint64_t s) { return (uint32_t)(s >> 32); }

double kappa_of(dg_schedule sc, double t) {
  switch (sc) {
    case DG_KAPPA_LINEAR: return 1.0 - t;
    case DG_KAPPA_QUADRATIC: return 1.0 - t * t;
    case DG_KAPPA_COSINE: return std::cos(M_PI * t / 2.0);
  }
  return 0.0;
}
double kappa_rate(dg_schedule sc, double t) {
  switch (sc) {
    case DG_KAPPA_LINEAR: return 1.0;
    case DG_KAPPA_QUADRATIC: return 2.0 * t;
    case DG_KAPPA_COSINE: return (M_PI / 2.0) * std::sin(M_PI * t / 2.0);
  }
  return 0.0;
}

// lambda = min(1, h |kappa'(t)| / (1 - kappa(t))): the Euler jump probability of one Step
float jump_prob(dg_schedule sc, double t, double h) {
  const double den = 1.0 - kappa_of(sc, t);
  const double lam = den <= 0.0 ? 1.0 : std::fmin(1.0, h * kappa_rate(sc, t) / den);
  return (float)lam;
}

// Records an event pair around the launches issued while it lives, if `cls` is being profiled.
struct ProfScope {
  Prof* p;
  int cls;
  hipStream_t s;
  hipEvent_t e0 = nullptr;
  ProfScope(const dg_ctx* c, int cls_, hipStream_t s_) : p(c->prof), cls(cls_), s(s_) {
    if (p && (p->mask >> cls & 1u)) {
      e0 = p->get();
      (void)hipEventRecord(e0, s);
    }
  }
  void close() {
    if (e0) {
      hipEvent_t e1 = p->get();
      (void)hipEventRecord(e1, s);
      p->recs[cls].emplace_back(e0, e1);
      e0 = nullptr;
    }
  }
  ~ProfScope() { close(); }
};

// ---------------------------------------------------------------- the layer stack -------------
struct Pass {
  const dg_ctx* c;
  const dg_kv* kv;
  int B, n;            // canvases, rows per canvas
  int causal;          // prefill
  void* ws;
  Layout w;
  hipStream_t s;
  const int32_t* seq_causal = nullptr;   // mixed batch: device [B] per-canvas kind (1 = append)
};

// Block tiles the dense GEMM launcher picks for M rows with bf16 / fp32 weights (mirrors k_gemm.hip's
// dense_pick).
int dense_blocks(int M, int N) {
  int bm = M > 256 ? 256 : (M > 64 ? 128 : 64), bn = M > 256 ? 128 : 64;
  if (M > 64 && N <= 256) bm = 64, bn = 32;
  return ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
}

// split-K parts for the attention output projection: the largest divisor of the K-tile count (at
// most MAX_KSPLIT, at least two K tiles per part) that keeps the block count at or below 512, or
// at or below 256 (one 8-wave block per CU) for the 8-wave tiles above 64 rows (128 x 64 up to 256
// rows, 256 x 128 above)
int ksplit_for(const dg_model_desc& d, int M, int N, int K) {
  const int nk = K / (d.act_dtype == DG_BF16 ? 64 : 32);
  const int blocks = dense_blocks(M, N);
  const int cap = (M > 64 && N > 256) ? 256 : 512;
  int best = 1;
  for (int s = 1; s <= MAX_KSPLIT; ++s)
    if (nk % s == 0 && nk / s >= 2 && blocks * s <= cap) best = s;
  return best;
}

// split-K parts for the router GEMM (N = n_experts is narrow): a divisor of the K-tile count
// that brings the block count near 256
int router_splits(const dg_model_desc& d, int R) {
  const int kt = d.d_model / (d.act_dtype == DG_BF16 ? 64 : 32);
  const int tiles = dense_blocks(R, d.n_experts);
  int best = 1;
  for (int s = 1; s <= MAX_RSPLIT; ++s)
    if (kt % s == 0 && kt / s >= 2 && tiles * s <= 512) best = s;
  return best;
}

int attn_splits(const dg_model_desc& d, int B, int n, int nkeys) {
  const int qtiles = (d.n_q_heads / d.n_kv_heads * n + 63) / 64;
  const int base = B * d.n_kv_heads * qtiles;
  const int tiles = (nkeys + 63) / 64;
  int sp = (512 + base - 1) / base;
  if (sp > tiles / 2) sp = tiles / 2;
  if (sp > MAX_SPLITS) sp = MAX_SPLITS;
  if (sp < 1) sp = 1;
  return sp;
}

// bf16 attention: blocks of 128 query rows, one block per CU (LDS ring of 128 KB); key splits
// bring the block count near 256, each split keeping at least two 64-key tiles
int flash_splits(const dg_model_desc& d, int B, int n, int ntiles) {
  const int qb = (d.n_q_heads / d.n_kv_heads * n + FLASH_QROWS - 1) / FLASH_QROWS;
  const int base = B * d.n_kv_heads * qb;
  int sp = (256 + base - 1) / base;
  if (sp > ntiles / 2) sp = ntiles / 2;
  if (sp > MAX_SPLITS) sp = MAX_SPLITS;
  if (sp < 1) sp = 1;
  return sp;
}

// One decoder layer.  xhat_ready: the previous layer's combine already wrote RMSNorm(resid) *
// attn_norm into xhat.  next_g / next_out: the combine also writes RMSNorm(resid) * next_g
// (the next layer's attention norm or the final norm) into next_out.
dg_status run_layer(const Pass& P, int l, bool do_ffn, bool xhat_ready, const void* next_g, void* next_out) {
  const dg_model_desc& d = P.c->d;
  const dg_layer_weights& L = P.c->layers[l];
  const int bf = d.act_dtype == DG_BF16;
  const int R = P.B * P.n;
  void* ws = P.ws;
  const Layout& w = P.w;
  int* status = at<int>(ws, w.status);
  const bool glob = is_global(d, l);

  if (!xhat_ready)
    HIPCHK(launch_rmsnorm(at<float>(ws, w.resid), L.attn_norm, at<void>(ws, w.xhat), R, d.d_model, d.norm_eps, bf,
                          status, P.s));
  // QKV + RoPE
  DenseArgs qa{};
  qa.epi = EPI_QKV;
  qa.A = at<void>(ws, w.xhat); qa.lda = d.d_model;
  qa.B = L.w_qkv; qa.ldb = d.d_model;
  qa.M = R; qa.N = (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim; qa.K = d.d_model;
  qa.q_out = at<void>(ws, w.q); qa.k_out = at<void>(ws, w.kn); qa.v_out = at<void>(ws, w.vn);
  qa.Hq = d.n_q_heads; qa.Hkv = d.n_kv_heads; qa.dh = d.head_dim; qa.rows_per_canvas = P.n; qa.v_ld = up8(P.n);
  qa.rope = at<float2>(ws, w.rope);
  {
    ProfScope ps(P.c, DG_PROF_QKV, P.s);
    HIPCHK(launch_dense(qa, bf, bf ? W_BF16 : W_F32, P.s));
  }
  // attention
  AttnArgs aa{};
  aa.q = at<void>(ws, w.q); aa.kn = at<void>(ws, w.kn); aa.vn = at<void>(ws, w.vn);
  aa.kc = P.kv->k[l]; aa.vc = P.kv->v[l];
  aa.B = P.B; aa.n = P.n; aa.Hq = d.n_q_heads; aa.Hkv = d.n_kv_heads; aa.dh = d.head_dim; aa.cap = P.kv->cap[l];
  aa.vn_ld = up8(P.n);
  aa.causal = P.causal; aa.window = d.window > 0 ? d.window : 1; aa.is_global = glob;
  aa.seq_causal = P.seq_causal;
  aa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d.head_dim));
  aa.plen = P.kv->prefix_len;
  aa.max_prefix = P.kv->max_prefix;
  // grids are sized for the host bound on the prefixes; a split past a canvas's own key tiles
  // writes an empty partial (m = -inf, l = 0) that the merge skips
  const int np_max = glob ? aa.max_prefix : std::min(aa.max_prefix, d.window);
  const int maxkeys = np_max + P.n;
  const int maxtiles = (np_max + 63) / 64 + (P.n + 63) / 64;
  if (bf) {
    aa.splits = flash_splits(d, P.B, P.n, maxtiles);
    aa.tiles_per_split = (maxtiles + aa.splits - 1) / aa.splits;
    aa.splits = (maxtiles + aa.tiles_per_split - 1) / aa.tiles_per_split;
  } else {
    aa.splits = attn_splits(d, P.B, P.n, maxkeys);
    aa.keys_per_split = ((maxkeys + aa.splits - 1) / aa.splits + 63) / 64 * 64;
    aa.splits = (maxkeys + aa.keys_per_split - 1) / aa.keys_per_split;
  }
  aa.part_o = at<float>(ws, w.part_o); aa.part_ml = at<float>(ws, w.part_ml);
  aa.out = at<void>(ws, w.attn_o);
  {
    ProfScope ps(P.c, DG_PROF_ATTENTION, P.s);
    HIPCHK(launch_attention(aa, bf, P.s));
    if (aa.splits > 1) HIPCHK(launch_attn_merge(aa, bf, P.s));
  }
  if (P.causal || P.seq_causal) {
    HIPCHK(launch_kv_append(at<void>(ws, w.kn), at<void>(ws, w.vn), aa.vn_ld, P.kv->k[l], P.kv->v[l], P.B, P.n,
                            d.n_kv_heads, d.head_dim, P.kv->cap[l], d.window, glob, aa.plen, aa.max_prefix,
                            P.seq_causal, bf, P.s));
  }
  // O projection as split-K partials; the fused kernel adds them to the residual (in part order)
  // and applies the FFN RMSNorm
  DenseArgs oa{};
  oa.epi = EPI_STORE_F32;
  oa.A = at<void>(ws, w.attn_o); oa.lda = d.n_q_heads * d.head_dim;
  oa.B = L.w_o; oa.ldb = d.n_q_heads * d.head_dim;
  oa.M = R; oa.N = d.d_model; oa.K = d.n_q_heads * d.head_dim;
  oa.C = at<void>(ws, w.o_parts); oa.ldc = d.d_model;
  oa.ksplit = ksplit_for(d, R, d.d_model, oa.K);
  oa.c_split = (int64_t)R * d.d_model;
  {
    ProfScope ps(P.c, DG_PROF_O_PROJ, P.s);
    HIPCHK(launch_dense(oa, bf, bf ? W_BF16 : W_F32, P.s));
  }
  {
    ProfScope ps(P.c, DG_PROF_NORM_COMBINE, P.s);
    HIPCHK(launch_resid_add_rmsnorm(at<float>(ws, w.resid), at<float>(ws, w.o_parts), oa.ksplit, oa.c_split,
                                    L.ffn_norm, at<void>(ws, w.xhat), R, d.d_model, d.norm_eps, bf, status, P.s));
  }
  if (!do_ffn) return DG_OK;

  // FFN: router, top-k, grouping
  // router logits: split-K partials, summed in order (+ bias) by the top-k kernel
  DenseArgs ra{};
  ra.epi = EPI_STORE_F32;
  ra.A = at<void>(ws, w.xhat); ra.lda = d.d_model;
  ra.B = L.w_router; ra.ldb = d.d_model;
  ra.M = R; ra.N = d.n_experts; ra.K = d.d_model;
  ra.C = at<void>(ws, w.rparts); ra.ldc = d.n_experts;
  ra.ksplit = router_splits(d, R);
  ra.c_split = (int64_t)R * d.n_experts;
  ProfScope route_scope(P.c, DG_PROF_ROUTING, P.s);
  HIPCHK(launch_dense(ra, bf, bf ? W_BF16 : W_F32, P.s));
  HIPCHK(launch_router_topk(at<float>(ws, w.rparts), ra.ksplit, ra.c_split, L.router_bias, R, d.n_experts, d.top_k,
                            at<float>(ws, w.rlogits), at<int32_t>(ws, w.idx), at<float>(ws, w.gates), P.s));
  const int wk = w_kind(d);
  const bool q8 = wk == W_FP8A8;
  int gbm = group_bm((int64_t)R * d.top_k, d.n_experts);
  if (q8 && gbm == GROUP_BM) gbm = GROUP_BM_Q8;
  // tiles the grouped launches may see: the workspace's bound is for GROUP_BM-row tiles
  const int max_items = gbm == GROUP_BM ? w.max_items : (R * d.top_k + gbm - 1) / gbm + d.n_experts;
  HIPCHK(launch_route_tables(at<int32_t>(ws, w.idx), R, d.n_experts, d.top_k, at<int32_t>(ws, w.counts),
                             at<int32_t>(ws, w.offsets), at<int32_t>(ws, w.perm), at<int32_t>(ws, w.inv_perm),
                             at<int32_t>(ws, w.tok), at<int32_t>(ws, w.work), at<int32_t>(ws, w.n_items),
                             gbm, P.s));
  route_scope.close();
  // routed experts and the shared expert in one launch each: gate/up + SwiGLU, then down
  GroupedArgs ga{};
  ga.epi = EPI_SWIGLU;
  ga.A = at<void>(ws, w.xhat); ga.lda = d.d_model; ga.a_tok = at<int32_t>(ws, w.tok);
  // storage units per weight row: MXFP4 packs two codes per byte and has one scale byte per 32
  // elements; fp8 has one bf16 scale per row
  const bool mx = wk == W_MXFP4;
  const int pk = mx ? 2 : 1;
  ga.B = L.w_gate; ga.B2 = L.w_up; ga.ldb = d.d_model / pk;
  ga.b_estride = (int64_t)d.expert_hidden * d.d_model / pk;
  ga.sB = L.s_gate; ga.sB2 = L.s_up; ga.s_ld = mx ? d.d_model / 32 : 2;
  ga.s_estride = (int64_t)d.expert_hidden * ga.s_ld;
  ga.N = d.expert_hidden; ga.K = d.d_model;
  ga.work = at<int32_t>(ws, w.work); ga.n_items = at<int32_t>(ws, w.n_items); ga.bm = gbm;
  ga.offsets = at<int32_t>(ws, w.offsets); ga.counts = at<int32_t>(ws, w.counts);
  ga.C = at<void>(ws, w.a_grp); ga.ldc = d.expert_hidden;
  ga.shA = at<void>(ws, w.xhat); ga.sh_lda = d.d_model;
  ga.shB = L.sh_gate; ga.shB2 = L.sh_up; ga.sh_ldb = d.d_model / pk;
  ga.sh_sB = L.sh_s_gate; ga.sh_sB2 = L.sh_s_up; ga.sh_s_ld = ga.s_ld;
  ga.shN = d.shared_hidden; ga.shK = d.d_model; ga.sh_rows = R;
  ga.shC = at<void>(ws, w.sh_a); ga.sh_ldc = d.shared_hidden;
  {
    ProfScope ps(P.c, DG_PROF_MOE_GATE_UP, P.s);
    if (q8) {
      // W8A8: the normalised rows as e4m3 codes with a float32 scale per row, for both expert kinds
      HIPCHK(launch_quant_rows(at<void>(ws, w.xhat), d.d_model, R, d.d_model, at<uint8_t>(ws, w.q_x),
                               at<float>(ws, w.q_xs), P.s));
      ga.A = ga.shA = at<void>(ws, w.q_x);
      ga.sA = ga.sh_sA = at<float>(ws, w.q_xs);
    }
    HIPCHK(launch_grouped(ga, bf, wk, max_items, P.s));
  }
  GroupedArgs da{};
  da.epi = EPI_STORE_ACT;           // expert outputs in the activation type
  da.A = at<void>(ws, w.a_grp); da.lda = d.expert_hidden; da.a_tok = nullptr;
  da.B = L.w_down; da.B2 = nullptr; da.ldb = d.expert_hidden / pk;
  da.b_estride = (int64_t)d.d_model * d.expert_hidden / pk;
  da.sB = L.s_down; da.sB2 = nullptr; da.s_ld = mx ? d.expert_hidden / 32 : 2;
  da.s_estride = (int64_t)d.d_model * da.s_ld;
  da.N = d.d_model; da.K = d.expert_hidden;
  da.work = ga.work; da.n_items = ga.n_items; da.offsets = ga.offsets; da.counts = ga.counts; da.bm = gbm;
  da.C = at<void>(ws, w.y); da.ldc = d.d_model;
  da.shA = at<void>(ws, w.sh_a); da.sh_lda = d.shared_hidden;
  da.shB = L.sh_down; da.shB2 = nullptr; da.sh_ldb = d.shared_hidden / pk;
  da.sh_sB = L.sh_s_down; da.sh_sB2 = nullptr; da.sh_s_ld = mx ? d.shared_hidden / 32 : 2;
  da.shN = d.d_model; da.shK = d.shared_hidden; da.sh_rows = R;
  da.shC = at<void>(ws, w.sh_parts); da.sh_ldc = d.d_model;
  {
    ProfScope ps(P.c, DG_PROF_MOE_DOWN, P.s);
    if (q8) {
      // the SwiGLU products (stored bf16) coded per row: routed rows in grouped order, shared rows in order
      HIPCHK(launch_quant_rows(at<void>(ws, w.a_grp), d.expert_hidden, R * d.top_k, d.expert_hidden,
                               at<uint8_t>(ws, w.q_a), at<float>(ws, w.q_as), P.s));
      HIPCHK(launch_quant_rows(at<void>(ws, w.sh_a), d.shared_hidden, R, d.shared_hidden, at<uint8_t>(ws, w.q_sh),
                               at<float>(ws, w.q_shs), P.s));
      da.A = at<void>(ws, w.q_a); da.sA = at<float>(ws, w.q_as);
      da.shA = at<void>(ws, w.q_sh); da.sh_sA = at<float>(ws, w.q_shs);
    }
    HIPCHK(launch_grouped(da, bf, wk, max_items, P.s));
  }
  {
    ProfScope ps(P.c, DG_PROF_NORM_COMBINE, P.s);
    HIPCHK(launch_moe_combine_norm(at<float>(ws, w.resid), at<void>(ws, w.y), at<void>(ws, w.sh_parts),
                                   at<float>(ws, w.gates), at<int32_t>(ws, w.inv_perm), R, d.d_model, d.top_k, next_g,
                                   next_out, d.norm_eps, bf, status, P.s));
  }
  return DG_OK;
}

dg_status check_desc(const dg_model_desc& d) {
  if (d.n_layers < 1 || d.d_model < 1 || d.n_q_heads < 1 || d.n_kv_heads < 1 || d.n_experts < 1 || d.top_k < 1 ||
      d.expert_hidden < 1 || d.shared_hidden < 1 || d.vocab < 1)
    return fail(DG_EINVAL, "model descriptor has a non-positive size");
  if (d.head_dim != 64 && d.head_dim != 128 && d.head_dim != 256)
    return fail(DG_EUNSUPPORTED, "head_dim %d not in {64, 128, 256}", d.head_dim);
  if (d.n_q_heads % d.n_kv_heads) return fail(DG_EUNSUPPORTED, "n_q_heads %% n_kv_heads != 0");
  if (d.d_model % 64 || d.expert_hidden % 64 || d.shared_hidden % 64)
    return fail(DG_EUNSUPPORTED, "d_model, expert_hidden and shared_hidden must be multiples of 64");
  if (d.d_model > 4096) return fail(DG_EUNSUPPORTED, "d_model %d > 4096", d.d_model);
  if (d.vocab % 16) return fail(DG_EUNSUPPORTED, "vocab %% 16 != 0");
  if (d.sc_hidden < 0 || d.sc_hidden % 64) return fail(DG_EUNSUPPORTED, "sc_hidden %d not a multiple of 64", d.sc_hidden);
  if (d.sc_hidden > 0 && d.vocab % 64) return fail(DG_EUNSUPPORTED, "self-conditioning needs vocab %% 64 == 0");
  if (d.n_experts > 256 || d.n_experts % 4 || d.top_k > 16 || d.top_k > d.n_experts)
    return fail(DG_EUNSUPPORTED, "need top_k <= 16, top_k <= n_experts <= 256 and n_experts %% 4 == 0");
  if (d.act_dtype != DG_F32 && d.act_dtype != DG_BF16) return fail(DG_EUNSUPPORTED, "act_dtype must be F32 or BF16");
  if (!(d.expert_dtype == d.act_dtype ||
        (d.act_dtype == DG_BF16 && (d.expert_dtype == DG_FP8E4M3 || d.expert_dtype == DG_MXFP4))))
    return fail(DG_EUNSUPPORTED, "expert_dtype must equal act_dtype, or be FP8E4M3 / MXFP4 with BF16 activations");
  if (d.expert_act_fp8 != 0 && d.expert_act_fp8 != 1) return fail(DG_EINVAL, "expert_act_fp8 must be 0 or 1");
  if (d.expert_act_fp8 && !(d.expert_dtype == DG_FP8E4M3 && d.act_dtype == DG_BF16))
    return fail(DG_EUNSUPPORTED, "expert_act_fp8 needs FP8E4M3 expert weights and BF16 activations");
  if (d.expert_act_fp8 && (d.expert_hidden > 4096 || d.shared_hidden > 4096))
    return fail(DG_EUNSUPPORTED, "expert_act_fp8 needs expert_hidden and shared_hidden <= 4096");
  if (!(d.norm_eps >= 0.f) || !(d.rope_theta > 0.f)) return fail(DG_EINVAL, "bad norm_eps or rope_theta");
  if (d.window > 0 && d.global_every > 0 && d.window < 1) return fail(DG_EINVAL, "bad window");
  return DG_OK;
}

dg_status check_rows(int B, int L) {
  if (B < 1 || B > MAX_BATCH) return fail(DG_EUNSUPPORTED, "batch %d not in [1, %d]", B, MAX_BATCH);
  if (L < 16 || L > 1024 || L % 16) return fail(DG_EUNSUPPORTED, "canvas length %d: need 16 <= L <= 1024, L %% 16 == 0", L);
  return DG_OK;
}

// Where the fused sampler and the Step keep their scratch: the status word, per-row statistics and
// the per-(slice, row) partials.
struct SampScratch {
  int* status;
  float* stats;
  float* part;
};
SampScratch samp_scratch(void* ws, const Layout& w) {
  return {at<int>(ws, w.status), at<float>(ws, w.stats), at<float>(ws, w.samp_part)};
}

// The self-conditioning signal s = FFW(p_hat_0 . E) of R rows [TR §디노이징 반복과 self-conditioning],
// once the fused sampler has written the tile-relative probabilities and the merge the statistics:
// p_hat_0 in place, the split-K product with E (through its transpose, K-contiguous), the parts
// summed in order into the block's input, then the gated feed-forward block into sc_out (fp32).
dg_status self_cond_into(const dg_ctx* c, int R, void* ws, const Layout& w, float* sc_out, hipStream_t s) {
  ProfScope ps(c, DG_PROF_SELF_COND, s);
  const dg_model_desc& d = c->d;
  const int bf = d.act_dtype == DG_BF16;
  const int bn = sampler_bn(bf);
  HIPCHK(launch_p_rescale(at<void>(ws, w.sc_p), at<float>(ws, w.sc_ptile), at<float>(ws, w.stats), R, d.vocab, bn,
                          (d.vocab + bn - 1) / bn, bf, s));
  DenseArgs pe{};
  pe.epi = EPI_STORE_F32;
  pe.A = at<void>(ws, w.sc_p); pe.lda = d.vocab;
  pe.B = c->embed_t; pe.ldb = d.vocab;
  pe.M = R; pe.N = d.d_model; pe.K = d.vocab;
  pe.C = at<void>(ws, w.sc_parts); pe.ldc = d.d_model;
  pe.ksplit = sc_splits(d, R);
  pe.c_split = (int64_t)R * d.d_model;
  HIPCHK(launch_dense(pe, bf, bf ? W_BF16 : W_F32, s));
  HIPCHK(launch_sum_parts_cast(at<float>(ws, w.sc_parts), pe.ksplit, pe.c_split, at<void>(ws, w.sc_x),
                               (int64_t)R * d.d_model, bf, s));
  DenseArgs g{};
  g.epi = EPI_SWIGLU;
  g.A = at<void>(ws, w.sc_x); g.lda = d.d_model;
  g.B = c->sc_gate; g.B2 = c->sc_up; g.ldb = d.d_model;
  g.M = R; g.N = d.sc_hidden; g.K = d.d_model;
  g.C = at<void>(ws, w.sc_a); g.ldc = d.sc_hidden;
  HIPCHK(launch_dense(g, bf, bf ? W_BF16 : W_F32, s));
  DenseArgs dn{};
  dn.epi = EPI_STORE_F32;
  dn.A = at<void>(ws, w.sc_a); dn.lda = d.sc_hidden;
  dn.B = c->sc_down; dn.ldb = d.sc_hidden;
  dn.M = R; dn.N = d.d_model; dn.K = d.sc_hidden;
  dn.C = sc_out; dn.ldc = d.d_model; dn.ksplit = 1; dn.c_split = 0;
  HIPCHK(launch_dense(dn, bf, bf ? W_BF16 : W_F32, s));
  return DG_OK;
}

// sampler arguments shared by the Euler and the entropy-bounded steps; with sc the probabilities
// are also written for the self-conditioning product
void samp_sc_args(const dg_ctx* c, SampArgs& sa, void* ws, const Layout& w, bool sc) {
  if (!sc) return;
  const int bn = sampler_bn(c->d.act_dtype == DG_BF16);
  sa.pmat = at<void>(ws, w.sc_p);
  sa.ptile = at<float>(ws, w.sc_ptile);
  sa.n_vtiles = (c->d.vocab + bn - 1) / bn;
}

dg_status sample_into(dg_ctx* c, const void* hidden, int32_t* canvas, uint8_t* lock, int32_t* n_locked,
                      const int32_t* done, int B, int L, const dg_step_params* p, float lam, const SampScratch& sc,
                      int32_t* steps_taken, int32_t* done_out, hipStream_t s,
                      const uint32_t* canvas_rng = nullptr, const float* lam_table = nullptr,
                      float* sc_out = nullptr, void* ws = nullptr, const Layout* w = nullptr) {
  const dg_model_desc& d = c->d;
  const int R = B * L;
  SampArgs sa{};
  if (sc_out) samp_sc_args(c, sa, ws, *w, true);
  sa.H = hidden; sa.E = c->embed;
  sa.rows = R; sa.d = d.d_model; sa.V = d.vocab; sa.L = L;
  sa.zscale_log2 = (float)(1.4426950408889634 / (double)p->tau);
  sa.k0 = key0(p->seed); sa.k1 = key1(p->seed); sa.step = p->step;
  sa.slices = sampler_slices(d, R, &sa.v_per_slice);
  sa.part = sc.part;
  sa.canvas_rng = canvas_rng;
  {
    ProfScope ps(c, DG_PROF_SAMPLER, s);
    HIPCHK(launch_lmhead_sampler(sa, d.act_dtype == DG_BF16, s));
  }
  StepArgs st{};
  st.part = sa.part; st.slices = sa.slices;
  st.B = B; st.L = L; st.canvas = canvas; st.lock = lock; st.n_locked = n_locked; st.done = done;
  st.lam = lam; st.theta = p->lock_threshold;
  st.k0 = sa.k0; st.k1 = sa.k1; st.step = p->step;
  st.stats = sc.stats; st.status = sc.status;
  st.steps_taken = steps_taken; st.done_out = done_out;
  st.canvas_rng = canvas_rng; st.lam_table = lam_table;
  {
    ProfScope ps(c, DG_PROF_STEP, s);
    HIPCHK(launch_step_merge(st, s));
  }
  if (sc_out) return self_cond_into(c, R, ws, *w, sc_out, s);
  return DG_OK;
}

dg_status check_eb_params(const dg_eb_params* p) {
  if (!p) return fail(DG_EINVAL, "params is NULL");
  if (!(p->t > 0.f) || p->t > 1.f) return fail(DG_EINVAL, "need 0 < t <= 1");
  if (!(p->tau_start > 0.f) || !(p->tau_end > 0.f) || !std::isfinite(p->tau_start) || !std::isfinite(p->tau_end))
    return fail(DG_EINVAL, "temperatures must be > 0");
  if (!(p->gamma >= 0.f) || !(p->stop_entropy >= 0.f)) return fail(DG_EINVAL, "gamma and stop_entropy must be >= 0");
  return DG_OK;
}

// tau_t = tau_end + (tau_start - tau_end) t, in double, as a float
float eb_tau(const dg_eb_params* p) {
  return (float)((double)p->tau_end + ((double)p->tau_start - (double)p->tau_end) * (double)p->t);
}

EbArgs eb_args(const dg_ctx* c, int32_t* canvas, int32_t* prev, int32_t* done, int32_t* n_accepted,
               float* mean_entropy, int B, int L, const dg_eb_params* p, void* ws, const Layout& w,
               int32_t* steps_taken) {
  EbArgs e{};
  e.stats = at<float>(ws, w.stats);
  e.B = B; e.L = L; e.canvas = canvas; e.prev = prev; e.done = done;
  e.n_accepted = n_accepted; e.mean_entropy = mean_entropy; e.steps_taken = steps_taken;
  e.gamma = p->gamma; e.stop_entropy = p->stop_entropy;
  e.has_prev = p->has_prev != 0; e.final_step = p->final_step != 0; e.adaptive = p->adaptive != 0;
  e.vocab = c->d.vocab;
  e.k0 = key0(p->seed); e.k1 = key1(p->seed); e.step = p->step;
  return e;
}

// the entropy-bounded step: statistics of every row (from the fused LM head over `src` = hidden
// states, or from given logits), merged without touching the canvas, then the per-canvas selection
dg_status eb_into(dg_ctx* c, const void* src, bool from_logits, int32_t* canvas, int32_t* prev, int32_t* done,
                  int32_t* n_accepted, float* mean_entropy, int B, int L, const dg_eb_params* p, void* ws,
                  const Layout& w, int32_t* steps_taken, hipStream_t s, float* sc_out = nullptr) {
  const dg_model_desc& d = c->d;
  const int R = B * L;
  const uint32_t k0 = key0(p->seed), k1 = key1(p->seed);
  const float zs = (float)(1.4426950408889634 / (double)eb_tau(p));
  int vps;
  const int slices = sampler_slices(d, R, &vps);
  float* part = at<float>(ws, w.samp_part);
  {
    ProfScope ps(c, DG_PROF_SAMPLER, s);
    if (from_logits) {
      HIPCHK(launch_logits_partials(static_cast<const float*>(src), R, d.vocab, L, zs, k0, k1, p->step, slices, vps,
                                    part, s));
    } else {
      SampArgs sa{};
      sa.H = src; sa.E = c->embed;
      sa.rows = R; sa.d = d.d_model; sa.V = d.vocab; sa.L = L;
      sa.zscale_log2 = zs; sa.k0 = k0; sa.k1 = k1; sa.step = p->step;
      sa.slices = slices; sa.v_per_slice = vps; sa.part = part;
      samp_sc_args(c, sa, ws, w, sc_out != nullptr);
      HIPCHK(launch_lmhead_sampler(sa, d.act_dtype == DG_BF16, s));
    }
  }
  StepArgs st{};
  st.part = part; st.slices = slices; st.B = B; st.L = L;
  st.stats = at<float>(ws, w.stats); st.status = at<int>(ws, w.status); st.stats_only = 1;
  HIPCHK(launch_step_merge(st, s));
  if (sc_out && !from_logits) {
    const dg_status r = self_cond_into(c, R, ws, w, sc_out, s);
    if (r != DG_OK) return r;
  }
  HIPCHK(launch_eb_select(eb_args(c, canvas, prev, done, n_accepted, mean_entropy, B, L, p, ws, w, steps_taken), s));
  return DG_OK;
}

dg_status check_step_params(const dg_step_params* p) {
  if (!p) return fail(DG_EINVAL, "params is NULL");
  if (!(p->tau > 0.f) || !std::isfinite(p->tau)) return fail(DG_EINVAL, "tau must be > 0");
  if (!(p->h > 0.f) || !(p->t > 0.f) || p->t > 1.f) return fail(DG_EINVAL, "need 0 < t <= 1 and h > 0");
  if (p->schedule < DG_KAPPA_LINEAR || p->schedule > DG_KAPPA_COSINE) return fail(DG_EINVAL, "bad schedule");
  if (!(p->lock_threshold > 0.f)) return fail(DG_EINVAL, "lock_threshold must be > 0");
  return DG_OK;
}

}  // namespace

// ================================================================ C ABI ==========================
extern "C" {

const char* dg_last_error(void) { return g_err.c_str(); }

float dg_jump_prob(dg_schedule schedule, float t, float h) { return jump_prob(schedule, t, h); }

dg_status dg_create(const dg_model_desc* desc, const dg_weights* wts, dg_ctx** out) {
  g_err.clear();
  if (!desc || !wts || !out) return fail(DG_EINVAL, "NULL argument");
  dg_status st = check_desc(*desc);
  if (st != DG_OK) return st;
  if (!wts->layers || !wts->final_norm) return fail(DG_EINVAL, "weights: NULL layer table or final_norm");
  const bool fp8 = desc->expert_dtype == DG_FP8E4M3 || desc->expert_dtype == DG_MXFP4;
  for (int l = 0; l < desc->n_layers; ++l) {
    const dg_layer_weights& L = wts->layers[l];
    if (!L.attn_norm || !L.w_qkv || !L.w_o || !L.ffn_norm || !L.w_router || !L.w_gate || !L.w_up || !L.w_down ||
        !L.sh_gate || !L.sh_up || !L.sh_down)
      return fail(DG_EINVAL, "weights: layer %d has a NULL matrix", l);
    if (fp8 && (!L.s_gate || !L.s_up || !L.s_down || !L.sh_s_gate || !L.sh_s_up || !L.sh_s_down))
      return fail(DG_EINVAL, "weights: layer %d: FP8 / MXFP4 experts need every scale", l);
    const void* ptrs[] = {L.attn_norm, L.w_qkv, L.w_o, L.ffn_norm, L.w_router, L.router_bias, L.w_gate, L.w_up,
                          L.w_down, L.sh_gate, L.sh_up, L.sh_down};
    for (const void* q : ptrs)
      if ((uintptr_t)q & 15) return fail(DG_EINVAL, "weights: layer %d has a pointer that is not 16-byte aligned", l);
  }
  if (((uintptr_t)wts->final_norm & 15) || ((uintptr_t)wts->embed & 15))
    return fail(DG_EINVAL, "weights: embed / final_norm not 16-byte aligned");
  if (desc->sc_hidden > 0) {
    if (!wts->embed || !wts->embed_t || !wts->sc_gate || !wts->sc_up || !wts->sc_down)
      return fail(DG_EINVAL, "weights: self-conditioning needs embed, embed_t, sc_gate, sc_up and sc_down");
    if (((uintptr_t)wts->embed_t | (uintptr_t)wts->sc_gate | (uintptr_t)wts->sc_up | (uintptr_t)wts->sc_down) & 15)
      return fail(DG_EINVAL, "weights: self-conditioning matrices not 16-byte aligned");
  }
  dg_ctx* c = new dg_ctx;
  c->d = *desc;
  c->layers.assign(wts->layers, wts->layers + desc->n_layers);
  c->embed = wts->embed;
  c->final_norm = wts->final_norm;
  c->embed_t = wts->embed_t;
  c->sc_gate = wts->sc_gate; c->sc_up = wts->sc_up; c->sc_down = wts->sc_down;
  c->prof = new Prof;
  *out = c;
  return DG_OK;
}

void dg_destroy(dg_ctx* ctx) {
  if (!ctx) return;
  delete ctx->prof;
  delete ctx;
}

dg_status dg_profile_enable(dg_ctx* ctx, uint32_t mask) {
  if (!ctx) return fail(DG_EINVAL, "NULL context");
  ctx->prof->mask = mask;
  return DG_OK;
}

dg_status dg_profile_read(dg_ctx* ctx, int32_t cls, double* total_ms, int32_t* launches) {
  if (!ctx || cls < 0 || cls >= DG_PROF_N) return fail(DG_EINVAL, "bad argument");
  Prof* p = ctx->prof;
  double tot = 0.0;
  int n = 0;
  for (auto& pr : p->recs[cls]) {
    HIPCHK(hipEventSynchronize(pr.second));
    float ms = 0.f;
    HIPCHK(hipEventElapsedTime(&ms, pr.first, pr.second));
    tot += ms;
    ++n;
    p->pool.push_back(pr.first);
    p->pool.push_back(pr.second);
  }
  p->recs[cls].clear();
  if (total_ms) *total_ms = tot;
  if (launches) *launches = n;
  return DG_OK;
}

dg_status dg_init_canvas(int32_t* canvas, uint8_t* lock, int32_t batch, int32_t L, int32_t vocab, uint64_t seed,
                         hipStream_t stream) {
  g_err.clear();
  if (!canvas || batch < 1 || L < 1 || vocab < 1) return fail(DG_EINVAL, "bad argument");
  HIPCHK(launch_init_canvas(canvas, lock, batch, L, vocab, key0(seed), key1(seed), stream));
  return DG_OK;
}

size_t dg_workspace_bytes(const dg_ctx* ctx, int32_t batch, int32_t rows_per_canvas, int32_t max_prefix) {
  if (!ctx || batch < 1 || rows_per_canvas < 1) return 0;
  return layout(ctx->d, batch, rows_per_canvas, max_prefix).total;
}

dg_status dg_query_status(const dg_ctx* ctx, const void* ws, hipStream_t stream) {
  if (!ctx || !ws) return fail(DG_EINVAL, "NULL argument");
  HIPCHK(hipStreamSynchronize(stream));
  int v = 0;
  HIPCHK(hipMemcpy(&v, ws, sizeof v, hipMemcpyDeviceToHost));
  if (v & 4) return fail(DG_EINVAL, "a device prefix_len was outside [0, max_prefix] (code %d)", v);
  return v ? fail(DG_ENONFINITE, "non-finite value flagged (code %d)", v) : DG_OK;
}

dg_status dg_clear_status(const dg_ctx* ctx, void* ws, hipStream_t stream) {
  if (!ctx || !ws) return fail(DG_EINVAL, "NULL argument");
  HIPCHK(launch_fill_i32(static_cast<int32_t*>(ws), 0, 64, stream));
  return DG_OK;
}

dg_status dg_prefill_kv(dg_ctx* ctx, const dg_kv* kv, const int32_t* tokens, int32_t n, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  g_err.clear();
  if (!ctx || !tokens) return fail(DG_EINVAL, "NULL argument");
  if (!ctx->embed) return fail(DG_EINVAL, "prefill needs the embedding");
  if (n < 1) return fail(DG_EINVAL, "n must be >= 1");
  int mp = 0;
  dg_status st = check_kv(ctx, kv, n, &mp);
  if (st != DG_OK) return st;
  if ((st = check_ws(ctx, ws, ws_bytes, kv->batch, n, mp)) != DG_OK) return st;
  Pass P{ctx, kv, kv->batch, n, 1, ws, layout(ctx->d, kv->batch, n, mp), stream};
  const dg_model_desc& d = ctx->d;
  HIPCHK(launch_embed(tokens, ctx->embed, at<float>(ws, P.w.resid), P.B * n, d.d_model, d.vocab,
                      d.act_dtype == DG_BF16, stream));
  HIPCHK(launch_rope_table(at<float2>(ws, P.w.rope), P.B * n, n, d.head_dim, std::log2((double)d.rope_theta),
                           kv->prefix_len, kv->max_prefix, at<int>(ws, P.w.status), stream));
  for (int l = 0; l < d.n_layers; ++l) {
    // the last layer's FFN feeds no cache; each combine writes the next layer's normalised rows
    const bool more = l + 1 < d.n_layers;
    if ((st = run_layer(P, l, more, l > 0, more ? ctx->layers[l + 1].attn_norm : nullptr,
                        at<void>(ws, P.w.xhat))) != DG_OK)
      return st;
  }
  HIPCHK(launch_advance_prefix(kv->prefix_len, P.B, n, nullptr, stream));
  return DG_OK;
}

dg_status dg_denoise_step(dg_ctx* ctx, const dg_kv* kv, const int32_t* canvas, const float* resid_in,
                          const float* sc_in, int32_t L, int32_t layer_begin, int32_t layer_end, void* hidden_out,
                          float* resid_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err.clear();
  if (!ctx) return fail(DG_EINVAL, "NULL context");
  const dg_model_desc& d = ctx->d;
  if (!canvas && !resid_in) return fail(DG_EINVAL, "need canvas or resid_in");
  if (sc_in && (resid_in || layer_begin != 0))
    return fail(DG_EINVAL, "sc_in is added to the embedded canvas: no resid_in, layer_begin 0");
  if (!resid_in && !ctx->embed) return fail(DG_EINVAL, "embedding canvas tokens needs the embedding");
  if (layer_begin < 0 || layer_end > d.n_layers || layer_begin > layer_end)
    return fail(DG_EINVAL, "layer range [%d, %d) outside [0, %d]", layer_begin, layer_end, d.n_layers);
  int mp = 0;
  dg_status st = check_kv(ctx, kv, 0, &mp);
  if (st != DG_OK) return st;
  if ((st = check_rows(kv->batch, L)) != DG_OK) return st;
  if ((st = check_ws(ctx, ws, ws_bytes, kv->batch, L, mp)) != DG_OK) return st;
  Pass P{ctx, kv, kv->batch, L, 0, ws, layout(d, kv->batch, L, mp), stream};
  const int R = P.B * L;
  const int bf = d.act_dtype == DG_BF16;
  {
    ProfScope ps(ctx, DG_PROF_EMBED, stream);
    if (resid_in) HIPCHK(launch_copy_f32(resid_in, at<float>(ws, P.w.resid), (int64_t)R * d.d_model, stream));
    else HIPCHK(launch_embed(canvas, ctx->embed, at<float>(ws, P.w.resid), R, d.d_model, d.vocab, bf, stream, sc_in));
    HIPCHK(launch_rope_table(at<float2>(ws, P.w.rope), R, L, d.head_dim, std::log2((double)d.rope_theta),
                             kv->prefix_len, kv->max_prefix, at<int>(ws, P.w.status), stream));
  }
  // each layer's combine writes the next layer's normalised rows, the last one the final norm
  for (int l = layer_begin; l < layer_end; ++l) {
    const bool last = l + 1 == layer_end;
    const void* ng = last ? (hidden_out ? ctx->final_norm : nullptr) : ctx->layers[l + 1].attn_norm;
    void* no = last ? hidden_out : at<void>(ws, P.w.xhat);
    if ((st = run_layer(P, l, true, l > layer_begin, ng, no)) != DG_OK) return st;
  }
  if (resid_out) HIPCHK(launch_copy_f32(at<float>(ws, P.w.resid), resid_out, (int64_t)R * d.d_model, stream));
  if (hidden_out && layer_begin == layer_end)
    HIPCHK(launch_rmsnorm(at<float>(ws, P.w.resid), ctx->final_norm, hidden_out, R, d.d_model, d.norm_eps, bf,
                          at<int>(ws, P.w.status), stream));
  return DG_OK;
}

// one mixed pass (arguments already validated): append canvases take the causal encoder pass and
// advance their device prefix length, the others the bidirectional decoder pass
dg_status mixed_pass(dg_ctx* ctx, const dg_kv* kv, const int32_t* tokens, const int32_t* append, int L,
                     void* hidden_out, float* resid_out, void* ws, const Layout& w, hipStream_t stream,
                     const float* sc_in = nullptr) {
  const dg_model_desc& d = ctx->d;
  Pass P{ctx, kv, kv->batch, L, 0, ws, w, stream, append};
  const int R = P.B * L;
  HIPCHK(launch_embed(tokens, ctx->embed, at<float>(ws, P.w.resid), R, d.d_model, d.vocab, d.act_dtype == DG_BF16,
                      stream, sc_in));
  HIPCHK(launch_rope_table(at<float2>(ws, P.w.rope), R, L, d.head_dim, std::log2((double)d.rope_theta),
                           kv->prefix_len, kv->max_prefix, at<int>(ws, P.w.status), stream));
  dg_status st;
  for (int l = 0; l < d.n_layers; ++l) {
    const bool last = l + 1 == d.n_layers;
    if ((st = run_layer(P, l, true, l > 0, last ? ctx->final_norm : ctx->layers[l + 1].attn_norm,
                        last ? hidden_out : at<void>(ws, P.w.xhat))) != DG_OK)
      return st;
  }
  if (resid_out) HIPCHK(launch_copy_f32(at<float>(ws, P.w.resid), resid_out, (int64_t)R * d.d_model, stream));
  HIPCHK(launch_advance_prefix(kv->prefix_len, P.B, L, append, stream));
  return DG_OK;
}

dg_status dg_mixed_forward(dg_ctx* ctx, const dg_kv* kv, const int32_t* tokens, const int32_t* append, int32_t L,
                           void* hidden_out, float* resid_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err.clear();
  if (!ctx || !tokens || !append || !hidden_out) return fail(DG_EINVAL, "NULL argument");
  if (!ctx->embed) return fail(DG_EINVAL, "embedding tokens needs the embedding");
  int mp = 0;
  // every canvas may be an append one: room for L more positions on the global layers
  dg_status st = check_kv(ctx, kv, L, &mp);
  if (st != DG_OK) return st;
  if ((st = check_rows(kv->batch, L)) != DG_OK) return st;
  if ((st = check_ws(ctx, ws, ws_bytes, kv->batch, L, mp)) != DG_OK) return st;
  return mixed_pass(ctx, kv, tokens, append, L, hidden_out, resid_out, ws, layout(ctx->d, kv->batch, L, mp), stream);
}

dg_status dg_step_sample(dg_ctx* ctx, const void* hidden, int32_t* canvas, uint8_t* lock, int32_t* n_locked,
                         const int32_t* done, float* sc_out, int32_t batch, int32_t L, const dg_step_params* params,
                         void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err.clear();
  if (!ctx || !hidden || !canvas || !lock) return fail(DG_EINVAL, "NULL argument");
  if (sc_out && ctx->d.sc_hidden <= 0) return fail(DG_EINVAL, "sc_out needs a model with a self-conditioning block");
  if (!ctx->embed) return fail(DG_EINVAL, "the LM head needs the embedding");
  dg_status st = check_step_params(params);
  if (st != DG_OK) return st;
  if ((st = check_rows(batch, L)) != DG_OK) return st;
  if ((st = check_ws(ctx, ws, ws_bytes, batch, L, 0)) != DG_OK) return st;
  const Layout w = layout(ctx->d, batch, L, 0);
  return sample_into(ctx, hidden, canvas, lock, n_locked, done, batch, L, params,
                     jump_prob(params->schedule, params->t, params->h), samp_scratch(ws, w), nullptr, nullptr,
                     stream, nullptr, nullptr, sc_out, ws, &w);
}

dg_status dg_step_sample_noalloc(dg_ctx* ctx, const void* hidden, int32_t* canvas, uint8_t* lock, int32_t* n_locked,
                                 const int32_t* done, int32_t batch, int32_t L, const dg_step_params* params,
                                 hipStream_t stream) {
  g_err.clear();
  if (!ctx || !hidden || !canvas || !lock) return fail(DG_EINVAL, "NULL argument");
  if (!ctx->embed) return fail(DG_EINVAL, "the LM head needs the embedding");
  dg_status st = check_step_params(params);
  if (st != DG_OK) return st;
  if ((st = check_rows(batch, L)) != DG_OK) return st;
  // the status word, the per-row statistics and the partials of every (vocabulary slice, row)
  const size_t R = (size_t)batch * L;
  int vps;
  const int slices = sampler_slices(ctx->d, (int)R, &vps);
  const size_t o_stats = up(256), o_part = o_stats + up(R * STAT_FIELDS * 4);
  const size_t need = o_part + up((size_t)slices * R * SAMPLER_PART * 4);
  if (need > STATIC_SCRATCH_BYTES)
    return fail(DG_EUNSUPPORTED, "%d x %d rows need %zu bytes of static scratch, more than its %zu; use dg_step_sample",
                batch, L, need, STATIC_SCRATCH_BYTES);
  void* base = nullptr;
  HIPCHK(static_scratch(&base));
  char* b = static_cast<char*>(base);
  const SampScratch sc{reinterpret_cast<int*>(b), reinterpret_cast<float*>(b + o_stats),
                       reinterpret_cast<float*>(b + o_part)};
  // the array keeps the previous call's contents: the status word starts from zero (a fill kernel);
  // statistics and partials are written in full before they are read
  HIPCHK(launch_fill_i32(sc.status, 0, 64, stream));
  return sample_into(ctx, hidden, canvas, lock, n_locked, done, batch, L, params,
                     jump_prob(params->schedule, params->t, params->h), sc, nullptr, nullptr, stream);
}

// dg_canvas_run with the entropy-bounded sampler
dg_status eb_run(dg_ctx* ctx, const dg_kv* kv, int32_t* canvas, uint8_t* lock, int32_t* steps_taken, int32_t L,
                 const dg_run_params* p, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ctx->embed) return fail(DG_EINVAL, "the canvas loop needs the embedding");
  if (p->max_steps < 1) return fail(DG_EINVAL, "max_steps must be >= 1");
  int mp = 0;
  dg_status st = check_kv(ctx, kv, 0, &mp);
  if (st != DG_OK) return st;
  if ((st = check_rows(kv->batch, L)) != DG_OK) return st;
  if ((st = check_ws(ctx, ws, ws_bytes, kv->batch, L, mp)) != DG_OK) return st;
  if (L > 1024) return fail(DG_EUNSUPPORTED, "entropy-bounded sampler: L %d > 1024", L);
  if (p->self_condition && ctx->d.sc_hidden <= 0) return fail(DG_EINVAL, "self_condition needs a self-conditioning block");
  dg_eb_params ep{};
  ep.t = 1.f; ep.tau_start = p->tau; ep.tau_end = p->tau_end; ep.gamma = p->gamma; ep.stop_entropy = p->stop_entropy;
  ep.seed = p->seed; ep.adaptive = p->adaptive != 0;
  if ((st = check_eb_params(&ep)) != DG_OK) return st;
  const Layout w = layout(ctx->d, kv->batch, L, mp);
  const int B = kv->batch;
  int32_t* done = at<int32_t>(ws, w.done);
  int32_t* all_done = at<int32_t>(ws, w.all_done);
  HIPCHK(launch_fill_i32(done, 0, B, stream));
  HIPCHK(launch_fill_i32(all_done, 0, 1, stream));
  if (steps_taken) HIPCHK(launch_fill_i32(steps_taken, 0, B, stream));
  if (p->init_canvas) HIPCHK(launch_init_canvas(canvas, lock, B, L, ctx->d.vocab, key0(p->seed), key1(p->seed), stream));
  const double h = 1.0 / p->max_steps;
  // every pass is enqueued up front; once all canvases have stopped, the gate turns the remaining
  // passes' kernels away at entry (adaptive mode)
  // self-conditioning: the signal of step s feeds the decoder of step s + 1 (none at step 0)
  float* sc = p->self_condition ? at<float>(ws, w.sc_state) : nullptr;
  GateScope gate(p->adaptive ? all_done : nullptr);
  for (int s = 0; s < p->max_steps; ++s) {
    if ((st = dg_denoise_step(ctx, kv, canvas, nullptr, s > 0 ? sc : nullptr, L, 0, ctx->d.n_layers,
                              at<void>(ws, w.hidden), nullptr, ws, ws_bytes, stream)) != DG_OK)
      return st;
    ep.t = (float)(1.0 - s * h);
    ep.step = (uint32_t)s;
    ep.has_prev = s > 0;
    ep.final_step = s == p->max_steps - 1;
    if ((st = eb_into(ctx, at<void>(ws, w.hidden), false, canvas, at<int32_t>(ws, w.prev), done, nullptr, nullptr,
                      B, L, &ep, ws, w, steps_taken, stream, s + 1 < p->max_steps ? sc : nullptr)) != DG_OK)
      return st;
    if (p->adaptive) HIPCHK(launch_all_set(done, B, all_done, stream));
  }
  return DG_OK;
}

dg_status dg_step_entropy_bounded(dg_ctx* ctx, const void* hidden, int32_t* canvas, int32_t* prev_argmax,
                                  int32_t* done, int32_t* n_accepted, float* mean_entropy, int32_t batch, int32_t L,
                                  const dg_eb_params* params, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err.clear();
  if (!ctx || !hidden || !canvas || !prev_argmax || !done) return fail(DG_EINVAL, "NULL argument");
  if (!ctx->embed) return fail(DG_EINVAL, "the LM head needs the embedding");
  dg_status st = check_eb_params(params);
  if (st != DG_OK) return st;
  if ((st = check_rows(batch, L)) != DG_OK) return st;
  if ((st = check_ws(ctx, ws, ws_bytes, batch, L, 0)) != DG_OK) return st;
  const Layout w = layout(ctx->d, batch, L, 0);
  return eb_into(ctx, hidden, false, canvas, prev_argmax, done, n_accepted, mean_entropy, batch, L, params, ws, w,
                 nullptr, stream);
}

dg_status dg_canvas_run(dg_ctx* ctx, const dg_kv* kv, int32_t* canvas, uint8_t* lock, int32_t* steps_taken, int32_t L,
                        const dg_run_params* p, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err.clear();
  if (!ctx || !canvas || !p) return fail(DG_EINVAL, "NULL argument");
  if (p->sampler != DG_SAMPLER_EULER && p->sampler != DG_SAMPLER_ENTROPY_BOUNDED)
    return fail(DG_EINVAL, "unknown sampler %d", (int)p->sampler);
  if (p->sampler == DG_SAMPLER_ENTROPY_BOUNDED) return eb_run(ctx, kv, canvas, lock, steps_taken, L, p, ws, ws_bytes,
                                                              stream);
  if (!lock) return fail(DG_EINVAL, "NULL argument");
  if (!ctx->embed) return fail(DG_EINVAL, "the canvas loop needs the embedding");
  if (p->max_steps < 1) return fail(DG_EINVAL, "max_steps must be >= 1");
  if (p->self_condition && ctx->d.sc_hidden <= 0) return fail(DG_EINVAL, "self_condition needs a self-conditioning block");
  int mp = 0;
  dg_status st = check_kv(ctx, kv, 0, &mp);
  if (st != DG_OK) return st;
  if ((st = check_rows(kv->batch, L)) != DG_OK) return st;
  if ((st = check_ws(ctx, ws, ws_bytes, kv->batch, L, mp)) != DG_OK) return st;
  dg_step_params sp{};
  sp.schedule = p->schedule; sp.tau = p->tau; sp.lock_threshold = p->lock_threshold; sp.seed = p->seed;
  sp.t = 1.f; sp.h = 1.f / p->max_steps;
  if ((st = check_step_params(&sp)) != DG_OK) return st;
  const Layout w = layout(ctx->d, kv->batch, L, mp);
  const int B = kv->batch;
  int32_t* done = at<int32_t>(ws, w.done);
  int32_t* all_done = at<int32_t>(ws, w.all_done);
  HIPCHK(launch_fill_i32(done, 0, B, stream));
  HIPCHK(launch_fill_i32(all_done, 0, 1, stream));
  if (steps_taken) HIPCHK(launch_fill_i32(steps_taken, 0, B, stream));
  if (p->init_canvas) HIPCHK(launch_init_canvas(canvas, lock, B, L, ctx->d.vocab, key0(p->seed), key1(p->seed), stream));
  const double h = 1.0 / p->max_steps;
  // every pass is enqueued up front (no host read of `done`); once all canvases have locked every
  // position, the gate turns the remaining passes' kernels away at entry (adaptive mode)
  // self-conditioning: the signal of step s feeds the decoder of step s + 1 (none at step 0)
  float* sc = p->self_condition ? at<float>(ws, w.sc_state) : nullptr;
  GateScope gate(p->adaptive ? all_done : nullptr);
  for (int s = 0; s < p->max_steps; ++s) {
    if ((st = dg_denoise_step(ctx, kv, canvas, nullptr, s > 0 ? sc : nullptr, L, 0, ctx->d.n_layers,
                              at<void>(ws, w.hidden), nullptr, ws, ws_bytes, stream)) != DG_OK)
      return st;
    const double t = 1.0 - s * h;
    sp.t = (float)t;
    sp.h = (float)h;
    sp.step = (uint32_t)s;
    // the jump probability is taken at the double-precision grid point t_s = 1 - s/T
    if ((st = sample_into(ctx, at<void>(ws, w.hidden), canvas, lock, at<int32_t>(ws, w.n_locked),
                          p->adaptive ? done : nullptr, B, L, &sp, jump_prob(p->schedule, t, h), samp_scratch(ws, w),
                          steps_taken, p->adaptive ? done : nullptr, stream, nullptr, nullptr,
                          s + 1 < p->max_steps ? sc : nullptr, ws, &w)) != DG_OK)
      return st;
    if (p->adaptive) HIPCHK(launch_all_set(done, B, all_done, stream));
  }
  return DG_OK;
}

dg_status dg_generate(dg_ctx* ctx, const dg_kv* kv, int32_t* out, int32_t* steps, int32_t* valid, int32_t* eos_seen,
                      int32_t K, int32_t L, int32_t eos_id, const dg_run_params* params, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  g_err.clear();
  if (!ctx || !kv || !out || !params || !kv->prefix_len) return fail(DG_EINVAL, "NULL argument");
  if (K < 1) return fail(DG_EINVAL, "K must be >= 1");
  const int B = kv->batch;
  if (B < 1 || B > MAX_BATCH) return fail(DG_EUNSUPPORTED, "batch %d not in [1, %d]", B, MAX_BATCH);
  // room for the appended canvases: checked up front so nothing is enqueued on failure
  dg_kv last = *kv;
  last.max_prefix = kv->max_prefix + (K - 1) * L;
  int mp = 0;
  dg_status st = check_kv(ctx, &last, 0, &mp);
  if (st != DG_OK) return st;
  if ((st = check_ws(ctx, ws, ws_bytes, B, L, mp)) != DG_OK) return st;
  const Layout w = layout(ctx->d, B, L, mp);
  uint8_t* lock = at<uint8_t>(ws, w.lockbuf);
  for (int k = 0; k < K; ++k) {
    // the device prefix lengths grow by L per appended canvas; the host bound follows
    dg_kv cur = *kv;
    cur.max_prefix = kv->max_prefix + k * L;
    dg_run_params p = *params;
    p.seed = params->seed + (uint64_t)k;
    p.init_canvas = 1;
    int32_t* canvas = out + (size_t)k * B * L;
    if ((st = dg_canvas_run(ctx, &cur, canvas, lock, steps ? steps + (size_t)k * B : nullptr, L, &p, ws, ws_bytes,
                            stream)) != DG_OK)
      return st;
    if (k + 1 < K && (st = dg_prefill_kv(ctx, &cur, canvas, L, ws, ws_bytes, stream)) != DG_OK) return st;
  }
  if (valid) HIPCHK(launch_valid_tokens(out, K, B, L, eos_id, valid, eos_seen, stream));
  return DG_OK;
}

dg_status dg_generate_continuous(dg_ctx* ctx, const dg_kv* kv, int32_t* out, int32_t* steps, int32_t* valid,
                                 int32_t* eos_seen, int32_t* passes, int32_t K, int32_t L, int32_t eos_id,
                                 const dg_run_params* params, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err.clear();
  if (!ctx || !kv || !out || !params || !kv->prefix_len) return fail(DG_EINVAL, "NULL argument");
  if (!ctx->embed) return fail(DG_EINVAL, "generation needs the embedding");
  if (K < 1) return fail(DG_EINVAL, "K must be >= 1");
  if (params->sampler != DG_SAMPLER_EULER) return fail(DG_EUNSUPPORTED, "continuous generation runs the Euler sampler");
  if (params->self_condition && ctx->d.sc_hidden <= 0)
    return fail(DG_EINVAL, "self_condition needs a self-conditioning block");
  const int T = params->max_steps;
  if (T < 1 || T > 256) return fail(DG_EUNSUPPORTED, "max_steps %d not in [1, 256]", T);
  dg_step_params sp{};
  sp.schedule = params->schedule; sp.tau = params->tau; sp.lock_threshold = params->lock_threshold;
  sp.seed = params->seed; sp.t = 1.f; sp.h = 1.f / T;
  dg_status st = check_step_params(&sp);
  if (st != DG_OK) return st;
  const int B = kv->batch;
  if ((st = check_rows(B, L)) != DG_OK) return st;
  // every pass reads prefixes up to the largest one a sequence reaches, (K - 1) canvases on; an append
  // starts at most one canvas earlier, so the caches need room for exactly that bound
  dg_kv run = *kv;
  run.max_prefix = kv->max_prefix + (K - 1) * L;
  int mp = 0;
  if ((st = check_kv(ctx, &run, 0, &mp)) != DG_OK) return st;
  if ((st = check_ws(ctx, ws, ws_bytes, B, L, mp)) != DG_OK) return st;
  const Layout w = layout(ctx->d, B, L, mp);
  // lambda of each grid point, as the step-by-step loop takes it (double grid point, float result)
  std::vector<float> lam(T);
  for (int s = 0; s < T; ++s) lam[s] = jump_prob(params->schedule, 1.0 - s * (1.0 / T), 1.0 / T);
  float* lam_dev = at<float>(ws, w.lam_table);
  HIPCHK(launch_write_f32(lam_dev, lam.data(), T, stream));
  int32_t* flags = at<int32_t>(ws, w.seq_flags);
  int32_t* append = flags, *skip = flags + B, *finished = flags + 2 * B;
  int32_t* all_done = at<int32_t>(ws, w.all_done);
  HIPCHK(launch_fill_i32(all_done, 0, 1, stream));
  SeqArgs sa{};
  sa.B = B; sa.L = L; sa.K = K; sa.T = T; sa.V = ctx->d.vocab; sa.adaptive = params->adaptive != 0;
  sa.seed = params->seed;
  sa.state = at<int32_t>(ws, w.seq_state); sa.rng = at<uint32_t>(ws, w.seq_rng);
  sa.cur = at<int32_t>(ws, w.prev); sa.lock = at<uint8_t>(ws, w.lockbuf);
  sa.n_locked = at<int32_t>(ws, w.n_locked);
  sa.out = out; sa.steps = steps; sa.append = append; sa.skip = skip; sa.finished = finished; sa.passes = passes;
  // self-conditioning: each sequence's signal, cleared whenever its next pass appends or starts a canvas
  sa.sc = params->self_condition ? at<float>(ws, w.sc_state) : nullptr;
  sa.d = ctx->d.d_model;
  {
    // every pass is enqueued up front; once every sequence has finished, the gate turns the rest away
    GateScope gate(all_done);
    sa.init = 1;
    HIPCHK(launch_seq_schedule(sa, stream));
    sa.init = 0;
    const int max_passes = K * T + K - 1;
    for (int p = 0; p < max_passes; ++p) {
      if ((st = mixed_pass(ctx, &run, sa.cur, append, L, at<void>(ws, w.hidden), nullptr, ws, w, stream, sa.sc)) !=
          DG_OK)
        return st;
      if ((st = sample_into(ctx, at<void>(ws, w.hidden), sa.cur, sa.lock, at<int32_t>(ws, w.n_locked), skip, B, L,
                            &sp, 0.f, samp_scratch(ws, w), nullptr, nullptr, stream, sa.rng, lam_dev, sa.sc, ws,
                            &w)) != DG_OK)
        return st;
      HIPCHK(launch_seq_schedule(sa, stream));
      HIPCHK(launch_all_set(finished, B, all_done, stream));
    }
  }
  if (valid) HIPCHK(launch_valid_tokens(out, K, B, L, eos_id, valid, eos_seen, stream));
  return DG_OK;
}

// ---- test hooks ------------------------------------------------------------------------------
dg_status dg_test_step_from_logits(dg_ctx* ctx, const float* logits, int32_t* canvas, uint8_t* lock,
                                   int32_t* n_locked, int32_t batch, int32_t L, const dg_step_params* p, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
  g_err.clear();
  if (!ctx || !logits || !canvas || !lock) return fail(DG_EINVAL, "NULL argument");
  dg_status st = check_step_params(p);
  if (st != DG_OK) return st;
  if ((st = check_rows(batch, L)) != DG_OK) return st;
  if ((st = check_ws(ctx, ws, ws_bytes, batch, L, 0)) != DG_OK) return st;
  const Layout w = layout(ctx->d, batch, L, 0);
  const int R = batch * L, V = ctx->d.vocab;
  int vps;
  int slices = sampler_slices(ctx->d, R, &vps);
  const uint32_t k0 = key0(p->seed), k1 = key1(p->seed);
  const float zs = (float)(1.4426950408889634 / (double)p->tau);
  HIPCHK(launch_logits_partials(logits, R, V, L, zs, k0, k1, p->step, slices, vps, at<float>(ws, w.samp_part),
                                stream));
  StepArgs sa{};
  sa.part = at<float>(ws, w.samp_part); sa.slices = slices;
  sa.B = batch; sa.L = L; sa.canvas = canvas; sa.lock = lock; sa.n_locked = n_locked; sa.done = nullptr;
  sa.lam = jump_prob(p->schedule, p->t, p->h); sa.theta = p->lock_threshold;
  sa.k0 = k0; sa.k1 = k1; sa.step = p->step;
  sa.stats = at<float>(ws, w.stats); sa.status = at<int>(ws, w.status);
  HIPCHK(launch_step_merge(sa, stream));
  return DG_OK;
}

dg_status dg_test_read_stats(const dg_ctx* ctx, const void* ws, int32_t rows, float* m, int32_t* a, float* c,
                             int32_t* y, float* best, float* entropy, hipStream_t stream) {
  if (!ctx || !ws || rows < 1) return fail(DG_EINVAL, "bad argument");
  const Layout w = layout(ctx->d, 1, rows, 0);
  const char* base = static_cast<const char*>(ws) + w.stats;
  void* outs[STAT_FIELDS] = {m, a, c, y, best, entropy};
  for (int j = 0; j < STAT_FIELDS; ++j)
    if (outs[j])
      HIPCHK(hipMemcpy2DAsync(outs[j], 4, base + 4 * j, 4 * STAT_FIELDS, 4, rows, hipMemcpyDeviceToDevice, stream));
  return DG_OK;
}

dg_status dg_test_eb_from_logits(dg_ctx* ctx, const float* logits, int32_t* canvas, int32_t* prev, int32_t* done,
                                 int32_t* n_accepted, float* mean_entropy, int32_t batch, int32_t L,
                                 const dg_eb_params* p, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err.clear();
  if (!ctx || !logits || !canvas || !prev || !done) return fail(DG_EINVAL, "NULL argument");
  dg_status st = check_eb_params(p);
  if (st != DG_OK) return st;
  if ((st = check_rows(batch, L)) != DG_OK) return st;
  if ((st = check_ws(ctx, ws, ws_bytes, batch, L, 0)) != DG_OK) return st;
  const Layout w = layout(ctx->d, batch, L, 0);
  return eb_into(ctx, logits, true, canvas, prev, done, n_accepted, mean_entropy, batch, L, p, ws, w, nullptr,
                 stream);
}

dg_status dg_test_eb_select(dg_ctx* ctx, const float* entropy, const int32_t* argmax, const int32_t* draw,
                            int32_t* canvas, int32_t* prev, int32_t* done, int32_t* n_accepted, float* mean_entropy,
                            int32_t batch, int32_t L, const dg_eb_params* p, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  g_err.clear();
  if (!ctx || !entropy || !argmax || !draw || !canvas || !prev || !done) return fail(DG_EINVAL, "NULL argument");
  dg_status st = check_eb_params(p);
  if (st != DG_OK) return st;
  if ((st = check_rows(batch, L)) != DG_OK) return st;
  if ((st = check_ws(ctx, ws, ws_bytes, batch, L, 0)) != DG_OK) return st;
  const Layout w = layout(ctx->d, batch, L, 0);
  const size_t R = (size_t)batch * L;
  char* base = static_cast<char*>(ws) + w.stats;
  HIPCHK(hipMemcpy2DAsync(base + 4 * 1, 4 * STAT_FIELDS, argmax, 4, 4, R, hipMemcpyDeviceToDevice, stream));
  HIPCHK(hipMemcpy2DAsync(base + 4 * 3, 4 * STAT_FIELDS, draw, 4, 4, R, hipMemcpyDeviceToDevice, stream));
  HIPCHK(hipMemcpy2DAsync(base + 4 * 5, 4 * STAT_FIELDS, entropy, 4, 4, R, hipMemcpyDeviceToDevice, stream));
  HIPCHK(launch_eb_select(eb_args(ctx, canvas, prev, done, n_accepted, mean_entropy, batch, L, p, ws, w, nullptr),
                          stream));
  return DG_OK;
}

dg_status dg_test_router_topk(const float* scores, int32_t T, int32_t E, int32_t k, int32_t* idx, float* gates,
                              int32_t* counts, int32_t* offsets, int32_t* perm, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  g_err.clear();
  if (!scores || T < 1 || E < 1 || E > 256 || k < 1 || k > 16 || k > E) return fail(DG_EINVAL, "bad argument");
  if (E % 4) return fail(DG_EUNSUPPORTED, "E %% 4 != 0");
  // scratch: idx, gates, counts, offsets, perm, inv_perm, tok, work, n_items
  const size_t A = (size_t)T * k;
  const int max_items = (int)((A + GROUP_BM - 1) / GROUP_BM) + E;
  const size_t need = 6 * up(A * 4) + 2 * up(E * 4) + up((size_t)max_items * 8) + up(4);
  if (!ws || ws_bytes < need) return fail(DG_EWORKSPACE, "workspace %zu < %zu", ws_bytes, need);
  char* p = static_cast<char*>(ws);
  auto take = [&](size_t b) { char* r = p; p += up(b); return r; };
  int32_t* i_idx = idx ? idx : (int32_t*)take(A * 4);
  float* i_g = gates ? gates : (float*)take(A * 4);
  int32_t* i_c = counts ? counts : (int32_t*)take(E * 4);
  int32_t* i_o = offsets ? offsets : (int32_t*)take(E * 4);
  int32_t* i_p = perm ? perm : (int32_t*)take(A * 4);
  int32_t* inv = (int32_t*)take(A * 4);
  int32_t* tok = (int32_t*)take(A * 4);
  int32_t* work = (int32_t*)take((size_t)max_items * 8);
  int32_t* nit = (int32_t*)take(4);
  HIPCHK(launch_router_topk(scores, 1, 0, nullptr, T, E, k, nullptr, i_idx, i_g, stream));
  HIPCHK(launch_route_tables(i_idx, T, E, k, i_c, i_o, i_p, inv, tok, work, nit, GROUP_BM, stream));
  return DG_OK;
}

dg_status dg_test_read_routing(const dg_ctx* ctx, const void* ws, int32_t rows, float* logits, int32_t* idx,
                               float* gates, hipStream_t stream) {
  if (!ctx || !ws || rows < 1) return fail(DG_EINVAL, "bad argument");
  const Layout w = layout(ctx->d, 1, rows, 0);
  const char* base = static_cast<const char*>(ws);
  const size_t Rk = (size_t)rows * ctx->d.top_k;
  if (logits) HIPCHK(hipMemcpyAsync(logits, base + w.rlogits, (size_t)rows * ctx->d.n_experts * 4, hipMemcpyDeviceToDevice, stream));
  if (idx) HIPCHK(hipMemcpyAsync(idx, base + w.idx, Rk * 4, hipMemcpyDeviceToDevice, stream));
  if (gates) HIPCHK(hipMemcpyAsync(gates, base + w.gates, Rk * 4, hipMemcpyDeviceToDevice, stream));
  return DG_OK;
}

dg_status dg_test_noise(const int32_t* x0, int32_t* xt, int32_t batch, int32_t L, int32_t vocab, dg_schedule schedule,
                        float t, uint64_t seed, uint32_t step, hipStream_t stream) {
  g_err.clear();
  if (!x0 || !xt || batch < 1 || L < 1 || vocab < 1 || !(t >= 0.f && t <= 1.f)) return fail(DG_EINVAL, "bad argument");
  const float kappa = (float)kappa_of(schedule, t);
  HIPCHK(launch_noise(x0, xt, batch, L, vocab, kappa, key0(seed), key1(seed), step, stream));
  return DG_OK;
}

dg_status dg_test_read_expert_inputs(const dg_ctx* ctx, const void* ws, int32_t batch, int32_t L, void* xhat,
                                     uint8_t* xq, float* xs, void* a_grp, uint8_t* aq, float* as, void* sh_a,
                                     uint8_t* shq, float* shs, hipStream_t stream) {
  g_err.clear();
  if (!ctx || !ws || batch < 1 || L < 1) return fail(DG_EINVAL, "bad argument");
  const dg_model_desc& d = ctx->d;
  if (!d.expert_act_fp8 && (xq || xs || aq || as || shq || shs))
    return fail(DG_EINVAL, "activation codes exist only with expert_act_fp8 = 1");
  const Layout w = layout(d, batch, L, 0);
  const char* base = static_cast<const char*>(ws);
  const size_t R = (size_t)batch * L, Rk = R * d.top_k, ab = act_bytes(d);
  auto cp = [&](void* dst, size_t off, size_t bytes) -> hipError_t {
    return dst ? hipMemcpyAsync(dst, base + off, bytes, hipMemcpyDeviceToDevice, stream) : hipSuccess;
  };
  HIPCHK(cp(xhat, w.xhat, R * d.d_model * ab));
  HIPCHK(cp(a_grp, w.a_grp, Rk * d.expert_hidden * ab));
  HIPCHK(cp(sh_a, w.sh_a, R * d.shared_hidden * ab));
  HIPCHK(cp(xq, w.q_x, R * d.d_model));
  HIPCHK(cp(xs, w.q_xs, R * 4));
  HIPCHK(cp(aq, w.q_a, Rk * d.expert_hidden));
  HIPCHK(cp(as, w.q_as, Rk * 4));
  HIPCHK(cp(shq, w.q_sh, R * d.shared_hidden));
  HIPCHK(cp(shs, w.q_shs, R * 4));
  return DG_OK;
}

dg_status dg_test_quant_rows(const void* x, int32_t rows, int32_t K, uint8_t* q, float* s, hipStream_t stream) {
  g_err.clear();
  if (!x || !q || !s || rows < 1 || K < 8 || K % 8 || K > 4096) return fail(DG_EINVAL, "bad argument");
  HIPCHK(launch_quant_rows(x, K, rows, K, q, s, stream));
  return DG_OK;
}

}  // extern "C"
