// Fused LM head -> Step.
//
// Logits z = H . E^T / tau are produced tile by tile by the MFMA engine and consumed in
// registers: per row the kernel keeps a running max and its argmax, the rescaled sum of
// exp(z - max), the rescaled sum of exp(z - max) * (z - max) (for the entropy of softmax(z)),
// and the best Gumbel-perturbed key z + G with its token (Gumbel-max sampling of softmax(z)).
// Nothing of size rows x vocab is ever written.  Everything is kept in the log2 domain
// (z2 = z * log2 e) so the exponentials are single exp2 instructions; with S = sum 2^(z2 - m2)
// and W = sum 2^(z2 - m2) (z2 - m2), the entropy in nats is ln 2 * (log2 S - W / S).
//
// Each block owns one vocabulary slice for one row tile and writes one partial per row; the
// Step kernel merges the partials of every slice in ascending slice order (deterministic), then
// applies the per-position update: lock-in of confident positions, else the Euler jump with
// probability lambda to the Gumbel-max draw [TR §Backward Denoising Process; PBD glossary].
#include "gemm_dma.h"
#include "internal.h"

namespace dg {

constexpr float LN2 = 0.69314718055994531f;
constexpr float LOG2E_F = 1.44269504088896341f;
// G * log2(e) = -log2(-log2(u)) - log2(ln 2)
constexpr float NEG_LOG2_LN2 = 0.52876637294904302f;
constexpr int PART = SAMPLER_PART;  // m2, s, a, g2, y, w

struct RowState {
  float m2, s, g2, w;
  int a, y;
};

DG_DEV void state_init(RowState& st) {
  st.m2 = -INFINITY; st.s = 0.f; st.g2 = -INFINITY; st.w = 0.f; st.a = 0x7fffffff; st.y = 0x7fffffff;
}

// merge b into a; ties in the max (or the Gumbel key) go to the lower token id.  Moving a sum
// from max m to max mn: S' = S 2^(m - mn), W' = 2^(m - mn) (W + (m - mn) S).
DG_DEV void state_merge(RowState& a, float m2, float s, float w, int ai, float g2, int y) {
  const float mn = fmaxf(a.m2, m2);
  float sa = a.s, sb = s, wa = a.w, wb = w;
  if (mn != -INFINITY) {
    if (a.m2 == -INFINITY) {
      sa = 0.f; wa = 0.f;
    } else {
      const float f = exp2f(a.m2 - mn);
      wa = f * (a.w + (a.m2 - mn) * a.s);
      sa = a.s * f;
    }
    if (m2 == -INFINITY) {
      sb = 0.f; wb = 0.f;
    } else {
      const float f = exp2f(m2 - mn);
      wb = f * (w + (m2 - mn) * s);
      sb = s * f;
    }
  }
  const bool take = (m2 > a.m2) || (m2 == a.m2 && ai < a.a);
  a.s = sa + sb;
  a.w = wa + wb;
  if (take) a.a = ai;
  a.m2 = mn;
  if ((g2 > a.g2) || (g2 == a.g2 && y < a.y)) { a.g2 = g2; a.y = y; }
}

// entropy in nats of softmax over a row, from the merged sums
DG_DEV float row_entropy(const RowState& r) { return LN2 * (__log2f(r.s) - r.w / r.s); }

// Gumbel-perturbed key in log2 units without the constant -log2(ln 2) (added once per row)
DG_DEV float gumbel_key2_nc(float z2, uint32_t w) {
  const float t1 = -__log2f(unit_oo(w));       // > 0
  return z2 - __log2f(t1);
}
DG_DEV float gumbel_key2(float z2, uint32_t w) { return gumbel_key2_nc(z2, w) + NEG_LOG2_LN2; }

// ------------------------------------------------------------------ fused LM head partials ------
// Block = (vocabulary slice, BM-row tile) on WM x WN waves; wave (wm, wn) owns rows
// [BM/WM * wm, +BM/WM) of the tile and columns [BN/WN * wn, +BN/WN).  The slice's vocabulary
// tiles stream through one continuous direct-to-LDS ring: step s = (tile t, K tile kt), so the
// ring never drains between vocabulary tiles.  After the last K tile of t the logits of t are
// consumed in registers: the 16 lanes holding a row reduce the tile's row max, the sums against
// it, the argmax and the best Gumbel key with shuffles, and one lane merges the result into the
// wave's running state of that row, which lives in LDS (the registers hold only the
// accumulators); the WN states of a row are merged in wave order at the end.
// PCR: each canvas takes its own Philox key and step index from p.canvas_rng.  PW: the tile's
// probabilities relative to each row's tile maximum, 2^(z2 - max), go to p.pmat (for the
// self-conditioning product), the maxima to p.ptile.
template <class TA, int BM, int BN, int WM, int WN, int NS, bool PCR, bool PW>
__global__ __launch_bounds__(WM * WN * 64) void lmhead_sampler_kernel(SampArgs p, int n_mt) {
  if (gate_closed(p.gate)) return;
  using G = GemmDma<TA, BM, BN, WM, WN, NS>;
  constexpr int NW = WM * WN;
  extern __shared__ __align__(16) char lds[];
  float* rowst_all = reinterpret_cast<float*>(lds + G::LDS_BYTES);   // [WN][BM][PART] running row states
  // blocks of one vocabulary slice run on the same XCD (block id mod 8) so E tiles are shared
  const int id = blockIdx.x, xcd = id & 7, local = id >> 3;
  const int mt = local % n_mt;
  const int slice = (local / n_mt) * 8 + xcd;
  if (slice >= p.slices) return;
  const int m0 = mt * BM;
  const int v_begin = slice * p.v_per_slice;
  const int v_end = min(p.V, v_begin + p.v_per_slice);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15;
  const int nk = p.d / G::KT;
  const int nsteps = (v_end - v_begin + BN - 1) / BN * nk;
  float* rowst = rowst_all + (size_t)(wave % WN) * BM * PART;

  for (int r = threadIdx.x; r < WN * BM; r += NW * 64) {    // visible after the ring's first barrier
    float* q = rowst_all + r * PART;
    q[0] = -INFINITY; q[1] = 0.f; q[2] = __int_as_float(0x7fffffff);
    q[3] = -INFINITY; q[4] = __int_as_float(0x7fffffff); q[5] = 0.f;
  }

  // DMA sources: this lane's H row (fixed) and E row index within a tile, each with its swizzled chunk
  const int rr = lane >> 3, slot = lane & 7;
  const char* a_src[G::IA];
#pragma unroll
  for (int i = 0; i < G::IA; ++i) {
    const int r = (wave + NW * i) * 8 + rr;
    const int m = m0 + r < p.rows ? m0 + r : m0;
    a_src[i] = static_cast<const char*>(p.H) + (int64_t)m * p.d * sizeof(TA) + ((slot ^ ((r >> 1) & 7)) * 16);
  }
  const char* E = static_cast<const char*>(p.E);
  int it_t = 0, it_k = 0;                      // (tile, K tile) of the next step to issue
  auto issue = [&](int stage) {
    char* st = lds + stage * G::STAGE;
    const size_t koff = (size_t)it_k * 128;
#pragma unroll
    for (int i = 0; i < G::IA; ++i) dma16(a_src[i] + koff, st + (wave + NW * i) * 8 * 128);
    const int v0 = v_begin + it_t * BN;
#pragma unroll
    for (int i = 0; i < G::IB; ++i) {
      const int r = (wave + NW * i) * 8 + rr;
      const int v = min(v0 + r, v_end - 1);
      dma16<DMA_STREAM>(E + (int64_t)v * p.d * sizeof(TA) + ((slot ^ ((r >> 1) & 7)) * 16) + koff,
            st + BM * 128 + (wave + NW * i) * 8 * 128);
    }
    if (++it_k == nk) { it_k = 0; ++it_t; }
  };

  f32x4_v acc[G::FM][G::FN];
#pragma unroll
  for (int i = 0; i < G::FM; ++i)
#pragma unroll
    for (int j = 0; j < G::FN; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};

  int issued = 0;
  for (; issued < NS - 1 && issued < nsteps; ++issued) issue(issued);
  int t = 0, kt = 0;
  for (int s = 0; s < nsteps; ++s) {
    G::wait_oldest(issued - s);
    lds_barrier();
    if (issued < nsteps) {
      issue(issued % NS);
      ++issued;
    }
    G::compute(lds + (s % NS) * G::STAGE, acc);
    if (++kt < nk) continue;
    kt = 0;
    // ---- logits of vocabulary tile t: z = acc / tau (log2 units) ---------------------------------
    const int v0 = v_begin + t * BN;
    ++t;
#pragma unroll
    for (int i = 0; i < G::FM; ++i) {
      const int rb = m0 + G::row_of(i, 0);       // first of this lane's 4 consecutive rows
      const int b = rb / p.L, ii = rb - b * p.L;
      uint32_t rk0 = p.k0, rk1 = p.k1, rstep = p.step;
      if constexpr (PCR) {
        const uint4 cr = *reinterpret_cast<const uint4*>(p.canvas_rng + 4 * min(b, p.rows / p.L - 1));
        rk0 = cr.x; rk1 = cr.y; rstep = cr.z;
      }
      // the row max over the tile (lowest token on ties): lane-local, then over the 16 lanes
      float rm[4];
      int ra[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float zmax = -INFINITY;
        int vmax = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < G::FN; ++j) {
          const int v = v0 + G::col_of(j);
          const float z = v < v_end ? acc[i][j][e] * p.zscale_log2 : -INFINITY;
          acc[i][j][e] = z;
          if (z > zmax) { zmax = z; vmax = v; }
        }
        const float m = row16_max(zmax);
        rm[e] = m;
        ra[e] = row16_min(zmax == m ? vmax : 0x7fffffff);
      }
      // sums against the row max and the Gumbel keys; one Philox block serves the lane's 4
      // consecutive rows of one token
      float ss[4] = {0.f, 0.f, 0.f, 0.f}, ww[4] = {0.f, 0.f, 0.f, 0.f};
      float g2[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      int yy[4] = {0x7fffffff, 0x7fffffff, 0x7fffffff, 0x7fffffff};
      TA* prow[4];
      if constexpr (PW) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + G::row_of(i, e);
          prow[e] = row < p.rows ? static_cast<TA*>(p.pmat) + (int64_t)row * p.V : nullptr;
          if (prow[e] && l16 == 0) p.ptile[(int64_t)row * p.n_vtiles + v0 / BN] = rm[e];
        }
      }
#pragma unroll
      for (int j = 0; j < G::FN; ++j) {
        const int v = v0 + G::col_of(j);
        if (v < v_end) {
          const u32x4 w = philox((uint32_t)v, (uint32_t)(ii >> 2), rstep, ((uint32_t)b << 8) | TAG_GUMBEL, rk0, rk1);
          const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float z = acc[i][j][e];
            const float dz = z - rm[e];
            const float ex = __builtin_amdgcn_exp2f(dz);   // dz <= 0; terms below 2^-126 do not count
            if constexpr (PW) {
              if (prow[e]) prow[e][v] = Elem<TA>::from_f(ex);
            }
            ss[e] += ex;
            ww[e] += ex * dz;
            const float key = gumbel_key2_nc(z, wd[e]);
            if (key > g2[e]) { g2[e] = key; yy[e] = v; }
          }
        }
        acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ss[e] = row16_sum(ss[e]);
        ww[e] = row16_sum(ww[e]);
        row16_argmax(g2[e], yy[e]);
      }
      // lane l16 = e merges row e of its group into the running state (one fixed lane per row,
      // so the sums it publishes do not depend on timing)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (l16 != e) continue;
        float* q = rowst + G::row_of(i, e) * PART;
        RowState r;
        r.m2 = q[0]; r.s = q[1]; r.a = __float_as_int(q[2]); r.g2 = q[3]; r.y = __float_as_int(q[4]); r.w = q[5];
        state_merge(r, rm[e], ss[e], ww[e], ra[e], g2[e] + NEG_LOG2_LN2, yy[e]);
        q[0] = r.m2; q[1] = r.s; q[2] = __int_as_float(r.a); q[3] = r.g2; q[4] = __int_as_float(r.y); q[5] = r.w;
      }
    }
  }

  __syncthreads();
  for (int r = threadIdx.x; r < BM; r += NW * 64) {
    const int m = m0 + r;
    if (m >= p.rows) continue;
    const float* q = rowst_all + r * PART;
    RowState s;
    s.m2 = q[0]; s.s = q[1]; s.a = __float_as_int(q[2]); s.g2 = q[3]; s.y = __float_as_int(q[4]); s.w = q[5];
    for (int w = 1; w < WN; ++w) {
      q = rowst_all + ((size_t)w * BM + r) * PART;
      state_merge(s, q[0], q[1], q[5], __float_as_int(q[2]), q[3], __float_as_int(q[4]));
    }
    float* o = p.part + ((size_t)slice * p.rows + m) * PART;
    o[0] = s.m2; o[1] = s.s; o[2] = __int_as_float(s.a); o[3] = s.g2; o[4] = __int_as_float(s.y); o[5] = s.w;
  }
}

template <class TA, int BM, int BN, int WM, int WN, int NS, bool PCR, bool PW>
static hipError_t launch_sampler_p(const SampArgs& a, hipStream_t s) {
  using G = GemmDma<TA, BM, BN, WM, WN, NS>;
  const int n_mt = (a.rows + BM - 1) / BM;
  const int blocks = n_mt * ((a.slices + 7) / 8 * 8);
  const size_t lds = G::LDS_BYTES + (size_t)WN * BM * PART * 4;
  if (a.d % G::KT) return hipErrorInvalidValue;
  if (PW && (a.v_per_slice % BN || a.n_vtiles != (a.V + BN - 1) / BN)) return hipErrorInvalidValue;
  static const hipError_t attr = allow_lds(lmhead_sampler_kernel<TA, BM, BN, WM, WN, NS, PCR, PW>, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((lmhead_sampler_kernel<TA, BM, BN, WM, WN, NS, PCR, PW>), dim3(blocks), dim3(WM * WN * 64), lds,
                     s, a, n_mt);
  return hipGetLastError();
}

template <class TA, int BM, int BN, int WM, int WN, int NS>
static hipError_t launch_sampler_t(SampArgs a, hipStream_t s) {
  a.gate = launch_gate();
  if (a.pmat) {
    if (a.canvas_rng) return launch_sampler_p<TA, BM, BN, WM, WN, NS, true, true>(a, s);
    return launch_sampler_p<TA, BM, BN, WM, WN, NS, false, true>(a, s);
  }
  if (a.canvas_rng) return launch_sampler_p<TA, BM, BN, WM, WN, NS, true, false>(a, s);
  return launch_sampler_p<TA, BM, BN, WM, WN, NS, false, false>(a, s);
}

// p_hat_0 = 2^(z2 - lse2): each thread rescales 8 consecutive probabilities of one row (one tile)
template <class T>
__global__ void p_rescale_kernel(T* P, const float* ptile, const float* stats, int V, int bn, int n_vtiles,
                                 const int32_t* gate) {
  if (gate_closed(gate)) return;
  const int r = blockIdx.y;
  const int v0 = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (v0 >= V) return;
  const float* st = stats + (size_t)r * STAT_FIELDS;
  const float lse2 = st[0] * LOG2E_F - __log2f(st[2]);      // m2 + log2(sum): c = 1 / sum
  const float f = exp2f(ptile[(size_t)r * n_vtiles + v0 / bn] - lse2);
  T* q = P + (size_t)r * V + v0;
#pragma unroll
  for (int e = 0; e < 8; ++e) q[e] = Elem<T>::from_f(Elem<T>::to_f(q[e]) * f);
}

hipError_t launch_p_rescale(void* P, const float* ptile, const float* stats, int rows, int V, int bn, int n_vtiles,
                            int bf, hipStream_t s) {
  if (V % 8 || bn % 8) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((V / 8 + 255) / 256), (unsigned)rows);
  if (bf)
    hipLaunchKernelGGL(p_rescale_kernel<bf16_t>, grid, dim3(256), 0, s, (bf16_t*)P, ptile, stats, V, bn, n_vtiles,
                       launch_gate());
  else
    hipLaunchKernelGGL(p_rescale_kernel<float>, grid, dim3(256), 0, s, (float*)P, ptile, stats, V, bn, n_vtiles,
                       launch_gate());
  return hipGetLastError();
}

// tiles: bf16 256 rows x 256 vocabulary entries on 8 waves of 32 rows (a row's statistics stay
// in one wave), two ring stages; fp32 128 x 128 on 4 waves of 32 rows, three stages
hipError_t launch_lmhead_sampler(const SampArgs& a, int act_bf16, hipStream_t s) {
  if (act_bf16) return launch_sampler_t<bf16_t, SAMPLER_BM_BF16, SAMPLER_BN_BF16, 8, 1, 2>(a, s);
  return launch_sampler_t<float, SAMPLER_BM_F32, SAMPLER_BN_F32, 4, 1, 3>(a, s);
}

// ------------------------------------------------------------------ partials from given logits --
// Test hook: the same partials from an fp32 logit array (one block per (row, slice)).
__global__ __launch_bounds__(256) void logits_partials_kernel(const float* z, int rows, int V, int L,
                                                              float zs, uint32_t k0, uint32_t k1,
                                                              uint32_t step, int v_per_slice, float* part) {
  const int row = blockIdx.x, slice = blockIdx.y;
  const int b = row / L, ii = row - b * L;
  const int v_begin = slice * v_per_slice, v_end = min(V, v_begin + v_per_slice);
  RowState st;
  state_init(st);
  for (int v = v_begin + threadIdx.x; v < v_end; v += 256) {
    const float z2 = z[(int64_t)row * V + v] * zs;
    const u32x4 w = philox((uint32_t)v, (uint32_t)(ii >> 2), step, ((uint32_t)b << 8) | TAG_GUMBEL, k0, k1);
    state_merge(st, z2, 1.f, 0.f, v, gumbel_key2(z2, pick(w, ii & 3)), v);
  }
  for (int o = 1; o < 64; o <<= 1) {
    const float m2 = __shfl_xor(st.m2, o, 64), ss = __shfl_xor(st.s, o, 64), g2 = __shfl_xor(st.g2, o, 64);
    const float ww = __shfl_xor(st.w, o, 64);
    const int a = __shfl_xor(st.a, o, 64), y = __shfl_xor(st.y, o, 64);
    state_merge(st, m2, ss, ww, a, g2, y);
  }
  __shared__ float xch[4][PART];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    xch[wave][0] = st.m2; xch[wave][1] = st.s; xch[wave][2] = __int_as_float(st.a);
    xch[wave][3] = st.g2; xch[wave][4] = __int_as_float(st.y); xch[wave][5] = st.w;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    RowState s;
    state_init(s);
    for (int w = 0; w < 4; ++w)
      state_merge(s, xch[w][0], xch[w][1], xch[w][5], __float_as_int(xch[w][2]), xch[w][3],
                  __float_as_int(xch[w][4]));
    float* o = part + ((size_t)slice * rows + row) * PART;
    o[0] = s.m2; o[1] = s.s; o[2] = __int_as_float(s.a); o[3] = s.g2; o[4] = __int_as_float(s.y); o[5] = s.w;
  }
}

hipError_t launch_logits_partials(const float* z, int rows, int V, int L, float zs, uint32_t k0,
                                  uint32_t k1, uint32_t step, int slices, int v_per_slice,
                                  float* part, hipStream_t s) {
  hipLaunchKernelGGL(logits_partials_kernel, dim3(rows, slices), dim3(256), 0, s, z, rows, V, L, zs,
                     k0, k1, step, v_per_slice, part);
  return hipGetLastError();
}

// ------------------------------------------------------------------ merge + Step -----------------
// One wave per position: lane j merges slices j, j+64, ... in ascending order, then a fixed xor
// tree combines the lanes (deterministic).  Lane 0 applies the Step to the position.
__global__ __launch_bounds__(256) void step_merge_kernel(StepArgs p) {
  if (gate_closed(p.gate)) return;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int rows = p.B * p.L;
  if (r >= rows) return;
  const int b = r / p.L, i = r - b * p.L;
  RowState s;
  state_init(s);
  // four slices per lane per round, loaded before they are merged in ascending order
  for (int base = lane; base < p.slices; base += 256) {
    float q[4][PART];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sl = min(base + 64 * u, p.slices - 1);
      const float* src = p.part + ((size_t)sl * rows + r) * PART;
#pragma unroll
      for (int f = 0; f < PART; ++f) q[u][f] = src[f];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (base + 64 * u < p.slices)
        state_merge(s, q[u][0], q[u][1], q[u][5], __float_as_int(q[u][2]), q[u][3], __float_as_int(q[u][4]));
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float m2 = __shfl_xor(s.m2, o, 64), ss = __shfl_xor(s.s, o, 64), g2 = __shfl_xor(s.g2, o, 64);
    const float ww = __shfl_xor(s.w, o, 64);
    const int a = __shfl_xor(s.a, o, 64), y = __shfl_xor(s.y, o, 64);
    state_merge(s, m2, ss, ww, a, g2, y);
  }
  if (lane != 0) return;
  const float c = 1.f / s.s;
  const float H = row_entropy(s);
  const bool bad = !(isfinite(s.m2) && isfinite(s.s) && isfinite(s.g2) && isfinite(H));
  if (p.stats) {
    float* o = p.stats + (size_t)r * STAT_FIELDS;
    o[0] = s.m2 * LN2; o[1] = __int_as_float(s.a); o[2] = c; o[3] = __int_as_float(s.y);
    o[4] = s.g2 * LN2; o[5] = H;
  }
  if (bad) {
    if (p.status) atomicOr(p.status, 1);
    return;
  }
  if (p.stats_only) return;
  const bool is_done = p.done && p.done[b] != 0;
  if (is_done || p.lock[r]) return;
  if (c >= p.theta) {
    p.canvas[r] = s.a;
    p.lock[r] = 1;
  } else {
    uint32_t k0 = p.k0, k1 = p.k1, stp = p.step;
    float lam = p.lam;
    if (p.canvas_rng) {
      const uint4 cr = *reinterpret_cast<const uint4*>(p.canvas_rng + 4 * b);
      k0 = cr.x; k1 = cr.y; stp = cr.z;
      lam = p.lam_table[stp];
    }
    const u32x4 w = philox((uint32_t)(i >> 2), 0u, stp, ((uint32_t)b << 8) | TAG_JUMP, k0, k1);
    if (unit_co(pick(w, i & 3)) < lam) p.canvas[r] = s.y;
  }
}

// One block per canvas: locked count (-1 if a non-finite statistic was seen in the canvas),
// steps taken and the done flag of the adaptive loop.
__global__ __launch_bounds__(256) void step_count_kernel(StepArgs p) {
  if (gate_closed(p.gate)) return;
  const int b = blockIdx.x;
  const int rows = p.B * p.L;
  int nl = 0, nb = 0;
  for (int i = threadIdx.x; i < p.L; i += 256) {
    const int r = b * p.L + i;
    nl += p.lock[r] != 0;
    if (p.stats) nb += !isfinite(p.stats[(size_t)r * STAT_FIELDS + 2]) || !isfinite(p.stats[(size_t)r * STAT_FIELDS]);
  }
  (void)rows;
  for (int o = 32; o > 0; o >>= 1) { nl += __shfl_xor(nl, o, 64); nb += __shfl_xor(nb, o, 64); }
  __shared__ int red[2][4];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { red[0][wave] = nl; red[1][wave] = nb; }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int tl = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    const int tb = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    const bool is_done = p.done && p.done[b] != 0;
    if (p.n_locked) p.n_locked[b] = tb ? -1 : tl;
    if (!is_done && p.steps_taken) p.steps_taken[b] += 1;
    if (p.done_out) p.done_out[b] = (tl == p.L) ? 1 : (p.done ? p.done[b] : 0);
  }
}

hipError_t launch_step_merge(StepArgs a, hipStream_t s) {
  a.gate = launch_gate();
  const int rows = a.B * a.L;
  hipLaunchKernelGGL(step_merge_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, a);
  if (!a.stats_only) hipLaunchKernelGGL(step_count_kernel, dim3(a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ entropy-bounded step ---------
// One block per canvas ([TR §DiffusionGemma 샘플러]): positions sorted by (entropy, position) with a
// bitonic sort of 64-bit keys in LDS (entropies are >= 0, so their float bits order like the
// values); one thread takes the float32 running sum in that order to find the largest k whose
// sum stays within gamma, and the mean entropy (the same sum over all L, divided by L).  The k
// lowest-entropy positions take the Gumbel-max draw y, the rest a uniform re-noise token; a canvas
// whose argmax sequence equals the previous step's and whose mean entropy is below the threshold
// stops (adaptive), and a stopped or final canvas takes its argmax sequence.
constexpr int EB_MAX_L = 1024;
__global__ __launch_bounds__(EB_MAX_L) void eb_select_kernel(EbArgs p) {
  __shared__ unsigned long long key[EB_MAX_L];
  __shared__ int rank[EB_MAX_L];
  __shared__ int sh_k, sh_unstable;
  __shared__ float sh_mean;
  const int b = blockIdx.x, i = threadIdx.x, NT = blockDim.x;
  if (gate_closed(p.gate) || p.done[b]) return;                              // the whole block leaves together
  const int r = b * p.L + i;
  float H = 0.f;
  int a = 0, y = 0;
  if (i < p.L) {
    const float* st = p.stats + (size_t)r * STAT_FIELDS;
    a = __float_as_int(st[1]);
    y = __float_as_int(st[3]);
    H = fmaxf(st[5], 0.f) + 0.f;                      // rounding below zero counts as (+)zero
  }
  key[i] = i < p.L ? ((unsigned long long)__float_as_uint(H) << 32) | (unsigned)i : ~0ull;
  if (i == 0) sh_unstable = 0;
  __syncthreads();
  if (i < p.L && p.has_prev && p.prev[r] != a) sh_unstable = 1;
  for (int k = 2; k <= NT; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      __syncthreads();
      const int ixj = i ^ j;
      if (ixj > i) {
        const unsigned long long x = key[i], z = key[ixj];
        if ((x > z) == ((i & k) == 0)) { key[i] = z; key[ixj] = x; }
      }
    }
  __syncthreads();
  if (i < p.L) rank[key[i] & 0xffffffffu] = i;
  if (i == 0) {
    float run = 0.f;
    int kk = 0;
    for (int q = 0; q < p.L; ++q) {
      run += __uint_as_float((unsigned)(key[q] >> 32));
      if (run <= p.gamma) kk = q + 1;
    }
    sh_k = kk;
    sh_mean = run / (float)p.L;
  }
  __syncthreads();
  const int k = sh_k;
  const float mean = sh_mean;
  const bool stop = p.adaptive && p.has_prev && !sh_unstable && mean < p.stop_entropy;
  const bool fin = stop || p.final_step;
  if (i < p.L) {
    int x;
    if (fin) {
      x = a;
    } else if (rank[i] < k) {
      x = y;
    } else {
      const u32x4 w = philox((uint32_t)(i >> 2), 0u, p.step, ((uint32_t)b << 8) | TAG_RENOISE, p.k0, p.k1);
      x = token_of(pick(w, i & 3), p.vocab, p.vocab_log2);
    }
    p.canvas[r] = x;
    p.prev[r] = a;
  }
  if (i == 0) {
    if (fin) p.done[b] = 1;
    if (p.n_accepted) p.n_accepted[b] = k;
    if (p.mean_entropy) p.mean_entropy[b] = mean;
    if (p.steps_taken) p.steps_taken[b] += 1;
  }
}

static int log2_exact(int v);

hipError_t launch_eb_select(EbArgs a, hipStream_t s) {
  if (a.L < 1 || a.L > EB_MAX_L) return hipErrorInvalidValue;
  int nt = 64;
  while (nt < a.L) nt <<= 1;
  a.vocab_log2 = log2_exact(a.vocab);
  a.gate = launch_gate();
  hipLaunchKernelGGL(eb_select_kernel, dim3(a.B), dim3(nt), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ canvas init / noise ----------
static int log2_exact(int v) {
  if (v <= 0 || (v & (v - 1))) return -1;
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

__global__ void init_canvas_kernel(int32_t* canvas, uint8_t* lock, int B, int L, int V, int vlog2,
                                   uint32_t k0, uint32_t k1) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= B * L) return;
  const int b = r / L, i = r - b * L;
  const u32x4 w = philox((uint32_t)(i >> 2), 0u, 0u, ((uint32_t)b << 8) | TAG_INIT, k0, k1);
  canvas[r] = token_of(pick(w, i & 3), V, vlog2);
  if (lock) lock[r] = 0;
}

hipError_t launch_init_canvas(int32_t* canvas, uint8_t* lock, int B, int L, int V, uint32_t k0,
                              uint32_t k1, hipStream_t s) {
  const int n = B * L;
  hipLaunchKernelGGL(init_canvas_kernel, dim3((n + 255) / 256), dim3(256), 0, s, canvas, lock, B, L, V,
                     log2_exact(V), k0, k1);
  return hipGetLastError();
}

__global__ void noise_kernel(const int32_t* x0, int32_t* xt, int B, int L, int V, int vlog2, float kappa,
                             uint32_t k0, uint32_t k1, uint32_t step) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= B * L) return;
  const int b = r / L, i = r - b * L;
  const u32x4 wk = philox((uint32_t)(i >> 2), 0u, step, ((uint32_t)b << 8) | TAG_NOISE_KEEP, k0, k1);
  const u32x4 wt = philox((uint32_t)(i >> 2), 0u, step, ((uint32_t)b << 8) | TAG_NOISE_TOKEN, k0, k1);
  xt[r] = unit_co(pick(wk, i & 3)) < kappa ? x0[r] : token_of(pick(wt, i & 3), V, vlog2);
}

hipError_t launch_noise(const int32_t* x0, int32_t* xt, int B, int L, int V, float kappa, uint32_t k0,
                        uint32_t k1, uint32_t step, hipStream_t s) {
  const int n = B * L;
  hipLaunchKernelGGL(noise_kernel, dim3((n + 255) / 256), dim3(256), 0, s, x0, xt, B, L, V, log2_exact(V),
                     kappa, k0, k1, step);
  return hipGetLastError();
}

// ------------------------------------------------------------------ continuous block-AR ----------
// One block per sequence.  After a pass: a denoising sequence counts the step; once it stops (all
// positions locked, adaptive) or reaches T steps, its canvas is stored as canvas k and the next pass
// appends it to the cache (or the sequence finishes after canvas K - 1).  After an append pass the
// sequence starts canvas k + 1 at t = 1: uniform tokens from the canvas-init stream of seed + k + 1,
// locks cleared.  The flags and Philox keys written here drive the next pass.
__global__ __launch_bounds__(256) void seq_schedule_kernel(SeqArgs a) {
  if (gate_closed(a.gate)) return;
  const int b = blockIdx.x;
  __shared__ int sh_copy, sh_fresh, sh_k, sh_phase;
  if (threadIdx.x == 0) {
    int32_t* st = a.state + 4 * b;
    int phase = SEQ_DENOISE, k = 0, s = 0, taken = 0, copy = -1, fresh = 1;
    if (!a.init) {
      phase = st[0]; k = st[1]; s = st[2]; taken = st[3];
      fresh = 0;
      if (phase == SEQ_DENOISE) {
        ++s;
        ++taken;
        if ((a.adaptive && a.n_locked[b] == a.L) || s == a.T) {
          copy = k;
          if (a.steps) a.steps[(int64_t)k * a.B + b] = taken;
          phase = k + 1 < a.K ? SEQ_APPEND : SEQ_FINISHED;
        }
      } else if (phase == SEQ_APPEND) {
        ++k;
        s = 0;
        taken = 0;
        phase = SEQ_DENOISE;
        fresh = 1;
      }
    }
    st[0] = phase; st[1] = k; st[2] = s; st[3] = taken;
    const uint64_t seed = a.seed + (uint64_t)k;
    uint32_t* r = a.rng + 4 * b;
    r[0] = (uint32_t)(seed & 0xffffffffu); r[1] = (uint32_t)(seed >> 32); r[2] = (uint32_t)s; r[3] = 0u;
    a.append[b] = phase == SEQ_APPEND;
    a.skip[b] = phase != SEQ_DENOISE;
    a.finished[b] = phase == SEQ_FINISHED;
    if (b == 0 && a.passes) a.passes[0] = a.init ? 0 : a.passes[0] + 1;
    sh_copy = copy; sh_fresh = fresh; sh_k = k; sh_phase = phase;
  }
  __syncthreads();
  const int copy = sh_copy, k = sh_k;
  int32_t* cur = a.cur + (int64_t)b * a.L;
  if (a.sc && (sh_phase != SEQ_DENOISE || sh_fresh)) {
    // the encoder pass of an appended canvas and the first step of a new one take no signal
    float* sc = a.sc + (int64_t)b * a.L * a.d;
    for (int64_t i = threadIdx.x; i < (int64_t)a.L * a.d; i += blockDim.x) sc[i] = 0.f;
  }
  if (copy >= 0)
    for (int i = threadIdx.x; i < a.L; i += blockDim.x) a.out[((int64_t)copy * a.B + b) * a.L + i] = cur[i];
  if (sh_fresh) {
    const uint64_t seed = a.seed + (uint64_t)k;
    const uint32_t k0 = (uint32_t)(seed & 0xffffffffu), k1 = (uint32_t)(seed >> 32);
    const int vlog2 = (a.V & (a.V - 1)) ? -1 : 31 - __clz(a.V);
    for (int i = threadIdx.x; i < a.L; i += blockDim.x) {
      const u32x4 w = philox((uint32_t)(i >> 2), 0u, 0u, ((uint32_t)b << 8) | TAG_INIT, k0, k1);
      cur[i] = token_of(pick(w, i & 3), a.V, vlog2);
      a.lock[(int64_t)b * a.L + i] = 0;
    }
  }
}

hipError_t launch_seq_schedule(SeqArgs a, hipStream_t s) {
  a.gate = launch_gate();
  hipLaunchKernelGGL(seq_schedule_kernel, dim3(a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

struct F32Vals { float v[256]; };
__global__ void write_f32_kernel(float* dst, F32Vals vals, int n) {
  if ((int)threadIdx.x < n) dst[threadIdx.x] = vals.v[threadIdx.x];
}

hipError_t launch_write_f32(float* dst, const float* vals, int n, hipStream_t s) {
  if (n < 0 || n > 256) return hipErrorInvalidValue;
  F32Vals v{};
  for (int i = 0; i < n; ++i) v.v[i] = vals[i];
  hipLaunchKernelGGL(write_f32_kernel, dim3(1), dim3(256), 0, s, dst, v, n);
  return hipGetLastError();
}

}  // namespace dg
