// Dense and expert-grouped GEMMs of the decoder layer with their fused epilogues:
//   QKV projection + RoPE + scatter to q / canvas k / canvas v,
//   attention output projection + residual add,
//   router logits (+ bias),
//   shared- and routed-expert SwiGLU (gate and up in one tile) and down projections.
// W8A16: fp8 e4m3 weights are widened to bf16 in the tile loader; the per-output-row scale is
// applied to the fp32 accumulator in the epilogue.
#include <type_traits>

#include "gemm_core.h"
#include "gemm_dma.h"
#include "internal.h"

namespace dg {

// bf16/fp32 weights stream through the direct-to-LDS engine; fp8 weights take the
// register-staged engine, which widens them to bf16 on the way into LDS.  Rings of 3-4 stages
// let two blocks share a CU (a single block per CU with a ring twice as deep was slower).
constexpr int ring_stages(int stage_bytes) { return stage_bytes <= 20480 ? 4 : stage_bytes <= 24576 ? 3 : 2; }
template <class TA, class TB, int BM, int BN, int WM, int WN, int NS = 0, int KPS = 1>
using TileFor = std::conditional_t<sizeof(TB) == 1, GemmTile<TA, TB, BM, BN, WM, WN, 4>,
                                   GemmDma<TA, BM, BN, WM, WN, NS ? NS : ring_stages((BM + BN) * 128), DMA_STREAM, KPS>>;
// grouped (expert) GEMMs: fp8 weights stream as raw codes on the direct-to-LDS ring, widened in
// registers (12 KB stages x 6, two blocks per CU); MXFP4 weights go through the register-staged
// engine, which measured faster for them (its stages carry 64 elements of all 128 rows widened
// once per block, where the ring's per-stage scale loads and short stages cost more)
// W8A8 (e4m3 activation codes with fp8 weights): both operands as codes on the ring, fp8 MFMA
template <class TA, class TB, int BM, int BN, int WM, int WN, int NS = 0, int QNS = 6>
using GroupTileFor = std::conditional_t<
    is_fp8a_v<TA>, GemmDmaQQ<BM, BN, WM, WN, QNS>,
    std::conditional_t<is_fp8_v<TB>, GemmDmaQ<TB, BM, BN, WM, WN, QNS>, TileFor<TA, TB, BM, BN, WM, WN, NS>>>;

// ---------------------------------------------------------------- B-row maps ----------------
// A tile column block of 16 columns; "paired" maps put the two members of a pair (gate/up, or
// RoPE partners j and j + dh/2) in adjacent blocks so one lane holds both.
enum BMap { MAP_PLAIN = 0, MAP_SWIGLU = 1, MAP_ROPE = 2 };

template <int BN>
DG_DEV void paired_col(int r, int& u, int& half, int& c) {
  const int nb = r >> 4;
  c = r & 15;
  u = nb >> 1;
  half = nb & 1;
}

// 1-D grid, XCD-aware: block id mod 8 picks the XCD; the n_mt row tiles of one column (weight)
// tile get ids congruent mod 8, so they run on one XCD and share its L2 copy of the weights.
// blockIdx.y is the split-K part.
// Epilogues that stage the output tile in LDS (rows padded by 16 bytes) when it fits in a CU's
// 160 KB: the QKV q / k rows (in the activation type) and the float32 (split-K) stores.  The dense
// launch's dynamic LDS is the larger of that and the ring.
template <class TA, int BM, int BN, int EPI>
constexpr int qkv_stage_bytes() {
  const int b = BM * (BN * (int)sizeof(TA) + 16);
  return EPI == EPI_QKV && b <= 160 * 1024 && (BN / 2) % (16 / (int)sizeof(TA)) == 0 ? b : 0;
}
template <int BM, int BN, int EPI>
constexpr int f32_stage_bytes() {
  const int b = BM * (BN * 4 + 16);
  return EPI == EPI_STORE_F32 && b <= 160 * 1024 && BN % 4 == 0 ? b : 0;
}
// the QKV v tile, transposed: BN dims of BM positions each (padded by 16 bytes)
template <class TA, int BM, int BN, int EPI>
constexpr int v_stage_bytes() {
  const int b = BN * (BM * (int)sizeof(TA) + 16);
  return EPI == EPI_QKV && b <= 160 * 1024 && BM % (16 / (int)sizeof(TA)) == 0 ? b : 0;
}
template <class G, class TA, int BM, int BN, int EPI>
constexpr size_t dense_lds_bytes() {
  size_t b = G::LDS_BYTES;
  if ((size_t)qkv_stage_bytes<TA, BM, BN, EPI>() > b) b = qkv_stage_bytes<TA, BM, BN, EPI>();
  if ((size_t)v_stage_bytes<TA, BM, BN, EPI>() > b) b = v_stage_bytes<TA, BM, BN, EPI>();
  if ((size_t)f32_stage_bytes<BM, BN, EPI>() > b) b = f32_stage_bytes<BM, BN, EPI>();
  return b;
}

template <class TA, class TB, int BM, int BN, int WM, int WN, int EPI, int MAP, int NS = 0, int KPS = 1>
__global__ __launch_bounds__(WM * WN * 64) void gemm_dense_kernel(DenseArgs p) {
  if (gate_closed(p.gate)) return;
  using G = TileFor<TA, TB, BM, BN, WM, WN, NS, KPS>;
  extern __shared__ __align__(16) char lds[];
  const int id = blockIdx.x, xcd = id & 7, local = id >> 3;
  const int mt = local % p.n_mt;
  const int nt = (local / p.n_mt) * 8 + xcd;
  if (nt >= p.n_nt) return;
  const int n0 = nt * BN, m0 = mt * BM;
  const int kpart = p.K / p.ksplit, k0 = blockIdx.y * kpart;
  const TA* A = static_cast<const TA*>(p.A);
  const TB* B = static_cast<const TB*>(p.B);
  const TB* B2 = static_cast<const TB*>(p.B2);
  auto arow = [&](int r) -> const TA* {
    const int m = m0 + r;
    return m < p.M ? A + (int64_t)m * p.lda + k0 : nullptr;
  };
  auto brow = [&](int r) -> const TB* {
    if constexpr (MAP == MAP_PLAIN) {
      const int n = n0 + r;
      return n < p.N ? B + (int64_t)n * p.ldb + k0 : nullptr;
    } else if constexpr (MAP == MAP_SWIGLU) {
      int u, half, c;
      paired_col<BN>(r, u, half, c);
      const int oc = n0 / 2 + u * 16 + c;
      if (oc >= p.N) return nullptr;
      return (half ? B2 : B) + (int64_t)oc * p.ldb + k0;
    } else {  // MAP_ROPE: tile inside one head
      int u, half, c;
      paired_col<BN>(r, u, half, c);
      const int head = n0 / p.dh, pb = (n0 % p.dh) / 2;
      const int row = head * p.dh + half * (p.dh / 2) + pb + u * 16 + c;
      return B + (int64_t)row * p.ldb + k0;
    }
  };
  G g;
  g.setup(arow, brow);
  const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) % WN;
  // QKV: where they take few registers, this lane's (cos, sin) table entries are loaded before the
  // K loop, so their latency passes under it instead of trailing it (rows past M read row M - 1)
  constexpr int NCS = G::FM * (G::FN / 2) * 4;
  constexpr bool CS_AHEAD = EPI == EPI_QKV && NCS <= 16;
  float2 cs_pre[CS_AHEAD ? NCS : 1];
  if constexpr (CS_AHEAD) {
    const int head = n0 / p.dh, pb = (n0 % p.dh) / 2, half_dh = p.dh / 2;
    if (head < p.Hq + p.Hkv) {
#pragma unroll
      for (int j = 0; j < G::FN; j += 2)
#pragma unroll
        for (int i = 0; i < G::FM; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = min(m0 + G::row_of(i, e), p.M - 1);
            const int jj = pb + ((wn * G::FN + j) >> 1) * 16 + (lane & 15);
            cs_pre[((j >> 1) * G::FM + i) * 4 + e] = p.rope[(int64_t)m * half_dh + jj];
          }
    }
  }
  f32x4_v acc[G::FM][G::FN];
  g.run(lds, kpart, acc);
  float* const C32 = static_cast<float*>(p.C) + (int64_t)blockIdx.y * p.c_split;

  if constexpr (f32_stage_bytes<BM, BN, EPI>() > 0) {
    // float32 tile through LDS, then whole 16-byte row chunks, streamed (the next launch reads
    // each partial once, from any XCD)
    constexpr int ROWB = BN * 4 + 16;
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
      const int c = G::col_of(j), n = n0 + c;
      float sc = 1.f, bias = 0.f;
      if (n < p.N) {
        if constexpr (sizeof(TB) == 1) sc = bf2f(p.sB[n]);
        if (p.bias) bias = p.bias[n];
      }
#pragma unroll
      for (int i = 0; i < G::FM; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          reinterpret_cast<float*>(lds + G::row_of(i, e) * ROWB)[c] = acc[i][j][e] * sc + bias;
    }
    __syncthreads();
    constexpr int CPR = BN / 4;
    for (int ch = threadIdx.x; ch < BM * CPR; ch += WM * WN * 64) {
      const int r = ch / CPR, col = (ch - r * CPR) * 4, m = m0 + r, n = n0 + col;
      if (m >= p.M || n >= p.N) continue;
      float* dst = C32 + (int64_t)m * p.ldc + n;
      const float* src = reinterpret_cast<const float*>(lds + r * ROWB) + col;
      if (n + 4 <= p.N && ((uintptr_t)dst & 15) == 0) {
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst));
      } else {
        for (int k = 0; k < 4 && n + k < p.N; ++k) dst[k] = src[k];
      }
    }
  } else if constexpr (EPI == EPI_STORE_F32 || EPI == EPI_ADD_F32 || EPI == EPI_STORE_ACT) {
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
      const int n = n0 + G::col_of(j);
      if (n >= p.N) continue;
      float sc = 1.f;
      if constexpr (sizeof(TB) == 1) sc = bf2f(p.sB[n]);
      const float bias = p.bias ? p.bias[n] : 0.f;
#pragma unroll
      for (int i = 0; i < G::FM; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + G::row_of(i, e);
          if (m >= p.M) continue;
          const float v = acc[i][j][e] * sc + bias;
          if constexpr (EPI == EPI_STORE_F32) {
            C32[(int64_t)m * p.ldc + n] = v;
          } else if constexpr (EPI == EPI_ADD_F32) {
            static_cast<float*>(p.C)[(int64_t)m * p.ldc + n] += v;
          } else {
            static_cast<TA*>(p.C)[(int64_t)m * p.ldc + n] = Elem<TA>::from_f(v);
          }
        }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int j = 0; j < G::FN; j += 2) {
      const int u = (wn * G::FN + j) >> 1;
      const int oc = n0 / 2 + u * 16 + (lane & 15);
      if (oc >= p.N) continue;
      float sg = 1.f, su = 1.f;
      if constexpr (sizeof(TB) == 1) { sg = bf2f(p.sB[oc]); su = bf2f(p.sB2[oc]); }
#pragma unroll
      for (int i = 0; i < G::FM; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + G::row_of(i, e);
          if (m >= p.M) continue;
          const float gt = acc[i][j][e] * sg, up = acc[i][j + 1][e] * su;
          const float a = silu(gt) * up;
          static_cast<TA*>(p.C)[(int64_t)m * p.ldc + oc] = Elem<TA>::from_f(a);
        }
    }
  } else if constexpr (EPI == EPI_QKV) {
    // rotation pairs (jj, jj + dh/2) sit in adjacent column blocks j, j + 1 of one lane; the
    // angle table holds (cos, sin) of row m's position for pair jj
    const int dh = p.dh, half_dh = dh / 2;
    const int head = n0 / dh, pb = (n0 % dh) / 2;
    // q / k rows of one head: the tile's BN columns are the dims pb + [0, BN/2) and half_dh + pb +
    // [0, BN/2).  Where the ring's LDS holds the tile (rows padded by 16 bytes), the rotated values
    // go there first, staged column c < BN/2 for dim pb + c and BN/2 + c for half_dh + pb + c, and
    // leave as whole 16-byte row chunks rather than one element per lane and store.
    constexpr int ROWB = BN * (int)sizeof(TA) + 16;
    constexpr int EPC = 16 / (int)sizeof(TA);            // elements per 16-byte chunk
    constexpr bool STAGED = qkv_stage_bytes<TA, BM, BN, EPI>() > 0;
    auto qk_row = [&](int m) -> TA* {
      if (head < p.Hq) return static_cast<TA*>(p.q_out) + ((int64_t)m * p.Hq + head) * dh;
      const int b = m / p.rows_per_canvas, ii = m - b * p.rows_per_canvas;
      return static_cast<TA*>(p.k_out) + (((int64_t)b * p.Hkv + head - p.Hq) * p.rows_per_canvas + ii) * dh;
    };
    if (head < p.Hq + p.Hkv) {           // q [rows][Hq][dh], canvas k [B][Hkv][n][dh], rotated
#pragma unroll
      for (int j = 0; j < G::FN; j += 2) {
        const int u = (wn * G::FN + j) >> 1;
        const int c = u * 16 + (lane & 15);              // pair index - pb
        const int jj = pb + c;                           // pair index in [0, dh/2)
#pragma unroll
        for (int i = 0; i < G::FM; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = G::row_of(i, e), m = m0 + r;
            if (m >= p.M) continue;
            float2 cs;
            if constexpr (CS_AHEAD) cs = cs_pre[((j >> 1) * G::FM + i) * 4 + e];
            else cs = p.rope[(int64_t)m * half_dh + jj];
            const float x1 = acc[i][j][e], x2 = acc[i][j + 1][e];
            const TA y1 = Elem<TA>::from_f(x1 * cs.x - x2 * cs.y), y2 = Elem<TA>::from_f(x2 * cs.x + x1 * cs.y);
            if constexpr (STAGED) {
              TA* row = reinterpret_cast<TA*>(lds + r * ROWB);
              row[c] = y1;
              row[BN / 2 + c] = y2;
            } else {
              TA* dst = qk_row(m);
              dst[jj] = y1;
              dst[jj + half_dh] = y2;
            }
          }
      }
      if constexpr (STAGED) {
        __syncthreads();
        constexpr int CPR = BN / EPC;                    // chunks per staged row
        for (int ch = threadIdx.x; ch < BM * CPR; ch += WM * WN * 64) {
          const int r = ch / CPR, col = (ch - r * CPR) * EPC, m = m0 + r;
          if (m >= p.M) continue;
          TA* dst = qk_row(m) + (col < BN / 2 ? pb + col : half_dh + pb + col - BN / 2);
          const char* src = lds + r * ROWB + col * (int)sizeof(TA);
          if (((uintptr_t)dst & 15) == 0) {
            *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
          } else {
            for (int k = 0; k < EPC; ++k) dst[k] = reinterpret_cast<const TA*>(src)[k];
          }
        }
      }
    } else if constexpr (v_stage_bytes<TA, BM, BN, EPI>() > 0) {
      // canvas v, d-major [B][Hkv][dh][v_ld], not rotated: the tile goes to LDS transposed (staged
      // row c < BN/2 holds dim pb + c, BN/2 + c dim half_dh + pb + c; four positions per 8- or
      // 16-byte write), then leaves as whole 16-byte chunks of consecutive positions of one dim
      constexpr int VROWB = BM * (int)sizeof(TA) + 16;
      TA* vbase = static_cast<TA*>(p.v_out) + (int64_t)(head - p.Hq - p.Hkv) * dh * p.v_ld;
      const int64_t bstride = (int64_t)p.Hkv * dh * p.v_ld;
#pragma unroll
      for (int j = 0; j < G::FN; ++j) {
        const int c = (j & 1) * (BN / 2) + ((wn * G::FN + j) >> 1) * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < G::FM; ++i) {
          char* dst = lds + c * VROWB + G::row_of(i, 0) * (int)sizeof(TA);
          if constexpr (sizeof(TA) == 2) {
            uint2 w;
            w.x = pack_bf2(acc[i][j][0], acc[i][j][1]);
            w.y = pack_bf2(acc[i][j][2], acc[i][j][3]);
            *reinterpret_cast<uint2*>(dst) = w;
          } else {
            *reinterpret_cast<f32x4_v*>(dst) = acc[i][j];
          }
        }
      }
      __syncthreads();
      constexpr int EPC = 16 / (int)sizeof(TA);
      constexpr int CPR = BM / EPC;                      // chunks per staged dim
      const bool whole = p.rows_per_canvas % EPC == 0 && (p.v_ld * (int)sizeof(TA)) % 16 == 0;
      for (int ch = threadIdx.x; ch < BN * CPR; ch += WM * WN * 64) {
        const int c = ch / CPR, r0 = (ch - c * CPR) * EPC, m = m0 + r0;
        if (m >= p.M) continue;
        const int d = c < BN / 2 ? pb + c : half_dh + pb + c - BN / 2;
        const TA* src = reinterpret_cast<const TA*>(lds + c * VROWB) + r0;
        const int b = m / p.rows_per_canvas, ii = m - b * p.rows_per_canvas;
        TA* dst = vbase + b * bstride + (int64_t)d * p.v_ld + ii;
        if (whole && m + EPC <= p.M && ((uintptr_t)dst & 15) == 0) {
          *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
        } else {
          for (int k = 0; k < EPC && m + k < p.M; ++k) {
            const int be = (m + k) / p.rows_per_canvas, ie = m + k - be * p.rows_per_canvas;
            vbase[be * bstride + (int64_t)d * p.v_ld + ie] = src[k];
          }
        }
      }
    } else {                             // canvas v, d-major [B][Hkv][dh][v_ld], not rotated
      TA* vbase = static_cast<TA*>(p.v_out) + (int64_t)(head - p.Hq - p.Hkv) * dh * p.v_ld;
      const int64_t bstride = (int64_t)p.Hkv * dh * p.v_ld;
#pragma unroll
      for (int j = 0; j < G::FN; ++j) {
        const int jj = pb + ((wn * G::FN + j) >> 1) * 16 + (lane & 15);
        const int d = jj + (j & 1) * half_dh;
#pragma unroll
        for (int i = 0; i < G::FM; ++i) {
          const int m = m0 + G::row_of(i, 0);      // rows m .. m + 3 of this lane
          const int b = m / p.rows_per_canvas, ii = m - b * p.rows_per_canvas;
          TA* dst = vbase + b * bstride + (int64_t)d * p.v_ld + ii;
          if (m + 3 < p.M && ii + 3 < p.rows_per_canvas && (p.rows_per_canvas & 3) == 0) {
            // four consecutive positions of one canvas: one 8-byte (bf16) / 16-byte (fp32) store
            if constexpr (sizeof(TA) == 2) {
              uint2 w;
              w.x = pack_bf2(acc[i][j][0], acc[i][j][1]);
              w.y = pack_bf2(acc[i][j][2], acc[i][j][3]);
              *reinterpret_cast<uint2*>(dst) = w;
            } else {
              *reinterpret_cast<f32x4_v*>(dst) = acc[i][j];
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int me = m + e;
              if (me >= p.M) continue;
              const int be = me / p.rows_per_canvas, ie = me - be * p.rows_per_canvas;
              vbase[be * bstride + (int64_t)d * p.v_ld + ie] = Elem<TA>::from_f(acc[i][j][e]);
            }
          }
        }
      }
    }
  }
}

// (cos, sin) of position pos0[b] + i for rotation pair jj: angle = pos * theta^(-2 jj / dh), taken
// in double and reduced to [0, 2 pi) before the single-precision sincos.  One entry per canvas row
// and pair: [rows][dh/2].
__global__ void rope_table_kernel(float2* tab, int rows, int rows_per_canvas, int half_dh, double log2_theta,
                                  const int32_t* plen, int max_prefix, int* status, const int32_t* gate) {
  if (gate_closed(gate)) return;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rows * half_dh) return;
  const int m = (int)(idx / half_dh), jj = (int)(idx - (int64_t)m * half_dh);
  const int b = m / rows_per_canvas, ii = m - b * rows_per_canvas;
  // a prefix length outside [0, max_prefix] is a caller error: flagged once per canvas, clamped
  if (ii == 0 && jj == 0 && status && (plen[b] < 0 || plen[b] > max_prefix)) atomicOr(status, 4);
  const double inv = exp2(-2.0 * jj / (2 * half_dh) * log2_theta);
  const double ang = (double)(prefix_of(plen, b, max_prefix) + ii) * inv;
  const double red = ang - 6.283185307179586 * floor(ang * 0.15915494309189535);
  float sn, cs;
  sincosf((float)red, &sn, &cs);
  tab[idx] = make_float2(cs, sn);
}

hipError_t launch_rope_table(float2* tab, int rows, int rows_per_canvas, int head_dim, double log2_theta,
                             const int32_t* plen, int max_prefix, int* status, hipStream_t s) {
  const int64_t n = (int64_t)rows * (head_dim / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, tab, rows, rows_per_canvas,
                     head_dim / 2, log2_theta, plen, max_prefix, status, launch_gate());
  return hipGetLastError();
}

// ---------------------------------------------------------------- grouped (MoE) ----------------
// One tile: rows [row0, row0 + rows) of A (through a_tok, or in order) times the weight rows from
// n0 (gate/up rows paired for SwiGLU) over the full K, then the tile's epilogue.
// W8A8: A holds e4m3 codes with the row scale sA[source row]; the SwiGLU product is stored in bf16.
template <class G, int BN, int WN, int EPI, class TA, class TB>
DG_DEV void grouped_tile(char* lds, const TA* A, int64_t lda, const int32_t* a_tok, int row0, int rows,
                         const TB* B, const TB* B2, int64_t ldb, const char* sB, const char* sB2, int64_t s_ld,
                         int N, int K, int n0, void* Cout, int64_t ldc, const float* sA) {
  using TO = std::conditional_t<is_fp8a_v<TA>, bf16_t, TA>;
  auto ascale = [&](int r) -> float {
    if constexpr (is_fp8a_v<TA>) return sA[a_tok ? a_tok[row0 + r] : row0 + r];
    else return 1.f;
  };
  auto arow = [&](int r) -> const TA* {
    if (r >= rows) return nullptr;
    const int src = a_tok ? a_tok[row0 + r] : row0 + r;
    return A + (int64_t)src * lda;
  };
  auto brow = [&](int r) -> const TB* {
    if constexpr (EPI == EPI_SWIGLU) {
      int u, half, c;
      paired_col<BN>(r, u, half, c);
      const int oc = n0 / 2 + u * 16 + c;
      if (oc >= N) return nullptr;
      return (half ? B2 : B) + (int64_t)oc * ldb;
    } else {
      const int n = n0 + r;
      return n < N ? B + (int64_t)n * ldb : nullptr;
    }
  };
  // MXFP4: the block-scale bytes of weight row r, paired like its weights
  auto srow = [&](int r) -> const uint8_t* {
    if constexpr (is_fp4_v<TB>) {
      if constexpr (EPI == EPI_SWIGLU) {
        int u, half, c;
        paired_col<BN>(r, u, half, c);
        const int oc = n0 / 2 + u * 16 + c;
        if (oc >= N) return nullptr;
        return reinterpret_cast<const uint8_t*>(half ? sB2 : sB) + (int64_t)oc * s_ld;
      } else {
        const int n = n0 + r;
        return n < N ? reinterpret_cast<const uint8_t*>(sB) + (int64_t)n * s_ld : nullptr;
      }
    } else {
      return nullptr;
    }
  };
  G g;
  g.setup(arow, brow, srow);
  f32x4_v acc[G::FM][G::FN];
  g.run(lds, K, acc);

  // Epilogue.  The output tile goes through LDS (the ring is idle once the K loop has ended) so
  // that the stores are whole 16-byte chunks of its rows, where a lane's own values (4 rows of one
  // column per fragment) would give 2- or 4-byte stores scattered over four rows, and they are
  // streaming stores; a tile whose rows do not fit the ring's bytes stores directly.
  const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) % WN;
  constexpr int NOUT = EPI == EPI_SWIGLU ? BN / 2 : BN;            // output columns of the tile
  using TS = std::conditional_t<EPI == EPI_STORE_F32, float, TO>;
  constexpr int ROWB = NOUT * (int)sizeof(TS) + 16;                 // padded LDS row
  constexpr bool STAGED = G::TILE_M * ROWB <= G::LDS_BYTES;
  const int c0 = EPI == EPI_SWIGLU ? n0 / 2 : n0;                   // first output column
  if constexpr (STAGED) __syncthreads();                            // every wave is done with the ring
  auto put = [&](int r, int cl, float v) {
    if constexpr (STAGED) *reinterpret_cast<TS*>(lds + r * ROWB + cl * (int)sizeof(TS)) = Elem<TS>::from_f(v);
    else static_cast<TS*>(Cout)[(int64_t)(row0 + r) * ldc + c0 + cl] = Elem<TS>::from_f(v);
  };
  if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int j = 0; j < G::FN; j += 2) {
      const int u = (wn * G::FN + j) >> 1;
      const int cl = u * 16 + (lane & 15), oc = c0 + cl;
      if (oc >= N) continue;
      float sg = 1.f, su = 1.f;
      if constexpr (is_fp8_v<TB>) {
        sg = bf2f(reinterpret_cast<const bf16_t*>(sB)[oc]);
        su = bf2f(reinterpret_cast<const bf16_t*>(sB2)[oc]);
      }
#pragma unroll
      for (int i = 0; i < G::FM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = G::row_of(i, q);
          if (r >= rows) continue;
          const float sa = ascale(r);
          const float gt = acc[i][j][q] * sg * sa, up = acc[i][j + 1][q] * su * sa;
          put(r, cl, silu(gt) * up);
        }
    }
  } else {  // EPI_STORE_F32 (fp32 rows) or EPI_STORE_ACT (rows of the activation type)
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
      const int cl = G::col_of(j), n = c0 + cl;
      if (n >= N) continue;
      float sc = 1.f;
      if constexpr (is_fp8_v<TB>) sc = bf2f(reinterpret_cast<const bf16_t*>(sB)[n]);
#pragma unroll
      for (int i = 0; i < G::FM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = G::row_of(i, q);
          if (r >= rows) continue;
          put(r, cl, acc[i][j][q] * sc * ascale(r));
        }
    }
  }
  if constexpr (STAGED) {
    __syncthreads();
    constexpr int EPC = 16 / (int)sizeof(TS);                       // elements per 16-byte chunk
    constexpr int CH = NOUT / EPC;                                   // chunks per tile row
    const int ncols = min(NOUT, N - c0);
    for (int idx = threadIdx.x; idx < rows * CH; idx += blockDim.x) {
      const int r = idx / CH, ch = idx - r * CH, cl = ch * EPC;
      if (cl >= ncols) continue;
      TS* dst = static_cast<TS*>(Cout) + (int64_t)(row0 + r) * ldc + c0 + cl;
      const char* src = lds + r * ROWB + ch * 16;
      if (cl + EPC <= ncols && ((uintptr_t)dst & 15) == 0) {
        // streaming stores: the rows go out to memory instead of staying dirty in this XCD's L2
        // (the next launch reads them, from any XCD)
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst));
      } else {
        for (int e = 0; e < EPC && cl + e < ncols; ++e) dst[e] = reinterpret_cast<const TS*>(src)[e];
      }
    }
  }
}

// 1-D grid.  Blocks [0, sh_blocks): the shared expert over all rows in row order, in row tiles of
// BMS rows (every shared weight tile passes through a CU once per row tile), first (its tiles are
// the longest, so they go before the routed tiles rather than into the tail); the n_sh_items row
// tiles of one column tile get ids congruent mod 8 (one XCD, one L2 copy of that weight tile).
// Blocks [sh_blocks, ...): routed tiles of BM rows; work item w < *n_items: expert e = work[2w],
// first row m0 = work[2w+1] of that expert's rows [offsets[e], offsets[e] + counts[e]) in grouped
// order.  XCDR = 0: block - sh_blocks = item * nt_r + column tile.  XCDR = 1 (large experts cut
// into many items): the items fall into groups of XG; unit u = group * nt_r + column tile holds
// that column tile of the group's XG items, and all XG blocks of unit u sit on XCD u mod 8 (block
// id mod 8).  An expert's items are consecutive, so its items in one group read each weight tile
// on one XCD and share its L2 copy, while consecutive units still cycle over all 8 XCDs; an
// expert's last item, when it holds BM/2 rows or fewer, runs on a BM/2-row tile.  The dynamic LDS
// holds the larger of the tile shapes' rings.
constexpr int XG = 16;

template <class TA, class TB, int BM, int BMS, int BN, int WM, int WN, int EPI, int NS = 0, int QNS = 6, int XCDR = 0>
__global__ __launch_bounds__(WM * WN * 64) void gemm_grouped_kernel(GroupedArgs p) {
  if (gate_closed(p.gate)) return;
  using G = GroupTileFor<TA, TB, BM, BN, WM, WN, NS, QNS>;
  using GS = GroupTileFor<TA, TB, BMS, BN, WM, WN, NS, QNS>;
  extern __shared__ __align__(16) char lds[];
  const int id = blockIdx.x;
  if (id >= p.sh_blocks) {
    const int rid = id - p.sh_blocks;      // sh_blocks is a multiple of 8: rid and id share an XCD
    int item, col;
    if constexpr (XCDR) {
      const int k = rid >> 3, u = 8 * (k / XG) + (rid & 7), g = u / p.nt_r;
      col = u - g * p.nt_r;
      item = g * XG + k % XG;
    } else {
      item = rid / p.nt_r;
      col = rid - item * p.nt_r;
    }
    if (item >= *p.n_items) return;
    const int e = p.work[2 * item], m0 = p.work[2 * item + 1], rows = min(BM, p.counts[e] - m0);
    if constexpr (XCDR && !is_fp8a_v<TA>) {
      if (rows <= BM / 2) {
        using GH = GroupTileFor<TA, TB, BM / 2, BN, WM, WN, NS, QNS>;
        grouped_tile<GH, BN, WN, EPI>(lds, static_cast<const TA*>(p.A), p.lda, p.a_tok, p.offsets[e] + m0, rows,
                                      static_cast<const TB*>(p.B) + (int64_t)e * p.b_estride,
                                      p.B2 ? static_cast<const TB*>(p.B2) + (int64_t)e * p.b_estride : nullptr, p.ldb,
                                      p.sB ? static_cast<const char*>(p.sB) + (int64_t)e * p.s_estride : nullptr,
                                      p.sB2 ? static_cast<const char*>(p.sB2) + (int64_t)e * p.s_estride : nullptr,
                                      p.s_ld, p.N, p.K, col * BN, p.C, p.ldc, p.sA);
        return;
      }
    }
    grouped_tile<G, BN, WN, EPI>(lds, static_cast<const TA*>(p.A), p.lda, p.a_tok, p.offsets[e] + m0,
                                 rows, static_cast<const TB*>(p.B) + (int64_t)e * p.b_estride,
                                 p.B2 ? static_cast<const TB*>(p.B2) + (int64_t)e * p.b_estride : nullptr, p.ldb,
                                 p.sB ? static_cast<const char*>(p.sB) + (int64_t)e * p.s_estride : nullptr,
                                 p.sB2 ? static_cast<const char*>(p.sB2) + (int64_t)e * p.s_estride : nullptr,
                                 p.s_ld, p.N, p.K, col * BN, p.C, p.ldc, p.sA);
  } else {
    const int j = id >> 3;
    const int it = j % p.n_sh_items, nt = (j / p.n_sh_items) * 8 + (id & 7);
    if (nt >= p.nt_s) return;
    grouped_tile<GS, BN, WN, EPI>(lds, static_cast<const TA*>(p.shA), p.sh_lda, nullptr, it * BMS,
                                  min(BMS, p.sh_rows - it * BMS), static_cast<const TB*>(p.shB),
                                  static_cast<const TB*>(p.shB2), p.sh_ldb, static_cast<const char*>(p.sh_sB),
                                  static_cast<const char*>(p.sh_sB2), p.sh_s_ld, p.shN, p.shK, nt * BN,
                                  p.shC, p.sh_ldc, p.sh_sA);
  }
}

// ---------------------------------------------------------------- launchers --------------------
template <class TA, class TB, int BM, int BN, int WM, int WN, int EPI, int MAP, int NS = 0, int KPS = 1>
static hipError_t launch_dense_t(DenseArgs a, int n_eff, hipStream_t s) {
  using G = TileFor<TA, TB, BM, BN, WM, WN, NS, KPS>;
  a.n_mt = (a.M + BM - 1) / BM;
  a.n_nt = (n_eff + BN - 1) / BN;
  if (a.ksplit < 1) a.ksplit = 1;
  if (a.K % (a.ksplit * G::KT * KPS)) return hipErrorInvalidValue;
  dim3 grid(a.n_mt * ((a.n_nt + 7) / 8 * 8), a.ksplit);
  a.gate = launch_gate();
  constexpr size_t LDS = dense_lds_bytes<G, TA, BM, BN, EPI>();
  static const hipError_t attr = allow_lds(gemm_dense_kernel<TA, TB, BM, BN, WM, WN, EPI, MAP, NS, KPS>, LDS);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((gemm_dense_kernel<TA, TB, BM, BN, WM, WN, EPI, MAP, NS, KPS>), grid, dim3(WM * WN * 64),
                     LDS, s, a);
  return hipGetLastError();
}

// Tiles.  Up to 256 rows: 128-row tiles (64 for tiny M) so each weight tile is read by at most
// two blocks, 64 (32 for SwiGLU) columns so enough blocks stream the weights; paired epilogues
// keep an even count of 16-column blocks per wave.  Above 256 rows: 128 x 128 tiles, except narrow
// outputs; with bf16 weights 256 x 128 tiles of 8 waves (3-stage ring): half the weight re-reads
// per output.  QKV up to
// 256 rows: 8 waves on the 128 x 64 tile with a 4-stage ring (one block per CU; 8 waves keep more
// loads and MFMAs in flight than 4).  Narrow outputs (the router, N <= 256) above 64 rows: 64 x 32
// tiles at any row count (few split-K parts where rows alone give enough blocks).
template <class TA, class TB, int EPI, int MAP>
static hipError_t dense_pick(const DenseArgs& a, int n_eff, hipStream_t s) {
  const bool small = a.M <= 64;
  if constexpr (MAP == MAP_ROPE) {
    // a column tile must stay inside one head; above 256 rows bf16 weights take 256 x 256 tiles
    // (128 x 64 per wave, two 64 KB ring stages) when a head spans 256 columns
    if (a.M > 256 && a.dh >= 128) {
      if constexpr (sizeof(TB) == 1) return launch_dense_t<TA, TB, 128, 128, 2, 2, EPI, MAP>(a, n_eff, s);
      else {
        if (a.dh % 256 == 0) return launch_dense_t<TA, TB, 256, 256, 2, 4, EPI, MAP, 2>(a, n_eff, s);
        return launch_dense_t<TA, TB, 256, 128, 4, 2, EPI, MAP, 3>(a, n_eff, s);
      }
    }
    if (small) return launch_dense_t<TA, TB, 64, 64, 2, 2, EPI, MAP>(a, n_eff, s);
    if constexpr (sizeof(TB) == 1) return launch_dense_t<TA, TB, 128, 64, 2, 2, EPI, MAP>(a, n_eff, s);
    else return launch_dense_t<TA, TB, 128, 64, 4, 2, EPI, MAP, 4>(a, n_eff, s);
  } else if constexpr (MAP == MAP_SWIGLU) {
    if (a.M > 256) return launch_dense_t<TA, TB, 128, 128, 2, 2, EPI, MAP>(a, n_eff, s);
    if (small) return launch_dense_t<TA, TB, 64, 32, 4, 1, EPI, MAP>(a, n_eff, s);
    return launch_dense_t<TA, TB, 128, 32, 4, 1, EPI, MAP>(a, n_eff, s);
  } else {
    if (small) return launch_dense_t<TA, TB, 64, 64, 2, 2, EPI, MAP>(a, n_eff, s);
    if (a.N <= 256) return launch_dense_t<TA, TB, 64, 32, 4, 1, EPI, MAP>(a, n_eff, s);
    if constexpr (sizeof(TB) == 2) {
      // a vocabulary-long contraction (the self-conditioning product, K = V) over one canvas: every
      // row in one 256 x 256 tile of 8 waves, split over K, so each K slice of the probabilities is
      // read once per 256 output columns and the embedding once
      if (a.K >= 16384 && a.M <= 256) return launch_dense_t<TA, TB, 256, 256, 2, 4, EPI, MAP, 2>(a, n_eff, s);
    }
    if (a.M > 256) {
      // bf16 weights: 128 x 192 tiles on 8 waves (64 x 48 per wave): at 2048 x 2816 (the attention
      // output projection of 8 canvases) 240 blocks where 256 x 128 tiles give 176 of 256 CUs
      if constexpr (sizeof(TB) == 1) return launch_dense_t<TA, TB, 128, 128, 2, 2, EPI, MAP>(a, n_eff, s);
      else return launch_dense_t<TA, TB, 128, 192, 2, 4, EPI, MAP, 3>(a, n_eff, s);
    }
    if constexpr (sizeof(TB) != 1) {
      // wide outputs up to 256 rows (the attention output projection): 8 waves, two K tiles per
      // ring stage, about one block per CU
      constexpr int KSTEP = 2 * 128 / (int)sizeof(TA);
      if ((a.K / a.ksplit) % KSTEP == 0) return launch_dense_t<TA, TB, 128, 64, 4, 2, EPI, MAP, 3, 2>(a, n_eff, s);
    }
    return launch_dense_t<TA, TB, 128, 64, 2, 2, EPI, MAP>(a, n_eff, s);
  }
}

template <class TA, class TB>
static hipError_t dense_dispatch(const DenseArgs& a, hipStream_t s) {
  if (a.ksplit > 1 && a.epi != EPI_STORE_F32) return hipErrorInvalidValue;
  switch (a.epi) {
    case EPI_STORE_F32: return dense_pick<TA, TB, EPI_STORE_F32, MAP_PLAIN>(a, a.N, s);
    case EPI_ADD_F32: return dense_pick<TA, TB, EPI_ADD_F32, MAP_PLAIN>(a, a.N, s);
    case EPI_STORE_ACT: return dense_pick<TA, TB, EPI_STORE_ACT, MAP_PLAIN>(a, a.N, s);
    case EPI_SWIGLU: return dense_pick<TA, TB, EPI_SWIGLU, MAP_SWIGLU>(a, 2 * a.N, s);
    case EPI_QKV: return dense_pick<TA, TB, EPI_QKV, MAP_ROPE>(a, a.N, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dense(const DenseArgs& a, int act_bf16, int w_kind, hipStream_t s) {
  if (!act_bf16) return dense_dispatch<float, float>(a, s);
  if (w_kind == W_FP8) {
    if (a.epi == EPI_QKV) return hipErrorInvalidValue;
    return dense_dispatch<bf16_t, fp8_t>(a, s);
  }
  return dense_dispatch<bf16_t, bf16_t>(a, s);
}

template <class TA, class TB, int BM, int BMS, int BN, int WM, int WN, int EPI, int NS = 0, int QNS = 6, int XCDR = 0>
static hipError_t launch_grouped_t(GroupedArgs a, int n_eff, int sh_eff, int max_items, hipStream_t s) {
  using G = GroupTileFor<TA, TB, BM, BN, WM, WN, NS, QNS>;
  using GS = GroupTileFor<TA, TB, BMS, BN, WM, WN, NS, QNS>;
  constexpr size_t LDS = G::LDS_BYTES > GS::LDS_BYTES ? G::LDS_BYTES : GS::LDS_BYTES;
  a.nt_r = (n_eff + BN - 1) / BN;
  a.nt_s = (sh_eff + BN - 1) / BN;
  a.n_sh_items = a.shB ? (a.sh_rows + BMS - 1) / BMS : 0;
  a.sh_blocks = (a.nt_s + 7) / 8 * a.n_sh_items * 8;
  const int units = (max_items + XG - 1) / XG * a.nt_r;
  const int blocks = a.sh_blocks + (XCDR ? (units + 7) / 8 * 8 * XG : max_items * a.nt_r);
  if (blocks == 0) return hipSuccess;
  // the W8A8 engine takes a K ending half-way through its 128-element stage
  constexpr int KQ = is_fp8a_v<TA> ? 64 : G::KT, KQS = is_fp8a_v<TA> ? 64 : GS::KT;
  if (a.K % KQ || (a.shB && a.shK % KQS)) return hipErrorInvalidValue;
  a.gate = launch_gate();
  static const hipError_t attr = allow_lds(gemm_grouped_kernel<TA, TB, BM, BMS, BN, WM, WN, EPI, NS, QNS, XCDR>, LDS);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((gemm_grouped_kernel<TA, TB, BM, BMS, BN, WM, WN, EPI, NS, QNS, XCDR>), dim3(blocks), dim3(WM * WN * 64),
                     LDS, s, a);
  return hipGetLastError();
}

// Routed tiles of GROUP_BM rows x 128 weight rows on 4 waves.  Weights of the activation type: the
// shared expert in tiles of 4 x GROUP_BM rows on a two-stage ring (32 KB stages: the launch's LDS
// stays the routed ring's 80 KB, two blocks per CU; its few long blocks start first); fp8 / MXFP4 weights (raw codes on the ring, widened in registers):
// GROUP_BM-row tiles for both.
// Batched canvases (experts averaging 64 rows or more): 128-row tiles for the routed experts and
// the shared expert, so a popular expert's weights stream once per 128 rows rather than per 32.
// bf16 and fp8 on 8 waves with 256-column tiles (the activation rows, which outweigh fp8 weights
// per stage, are re-read by half as many column tiles),
// MXFP4 on the 4-wave register-staged engine (128 columns).
template <class TA, class TB, int EPI>
static hipError_t grouped_wide(const GroupedArgs& a, int n_eff, int sh_eff, int max_items, hipStream_t s) {
  constexpr int W = GROUP_BM_WIDE;
  if constexpr (is_fp4_v<TB>) return launch_grouped_t<TA, TB, W, W, 128, 2, 2, EPI, 0, 6, 1>(a, n_eff, sh_eff, max_items, s);
  else if constexpr (is_fp8_v<TB>) {
    // fp8 rings: 3 stages (96 KB, one block per CU) for gate/up over K = d_model; 2 stages (64 KB,
    // two blocks per CU, which hide each other's short K loops) for down over K = expert width
    constexpr int Q = EPI == EPI_SWIGLU ? 3 : 2;
    return launch_grouped_t<TA, TB, W, W, 256, 2, 4, EPI, 3, Q, 1>(a, n_eff, sh_eff, max_items, s);
  } else return launch_grouped_t<TA, TB, W, W, 256, 2, 4, EPI, 3, 4, 1>(a, n_eff, sh_eff, max_items, s);
}

template <class TA, class TB>
static hipError_t grouped_dispatch(const GroupedArgs& a, int max_items, hipStream_t s) {
  if (a.bm == GROUP_BM_WIDE) {
    if (a.epi == EPI_SWIGLU) return grouped_wide<TA, TB, EPI_SWIGLU>(a, 2 * a.N, 2 * a.shN, max_items, s);
    return grouped_wide<TA, TB, EPI_STORE_ACT>(a, a.N, a.shN, max_items, s);
  }
  if (a.bm != GROUP_BM) return hipErrorInvalidValue;
  if constexpr (sizeof(TB) == 1) {
    if (a.epi == EPI_SWIGLU)
      return launch_grouped_t<TA, TB, GROUP_BM, GROUP_BM, 128, 1, 4, EPI_SWIGLU>(a, 2 * a.N, 2 * a.shN, max_items, s);
    return launch_grouped_t<TA, TB, GROUP_BM, GROUP_BM, 128, 1, 4, EPI_STORE_ACT>(a, a.N, a.shN, max_items, s);
  } else {
    if (a.epi == EPI_SWIGLU)
      return launch_grouped_t<TA, TB, GROUP_BM, 4 * GROUP_BM, 128, 1, 4, EPI_SWIGLU>(a, 2 * a.N, 2 * a.shN, max_items, s);
    return launch_grouped_t<TA, TB, GROUP_BM, 4 * GROUP_BM, 128, 1, 4, EPI_STORE_ACT>(a, a.N, a.shN, max_items, s);
  }
}

// W8A8: routed tiles of GROUP_BM_Q8 rows (four waves side by side) or, for batched canvases, 128 x 256
// tiles on 8 waves (2 x 4); shared-expert tiles of 128 rows; block-scaled fp8 MFMA throughout.
// Rings of 128-element stages: 3 x 48 KB for the batched gate/up (one block per CU, K = d_model);
// the batched down (K = expert width: six stages) on 128 x 128 tiles, 2 x 32 KB, two blocks per CU
// to hide each other's ring fill (measured at eight canvases: 199 us per launch against 264 us
// for 128 x 256 tiles on one block per CU); 3 stages of 24 / 32 KB otherwise.
static hipError_t grouped_q8(const GroupedArgs& a, int max_items, hipStream_t s) {
  if (a.bm == GROUP_BM_WIDE) {
    constexpr int W = GROUP_BM_WIDE;
    if (a.epi == EPI_SWIGLU)
      return launch_grouped_t<fp8a_t, fp8_t, W, W, 256, 2, 4, EPI_SWIGLU, 0, 3, 1>(a, 2 * a.N, 2 * a.shN, max_items, s);
    return launch_grouped_t<fp8a_t, fp8_t, W, W, 128, 2, 4, EPI_STORE_ACT, 0, 2, 1>(a, a.N, a.shN, max_items, s);
  }
  if (a.bm != GROUP_BM_Q8) return hipErrorInvalidValue;
  if (a.epi == EPI_SWIGLU)
    return launch_grouped_t<fp8a_t, fp8_t, GROUP_BM_Q8, 128, 128, 1, 4, EPI_SWIGLU, 0, 3>(a, 2 * a.N, 2 * a.shN,
                                                                                       max_items, s);
  return launch_grouped_t<fp8a_t, fp8_t, GROUP_BM_Q8, 128, 128, 1, 4, EPI_STORE_ACT, 0, 3>(a, a.N, a.shN, max_items, s);
}

hipError_t launch_grouped(const GroupedArgs& a, int act_bf16, int w_kind, int max_items, hipStream_t s) {
  if (a.epi != EPI_SWIGLU && a.epi != EPI_STORE_ACT) return hipErrorInvalidValue;
  if (w_kind == W_FP8A8) return grouped_q8(a, max_items, s);
  if (!act_bf16) return grouped_dispatch<float, float>(a, max_items, s);
  if (w_kind == W_FP8) return grouped_dispatch<bf16_t, fp8_t>(a, max_items, s);
  if (w_kind == W_MXFP4) return grouped_dispatch<bf16_t, fp4x2_t>(a, max_items, s);
  return grouped_dispatch<bf16_t, bf16_t>(a, max_items, s);
}

}  // namespace dg
