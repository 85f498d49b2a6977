// Canvas attention with fp32 activations (bf16 activations take flash_kernel): every query row
// of the canvas attends to the visible prefix cache slots and to all canvas keys (bidirectional,
// [TR §아키텍처와 블록 자기회귀 생성]); the same kernel with `causal` set serves the causal
// encoder (prefill), with the sliding window on local layers.
//
// Work item = (canvas b, KV head g, 64 query rows of the G = Hq/Hkv heads sharing g, key split).
// Each wave owns 16 query rows.  Per 64-key tile (K row-major and V transposed in LDS):
//   S^T = K . Q^T     (A = K from LDS, B = Q^T from registers)   -> lane holds one query column
//   online softmax    (per lane; row max over the 4 lanes of a column by two xor-shuffles)
//   O^T += V^T . P^T  (A = V^T from LDS, B = P^T straight from the S^T registers)
// so probabilities never leave registers and the row rescale is lane-local.  With one split the
// kernel normalises and writes o; otherwise it writes (O, m, l) partials merged by
// attn_merge_kernel in split order.
#include "common.h"
#include "internal.h"

namespace dg {

constexpr int AT_KEYS = 64;

template <class T, int DH>
struct AttnCfg {
  static constexpr int ESZ = sizeof(T);
  static constexpr int EPL = 16 / ESZ;                    // elements per 16-byte fragment
  static constexpr int KPF = Mfma<T>::K_PER_FRAG;         // k per fragment (32 bf16, 16 f32)
  static constexpr int NCH = DH / KPF;                    // fragments along head_dim
  static constexpr int K_STRIDE = DH * ESZ + 16;          // bytes per K row in LDS
  static constexpr int V_STRIDE = AT_KEYS * ESZ + 16;     // bytes per V^T row (one d) in LDS
  static constexpr int LDS_K = AT_KEYS * K_STRIDE;
  static constexpr int LDS_V = DH * V_STRIDE;
  static constexpr int LDS = LDS_K + LDS_V;
  static constexpr int CH_ROW = DH * ESZ / 16;            // 16-byte chunks per key row
  static constexpr int CHUNKS = AT_KEYS * CH_ROW / 256;   // per thread, per tensor
  static constexpr int DB = DH / 16;                      // 16-row blocks of head_dim
};

template <class T>
DG_DEV void put_elem(char* p, float v);
template <> DG_DEV void put_elem<bf16_t>(char* p, float v) { *reinterpret_cast<bf16_t*>(p) = f2bf(v); }
template <> DG_DEV void put_elem<float>(char* p, float v) { *reinterpret_cast<float*>(p) = v; }

template <class T, int DH>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs p) {
  if (gate_closed(p.gate)) return;
  using C = AttnCfg<T, DH>;
  extern __shared__ __align__(16) char lds[];
  char* lk = lds;
  char* lv = lds + C::LDS_K;
  const int G = p.Hq / p.Hkv;
  const int mrows = G * p.n;                     // query rows sharing one KV head
  const int qtiles = (mrows + 63) / 64;
  int id = blockIdx.x;
  const int split = id % p.splits; id /= p.splits;
  const int qt = id % qtiles; id /= qtiles;
  const int g = id % p.Hkv;
  const int b = id / p.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int P = prefix_of(p.plen, b, p.max_prefix);
  const bool causal = p.seq_causal ? p.seq_causal[b] != 0 : p.causal != 0;
  const int np = p.is_global ? P : min(P, p.window);       // visible prefix slots
  const int nkeys = np + p.n;
  const int k_begin = split * p.keys_per_split;
  const int k_end = min(nkeys, k_begin + p.keys_per_split);

  // this lane's query column
  const int mq = qt * 64 + wave * 16 + (lane & 15);
  const bool q_ok = mq < mrows;
  const int hj = q_ok ? mq / p.n : 0, qi = q_ok ? mq - hj * p.n : 0;
  const int head = g * G + hj;
  const int qpos = P + qi;
  const int kg = lane >> 4;

  u32x4 qf[C::NCH];
  {
    const char* qrow = static_cast<const char*>(p.q) + (((int64_t)(b * p.n + qi) * p.Hq + head) * DH) * C::ESZ;
#pragma unroll
    for (int c = 0; c < C::NCH; ++c)
      qf[c] = q_ok ? *reinterpret_cast<const u32x4*>(qrow + (c * C::KPF + kg * C::EPL) * C::ESZ)
                   : u32x4{0, 0, 0, 0};
  }

  f32x4_v acc[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) acc[i] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_lane = 0.f;

  const char* kc = static_cast<const char*>(p.kc) + ((int64_t)(b * p.Hkv + g) * p.cap) * DH * C::ESZ;
  const char* vc = static_cast<const char*>(p.vc) + ((int64_t)(b * p.Hkv + g) * p.cap) * DH * C::ESZ;  // [dh][cap]
  const char* kn = static_cast<const char*>(p.kn) + ((int64_t)(b * p.Hkv + g) * p.n) * DH * C::ESZ;
  const char* vn = static_cast<const char*>(p.vn) + ((int64_t)(b * p.Hkv + g) * p.vn_ld) * DH * C::ESZ;  // [dh][vn_ld]
  const int ring_lo = max(0, P - p.window);

  // ---- staging: K rows and V^T rows of one 64-key tile go global -> registers (all loads
  // issued back to back, for the next tile while the current one is computed) -> LDS.  Keys
  // past the split's end are clamped to its last key: they are masked out of the softmax (P = 0).
  // K: chunk q -> key q / CH_ROW, 16-byte column q % CH_ROW (coalesced rows).
  // V: task q -> head-dim row q / 16 and keys 4 * (q % 16) .. + 3, read from the d-major value
  //    rows (prefix slots, then canvas keys) and written to LDS as one 4-key vector.
  constexpr int VTASKS = DH * (AT_KEYS / 4);
  constexpr int VT = VTASKS / 256;                           // V tasks per thread
  static_assert(VTASKS % 256 == 0, "V tasks");
  u32x4 kreg[C::CHUNKS], vreg[VT];
  auto key_row = [&](int kk) -> const char* {
    kk = min(kk, k_end - 1);
    return kk < np ? kc + (int64_t)kk * DH * C::ESZ : kn + (int64_t)(kk - np) * DH * C::ESZ;
  };
  auto val_elem = [&](int kk, int d) -> const char* {
    kk = min(kk, k_end - 1);
    return kk < np ? vc + ((int64_t)d * p.cap + kk) * C::ESZ : vn + ((int64_t)d * p.vn_ld + (kk - np)) * C::ESZ;
  };
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int it = 0; it < C::CHUNKS; ++it) {
      const int q = threadIdx.x + 256 * it;
      kreg[it] = *reinterpret_cast<const u32x4*>(key_row(k0 + q / C::CH_ROW) + (q % C::CH_ROW) * 16);
    }
#pragma unroll
    for (int it = 0; it < VT; ++it) {
      const int q = threadIdx.x + 256 * it;
      const int d = q >> 4, kq = q & 15;
      uint32_t e[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const char* src = val_elem(k0 + 4 * kq + m, d);
        e[m] = C::ESZ == 2 ? (uint32_t)*reinterpret_cast<const uint16_t*>(src) : *reinterpret_cast<const uint32_t*>(src);
      }
      if constexpr (C::ESZ == 2) vreg[it] = u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), 0, 0};
      else vreg[it] = u32x4{e[0], e[1], e[2], e[3]};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < C::CHUNKS; ++it) {
      const int q = threadIdx.x + 256 * it;
      *reinterpret_cast<u32x4*>(lk + (q / C::CH_ROW) * C::K_STRIDE + (q % C::CH_ROW) * 16) = kreg[it];
    }
#pragma unroll
    for (int it = 0; it < VT; ++it) {
      const int q = threadIdx.x + 256 * it;
      const int d = q >> 4, kq = q & 15;
      char* dst = lv + d * C::V_STRIDE + kq * 4 * C::ESZ;
      if constexpr (C::ESZ == 2) *reinterpret_cast<uint2*>(dst) = make_uint2(vreg[it].x, vreg[it].y);
      else *reinterpret_cast<u32x4*>(dst) = vreg[it];
    }
  };

  if (k_begin < k_end) load_tile(k_begin);
  for (int k0 = k_begin; k0 < k_end; k0 += AT_KEYS) {
    __syncthreads();                  // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (k0 + AT_KEYS < k_end) load_tile(k0 + AT_KEYS);   // in flight during this tile's math

    // ---- S^T = K . Q^T --------------------------------------------------------------------
    f32x4_v s[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      s[nb] = f32x4_v{0.f, 0.f, 0.f, 0.f};
      const char* krow = lk + (nb * 16 + (lane & 15)) * C::K_STRIDE + kg * 16;
#pragma unroll
      for (int c = 0; c < C::NCH; ++c)
        Mfma<T>::mma(s[nb], *reinterpret_cast<const u32x4*>(krow + c * C::KPF * C::ESZ), qf[c]);
    }
    // ---- scale, mask, online softmax --------------------------------------------------------
    float mt = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kk = k0 + nb * 16 + 4 * kg + j;
        bool vis = kk < k_end;
        if (causal && vis) {
          int kpos;
          if (kk >= np) kpos = P + (kk - np);
          else kpos = p.is_global ? kk : ring_lo + ((kk - ring_lo) % p.window + p.window) % p.window;
          vis = kpos <= qpos && (p.is_global || qpos - kpos < p.window);
        }
        const float v = vis ? s[nb][j] * p.scale_log2 : -INFINITY;
        s[nb][j] = v;
        mt = fmaxf(mt, v);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = (m_new == -INFINITY || m_run == -INFINITY) ? (m_run == -INFINITY ? 0.f : 1.f)
                                                                 : exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e = (s[nb][j] == -INFINITY) ? 0.f : exp2f(s[nb][j] - m_new);
        s[nb][j] = e;
        psum += e;
      }
    l_lane = l_lane * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < C::DB; ++i) acc[i] *= alpha;

    // ---- O^T += V^T . P^T --------------------------------------------------------------------
    if constexpr (C::ESZ == 2) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        u32x4 pb;
        pb.x = pack_bf2(s[2 * c2][0], s[2 * c2][1]);
        pb.y = pack_bf2(s[2 * c2][2], s[2 * c2][3]);
        pb.z = pack_bf2(s[2 * c2 + 1][0], s[2 * c2 + 1][1]);
        pb.w = pack_bf2(s[2 * c2 + 1][2], s[2 * c2 + 1][3]);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const char* vrow = lv + (db * 16 + (lane & 15)) * C::V_STRIDE;
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow + (32 * c2 + 4 * kg) * 2);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + (32 * c2 + 16 + 4 * kg) * 2);
          const u32x4 va = {lo.x, lo.y, hi.x, hi.y};
          Mfma<T>::mma(acc[db], va, pb);
        }
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const u32x4 pb = {__float_as_uint(s[nb][0]), __float_as_uint(s[nb][1]),
                          __float_as_uint(s[nb][2]), __float_as_uint(s[nb][3])};
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const char* vrow = lv + (db * 16 + (lane & 15)) * C::V_STRIDE;
          const u32x4 va = *reinterpret_cast<const u32x4*>(vrow + (16 * nb + 4 * kg) * 4);
          Mfma<T>::mma(acc[db], va, pb);
        }
      }
    }
  }

  // ---- finish: total l over the 4 lanes of the column ----------------------------------------
  float l = l_lane + __shfl_xor(l_lane, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (!q_ok) return;
  const int64_t row = (int64_t)b * p.n + qi;
  if (p.splits == 1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    char* o = static_cast<char*>(p.out) + ((row * p.Hq + head) * DH) * C::ESZ;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) put_elem<T>(o + (db * 16 + 4 * kg + j) * C::ESZ, acc[db][j] * inv);
  } else {
    float* o = p.part_o + (((int64_t)split * p.B * p.n + row) * p.Hq + head) * DH;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
      *reinterpret_cast<f32x4_v*>(o + db * 16 + 4 * kg) = acc[db];
    if (kg == 0) {
      float* ml = p.part_ml + (((int64_t)split * p.B * p.n + row) * p.Hq + head) * 2;
      ml[0] = m_run;
      ml[1] = l;
    }
  }
}

// merge split partials in split order: o = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M), where
// the fp32 kernel stores the sums O_s (fp32) and the bf16 kernel the normalised O_s / l_s (IEEE
// half).  S (the split count) is a compile-time constant, so every partial of a thread is loaded
// before the sums and nothing beyond the S partials is read.
constexpr int MERGE_MAX = 16;
template <class T>
DG_DEV void put4(T* dst, f32x4_v v);
template <>
DG_DEV void put4<float>(float* dst, f32x4_v v) { *reinterpret_cast<f32x4_v*>(dst) = v; }
template <>
DG_DEV void put4<bf16_t>(bf16_t* dst, f32x4_v v) {
  uint2 w;
  w.x = pack_bf2(v[0], v[1]);
  w.y = pack_bf2(v[2], v[3]);
  *reinterpret_cast<uint2*>(dst) = w;
}

template <class T, int S>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs p) {
  if (gate_closed(p.gate)) return;
  constexpr bool HALF = sizeof(T) == 2;            // bf16 path: IEEE-half O_s / l_s partials
  constexpr int DPT = HALF ? 8 : 4;                // head-dim entries per thread (one 16-byte load)
  constexpr int NV = DPT / 4;
  const int64_t rows = (int64_t)p.B * p.n * p.Hq;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (row, head, d/DPT)
  const int dq = p.dh / DPT;
  if (idx >= rows * dq) return;
  const int64_t rh = idx / dq;
  const int d0 = (int)(idx - rh * dq) * DPT;
  float mv[S], lv[S];
  f32x4_v ov[S][NV];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int64_t sr = (int64_t)s * rows + rh;
    const float2 ml = *reinterpret_cast<const float2*>(p.part_ml + sr * 2);
    mv[s] = ml.x;
    lv[s] = ml.y;
    if constexpr (HALF) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(p.part_o) + (sr * p.dh + d0) * 2);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        float a, b, c, d;
        unpack_h2(w[2 * v], a, b);
        unpack_h2(w[2 * v + 1], c, d);
        ov[s][v] = f32x4_v{a, b, c, d};
      }
    } else {
      ov[s][0] = *reinterpret_cast<const f32x4_v*>(p.part_o + sr * p.dh + d0);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < S; ++s) M = fmaxf(M, mv[s]);
  float L = 0.f;
  f32x4_v o[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) o[v] = f32x4_v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if (mv[s] == -INFINITY) continue;
    const float w = exp2f(mv[s] - M);
    L += lv[s] * w;
#pragma unroll
    for (int v = 0; v < NV; ++v) o[v] += ov[s][v] * (HALF ? lv[s] * w : w);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int v = 0; v < NV; ++v) put4<T>(static_cast<T*>(p.out) + rh * p.dh + d0 + 4 * v, o[v] * inv);
}

template <class T, int S>
static void launch_merge_s(AttnArgs a, int blocks, hipStream_t s) {
  a.gate = launch_gate();
  if constexpr (S < MERGE_MAX) {
    if (a.splits > S) return launch_merge_s<T, S + 1>(a, blocks, s);
  }
  hipLaunchKernelGGL((attn_merge_kernel<T, S>), dim3(blocks), dim3(256), 0, s, a);
}

template <class T, int DH>
static hipError_t launch_attn_t(AttnArgs a, hipStream_t s) {
  a.gate = launch_gate();
  using C = AttnCfg<T, DH>;
  const int qtiles = (a.Hq / a.Hkv * a.n + 63) / 64;
  const int blocks = a.B * a.Hkv * qtiles * a.splits;
  static const hipError_t attr = allow_lds(attn_kernel<T, DH>, C::LDS);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((attn_kernel<T, DH>), dim3(blocks), dim3(256), C::LDS, s, a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, int act_bf16, hipStream_t s) {
  if (act_bf16) return launch_flash(a, s);
  switch (a.dh) {
    case 64: return launch_attn_t<float, 64>(a, s);
    case 128: return launch_attn_t<float, 128>(a, s);
    case 256: return launch_attn_t<float, 256>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_merge(const AttnArgs& a, int act_bf16, hipStream_t s) {
  const int dpt = act_bf16 ? 8 : 4;                  // head-dim entries per merge thread
  if (a.splits < 2 || a.splits > MERGE_MAX || a.dh % dpt) return hipErrorInvalidValue;
  const int64_t n = (int64_t)a.B * a.n * a.Hq * (a.dh / dpt);
  const int blocks = (int)((n + 255) / 256);
  if (act_bf16) launch_merge_s<bf16_t, 2>(a, blocks, s);
  else launch_merge_s<float, 2>(a, blocks, s);
  return hipGetLastError();
}

}  // namespace dg
