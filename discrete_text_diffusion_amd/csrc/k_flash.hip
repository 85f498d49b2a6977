// Canvas attention in bf16 for gfx950: every canvas query attends to the visible prefix cache
// slots and to all canvas keys (bidirectional, [TR §아키텍처와 블록 자기회귀 생성]); with `causal`
// set it serves the causal encoder (sliding window on local layers), and with per-canvas flags a
// batch that mixes the two kinds of pass ([TR §CPU-GPU 동기화 제거]).
//
// Block = FLASH_WAVES waves over 128 query rows of the G = Hq/Hkv heads that share KV head g;
// each wave owns 16 rows (one MFMA column block), two waves per SIMD, so one wave's softmax
// overlaps the other's matrix work.  Keys stream in 64-key tiles straight from global memory
// into LDS (one global_load_lds_dwordx4 moves 16 bytes per lane, no VGPR staging) through an
// NS-stage ring:
//   K tile   [64 keys][dh]   as dh/64 sub-tiles of 128-byte rows, rows in the key order of
//                            key_of_row (below),
//   V^T tile [dh][64 keys]   one 128-byte row per head-dim index (the value cache is d-major),
// both with the 16-byte chunk c of row r stored in slot c ^ ((r >> 1) & 7) (conflict-free
// 16-byte fragment reads).  Per tile:
//   S^T = K . Q^T      (A = K from LDS, B = Q^T held in registers for the whole key loop)
//   online softmax     lane-local per query column; the running max is raised (and O, l
//                      rescaled) only when a tile's scores exceed it by more than 8 in log2 units,
//                      otherwise probabilities are taken against the stale max (at most 256,
//                      exact in fp32; O / l is unchanged)
//   O^T += V^T . P^T   (A = V^T from LDS, B = P^T built in registers from the S^T accumulators)
// The key list is the prefix slots [0, np) in 64-key tiles, then the canvas keys [0, n) in
// 64-key tiles (for the causal encoder only the canvas tiles that some query of the block can see);
// a split covers a contiguous run of tiles.  Rows of a partial tile are loaded
// from the range's last valid key (finite data) and masked out of the softmax; the value
// columns of a partial tile are zeroed in LDS so that P = 0 never meets an unwritten slot.
#include "common.h"
#include "gemm_dma.h"
#include "internal.h"

namespace dg {

// Key held by LDS row p of a K tile.  S^T row p = 32c + 16h + 4g + j (lane group g, element j
// of 16-key block 2c + h) holds key 32c + 8g + 4h + j, so the eight probabilities a lane packs for
// k-step c are eight consecutive keys and its V^T fragment is one 16-byte read.
DG_DEV int key_of_row(int p) { return (p & 0x23) | ((p & 0x0c) << 1) | ((p & 0x10) >> 2); }

template <int DH, int QPW, int NW>
struct FlashCfg {
  static constexpr int KEYS = 64;
  static constexpr int QPW_ = QPW;                 // 16-column query blocks per wave
  static constexpr int QW = 16 * QPW;              // query rows per wave
  static constexpr int WAVES = NW;
  static constexpr int QROWS = QW * WAVES;         // query rows per block
  static constexpr int KSUB = DH / 64;             // 128-byte sub-rows of one key row
  static constexpr int K_BYTES = KEYS * DH * 2;
  static constexpr int V_BYTES = DH * KEYS * 2;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int NS = STAGE * 4 <= 131072 ? 4 : (STAGE * 3 <= 131072 ? 3 : 2);
  static constexpr int LDS = NS * STAGE;
  static constexpr int NCH = DH / 32;              // MFMA k-steps along head_dim
  static constexpr int DB = DH / 16;               // 16-row blocks of head_dim
  static constexpr int K_INS = KEYS * KSUB / 8 / WAVES;   // DMA instructions per wave per tile
  static constexpr int V_INS = DH / 8 / WAVES;
  static constexpr int LPT = K_INS + V_INS;
  static_assert(K_INS >= 1 && V_INS >= 1 && (NS - 2) * LPT < 64, "tile shape");
};

template <int DH, bool CAUSAL, int QPW, int NW>
__global__ __launch_bounds__(NW * 64) void flash_kernel(AttnArgs p) {
  if (gate_closed(p.gate)) return;
  using C = FlashCfg<DH, QPW, NW>;
  extern __shared__ __align__(16) char lds[];
  const int G = p.Hq / p.Hkv;
  const int mrows = G * p.n;
  const int QB = (mrows + C::QROWS - 1) / C::QROWS;
  // XCD-aware: the QB query blocks of one (canvas, KV head, split) get ids congruent mod 8
  const int id = blockIdx.x, xcd = id & 7, local = id >> 3;
  const int qblk = local % QB;
  int r = (local / QB) * 8 + xcd;
  if (r >= p.B * p.Hkv * p.splits) return;
  const int split = r % p.splits; r /= p.splits;
  const int g = r % p.Hkv;
  const int b = r / p.Hkv;
  // a mixed batch runs both instantiations over the whole grid: each takes the canvases of its kind
  if (p.seq_causal && (p.seq_causal[b] != 0) != CAUSAL) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kg = lane >> 4, l16 = lane & 15;

  const int P = prefix_of(p.plen, b, p.max_prefix);
  const int np = p.is_global ? P : min(P, p.window);
  const int TP = (np + C::KEYS - 1) / C::KEYS;
  // canvas key tiles [c_lo, c_hi] are the ones some query of this block can see: all of them for a
  // bidirectional pass; for the causal encoder, none past the block's last query position and, on
  // a sliding-window layer, none wholly older than its first query's window.  The block's rows are
  // (head, position) pairs in head-major order, so the positions form one range unless the block
  // straddles two heads (then every position counts).
  int c_lo = 0, c_hi = (p.n + C::KEYS - 1) / C::KEYS - 1;
  if constexpr (CAUSAL) {
    const int mq0 = qblk * C::QROWS, mq1 = min(mrows, mq0 + C::QROWS) - 1;
    const bool one_head = mq0 / p.n == mq1 / p.n;
    const int qlo = one_head ? mq0 % p.n : 0, qhi = one_head ? mq1 % p.n : p.n - 1;
    c_hi = min(c_hi, qhi / C::KEYS);
    if (!p.is_global) c_lo = max(0, qlo - p.window + 1) / C::KEYS;
  }
  const int TC = c_hi - c_lo + 1;
  const int t_begin = split * p.tiles_per_split;
  const int t_end = min(TP + TC, t_begin + p.tiles_per_split);
  const int ring_lo = max(0, P - p.window);
  const int ring_mod = ring_lo % p.window, ring_base = ring_lo - ring_mod;

  // ---- query fragments: column q = l16 of block qb holds head_dim 32c + 8kg .. + 7 ----------
  int qpos[QPW], qrow[QPW], qhead[QPW];
  bool qok[QPW];
  u32x4 qf[QPW][C::NCH];
#pragma unroll
  for (int qb = 0; qb < QPW; ++qb) {
    const int mq = qblk * C::QROWS + wave * C::QW + qb * 16 + l16;
    qok[qb] = mq < mrows;
    const int hj = qok[qb] ? mq / p.n : 0, qi = qok[qb] ? mq - hj * p.n : 0;
    qhead[qb] = g * G + hj;
    qrow[qb] = b * p.n + qi;
    qpos[qb] = P + qi;
    const char* qp = static_cast<const char*>(p.q) + ((int64_t)qrow[qb] * p.Hq + qhead[qb]) * DH * 2;
#pragma unroll
    for (int c = 0; c < C::NCH; ++c)
      qf[qb][c] = qok[qb] ? *reinterpret_cast<const u32x4*>(qp + (32 * c + 8 * kg) * 2) : u32x4{0, 0, 0, 0};
  }

  const int64_t bg = (int64_t)b * p.Hkv + g;
  const char* kpre = static_cast<const char*>(p.kc) + bg * p.cap * DH * 2;
  const char* kcan = static_cast<const char*>(p.kn) + bg * p.n * DH * 2;
  const char* vpre = static_cast<const char*>(p.vc) + bg * DH * p.cap * 2;   // [dh][cap]
  const char* vcan = static_cast<const char*>(p.vn) + bg * DH * p.vn_ld * 2; // [dh][vn_ld]

  // tile t -> range (prefix / canvas), first key of the tile within the range, valid keys
  auto tile_info = [&](int t, bool& canvas, int& kt0, int& nv) {
    canvas = t >= TP;
    kt0 = (canvas ? c_lo + t - TP : t) * C::KEYS;
    nv = min(C::KEYS, (canvas ? p.n : np) - kt0);
  };

  auto issue_k = [&](int t, int stage) {
    bool canvas; int kt0, nv;
    tile_info(t, canvas, kt0, nv);
    char* st = lds + stage * C::STAGE;
    const int rr = lane >> 3, slot = lane & 7;
    const char* kb = canvas ? kcan : kpre;
#pragma unroll
    for (int i = 0; i < C::K_INS; ++i) {
      const int gi = wave + C::WAVES * i;          // sub-tile gi / 8, rows (gi % 8) * 8 + rr
      const int sub = gi >> 3, row = (gi & 7) * 8 + rr;
      const int key = kt0 + min(key_of_row(row), nv - 1);
      const char* src = kb + (int64_t)key * DH * 2 + sub * 128 + ((slot ^ ((row >> 1) & 7)) * 16);
      dma16(src, st + sub * 8192 + (gi & 7) * 8 * 128);
    }
  };
  auto issue_v = [&](int t, int stage) {
    bool canvas; int kt0, nv;
    tile_info(t, canvas, kt0, nv);
    char* st = lds + stage * C::STAGE;
    const int rr = lane >> 3, slot = lane & 7;
    const char* vb = canvas ? vcan : vpre;
    const int vstride = canvas ? p.vn_ld : p.cap;
    const int last_chunk = ((canvas ? p.n : np) - 1) & ~7;    // first key of the range's last 8-key chunk
#pragma unroll
    for (int i = 0; i < C::V_INS; ++i) {
      const int gi = wave + C::WAVES * i;
      const int d = gi * 8 + rr;
      const int key = min(kt0 + 8 * (slot ^ ((d >> 1) & 7)), last_chunk);
      const char* src = vb + ((int64_t)d * vstride + key) * 2;
      dma16(src, st + C::K_BYTES + gi * 8 * 128);
    }
  };

  f32x4_v acc[C::DB][QPW];
  float m_run[QPW], l_lane[QPW];
#pragma unroll
  for (int qb = 0; qb < QPW; ++qb) {
    m_run[qb] = -INFINITY;
    l_lane[qb] = 0.f;
#pragma unroll
    for (int i = 0; i < C::DB; ++i) acc[i][qb] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  }

  // ---- phases of one tile ----------------------------------------------------------------------
  // S^T = K . Q^T.  K fragments of head-dim chunk c+1 are read while the MFMAs of chunk c run (two
  // register sets), so each group of reads has a group of MFMAs to hide behind.
  const int swz = l16 >> 1;
  auto phase_s = [&](const char* st, f32x4_v (&s)[4][QPW]) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int qb = 0; qb < QPW; ++qb) s[nb][qb] = f32x4_v{0.f, 0.f, 0.f, 0.f};
    auto kfrag = [&](int c, int nb) -> u32x4 {
      return *reinterpret_cast<const u32x4*>(st + (c >> 1) * 8192 + l16 * 128 + (((4 * (c & 1) + kg) ^ swz) * 16) +
                                             nb * 16 * 128);
    };
    u32x4 kf[2][4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) kf[0][nb] = kfrag(0, nb);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);         // the first group's 4 LDS reads
#pragma unroll
    for (int c = 0; c < C::NCH; ++c) {
      if (c + 1 < C::NCH) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) kf[(c + 1) & 1][nb] = kfrag(c + 1, nb);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);     // then the next group's reads ...
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int qb = 0; qb < QPW; ++qb) Mfma<bf16_t>::mma(s[nb][qb], kf[c & 1][nb], qf[qb][c]);
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * QPW, 0);  // ... ahead of this group's MFMAs
    }
  };

  // mask, scale, online softmax with conditional rescale, P^T packed to bf16.  The column max (over
  // the 4 lanes sharing a query column) is only formed when some lane's scores exceed its running
  // max by more than 8 (log2 units): rare after the first tile.
  auto phase_softmax = [&](int t, f32x4_v (&s)[4][QPW], u32x4 (&pb)[QPW][2]) {
    bool canvas; int kt0, nv;
    tile_info(t, canvas, kt0, nv);
    const bool full = !CAUSAL && nv == C::KEYS;
#pragma unroll
    for (int qb = 0; qb < QPW; ++qb) {
      float ml = -INFINITY;
      if (full) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float v = s[nb][qb][j] * p.scale_log2;
            s[nb][qb][j] = v;
            ml = fmaxf(ml, v);
          }
      } else {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int kl = key_of_row(nb * 16 + 4 * kg + j);     // key within the tile
            bool vis = kl < nv;
            if constexpr (CAUSAL) {
              const int kk = kt0 + kl;
              // ring slot -> position: the ring holds positions [ring_lo, ring_lo + window)
              const int kpos = canvas ? P + kk : (p.is_global ? kk : kk + ring_base + (kk < ring_mod ? p.window : 0));
              vis = vis && kpos <= qpos[qb] && (p.is_global || qpos[qb] - kpos < p.window);
            }
            const float v = vis ? s[nb][qb][j] * p.scale_log2 : -INFINITY;
            s[nb][qb][j] = v;
            ml = fmaxf(ml, v);
          }
      }
      if (__any(ml > m_run[qb] + 8.f)) {
        float mt = fmaxf(ml, __shfl_xor(ml, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const bool need = mt > m_run[qb] + 8.f;     // also true for the first visible scores
        const float alpha = need ? (m_run[qb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[qb] - mt)) : 1.f;
        m_run[qb] = need ? mt : m_run[qb];
        l_lane[qb] *= alpha;
#pragma unroll
        for (int i = 0; i < C::DB; ++i) acc[i][qb] *= alpha;
      }
      const float mr = m_run[qb] == -INFINITY ? 0.f : m_run[qb];   // all -inf so far: p = 0 below
      float psum = 0.f;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float e = __builtin_amdgcn_exp2f(s[nb][qb][j] - mr);   // exp2(-inf) = 0
          s[nb][qb][j] = e;
          psum += e;
        }
      l_lane[qb] += psum;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        pb[qb][c2].x = pack_bf2(s[2 * c2][qb][0], s[2 * c2][qb][1]);
        pb[qb][c2].y = pack_bf2(s[2 * c2][qb][2], s[2 * c2][qb][3]);
        pb[qb][c2].z = pack_bf2(s[2 * c2 + 1][qb][0], s[2 * c2 + 1][qb][1]);
        pb[qb][c2].w = pack_bf2(s[2 * c2 + 1][qb][2], s[2 * c2 + 1][qb][3]);
      }
    }
  };

  // O^T += V^T . P^T: lane (d = l16, kg) supplies keys 32c2 + 8kg .. + 7 of row d.  The key half c2
  // is outermost, so consecutive MFMAs feed different accumulators (each accumulator still takes
  // its two halves in the order c2 = 0, 1); V fragments are read one group of four ahead of the
  // MFMAs that use them, as for K above.
  auto phase_pv = [&](const char* st, const u32x4 (&pb)[QPW][2]) {
    const char* vt = st + C::K_BYTES;
    auto vfrag = [&](int g) -> u32x4 {            // g = c2 * DB + db
      const int c2 = g / C::DB, d = (g % C::DB) * 16 + l16;
      return *reinterpret_cast<const u32x4*>(vt + d * 128 + (((4 * c2 + kg) ^ ((d >> 1) & 7)) * 16));
    };
    constexpr int NG = 2 * C::DB / 4;             // groups of four fragments
    u32x4 vf[2][4];
#pragma unroll
    for (int e = 0; e < 4; ++e) vf[0][e] = vfrag(e);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      if (gi + 1 < NG) {
#pragma unroll
        for (int e = 0; e < 4; ++e) vf[(gi + 1) & 1][e] = vfrag(4 * (gi + 1) + e);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int g = 4 * gi + e, c2 = g / C::DB, db = g % C::DB;
#pragma unroll
        for (int qb = 0; qb < QPW; ++qb) Mfma<bf16_t>::mma(acc[db][qb], vf[gi & 1][e], pb[qb][c2]);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * QPW, 0);
    }
  };

  // ---- key loop ----------------------------------------------------------------------------------
  // Two wave groups, one wave of each per SIMD, half a tile apart.  Between the tile's two barriers
  // the leading group (waves 0 .. NW/2-1) forms S(t) while the lagging group adds P(t-1) V(t-1);
  // after the second, the leading group takes the softmax and P(t) V(t) while the lagging group forms
  // S(t) and its softmax.  One group's softmax thus meets the other's matrix products on each SIMD
  // (a single barrier per tile would keep the two waves of a SIMD in the same phase).  Each
  // accumulator still sees rescale(t), then + P(t) V(t), in tile order.  K(t+1) is loaded after the
  // first barrier (every wave is done with S(t-1)); V(t+1) after the second (the lagging group is
  // done with P(t-1) V(t-1)).
  const bool lag = wave >= NW / 2;
  auto stage_of = [&](int t) -> char* { return lds + ((t - t_begin) % C::NS) * C::STAGE; };
  u32x4 pb[QPW][2];
  if (t_begin < t_end) {
    issue_k(t_begin, 0);
    issue_v(t_begin, 0);
  }
  for (int t = t_begin; t < t_end; ++t) {
    const bool more = t + 1 < t_end;
    char* st = stage_of(t);
    wait_vm<C::V_INS>();                 // K(t): only V(t) was issued after it
    lds_barrier();
    if (more) issue_k(t + 1, (t + 1 - t_begin) % C::NS);
    f32x4_v s[4][QPW];
    if (!lag) phase_s(st, s);
    else if (t > t_begin) phase_pv(stage_of(t - 1), pb);
    if (more) wait_vm<C::K_INS>();       // V(t): only K(t+1) was issued after it
    else wait_vm<0>();
    lds_barrier();
    bool canvas; int kt0, nv;
    tile_info(t, canvas, kt0, nv);
    if (nv < C::KEYS) {
      // zero the value columns of keys nv..63 (their slots may hold anything)
      char* vt = st + C::K_BYTES;
      for (int idx = threadIdx.x; idx < DH * 8; idx += NW * 64) {
        const int d = idx >> 3, c = idx & 7;
        if (8 * c + 8 <= nv) continue;
        u32x4* w = reinterpret_cast<u32x4*>(vt + d * 128 + ((c ^ ((d >> 1) & 7)) * 16));
        u32x4 v = *w;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (8 * c + e < nv) continue;
          const uint32_t mask = (e & 1) ? 0x0000ffffu : 0xffff0000u;
          v[e >> 1] &= mask;
        }
        *w = v;
      }
      lds_barrier();
    }
    if (more) issue_v(t + 1, (t + 1 - t_begin) % C::NS);
    if (!lag) {
      phase_softmax(t, s, pb);
      phase_pv(st, pb);
    } else {
      phase_s(st, s);
      phase_softmax(t, s, pb);
    }
  }
  if (lag && t_begin < t_end) phase_pv(stage_of(t_end - 1), pb);

  // ---- finish --------------------------------------------------------------------------------
  // Lane (l16, kg) holds head-dim indices 16db + 4kg .. + 3 of query column l16: stored directly,
  // each instruction would write 32 bytes into each of 16 rows.  The wave's 16 x DH block goes
  // through LDS instead (the ring is idle once every wave has left the key loop), and each store
  // instruction then writes whole rows.
  // Split partials are the split's output normalised by its own sum, O_s / l_s (a convex
  // combination of value rows, so bounded by max |v|), as IEEE half: half the bytes of fp32 sums at
  // 2^-11 relative precision; (m_s, l_s) stay fp32.  One split writes the bf16 output itself.
  constexpr int ROWB = DH * 2 + 16;                  // padded LDS row of one query (bytes)
  static_assert(NW * 16 * ROWB <= C::LDS, "finish staging");
  char* tb = lds + wave * 16 * ROWB;
  const bool partial = p.splits > 1;
  lds_barrier();
#pragma unroll
  for (int qb = 0; qb < QPW; ++qb) {
    float l = l_lane[qb] + __shfl_xor(l_lane[qb], 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const f32x4_v v = acc[db][qb] * inv;
      uint2 w;
      w.x = partial ? pack_h2(v[0], v[1]) : pack_bf2(v[0], v[1]);
      w.y = partial ? pack_h2(v[2], v[3]) : pack_bf2(v[2], v[3]);
      *reinterpret_cast<uint2*>(tb + l16 * ROWB + (db * 16 + 4 * kg) * 2) = w;
    }
    if (partial && kg == 0 && qok[qb]) {
      float* ml = p.part_ml + (((int64_t)split * p.B * p.n + qrow[qb]) * p.Hq + qhead[qb]) * 2;
      ml[0] = m_run[qb];
      ml[1] = l;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's own LDS writes, in order
    constexpr int CPR = DH / 8, RPI = 64 / CPR;          // 16-byte chunks per row, rows per store
    static_assert(CPR * RPI == 64 && 16 % RPI == 0, "finish store shape");
    const int ch = lane % CPR;
#pragma unroll
    for (int it = 0; it < 16 / RPI; ++it) {
      const int r = RPI * it + lane / CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(tb + r * ROWB + ch * 16);
      const int mq = qblk * C::QROWS + wave * C::QW + qb * 16 + r;
      if (mq >= mrows) continue;
      const int hj = mq / p.n, qi = mq - hj * p.n;
      const int64_t rh = (int64_t)(b * p.n + qi) * p.Hq + g * G + hj;
      char* dst = partial ? reinterpret_cast<char*>(p.part_o) + (((int64_t)split * p.B * p.n * p.Hq + rh) * DH) * 2
                          : static_cast<char*>(p.out) + rh * DH * 2;
      // streaming stores: the merge or the output projection reads these rows from any XCD
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst + ch * 16));
    }
    if (qb + 1 < QPW) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

template <int DH, bool CAUSAL>
static hipError_t launch_flash_t(AttnArgs a, hipStream_t s) {
  a.gate = launch_gate();
  using C = FlashCfg<DH, FLASH_QPW, FLASH_WAVES>;
  const int QB = (a.Hq / a.Hkv * a.n + C::QROWS - 1) / C::QROWS;
  const int groups = a.B * a.Hkv * a.splits;
  const int blocks = QB * ((groups + 7) / 8 * 8);
  auto* k = flash_kernel<DH, CAUSAL, FLASH_QPW, FLASH_WAVES>;
  static const hipError_t attr = allow_lds(k, C::LDS);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(k, dim3(blocks), dim3(FLASH_WAVES * 64), C::LDS, s, a);
  return hipGetLastError();
}

hipError_t launch_flash(const AttnArgs& a, hipStream_t s) {
  // a mixed batch (per-canvas kinds, flags on the device): the bidirectional and the causal
  // kernel each cover the grid and leave the other kind's blocks at once
  if (a.seq_causal) {
    hipError_t e = hipErrorInvalidValue;
    switch (a.dh) {
      case 64: e = launch_flash_t<64, false>(a, s); break;
      case 128: e = launch_flash_t<128, false>(a, s); break;
      case 256: e = launch_flash_t<256, false>(a, s); break;
    }
    if (e != hipSuccess) return e;
    switch (a.dh) {
      case 64: return launch_flash_t<64, true>(a, s);
      case 128: return launch_flash_t<128, true>(a, s);
      case 256: return launch_flash_t<256, true>(a, s);
    }
    return hipErrorInvalidValue;
  }
  if (a.causal) {
    switch (a.dh) {
      case 64: return launch_flash_t<64, true>(a, s);
      case 128: return launch_flash_t<128, true>(a, s);
      case 256: return launch_flash_t<256, true>(a, s);
    }
  } else {
    switch (a.dh) {
      case 64: return launch_flash_t<64, false>(a, s);
      case 128: return launch_flash_t<128, false>(a, s);
      case 256: return launch_flash_t<256, false>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace dg
