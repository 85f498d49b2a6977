// MoE routing: top-k experts per row (ties to the lower expert id), gates = softmax over the
// selected router logits, then per-expert row counts, the expert-grouped row order (rows of each
// expert in ascending (token, slot) order), its inverse, and the tile work list of the grouped
// GEMMs.  Everything is deterministic: counts are integer sums and no atomic decides an order.
#include "common.h"
#include "internal.h"

namespace dg {

constexpr int MAX_PARTS = 16;   // split-K parts of the router GEMM

// Candidate order as one 64-bit key: the score mapped to an order-preserving uint32 (NaN counts as
// -inf, -0 as +0) above 0xffff - expert id, so a larger key is a larger score, then a lower id;
// 0 (below every candidate) marks "none".
DG_DEV uint64_t topk_key(float v, int e) {
  if (!(v == v)) v = -INFINITY;
  if (v == 0.f) v = 0.f;
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(0xffff - e);
}
DG_DEV float key_score(uint64_t k) {
  const uint32_t u = (uint32_t)(k >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}
DG_DEV int key_expert(uint64_t k) { return 0xffff - (int)(uint32_t)k; }

DG_DEV uint64_t key_max(uint64_t a, uint32_t blo, uint32_t bhi) {
  const uint64_t b = ((uint64_t)bhi << 32) | blo;
  return b > a ? b : a;
}
// lane key combined with the key of the lane that the DPP control names (full row and bank masks:
// quad permutes and row rotations have a source in every lane)
template <int CTRL>
DG_DEV uint64_t key_max_dpp(uint64_t k) {
  const uint32_t lo = (uint32_t)k, hi = (uint32_t)(k >> 32);
  return key_max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, CTRL, 0xf, 0xf, false),
                 (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, CTRL, 0xf, 0xf, false));
}
// the maximum key over the wave, in every lane, without LDS: quad swaps (xor 1, xor 2) and row
// rotations (4, 8) give every lane its 16-lane row's maximum; the row-pair and half swaps of
// gfx950 (permlane16 / permlane32) then combine rows
DG_DEV uint64_t wave_max_key(uint64_t k) {
  k = key_max_dpp<0xB1>(k);    // quad_perm [1, 0, 3, 2]
  k = key_max_dpp<0x4E>(k);    // quad_perm [2, 3, 0, 1]
  k = key_max_dpp<0x124>(k);   // row_ror 4
  k = key_max_dpp<0x128>(k);   // row_ror 8
  {
    const auto l = __builtin_amdgcn_permlane16_swap((uint32_t)k, (uint32_t)k, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap((uint32_t)(k >> 32), (uint32_t)(k >> 32), false, false);
    k = key_max(key_max(0, l[0], h[0]), l[1], h[1]);
  }
  {
    const auto l = __builtin_amdgcn_permlane32_swap((uint32_t)k, (uint32_t)k, false, false);
    const auto h = __builtin_amdgcn_permlane32_swap((uint32_t)(k >> 32), (uint32_t)(k >> 32), false, false);
    k = key_max(key_max(0, l[0], h[0]), l[1], h[1]);
  }
  return k;
}

// One wave (one block) per row; lane l holds experts 4l .. 4l+3 (E <= 256, E % 4 == 0), k <= E,
// k <= 16.  The router logits arrive as `nparts` split-K partial sums, added in part order
// (deterministic), plus the optional bias.  Each of the k rounds takes the wave's largest key
// among the untaken candidates.
template <int K>
__global__ __launch_bounds__(64) void router_topk_kernel(const float* parts, int nparts, int64_t part_stride,
                                                         const float* bias, int T, int E, int k, float* logits_out,
                                                         int32_t* idx, float* gates, const int32_t* gate) {
  if (gate_closed(gate)) return;
  const int lane = threadIdx.x;
  const int t = blockIdx.x;
  const int e0 = 4 * lane;
  const bool on = e0 < E;
  uint64_t key[4] = {0, 0, 0, 0};
  if (on) {
    const float* src = parts + (int64_t)t * E + e0;
    f32x4_v pv[MAX_PARTS];
#pragma unroll
    for (int p = 0; p < MAX_PARTS; ++p)
      if (p < nparts) pv[p] = *reinterpret_cast<const f32x4_v*>(src + p * part_stride);
    f32x4_v acc = pv[0];
#pragma unroll
    for (int p = 1; p < MAX_PARTS; ++p)
      if (p < nparts) acc += pv[p];
    if (bias) acc += *reinterpret_cast<const f32x4_v*>(bias + e0);
    if (logits_out) *reinterpret_cast<f32x4_v*>(logits_out + (int64_t)t * E + e0) = acc;
#pragma unroll
    for (int j = 0; j < 4; ++j) key[j] = topk_key(acc[j], e0 + j);
  }
  float sel_v[K];
  int sel_i[K];
#pragma unroll
  for (int s = 0; s < K; ++s) {
    if (s >= k) break;
    uint64_t b = key[0];
#pragma unroll
    for (int j = 1; j < 4; ++j) b = key[j] > b ? key[j] : b;
    b = wave_max_key(b);
    sel_v[s] = key_score(b);
    sel_i[s] = key_expert(b);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (key[j] == b) key[j] = 0;     // keys are distinct (distinct expert ids)
  }
  if (lane == 0) {
    const float mx = sel_v[0];
    float tot = 0.f;
#pragma unroll
    for (int s = 0; s < K; ++s)
      if (s < k) tot += sel_v[s] == -INFINITY ? 0.f : __expf(sel_v[s] - mx);
#pragma unroll
    for (int s = 0; s < K; ++s)
      if (s < k) {
        idx[(int64_t)t * k + s] = sel_i[s];
        gates[(int64_t)t * k + s] = tot > 0.f && sel_v[s] != -INFINITY ? __expf(sel_v[s] - mx) / tot : 0.f;
      }
  }
}

hipError_t launch_router_topk(const float* parts, int nparts, int64_t part_stride, const float* bias, int T, int E,
                              int k, float* logits_out, int32_t* idx, float* gates, hipStream_t s) {
  if (E > 256 || E % 4 || k > 16 || k > E || nparts < 1 || nparts > MAX_PARTS || part_stride % 4)
    return hipErrorInvalidValue;
  if (((uintptr_t)parts & 15) || ((uintptr_t)bias & 15) || ((uintptr_t)logits_out & 15)) return hipErrorInvalidValue;
  if (T == 0) return hipSuccess;
  const dim3 grid(T);
  if (k <= 2)
    hipLaunchKernelGGL(router_topk_kernel<2>, grid, dim3(64), 0, s, parts, nparts, part_stride, bias, T, E, k, logits_out, idx, gates, launch_gate());
  else if (k <= 8)
    hipLaunchKernelGGL(router_topk_kernel<8>, grid, dim3(64), 0, s, parts, nparts, part_stride, bias, T, E, k, logits_out, idx, gates, launch_gate());
  else
    hipLaunchKernelGGL(router_topk_kernel<16>, grid, dim3(64), 0, s, parts, nparts, part_stride, bias, T, E, k, logits_out, idx, gates, launch_gate());
  return hipGetLastError();
}

// ---- grouping -------------------------------------------------------------------------------
// The experts of one row are distinct, so for expert e the flag "row t chose e" is 0/1 and the
// grouped position of (t, s) is offsets[e] + (number of earlier rows that chose e).

template <int K, class P>
DG_DEV int chosen_slot(P idx, int t, int k, int e) {
  int v[K];
#pragma unroll
  for (int s = 0; s < K; ++s) v[s] = idx[(int64_t)t * k + min(s, k - 1)];
  int slot = -1;
#pragma unroll
  for (int s = 0; s < K; ++s)
    if (s < k && v[s] == e) slot = s;
  return slot;
}

// Block e (one launch for all experts): every block forms the per-expert row counts of all T*k
// picks in LDS; offsets[e] and expert e's first tile index are the sums of counts / tiles of the
// experts below e; expert e's work-list tiles (e, m0); then the positions of its rows in
// ascending row order (wave ballots over row chunks).
DG_DEV int block_sum_int(int v, int* red) {
  v = wave_sum_i(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// STAGED: the T*k picks are first copied to LDS (every block reads all of them twice).
constexpr int ROUTE_STAGE_MAX = 16384;   // picks staged in LDS (64 KB)

template <int K, bool STAGED>
__global__ __launch_bounds__(256) void route_place_kernel(const int32_t* idx_g, int T, int E, int k, int32_t* counts,
                                                          int bm, int32_t* offsets, int32_t* work,
                                                          int32_t* n_items, int32_t* perm, int32_t* inv_perm,
                                                          int32_t* tok, const int32_t* gate) {
  if (gate_closed(gate)) return;
  const int e = blockIdx.x;
  __shared__ int red[4];
  __shared__ int wsum[4];
  __shared__ int hist[256];
  extern __shared__ __align__(16) int32_t idx_s[];
  for (int q = threadIdx.x; q < 256; q += 256) hist[q] = 0;
  if constexpr (STAGED) {
    // 16-byte loads when the picks are 16-byte aligned, then the tail one by one
    const int n4 = (reinterpret_cast<uintptr_t>(idx_g) & 15) == 0 ? (T * k) >> 2 : 0;
    for (int i = threadIdx.x; i < n4; i += 256)
      reinterpret_cast<int4*>(idx_s)[i] = reinterpret_cast<const int4*>(idx_g)[i];
    for (int i = 4 * n4 + threadIdx.x; i < T * k; i += 256) idx_s[i] = idx_g[i];
  }
  __syncthreads();
  const int32_t* idx = STAGED ? idx_s : idx_g;
  for (int i = threadIdx.x; i < T * k; i += 256) atomicAdd(&hist[min(max(idx[i], 0), E - 1)], 1);
  __syncthreads();
  int ro = 0, rt = 0;
  for (int q = threadIdx.x; q < e; q += 256) {
    const int c = hist[q];
    ro += c;
    rt += (c + bm - 1) / bm;
  }
  int base = block_sum_int(ro, red);
  const int tile0 = block_sum_int(rt, red);
  const int c = hist[e];
  if (threadIdx.x == 0) {
    counts[e] = c;
    offsets[e] = base;
    if (e == E - 1) *n_items = tile0 + (c + bm - 1) / bm;
  }
  for (int m0 = threadIdx.x * bm; m0 < c; m0 += 256 * bm) {
    const int w = tile0 + m0 / bm;
    work[2 * w] = e;
    work[2 * w + 1] = m0;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int t0 = 0; t0 < T; t0 += 256) {
    const int t = t0 + threadIdx.x;
    const int slot = t < T ? chosen_slot<K>(idx, t, k, e) : -1;
    const uint64_t m = __ballot(slot >= 0);
    const int rank_in_wave = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(m);
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    if (slot >= 0) {
      const int pos = base + before + rank_in_wave;
      const int a = t * k + slot;
      perm[pos] = a;
      inv_perm[a] = pos;
      tok[pos] = t;
    }
    base += total;
    __syncthreads();
  }
}

template <int K>
static hipError_t launch_place(const int32_t* idx, int T, int E, int k, int32_t* counts, int32_t* offsets,
                               int32_t* perm, int32_t* inv_perm, int32_t* tok, int32_t* work, int32_t* n_items,
                               int bm, hipStream_t s) {
  if ((int64_t)T * k <= ROUTE_STAGE_MAX) {
    static const hipError_t attr = allow_lds(route_place_kernel<K, true>, ROUTE_STAGE_MAX * 4);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((route_place_kernel<K, true>), dim3(E), dim3(256), (size_t)T * k * 4, s, idx, T, E, k, counts,
                       bm, offsets, work, n_items, perm, inv_perm, tok, launch_gate());
  } else {
    hipLaunchKernelGGL((route_place_kernel<K, false>), dim3(E), dim3(256), 0, s, idx, T, E, k, counts, bm, offsets,
                       work, n_items, perm, inv_perm, tok, launch_gate());
  }
  return hipGetLastError();
}

hipError_t launch_route_tables(const int32_t* idx, int T, int E, int k, int32_t* counts, int32_t* offsets,
                               int32_t* perm, int32_t* inv_perm, int32_t* tok, int32_t* work, int32_t* n_items,
                               int bm, hipStream_t s) {
  if (k <= 2) return launch_place<2>(idx, T, E, k, counts, offsets, perm, inv_perm, tok, work, n_items, bm, s);
  if (k <= 8) return launch_place<8>(idx, T, E, k, counts, offsets, perm, inv_perm, tok, work, n_items, bm, s);
  return launch_place<16>(idx, T, E, k, counts, offsets, perm, inv_perm, tok, work, n_items, bm, s);
}

}  // namespace dg
