// MoE routing: top-k experts per row (ties to the lower expert id), gates = softmax over the
// selected router logits, then the expert-grouped row order (rows of each expert in ascending
// (token, slot) order), its inverse, and the tile work list of the grouped GEMMs.  Everything is
// deterministic: no atomics decide an order.
#include "common.h"
#include "internal.h"

namespace dg {

// one wave per row; E <= 256 (4 values per lane), k <= 16
__global__ __launch_bounds__(256) void router_topk_kernel(const float* logits, int T, int E, int k,
                                                          int32_t* idx, float* gates) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? logits[(int64_t)t * E + e] : -INFINITY;
  }
  float sel_v[16];
  int sel_i[16];
  for (int s = 0; s < k; ++s) {
    // lane-local best (lowest id on ties: j ascending = id ascending)
    float bv = v[0]; int bi = lane;
#pragma unroll
    for (int j = 1; j < 4; ++j)
      if (v[j] > bv) { bv = v[j]; bi = lane + 64 * j; }
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    sel_v[s] = bv;
    sel_i[s] = bi;
    if ((bi & 63) == lane) v[bi >> 6] = -INFINITY;
  }
  if (lane == 0) {
    float mx = sel_v[0];
    float w[16], tot = 0.f;
    for (int s = 0; s < k; ++s) { w[s] = __expf(sel_v[s] - mx); tot += w[s]; }
    for (int s = 0; s < k; ++s) {
      idx[(int64_t)t * k + s] = sel_i[s];
      gates[(int64_t)t * k + s] = w[s] / tot;
    }
  }
}

hipError_t launch_router_topk(const float* logits, int T, int E, int k, int32_t* idx, float* gates,
                              hipStream_t s) {
  hipLaunchKernelGGL(router_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, idx, gates);
  return hipGetLastError();
}

// Single block.  Thread t owns the contiguous assignment range [t*chunk, (t+1)*chunk) and a
// private counter column cnt[e][t]; an exclusive scan over (expert, thread) gives each thread
// its write base per expert, so the grouped order is ascending assignment id within an expert.
static int route_threads(int E) { return E <= 128 ? 256 : 128; }

size_t route_tables_lds(int E) { return (size_t)E * route_threads(E) * 4 + 1024 * 4; }

__global__ void route_tables_kernel(const int32_t* idx, int T, int E, int k, int32_t* counts,
                                    int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* tok,
                                    int32_t* work, int32_t* n_items, int bm) {
  extern __shared__ int32_t sm[];
  const int NT = blockDim.x, tid = threadIdx.x;
  int32_t* cnt = sm;                     // [E][NT]
  int32_t* tsum = sm + E * NT;           // [NT] scan scratch (+ tile scan)
  const int A = T * k;
  const int chunk = (A + NT - 1) / NT;
  const int a0 = min(A, tid * chunk), a1 = min(A, a0 + chunk);
  for (int e = 0; e < E; ++e) cnt[e * NT + tid] = 0;
  // ids come from router_topk and are always in [0, E); the clamp keeps a corrupted id in bounds
  for (int a = a0; a < a1; ++a) cnt[min(max(idx[a], 0), E - 1) * NT + tid] += 1;
  __syncthreads();
  // exclusive scan over the flattened [E][NT] array: thread t scans segment [t*E, (t+1)*E)
  const int seg0 = tid * E;
  int s = 0;
  for (int q = 0; q < E; ++q) s += cnt[seg0 + q];
  tsum[tid] = s;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int q = 0; q < NT; ++q) { const int v = tsum[q]; tsum[q] = run; run += v; }
  }
  __syncthreads();
  int run = tsum[tid];
  for (int q = 0; q < E; ++q) { const int v = cnt[seg0 + q]; cnt[seg0 + q] = run; run += v; }
  __syncthreads();
  // per-expert counts/offsets and tile counts
  int32_t* tiles = tsum;                 // reuse: [E] tile offsets
  if (tid == 0) {
    int acc = 0;
    for (int e = 0; e < E; ++e) {
      const int off = cnt[e * NT];
      const int nxt = e + 1 < E ? cnt[(e + 1) * NT] : A;
      offsets[e] = off;
      counts[e] = nxt - off;
      tiles[e] = acc;
      acc += (nxt - off + bm - 1) / bm;
    }
    *n_items = acc;
  }
  __syncthreads();
  for (int e = tid; e < E; e += NT) {
    const int off = cnt[e * NT];
    const int c = (e + 1 < E ? cnt[(e + 1) * NT] : A) - off;
    int w = tiles[e];
    for (int m0 = 0; m0 < c; m0 += bm, ++w) { work[2 * w] = e; work[2 * w + 1] = m0; }
  }
  // scatter: positions in ascending assignment order within each expert
  for (int a = a0; a < a1; ++a) {
    const int e = min(max(idx[a], 0), E - 1);
    const int pos = cnt[e * NT + tid]++;
    perm[pos] = a;
    inv_perm[a] = pos;
    tok[pos] = a / k;
  }
}

hipError_t launch_route_tables(const int32_t* idx, int T, int E, int k, int32_t* counts, int32_t* offsets,
                               int32_t* perm, int32_t* inv_perm, int32_t* tok, int32_t* work,
                               int32_t* n_items, int bm, hipStream_t s) {
  const int NT = route_threads(E);
  static const hipError_t attr = allow_lds(route_tables_kernel, route_tables_lds(256));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(route_tables_kernel, dim3(1), dim3(NT), route_tables_lds(E), s, idx, T, E, k, counts,
                     offsets, perm, inv_perm, tok, work, n_items, bm);
  return hipGetLastError();
}

}  // namespace dg
