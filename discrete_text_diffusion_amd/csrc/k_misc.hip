// Row-wise and elementwise kernels of the decoder layer: embedding lookup into the fp32 residual
// stream, RMSNorm into the activation dtype, appending encoded keys/values to the caches, and
// the MoE combine (slot-ordered gate-weighted sum of expert outputs + shared expert + residual).
#include "common.h"
#include "internal.h"

namespace dg {

// The host side of the launch gate: one current gate per host thread.
namespace {
thread_local const int32_t* t_gate = nullptr;
}
const int32_t* launch_gate() { return t_gate; }
GateScope::GateScope(const int32_t* gate) : prev(t_gate) { t_gate = gate; }
GateScope::~GateScope() { t_gate = prev; }

template <class T>
__global__ void embed_kernel(const int32_t* tok, const T* E, float* resid, int d, int V, const float* add,
                             const int32_t* gate) {
  if (gate_closed(gate)) return;
  const int r = blockIdx.x;
  const int t = min(max(tok[r], 0), V - 1);     // out-of-range ids are clamped, never read past E
  const T* src = E + (int64_t)t * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x)
    resid[(int64_t)r * d + c] = Elem<T>::to_f(src[c]) + (add ? add[(int64_t)r * d + c] : 0.f);
}

hipError_t launch_embed(const int32_t* tok, const void* E, float* resid, int rows, int d, int V, int bf,
                        hipStream_t s, const float* add) {
  if (bf)
    hipLaunchKernelGGL(embed_kernel<bf16_t>, dim3(rows), dim3(256), 0, s, tok, (const bf16_t*)E, resid, d, V, add,
                       launch_gate());
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(rows), dim3(256), 0, s, tok, (const float*)E, resid, d, V, add,
                       launch_gate());
  return hipGetLastError();
}

template <class T>
__global__ void sum_parts_cast_kernel(const float* parts, int nparts, int64_t pstride, T* out, int64_t n,
                                      const int32_t* gate) {
  if (gate_closed(gate)) return;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float a = 0.f;
  for (int q = 0; q < nparts; ++q) a += parts[q * pstride + i];
  out[i] = Elem<T>::from_f(a);
}

hipError_t launch_sum_parts_cast(const float* parts, int nparts, int64_t pstride, void* out, int64_t n, int bf,
                                 hipStream_t s) {
  const dim3 grid((unsigned)((n + 255) / 256));
  if (bf)
    hipLaunchKernelGGL(sum_parts_cast_kernel<bf16_t>, grid, dim3(256), 0, s, parts, nparts, pstride, (bf16_t*)out, n,
                       launch_gate());
  else
    hipLaunchKernelGGL(sum_parts_cast_kernel<float>, grid, dim3(256), 0, s, parts, nparts, pstride, (float*)out, n,
                       launch_gate());
  return hipGetLastError();
}

// ---------------------------------------------------------------- W8A8 activation codes --------
// One wave per row: s = max|x| / 448 in float32 (1 for a zero row), and the nearest OCP e4m3
// (e4m3fn: bias 7, 3 mantissa bits, largest finite 448) codes of the float32 products x * r with
// r = 448 / max|x| (1 for a zero row), one division per row; ties go to the even code and values
// beyond 448 saturate.  The row stays in registers between the max and the coding (CH 16-byte
// chunks per lane, K <= 512 CH), so it is read once.  The build keeps IEEE float division (no
// fast-math): s and r are correctly rounded, and each product is a single rounded multiply.
template <int WPB, int CH>
__global__ __launch_bounds__(WPB * 64) void quant_rows_kernel(const bf16_t* x, int64_t ldx, int rows, int K,
                                                             uint8_t* q, float* s, const int32_t* gate) {
  if (gate_closed(gate)) return;
  const int lane = threadIdx.x & 63, r = blockIdx.x * WPB + (threadIdx.x >> 6);
  if (r >= rows) return;
  const bf16_t* xr = x + (int64_t)r * ldx;
  uint4 v[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int k = (c * 64 + lane) * 8;
    v[c] = k < K ? *reinterpret_cast<const uint4*>(xr + k) : make_uint4(0u, 0u, 0u, 0u);
  }
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
    for (int h = 0; h < 4; ++h)
      amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(w[h] << 16)), fabsf(__uint_as_float(w[h] & 0xffff0000u))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const float sc = amax > 0.f ? amax / 448.f : 1.f;
  const float rc = amax > 0.f ? 448.f / amax : 1.f;
  if (lane == 0) s[r] = sc;
  uint8_t* qr = q + (int64_t)r * K;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int k = (c * 64 + lane) * 8;
    if (k >= K) continue;
    const uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
    // the hardware conversion rounds to nearest even; the clamp to +-448 makes it saturate.  Two
    // bf16 elements per word, four codes per output word (the second pair into its upper half)
    auto prod = [&](uint32_t word, bool upper) {
      const float v = __fmul_rn(__uint_as_float(upper ? word & 0xffff0000u : word << 16), rc);
      return fminf(fmaxf(v, -448.f), 448.f);
    };
    uint32_t out[2];
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(prod(w[2 * o], false), prod(w[2 * o], true), 0, false);
      out[o] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(prod(w[2 * o + 1], false), prod(w[2 * o + 1], true), lo, true);
    }
    *reinterpret_cast<uint2*>(qr + k) = make_uint2(out[0], out[1]);
  }
}

template <int CH>
static hipError_t launch_quant_ch(const void* x, int64_t ldx, int rows, int K, uint8_t* q, float* s, hipStream_t st) {
  constexpr int WPB = 4;
  hipLaunchKernelGGL((quant_rows_kernel<WPB, CH>), dim3((unsigned)((rows + WPB - 1) / WPB)), dim3(WPB * 64), 0, st,
                     static_cast<const bf16_t*>(x), ldx, rows, K, q, s, launch_gate());
  return hipGetLastError();
}

hipError_t launch_quant_rows(const void* x, int64_t ldx, int rows, int K, uint8_t* q, float* s, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  if (K % 8 || ldx % 8 || K > 4096) return hipErrorInvalidValue;
  switch ((K + 511) / 512) {
    case 1: return launch_quant_ch<1>(x, ldx, rows, K, q, s, st);
    case 2: return launch_quant_ch<2>(x, ldx, rows, K, q, s, st);
    case 3: return launch_quant_ch<3>(x, ldx, rows, K, q, s, st);
    case 4: return launch_quant_ch<4>(x, ldx, rows, K, q, s, st);
    case 5: return launch_quant_ch<5>(x, ldx, rows, K, q, s, st);
    case 6: return launch_quant_ch<6>(x, ldx, rows, K, q, s, st);
    case 7: return launch_quant_ch<7>(x, ldx, rows, K, q, s, st);
    default: return launch_quant_ch<8>(x, ldx, rows, K, q, s, st);
  }
}

__global__ void copy_f32_kernel(const float* a, float* b, int64_t n, const int32_t* gate) {
  if (gate_closed(gate)) return;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) b[i] = a[i];
}

hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(copy_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, dst, n, launch_gate());
  return hipGetLastError();
}

__global__ void fill_i32_kernel(int32_t* p, int32_t v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

// forward declaration: plain RMSNorm is the fused kernel with no partials to add
hipError_t launch_resid_add_rmsnorm(float* resid, const float* parts, int nparts, int64_t pstride, const void* g,
                                    void* y, int rows, int d, float eps, int bf, int* status, hipStream_t s);

hipError_t launch_rmsnorm(const float* x, const void* g, void* y, int rows, int d, float eps, int bf,
                          int* status, hipStream_t s) {
  return launch_resid_add_rmsnorm(const_cast<float*>(x), nullptr, 0, 0, g, y, rows, d, eps, bf, status, s);
}

// resid += sum_s parts[s] (split-K partials, in part order); y = RMSNorm(resid) * g.  One block per
// row and one thread per 4 columns (d / 4 threads rounded up to whole waves, d <= 4096), so a row's
// loads are spread over up to 16 waves and every load of a thread issues before its sums.
constexpr int MAX_PARTS_ADD = 8;
DG_DEV float block_sum_f(float v, float* red) {
  v = wave_sum(v);
  const int nw = (blockDim.x + 63) >> 6;
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < nw; ++w) tot += red[w];   // fixed order: every thread gets the same sum
  return tot;
}

template <class T>
DG_DEV void store4(T* dst, f32x4_v v);
template <>
DG_DEV void store4<float>(float* dst, f32x4_v v) { *reinterpret_cast<f32x4_v*>(dst) = v; }
template <>
DG_DEV void store4<bf16_t>(bf16_t* dst, f32x4_v v) {
  uint2 w;
  w.x = pack_bf2(v[0], v[1]);
  w.y = pack_bf2(v[2], v[3]);
  *reinterpret_cast<uint2*>(dst) = w;
}
template <class T>
DG_DEV f32x4_v load4(const T* src);
template <>
DG_DEV f32x4_v load4<float>(const float* src) { return *reinterpret_cast<const f32x4_v*>(src); }
template <>
DG_DEV f32x4_v load4<bf16_t>(const bf16_t* src) {
  const uint2 w = *reinterpret_cast<const uint2*>(src);
  return f32x4_v{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                 __uint_as_float(w.y & 0xffff0000u)};
}

// NP = number of partials, a compile-time constant so the loads stay in registers
template <class T, int NP>
__global__ __launch_bounds__(1024) void resid_add_rmsnorm_kernel(float* resid, const float* parts, int64_t pstride,
                                                                 const T* g, T* y, int d, float eps, int* status,
                                                                 const int32_t* gate) {
  if (gate_closed(gate)) return;
  __shared__ float red[16];
  const int r = blockIdx.x;
  const int c = threadIdx.x * 4;
  f32x4_v a = {0.f, 0.f, 0.f, 0.f};
  if (c < d) {
    float* xr = resid + (int64_t)r * d + c;
    f32x4_v pv[NP > 0 ? NP : 1];
#pragma unroll
    for (int q = 0; q < NP; ++q) pv[q] = *reinterpret_cast<const f32x4_v*>(parts + q * pstride + (int64_t)r * d + c);
    a = *reinterpret_cast<const f32x4_v*>(xr);
#pragma unroll
    for (int q = 0; q < NP; ++q) a += pv[q];
    if constexpr (NP > 0) *reinterpret_cast<f32x4_v*>(xr) = a;
  }
  const float tot = block_sum_f(a[0] * a[0] + a[1] * a[1] + a[2] * a[2] + a[3] * a[3], red);
  const float inv = rsqrtf(tot / (float)d + eps);
  if (threadIdx.x == 0 && status && !isfinite(tot)) atomicOr(status, 2);
  if (c < d) store4<T>(y + (int64_t)r * d + c, a * inv * load4<T>(g + c));
}

template <class T, int NP>
static void launch_ran(dim3 grid, dim3 block, hipStream_t s, float* resid, const float* parts, int nparts,
                       int64_t pstride, const void* g, void* y, int d, float eps, int* status) {
  if constexpr (NP < MAX_PARTS_ADD) {
    if (nparts > NP) return launch_ran<T, NP + 1>(grid, block, s, resid, parts, nparts, pstride, g, y, d, eps, status);
  }
  hipLaunchKernelGGL((resid_add_rmsnorm_kernel<T, NP>), grid, block, 0, s, resid, parts, pstride, (const T*)g, (T*)y,
                     d, eps, status, launch_gate());
}

hipError_t launch_resid_add_rmsnorm(float* resid, const float* parts, int nparts, int64_t pstride, const void* g,
                                    void* y, int rows, int d, float eps, int bf, int* status, hipStream_t s) {
  if (d % 4 || d > 4096 || nparts < 0 || nparts > MAX_PARTS_ADD) return hipErrorInvalidValue;
  const uintptr_t al = bf ? 7 : 15;   // 4-column vector accesses of g and y
  if (((uintptr_t)g & al) || ((uintptr_t)y & al)) return hipErrorInvalidValue;
  const dim3 block((d / 4 + 63) / 64 * 64);
  if (bf) launch_ran<bf16_t, 0>(dim3(rows), block, s, resid, parts, nparts, pstride, g, y, d, eps, status);
  else launch_ran<float, 0>(dim3(rows), block, s, resid, parts, nparts, pstride, g, y, d, eps, status);
  return hipGetLastError();
}

// new keys [B][Hkv][n][dh] -> cache rows, new values d-major [B][Hkv][dh][vn_ld] -> cache columns
// ([B][Hkv][dh][cap]): position p in slot p (global) or p % window (local ring; only the last
// `window` of the new positions are kept)
struct AppendArgs {
  const char* kn; const char* vn; char* kc; char* vc;
  const int32_t* mask;    // device [B] or null: canvases with mask[b] == 0 are not appended
  int B, n, vn_ld, Hkv, esz, row_bytes, cap, window, is_global;
  const int32_t* plen;    // device [B] prefix lengths (first position of the new rows)
  int max_prefix;
  const int32_t* gate;
};

__global__ void kv_append_kernel(AppendArgs a) {
  if (gate_closed(a.gate)) return;
  // keys: one 16-byte chunk of a key row per thread
  const int chunks = a.row_bytes / 16;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total_k = (int64_t)a.B * a.Hkv * a.n * chunks;
  if (idx < total_k) {
    const int ch = (int)(idx % chunks);
    int64_t t = idx / chunks;
    const int j = (int)(t % a.n); t /= a.n;
    const int g = (int)(t % a.Hkv);
    const int b = (int)(t / a.Hkv);
    if (!a.is_global && j < a.n - a.window) return;
    if (a.mask && a.mask[b] == 0) return;
    const int pos = prefix_of(a.plen, b, a.max_prefix) + j;
    const int slot = a.is_global ? pos : pos % a.window;
    if (slot >= a.cap) return;                      // never past the slots the host validated
    const int64_t src = (((int64_t)b * a.Hkv + g) * a.n + j) * a.row_bytes + ch * 16;
    const int64_t dst = (((int64_t)b * a.Hkv + g) * a.cap + slot) * a.row_bytes + ch * 16;
    *reinterpret_cast<u32x4*>(a.kc + dst) = *reinterpret_cast<const u32x4*>(a.kn + src);
    return;
  }
  // values (d-major): one element per thread, (b, g, d, j) -> column slot of row d
  const int64_t v = idx - total_k;
  const int dh = a.row_bytes / a.esz;
  if (v >= (int64_t)a.B * a.Hkv * dh * a.n) return;
  const int j = (int)(v % a.n);
  const int64_t row = v / a.n;                      // (b * Hkv + g) * dh + d
  const int b = (int)(row / ((int64_t)a.Hkv * dh));
  if (!a.is_global && j < a.n - a.window) return;
  if (a.mask && a.mask[b] == 0) return;
  const int pos = prefix_of(a.plen, b, a.max_prefix) + j;
  const int slot = a.is_global ? pos : pos % a.window;
  if (slot >= a.cap) return;
  if (a.esz == 2)
    reinterpret_cast<uint16_t*>(a.vc)[row * a.cap + slot] = reinterpret_cast<const uint16_t*>(a.vn)[row * a.vn_ld + j];
  else
    reinterpret_cast<uint32_t*>(a.vc)[row * a.cap + slot] = reinterpret_cast<const uint32_t*>(a.vn)[row * a.vn_ld + j];
}

hipError_t launch_kv_append(const void* kn, const void* vn, int vn_ld, void* kc, void* vc, int B, int n, int Hkv,
                            int dh, int cap, int window, int is_global, const int32_t* plen, int max_prefix,
                            const int32_t* seq_mask, int bf, hipStream_t s) {
  AppendArgs a;
  a.kn = (const char*)kn; a.vn = (const char*)vn; a.kc = (char*)kc; a.vc = (char*)vc;
  a.mask = seq_mask;
  a.B = B; a.n = n; a.vn_ld = vn_ld; a.Hkv = Hkv; a.esz = bf ? 2 : 4; a.row_bytes = dh * a.esz; a.cap = cap; a.window = window;
  a.is_global = is_global;
  a.plen = plen;
  a.max_prefix = max_prefix;
  a.gate = launch_gate();
  const int64_t total = (int64_t)B * Hkv * n * (a.row_bytes / 16) + (int64_t)B * Hkv * dh * n;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// resid[t] += (sum_{s<k} gate[t][s] * y[inv_perm[t*k+s]] + shared[t]), slots in order, with the
// expert rows y and shared in the activation type T; then, when g is given, out[t] =
// RMSNorm(resid[t]) * g (the next layer's attention norm, or the final norm).  One block per row and one thread per 4 columns (d / 4 threads rounded up to whole waves,
// so a 2816-wide row runs 11 waves): every load of the row (k gathered expert rows, the shared
// row, the residual) issues before the sums.
template <int K, class T>
__global__ __launch_bounds__(1024) void moe_combine_norm_kernel(float* resid, const T* y, const T* shared,
                                                                const float* gates, const int32_t* inv_perm,
                                                                int rows, int d, int k, const T* g, T* out,
                                                                float eps, int* status, const int32_t* gate) {
  if (gate_closed(gate)) return;
  __shared__ float red[16];
  const int t = blockIdx.x;
  const int c = threadIdx.x * 4;
  f32x4_v a = {0.f, 0.f, 0.f, 0.f};
  if (c < d) {
    f32x4_v yv[K];
    float gv[K];
#pragma unroll
    for (int s = 0; s < K; ++s) {
      const int sc = min(s, k - 1);
      // grouped positions are a permutation of [0, rows*k); the clamp only guards the read
      const int pos = min(max(inv_perm[(int64_t)t * k + sc], 0), rows * k - 1);
      gv[s] = s < k ? gates[(int64_t)t * k + sc] : 0.f;
      yv[s] = load4<T>(y + (int64_t)pos * d + c);
    }
    const f32x4_v sh = load4<T>(shared + (int64_t)t * d + c);
    f32x4_v* rp = reinterpret_cast<f32x4_v*>(resid + (int64_t)t * d + c);
    const f32x4_v r0 = *rp;
    f32x4_v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < K; ++s)
      if (s < k) acc += gv[s] * yv[s];
    a = r0 + (acc + sh);
    *rp = a;
  }
  if (!g) return;
  const float tot = block_sum_f(a[0] * a[0] + a[1] * a[1] + a[2] * a[2] + a[3] * a[3], red);
  const float inv = rsqrtf(tot / (float)d + eps);
  if (threadIdx.x == 0 && status && !isfinite(tot)) atomicOr(status, 2);
  if (c < d) store4<T>(out + (int64_t)t * d + c, a * inv * load4<T>(g + c));
}

template <int K>
static void combine_k(int bf, float* resid, const void* y, const void* shared, const float* gates,
                      const int32_t* inv_perm, int rows, int d, int k, const void* g, void* out, float eps,
                      int* status, hipStream_t s) {
  const dim3 block((d / 4 + 63) / 64 * 64);
  if (bf)
    hipLaunchKernelGGL((moe_combine_norm_kernel<K, bf16_t>), dim3(rows), block, 0, s, resid, (const bf16_t*)y,
                       (const bf16_t*)shared, gates, inv_perm, rows, d, k, (const bf16_t*)g, (bf16_t*)out, eps, status,
                       launch_gate());
  else
    hipLaunchKernelGGL((moe_combine_norm_kernel<K, float>), dim3(rows), block, 0, s, resid, (const float*)y,
                       (const float*)shared, gates, inv_perm, rows, d, k, (const float*)g, (float*)out, eps, status,
                       launch_gate());
}

hipError_t launch_moe_combine_norm(float* resid, const void* y, const void* shared, const float* gates,
                                   const int32_t* inv_perm, int rows, int d, int k, const void* g, void* out,
                                   float eps, int bf, int* status, hipStream_t s) {
  if (d % 4 || d > 4096) return hipErrorInvalidValue;
  const uintptr_t al = bf ? 7 : 15;   // 4-column vector accesses of g and out
  if (g && (((uintptr_t)g & al) || ((uintptr_t)out & al))) return hipErrorInvalidValue;
  if (k <= 2) combine_k<2>(bf, resid, y, shared, gates, inv_perm, rows, d, k, g, out, eps, status, s);
  else if (k <= 8) combine_k<8>(bf, resid, y, shared, gates, inv_perm, rows, d, k, g, out, eps, status, s);
  else combine_k<16>(bf, resid, y, shared, gates, inv_perm, rows, d, k, g, out, eps, status, s);
  return hipGetLastError();
}

__global__ void advance_prefix_kernel(int32_t* plen, int B, int n, const int32_t* mask, const int32_t* gate) {
  if (gate_closed(gate)) return;
  const int b = threadIdx.x;
  if (b < B && (!mask || mask[b] != 0)) plen[b] += n;
}

hipError_t launch_advance_prefix(int32_t* plen, int B, int n, const int32_t* seq_mask, hipStream_t s) {
  if (B > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(advance_prefix_kernel, dim3(1), dim3(1024), 0, s, plen, B, n, seq_mask, launch_gate());
  return hipGetLastError();
}

__global__ void all_set_kernel(const int32_t* v, int n, int32_t* flag) {
  int all = 1;
  for (int i = threadIdx.x; i < n; i += 64) all &= v[i] != 0;
  for (int o = 32; o > 0; o >>= 1) all &= __shfl_xor(all, o, 64);
  if (threadIdx.x == 0) *flag = all;
}

hipError_t launch_all_set(const int32_t* v, int n, int32_t* flag, hipStream_t s) {
  hipLaunchKernelGGL(all_set_kernel, dim3(1), dim3(64), 0, s, v, n, flag);
  return hipGetLastError();
}

// Valid tokens of block-AR canvases out [K][B][L]: one wave per sequence b walks the canvases in
// order; n[k][b] = position of the sequence's first eos in canvas k (tokens before it), L when
// the canvas holds none, 0 for canvases after the first eos; seen[k][b] = canvas k holds an eos.
__global__ __launch_bounds__(64) void valid_tokens_kernel(const int32_t* out, int K, int B, int L, int32_t eos,
                                                          int32_t* valid, int32_t* seen) {
  const int b = blockIdx.x, lane = threadIdx.x;
  bool ended = false;
  for (int k = 0; k < K; ++k) {
    const int32_t* c = out + ((int64_t)k * B + b) * L;
    int first = L;
    for (int i = lane; i < L; i += 64)
      if (c[i] == eos) { first = i; break; }
    for (int o = 32; o > 0; o >>= 1) first = min(first, __shfl_xor(first, o, 64));
    if (lane == 0) {
      valid[(int64_t)k * B + b] = ended ? 0 : first;
      if (seen) seen[(int64_t)k * B + b] = first < L;
    }
    ended = ended || first < L;
  }
}

hipError_t launch_valid_tokens(const int32_t* out, int K, int B, int L, int32_t eos, int32_t* valid, int32_t* seen,
                               hipStream_t s) {
  hipLaunchKernelGGL(valid_tokens_kernel, dim3(B), dim3(64), 0, s, out, K, B, L, eos, valid, seen);
  return hipGetLastError();
}

}  // namespace dg
