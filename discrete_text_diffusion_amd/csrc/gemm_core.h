// The MFMA tile engine behind every GEMM-shaped step of the denoise step (projections, expert
// FFNs, router, LM head).  C[BM x BN] += A[BM x K] . B[BN x K]^T with both operands K-contiguous.
//
// Block: 256 threads = 4 waves arranged WM x WN; wave tile (BM/WM) x (BN/WN) in 16x16 MFMA
// blocks.  K advances in tiles of 128 bytes per row (64 bf16 or 32 fp32); each tile goes
// global -> registers -> LDS (double buffered, one barrier per tile).  Rows beyond the operand
// are zero-filled.  fp8 e4m3 B rows are widened to bf16 on the way into LDS (exact).
#pragma once
#include "common.h"

namespace dg {

struct fp8_t { uint8_t v; };  // storage tag for e4m3 weights

constexpr int ROW_BYTES = 128;            // data bytes of one operand row per K tile
constexpr int ROW_STRIDE = 144;           // + 16 bytes of padding against bank conflicts

// e4m3 (OCP, finite only) -> bf16 word, exact: normal codes shift into place with the exponent
// re-biased from 7 to 127; subnormal codes m * 2^-9 are normalised.
DG_DEV uint32_t e4m3_to_bf16(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 8;
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  if (e) return s | ((e + 120u) << 7) | (m << 4);
  if (m == 0) return s;
  // m in 1..7: value m * 2^-9; leading bit position p (0..2)
  const uint32_t p = 31u - __builtin_clz(m);
  const uint32_t frac = (m << (3 - p)) & 7u;           // bits below the leading one
  return s | ((p + 118u) << 7) | (frac << 4);          // 2^(p-9) -> biased exponent p+118
}

DG_DEV u32x4 widen_fp8_lo(const u32x4& w) {           // bytes 0..7 -> 8 bf16
  u32x4 r;
  r.x = e4m3_to_bf16(w.x & 0xff) | (e4m3_to_bf16((w.x >> 8) & 0xff) << 16);
  r.y = e4m3_to_bf16((w.x >> 16) & 0xff) | (e4m3_to_bf16(w.x >> 24) << 16);
  r.z = e4m3_to_bf16(w.y & 0xff) | (e4m3_to_bf16((w.y >> 8) & 0xff) << 16);
  r.w = e4m3_to_bf16((w.y >> 16) & 0xff) | (e4m3_to_bf16(w.y >> 24) << 16);
  return r;
}
DG_DEV u32x4 widen_fp8_hi(const u32x4& w) {           // bytes 8..15
  u32x4 t{w.z, w.w, 0, 0};
  return widen_fp8_lo(t);
}

// DEPTH = K tiles in flight from global memory while one is computed (1 or 2).
template <class TA, class TB, int BM, int BN, int WM, int WN, int DEPTH = 1>
struct GemmTile {
  static_assert(WM * WN == 4, "4 waves");
  static constexpr int FM = BM / WM / 16;
  static constexpr int FN = BN / WN / 16;
  static_assert(FM >= 1 && FN >= 1, "wave tile at least 16x16");
  static constexpr bool B_FP8 = sizeof(TB) == 1;
  static constexpr int KT = ROW_BYTES / sizeof(TA);             // K elements per tile
  static constexpr int A_CHUNKS = BM * 8 / 256;                 // 16-byte loads per thread
  static constexpr int B_ROWCH = B_FP8 ? 4 : 8;                 // global 16-byte chunks per row
  static constexpr int B_CHUNKS = (BN * B_ROWCH + 255) / 256;
  static constexpr int LDS_A = BM * ROW_STRIDE;
  static constexpr int LDS_B = BN * ROW_STRIDE;
  static constexpr int LDS_BYTES = 2 * (LDS_A + LDS_B);
  static_assert(BM * 8 % 256 == 0, "A tile must split evenly over 256 threads");

  static_assert(DEPTH == 1 || DEPTH == 2, "pipeline depth");
  const char* a_ptr[A_CHUNKS];   // row base + chunk offset, or null (zero row)
  const char* b_ptr[B_CHUNKS];
  u32x4 ra[DEPTH][A_CHUNKS], rb[DEPTH][B_CHUNKS];

  // arow(r): pointer to A row r of the tile (element 0) or nullptr; likewise brow.
  template <class ARow, class BRow>
  DG_DEV void setup(ARow arow, BRow brow) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int q = t + 256 * i, r = q >> 3, kc = q & 7;
      const char* p = reinterpret_cast<const char*>(arow(r));
      a_ptr[i] = p ? p + kc * 16 : nullptr;
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
      const int q = t + 256 * i, r = q / B_ROWCH, kc = q % B_ROWCH;
      const char* p = (q < BN * B_ROWCH) ? reinterpret_cast<const char*>(brow(r)) : nullptr;
      b_ptr[i] = p ? p + kc * 16 : nullptr;
    }
  }

  template <int S>
  DG_DEV void load(int kt) {  // global -> register set S for K tile kt
    const size_t offa = (size_t)kt * ROW_BYTES;
    const size_t offb = (size_t)kt * (B_FP8 ? ROW_BYTES / 2 : ROW_BYTES);
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i)
      ra[S][i] = a_ptr[i] ? *reinterpret_cast<const u32x4*>(a_ptr[i] + offa) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i)
      rb[S][i] = b_ptr[i] ? *reinterpret_cast<const u32x4*>(b_ptr[i] + offb) : u32x4{0, 0, 0, 0};
  }

  template <int S>
  DG_DEV void store(char* lds) {  // register set S -> LDS buffer
    const int t = threadIdx.x;
    char* la = lds;
    char* lb = lds + LDS_A;
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int q = t + 256 * i, r = q >> 3, kc = q & 7;
      *reinterpret_cast<u32x4*>(la + r * ROW_STRIDE + kc * 16) = ra[S][i];
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
      const int q = t + 256 * i;
      if (q >= BN * B_ROWCH) continue;
      const int r = q / B_ROWCH, kc = q % B_ROWCH;
      if constexpr (B_FP8) {
        *reinterpret_cast<u32x4*>(lb + r * ROW_STRIDE + kc * 32) = widen_fp8_lo(rb[S][i]);
        *reinterpret_cast<u32x4*>(lb + r * ROW_STRIDE + kc * 32 + 16) = widen_fp8_hi(rb[S][i]);
      } else {
        *reinterpret_cast<u32x4*>(lb + r * ROW_STRIDE + kc * 16) = rb[S][i];
      }
    }
  }

  DG_DEV static void compute(const char* lds, f32x4_v (&acc)[FM][FN]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const char* la = lds + (wm * FM * 16 + (lane & 15)) * ROW_STRIDE + (lane >> 4) * 16;
    const char* lb = lds + LDS_A + (wn * FN * 16 + (lane & 15)) * ROW_STRIDE + (lane >> 4) * 16;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const u32x4*>(la + i * 16 * ROW_STRIDE + c * 64);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const u32x4*>(lb + j * 16 * ROW_STRIDE + c * 64);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) Mfma<TA>::mma(acc[i][j], af[i], bfr[j]);
    }
  }

  // Full K loop; K must be a multiple of KT.  `lds` holds LDS_BYTES (two tile buffers).
  // DEPTH 1: tile kt+1 is loaded while kt is computed.  DEPTH 2: tiles kt+1 and kt+2 are in
  // flight; the loop is unrolled by two so every register set index is a constant.
  DG_DEV void run(char* lds, int K, f32x4_v (&acc)[FM][FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};
    const int nk = K / KT;
    char* buf0 = lds;
    char* buf1 = lds + LDS_A + LDS_B;
    if constexpr (DEPTH == 1) {
      load<0>(0);
      store<0>(buf0);
      __syncthreads();
      for (int kt = 0; kt < nk; ++kt) {
        char* cur = (kt & 1) ? buf1 : buf0;
        char* nxt = (kt & 1) ? buf0 : buf1;
        if (kt + 1 < nk) load<0>(kt + 1);
        compute(cur, acc);
        if (kt + 1 < nk) store<0>(nxt);
        __syncthreads();
      }
    } else {
      // set 0 carries even tiles, set 1 odd tiles; buffer 0 even tiles, buffer 1 odd tiles
      load<0>(0);
      if (nk > 1) load<1>(1);
      store<0>(buf0);
      __syncthreads();
      for (int kt = 0; kt < nk; kt += 2) {
        // even tile kt in buf0; tile kt+1 in flight in set 1
        if (kt + 2 < nk) load<0>(kt + 2);
        compute(buf0, acc);
        if (kt + 1 < nk) store<1>(buf1);
        __syncthreads();
        if (kt + 1 >= nk) break;
        // odd tile kt+1 in buf1; tile kt+2 in flight in set 0
        if (kt + 3 < nk) load<1>(kt + 3);
        compute(buf1, acc);
        if (kt + 2 < nk) store<0>(buf0);
        __syncthreads();
      }
    }
  }

  // position of accumulator element (i, j, e) inside the block tile
  DG_DEV static int row_of(int i, int e) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    return (wave / WN) * FM * 16 + i * 16 + 4 * (lane >> 4) + e;
  }
  DG_DEV static int col_of(int j) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    return (wave % WN) * FN * 16 + j * 16 + (lane & 15);
  }
};

}  // namespace dg
