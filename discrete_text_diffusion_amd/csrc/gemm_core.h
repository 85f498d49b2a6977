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

template <class TA, class TB, int BM, int BN, int WM, int WN>
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

  const char* a_ptr[A_CHUNKS];   // row base + chunk offset, or null (zero row)
  const char* b_ptr[B_CHUNKS];
  u32x4 ra[A_CHUNKS], rb[B_CHUNKS];

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

  DG_DEV void load(int kt) {  // global -> registers for K tile kt
    const size_t offa = (size_t)kt * ROW_BYTES;
    const size_t offb = (size_t)kt * (B_FP8 ? ROW_BYTES / 2 : ROW_BYTES);
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i)
      ra[i] = a_ptr[i] ? *reinterpret_cast<const u32x4*>(a_ptr[i] + offa) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i)
      rb[i] = b_ptr[i] ? *reinterpret_cast<const u32x4*>(b_ptr[i] + offb) : u32x4{0, 0, 0, 0};
  }

  DG_DEV void store(char* lds) {  // registers -> LDS buffer
    const int t = threadIdx.x;
    char* la = lds;
    char* lb = lds + LDS_A;
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int q = t + 256 * i, r = q >> 3, kc = q & 7;
      *reinterpret_cast<u32x4*>(la + r * ROW_STRIDE + kc * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
      const int q = t + 256 * i;
      if (q >= BN * B_ROWCH) continue;
      const int r = q / B_ROWCH, kc = q % B_ROWCH;
      if constexpr (B_FP8) {
        *reinterpret_cast<u32x4*>(lb + r * ROW_STRIDE + kc * 32) = widen_fp8_lo(rb[i]);
        *reinterpret_cast<u32x4*>(lb + r * ROW_STRIDE + kc * 32 + 16) = widen_fp8_hi(rb[i]);
      } else {
        *reinterpret_cast<u32x4*>(lb + r * ROW_STRIDE + kc * 16) = rb[i];
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

  // Full K loop; K must be a multiple of KT.  `lds` holds LDS_BYTES.
  DG_DEV void run(char* lds, int K, f32x4_v (&acc)[FM][FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};
    const int nk = K / KT;
    load(0);
    store(lds);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      char* cur = lds + (kt & 1) * (LDS_A + LDS_B);
      char* nxt = lds + ((kt + 1) & 1) * (LDS_A + LDS_B);
      if (kt + 1 < nk) load(kt + 1);
      compute(cur, acc);
      if (kt + 1 < nk) store(nxt);
      __syncthreads();
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
