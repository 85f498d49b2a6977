// The MFMA tile engine behind every GEMM-shaped step of the denoise step (projections, expert
// FFNs, router, LM head).  C[BM x BN] += A[BM x K] . B[BN x K]^T with both operands K-contiguous.
//
// Block: 256 threads = 4 waves arranged WM x WN; wave tile (BM/WM) x (BN/WN) in 16x16 MFMA
// blocks.  K advances in tiles of 128 bytes per row (64 bf16 or 32 fp32); each tile goes
// global -> registers -> LDS (double buffered, one barrier per tile).  Rows beyond the operand
// are zero-filled.  fp8 e4m3 B rows are widened to bf16 on the way into LDS (exact); MXFP4 B rows
// (e2m1 codes with one power-of-two scale per 32 elements) are widened with their scale applied
// (exact: an e2m1 value times a power of two is a bf16 value).
#pragma once
#include <type_traits>
#include "common.h"

namespace dg {

struct fp8_t { uint8_t v; };    // storage tag for e4m3 weights
struct fp4x2_t { uint8_t v; };  // storage tag for MXFP4 weights: two e2m1 codes per byte, element 2j low
struct fp8a_t { uint8_t v; };   // storage tag for e4m3 activation codes (W8A8: a scale per row)
template <class T> constexpr bool is_fp8_v = std::is_same<T, fp8_t>::value;
template <class T> constexpr bool is_fp4_v = std::is_same<T, fp4x2_t>::value;
template <class T> constexpr bool is_fp8a_v = std::is_same<T, fp8a_t>::value;

constexpr int ROW_BYTES = 128;            // data bytes of one operand row per K tile
constexpr int ROW_STRIDE = 144;           // + 16 bytes of padding against bank conflicts

// e4m3 codes -> bf16, exact (gfx950 scaled conversion with scale 1; the lower byte of each
// selected 16-bit half goes to the low bf16): bytes 0..7 of w, then bytes 8..15
DG_DEV uint32_t cvt_fp8_pair(uint32_t w, bool upper) {
  return upper ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))
               : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}
DG_DEV u32x4 widen_fp8_lo(const u32x4& w) {
  return u32x4{cvt_fp8_pair(w.x, false), cvt_fp8_pair(w.x, true), cvt_fp8_pair(w.y, false), cvt_fp8_pair(w.y, true)};
}
DG_DEV u32x4 widen_fp8_hi(const u32x4& w) {
  return u32x4{cvt_fp8_pair(w.z, false), cvt_fp8_pair(w.z, true), cvt_fp8_pair(w.w, false), cvt_fp8_pair(w.w, true)};
}

// e8m0 scale byte -> float 2^(s - 127) (s = 0: the subnormal 2^-127; s = 255: NaN)
DG_DEV float e8m0_scale(uint32_t s) {
  return __uint_as_float(s == 0 ? 0x00400000u : s == 255 ? 0x7fc00000u : s << 23);
}
// eight e2m1 codes (one word, element 2j in the low nibble of byte j) times the scale -> eight
// bf16 in element order (gfx950 scaled conversion; low nibble to the low half)
DG_DEV u32x4 widen_fp4_word(uint32_t w, float sc) {
  u32x4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
  return r;
}

// DEPTH = K tiles in flight from global memory while one is computed (1..4): register set s
// carries the tiles congruent to s mod DEPTH, LDS double-buffers the tile being computed.
template <class TA, class TB, int BM, int BN, int WM, int WN, int DEPTH = 1>
struct GemmTile {
  static constexpr int TILE_M = BM;
  static_assert(WM * WN == 4, "4 waves");
  static constexpr int FM = BM / WM / 16;
  static constexpr int FN = BN / WN / 16;
  static_assert(FM >= 1 && FN >= 1, "wave tile at least 16x16");
  static constexpr bool B_FP8 = is_fp8_v<TB>;
  static constexpr bool B_FP4 = is_fp4_v<TB>;
  static_assert(!(B_FP8 || B_FP4) || sizeof(TA) == 2, "quantised weights widen to bf16");
  static constexpr int KT = ROW_BYTES / sizeof(TA);             // K elements per tile
  static constexpr int A_CHUNKS = BM * 8 / 256;                 // 16-byte loads per thread
  static constexpr int B_ROWCH = B_FP8 ? 4 : B_FP4 ? 2 : 8;     // global 16-byte chunks per row
  static constexpr int B_TILE = B_ROWCH * 16;                   // stored bytes of a B row per K tile
  static constexpr int B_CHUNKS = (BN * B_ROWCH + 255) / 256;
  static constexpr int LDS_A = BM * ROW_STRIDE;
  static constexpr int LDS_B = BN * ROW_STRIDE;
  static constexpr int LDS_BYTES = 2 * (LDS_A + LDS_B);
  static_assert(BM * 8 % 256 == 0, "A tile must split evenly over 256 threads");

  static_assert(DEPTH >= 1 && DEPTH <= 4, "pipeline depth");
  const char* a_ptr[A_CHUNKS];   // row base + chunk offset, or null (zero row)
  const char* b_ptr[B_CHUNKS];
  const uint8_t* s_ptr[B_CHUNKS];   // MXFP4: the chunk's scale byte in K tile 0, or null
  u32x4 ra[DEPTH][A_CHUNKS], rb[DEPTH][B_CHUNKS];
  uint32_t rs[DEPTH][B_CHUNKS];

  // arow(r): pointer to A row r of the tile (element 0) or nullptr; likewise brow; srow (MXFP4):
  // the scale bytes of B row r (one per 32 elements) or nullptr.
  template <class ARow, class BRow>
  DG_DEV void setup(ARow arow, BRow brow) {
    setup(arow, brow, [](int) -> const uint8_t* { return nullptr; });
  }
  template <class ARow, class BRow, class SRow>
  DG_DEV void setup(ARow arow, BRow brow, SRow srow) {
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
      if constexpr (B_FP4) {
        const uint8_t* sp = p ? srow(r) : nullptr;
        s_ptr[i] = sp ? sp + kc : nullptr;
      }
    }
  }

  template <int S>
  DG_DEV void load(int kt) {  // global -> register set S for K tile kt
    const size_t offa = (size_t)kt * ROW_BYTES;
    const size_t offb = (size_t)kt * B_TILE;
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i)
      ra[S][i] = a_ptr[i] ? *reinterpret_cast<const u32x4*>(a_ptr[i] + offa) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
      rb[S][i] = b_ptr[i] ? *reinterpret_cast<const u32x4*>(b_ptr[i] + offb) : u32x4{0, 0, 0, 0};
      if constexpr (B_FP4) rs[S][i] = s_ptr[i] ? s_ptr[i][(size_t)kt * B_ROWCH] : 0u;
    }
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
      } else if constexpr (B_FP4) {
        const float sc = e8m0_scale(rs[S][i]);
        char* d = lb + r * ROW_STRIDE + kc * 64;
        *reinterpret_cast<u32x4*>(d) = widen_fp4_word(rb[S][i].x, sc);
        *reinterpret_cast<u32x4*>(d + 16) = widen_fp4_word(rb[S][i].y, sc);
        *reinterpret_cast<u32x4*>(d + 32) = widen_fp4_word(rb[S][i].z, sc);
        *reinterpret_cast<u32x4*>(d + 48) = widen_fp4_word(rb[S][i].w, sc);
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

  // Full K loop; K must be a multiple of KT.  `lds` holds LDS_BYTES (two tile buffers).  Tile kt
  // is computed from LDS buffer kt & 1 while tiles kt+1 .. kt+DEPTH are in flight in registers;
  // the loop is unrolled by DEPTH so every register set index is a constant.
  template <int J>
  DG_DEV void iter(int kt0, int nk, char* const (&buf)[2], f32x4_v (&acc)[FM][FN]) {
    const int kt = kt0 + J;
    if (kt >= nk) return;
    if (kt + DEPTH < nk) load<J>(kt + DEPTH);        // set J's tile kt is already in LDS
    compute(buf[kt & 1], acc);
    if (kt + 1 < nk) store<(J + 1) % DEPTH>(buf[(kt + 1) & 1]);
    __syncthreads();
  }
  template <int J>
  DG_DEV void prologue(int nk) {
    if constexpr (J < DEPTH) {
      if (J < nk) load<J>(J);
      prologue<J + 1>(nk);
    }
  }
  template <int J>
  DG_DEV void round(int kt0, int nk, char* const (&buf)[2], f32x4_v (&acc)[FM][FN]) {
    if constexpr (J < DEPTH) {
      iter<J>(kt0, nk, buf, acc);
      round<J + 1>(kt0, nk, buf, acc);
    }
  }
  DG_DEV void run(char* lds, int K, f32x4_v (&acc)[FM][FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};
    const int nk = K / KT;
    char* const buf[2] = {lds, lds + LDS_A + LDS_B};
    prologue<0>(nk);
    if (nk > 0) store<0>(buf[0]);
    __syncthreads();
    for (int kt0 = 0; kt0 < nk; kt0 += DEPTH) round<0>(kt0, nk, buf, acc);
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
