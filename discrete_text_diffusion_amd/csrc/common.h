// Device-side building blocks shared by the gfx950 kernels of libdg.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define DG_DEV __device__ __forceinline__

namespace dg {

// A closed launch gate (see launch_gate): the whole grid returns before doing anything.
DG_DEV bool gate_closed(const int32_t* gate) { return gate != nullptr && *gate != 0; }

// A canvas's prefix length from the device array, clamped to [0, max_prefix] so that no cache
// access can leave the slots the host validated.
DG_DEV int prefix_of(const int32_t* plen, int b, int max_prefix) { return min(max(plen[b], 0), max_prefix); }

typedef uint16_t bf16_t;  // raw bf16 word

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_v;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_v;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16 bytes, lives in VGPRs
typedef int i32x8 __attribute__((ext_vector_type(8)));       // 32 bytes: one f8f6f4 MFMA operand

// ---------------------------------------------------------------- bf16 <-> f32 -------------------
DG_DEV float bf2f(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// round to nearest even (gfx950 v_cvt_pk_bf16_f32); NaN stays NaN
typedef __bf16 hw_bf16x2 __attribute__((ext_vector_type(2)));
typedef float hw_f32x2 __attribute__((ext_vector_type(2)));
DG_DEV bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

DG_DEV uint32_t pack_bf2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((hw_f32x2){a, b}, hw_bf16x2));
}

// two floats as IEEE half (round to nearest even) in one word, and back
typedef _Float16 hw_f16x2 __attribute__((ext_vector_type(2)));
DG_DEV uint32_t pack_h2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((hw_f32x2){a, b}, hw_f16x2));
}
DG_DEV void unpack_h2(uint32_t w, float& a, float& b) {
  const hw_f32x2 f = __builtin_convertvector(__builtin_bit_cast(hw_f16x2, w), hw_f32x2);
  a = f[0];
  b = f[1];
}

// All-reduce over the 16 lanes of each row (lanes 16r .. 16r + 15) with DPP moves, no LDS: quad
// swaps (xor 1, xor 2), then the half-row and row mirrors.  Every step pairs lanes (i with its
// partner, the partner with i), so all lanes of a row end with the same value, sums included.
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;
template <int CTRL>
DG_DEV int dpp_mov(int v) { return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false); }
template <int CTRL>
DG_DEV float dpp_movf(float v) { return __int_as_float(dpp_mov<CTRL>(__float_as_int(v))); }
DG_DEV float row16_max(float v) {
  v = fmaxf(v, dpp_movf<DPP_XOR1>(v));
  v = fmaxf(v, dpp_movf<DPP_XOR2>(v));
  v = fmaxf(v, dpp_movf<DPP_HALF_MIRROR>(v));
  return fmaxf(v, dpp_movf<DPP_MIRROR>(v));
}
DG_DEV int row16_min(int v) {
  v = min(v, dpp_mov<DPP_XOR1>(v));
  v = min(v, dpp_mov<DPP_XOR2>(v));
  v = min(v, dpp_mov<DPP_HALF_MIRROR>(v));
  return min(v, dpp_mov<DPP_MIRROR>(v));
}
DG_DEV float row16_sum(float v) {
  v += dpp_movf<DPP_XOR1>(v);
  v += dpp_movf<DPP_XOR2>(v);
  v += dpp_movf<DPP_HALF_MIRROR>(v);
  return v + dpp_movf<DPP_MIRROR>(v);
}
DG_DEV int row16_sum_i(int v) {
  v += dpp_mov<DPP_XOR1>(v);
  v += dpp_mov<DPP_XOR2>(v);
  v += dpp_mov<DPP_HALF_MIRROR>(v);
  return v + dpp_mov<DPP_MIRROR>(v);
}
// largest key, ties to the lower id
template <int CTRL>
DG_DEV void argmax_step(float& k, int& id) {
  const float ok = dpp_movf<CTRL>(k);
  const int oi = dpp_mov<CTRL>(id);
  if (ok > k || (ok == k && oi < id)) { k = ok; id = oi; }
}
DG_DEV void row16_argmax(float& k, int& id) {
  argmax_step<DPP_XOR1>(k, id);
  argmax_step<DPP_XOR2>(k, id);
  argmax_step<DPP_HALF_MIRROR>(k, id);
  argmax_step<DPP_MIRROR>(k, id);
}
// the two values a lane sees after the gfx950 row-pair swap (rows 2j, 2j + 1) or half swap
// (lanes 0..31, 32..63) of v with itself: its own and its partner's, in the same order in both
DG_DEV void pair16(uint32_t v, uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  a = r[0];
  b = r[1];
}
DG_DEV void pair32(uint32_t v, uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  a = r[0];
  b = r[1];
}

// element access for the two activation types
template <class T> struct Elem;
template <> struct Elem<float> {
  static DG_DEV float load(const float* p) { return *p; }
  static DG_DEV float to_f(float v) { return v; }
  static DG_DEV float from_f(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static DG_DEV float load(const bf16_t* p) { return bf2f(*p); }
  static DG_DEV float to_f(bf16_t v) { return bf2f(v); }
  static DG_DEV bf16_t from_f(float v) { return f2bf(v); }
};

// ---------------------------------------------------------------- MFMA -------------------------
// 16x16 output tile; lane l holds rows 4*(l/16)+j (j = 0..3) of column l%16.
// bf16: one 16x16x32 product; A lane supplies A[l%16][8*(l/16)..+7], B lane B[8*(l/16)..+7][l%16].
// f32 : a 16-byte fragment holds 4 consecutive k; four 16x16x4 products, product j taking
//       element j, so the 16 k of a fragment column are summed in full.
template <class T> struct Mfma;
template <> struct Mfma<bf16_t> {
  static constexpr int K_PER_FRAG = 32;  // k covered by one 16-byte-per-lane fragment
  static DG_DEV void mma(f32x4_v& acc, const u32x4& a, const u32x4& b) {
    bf16x8_v av = *reinterpret_cast<const bf16x8_v*>(&a);
    bf16x8_v bv = *reinterpret_cast<const bf16x8_v*>(&b);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  static constexpr int K_PER_FRAG = 16;
  static DG_DEV void mma(f32x4_v& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

// ---------------------------------------------------------------- wave reductions --------------
// over the wave, the same value in every lane: row all-reduce, then rows paired, then halves
DG_DEV float wave_sum(float v) {
  uint32_t a, b;
  v = row16_sum(v);
  pair16(__float_as_uint(v), a, b);
  v = __uint_as_float(a) + __uint_as_float(b);
  pair32(__float_as_uint(v), a, b);
  return __uint_as_float(a) + __uint_as_float(b);
}
DG_DEV int wave_sum_i(int v) {
  uint32_t a, b;
  v = row16_sum_i(v);
  pair16((uint32_t)v, a, b);
  v = (int)(a + b);
  pair32((uint32_t)v, a, b);
  return (int)(a + b);
}
DG_DEV float wave_max(float v) {
  uint32_t a, b;
  v = row16_max(v);
  pair16(__float_as_uint(v), a, b);
  v = fmaxf(__uint_as_float(a), __uint_as_float(b));
  pair32(__float_as_uint(v), a, b);
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}

// SiLU g * sigmoid(g) with the hardware reciprocal (about 1 ulp) in place of an IEEE division:
// exp(-g) overflows to +inf for very negative g, whose reciprocal is 0, so the result is -0 as
// with the division
DG_DEV float silu(float g) { return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)); }

// ---------------------------------------------------------------- Philox4x32-10 ---------------
// Salmon et al., SC'11: ten rounds; each multiplies counter words 0 and 2 by fixed constants,
// mixes the high halves with words 1, 3 and the round key; the key is bumped by Weyl constants.
// One 32 x 32 -> 64-bit product per word (v_mad_u64_u32 gives both halves in one instruction);
// the three-way exclusive or is one v_bitop3_b32 (truth table 0x96).
DG_DEV uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) { return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96); }

DG_DEV void philox_round(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3, uint32_t k0, uint32_t k1) {
  const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u, p1 = (uint64_t)c2 * 0xCD9E8D57u;
  const uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0), n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
  c0 = n0; c1 = (uint32_t)p1; c2 = n2; c3 = (uint32_t)p0;
}

DG_DEV u32x4 philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    philox_round(c0, c1, c2, c3, k0, k1);
    k0 += 0x9E3779B9u; k1 += 0xBB67AE85u;
  }
  return u32x4{c0, c1, c2, c3};
}

enum : uint32_t { TAG_GUMBEL = 0, TAG_JUMP = 1, TAG_INIT = 2, TAG_NOISE_KEEP = 3, TAG_NOISE_TOKEN = 4, TAG_RENOISE = 5 };

DG_DEV uint32_t pick(const u32x4& w, int j) {
  return j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w;
}

// (w >> 8) * 2^-24 in [0, 1): exact in float
DG_DEV float unit_co(uint32_t w) { return (float)(w >> 8) * 5.9604644775390625e-08f; }
// ((w >> 9) + 1/2) * 2^-23 in (0, 1), exact in float: the float 1 + (w >> 9) 2^-23 (mantissa bits
// set directly) minus (1 - 2^-24); the difference of two floats within a factor 2 is exact
DG_DEV float unit_oo(uint32_t w) { return __uint_as_float(0x3f800000u | (w >> 9)) - 0.999999940395355224609375f; }

DG_DEV int32_t token_of(uint32_t w, int32_t vocab, int32_t vocab_log2) {
  if (vocab_log2 >= 0) return vocab_log2 == 0 ? 0 : (int32_t)(w >> (32 - vocab_log2));
  return (int32_t)(((uint64_t)w * (uint64_t)vocab) >> 32);
}

}  // namespace dg
