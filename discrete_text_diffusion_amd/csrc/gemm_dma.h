// MFMA tile engine with direct global -> LDS loads (gfx950 global_load_lds_dwordx4).
//
// C[BM x BN] += A[BM x K] . B[BN x K]^T, both operands K-contiguous, bf16 or fp32.  Each K tile
// is 128 bytes of every operand row.  One load instruction moves 16 bytes per lane straight
// into LDS at (wave-uniform base + 16 * lane), so a wave fills 8 consecutive 128-byte rows per
// instruction; no registers hold tiles in flight, which lets NS - 1 tiles stream from memory
// while one is multiplied (an NS-stage LDS ring, one barrier per tile).
//
// Bank-conflict-free fragment reads without padding: the 16-byte chunk c of row r lives in slot
// c ^ ((r >> 1) & 7) of that row.  A fragment read touches 16 consecutive rows at one logical
// chunk; rows of one parity share a half of the 64 banks and the swizzle gives the 8 rows of
// each parity 8 different slots, so the 16 lanes hit 64 distinct banks.
//
// Rows outside the operand are loaded from a clamped (valid) row: their products land only in
// output rows/columns that the caller never stores.
#pragma once
#include "common.h"
#include "gemm_core.h"

namespace dg {

#define DG_LDS_AS __attribute__((address_space(3)))
#define DG_GLOBAL_AS __attribute__((address_space(1)))

// Cache policy of a direct-to-LDS load (gfx950 CPol bits): DMA_CACHED for operands other blocks
// re-read from L2 (activations), DMA_STREAM (nt) for data read once per launch (weights, the
// embedding, KV caches): measured on MI355X, nt streams reach ~6.8 TB/s where cached loads of the
// same bytes reach ~6.0 TB/s.
constexpr int DMA_CACHED = 0, DMA_STREAM = 2;
template <int AUX = DMA_CACHED>
DG_DEV void dma16(const void* gsrc, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const DG_GLOBAL_AS void*)gsrc, (DG_LDS_AS void*)lds_wave_base, 16, 0, AUX);
}

// Workgroup barrier for LDS hand-offs: waits for this wave's LDS operations only.  A
// __syncthreads() carries a release fence, for which the compiler also drains every
// direct-to-LDS load still in flight (vmcnt(0)) and so serialises the load ring.  The memory
// clobber keeps the compiler from moving memory operations across it.
DG_DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// wait until at most n of this wave's vector-memory loads are outstanding (n <= 63)
template <int N>
DG_DEV void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] in [15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// B_AUX: cache policy of the B (weight) operand loads.  KPS: K tiles per ring stage (one wait and
// one barrier per stage: two tiles per stage halve the per-step synchronisation of long K loops).
template <class T, int BM, int BN, int WM, int WN, int NS, int B_AUX = DMA_STREAM, int KPS = 1>
struct GemmDma {
  static constexpr int TILE_M = BM;
  static constexpr int NW = WM * WN;                   // waves per block
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "rows per tile: multiples of 8 x waves");
  static_assert(NS >= 2 && NS <= 8, "stages");
  static_assert(KPS == 1 || KPS == 2, "K tiles per stage");
  static constexpr int FM = BM / WM / 16;
  static constexpr int FN = BN / WN / 16;
  static constexpr int KT = 128 / sizeof(T);          // K elements per tile
  static constexpr int KSTEP = KT * KPS;              // K elements per ring stage
  static constexpr int IA = BM / (8 * NW), IB = BN / (8 * NW);   // load instructions per wave per tile
  static constexpr int LPT = (IA + IB) * KPS;         // load instructions per wave per stage
  static constexpr int SUB = (BM + BN) * 128;         // one K tile of both operands
  static constexpr int STAGE = SUB * KPS;
  static constexpr int LDS_BYTES = NS * STAGE;
  static_assert((NS - 2) * LPT < 64, "vmcnt range");

  const char* a_src[IA];   // this lane's source row (+ its swizzled chunk) for each instruction
  const char* b_src[IB];

  // arow(r)/brow(r): pointer to element 0 of tile row r, or nullptr for rows past the operand,
  // for which row 0 of the tile (always valid) is loaded instead.
  template <class ARow, class BRow>
  DG_DEV void setup(ARow arow, BRow brow) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rr = lane >> 3, slot = lane & 7;
#pragma unroll
    for (int i = 0; i < IA; ++i) {
      const int r = (wave + NW * i) * 8 + rr;
      const char* p = reinterpret_cast<const char*>(arow(r));
      if (!p) p = reinterpret_cast<const char*>(arow(0));
      a_src[i] = p + ((slot ^ ((r >> 1) & 7)) * 16);
    }
#pragma unroll
    for (int i = 0; i < IB; ++i) {
      const int r = (wave + NW * i) * 8 + rr;
      const char* p = reinterpret_cast<const char*>(brow(r));
      if (!p) p = reinterpret_cast<const char*>(brow(0));
      b_src[i] = p + ((slot ^ ((r >> 1) & 7)) * 16);
    }
  }

  // weights of the activation type carry no scales
  template <class ARow, class BRow, class SRow>
  DG_DEV void setup(ARow arow, BRow brow, SRow) { setup(arow, brow); }

  // stage `stage` <- K tiles kt * KPS .. kt * KPS + KPS - 1
  DG_DEV void issue(char* lds, int kt, int stage) {
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int p = 0; p < KPS; ++p) {
      char* st = lds + stage * STAGE + p * SUB;
      const size_t off = (size_t)(kt * KPS + p) * 128;
#pragma unroll
      for (int i = 0; i < IA; ++i) dma16(a_src[i] + off, st + (wave + NW * i) * 8 * 128);
#pragma unroll
      for (int i = 0; i < IB; ++i) dma16<B_AUX>(b_src[i] + off, st + BM * 128 + (wave + NW * i) * 8 * 128);
    }
  }

  // wait for the oldest of `pending` outstanding tiles (pending = tiles issued and not yet
  // waited for): at most (pending - 1) tiles' loads may stay in flight
  template <int P>
  DG_DEV static void wait_pending(int pending) {
    if constexpr (P > 1) {
      if (pending >= P) { wait_vm<(P - 1) * LPT>(); return; }
      wait_pending<P - 1>(pending);
    } else {
      wait_vm<0>();
    }
  }
  DG_DEV static void wait_oldest(int pending) { wait_pending<NS - 1>(pending); }

  DG_DEV static void compute(const char* st, f32x4_v (&acc)[FM][FN]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int swz = (lane & 15) >> 1, kg = lane >> 4;
    if constexpr (FN >= 8 && KPS == 1) {
      // wide wave tiles (a row strip against many columns): the second chunk's B fragments are
      // read one by one as the first chunk's products free their registers, so those reads run
      // under the matrix work instead of after it (scheduling groups pin the interleaving; each
      // accumulator still adds chunk 0, then chunk 1)
      const char* la = st + (wm * FM * 16 + (lane & 15)) * 128;
      const char* lb = st + BM * 128 + (wn * FN * 16 + (lane & 15)) * 128;
      const int s0 = (kg ^ swz) * 16, s1 = ((4 + kg) ^ swz) * 16;
      u32x4 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const u32x4*>(la + i * 16 * 128 + s0);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const u32x4*>(lb + j * 16 * 128 + s0);
      __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int i = 0; i < FM; ++i) Mfma<T>::mma(acc[i][j], af[i], bfr[j]);
        bfr[j] = *reinterpret_cast<const u32x4*>(lb + j * 16 * 128 + s1);
        __builtin_amdgcn_sched_group_barrier(0x008, FM, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const u32x4*>(la + i * 16 * 128 + s1);
      __builtin_amdgcn_sched_group_barrier(0x100, FM, 0);
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) Mfma<T>::mma(acc[i][j], af[i], bfr[j]);
      __builtin_amdgcn_sched_group_barrier(0x008, FM * FN, 0);
      return;
    }
#pragma unroll
    for (int p = 0; p < KPS; ++p) {
      const char* la = st + p * SUB + (wm * FM * 16 + (lane & 15)) * 128;
      const char* lb = st + p * SUB + BM * 128 + (wn * FN * 16 + (lane & 15)) * 128;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int so = (((4 * c + kg) ^ swz)) * 16;
        u32x4 af[FM], bfr[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const u32x4*>(la + i * 16 * 128 + so);
#pragma unroll
        for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const u32x4*>(lb + j * 16 * 128 + so);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) Mfma<T>::mma(acc[i][j], af[i], bfr[j]);
      }
    }
  }

  // Full K loop over nk = K / KSTEP stages (K a multiple of KSTEP).  The stage computed at step
  // kt - 1 is refilled at step kt only after the barrier that follows every wave's wait for kt.
  DG_DEV void run(char* lds, int K, f32x4_v (&acc)[FM][FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};
    const int nk = K / KSTEP;
    int issued = 0;
    for (; issued < NS - 1 && issued < nk; ++issued) issue(lds, issued, issued);
    for (int kt = 0; kt < nk; ++kt) {
      wait_oldest(issued - kt);
      lds_barrier();
      if (issued < nk) {
        issue(lds, issued, issued % NS);
        ++issued;
      }
      compute(lds + (kt % NS) * STAGE, acc);
    }
    __syncthreads();   // the LDS ring may be reused by the caller after this
  }

  DG_DEV static int row_of(int i, int e) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    return (wave / WN) * FM * 16 + i * 16 + 4 * (lane >> 4) + e;
  }
  DG_DEV static int col_of(int j) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    return (wave % WN) * FN * 16 + j * 16 + (lane & 15);
  }
};

// Weights-only quantised B on the same direct-to-LDS ring: fp8 e4m3 codes (their per-row scale is
// applied by the caller's epilogue) or MXFP4 (e2m1 codes with one e8m0 scale per 32 elements).  A
// stage is 64 K-elements: A (bf16) as 128-byte rows; B as its raw codes, 64 bytes (fp8) or 32 bytes
// (MXFP4) per row, the 16-byte chunk c of row r stored in slot c ^ ((r >> 1) & 3) (fp8) or
// c ^ ((r >> 3) & 1) (MXFP4); MXFP4 scales as one 32-bit word per (row, 32-element block) (a
// byte-sized direct load writes each byte zero-extended to a word).  Codes are widened to bf16 in
// registers just before the MFMA, so no widened copy passes through LDS.
// K order inside a stage: lane group kg = lane >> 4 owns elements [16 kg, 16 kg + 16) of every
// row (half an MXFP4 scale block, one fp8 chunk), its MFMA chunk c in {0, 1} the elements
// 16 kg + 8 c .. + 7; A is read with the same map, so the sum over the stage is unchanged.  The A
// row keeps that chunk (2 kg + c) in slot (4 c + kg) ^ ((r >> 1) & 7): a 16-row fragment read then
// has the bank pattern of the bf16 ring's.  Measured on gfx950 (16-byte reads, 8 waves): this A
// pattern and the fp8 B swizzle on r >> 1 read at ~188 B/clock per CU; kg in the high chunk bits
// (2 kg + c) ^ (r >> 1), or a B swizzle on r >> 2, r & 3 or none, at ~110 (bank conflicts).
template <class TB, int BM, int BN, int WM, int WN, int NS>
struct GemmDmaQ {
  static constexpr int TILE_M = BM;
  static constexpr bool FP4 = is_fp4_v<TB>;
  static_assert(FP4 || is_fp8_v<TB>, "quantised weights");
  static constexpr int NW = WM * WN;
  static constexpr int FM = BM / WM / 16, FN = BN / WN / 16;
  static_assert(FM >= 1 && FN >= 1, "wave tile at least 16 x 16");
  static constexpr int KT = 64;                          // K elements per stage
  static constexpr int BROW = FP4 ? 32 : 64;             // code bytes per B row per stage
  static constexpr int BRPI = 1024 / BROW;               // B rows per load instruction
  static constexpr int IA = BM / (8 * NW), IB = BN / (BRPI * NW), IS = FP4 ? 1 : 0;
  static_assert(IA * 8 * NW == BM && IB * BRPI * NW == BN, "rows per tile: whole load instructions");
  static_assert(!FP4 || BN * 2 == 64 * NW, "MXFP4: one scale entry per lane of each wave");
  static constexpr int LPT = IA + IB + IS;               // load instructions per wave per stage
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * BROW, S_BYTES = FP4 ? BN * 2 * 4 : 0;
  static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
  static constexpr int LDS_BYTES = NS * STAGE;
  static_assert(NS >= 2 && (NS - 2) * LPT < 64, "stages / vmcnt range");

  const char* a_src[IA];
  const char* b_src[IB];
  const uint8_t* s_src;

  // arow / brow as in GemmDma; srow(r): the scale bytes of B row r (MXFP4) or nullptr
  template <class ARow, class BRow, class SRow>
  DG_DEV void setup(ARow arow, BRow brow, SRow srow) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    {
      const int rr = lane >> 3, slot = lane & 7;
#pragma unroll
      for (int i = 0; i < IA; ++i) {
        const int r = (wave + NW * i) * 8 + rr;
        const char* p = reinterpret_cast<const char*>(arow(r));
        if (!p) p = reinterpret_cast<const char*>(arow(0));
        const int s = slot ^ ((r >> 1) & 7);             // = 4 c + kg of the chunk this lane fetches
        a_src[i] = p + ((((s & 3) << 1) | (s >> 2)) * 16);
      }
    }
    {
      constexpr int CPR = BROW / 16;                     // 16-byte chunks per row
      const int rr = lane / CPR, slot = lane % CPR;
#pragma unroll
      for (int i = 0; i < IB; ++i) {
        const int r = (wave + NW * i) * BRPI + rr;
        const char* p = reinterpret_cast<const char*>(brow(r));
        if (!p) p = reinterpret_cast<const char*>(brow(0));
        const int sw = FP4 ? ((r >> 3) & 1) : ((r >> 1) & 3);
        b_src[i] = p + ((slot ^ sw) * 16);
      }
    }
    if constexpr (FP4) {
      const int e = wave * 64 + lane, r = e >> 1;        // entry e = (row r, block e & 1)
      const uint8_t* sp = srow(r);
      if (!sp) sp = srow(0);
      s_src = sp + (e & 1);
    }
  }

  DG_DEV void issue(char* lds, int kt, int stage) {
    const int wave = threadIdx.x >> 6;
    char* st = lds + stage * STAGE;
#pragma unroll
    for (int i = 0; i < IA; ++i) dma16(a_src[i] + (size_t)kt * 128, st + (wave + NW * i) * 8 * 128);
#pragma unroll
    for (int i = 0; i < IB; ++i)
      dma16<DMA_STREAM>(b_src[i] + (size_t)kt * BROW, st + A_BYTES + (wave + NW * i) * 1024);
    if constexpr (FP4)
      __builtin_amdgcn_global_load_lds((const DG_GLOBAL_AS void*)(s_src + (size_t)kt * 2),
                                       (DG_LDS_AS void*)(st + A_BYTES + B_BYTES + wave * 256), 1, 0, DMA_CACHED);
  }

  template <int P>
  DG_DEV static void wait_pending(int pending) {
    if constexpr (P > 1) {
      if (pending >= P) { wait_vm<(P - 1) * LPT>(); return; }
      wait_pending<P - 1>(pending);
    } else {
      wait_vm<0>();
    }
  }
  DG_DEV static void wait_oldest(int pending) { wait_pending<NS - 1>(pending); }

  DG_DEV static void compute(const char* st, f32x4_v (&acc)[FM][FN]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int l16 = lane & 15, kg = lane >> 4, swa = l16 >> 1;
    u32x4 bfr[FN][2];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = wn * FN * 16 + j * 16 + l16;
      if constexpr (FP4) {
        // elements [16 kg, 16 kg + 16) = bytes [8 kg, 8 kg + 8) of the row: chunk kg >> 1, half kg & 1
        const char* row = st + A_BYTES + n * 32;
        const uint2 w = *reinterpret_cast<const uint2*>(row + (((kg >> 1) ^ ((n >> 3) & 1)) * 16) + (kg & 1) * 8);
        const uint32_t s = *reinterpret_cast<const uint32_t*>(st + A_BYTES + B_BYTES + (n * 2 + (kg >> 1)) * 4);
        const float sc = e8m0_scale(s & 0xffu);
        bfr[j][0] = widen_fp4_word(w.x, sc);
        bfr[j][1] = widen_fp4_word(w.y, sc);
      } else {
        const char* row = st + A_BYTES + n * 64;
        const u32x4 w = *reinterpret_cast<const u32x4*>(row + ((kg ^ ((n >> 1) & 3)) * 16));
        bfr[j][0] = widen_fp8_lo(w);
        bfr[j][1] = widen_fp8_hi(w);
      }
    }
    const char* la = st + (wm * FM * 16 + l16) * 128;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int so = (((4 * c + kg) ^ swa)) * 16;     // A elements 16 kg + 8 c .. + 7
      u32x4 af[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const u32x4*>(la + i * 16 * 128 + so);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) Mfma<bf16_t>::mma(acc[i][j], af[i], bfr[j][c]);
    }
  }

  DG_DEV void run(char* lds, int K, f32x4_v (&acc)[FM][FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};
    const int nk = K / KT;
    int issued = 0;
    for (; issued < NS - 1 && issued < nk; ++issued) issue(lds, issued, issued);
    for (int kt = 0; kt < nk; ++kt) {
      wait_oldest(issued - kt);
      lds_barrier();
      if (issued < nk) {
        issue(lds, issued, issued % NS);
        ++issued;
      }
      compute(lds + (kt % NS) * STAGE, acc);
    }
    __syncthreads();
  }

  DG_DEV static int row_of(int i, int e) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    return (wave / WN) * FM * 16 + i * 16 + 4 * (lane >> 4) + e;
  }
  DG_DEV static int col_of(int j) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    return (wave % WN) * FN * 16 + j * 16 + (lane & 15);
  }
};

// W8A8: both operands as e4m3 codes on the direct-to-LDS ring, multiplied by the gfx950
// block-scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4 with both formats e4m3 and both block
// scales 1 (e8m0 code 127): 128 K-elements per instruction at twice the bf16 rate, fp32
// accumulation; the per-row and per-column scales are the caller's epilogue.  A stage is 128
// K-elements: A and B rows of 128 bytes laid out like the bf16 ring's (8 rows per load
// instruction, the 16-byte chunk c of row r in slot c ^ ((r >> 1) & 7)).  Lane group kg = lane >> 4
// feeds the MFMA chunks kg and 4 + kg of its A row and of its B row as its 32 bytes, the same
// 16-byte reads as the bf16 ring's (conflict-free); A and B use the same map, so the sum over the
// stage is the plain dot product.  K may end half-way through a stage (K % 128 == 64): there the
// lanes of chunks 4..7 fetch chunk c - 4 of the same row instead (no access past K), and their A
// halves are zeroed in registers, so those products add exact zeros.
template <int BM, int BN, int WM, int WN, int NS>
struct GemmDmaQQ {
  static constexpr int TILE_M = BM;
  static constexpr int NW = WM * WN;
  static constexpr int FM = BM / WM / 16, FN = BN / WN / 16;
  static_assert(FM >= 1 && FN >= 1, "wave tile at least 16 x 16");
  static constexpr int KT = 128;                         // K elements (bytes) per stage
  static constexpr int IA = BM / (8 * NW), IB = BN / (8 * NW);   // 8 rows per load instruction
  static_assert(IA * 8 * NW == BM && IB * 8 * NW == BN, "rows per tile: whole load instructions");
  static constexpr int LPT = IA + IB;                    // load instructions per wave per stage
  static constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = NS * STAGE;
  static_assert(NS >= 2 && (NS - 2) * LPT < 64, "stages / vmcnt range");

  const char* a_src[IA];
  const char* b_src[IB];
  int hi_back;                 // bytes this lane steps back on a half stage (64 for chunks 4..7, else 0)

  template <class ARow, class BRow, class SRow>
  DG_DEV void setup(ARow arow, BRow brow, SRow) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rr = lane >> 3, slot = lane & 7;
#pragma unroll
    for (int i = 0; i < IA; ++i) {
      const int r = (wave + NW * i) * 8 + rr;
      const char* p = reinterpret_cast<const char*>(arow(r));
      if (!p) p = reinterpret_cast<const char*>(arow(0));
      a_src[i] = p + ((slot ^ ((r >> 1) & 7)) * 16);
    }
#pragma unroll
    for (int i = 0; i < IB; ++i) {
      const int r = (wave + NW * i) * 8 + rr;
      const char* p = reinterpret_cast<const char*>(brow(r));
      if (!p) p = reinterpret_cast<const char*>(brow(0));
      b_src[i] = p + ((slot ^ ((r >> 1) & 7)) * 16);
    }
    // the chunk this lane fetches, slot ^ ((r >> 1) & 7), is the same for all its instructions:
    // their rows differ by multiples of 8 x NW (NW even), which leave (r >> 1) & 7 unchanged
    static_assert(NW % 2 == 0, "even wave count");
    hi_back = ((slot ^ (((wave * 8 + rr) >> 1) & 7)) >= 4) ? 64 : 0;
  }

  // stage `stage` <- K elements [128 kt, 128 kt + 128); half: only [128 kt, 128 kt + 64) exist
  DG_DEV void issue(char* lds, int kt, int stage, bool half = false) {
    const int wave = threadIdx.x >> 6;
    char* st = lds + stage * STAGE;
    const size_t off = (size_t)kt * 128 - (half ? hi_back : 0);
#pragma unroll
    for (int i = 0; i < IA; ++i) dma16(a_src[i] + off, st + (wave + NW * i) * 8 * 128);
#pragma unroll
    for (int i = 0; i < IB; ++i) dma16<DMA_STREAM>(b_src[i] + off, st + A_BYTES + (wave + NW * i) * 8 * 128);
  }

  template <int P>
  DG_DEV static void wait_pending(int pending) {
    if constexpr (P > 1) {
      if (pending >= P) { wait_vm<(P - 1) * LPT>(); return; }
      wait_pending<P - 1>(pending);
    } else {
      wait_vm<0>();
    }
  }
  DG_DEV static void wait_oldest(int pending) { wait_pending<NS - 1>(pending); }

  DG_DEV static void compute(const char* st, f32x4_v (&acc)[FM][FN], bool half = false) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int l16 = lane & 15, kg = lane >> 4, swz = l16 >> 1;
    const int s0 = (kg ^ swz) * 16, s1 = ((4 + kg) ^ swz) * 16;
    i32x8 bf[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const char* row = st + A_BYTES + (wn * FN * 16 + j * 16 + l16) * 128;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(row + s0), hi = *reinterpret_cast<const u32x4*>(row + s1);
      bf[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const char* row = st + (wm * FM * 16 + i * 16 + l16) * 128;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(row + s0);
      u32x4 hi = *reinterpret_cast<const u32x4*>(row + s1);
      if (half) hi = u32x4{0u, 0u, 0u, 0u};
      const i32x8 af = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], acc[i][j], 0, 0, 0, 127, 0, 127);
    }
  }

  // nk = ceil(K / 128) stages, the last one half when K % 128 == 64
  DG_DEV void run(char* lds, int K, f32x4_v (&acc)[FM][FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};
    const int nk = (K + KT - 1) / KT;
    const bool tail = (K % KT) != 0;
    int issued = 0;
    for (; issued < NS - 1 && issued < nk; ++issued) issue(lds, issued, issued, tail && issued == nk - 1);
    for (int kt = 0; kt < nk; ++kt) {
      wait_oldest(issued - kt);
      lds_barrier();
      if (issued < nk) {
        issue(lds, issued, issued % NS, tail && issued == nk - 1);
        ++issued;
      }
      compute(lds + (kt % NS) * STAGE, acc, tail && kt == nk - 1);
    }
    __syncthreads();
  }

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
