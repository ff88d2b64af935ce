// encode_impl.h -- the encoder kernels (templates instantiated per stage count
// in the encode_s*.hip units).
#pragma once
//
// Method: "LongCat-2.5 Native Multimodality for Agentic Tasks", section
// "Visual Primitive Modeling", paragraph "Discrete Native Resolution Vision
// Transformer" (RVQ on native-resolution features), and "LongCat-2.5 Open
// Source Release ...", section "02 Visual Coding and 3D" (detail added level
// by level).  Per level and row r the nearest codeword under the squared
// Euclidean distance ||r||^2 - 2 r.c + ||c||^2 is chosen; ||r||^2 is the
// same for every codeword, so codewords are ranked by the score
// ||c||^2 - 2 r.c.
//
// Design (one workgroup = 4 waves = 128 rows, one workgroup per CU):
//  * Each wave keeps its 32 rows resident in VGPRs as bf16 B-fragments of
//    v_mfma_f32_32x32x16_bf16 covering the whole feature dimension, so rows
//    are read from memory once per level, never once per codeword tile.
//  * The prepared codebook (common.h) is one contiguous stream of A-fragments
//    per level.  All workgroups sweep it in the same order, so the 32 CUs of
//    an XCD share every line in L2.  Each 16 KB stage goes through a 7-slot
//    LDS ring filled by direct global->LDS loads six stages ahead, and
//    every wave reads all A-fragments of a stage from LDS (no bank
//    conflicts: lane L reads bytes 16L..16L+15 of a 1 KB fragment).
//  * A per-tile norm k-step folds ||c||^2 into the accumulator, so the
//    accumulator holds the score.  The epilogue packs each score with a
//    5-bit lane-local codeword tag into a key (score bits 0..4 replaced) and
//    keeps the two smallest keys per 64-codeword block with v_min / v_med3
//    (3 VALU ops per score); block winners are merged exactly under the
//    (key, index) order.
//  * Fused mode (enough rows to fill the GPU): all levels run in one launch;
//    after a level's sweep, lanes L and L+32 of a wave rescore their row's
//    two candidates exactly in fp32 (sum of squared differences, each lane
//    one half of the features in a fixed order), pick the smaller (lower
//    index on a tie), subtract it from the fp32 residual and rebuild the
//    B-fragments for the next level in registers.
//  * Split mode (few rows): a level's codeword tiles are split over
//    several workgroups per row block, each writing its top-2 list; a second
//    kernel merges the lists and runs the same rescoring and update.
// Every score depends only on (row, codeword): one MFMA shape, one k-step
// order, one key rule and a total order for merging, so the IDs and
// residuals are bitwise independent of batch size, row position and mode.
#include <type_traits>

#include "common.h"

namespace rvq {

namespace {

constexpr int NT = 256;

__device__ __forceinline__ float pack_key(float score, uint32_t tag) {
  return __uint_as_float((__float_as_uint(score) & ~31u) | tag);
}

// Codeword index of a key found in the 64-codeword block whose lane-half
// base is b (kNoIndex when nothing was found).
__device__ __forceinline__ int block_index(float key, int b) {
  const uint32_t g = __float_as_uint(key) & 31u;
  return b == kNoIndex ? kNoIndex : b + (int)((g >> 4) * 32 + ((g >> 2) & 3) * 8 + (g & 3));
}

// The row fragments do not fit in the 256 arch VGPRs next to everything
// else, so the first kFragsInAgpr k-steps fill the 256 AGPRs and feed the
// MFMA B operand from there (the compiler only emits the VGPR form, so a
// stage's MFMAs are written out below); the accumulators stay in VGPRs,
// where the epilogue reads them without copies.  A fragment is one 128-bit
// value (8 bf16 packed in 4 words).
constexpr int kFragsInAgpr = 64;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Stage blocks.  A slot holds a 4 KB norm area and one 16 KB stage; in the
// stage, k-step ks of sub-tile j is the 1 KB A-fragment at byte
// 4096 + (4*j + ks)*1024, and lane L reads its 16 bytes at slot base + 16*L.
// A block runs one stage's MFMAs with each LDS read five MFMAs ahead of its
// use, and during its last k-steps it reads the first
// A-fragments of the next stage (norm fragments when the next stage opens a
// tile) into p, so the next block starts its MFMAs without waiting for LDS.  Every read has completed
// when a block ends (no load is in flight across blocks).  The leading
// wait covers any scalar load the compiler left in flight, so the counted
// waits below see only this block's reads.
#define RVQ_RD(t, base, off) "ds_read_b128 %[" #t "], %[" #base "] offset:" #off "\n\t"
#define RVQ_MF(c, a, b) "v_mfma_f32_32x32x16_bf16 %[" #c "], %[" #a "], %[" #b "], %[" #c "]\n\t"
// First A-fragments of the next stage (its k-step 0), or of the next tile
// (its norm k-step), one sub-tile at a time
#define RVQ_NEXT_STAGE_0 RVQ_RD(p0, naddr, 4096)
#define RVQ_NEXT_STAGE_1 RVQ_RD(p1, naddr, 8192)
#define RVQ_NEXT_STAGE_2 RVQ_RD(p2, naddr, 12288)
#define RVQ_NEXT_STAGE_3 RVQ_RD(p3, naddr, 16384)
#define RVQ_NEXT_TILE_0 RVQ_RD(p0, naddr, 0)
#define RVQ_NEXT_TILE_1 RVQ_RD(p1, naddr, 1024)
#define RVQ_NEXT_TILE_2 RVQ_RD(p2, naddr, 2048)
#define RVQ_NEXT_TILE_3 RVQ_RD(p3, naddr, 3072)
#define RVQ_WAIT(n) "s_waitcnt lgkmcnt(" #n ")\n\t"


// Refill loads placed inside a block, one after the first MFMA of each
// k-step, so they issue while the matrix core is busy: this wave's four 1 KB blocks of the
// stage being refilled (uniform global base gsb in SGPRs plus the lane's
// 32-bit offset voff; LDS destination lds).  Lane i's 16 bytes land at
// M0 + offset + 16*i: the instruction offset moves the global and the LDS
// address alike, so M0 is set once.  The scalar-base form keeps the
// per-lane address at 32 bits, which costs the issuing wave measurably
// fewer cycles than a 64-bit per-lane address.
#define RVQ_D0 "s_mov_b32 m0, %[lds]\n\tglobal_load_lds_dwordx4 %[voff], %[gsb]\n\t"
#define RVQ_D1 "global_load_lds_dwordx4 %[voff], %[gsb] offset:1024\n\t"
#define RVQ_D2 "global_load_lds_dwordx4 %[voff], %[gsb] offset:2048\n\t"
#define RVQ_D3 "global_load_lds_dwordx4 %[voff], %[gsb] offset:3072\n\t"

// A stage inside a tile: p holds its k-step 0 on entry.  Reads are spread
// one per MFMA, each five MFMAs ahead of its use, and a refill load follows
// the first MFMA of each k-step: evenly spaced requests keep the LDS queue
// short.  (Probes of this block measured 682 cycles with reads in bursts of
// four one k-step ahead, 657 spread four ahead, 635 as here.)
#define RVQ_STAGE_BODY(NX, D0, D1, D2, D3)                                               \
  RVQ_WAIT(0) RVQ_RD(t0, addr, 5120) RVQ_RD(t1, addr, 9216) RVQ_MF(c0, p0, b0) D0        \
  RVQ_RD(t2, addr, 13312) RVQ_MF(c1, p1, b0) RVQ_RD(t3, addr, 17408) RVQ_MF(c2, p2, b0)  \
  RVQ_RD(t4, addr, 6144) RVQ_MF(c3, p3, b0) RVQ_RD(t5, addr, 10240) RVQ_WAIT(5)          \
  RVQ_MF(c0, t0, b1) D1 RVQ_RD(t6, addr, 14336) RVQ_WAIT(5) RVQ_MF(c1, t1, b1)           \
  RVQ_RD(t7, addr, 18432) RVQ_WAIT(5) RVQ_MF(c2, t2, b1) RVQ_RD(t0, addr, 7168)          \
  RVQ_WAIT(5) RVQ_MF(c3, t3, b1) RVQ_RD(t1, addr, 11264) RVQ_WAIT(5) RVQ_MF(c0, t4, b2)  \
  D2 RVQ_RD(t2, addr, 15360) RVQ_WAIT(5) RVQ_MF(c1, t5, b2) RVQ_RD(t3, addr, 19456)      \
  RVQ_WAIT(5) RVQ_MF(c2, t6, b2) NX##_0 RVQ_WAIT(5) RVQ_MF(c3, t7, b2) NX##_1            \
  RVQ_WAIT(5) RVQ_MF(c0, t0, b3) D3 NX##_2 RVQ_WAIT(5) RVQ_MF(c1, t1, b3) NX##_3         \
  RVQ_WAIT(5) RVQ_MF(c2, t2, b3) RVQ_WAIT(4) RVQ_MF(c3, t3, b3) RVQ_WAIT(0)             

// The stage opening a tile: p holds the norm k-step on entry, and the
// accumulators start from ||c||^2 (B = ones at k = 0, 1).
#define RVQ_MFN(c, a) "v_mfma_f32_32x32x16_bf16 %[" #c "], %[" #a "], %[bn], 0\n\t"
#define RVQ_STAGE0_BODY(NX, D0, D1, D2, D3)                                              \
  RVQ_WAIT(0) RVQ_RD(t0, addr, 4096) RVQ_RD(t1, addr, 8192) RVQ_MFN(c0, p0)              \
  RVQ_RD(t2, addr, 12288) RVQ_MFN(c1, p1) RVQ_RD(t3, addr, 16384) RVQ_MFN(c2, p2)        \
  RVQ_RD(t4, addr, 5120) RVQ_MFN(c3, p3) RVQ_RD(t5, addr, 9216) RVQ_WAIT(5)              \
  RVQ_MF(c0, t0, b0) D0 RVQ_RD(t6, addr, 13312) RVQ_WAIT(5) RVQ_MF(c1, t1, b0)           \
  RVQ_RD(t7, addr, 17408) RVQ_WAIT(5) RVQ_MF(c2, t2, b0) RVQ_RD(t0, addr, 6144)          \
  RVQ_WAIT(5) RVQ_MF(c3, t3, b0) RVQ_RD(t1, addr, 10240) RVQ_WAIT(5) RVQ_MF(c0, t4, b1)  \
  D1 RVQ_RD(t2, addr, 14336) RVQ_WAIT(5) RVQ_MF(c1, t5, b1) RVQ_RD(t3, addr, 18432)      \
  RVQ_WAIT(5) RVQ_MF(c2, t6, b1) RVQ_RD(t4, addr, 7168) RVQ_WAIT(5) RVQ_MF(c3, t7, b1)   \
  RVQ_RD(t5, addr, 11264) RVQ_WAIT(5) RVQ_MF(c0, t0, b2) D2 RVQ_RD(t6, addr, 15360)      \
  RVQ_WAIT(5) RVQ_MF(c1, t1, b2) RVQ_RD(t7, addr, 19456) RVQ_WAIT(5) RVQ_MF(c2, t2, b2)  \
  NX##_0 RVQ_WAIT(5) RVQ_MF(c3, t3, b2) NX##_1 RVQ_WAIT(5) RVQ_MF(c0, t4, b3) D3 NX##_2  \
  RVQ_WAIT(5) RVQ_MF(c1, t5, b3) NX##_3 RVQ_WAIT(5) RVQ_MF(c2, t6, b3) RVQ_WAIT(4)       \
  RVQ_MF(c3, t7, b3) RVQ_WAIT(0)

#define RVQ_TEMPS                                                                          \
  [t0] "=&v"(t[0]), [t1] "=&v"(t[1]), [t2] "=&v"(t[2]), [t3] "=&v"(t[3]), [t4] "=&v"(t[4]), \
      [t5] "=&v"(t[5]), [t6] "=&v"(t[6]), [t7] "=&v"(t[7])
#define RVQ_PREF [p0] "+v"(p[0]), [p1] "+v"(p[1]), [p2] "+v"(p[2]), [p3] "+v"(p[3])

// FIRST: the stage opens a tile.  NEXT_TILE: the next stage opens a tile.
// B_IN_AGPR: the stage's row fragments live in AGPRs.  DMA: the block also
// issues this wave's refill loads (gsb + voff, lds).
template <bool FIRST, bool NEXT_TILE, bool B_IN_AGPR, bool DMA>
__device__ __forceinline__ void stage_block(f32x16 (&c)[4], u32x4 (&p)[4], uint32_t addr,
                                            uint32_t naddr, const u32x4 &bn, const u32x4 &b0,
                                            const u32x4 &b1, const u32x4 &b2, const u32x4 &b3,
                                            const uint4 *gsb, uint32_t voff, uint32_t lds) {
  u32x4 t[8];
  uint32_t m0_out;
#define RVQ_IN(cls)                                                                        \
  [addr] "v"(addr), [naddr] "v"(naddr), [b0] cls(b0), [b1] cls(b1), [b2] cls(b2), [b3] cls(b3), \
      [gsb] "s"(gsb), [voff] "v"(voff), [lds] "s"(lds)
#define RVQ_OUTSEL_0 \
  [c0] "=&v"(c[0]), [c1] "=&v"(c[1]), [c2] "=&v"(c[2]), [c3] "=&v"(c[3]), RVQ_PREF, RVQ_TEMPS, [m0o] "=&{m0}"(m0_out)
#define RVQ_OUTSEL_1 \
  [c0] "+v"(c[0]), [c1] "+v"(c[1]), [c2] "+v"(c[2]), [c3] "+v"(c[3]), RVQ_PREF, RVQ_TEMPS, [m0o] "=&{m0}"(m0_out)
#define RVQ_EMIT(BODY, OSEL, CLS, ...)                                                     \
  asm volatile(BODY : RVQ_OUTSEL_##OSEL : RVQ_IN(CLS) __VA_ARGS__ : "memory")
#define RVQ_NEXT_SEL(B0DY, NX) \
  B0DY(NX, RVQ_D0, RVQ_D1, RVQ_D2, RVQ_D3)
#define RVQ_NEXT_NODMA(B0DY, NX) B0DY(NX, "", "", "", "")
#define RVQ_CASES(B0DY, OSEL, ...)                                                          \
  if constexpr (NEXT_TILE) {                                                                \
    if constexpr (DMA) {                                                                    \
      if constexpr (B_IN_AGPR) RVQ_EMIT(RVQ_NEXT_SEL(B0DY, RVQ_NEXT_TILE), OSEL, "a", __VA_ARGS__); \
      else RVQ_EMIT(RVQ_NEXT_SEL(B0DY, RVQ_NEXT_TILE), OSEL, "v", __VA_ARGS__);              \
    } else {                                                                                \
      if constexpr (B_IN_AGPR) RVQ_EMIT(RVQ_NEXT_NODMA(B0DY, RVQ_NEXT_TILE), OSEL, "a", __VA_ARGS__); \
      else RVQ_EMIT(RVQ_NEXT_NODMA(B0DY, RVQ_NEXT_TILE), OSEL, "v", __VA_ARGS__);            \
    }                                                                                       \
  } else {                                                                                  \
    if constexpr (DMA) {                                                                    \
      if constexpr (B_IN_AGPR) RVQ_EMIT(RVQ_NEXT_SEL(B0DY, RVQ_NEXT_STAGE), OSEL, "a", __VA_ARGS__); \
      else RVQ_EMIT(RVQ_NEXT_SEL(B0DY, RVQ_NEXT_STAGE), OSEL, "v", __VA_ARGS__);             \
    } else {                                                                                \
      if constexpr (B_IN_AGPR) RVQ_EMIT(RVQ_NEXT_NODMA(B0DY, RVQ_NEXT_STAGE), OSEL, "a", __VA_ARGS__); \
      else RVQ_EMIT(RVQ_NEXT_NODMA(B0DY, RVQ_NEXT_STAGE), OSEL, "v", __VA_ARGS__);           \
    }                                                                                       \
  }
  if constexpr (FIRST) {
    RVQ_CASES(RVQ_STAGE0_BODY, 0, , [bn] "v"(bn))
  } else {
    RVQ_CASES(RVQ_STAGE_BODY, 1, )
  }
#undef RVQ_CASES
#undef RVQ_NEXT_NODMA
#undef RVQ_NEXT_SEL
#undef RVQ_EMIT
#undef RVQ_OUTSEL_1
#undef RVQ_OUTSEL_0
#undef RVQ_IN
  (void)m0_out;
}

// The norm fragments of the tile opening a level (slot base + 16*lane).
__device__ __forceinline__ void read_tile_norms(u32x4 (&p)[4], uint32_t naddr) {
  asm volatile(RVQ_WAIT(0) RVQ_NEXT_TILE_0 RVQ_NEXT_TILE_1 RVQ_NEXT_TILE_2 RVQ_NEXT_TILE_3
                   RVQ_WAIT(0)
               : [p0] "=&v"(p[0]), [p1] "=&v"(p[1]), [p2] "=&v"(p[2]), [p3] "=&v"(p[3])
               : [naddr] "v"(naddr));
}

// Orders the epilogue's accumulator reads after the last MFMA's result
// latency (the compiler does not see the MFMAs above).
__device__ __forceinline__ void mfma_drain(f32x16 (&acc)[4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
}

// Row fragments split over AGPRs (k-steps < NA) and VGPRs (the rest); NA
// is a multiple of 4 so a stage's four k-steps sit in one register file.
template <int KS>
struct RowFrags {
  static constexpr int NA = KS < kFragsInAgpr ? KS : kFragsInAgpr;
  static constexpr int NV = KS - NA;
  u32x4 fa[NA];
  u32x4 fv[NV > 0 ? NV : 1];
  // The empty asm pins a new fragment to its register file from the start
  // (an AGPR-class value never needs copying before an MFMA that reads it).
  template <int k>
  __device__ __forceinline__ void set(const u32x4 &v) {
    u32x4 t = v;
    if constexpr (k < NA) {
      asm volatile("" : "+a"(t));
      fa[k] = t;
    } else {
      asm volatile("" : "+v"(t));
      fv[k - NA] = t;
    }
  }
  template <int k>
  __device__ __forceinline__ const u32x4 &get() const {
    if constexpr (k < NA) return fa[k];
    else return fv[k - NA];
  }
  template <int s, int S, bool DMA>
  __device__ __forceinline__ void stage(f32x16 (&c)[4], u32x4 (&p)[4], uint32_t addr,
                                        uint32_t naddr, const u32x4 &bn, const uint4 *gsb,
                                        uint32_t voff, uint32_t lds) const {
    static_assert(NA % 4 == 0, "a stage's k-steps must share a register file");
    stage_block<s == 0, s == S - 1, (s * 4 < NA), DMA>(c, p, addr, naddr, bn, get<s * 4>(),
                                                        get<s * 4 + 1>(), get<s * 4 + 2>(),
                                                        get<s * 4 + 3>(), gsb, voff, lds);
  }};

// Compile-time loop: f(integral_constant<int, i>) for i in [0, N).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Rows seen by the sweep are fp32 with a stride dp that is a multiple of 16
// and zero padding past the true width, so a k-step (16 features) is either
// wholly inside the row or wholly past it -- the same for every lane of a
// wave -- and every access is an aligned 32-byte vector access.  Reads past
// the row use a clamped address and select zero, so no lane branches.
__device__ __forceinline__ void read8(const float *base, int64_t row, int dp, int i0, bool active,
                                      float (&v)[8]) {
  const float *p = base + row * dp + (active ? i0 : 0);
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 4);
  v[0] = active ? a.x : 0.f; v[1] = active ? a.y : 0.f;
  v[2] = active ? a.z : 0.f; v[3] = active ? a.w : 0.f;
  v[4] = active ? b.x : 0.f; v[5] = active ? b.y : 0.f;
  v[6] = active ? b.z : 0.f; v[7] = active ? b.w : 0.f;
}

__device__ __forceinline__ void write8(float *base, int64_t row, int dp, int i0,
                                       const float (&v)[8]) {
  *reinterpret_cast<float4 *>(base + row * dp + i0) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4 *>(base + row * dp + i0 + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Eight bf16 features (16 bytes) widened exactly to fp32; q is returned too,
// since it already is the B-fragment of these features.
__device__ __forceinline__ uint4 read8_bf16(const uint16_t *base, int64_t row, int dp, int i0,
                                            float (&v)[8]) {
  const uint4 q = *reinterpret_cast<const uint4 *>(base + row * dp + i0);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(w[e] << 16);
    v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
  return q;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x4 to_bf16x8(const float (&v)[8]) {
  u32x4 q;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16x2 p = {(__bf16)v[2 * e], (__bf16)v[2 * e + 1]};
    q[e] = __builtin_bit_cast(uint32_t, p);
  }
  return q;
}

// Re-defines values through an empty asm: code that computes addresses from
// them cannot move above this point, which bounds how far the compiler
// hoists loads (and so the registers they hold).
template <typename T>
__device__ __forceinline__ void opaque1(T &v) {
  asm volatile("" : "+v"(v) : : "memory");
}
template <typename... T>
__device__ __forceinline__ void opaque(T &...v) {
  (opaque1(v), ...);
}

// B-fragments of one row half: lane half h holds features ks*16 + h*8 + e.
// Loads are issued eight k-steps at a time before any fragment is pinned,
// so the waits for them overlap.
template <int KS>
__device__ __forceinline__ void build_bfrags(RowFrags<KS> &bfr, const float *src, int64_t row,
                                             int dp, int h) {
  static_for<0, (KS + 7) / 8>([&](auto G_) {
    constexpr int g = decltype(G_)::value;
    constexpr int n = KS - g * 8 < 8 ? KS - g * 8 : 8;
    float v[8][8];
    static_for<0, n>([&](auto U_) {
      constexpr int ks = g * 8 + decltype(U_)::value;
      read8(src, row, dp, ks * 16 + h * 8, ks * 16 < dp, v[decltype(U_)::value]);
    });
    static_for<0, n>([&](auto U_) {
      constexpr int ks = g * 8 + decltype(U_)::value;
      bfr.template set<ks>(to_bf16x8(v[decltype(U_)::value]));
    });
    opaque(row);
  });
}

__device__ __forceinline__ void read_src(const float *src, int64_t row, int dp, int i0,
                                         float (&v)[8]) {
  read8(src, row, dp, i0, true, v);
}
__device__ __forceinline__ void read_src(const uint16_t *src, int64_t row, int dp, int i0,
                                         float (&v)[8]) {
  read8_bf16(src, row, dp, i0, v);
}

// The same fragments from the bf16 fragment copy of a block of 32 rows
// (split mode): k-step ks of lane L is the 16 bytes at blk[ks * 64 + L], so
// every load of a wave is 1 KB of consecutive bytes.  K-steps past the row
// (ks >= ksp) are zero.
template <int KS>
__device__ __forceinline__ void build_bfrags_frag(RowFrags<KS> &bfr, const uint4 *blk, int ksp,
                                                  int lane) {
  static_for<0, (KS + 15) / 16>([&](auto G_) {
    constexpr int g = decltype(G_)::value;
    constexpr int n = KS - g * 16 < 16 ? KS - g * 16 : 16;
    u32x4 f[16];
    static_for<0, n>([&](auto U_) {
      constexpr int ks = g * 16 + decltype(U_)::value;
      const bool active = ks < ksp;
      const uint4 q = blk[(active ? ks : 0) * 64 + lane];
      f[decltype(U_)::value] = active ? u32x4{q.x, q.y, q.z, q.w} : u32x4{0u, 0u, 0u, 0u};
    });
    static_for<0, n>([&](auto U_) {
      constexpr int ks = g * 16 + decltype(U_)::value;
      bfr.template set<ks>(f[decltype(U_)::value]);
    });
    opaque(blk);
  });
}

// The same fragments straight from bf16 rows (stride dp): the stored bits
// are the fragment.
template <int KS>
__device__ __forceinline__ void build_bfrags_bf16(RowFrags<KS> &bfr, const uint16_t *src,
                                                  int64_t row, int dp, int h) {
  static_for<0, (KS + 7) / 8>([&](auto G_) {
    constexpr int g = decltype(G_)::value;
    constexpr int n = KS - g * 8 < 8 ? KS - g * 8 : 8;
    u32x4 f[8];
    static_for<0, n>([&](auto U_) {
      constexpr int ks = g * 8 + decltype(U_)::value;
      const bool active = ks * 16 < dp;
      const uint4 q = *reinterpret_cast<const uint4 *>(src + row * dp + (active ? ks * 16 + h * 8 : 0));
      f[decltype(U_)::value] = active ? u32x4{q.x, q.y, q.z, q.w} : u32x4{0u, 0u, 0u, 0u};
    });
    static_for<0, n>([&](auto U_) {
      constexpr int ks = g * 8 + decltype(U_)::value;
      bfr.template set<ks>(f[decltype(U_)::value]);
    });
    opaque(row);
  });
}

// First two candidates of a row's top-2 list as valid codeword indices.
__device__ __forceinline__ void candidates(int i1, int i2, int K, int &c1, int &c2, bool &v2) {
  c1 = (i1 >= 0 && i1 < K) ? i1 : 0;  // finite inputs always give a valid first candidate
  v2 = i2 >= 0 && i2 < K && i2 != i1;
  c2 = v2 ? i2 : c1;
}

// ---- LDS ring of codebook stages fed by direct global->LDS loads ----
// A slot holds one stage (16 KB of A-fragments) after a 4 KB area that
// receives the tile's norm k-step when the stage starts a tile.  The loads
// (global_load_lds_dwordx4: lane i's 16 bytes land at M0 + 16*i) are
// written out because the compiler, unable to tell the slots apart, would
// otherwise wait for every outstanding load before each LDS read; the
// waits below are exact per-wave counts instead.
constexpr int kSlots = 7;                  // stages resident in LDS
constexpr int kAhead = kSlots - 1;         // stages loaded ahead of the one in use
constexpr int kSlotBytes = kNormBytes + kStageBytes;

// One 1 KB block: lane i's 16 bytes from base + voff (base uniform, in
// SGPRs) land at lds_addr + 16*i.
__device__ __forceinline__ void dma16(const uint4 *base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds_addr) : "memory");
}

// This wave's four 1 KB blocks of a stage (gsb + voff, landing at lds), as
// one statement; the instruction offset moves both addresses.
__device__ __forceinline__ void dma_stage(const uint4 *gsb, uint32_t voff, uint32_t lds) {
  uint32_t m0_out;
  asm volatile(RVQ_D0 RVQ_D1 RVQ_D2 RVQ_D3
               : [m0o] "=&{m0}"(m0_out)
               : [gsb] "s"(gsb), [voff] "v"(voff), [lds] "s"(lds)
               : "memory");
  (void)m0_out;
}

// Load instructions one wave issues for a stage: 4 x 1 KB blocks, plus its
// norm block when the stage starts a tile.
__host__ __device__ constexpr int dma_count(int s) { return s == 0 ? 5 : 4; }

// Loads issued after stage s+1's, for the stages s+2 .. s+kAhead-1.
template <int S>
__host__ __device__ constexpr int dma_after_next(int s) {
  int c = 0;
  for (int k = 2; k < kAhead; ++k) c += dma_count((s + k) % S);
  return c;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// Issue this wave's loads of stream stage (tt, s) into ring slot `slot`.
__device__ __forceinline__ void issue_stage(const uint4 *ls, int64_t tile_u4, int tt, int s,
                                            int slot, uint32_t ring_lds, int wave, int lane) {
  const uint4 *tp = ls + (int64_t)tt * tile_u4;
  const uint4 *sp = tp + 256 + (int64_t)s * 1024;
  const uint32_t base = ring_lds + (uint32_t)slot * kSlotBytes;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    dma16(sp, (uint32_t)(wave * 256 + q * 64 + lane) * 16u,
          base + kNormBytes + (uint32_t)(wave * 4 + q) * kBlockBytes);
  if (s == 0) dma16(tp, (uint32_t)(wave * 64 + lane) * 16u, base + (uint32_t)wave * kBlockBytes);
}

// ---- fused update through LDS ----
// After a level's sweep each lane-row needs three rows: its residual and its
// two candidate codewords.  Loaded straight into fragment layout, every load
// instruction touches 32 rows at 32 bytes each, which the memory pipeline
// serves slowly per cache line.  Instead each row is copied global->LDS in a
// coalesced pattern (8 lanes per 128-byte row piece, 8 rows per instruction;
// the residual, kept in fragment-major order between levels, as 1 KB runs)
// and read back in fragment layout with ds_read_b128.  Work goes in half
// groups of two k-steps, double-buffered in this wave's own 4 KB stage areas
// of ring slots 0..5: the ring is idle between a level's sweep and the next
// level's first loads, which the wave issues only after its update, and no
// other wave touches these areas in the meantime.
//
// Fragment-major residual (the fused encoder's internal buffers): for each
// block of 32 rows and each k-step ks < dp/16, two 1 KB runs (q = 0, 1);
// lane L's 16 bytes hold row 32*blk + L%32, features ks*16 + (L/32)*8 +
// q*4 .. +3.  One block is 32*dp floats; buffers cover n rounded up to 128.

enum class RSrc { kFragMajor, kRowF32, kRowBF16 };

// LDS byte offset, within a 4 KB area, of 16-byte chunk m (0..7) of row rho
// (0..31) of a 128-byte fp32 row piece: 8 rows per 1 KB, chunks swizzled so
// that any 16 consecutive lanes reading one chunk index of 16 rows (and any
// 8 consecutive lanes) hit distinct 16-byte bank groups.
__device__ __forceinline__ uint32_t swz_f32(int rho, int m) {
  const int f = (rho & 7) ^ ((rho >> 3) & 1);
  return (uint32_t)((rho >> 3) * 1024 + (rho & 7) * 128 + ((m ^ f) << 4));
}
// The same for a 64-byte bf16 row piece (4 chunks): 16 rows per 1 KB.
__device__ __forceinline__ uint32_t swz_bf16(int rho, int m) {
  const int f = ((rho >> 1) ^ (rho >> 3)) & 3;
  return (uint32_t)((rho >> 4) * 1024 + (rho & 15) * 64 + ((m ^ f) << 4));
}

// This wave's 4 KB area in ring slot k (0..5).
__device__ __forceinline__ uint32_t upd_area(uint32_t ring_lds, int wave, int k) {
  return ring_lds + (uint32_t)k * kSlotBytes + kNormBytes + (uint32_t)wave * 4096u;
}

#define RVQ_DL(o, b) "global_load_lds_dwordx4 %[" #o "], %[" #b "]\n\t"
#define RVQ_M0(a, off) "s_add_u32 m0, %[" #a "], " #off "\n\t"

// Four 1 KB copies into the area at lds: lane offsets o0..o3 from base b
// (one instruction each, the i-th landing at lds + 1 KB * i).
__device__ __forceinline__ void dma_rows4(const void *b, uint32_t lds, uint32_t o0, uint32_t o1,
                                          uint32_t o2, uint32_t o3) {
  uint32_t m0_out;
  asm volatile("s_mov_b32 m0, %[a]\n\t" RVQ_DL(o0, b) RVQ_M0(a, 0x400) RVQ_DL(o1, b)
                   RVQ_M0(a, 0x800) RVQ_DL(o2, b) RVQ_M0(a, 0xc00) RVQ_DL(o3, b)
               : [m0o] "=&{m0}"(m0_out)
               : [a] "s"(lds), [b] "s"(b), [o0] "v"(o0), [o1] "v"(o1), [o2] "v"(o2), [o3] "v"(o3)
               : "memory", "scc");
  (void)m0_out;
}
// Two 1 KB copies (lanes offsets o0, o1).
__device__ __forceinline__ void dma_rows2(const void *b, uint32_t lds, uint32_t o0, uint32_t o1) {
  uint32_t m0_out;
  asm volatile("s_mov_b32 m0, %[a]\n\t" RVQ_DL(o0, b) RVQ_M0(a, 0x400) RVQ_DL(o1, b)
               : [m0o] "=&{m0}"(m0_out)
               : [a] "s"(lds), [b] "s"(b), [o0] "v"(o0), [o1] "v"(o1)
               : "memory", "scc");
  (void)m0_out;
}
#undef RVQ_M0
#undef RVQ_DL

template <int N>
__device__ __forceinline__ void wait_vmcnt_upd() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Lane offsets of this wave's row copies for one level.  Copy instruction i
// (0..3) of an fp32 row piece serves rows 8i .. 8i+7: lane l fetches chunk
// m = (l%8) ^ f(row) of row 8i + l/8.  crow(i) gives that row's index into
// the source (a codeword or an input row), stride the row stride in bytes.
struct RowCopy {
  uint32_t off[4];  // byte offset of the lane's chunk from the copy base, per instruction
  uint32_t hi;      // 64 when the lane's chunk lies in the second k-step (for odd tails,
                    // which fetch the chunk 64 bytes lower instead and never read it)
};

__device__ __forceinline__ RowCopy row_copy_f32(int lane, int64_t stride_bytes,
                                                const int (&rows)[4]) {
  RowCopy c;
  const int p = lane & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rho = 8 * i + (lane >> 3);
    const int f = (rho & 7) ^ ((rho >> 3) & 1);
    const int m = p ^ f;
    c.off[i] = (uint32_t)((int64_t)rows[i] * stride_bytes + m * 16);
  }
  // f(8i + l/8) = (l/8) ^ (i & 1) changes only bit 0 of m across i, so
  // whether m >= 4 is the same for every instruction
  c.hi = ((p ^ (lane >> 3)) >= 4) ? 64u : 0u;
  return c;
}

// Row indices (relative to the copy base) that copy instruction i of an fp32
// piece serves, from per-lane values held by lanes 0..31 (one per row).
__device__ __forceinline__ void rows_f32(int v, int (&rows)[4], int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) rows[i] = __shfl(v, 8 * i + (lane >> 3), 64);
}

// Exact fp32 rescoring of the two candidates and residual update for the
// fused encoder, through LDS.  Lanes L and L+32 hold one row (h = 0, 1) and
// each takes features ks*16 + h*8 + e in order ks, e, accumulating (r - c)^2
// with fmaf; the row's distance is (half 0) + (half 1).  r - c1 is written as
// it goes (fragment-major, when STORE) and becomes the next level's
// B-fragments; rows where c2 wins are redone with every lane taking part.
// Returns the chosen index.  rsrc: the level's residual (fragment-major
// buffer, or for level 0 the fp32 / bf16 input rows of stride dp, based at
// row wbase of this wave, rrow = this lane's row relative to wbase).
template <int KS, RSrc SRC, bool STORE>
__device__ __forceinline__ int update_staged(RowFrags<KS> &bfr, const void *rsrc, int rrow,
                                             float *dst_blk, int dp, const float *cb_l, int c1,
                                             int c2, bool v2, int lane_in, uint32_t ring_lds,
                                             int wave) {
  // Everything below derives from this opaque copy of the lane index, so the
  // compiler cannot hoist lane-dependent addresses out of the level loop and
  // keep them live through the sweep.
  int lane = lane_in;
  opaque1(lane);
  const int h = lane >> 5;
  const int rho = lane & 31;
  const int nks = dp >> 4;                // k-steps inside the row
  const int nhg = (nks + 1) >> 1;         // half groups
  const bool odd = nks & 1;               // the last half group has one k-step
  constexpr int kStores = STORE ? 4 : 0;  // stores a full half group issues

  // residual copies (the same in the first pass and the redo)
  RowCopy rc{};
  uint32_t rc2[2] = {0u, 0u}, rhi2[2] = {0u, 0u};
  if constexpr (SRC == RSrc::kRowF32) {
    int rows[4];
    rows_f32(rrow, rows, lane);
    rc = row_copy_f32(lane, (int64_t)dp * 4, rows);
  } else if constexpr (SRC == RSrc::kRowBF16) {
    // copy instruction i (0, 1) serves rows 16i .. 16i+15: lane l fetches
    // chunk (l%4) ^ f(row) of row 16i + l/4
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 16 * i + (lane >> 2);
      const int rr = __shfl(rrow, r, 64);
      const int f = ((r >> 1) ^ (r >> 3)) & 3;
      const int m = (lane & 3) ^ f;
      rc2[i] = (uint32_t)((int64_t)rr * dp * 2 + m * 16);
      rhi2[i] = m >= 2 ? 32u : 0u;  // chunk in the second k-step (odd tails)
    }
  }
  const uint32_t fm_off = (uint32_t)lane * 16u;

  // Issues the copies of half group hg into buffer b: the residual, then
  // codewords ca (and cb when TWO).
  // Issues the copies of the next half group (hg, in increasing order within
  // a pass) into buffer b: the residual, then codewords ca (and cb when
  // TWO).  The source bases advance by one half group per call through an
  // opaque scalar, so the compiler cannot precompute (and hold) all of them.
  const char *rnext = static_cast<const char *>(rsrc);
  const char *cnext = reinterpret_cast<const char *>(cb_l);
  auto restart = [&]() {
    rnext = static_cast<const char *>(rsrc);
    cnext = reinterpret_cast<const char *>(cb_l);
  };
  auto issue = [&](int hg, int b, const RowCopy &ca, const RowCopy &cbw, auto TWO_) {
    constexpr bool TWO = decltype(TWO_)::value;
    const bool part = odd && hg == nhg - 1;
    const uint32_t ar = upd_area(ring_lds, wave, 3 * b);
    if constexpr (SRC == RSrc::kFragMajor) {
      if (part) dma_rows2(rnext, ar, fm_off, fm_off + 1024u);
      else dma_rows4(rnext, ar, fm_off, fm_off + 1024u, fm_off + 2048u, fm_off + 3072u);
      rnext += 4096;  // two k-steps of 2 KB
    } else if constexpr (SRC == RSrc::kRowF32) {
      const uint32_t d = part ? rc.hi : 0u;
      dma_rows4(rnext, ar, rc.off[0] - d, rc.off[1] - d, rc.off[2] - d, rc.off[3] - d);
      rnext += 128;  // 32 fp32 features
    } else {
      dma_rows2(rnext, ar, rc2[0] - (part ? rhi2[0] : 0u), rc2[1] - (part ? rhi2[1] : 0u));
      rnext += 64;  // 32 bf16 features
    }
    {
      const uint32_t d = part ? ca.hi : 0u;
      dma_rows4(cnext, upd_area(ring_lds, wave, 3 * b + 1), ca.off[0] - d, ca.off[1] - d,
                ca.off[2] - d, ca.off[3] - d);
    }
    if constexpr (TWO) {
      const uint32_t d = part ? cbw.hi : 0u;
      dma_rows4(cnext, upd_area(ring_lds, wave, 3 * b + 2), cbw.off[0] - d, cbw.off[1] - d,
                cbw.off[2] - d, cbw.off[3] - d);
    }
    cnext += 128;
    asm volatile("" : "+s"(rnext), "+s"(cnext));
  };

  // Eight residual features of k-step j (0, 1) of the half group in buffer b.
  auto lds16 = [](uint32_t addr) {
    return *reinterpret_cast<const __attribute__((address_space(3))) f32x4 *>((size_t)addr);
  };
  auto read_r = [&](int b, int j, float (&r)[8]) {
    const uint32_t ar = upd_area(ring_lds, wave, 3 * b);
    if constexpr (SRC == RSrc::kRowBF16) {
      const f32x4 q = lds16(ar + swz_bf16(rho, 2 * j + h));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = __float_as_uint(q[e]);
        r[2 * e] = __uint_as_float(w << 16);
        r[2 * e + 1] = __uint_as_float(w & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint32_t a = SRC == RSrc::kFragMajor
                               ? ar + (uint32_t)(2 * j + q) * 1024u + fm_off
                               : ar + swz_f32(rho, 4 * j + 2 * h + q);
        const f32x4 v = lds16(a);
        r[4 * q] = v[0]; r[4 * q + 1] = v[1]; r[4 * q + 2] = v[2]; r[4 * q + 3] = v[3];
      }
    }
  };
  auto read_c = [&](uint32_t area, int j, float (&c)[8]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const f32x4 v = lds16(area + swz_f32(rho, 4 * j + 2 * h + q));
      c[4 * q] = v[0]; c[4 * q + 1] = v[1]; c[4 * q + 2] = v[2]; c[4 * q + 3] = v[3];
    }
  };
  // r - c of k-step ks into the fragment-major buffer: a uniform base per
  // k-step plus the lane's 32-bit offset (scalar-base stores, so no 64-bit
  // address per k-step is held in VGPRs).
  // (st_off is re-made opaque at the start of each pass, so the redo does not
  // share address values with the first pass and keep them alive between.)
  uint32_t st_off = fm_off;
  auto store = [&](int ks, const float (&v)[8]) {
    char *sb = reinterpret_cast<char *>(dst_blk) + (int64_t)ks * 2048;
    *reinterpret_cast<f32x4 *>(sb + st_off) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4 *>(sb + 1024 + st_off) = f32x4{v[4], v[5], v[6], v[7]};
  };

  // Half groups whose k-steps all lie inside every row this stage count
  // serves need no run-time test; k-steps past the row are never touched
  // (their fragments were built as zeros and stay zero).
  constexpr int kSure = 4 * prev_stage_count(KS / 4);  // k-steps inside every row
  auto sure = [](int hg) { return 2 * hg + 1 < kSure; };

  // First pass: both distances, r - c1 stored and made the next fragments.
  int rows[4];
  rows_f32(c1, rows, lane);
  const RowCopy k1 = row_copy_f32(lane, (int64_t)dp * 4, rows);
  rows_f32(c2, rows, lane);
  const RowCopy k2 = row_copy_f32(lane, (int64_t)dp * 4, rows);
  float p1 = 0.f, p2 = 0.f;
  opaque1(st_off);
  auto first = [&](auto HG_) {
    constexpr int hg = decltype(HG_)::value;
    constexpr int b = hg & 1;
    // this half group's copies have landed (only the previous half group's
    // stores may be newer)
    if constexpr (hg == 0) wait_vmcnt_upd<0>();
    else wait_vmcnt_upd<kStores>();
    if (sure(hg + 1) || hg + 1 < nhg) issue(hg + 1, b ^ 1, k1, k2, std::true_type{});
    static_for<0, 2>([&](auto J_) {
      constexpr int j = decltype(J_)::value;
      constexpr int ks = 2 * hg + j;
      if (ks < kSure || ks < nks) {
        float r[8], a[8], c[8], v[8];
        read_r(b, j, r);
        read_c(upd_area(ring_lds, wave, 3 * b + 1), j, a);
        read_c(upd_area(ring_lds, wave, 3 * b + 2), j, c);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float t = r[e] - a[e];
          const float u = r[e] - c[e];
          p1 = fmaf(t, t, p1);
          p2 = fmaf(u, u, p2);
          v[e] = t;
        }
        if constexpr (STORE) store(ks, v);
        bfr.template set<ks>(to_bf16x8(v));
        // the distance sums are finished here, in order, so the compiler
        // cannot defer them and keep every difference alive
        opaque(p1, p2);
      }
    });
  };
  issue(0, 0, k1, k2, std::true_type{});
  static_for<0, KS / 2>([&](auto G_) {
    constexpr int hg = decltype(G_)::value;
    if (sure(hg) || hg < nhg) first(G_);
  });
  const float q1 = __shfl_xor(p1, 32, 64);
  const float q2 = __shfl_xor(p2, 32, 64);
  const float d1 = h ? q1 + p1 : p1 + q1;
  const float d2 = h ? q2 + p2 : p2 + q2;
  const bool take2 = v2 && (d2 < d1 || (d2 == d1 && c2 < c1));
  // Rows where the second candidate won are redone.  Every lane of the wave
  // takes part (no divergent branch, so fragments are rewritten in place):
  // a lane whose first candidate won recomputes exactly r - c1 again.
  if (__ballot(take2)) {
    const int cs = take2 ? c2 : c1;
    rows_f32(cs, rows, lane);
    const RowCopy kc = row_copy_f32(lane, (int64_t)dp * 4, rows);
    auto redo = [&](auto HG_) {
      constexpr int hg = decltype(HG_)::value;
      constexpr int b = hg & 1;
      if constexpr (hg == 0) wait_vmcnt_upd<0>();
      else wait_vmcnt_upd<kStores>();
      if (sure(hg + 1) || hg + 1 < nhg) issue(hg + 1, b ^ 1, kc, kc, std::false_type{});
      static_for<0, 2>([&](auto J_) {
        constexpr int j = decltype(J_)::value;
        constexpr int ks = 2 * hg + j;
        if (ks < kSure || ks < nks) {
          float r[8], c[8], v[8];
          read_r(b, j, r);
          read_c(upd_area(ring_lds, wave, 3 * b + 1), j, c);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = r[e] - c[e];
          if constexpr (STORE) store(ks, v);
          bfr.template set<ks>(to_bf16x8(v));
        }
      });
    };
    restart();
    st_off = fm_off;
    opaque1(st_off);
    issue(0, 0, kc, kc, std::false_type{});
    static_for<0, KS / 2>([&](auto G_) {
      constexpr int hg = decltype(G_)::value;
      if (sure(hg) || hg < nhg) redo(G_);
    });
  }
  return take2 ? c2 : c1;
}

}  // namespace

template <int S, bool FUSED>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void sweep_kernel(
    EncodeArgs a, int T, int level, int splits, int tiles_per_split) {
  constexpr int KS = 4 * S;
  __shared__ uint4 ring[kSlots * (kSlotBytes / 16)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int rb, sp;
  if (FUSED) {
    rb = blockIdx.x;
    sp = 0;
  } else {
    rb = blockIdx.x / splits;
    sp = blockIdx.x % splits;
  }
  const int64_t row = (int64_t)rb * kRowsPerWG + wave * 32 + (lane & 31);
  const bool live = row < a.n;
  const int64_t rowc = live ? row : a.n - 1;
  const int t0 = FUSED ? 0 : sp * tiles_per_split;
  const int t1 = FUSED ? T : min(T, t0 + tiles_per_split);
  const int ntiles = t1 - t0;
  const int nst = ntiles * S;
  const int l_begin = FUSED ? 0 : level;
  const int l_end = FUSED ? a.L : level + 1;
  const int64_t tile_u4 = tile_bytes(S) / 16;
  const uint32_t ring_lds = (uint32_t)(size_t)((__attribute__((address_space(3))) uint4 *)ring);
  const uint32_t lane_lds = ring_lds + (uint32_t)lane * 16u;

  const uint4 *ls = reinterpret_cast<const uint4 *>(a.stream) + ((int64_t)l_begin * T + t0) * tile_u4;
  // prologue of the first level: stages 0 .. kAhead-1
  auto prologue = [&]() {
    static_for<0, kAhead>([&](auto K_) {
      constexpr int k = decltype(K_)::value;
      if (k < nst) issue_stage(ls, tile_u4, k / S, k % S, k, ring_lds, wave, lane);
    });
  };
  RowFrags<KS> bfr;
  if (FUSED) {
    if (a.x16)
      build_bfrags_bf16<KS>(bfr, a.x16, rowc, a.dp, h);
    else
      build_bfrags<KS>(bfr, a.src0, rowc, a.dp, h);
    prologue();
  } else {
    // one sweep per level and workgroup: the ring fills while the
    // fragments load
    prologue();
    const int ksp = a.dp >> 4;
    build_bfrags_frag<KS>(bfr, a.xfrag + ((int64_t)rb * 4 + wave) * ksp * 64, ksp, lane);
  }
  // B-fragment of the norm k-step: ones at k = 0, 1 (lanes of half 0)
  u32x4 bnorm = {0u, 0u, 0u, 0u};
  if (h == 0) bnorm[0] = 0x3F803F80u;  // two bf16 ones

  for (int l = l_begin; l < l_end; ++l) {
    ls = reinterpret_cast<const uint4 *>(a.stream) + ((int64_t)l * T + t0) * tile_u4;
    // Running top-2 of this lane as (key, base of the key's 64-codeword
    // block).  Blocks come in increasing codeword order and a key's tag is
    // its position in the block, so keeping the earlier entry on equal keys
    // is the (key, index) order.
    float R1 = __builtin_inff(), R2 = __builtin_inff();
    int B1 = kNoIndex, B2 = kNoIndex;

    // byte offsets in the ring of the slots of stages g-1, g and g+1 (the
    // refill of stage g + kAhead goes to the slot of stage g-1)
    uint32_t prv = (kSlots - 1) * kSlotBytes, cur = 0, nxt = kSlotBytes;
    u32x4 pre[4];  // first A-fragments of the next stage, read ahead
    // byte offsets of this wave's lanes in a stage and in a norm block
    const uint32_t soff = (uint32_t)(wave * 256 + lane) * 16u;
    const uint32_t noff = (uint32_t)(wave * 64 + lane) * 16u;
    // One tile: FIRST / LAST say whether it is the level's first / last tile
    // (0 no, 1 yes, 2 only known at run time), so the middle tiles carry no
    // run-time tests of the level's boundaries.
    auto tile = [&](int tt, auto FIRST_, auto LAST_) {
      constexpr int FIRST = decltype(FIRST_)::value, LAST = decltype(LAST_)::value;
      f32x16 acc[4];
      const uint4 *tsb = ls + (int64_t)tt * tile_u4;  // the tile in the stream
      static_for<0, S>([&](auto S_) {
        constexpr int s = decltype(S_)::value;
        const int g = tt * S + s;
        // Stage g+1 must be in LDS for every wave before this stage's block
        // reads ahead into it: wait for this wave's loads of stage g+1 (at
        // most dma_after_next<S>(s) newer loads outstanding), then the
        // barrier, which also means every wave is done with stage g-1, whose
        // slot the refill overwrites.  At the start of a level (update-phase
        // accesses may be interleaved) and near its end, wait for every load.
        if constexpr (FIRST == 2 || LAST == 2) {
          if (g == 0 || g + kAhead - 1 >= nst) wait_vmcnt<0>();
          else wait_vmcnt<dma_after_next<S>(s)>();
        } else if constexpr ((FIRST == 1 && s == 0) || (LAST == 1 && s + kAhead - 1 >= S)) {
          wait_vmcnt<0>();
        } else {
          wait_vmcnt<dma_after_next<S>(s)>();
        }
        barrier_only();
        const uint32_t addr = lane_lds + cur;
        const uint32_t naddr = lane_lds + nxt;
        if constexpr (s == 0 && FIRST == 1) read_tile_norms(pre, addr);
        if constexpr (s == 0 && FIRST == 2) {
          if (tt == 0) read_tile_norms(pre, addr);
        }
        // refill: stage g + kAhead is stage sr of tile tt + dt; the block
        // issues its four stage loads, and its norm block goes first when it
        // opens a tile
        constexpr int sr = (s + kAhead) % S, dt = (s + kAhead) / S;
        const uint4 *gsb = tsb + (dt * tile_u4 + 256 + sr * 1024);
        // (uniform: read from lane 0 so that it is kept in an SGPR for M0)
        const uint32_t lds =
            __builtin_amdgcn_readfirstlane(ring_lds + prv + kNormBytes + (uint32_t)wave * 4096u);
        auto with_refill = [&]() {
          if constexpr (sr == 0)
            dma16(tsb + dt * tile_u4, noff, ring_lds + prv + (uint32_t)wave * kBlockBytes);
          bfr.template stage<s, S, true>(acc, pre, addr, naddr, bnorm, gsb, soff, lds);
        };
        // (the last stage of a level reads ahead into a slot it never uses)
        if constexpr (LAST == 2) {
          // Whether this stage refills is known only at run time.  The block
          // itself must be one asm statement on both paths: two variants
          // would let the compiler give their accumulators different
          // registers and copy them at the join, reading MFMA results whose
          // latency it cannot see.  So the refill loads go first, on their
          // own, and the block is always the one without loads.
          if (g + kAhead < nst) {
            if constexpr (sr == 0)
              dma16(tsb + dt * tile_u4, noff, ring_lds + prv + (uint32_t)wave * kBlockBytes);
            dma_stage(gsb, soff, lds);
          }
          bfr.template stage<s, S, false>(acc, pre, addr, naddr, bnorm, gsb, soff, lds);
        } else if constexpr (LAST == 0 || s + kAhead < S) {
          with_refill();
        } else {
          bfr.template stage<s, S, false>(acc, pre, addr, naddr, bnorm, gsb, soff, lds);
        }
        prv = cur;
        cur = nxt;
        nxt = nxt == (kSlots - 1) * kSlotBytes ? 0u : nxt + kSlotBytes;
      });
      mfma_drain(acc);
      // Epilogue: accumulator element i of sub-tile j is codeword
      // j*32 + (i/4)*8 + h*4 + i%4 of the tile for this lane's row.  Per
      // 64-codeword block p (sub-tiles 2p, 2p+1) the tag jj*16 + i is unique.
      // Each key costs three VALU ops: pack, then the two-smallest update
      // with med3 (med3(a, b, -inf) is min(a, b)).
      const float ninf = -__builtin_inff();
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        float k1 = __builtin_inff(), k2 = __builtin_inff();
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float key = pack_key(acc[2 * p + jj][i], (uint32_t)(jj * 16 + i));
            k2 = __builtin_amdgcn_fmed3f(k1, k2, key);
            k1 = __builtin_amdgcn_fmed3f(k1, key, ninf);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        const int base = (t0 + tt) * kTileCw + p * 64 + h * 4;
        const bool c = k1 < R1;
        const float old = c ? R1 : R2;
        const int oldb = c ? B1 : B2;
        const float nw = c ? k2 : k1;
        R1 = c ? k1 : R1;
        B1 = c ? base : B1;
        const bool d = nw < old;
        R2 = d ? nw : old;
        B2 = d ? base : oldb;
      }
    };
    using TNo = std::integral_constant<int, 0>;
    using TYes = std::integral_constant<int, 1>;
    using TRun = std::integral_constant<int, 2>;
    if constexpr (S >= kAhead) {
      // with at least kAhead stages per tile only the first and the last
      // tile of a level see its boundaries
      if (ntiles == 1) {
        tile(0, TYes{}, TYes{});
      } else {
        tile(0, TYes{}, TNo{});
        for (int tt = 1; tt + 1 < ntiles; ++tt) tile(tt, TNo{}, TNo{});
        tile(ntiles - 1, TNo{}, TYes{});
      }
    } else {
      for (int tt = 0; tt < ntiles; ++tt) tile(tt, TRun{}, TRun{});
    }

    // Decode the tags, then merge with the other half of the row (lanes L
    // and L+32 hold the same row over disjoint codewords).
    float S1 = R1, S2 = R2;
    int I1 = block_index(R1, B1), I2 = block_index(R2, B2);
    {
      const float t1 = __shfl_xor(S1, 32, 64), t2 = __shfl_xor(S2, 32, 64);
      const int j1 = __shfl_xor(I1, 32, 64), j2 = __shfl_xor(I2, 32, 64);
      merge_top2(S1, I1, S2, I2, t1, j1, t2, j2);
    }

    if (FUSED) {
      // every wave is done with the ring: the update may use this wave's
      // areas of it
      barrier_only();
      int c1, c2;
      bool v2;
      candidates(I1, I2, a.K, c1, c2, v2);
      const bool store = l + 1 < a.L || a.res_final != nullptr;
      // this wave's block of 32 rows in the fragment-major buffers
      const int64_t blk_off = ((int64_t)rb * 4 + wave) * 32 * a.dp;
      float *dst = a.rbuf[(l + 1) & 1] + blk_off;
      const float *cb_l = a.cb + (int64_t)l * a.K * a.dp;
      int id;
      if (l == 0) {
        // input rows, based at this wave's first row (clamped into the batch)
        const int64_t w0 = (int64_t)rb * kRowsPerWG + wave * 32;
        const int64_t wbase = w0 < a.n ? w0 : a.n - 1;
        const int rrow = (int)(rowc - wbase);
        if (a.x16)
          id = update_staged<KS, RSrc::kRowBF16, true>(bfr, a.x16 + wbase * a.dp, rrow, dst, a.dp,
                                                       cb_l, c1, c2, v2, lane, ring_lds, wave);
        else
          id = update_staged<KS, RSrc::kRowF32, true>(bfr, a.src0 + wbase * a.dp, rrow, dst, a.dp,
                                                      cb_l, c1, c2, v2, lane, ring_lds, wave);
      } else if (store) {
        id = update_staged<KS, RSrc::kFragMajor, true>(bfr, a.rbuf[l & 1] + blk_off, 0, dst, a.dp,
                                                       cb_l, c1, c2, v2, lane, ring_lds, wave);
      } else {
        id = update_staged<KS, RSrc::kFragMajor, false>(bfr, a.rbuf[l & 1] + blk_off, 0, dst,
                                                         a.dp, cb_l, c1, c2, v2, lane, ring_lds,
                                                         wave);
      }
      if (live && h == 0) a.ids[row * a.L + l] = id;
      if (l + 1 < l_end) {
        // the next level's first stages, into this wave's areas of the ring
        // (its own update is done with them; other waves touch only theirs)
        const uint4 *ln =
            reinterpret_cast<const uint4 *>(a.stream) + ((int64_t)(l + 1) * T + t0) * tile_u4;
        static_for<0, kAhead>([&](auto K_) {
          constexpr int k = decltype(K_)::value;
          if (k < nst) issue_stage(ln, tile_u4, k / S, k % S, k, ring_lds, wave, lane);
        });
      }
    } else {
      if (live && h == 0)
        a.part[row * splits + sp] = make_float4(S1, __int_as_float(I1), S2, __int_as_float(I2));
    }
  }
}

// c ? a : b by components (a select of whole array elements becomes a
// select of their addresses, which keeps the arrays in scratch memory)
__device__ __forceinline__ float4 select4(bool c, float4 a, float4 b) {
  return make_float4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}

// Split mode, after every split of a level wrote its list: one wave per
// row, four rows per workgroup.  The wave merges the row's lists, then
// rescores the two candidates exactly as the fused kernel does: for
// candidate c and half h, one lane accumulates (r - c)^2 over features
// ks*16 + h*8 + e, in order ks, e, with fmaf, and the distance is
// (half 0) + (half 1).  The smaller distance wins, the lower index on a tie.
// Every lane loads 16-byte pieces of the row and of both candidates, all in
// flight at once, and forms r - c for both; the four accumulating lanes read
// these back from this wave's area of LDS, and the winner's r - c is written
// from the registers.
template <int S>
__global__ __launch_bounds__(NT) void split_update_kernel(EncodeArgs a, int level, int splits) {
  constexpr int kRow4 = S * kStageCols / 4;  // float4 capacity of a row (dp <= 64 S)
  constexpr int NV = (kRow4 + 63) / 64;      // float4 of a row per lane
  __shared__ float4 area[4][2][kRow4];       // per wave: r - c1, r - c2
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= a.n) return;
  const int dp4 = a.dp >> 2;
  // (selects, not a run-time index into the argument struct, which would
  // copy it to scratch)
  const float *src = level == 0 ? a.src0 : (level & 1) ? a.rbuf[1] : a.rbuf[0];
  const float4 *rs = reinterpret_cast<const float4 *>(src + row * a.dp);
  float4 r[NV], x1[NV], x2[NV];
  static_for<0, NV>([&](auto V_) {
    constexpr int v = decltype(V_)::value;
    const int i = lane + 64 * v;
    if (i < dp4) r[v] = rs[i];
  });

  // Lane j merges the lists of splits j, j + 64, ..., then a butterfly
  // merges the lanes' lists.  Every split holds at least one tile, so its
  // list has two real, distinct codewords, and with finite scores the two
  // smallest of all of them under the total order are unique: any merge
  // order, the fused kernel's included, gives the same pair.
  float S1 = __builtin_inff(), S2 = __builtin_inff();
  int I1 = kNoIndex, I2 = kNoIndex;
  const float4 *pp = a.part + row * splits;
  for (int sp = lane; sp < splits; sp += 64) {
    const float4 e = pp[sp];
    merge_top2(S1, I1, S2, I2, e.x, __float_as_int(e.y), e.z, __float_as_int(e.w));
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float u1 = __shfl_xor(S1, off, 64), u2 = __shfl_xor(S2, off, 64);
    const int j1 = __shfl_xor(I1, off, 64), j2 = __shfl_xor(I2, off, 64);
    merge_top2(S1, I1, S2, I2, u1, j1, u2, j2);
  }
  int c1, c2;
  bool v2;
  candidates(I1, I2, a.K, c1, c2, v2);  // c2 == c1 when there is no second
  c1 = __builtin_amdgcn_readfirstlane(c1);  // (the same in every lane)
  c2 = __builtin_amdgcn_readfirstlane(c2);
  const float *cb_l = a.cb + (int64_t)level * a.K * a.dp;
  const float4 *p1 = reinterpret_cast<const float4 *>(cb_l + (int64_t)c1 * a.dp);
  const float4 *p2 = reinterpret_cast<const float4 *>(cb_l + (int64_t)c2 * a.dp);
  static_for<0, NV>([&](auto V_) {
    constexpr int v = decltype(V_)::value;
    const int i = lane + 64 * v;
    if (i < dp4) {
      x1[v] = p1[i];
      x2[v] = p2[i];
    }
  });
  // r - c for both candidates, elementwise in every lane (the residual
  // of whichever wins), then into this wave's area for the accumulating lanes
  float4 t1[NV], t2[NV];
  static_for<0, NV>([&](auto V_) {
    constexpr int v = decltype(V_)::value;
    const int i = lane + 64 * v;
    if (i < dp4) {
      t1[v] = make_float4(r[v].x - x1[v].x, r[v].y - x1[v].y, r[v].z - x1[v].z, r[v].w - x1[v].w);
      t2[v] = make_float4(r[v].x - x2[v].x, r[v].y - x2[v].y, r[v].z - x2[v].z, r[v].w - x2[v].w);
      area[wave][0][i] = t1[v];
      area[wave][1][i] = t2[v];
    }
  });
  // the area is this wave's alone: order its writes before the reads of
  // other lanes of the same wave
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float p = 0.f;
  if (lane < 4) {
    // lane 2c + h: candidate c + 1, half h
    const float4 *tl = &area[wave][lane >> 1][(lane & 1) * 2];
    const int kend = a.dp >> 4;
#pragma unroll 4
    for (int ks = 0; ks < kend; ++ks) {
      const float4 ta = tl[ks * 4], tb = tl[ks * 4 + 1];
      const float tv[8] = {ta.x, ta.y, ta.z, ta.w, tb.x, tb.y, tb.z, tb.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) p = fmaf(tv[e], tv[e], p);
    }
  }
  const float d1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), 0)) +
                   __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), 1));
  const float d2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), 2)) +
                   __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), 3));
  const bool take2 = v2 && (d2 < d1 || (d2 == d1 && c2 < c1));
  float *dst = level == a.L - 1 ? a.res_final : (level & 1) ? a.rbuf[0] : a.rbuf[1];
  if (dst != nullptr) {
    float4 *ds = reinterpret_cast<float4 *>(dst + row * a.dp);
    static_for<0, NV>([&](auto V_) {
      constexpr int v = decltype(V_)::value;
      const int i = lane + 64 * v;
      if (i < dp4) ds[i] = select4(take2, t2[v], t1[v]);
    });
  }
  if (level + 1 < a.L) {
    // bf16 fragment copy for the next level's sweep: the 4 features of a
    // float4 are half q of lane (h*32 + row%32)'s 16 bytes of k-step ks
    uint2 *fr = reinterpret_cast<uint2 *>(a.xfrag + (row >> 5) * (a.dp >> 4) * 64);
    const int rl = (int)(row & 31);
    static_for<0, NV>([&](auto V_) {
      constexpr int v = decltype(V_)::value;
      const int i = lane + 64 * v;
      if (i < dp4) {
        const float4 t = select4(take2, t2[v], t1[v]);
        const bf16x2 lo = {(__bf16)t.x, (__bf16)t.y};
        const bf16x2 hi = {(__bf16)t.z, (__bf16)t.w};
        const int ks = i >> 2, hq = i & 3;
        fr[((ks * 64 + (hq >> 1) * 32 + rl) << 1) + (hq & 1)] =
            make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
      }
    });
  }
  if (lane == 0) a.ids[row * a.L + level] = take2 ? c2 : c1;
}

template <int S>
hipError_t launch_stage_count(const EncodePlan &p, const EncodeArgs &a, hipEvent_t *ev, hipStream_t s) {
  hipError_t e;
  if (p.fused) {
    if (ev && (e = hipEventRecord(ev[0], s)) != hipSuccess) return e;
    sweep_kernel<S, true><<<dim3(p.row_blocks), dim3(NT), 0, s>>>(a, p.tiles, 0, 1, p.tiles);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev && (e = hipEventRecord(ev[1], s)) != hipSuccess) return e;
    return hipSuccess;
  }
  for (int l = 0; l < a.L; ++l) {
    if (ev && (e = hipEventRecord(ev[2 * l], s)) != hipSuccess) return e;
    sweep_kernel<S, false><<<dim3(p.row_blocks * p.splits), dim3(NT), 0, s>>>(
        a, p.tiles, l, p.splits, p.tiles_per_split);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev && (e = hipEventRecord(ev[2 * l + 1], s)) != hipSuccess) return e;
    split_update_kernel<S><<<dim3((unsigned)ceil_div(a.n, 4)), dim3(NT), 0, s>>>(a, l, p.splits);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}


}  // namespace rvq
