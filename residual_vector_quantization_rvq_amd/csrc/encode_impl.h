// encode_impl.h -- the encoder kernels (templates instantiated per stage count
// in the encode_s*.hip units).
#pragma once
//
// Method: "LongCat-2.5 发布：面向智能体任务的原生多模态大模型", section
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
//    (3 VALU ops per score); a block whose smallest key lies within the
//    row's screening band (common.h, screen_band) of the running minimum
//    goes on the lane's list.  Minima are merged exactly under the
//    (key, index) order.
//  * Fused mode (enough rows to fill the GPU): all levels run in one launch;
//    after a level's sweep the row's smallest key fixes the band, and lanes
//    L and L+32 of a wave rescore every candidate inside it exactly in fp32
//    (sum of squared differences, each lane one half of the features in a
//    fixed order); a block whose second key is inside the band too is
//    rescored whole, and a level whose candidates could not all be kept is
//    flagged for the exact scan after the launch.  The smallest distance
//    wins (lower index on a tie); it is subtracted from the fp32 residual
//    and the B-fragments for the next level are rebuilt in registers.
//  * Split mode (few rows): a level's codeword tiles are split over
//    several workgroups per row block, each writing its band list as a
//    record; a second kernel merges the records and runs the same
//    rescoring and update.
// Every score depends only on (row, codeword): one MFMA shape, one k-step
// order, one key rule and a total order for merging, so the IDs and
// residuals are bitwise independent of batch size, row position and mode.
#include <type_traits>

#include "common.h"

namespace rvq {

namespace {

constexpr int NT = 256;

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
// Sub-tiles of a tile whose keys are formed during the next tile's first
// stage blocks (2 or 4; the rest right after the tile).
constexpr int kCarry = 1;
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
// fewer cycles than a 64-bit per-lane address.  (Prefix RVQ_DY: with
// refill loads, RVQ_DN: without.)
#define RVQ_DY_0 "s_mov_b32 m0, %[lds]\n\tglobal_load_lds_dwordx4 %[voff], %[gsb]\n\t"
#define RVQ_DY_1 "global_load_lds_dwordx4 %[voff], %[gsb] offset:1024\n\t"
#define RVQ_DY_2 "global_load_lds_dwordx4 %[voff], %[gsb] offset:2048\n\t"
#define RVQ_DY_3 "global_load_lds_dwordx4 %[voff], %[gsb] offset:3072\n\t"
#define RVQ_DN_0 ""
#define RVQ_DN_1 ""
#define RVQ_DN_2 ""
#define RVQ_DN_3 ""

// Epilogue keys.  Accumulator element i of a sub-tile becomes a key: the
// score with the 5-bit tag t in its low bits (v_and_or), then the block's two
// smallest keys k2 = med3(k1, k2, key) and k1 = min(k1, key): three VALU ops
// per score.  Written out: compiled, each min would first canonicalise both
// operands.
#define RVQ_KEY(i, t)                                     \
  "v_and_or_b32 %[key], %[a" #i "], %[keep], " #t "\n\t" \
  "v_med3_f32 %[k2], %[k1], %[k2], %[key]\n\t"           \
  "v_min_f32 %[k1], %[k1], %[key]\n\t"
// A block can carry the keys of the previous tile's sub-tile, one score
// after each of its sixteen k-step MFMAs, so they issue while the matrix
// core works.  Prefix RVQ_EL: tags 0..15 (an even sub-tile), RVQ_EH: tags
// 16..31 (an odd one), RVQ_EN: none.
#define RVQ_EN_0 ""
#define RVQ_EN_1 ""
#define RVQ_EN_2 ""
#define RVQ_EN_3 ""
#define RVQ_EN_4 ""
#define RVQ_EN_5 ""
#define RVQ_EN_6 ""
#define RVQ_EN_7 ""
#define RVQ_EN_8 ""
#define RVQ_EN_9 ""
#define RVQ_EN_10 ""
#define RVQ_EN_11 ""
#define RVQ_EN_12 ""
#define RVQ_EN_13 ""
#define RVQ_EN_14 ""
#define RVQ_EN_15 ""
#define RVQ_EL_0 RVQ_KEY(0, 0)
#define RVQ_EL_1 RVQ_KEY(1, 1)
#define RVQ_EL_2 RVQ_KEY(2, 2)
#define RVQ_EL_3 RVQ_KEY(3, 3)
#define RVQ_EL_4 RVQ_KEY(4, 4)
#define RVQ_EL_5 RVQ_KEY(5, 5)
#define RVQ_EL_6 RVQ_KEY(6, 6)
#define RVQ_EL_7 RVQ_KEY(7, 7)
#define RVQ_EL_8 RVQ_KEY(8, 8)
#define RVQ_EL_9 RVQ_KEY(9, 9)
#define RVQ_EL_10 RVQ_KEY(10, 10)
#define RVQ_EL_11 RVQ_KEY(11, 11)
#define RVQ_EL_12 RVQ_KEY(12, 12)
#define RVQ_EL_13 RVQ_KEY(13, 13)
#define RVQ_EL_14 RVQ_KEY(14, 14)
#define RVQ_EL_15 RVQ_KEY(15, 15)
#define RVQ_EH_0 RVQ_KEY(0, 16)
#define RVQ_EH_1 RVQ_KEY(1, 17)
#define RVQ_EH_2 RVQ_KEY(2, 18)
#define RVQ_EH_3 RVQ_KEY(3, 19)
#define RVQ_EH_4 RVQ_KEY(4, 20)
#define RVQ_EH_5 RVQ_KEY(5, 21)
#define RVQ_EH_6 RVQ_KEY(6, 22)
#define RVQ_EH_7 RVQ_KEY(7, 23)
#define RVQ_EH_8 RVQ_KEY(8, 24)
#define RVQ_EH_9 RVQ_KEY(9, 25)
#define RVQ_EH_10 RVQ_KEY(10, 26)
#define RVQ_EH_11 RVQ_KEY(11, 27)
#define RVQ_EH_12 RVQ_KEY(12, 28)
#define RVQ_EH_13 RVQ_KEY(13, 29)
#define RVQ_EH_14 RVQ_KEY(14, 30)
#define RVQ_EH_15 RVQ_KEY(15, 31)

// A stage inside a tile: p holds its k-step 0 on entry.  Reads are spread
// one per MFMA, each five MFMAs ahead of its use, and a refill load follows
// the first MFMA of each k-step: evenly spaced requests keep the LDS queue
// short.  (Probes of this block measured 682 cycles with reads in bursts of
// four one k-step ahead, 657 spread four ahead, 635 as here.)
#define RVQ_STAGE_BODY(NX, D, E)                                                                 \
  RVQ_WAIT(0) RVQ_RD(t0, addr, 5120) RVQ_RD(t1, addr, 9216) RVQ_MF(c0, p0, b0) D##_0 E##_0       \
  RVQ_RD(t2, addr, 13312) RVQ_MF(c1, p1, b0) E##_1 RVQ_RD(t3, addr, 17408) RVQ_MF(c2, p2, b0)    \
  E##_2 RVQ_RD(t4, addr, 6144) RVQ_MF(c3, p3, b0) E##_3 RVQ_RD(t5, addr, 10240) RVQ_WAIT(5)      \
  RVQ_MF(c0, t0, b1) D##_1 E##_4 RVQ_RD(t6, addr, 14336) RVQ_WAIT(5) RVQ_MF(c1, t1, b1) E##_5    \
  RVQ_RD(t7, addr, 18432) RVQ_WAIT(5) RVQ_MF(c2, t2, b1) E##_6 RVQ_RD(t0, addr, 7168)            \
  RVQ_WAIT(5) RVQ_MF(c3, t3, b1) E##_7 RVQ_RD(t1, addr, 11264) RVQ_WAIT(5) RVQ_MF(c0, t4, b2)    \
  D##_2 E##_8 RVQ_RD(t2, addr, 15360) RVQ_WAIT(5) RVQ_MF(c1, t5, b2) E##_9                       \
  RVQ_RD(t3, addr, 19456) RVQ_WAIT(5) RVQ_MF(c2, t6, b2) E##_10 NX##_0 RVQ_WAIT(5)               \
  RVQ_MF(c3, t7, b2) E##_11 NX##_1 RVQ_WAIT(5) RVQ_MF(c0, t0, b3) D##_3 E##_12 NX##_2            \
  RVQ_WAIT(5) RVQ_MF(c1, t1, b3) E##_13 NX##_3 RVQ_WAIT(5) RVQ_MF(c2, t2, b3) E##_14 RVQ_WAIT(4) \
  RVQ_MF(c3, t3, b3) E##_15 RVQ_WAIT(0)

// The stage opening a tile: p holds the norm k-step on entry, and the
// accumulators start from ||c||^2 (B = ones at k = 0, 1).  Its keys start
// after five MFMAs, long after the previous tile's last accumulator write
// has landed.
#define RVQ_MFN(c, a) "v_mfma_f32_32x32x16_bf16 %[" #c "], %[" #a "], %[bn], 0\n\t"
#define RVQ_STAGE0_BODY(NX, D, E)                                                                \
  RVQ_WAIT(0) RVQ_RD(t0, addr, 4096) RVQ_RD(t1, addr, 8192) RVQ_MFN(c0, p0)                      \
  RVQ_RD(t2, addr, 12288) RVQ_MFN(c1, p1) RVQ_RD(t3, addr, 16384) RVQ_MFN(c2, p2)                \
  RVQ_RD(t4, addr, 5120) RVQ_MFN(c3, p3) RVQ_RD(t5, addr, 9216) RVQ_WAIT(5)                      \
  RVQ_MF(c0, t0, b0) D##_0 E##_0 RVQ_RD(t6, addr, 13312) RVQ_WAIT(5) RVQ_MF(c1, t1, b0) E##_1    \
  RVQ_RD(t7, addr, 17408) RVQ_WAIT(5) RVQ_MF(c2, t2, b0) E##_2 RVQ_RD(t0, addr, 6144)            \
  RVQ_WAIT(5) RVQ_MF(c3, t3, b0) E##_3 RVQ_RD(t1, addr, 10240) RVQ_WAIT(5) RVQ_MF(c0, t4, b1)    \
  D##_1 E##_4 RVQ_RD(t2, addr, 14336) RVQ_WAIT(5) RVQ_MF(c1, t5, b1) E##_5                       \
  RVQ_RD(t3, addr, 18432) RVQ_WAIT(5) RVQ_MF(c2, t6, b1) E##_6 RVQ_RD(t4, addr, 7168)            \
  RVQ_WAIT(5) RVQ_MF(c3, t7, b1) E##_7 RVQ_RD(t5, addr, 11264) RVQ_WAIT(5) RVQ_MF(c0, t0, b2)    \
  D##_2 E##_8 RVQ_RD(t6, addr, 15360) RVQ_WAIT(5) RVQ_MF(c1, t1, b2) E##_9                       \
  RVQ_RD(t7, addr, 19456) RVQ_WAIT(5) RVQ_MF(c2, t2, b2) E##_10 NX##_0 RVQ_WAIT(5)               \
  RVQ_MF(c3, t3, b2) E##_11 NX##_1 RVQ_WAIT(5) RVQ_MF(c0, t4, b3) D##_3 E##_12 NX##_2            \
  RVQ_WAIT(5) RVQ_MF(c1, t5, b3) E##_13 NX##_3 RVQ_WAIT(5) RVQ_MF(c2, t6, b3) E##_14 RVQ_WAIT(4) \
  RVQ_MF(c3, t7, b3) E##_15 RVQ_WAIT(0)

// Operand lists, as function-like macros so that they expand only where
// the asm statement is formed.
#define RVQ_OA_W() [c0] "=&v"(c[0]), [c1] "=&v"(c[1]), [c2] "=&v"(c[2]), [c3] "=&v"(c[3])
#define RVQ_OA_RW() [c0] "+v"(c[0]), [c1] "+v"(c[1]), [c2] "+v"(c[2]), [c3] "+v"(c[3])
#define RVQ_OUT_COMMON                                                                         \
  [p0] "+v"(p[0]), [p1] "+v"(p[1]), [p2] "+v"(p[2]), [p3] "+v"(p[3]), [t0] "=&v"(t[0]),      \
      [t1] "=&v"(t[1]), [t2] "=&v"(t[2]), [t3] "=&v"(t[3]), [t4] "=&v"(t[4]), [t5] "=&v"(t[5]), \
      [t6] "=&v"(t[6]), [t7] "=&v"(t[7]), [m0o] "=&{m0}"(m0_out)
#define RVQ_IN_COMMON(cls)                                                                       \
  [addr] "v"(addr), [naddr] "v"(naddr), [b0] #cls(b0), [b1] #cls(b1), [b2] #cls(b2),          \
      [b3] #cls(b3), [gsb] "s"(gsb), [voff] "v"(voff), [lds] "s"(lds)
#define RVQ_NONE()
#define RVQ_IN_BN() , [bn] "v"(bn)
#define RVQ_OUT_KEYS() , [k1] "+v"(k1), [k2] "+v"(k2), [key] "=&v"(key)
#define RVQ_IN_KEYS_LIST                                                                      \
  [a0] "v"(e[0]), [a1] "v"(e[1]), [a2] "v"(e[2]), [a3] "v"(e[3]), [a4] "v"(e[4]),               \
      [a5] "v"(e[5]), [a6] "v"(e[6]), [a7] "v"(e[7]), [a8] "v"(e[8]), [a9] "v"(e[9]),           \
      [a10] "v"(e[10]), [a11] "v"(e[11]), [a12] "v"(e[12]), [a13] "v"(e[13]), [a14] "v"(e[14]), \
      [a15] "v"(e[15]), [keep] "s"(keep)
#define RVQ_IN_KEYS() , RVQ_IN_KEYS_LIST

// FIRST: the stage opens a tile.  NEXT_TILE: the next stage opens a tile.
// B_IN_AGPR: the stage's row fragments live in AGPRs.  DMA: the block also
// issues this wave's refill loads (gsb + voff, lds).  EPI: -1 no keys, 0 / 1
// the keys of sub-tile accumulator e with tags 0..15 / 16..31 folded into
// the block's running pair (k1, k2).
template <bool FIRST, bool NEXT_TILE, bool B_IN_AGPR, bool DMA, int EPI>
__device__ __forceinline__ void stage_block(f32x16 (&c)[4], u32x4 (&p)[4], uint32_t addr,
                                            uint32_t naddr, const u32x4 &bn, const u32x4 &b0,
                                            const u32x4 &b1, const u32x4 &b2, const u32x4 &b3,
                                            const uint4 *gsb, uint32_t voff, uint32_t lds,
                                            const f32x16 &e, float &k1, float &k2) {
  u32x4 t[8];
  uint32_t m0_out;
  float key;
  const uint32_t keep = ~31u;
#define RVQ_SEL4(B, NX, D, E, OA, OK, IB, IK)                                                 \
  if constexpr (B_IN_AGPR)                                                                    \
    asm volatile(B(NX, D, E) : OA(), RVQ_OUT_COMMON OK() : RVQ_IN_COMMON(a) IB() IK() : "memory"); \
  else                                                                                        \
    asm volatile(B(NX, D, E) : OA(), RVQ_OUT_COMMON OK() : RVQ_IN_COMMON(v) IB() IK() : "memory");
#define RVQ_SEL3(B, NX, E, OA, OK, IB, IK)                  \
  if constexpr (DMA) {                                      \
    RVQ_SEL4(B, NX, RVQ_DY, E, OA, OK, IB, IK)              \
  } else {                                                  \
    RVQ_SEL4(B, NX, RVQ_DN, E, OA, OK, IB, IK)              \
  }
#define RVQ_SEL2(B, E, OA, OK, IB, IK)                      \
  if constexpr (NEXT_TILE) {                                \
    RVQ_SEL3(B, RVQ_NEXT_TILE, E, OA, OK, IB, IK)           \
  } else {                                                  \
    RVQ_SEL3(B, RVQ_NEXT_STAGE, E, OA, OK, IB, IK)          \
  }
#define RVQ_SEL1(E, OK, IK)                                           \
  if constexpr (FIRST) {                                              \
    RVQ_SEL2(RVQ_STAGE0_BODY, E, RVQ_OA_W, OK, RVQ_IN_BN, IK)         \
  } else {                                                            \
    RVQ_SEL2(RVQ_STAGE_BODY, E, RVQ_OA_RW, OK, RVQ_NONE, IK)          \
  }
  if constexpr (EPI < 0) {
    RVQ_SEL1(RVQ_EN, RVQ_NONE, RVQ_NONE)
  } else if constexpr (EPI == 0) {
    RVQ_SEL1(RVQ_EL, RVQ_OUT_KEYS, RVQ_IN_KEYS)
  } else {
    RVQ_SEL1(RVQ_EH, RVQ_OUT_KEYS, RVQ_IN_KEYS)
  }
#undef RVQ_SEL1
#undef RVQ_SEL2
#undef RVQ_SEL3
#undef RVQ_SEL4
  (void)m0_out;
  (void)key;
  (void)keep;
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
  template <int s, int S, bool DMA, int EPI = -1>
  __device__ __forceinline__ void stage(f32x16 (&c)[4], u32x4 (&p)[4], uint32_t addr,
                                        uint32_t naddr, const u32x4 &bn, const uint4 *gsb,
                                        uint32_t voff, uint32_t lds, const f32x16 &e, float &k1,
                                        float &k2) const {
    static_assert(NA % 4 == 0, "a stage's k-steps must share a register file");
    stage_block<s == 0, s == S - 1, (s * 4 < NA), DMA, EPI>(
        c, p, addr, naddr, bn, get<s * 4>(), get<s * 4 + 1>(), get<s * 4 + 2>(), get<s * 4 + 3>(),
        gsb, voff, lds, e, k1, k2);
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
// Also returns the band inputs of the row half: srb = sum bf16(v)^2 and
// sdr = sum (v - bf16(v))^2 in feature order (k-steps past the row add zeros).
template <int KS>
__device__ __forceinline__ void build_bfrags(RowFrags<KS> &bfr, const float *src, int64_t row,
                                             int dp, int h, float &srb, float &sdr) {
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
      const float(&w)[8] = v[decltype(U_)::value];
      const u32x4 q = to_bf16x8(w);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float b0 = __uint_as_float(q[e] << 16);
        const float b1 = __uint_as_float(q[e] & 0xffff0000u);
        const float t0 = w[2 * e] - b0, t1 = w[2 * e + 1] - b1;
        srb = fmaf(b0, b0, srb);
        sdr = fmaf(t0, t0, sdr);
        srb = fmaf(b1, b1, srb);
        sdr = fmaf(t1, t1, sdr);
      }
      bfr.template set<ks>(q);
    });
    opaque(row, srb, sdr);
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
// every load of a wave is 1 KB of consecutive bytes.  All KS loads issue
// back to back, straight into the fragment registers, and nothing waits
// for them here: each stage block's first use of its four fragments is
// where the wait goes, so the loads complete under the sweep's first
// stages.  K-steps past the row (ks >= ksp) load k-step ksp-1 again: their
// codebook A-fragments are zero, so any finite fragment adds exactly zero.
template <int KS>
__device__ __forceinline__ void build_bfrags_frag(RowFrags<KS> &bfr, const uint4 *blk, int ksp,
                                                  int lane) {
  static_for<0, KS>([&](auto K_) {
    constexpr int ks = decltype(K_)::value;
    const uint4 q = blk[(ks < ksp ? ks : ksp - 1) * 64 + lane];
    const u32x4 v = u32x4{q.x, q.y, q.z, q.w};
    if constexpr (ks < RowFrags<KS>::NA) bfr.fa[ks] = v;
    else bfr.fv[ks - RowFrags<KS>::NA] = v;
  });
}

// The same fragments straight from bf16 rows (stride dp): the stored bits
// are the fragment.
// (bf16 rows are their own bf16 copy: srb = sum v^2, and the rounding
// part sdr stays zero)
template <int KS>
__device__ __forceinline__ void build_bfrags_bf16(RowFrags<KS> &bfr, const uint16_t *src,
                                                  int64_t row, int dp, int h, float &srb) {
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
      const u32x4 &q = f[decltype(U_)::value];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float b0 = __uint_as_float(q[e] << 16);
        const float b1 = __uint_as_float(q[e] & 0xffff0000u);
        srb = fmaf(b0, b0, srb);
        srb = fmaf(b1, b1, srb);
      }
      bfr.template set<ks>(q);
    });
    opaque(row, srb);
  });
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
  asm volatile(RVQ_DY_0 RVQ_DY_1 RVQ_DY_2 RVQ_DY_3
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

// Split mode, first tile, stage s < kAhead - 1 (stage s+1 still one of the
// prologue's): a lower bound on the loads this wave issued after stage
// s+1's, namely the rest of the prologue (stages s+2 .. kAhead-1), the 4S
// row-fragment loads that follow it, and the refills of stages 0 .. s-1
// (all refills before the level's end when LAST; capped at the counter's
// range).
template <int S, bool LAST>
__host__ __device__ constexpr int split_after_next(int s) {
  int c = 4 * S;
  for (int k = s + 2; k < kAhead; ++k) c += dma_count(k % S);
  for (int k = 0; k < s; ++k)
    if (!LAST || k + kAhead < S) c += dma_count((k + kAhead) % S);
  return c < 63 ? c : 63;
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

// Exact fp32 rescoring of a row's candidates and residual update for the
// fused encoder, through LDS.  Lanes L and L+32 hold one row (h = 0, 1) and
// each takes features ks*16 + h*8 + e in order ks, e, accumulating (r - c)^2
// with fmaf; the row's distance is (half 0) + (half 1).  The candidates are
// ca (the smallest key) and nx more, xc(0) .. xc(nx-1).  The first pass
// scores ca and xc(0), writes r - ca as it goes (fragment-major, when STORE)
// and makes it the next level's B-fragments; further passes score two more
// candidates each; the smallest distance wins, the lower index on a tie, and
// rows where another candidate won are redone with every lane taking part.
// Returns the winner.  st_rb / st_dr: sum bf16(v)^2 and sum (v - bf16(v))^2
// over this lane's half of the winner's v = r - c, in the same feature order
// (the next level's band inputs).  rsrc: the level's residual
// (fragment-major buffer, or for level 0 the fp32 / bf16 input rows of
// stride dp, based at row wbase of this wave, rrow = this lane's row
// relative to wbase).
template <int KS, RSrc SRC, bool STORE, typename XC>
__device__ __forceinline__ int update_staged(RowFrags<KS> &bfr, const void *rsrc, int rrow,
                                             float *dst_blk, int dp, const float *cb_l, int ca,
                                             int nx, XC &&xc, int lane_in, uint32_t ring_lds,
                                             int wave, float &st_rb, float &st_dr) {
  // Everything below derives from this opaque copy of the lane index, so the
  // compiler cannot hoist lane-dependent addresses out of the level loop and
  // keep them live through the sweep.
  int lane = lane_in;
  opaque1(lane);
  int h = lane >> 5;
  int rho = lane & 31;
  const int nks = dp >> 4;                // k-steps inside the row
  const int nhg = (nks + 1) >> 1;         // half groups
  const bool odd = nks & 1;               // the last half group has one k-step
  constexpr int kStores = STORE ? 4 : 0;  // stores a full half group issues

  // residual copies (the same in every pass)
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
  uint32_t fm_off = (uint32_t)lane * 16u;

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
  auto issue = [&](int hg, int b, const RowCopy &ka, const RowCopy &kb, auto TWO_) {
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
      const uint32_t d = part ? ka.hi : 0u;
      dma_rows4(cnext, upd_area(ring_lds, wave, 3 * b + 1), ka.off[0] - d, ka.off[1] - d,
                ka.off[2] - d, ka.off[3] - d);
    }
    if constexpr (TWO) {
      const uint32_t d = part ? kb.hi : 0u;
      dma_rows4(cnext, upd_area(ring_lds, wave, 3 * b + 2), kb.off[0] - d, kb.off[1] - d,
                kb.off[2] - d, kb.off[3] - d);
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
  // band inputs of the next level: bf16(v)^2 and (v - bf16(v))^2 in feature
  // order (q packs the bf16 values of v[2e], v[2e+1] in its low, high half)
  float srb = 0.f, sdr = 0.f;
  auto stat8 = [&](const float (&v)[8], const u32x4 &q) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float b0 = __uint_as_float(q[e] << 16);
      const float b1 = __uint_as_float(q[e] & 0xffff0000u);
      const float t0 = v[2 * e] - b0, t1 = v[2 * e + 1] - b1;
      srb = fmaf(b0, b0, srb);
      sdr = fmaf(t0, t0, sdr);
      srb = fmaf(b1, b1, srb);
      sdr = fmaf(t1, t1, sdr);
    }
  };

  // Half groups whose k-steps all lie inside every row this stage count
  // serves need no run-time test; k-steps past the row are never touched
  // (their fragments were built as zeros and stay zero).
  constexpr int kSure = 4 * prev_stage_count(KS / 4);  // k-steps inside every row
  auto sure = [](int hg) { return 2 * hg + 1 < kSure; };
  auto combine = [&](float p) {
    const float q = __shfl_xor(p, 32, 64);
    return h ? q + p : p + q;
  };

  // First pass: distances of ca and cb0, r - ca stored and made the next
  // fragments.  Without a second candidate in any row of the wave only ca
  // is copied.
  int rows[4];
  const int cb0 = nx > 0 ? xc(0) : ca;
  rows_f32(ca, rows, lane);
  const RowCopy k1 = row_copy_f32(lane, (int64_t)dp * 4, rows);
  rows_f32(cb0, rows, lane);
  const RowCopy k2 = row_copy_f32(lane, (int64_t)dp * 4, rows);
  float p1 = 0.f, p2 = 0.f;
  opaque1(st_off);
  auto first = [&](auto HG_, auto TWO_) {
    constexpr int hg = decltype(HG_)::value;
    constexpr bool TWO = decltype(TWO_)::value;
    constexpr int b = hg & 1;
    // this half group's copies have landed (only the previous half group's
    // stores may be newer)
    if constexpr (hg == 0) wait_vmcnt_upd<0>();
    else wait_vmcnt_upd<kStores>();
    if (sure(hg + 1) || hg + 1 < nhg) issue(hg + 1, b ^ 1, k1, k2, TWO_);
    static_for<0, 2>([&](auto J_) {
      constexpr int j = decltype(J_)::value;
      constexpr int ks = 2 * hg + j;
      if (ks < kSure || ks < nks) {
        float r[8], a[8], v[8];
        read_r(b, j, r);
        read_c(upd_area(ring_lds, wave, 3 * b + 1), j, a);
        if constexpr (TWO) {
          float c[8];
          read_c(upd_area(ring_lds, wave, 3 * b + 2), j, c);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float u = r[e] - c[e];
            p2 = fmaf(u, u, p2);
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float t = r[e] - a[e];
          p1 = fmaf(t, t, p1);
          v[e] = t;
        }
        if constexpr (STORE) store(ks, v);
        const u32x4 q = to_bf16x8(v);
        stat8(v, q);
        bfr.template set<ks>(q);
        // the sums are finished here, in order, so the compiler cannot defer
        // them and keep every difference alive
        opaque(p1, p2, srb, sdr);
      }
    });
  };
  if (__ballot(nx > 0)) {
    issue(0, 0, k1, k2, std::true_type{});
    static_for<0, KS / 2>([&](auto G_) {
      constexpr int hg = decltype(G_)::value;
      if (sure(hg) || hg < nhg) first(G_, std::true_type{});
    });
  } else {
    issue(0, 0, k1, k1, std::false_type{});
    static_for<0, KS / 2>([&](auto G_) {
      constexpr int hg = decltype(G_)::value;
      if (sure(hg) || hg < nhg) first(G_, std::false_type{});
    });
  }
  int best = ca;
  float dbest = combine(p1);
  {
    const float d2 = combine(p2);
    if (nx > 0 && lex_lt(d2, cb0, dbest, best)) {
      best = cb0;
      dbest = d2;
    }
  }
  // Further candidates, two per pass (distances only), at most two passes
  // (kMaxRescore candidates in all; a row with more is left to the exact
  // scan).  Rows with fewer score ca again, which is never taken.  (The
  // passes are unrolled: as a loop, the compiler keeps more values alive
  // across it than the registers hold.)
  static_for<0, 2>([&](auto P_) {
    const int j = 1 + 2 * decltype(P_)::value;
    if (!__ballot(nx > j)) return;
    // (the lane-derived values are re-made opaque each pass, so the compiler
    // cannot hoist the pass's addresses out of the loop and hold them all)
    opaque(h, rho, fm_off);
    const int ea = nx > j ? xc(j) : ca;
    const int eb = nx > j + 1 ? xc(j + 1) : ea;
    rows_f32(ea, rows, lane);
    const RowCopy ke = row_copy_f32(lane, (int64_t)dp * 4, rows);
    rows_f32(eb, rows, lane);
    const RowCopy kf = row_copy_f32(lane, (int64_t)dp * 4, rows);
    float pa = 0.f, pb = 0.f;
    auto scan = [&](auto HG_) {
      constexpr int hg = decltype(HG_)::value;
      constexpr int b = hg & 1;
      wait_vmcnt_upd<0>();
      if (sure(hg + 1) || hg + 1 < nhg) issue(hg + 1, b ^ 1, ke, kf, std::true_type{});
      static_for<0, 2>([&](auto J_) {
        constexpr int jj = decltype(J_)::value;
        constexpr int ks = 2 * hg + jj;
        if (ks < kSure || ks < nks) {
          float r[8], a[8], c[8];
          read_r(b, jj, r);
          read_c(upd_area(ring_lds, wave, 3 * b + 1), jj, a);
          read_c(upd_area(ring_lds, wave, 3 * b + 2), jj, c);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float t = r[e] - a[e];
            const float u = r[e] - c[e];
            pa = fmaf(t, t, pa);
            pb = fmaf(u, u, pb);
          }
          opaque(pa, pb);
        }
      });
    };
    restart();
    issue(0, 0, ke, kf, std::true_type{});
    static_for<0, KS / 2>([&](auto G_) {
      constexpr int hg = decltype(G_)::value;
      if (sure(hg) || hg < nhg) scan(G_);
    });
    const float da = combine(pa), db = combine(pb);
    if (nx > j && lex_lt(da, ea, dbest, best)) {
      best = ea;
      dbest = da;
    }
    if (nx > j + 1 && lex_lt(db, eb, dbest, best)) {
      best = eb;
      dbest = db;
    }
    });
  // Rows where another candidate won are redone.  Every lane of the wave
  // takes part (no divergent branch, so fragments are rewritten in place):
  // a lane whose first candidate won recomputes exactly r - ca again.
  if (__ballot(best != ca)) {
    rows_f32(best, rows, lane);
    const RowCopy kc = row_copy_f32(lane, (int64_t)dp * 4, rows);
    srb = 0.f;
    sdr = 0.f;
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
          const u32x4 q = to_bf16x8(v);
          stat8(v, q);
          bfr.template set<ks>(q);
          opaque(srb, sdr);
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
  st_rb = srb;
  st_dr = sdr;
  return best;
}


// Exact fp32 distances of the 64 codewords of block blk to one row, and the
// nearest of them (the lower index on a tie); used when a block held two
// keys inside the band, so that its third and later keys, which the sweep
// does not keep, may be inside it too.  rget(ks, h, r) reads features
// ks*16 + h*8 .. +7 of the row.  Lane l takes codewords blk*64 + l%32 and
// blk*64 + 32 + l%32 over feature half l/32, summed in the rescoring's order
// (half 0 + half 1), so the winner's distance equals its rescoring.  Every
// lane returns the same index.
template <typename RG>
__device__ __forceinline__ int rescore_block(RG &&rget, int nks, const float *cb_l, int dp, int K,
                                             int blk, int lane) {
  const int h = lane >> 5;
  const int k0 = blk * 64 + (lane & 31), k1 = k0 + 32;
  const float *c0 = cb_l + (int64_t)(k0 < K ? k0 : K - 1) * dp;
  const float *c1 = cb_l + (int64_t)(k1 < K ? k1 : K - 1) * dp;
  float p0 = 0.f, p1 = 0.f;
  // k-steps four at a time, every load of a group issued before its sums
  // (one round trip per group instead of one per k-step); the sums keep
  // their order
  constexpr int G = 4;
  int ks = 0;
  for (; ks + G <= nks; ks += G) {
    float r[G][8], x0[G][8], x1[G][8];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      rget(ks + u, h, r[u]);
      read8(c0, 0, dp, (ks + u) * 16 + h * 8, true, x0[u]);
      read8(c1, 0, dp, (ks + u) * 16 + h * 8, true, x1[u]);
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float t = r[u][e] - x0[u][e], v = r[u][e] - x1[u][e];
        p0 = fmaf(t, t, p0);
        p1 = fmaf(v, v, p1);
      }
    }
  }
  for (; ks < nks; ++ks) {
    float r[8], x0[8], x1[8];
    rget(ks, h, r);
    read8(c0, 0, dp, ks * 16 + h * 8, true, x0);
    read8(c1, 0, dp, ks * 16 + h * 8, true, x1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float t = r[e] - x0[e], u = r[e] - x1[e];
      p0 = fmaf(t, t, p0);
      p1 = fmaf(u, u, p1);
    }
  }
  const float q0 = __shfl_xor(p0, 32, 64), q1 = __shfl_xor(p1, 32, 64);
  const float d0 = h ? q0 + p0 : p0 + q0;
  const float d1 = h ? q1 + p1 : p1 + q1;
  float bd = k0 < K ? d0 : __builtin_inff();
  int bi = k0;
  if (k1 < K && lex_lt(d1, k1, bd, bi)) {
    bd = d1;
    bi = k1;
  }
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) {
    const float od = __shfl_xor(bd, off, 64);
    const int oi = __shfl_xor(bi, off, 64);
    if (lex_lt(od, oi, bd, bi)) {
      bd = od;
      bi = oi;
    }
  }
  return bi;
}

// Per-lane candidate list entry: a 64-codeword block's two smallest keys
// and the block's base (as in block_index).
struct BandEntry {
  float k1, k2;
  int base;
};

// Per-lane state of the candidate band over one level's blocks: the
// smallest key so far and the list entries appended since the last reset
// (more than kList: the list overflowed).
struct BandState {
  float R1;
  int cnt;
};

__device__ __forceinline__ void band_reset(BandState &b) {
  b.R1 = __builtin_inff();
  b.cnt = 0;
}

// One 64-codeword block of this lane (two smallest keys k1 <= k2, block
// base): update the running minimum, and append the block to the lane's
// list when k1 is within the band of the row's running minimum (ref: this
// lane's minimum and the other half's as last exchanged, which is never
// below the row's final minimum).  Every block holding a key inside the
// final band has k1 inside it, and so k1 was inside the band of ref when it
// came; the list (filtered at the end) therefore holds every such block.
// A new minimum more than the band below every earlier key of the lane
// makes all its entries stale, which empties the list; a full list first
// drops the entries that are no longer inside the band of ref, and only
// overflows (cnt > kList) when kList entries still are.
__device__ __forceinline__ void band_block(BandState &b, float k1, float k2, int base, float band,
                                           float r_other, BandEntry *list) {
  const float r_old = b.R1;
  b.R1 = __builtin_amdgcn_fmed3f(b.R1, k1, -__builtin_inff());  // min
  b.cnt = __fadd_rn(k1, band) < r_old ? 0 : b.cnt;
  const float lim = __fadd_rn(__builtin_amdgcn_fmed3f(b.R1, r_other, -__builtin_inff()), band);
  if (k1 <= lim) {
    if (b.cnt == kList) {
      int m = 0;
      for (int j = 0; j < kList; ++j) {
        const BandEntry e = list[j];
        if (e.k1 <= lim) list[m++] = e;
      }
      b.cnt = m;
    }
    if (b.cnt < kList) list[b.cnt] = BandEntry{k1, k2, base};
    ++b.cnt;
  }
}

// The end of a level for one lane: from its list, the smallest key's
// codeword (ca, key ka; (key, index) order), and the blocks inside the
// final band thr.  Indices of blocks whose k1 is inside the band but whose
// k2 is not are compacted, in place, into list[0 .. nx) (base field), as
// candidates next to ca; a block with k2 inside the band may hold more keys
// inside it than the two the sweep keeps, so it is reported as fblk (block
// id, base / 64) and counted in nfail instead.
__device__ __forceinline__ void band_finish(const BandState &b, BandEntry *list, float &ka,
                                            int &ia) {
  ka = __builtin_inff();
  ia = kNoIndex;
  const int nl = b.cnt < kList ? b.cnt : kList;
  for (int j = 0; j < kList; ++j) {
    if (j < nl) {
      const BandEntry e = list[j];
      const int i = block_index(e.k1, e.base);
      if (lex_lt(e.k1, i, ka, ia)) {
        ka = e.k1;
        ia = i;
      }
    }
  }
}
__device__ __forceinline__ int band_collect(const BandState &b, BandEntry *list, float thr,
                                            int ca, int K, int &nfail, int &fblk) {
  int nx = 0;
  nfail = 0;
  fblk = -1;
  const int nl = b.cnt < kList ? b.cnt : kList;
  for (int j = 0; j < kList; ++j) {
    if (j < nl) {
      const BandEntry e = list[j];
      if (e.k2 <= thr) {
        ++nfail;
        fblk = e.base >> 6;
      } else if (e.k1 <= thr) {
        const int i = block_index(e.k1, e.base);
        if (i != ca && i >= 0 && i < K) {
          list[nx].base = i;
          ++nx;
        }
      }
    }
  }
  return nx;
}

}  // namespace

template <int S, bool FUSED>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void sweep_kernel(
    EncodeArgs a, int T, int level, int splits, int tiles_per_split) {
  constexpr int KS = 4 * S;
  __shared__ uint4 ring[kSlots * (kSlotBytes / 16)];
  __shared__ BandEntry clist[NT * kList];  // per-lane candidate lists

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
  BandEntry *const mylist = clist + tid * kList;
  // band inputs of the row's residual at the current level: sum bf16(r)^2
  // and sum (r - bf16(r))^2, each half in feature order, half 0 + half 1
  float rbn2 = 0.f, drn2 = 0.f;
  auto halves = [&](float v) {
    const float o = __shfl_xor(v, 32, 64);
    return h ? o + v : v + o;
  };
  if (FUSED) {
    float srb = 0.f, sdr = 0.f;
    if (a.x16)
      build_bfrags_bf16<KS>(bfr, a.x16, rowc, a.dp, h, srb);
    else
      build_bfrags<KS>(bfr, a.src0, rowc, a.dp, h, srb, sdr);
    rbn2 = halves(srb);
    drn2 = halves(sdr);
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
    // The candidate band of this row at this level (common.h).  Blocks come
    // in increasing codeword order and a key's tag is its position in the
    // block, so keeping the earlier entry on equal keys is the (key, index)
    // order.
    if (!FUSED) {
      const float2 st = a.rstat[rowc];
      rbn2 = st.x;
      drn2 = st.y;
    }
    const float band = screen_band(rbn2, drn2, a.lstat[4 * l], a.lstat[4 * l + 1], a.d);
    BandState bs;
    band_reset(bs);
    float r_other = __builtin_inff();

    // byte offsets in the ring of the slots of stages g-1, g and g+1 (the
    // refill of stage g + kAhead goes to the slot of stage g-1)
    uint32_t prv = (kSlots - 1) * kSlotBytes, cur = 0, nxt = kSlotBytes;
    u32x4 pre[4];  // first A-fragments of the next stage, read ahead
    // byte offsets of this wave's lanes in a stage and in a norm block
    const uint32_t soff = (uint32_t)(wave * 256 + lane) * 16u;
    const uint32_t noff = (uint32_t)(wave * 64 + lane) * 16u;
    // Epilogue of a tile whose scores are in acc, on its own, for sub-tiles
    // 0 .. nsub-1: the level's last tile (all four), every tile when a tile
    // has too few stages to carry keys into the next one, else the
    // sub-tiles not carried.  Accumulator element i of sub-tile j is
    // codeword j*32 + (i/4)*8 + h*4 + i%4 of the tile for this lane's row.
    // Per 64-codeword block p (sub-tiles 2p, 2p+1) the tag jj*16 + i is
    // unique.  A block left half done (odd nsub) keeps its pair in (ck1, ck2)
    // for the next tile's first carried stage.
    float ck1 = __builtin_inff(), ck2 = __builtin_inff();
    auto epilogue = [&](f32x16(&acc)[4], int tt, auto NSUB_) {
      constexpr int nsub = decltype(NSUB_)::value;
      if constexpr (nsub > 0) {
        mfma_drain(acc);
        const uint32_t keep = ~31u;
        static_for<0, nsub>([&](auto J_) {
          constexpr int j = decltype(J_)::value;
          if constexpr ((j & 1) == 0) {
            ck1 = __builtin_inff();
            ck2 = __builtin_inff();
          }
          const f32x16 &e = acc[j];
          float key;
          if constexpr ((j & 1) == 0)
            asm(RVQ_EL_0 RVQ_EL_1 RVQ_EL_2 RVQ_EL_3 RVQ_EL_4 RVQ_EL_5 RVQ_EL_6 RVQ_EL_7 RVQ_EL_8
                    RVQ_EL_9 RVQ_EL_10 RVQ_EL_11 RVQ_EL_12 RVQ_EL_13 RVQ_EL_14 RVQ_EL_15
                : [k1] "+v"(ck1), [k2] "+v"(ck2), [key] "=&v"(key)
                : RVQ_IN_KEYS_LIST);
          else
            asm(RVQ_EH_0 RVQ_EH_1 RVQ_EH_2 RVQ_EH_3 RVQ_EH_4 RVQ_EH_5 RVQ_EH_6 RVQ_EH_7 RVQ_EH_8
                    RVQ_EH_9 RVQ_EH_10 RVQ_EH_11 RVQ_EH_12 RVQ_EH_13 RVQ_EH_14 RVQ_EH_15
                : [k1] "+v"(ck1), [k2] "+v"(ck2), [key] "=&v"(key)
                : RVQ_IN_KEYS_LIST);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr ((j & 1) == 1) {
            const int base = (t0 + tt) * kTileCw + (j >> 1) * 64 + h * 4;
            // both keys are formed here, key by key (the compiler would
            // otherwise sink k2's chain into the rare append and keep all
            // of the block's keys alive)
            asm volatile("" : "+v"(ck1), "+v"(ck2));
            band_block(bs, ck1, ck2, base, band, r_other, mylist);
          }
        });
        // the other half's running minimum, for the next tile's blocks (the
        // exchange completes under that tile's matrix work)
        if constexpr (nsub == 4) r_other = __shfl_xor(bs.R1, 32, 64);
      }
    };
    // One tile into acc: FIRST / LAST say whether it is the level's first /
    // last tile (0 no, 1 yes, 2 only known at run time), so the middle tiles
    // carry no run-time tests of the level's boundaries.  With PREV, the
    // previous tile's scores are in prev, and this tile's first four stage
    // blocks form their keys, sub-tile s in block s, between their MFMAs;
    // the block pair of sub-tiles 0, 1 goes to the band after stage 1, that
    // of 2, 3 after stage 3.
    auto tile = [&](int tt, auto FIRST_, auto LAST_, f32x16(&acc)[4], f32x16(&prev)[4],
                    auto PREV_) {
      constexpr int FIRST = decltype(FIRST_)::value, LAST = decltype(LAST_)::value;
      constexpr bool PREV = decltype(PREV_)::value;
      static_assert(!PREV || S >= 4, "the previous tile's keys need four stages");
      const uint4 *tsb = ls + (int64_t)tt * tile_u4;  // the tile in the stream
      static_for<0, S>([&](auto S_) {
        constexpr int s = decltype(S_)::value;
        // stage s < kCarry carries sub-tile j of the previous tile
        constexpr int j = 4 - kCarry + s;
        constexpr int EPI = (PREV && s < kCarry) ? (j & 1) : -1;
        const f32x16 &pe = prev[s < kCarry ? j : 0];
        if constexpr (EPI == 0) {
          ck1 = __builtin_inff();
          ck2 = __builtin_inff();
        }
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
        } else if constexpr (!FUSED && FIRST == 1 && s + 1 < kAhead &&
                             !(LAST == 1 && s + kAhead - 1 >= S)) {
          // the row fragments, issued after the prologue, are still on
          // their way: stage s+1's loads are older than all of them
          wait_vmcnt<split_after_next<S, LAST == 1>(s)>();
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
          bfr.template stage<s, S, false, EPI>(acc, pre, addr, naddr, bnorm, gsb, soff, lds, pe,
                                               ck1, ck2);
        } else if constexpr (LAST == 0 || s + kAhead < S) {
          if constexpr (sr == 0)
            dma16(tsb + dt * tile_u4, noff, ring_lds + prv + (uint32_t)wave * kBlockBytes);
          bfr.template stage<s, S, true, EPI>(acc, pre, addr, naddr, bnorm, gsb, soff, lds, pe,
                                              ck1, ck2);
        } else {
          bfr.template stage<s, S, false, EPI>(acc, pre, addr, naddr, bnorm, gsb, soff, lds, pe,
                                               ck1, ck2);
        }
        if constexpr (EPI == 1) {
          // a 64-codeword block of the previous tile is complete
          const int base = (t0 + tt - 1) * kTileCw + (j >> 1) * 64 + h * 4;
          band_block(bs, ck1, ck2, base, band, r_other, mylist);
          if constexpr (j == 3) r_other = __shfl_xor(bs.R1, 32, 64);
        }
        prv = cur;
        cur = nxt;
        nxt = nxt == (kSlots - 1) * kSlotBytes ? 0u : nxt + kSlotBytes;
      });
    };
    using TNo = std::integral_constant<int, 0>;
    using TYes = std::integral_constant<int, 1>;
    using TRun = std::integral_constant<int, 2>;
    using PNo = std::integral_constant<bool, false>;
    using PYes = std::integral_constant<bool, true>;
    // two accumulator sets: tile i writes set i % 2 while its first blocks
    // read the other's last kCarry sub-tiles; the rest of a tile's epilogue
    // runs right after it
    f32x16 accA[4], accB[4];
    using NAll = std::integral_constant<int, 4>;
    using NOwn = std::integral_constant<int, 4 - kCarry>;
    if constexpr (S >= kAhead) {
      // with at least kAhead stages per tile only the first and the last
      // tile of a level see its boundaries
      if (ntiles == 1) {
        tile(0, TYes{}, TYes{}, accA, accB, PNo{});
        epilogue(accA, 0, NAll{});
      } else {
        tile(0, TYes{}, TNo{}, accA, accB, PNo{});
        epilogue(accA, 0, NOwn{});
        for (int tt = 1;; tt += 2) {
          if (tt == ntiles - 1) {
            tile(tt, TNo{}, TYes{}, accB, accA, PYes{});
            epilogue(accB, tt, NAll{});
            break;
          }
          tile(tt, TNo{}, TNo{}, accB, accA, PYes{});
          epilogue(accB, tt, NOwn{});
          if (tt + 1 == ntiles - 1) {
            tile(tt + 1, TNo{}, TYes{}, accA, accB, PYes{});
            epilogue(accA, tt + 1, NAll{});
            break;
          }
          tile(tt + 1, TNo{}, TNo{}, accA, accB, PYes{});
          epilogue(accA, tt + 1, NOwn{});
        }
      }
    } else {
      for (int tt = 0; tt < ntiles; ++tt) {
        tile(tt, TRun{}, TRun{}, accA, accB, PNo{});
        epilogue(accA, tt, NAll{});
      }
    }

    if (FUSED) {
      // smallest key of the row over both halves, (key, index) order
      float ka;
      int i1;
      band_finish(bs, mylist, ka, i1);
      const float o1 = __shfl_xor(ka, 32, 64);
      const int oi1 = __shfl_xor(i1, 32, 64);
      const bool oth = lex_lt(o1, oi1, ka, i1);
      const float rmin = oth ? o1 : ka;
      int ca = oth ? oi1 : i1;
      ca = (ca >= 0 && ca < a.K) ? ca : 0;  // finite inputs always give a valid codeword
      const float thr = __fadd_rn(rmin, band);
      // This lane's other candidates, compacted into its list.  A block
      // whose second key lies inside the band may hold more keys inside it,
      // so that block is rescored whole below; two such blocks, or an
      // overflowing list, leave the level to the exact scan after the launch.
      int nfail, fblk;
      const int nx = band_collect(bs, mylist, thr, ca, a.K, nfail, fblk);
      const int onf = __shfl_xor(nfail, 32, 64);
      const int ofb = __shfl_xor(fblk, 32, 64);
      const bool ovf = __shfl_xor(bs.cnt, 32, 64) > kList || bs.cnt > kList;
      int rcode;
      if (ovf || nfail + onf > 2 || nfail > 1 || onf > 1 ||
          (nfail == 1 && onf == 1 && fblk != ofb))
        rcode = kAuxScan;
      else
        rcode = nfail ? fblk : (onf ? ofb : kAuxOk);

      // every wave is done with the ring: the update may use this wave's
      // areas of it
      barrier_only();
      const bool store = l + 1 < a.L || a.res_final != nullptr;
      // this wave's block of 32 rows in the fragment-major buffers
      const int64_t blk_off = ((int64_t)rb * 4 + wave) * 32 * a.dp;
      float *dst = a.rbuf[(l + 1) & 1] + blk_off;
      const float *cb_l = a.cb + (int64_t)l * a.K * a.dp;
      const int64_t w0 = (int64_t)rb * kRowsPerWG + wave * 32;
      const int64_t wbase = w0 < a.n ? w0 : a.n - 1;
      const int nks = a.dp >> 4;

      // rows with one block to rescore whole (rare): its nearest codeword
      // joins the row's candidates
      int bonus = -1;
      for (uint64_t need = __ballot(h == 0 && rcode >= 0); need; need &= need - 1) {
        const int rl = __builtin_ctzll(need);
        const int blk = __shfl(rcode, rl, 64);
        int bi;
        if (l == 0) {
          const int64_t rr = w0 + rl < a.n ? w0 + rl : a.n - 1;
          if (a.x16)
            bi = rescore_block([&](int ks, int hh, float(&r)[8]) {
              read8_bf16(a.x16, rr, a.dp, ks * 16 + hh * 8, r);
            }, nks, cb_l, a.dp, a.K, blk, lane);
          else
            bi = rescore_block([&](int ks, int hh, float(&r)[8]) {
              read8(a.src0, rr, a.dp, ks * 16 + hh * 8, true, r);
            }, nks, cb_l, a.dp, a.K, blk, lane);
        } else {
          const float4 *fb = reinterpret_cast<const float4 *>(a.rbuf[l & 1] + blk_off);
          bi = rescore_block([&](int ks, int hh, float(&r)[8]) {
            const float4 x = fb[(ks * 2) * 64 + hh * 32 + rl];
            const float4 y = fb[(ks * 2 + 1) * 64 + hh * 32 + rl];
            r[0] = x.x; r[1] = x.y; r[2] = x.z; r[3] = x.w;
            r[4] = y.x; r[5] = y.y; r[6] = y.z; r[7] = y.w;
          }, nks, cb_l, a.dp, a.K, blk, lane);
        }
        if ((lane & 31) == rl && bi >= 0 && bi < a.K) bonus = bi;
      }

      // the row's candidates after ca: half 0's list, half 1's list, then
      // the rescored block's nearest
      const int onx = __shfl_xor(nx, 32, 64);
      const int nx0 = h ? onx : nx;
      const int nxt = nx + onx;
      const BandEntry *lst0 = clist + (wave * 64 + (lane & 31)) * kList;
      const BandEntry *lst1 = lst0 + 32 * kList;
      auto xc = [&](int j) -> int {
        if (j < nx0) return lst0[j].base;
        if (j < nxt) return lst1[j - nx0].base;
        return bonus;
      };
      const int nxa = nxt + (bonus >= 0 ? 1 : 0);
      if (nxa + 1 > kMaxRescore) rcode = kAuxScan;
      float srb = 0.f, sdr = 0.f;
      int id;
      if (l == 0) {
        // input rows, based at this wave's first row (clamped into the batch)
        const int rrow = (int)(rowc - wbase);
        if (a.x16)
          id = update_staged<KS, RSrc::kRowBF16, true>(bfr, a.x16 + wbase * a.dp, rrow, dst, a.dp,
                                                       cb_l, ca, nxa, xc, lane, ring_lds, wave,
                                                       srb, sdr);
        else
          id = update_staged<KS, RSrc::kRowF32, true>(bfr, a.src0 + wbase * a.dp, rrow, dst, a.dp,
                                                      cb_l, ca, nxa, xc, lane, ring_lds, wave, srb,
                                                      sdr);
      } else if (store) {
        id = update_staged<KS, RSrc::kFragMajor, true>(bfr, a.rbuf[l & 1] + blk_off, 0, dst, a.dp,
                                                       cb_l, ca, nxa, xc, lane, ring_lds, wave, srb,
                                                       sdr);
      } else {
        id = update_staged<KS, RSrc::kFragMajor, false>(bfr, a.rbuf[l & 1] + blk_off, 0, dst,
                                                        a.dp, cb_l, ca, nxa, xc, lane, ring_lds,
                                                        wave, srb, sdr);
      }
      rbn2 = halves(srb);
      drn2 = halves(sdr);
      if (live && h == 0) {
        a.ids[row * a.L + l] = id;
        a.aux[row * a.L + l] = rcode == kAuxScan ? kAuxScan : kAuxOk;
      }
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
      // this split's record of the row half (merged by split_update_kernel):
      // [cnt, 0, 0, 0], then the list entries [k1, k2, base, 0]
      if (live) {
        float4 *rec = a.part + (((int64_t)row * splits + sp) * 2 + h) * kRecF4;
        rec[0] = make_float4(__int_as_float(bs.cnt), 0.f, 0.f, 0.f);
        const int nl = bs.cnt < kList ? bs.cnt : kList;
        for (int j = 0; j < nl; ++j) {
          const BandEntry e = mylist[j];
          rec[1 + j] = make_float4(e.k1, e.k2, __int_as_float(e.base), 0.f);
        }
      }
    }
  }
}

// Split mode, after every split of a level wrote its records: one wave per
// row, four rows per workgroup.  The wave merges the records of the row's
// two halves over all splits (the same running minimum, block-second keys
// and band lists the fused kernel keeps for the whole level), collects the
// candidates inside the band, rescores a block whose second key lies inside
// it, and rescores every candidate exactly as the fused kernel does: for
// candidate c and half h, one lane accumulates (r - c)^2 over features
// ks*16 + h*8 + e, in order ks, e, with fmaf, and the distance is
// (half 0) + (half 1).  The smallest distance wins, the lower index on a
// tie.  Candidates go two at a time: every lane loads 16-byte pieces of the
// row and of both codewords, all in flight at once, and forms r - c for
// both; four accumulating lanes read these back from this wave's area of
// LDS, and the winner's r - c is written from the registers.
template <int S>
__global__ __launch_bounds__(NT) void split_update_kernel(EncodeArgs a, int level, int splits,
                                                          int rec_f4) {
  constexpr int kRow4 = S * kStageCols / 4;  // float4 capacity of a row (dp <= 64 S)
  constexpr int NV = (kRow4 + 63) / 64;      // float4 of a row per lane
  constexpr int kMaxCand = 64;
  __shared__ float4 area[4][2][kRow4];       // per wave: r - c of the pair of candidates rescored
  __shared__ int cand[4][kMaxCand + 1];
  __shared__ int ncand[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= a.n) return;
  const int dp4 = a.dp >> 2;
  // (selects, not a run-time index into the argument struct, which would
  // copy it to scratch)
  const float *src = level == 0 ? a.src0 : (level & 1) ? a.rbuf[1] : a.rbuf[0];
  const float4 *rs = reinterpret_cast<const float4 *>(src + row * a.dp);
  float4 r[NV];
  static_for<0, NV>([&](auto V_) {
    constexpr int v = decltype(V_)::value;
    const int i = lane + 64 * v;
    if (i < dp4) r[v] = rs[i];
  });

  // Lane j reads the records of half j & 1 of splits j/2, j/2 + 32, ...:
  // the smallest list key of the row ((key, index) order, over both halves),
  // then with its band, the candidates, the blocks whose second key is
  // inside the band, and overflow, as the fused kernel finds them from its
  // one list per half (the union of a half's split lists holds the blocks
  // its full list would).
  const int hh = lane & 1;
  float R1 = __builtin_inff();
  int I1 = kNoIndex, ovf = 0;
  // (a record is read at once, count and entries: the first rec_f4 float4,
  // which hold every entry a split of this many tiles can list (one per
  // 64-codeword block); the lane's first two records stay in registers for
  // the second pass, and a lane past the last split reads nothing)
  auto rec_at = [&](int sp2) { return a.part + ((row * splits + sp2) * 2 + hh) * kRecF4; };
  auto read_rec = [&](const float4 *rec, float4(&e)[kRecF4], bool have) {
#pragma unroll
    for (int j = 0; j < kRecF4; ++j)
      e[j] = (have && j < rec_f4) ? rec[j] : make_float4(0.f, 0.f, 0.f, 0.f);
  };
  float4 rc[2][kRecF4];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int sp2 = (lane >> 1) + 32 * q;
    read_rec(rec_at(sp2 < splits ? sp2 : 0), rc[q], sp2 < splits);
  }
  auto first_pass = [&](const float4(&e)[kRecF4]) {
    const int c = __float_as_int(e[0].x);
    ovf |= c > kList ? 1 : 0;
#pragma unroll
    for (int j = 0; j < kList; ++j) {
      const int i = block_index(e[1 + j].x, __float_as_int(e[1 + j].z));
      if (j < c && lex_lt(e[1 + j].x, i, R1, I1)) {
        R1 = e[1 + j].x;
        I1 = i;
      }
    }
  };
  first_pass(rc[0]);
  first_pass(rc[1]);
  for (int sp2 = (lane >> 1) + 64; sp2 < splits; sp2 += 32) {
    float4 e[kRecF4];
    read_rec(rec_at(sp2), e, true);
    first_pass(e);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float oR = __shfl_xor(R1, off, 64);
    const int oI = __shfl_xor(I1, off, 64);
    if (lex_lt(oR, oI, R1, I1)) {
      R1 = oR;
      I1 = oI;
    }
  }
  const int Im = (I1 >= 0 && I1 < a.K) ? I1 : 0;  // finite inputs always give a valid codeword
  // the nearest key's codeword, the winner unless another candidate turns
  // up: its load overlaps the second pass
  const float *cb_l = a.cb + (int64_t)level * a.K * a.dp;
  const float4 *pim = reinterpret_cast<const float4 *>(cb_l + (int64_t)Im * a.dp);
  float4 xim[NV];
  static_for<0, NV>([&](auto V_) {
    constexpr int v = decltype(V_)::value;
    const int i = lane + 64 * v;
    if (i < dp4) xim[v] = pim[i];
  });
  const float2 st = a.rstat[row];
  const float band = screen_band(st.x, st.y, a.lstat[4 * level], a.lstat[4 * level + 1], a.d);
  const float thr = __fadd_rn(R1, band);

  // candidates other than Im (any order; the winner does not depend on it)
  // and the failing blocks of each half
  if (lane == 0) ncand[wave] = 0;
  int nfail = 0, fblk = -1;
  auto second_pass = [&](const float4(&er)[kRecF4]) {
    const int c = __float_as_int(er[0].x);
    const int nl = c < kList ? c : kList;
    for (int j = 0; j < nl; ++j) {
      const float4 e = er[1 + j];
      const int base = __float_as_int(e.z);
      if (e.y <= thr) {
        ++nfail;
        fblk = base >> 6;
      } else if (e.x <= thr) {
        const int idx = block_index(e.x, base);
        if (idx != Im && idx >= 0 && idx < a.K) {
          const int pos = atomicAdd(&ncand[wave], 1);
          if (pos < kMaxCand) cand[wave][pos] = idx;
        }
      }
    }
  };
  second_pass(rc[0]);
  second_pass(rc[1]);
  for (int sp2 = (lane >> 1) + 64; sp2 < splits; sp2 += 32) {
    float4 er[kRecF4];
    read_rec(rec_at(sp2), er, true);
    second_pass(er);
  }
  // per half: failing blocks (counts add; any one of them), overflow
  int fb_any = fblk;
#pragma unroll
  for (int off = 2; off < 64; off <<= 1) {
    nfail += __shfl_xor(nfail, off, 64);
    ovf |= __shfl_xor(ovf, off, 64);
    const int o = __shfl_xor(fb_any, off, 64);
    fb_any = fb_any >= 0 ? fb_any : o;
  }
  const int onf = __shfl_xor(nfail, 1, 64);
  const int ofb = __shfl_xor(fb_any, 1, 64);
  ovf |= __shfl_xor(ovf, 1, 64);
  int rcode;
  if (ovf || nfail > 1 || onf > 1 || (nfail == 1 && onf == 1 && fb_any != ofb))
    rcode = kAuxScan;
  else
    rcode = nfail ? fb_any : (onf ? ofb : kAuxOk);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int nc = __builtin_amdgcn_readfirstlane(ncand[wave]);
  if (nc > kMaxCand) {
    nc = kMaxCand;
    rcode = kAuxScan;
  }
  // (as in the fused kernel: more than kMaxRescore candidates, counting the
  // rescored block's nearest, leave the level to the exact scan)
  if (nc + 1 + (rcode >= 0 ? 1 : 0) > kMaxRescore) rcode = kAuxScan;
  if (rcode >= 0) {
    // a block whose second key is inside the band: its nearest codeword
    // joins the candidates
    const float *rrow = src + row * a.dp;
    const int bi = rescore_block([&](int ks, int h, float(&v)[8]) {
      read8(rrow, 0, a.dp, ks * 16 + h * 8, true, v);
    }, a.dp >> 4, cb_l, a.dp, a.K, rcode, lane);
    if (lane == 0) cand[wave][nc] = bi < a.K ? bi : Im;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    ++nc;
  }

  // rescoring, two candidates at a time; tw keeps the winner's r - c.  A
  // lone candidate wins without a distance.
  int best = Im;
  float dbest = __builtin_inff();
  float4 tw[NV];
  static_for<0, NV>([&](auto V_) {
    constexpr int v = decltype(V_)::value;
    tw[v] = make_float4(r[v].x - xim[v].x, r[v].y - xim[v].y, r[v].z - xim[v].z,
                        r[v].w - xim[v].w);
  });
  for (int j = -1; nc > 0 && j < nc; j += 2) {
    const int ua = __builtin_amdgcn_readfirstlane(j < 0 ? Im : cand[wave][j]);
    const int ub = __builtin_amdgcn_readfirstlane(j + 1 < nc ? cand[wave][j + 1] : ua);
    const float4 *p1 = reinterpret_cast<const float4 *>(cb_l + (int64_t)ua * a.dp);
    const float4 *p2 = reinterpret_cast<const float4 *>(cb_l + (int64_t)ub * a.dp);
    float4 x1[NV], x2[NV];
    static_for<0, NV>([&](auto V_) {
      constexpr int v = decltype(V_)::value;
      const int i = lane + 64 * v;
      if (i < dp4) {
        x1[v] = j < 0 ? xim[v] : p1[i];
        x2[v] = p2[i];
      }
    });
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
      // lane 2c + h: candidate c, half h
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
    if (j < 0 || lex_lt(d1, ua, dbest, best)) {
      best = ua;
      dbest = d1;
      static_for<0, NV>([&](auto V_) { tw[decltype(V_)::value] = t1[decltype(V_)::value]; });
    }
    if (ub != ua && lex_lt(d2, ub, dbest, best)) {
      best = ub;
      dbest = d2;
      static_for<0, NV>([&](auto V_) { tw[decltype(V_)::value] = t2[decltype(V_)::value]; });
    }
    // the accumulating lanes are done with the area before it is rewritten
    __builtin_amdgcn_wave_barrier();
  }
  float *dst = level == a.L - 1 ? a.res_final : (level & 1) ? a.rbuf[0] : a.rbuf[1];
  if (dst != nullptr) {
    float4 *ds = reinterpret_cast<float4 *>(dst + row * a.dp);
    static_for<0, NV>([&](auto V_) {
      constexpr int v = decltype(V_)::value;
      const int i = lane + 64 * v;
      if (i < dp4) ds[i] = tw[v];
    });
  }
  if (level + 1 < a.L) {
    // bf16 fragment copy for the next level's sweep: the 4 features of a
    // float4 are half q of lane (h*32 + row%32)'s 16 bytes of k-step ks.
    // The same rounding gives the next level's band inputs: every lane puts
    // b = bf16(t) and u = t - b of its features into this wave's area.
    uint2 *fr = reinterpret_cast<uint2 *>(a.xfrag + (row >> 5) * (a.dp >> 4) * 64);
    const int rl = (int)(row & 31);
    static_for<0, NV>([&](auto V_) {
      constexpr int v = decltype(V_)::value;
      const int i = lane + 64 * v;
      if (i < dp4) {
        const float4 t = tw[v];
        const uint16_t q0 = f32_to_bf16_bits(t.x), q1 = f32_to_bf16_bits(t.y);
        const uint16_t q2 = f32_to_bf16_bits(t.z), q3 = f32_to_bf16_bits(t.w);
        const int ks = i >> 2, hq = i & 3;
        fr[((ks * 64 + (hq >> 1) * 32 + rl) << 1) + (hq & 1)] =
            make_uint2((uint32_t)q0 | ((uint32_t)q1 << 16), (uint32_t)q2 | ((uint32_t)q3 << 16));
        const float4 b4 = make_float4(bf16_bits_to_f32(q0), bf16_bits_to_f32(q1),
                                      bf16_bits_to_f32(q2), bf16_bits_to_f32(q3));
        area[wave][0][i] = b4;
        area[wave][1][i] = make_float4(t.x - b4.x, t.y - b4.y, t.z - b4.z, t.w - b4.w);
      }
    });
    // summed as the fused kernel sums them: over features ks*16 + h*8 + e of
    // half h, in order, with fmaf, then half 0 + half 1; lane 2q + h takes
    // sum b^2 (q = 0) or sum u^2 (q = 1) of half h, so one instruction
    // stream runs all four chains
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float acc = 0.f;
    if (lane < 4) {
      const float4 *tl = &area[wave][lane >> 1][(lane & 1) * 2];
      const int kend = a.dp >> 4;
#pragma unroll 4
      for (int ks = 0; ks < kend; ++ks) {
        const float4 ta = tl[ks * 4], tb = tl[ks * 4 + 1];
        const float tv[8] = {ta.x, ta.y, ta.z, ta.w, tb.x, tb.y, tb.z, tb.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(tv[e], tv[e], acc);
      }
    }
    const float rb0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 0));
    const float rb1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 1));
    const float dr0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 2));
    const float dr1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 3));
    if (lane == 0) a.rstat[row] = make_float2(rb0 + rb1, dr0 + dr1);
  }
  if (lane == 0) {
    a.ids[row * a.L + level] = best;
    a.aux[row * a.L + level] = rcode == kAuxScan ? kAuxScan : kAuxOk;
  }
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
    // a split's list has at most one entry per 64-codeword block it swept
    const int rec_f4 = 1 + (2 * p.tiles_per_split < kList ? 2 * p.tiles_per_split : kList);
    split_update_kernel<S><<<dim3((unsigned)ceil_div(a.n, 4)), dim3(NT), 0, s>>>(a, l, p.splits,
                                                                                rec_f4);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}


}  // namespace rvq
