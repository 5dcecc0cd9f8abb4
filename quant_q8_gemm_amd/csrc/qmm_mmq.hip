// qmm_mmq.hip -- the q4_K / q6_K x q8 MMQ for gfx950 (MI355X).
//
// Method (engineering log "minfer / cuda_optimization_steps", pages r45, r56,
// r58): activations are quantized by a prepass into q8 blocks of 32 with a
// (d, scaled sum) pair; weights are expanded once at registration into planes
// that the GEMM streams without arithmetic; the GEMM forms exact integer dots
// per 32-block on int8 matrix cores and applies the per-block scales in f32.
//
// MI355X design (differs from the pages' GB10 kernels on purpose):
//  * the d*scale pair plane of r56 section 2.2 becomes integer arithmetic: the
//    block dot of a 32-block carries the small integer group scales exactly,
//    and only the f16 d (and q4_K's dmin) of the 256-weight super-block stays a
//    float, applied once per super-block.  q6_K (two 16-groups per 32-block,
//    int8 scales): the scale is multiplied into the codes at registration and
//    the folded weight split into two int8 planes (hi = w >> 6, lo = w & 63), so
//    one K=32 int8 MFMA per plane gives J = 64*J_hi + J_lo.  q4_K (one 6-bit
//    scale per 32-block): the 4-bit codes are int8 bytes, one K=32 MFMA gives
//    the code dot D, and the products sc(row)*dh(token) of the block's scale
//    and the activation scale come from one small f16 MFMA (an outer product of
//    exact f16 values, so every product is exact);
//  * q4_K's block dot leaves the matrix core already as an f32: the MFMA's
//    accumulator input is the inline constant 1/(2 pi), whose bit pattern
//    0x3E22F983 plus any |D| < 2^21 is the f32 value c0 + D*2^-26 (one binade,
//    spacing 2^-26), so D*2^-26 = that value - c0 exactly, one full-rate
//    subtraction where an integer-to-float conversion issues at half rate;
//  * planes are stored in MFMA fragment order, so every lane's operand is one
//    contiguous 16-byte load and a wave's load is one contiguous 1 KiB;
//  * the q4_K min term sum_c dmin*min_c*s_c is a small matrix product over
//    chunks: per super-block, one f16 MFMA (32x32x8) of the 6-bit mins and the
//    f16 scaled sums, times dmin.
#include "qmm_internal.h"
#include "qmm_common.h"

#include <algorithm>
#include <mutex>

#include "../../include/qmm.h"

namespace qmm {

// ---------------------------------------------------------------------------
// MMQ.  A work-group of KS x WR x WT waves owns a (32*WR rows) x (32*WT tokens)
// output tile, one 32 x 32 block per wave and k-group.  With KS = 2 the two
// k-groups take the first and the second half of the super-blocks, each with
// its own LDS stages, and their sums are added once at the end (k-group 0's
// plus k-group 1's, always in that order): twice the waves per tile for shapes
// with too few tiles to keep the CUs busy.  The inner dimension is walked in
// stages of KC chunks of 32 (KC = 2, 4 or 8: a quarter, half or whole 256-wide
// super-block).  Each stage's operands -- the weight fragments of the WR row
// blocks, the q8 codes and scale pairs of the WT token blocks, and q6_K's d or
// q4_K's stage records (scales, mins, d and dmin) of the row blocks -- are
// copied once per work-group into LDS with direct global->LDS loads
// (global_load_lds_dwordx4 puts lane l's 16 bytes at the LDS base + 16*l, so
// one wave instruction moves 1 KiB), and read from there by every wave that
// shares them.  Two LDS stages alternate: the loads of stage g+1 are issued
// during stage g, one job of a wave per chunk step; one barrier per stage.
// A small tile and a small LDS footprint let several work-groups share a CU, so
// one group's barrier wait is covered by the others' work.
// MFMA orientation: A = weights (rows j), B = activations (columns t), so each
// lane's 16 outputs share one token: q6_K's activation scale dh is one register
// per chunk and its super-block d is applied once per 8 chunks; q4_K's scale
// products come as a 32 x 32 block from the matrix core.
// ---------------------------------------------------------------------------
// Direct global->LDS copy of 16 bytes per lane (global_load_lds_dwordx4: lane
// l's bytes land at the LDS byte address held in M0 plus 16*l).  Written out so
// that a wave-uniform source is addressed as scalar base + the lane's offset;
// the builtin form lets the compiler turn the source into a per-lane 64-bit
// induction variable, a few vector instructions per copy (6-9% of the 512-token
// ffn_down MMQ).  M0 is set by each copy itself; the kernel issues no other
// instruction that reads M0.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
// N consecutive 1 KiB copies (N <= 4) from base + lane_off + 1024*i to the LDS
// bytes at lds + 1024*i: one M0 write, and the instruction offset, which the
// load adds to both its global and its LDS address, steps through the run.
template <int N>
__device__ __forceinline__ void copy16_run(const void* base, uint32_t lane_off, uint32_t lds) {
  static_assert(N >= 1 && N <= 4, "a run of 1 to 4 KiB (13-bit instruction offsets)");
  if constexpr (N == 1)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(lane_off), "s"(base), "s"(lds) : "memory");
  else if constexpr (N == 2)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1\n\t"
                 "global_load_lds_dwordx4 %0, %1 offset:1024"
                 :: "v"(lane_off), "s"(base), "s"(lds) : "memory");
  else if constexpr (N == 3)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1\n\t"
                 "global_load_lds_dwordx4 %0, %1 offset:1024\n\tglobal_load_lds_dwordx4 %0, %1 offset:2048"
                 :: "v"(lane_off), "s"(base), "s"(lds) : "memory");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1\n\t"
                 "global_load_lds_dwordx4 %0, %1 offset:1024\n\tglobal_load_lds_dwordx4 %0, %1 offset:2048\n\t"
                 "global_load_lds_dwordx4 %0, %1 offset:3072"
                 :: "v"(lane_off), "s"(base), "s"(lds) : "memory");
}

// Weight fragment bytes per (32-row block, chunk): q6_K hi and lo planes of
// 1 KiB each; q4_K codes (16 bytes per lane).
template <int TYPE>
constexpr int kFragA = TYPE == QMM_Q6_K ? 2048 : TYPE == QMM_Q4_K_PACKED ? kQ4PackedFrag : kQ4CodeFrag;

// q4_K's stage record of one 32-row block (the wsm plane's 1 KiB record): the
// stage's 4 scales and the super-block's 8 mins as f16 integers, d*2^25 and
// -dmin in f32.
struct Q4Rec {
  uint16_t sc[32][4];     // [row][chunk of the stage]
  uint16_t mn[2][32][4];  // [chunk/4][row][chunk%4] of the super-block
  float d[2][32];         // [d*2^25, -dmin][row]
};
static_assert(sizeof(Q4Rec) == kQ4RecBytes && __builtin_offsetof(Q4Rec, mn) == kQ4RecMnOff &&
                  __builtin_offsetof(Q4Rec, d) == kQ4RecDOff,
              "the record as the repack writes it");

template <int TYPE, int WR, int WT, int KC>
struct alignas(16) Stage {
  static constexpr bool kQ4 = is_q4k(TYPE);
  int8_t a[WR][KC][kFragA<TYPE>];    // weight fragments: [row block][chunk]
  int8_t b[WT][KC][1024];            // q8 codes: [token block][chunk][fragment]
  // The small region, copied in whole 1 KiB jobs of one kind each:
  uint32_t s[WT][KC][32];            // (dh, s) pairs: [token block][chunk][token]
  Q4Rec rec[kQ4 ? WR : 0];           // q4_K: the row blocks' stage records
  float d[kQ4 ? 0 : WR][32];         // q6_K: super-block d: [row block][row]
  // jobs: pairs (8/KC token blocks each), then q4_K one per record, or q6_K
  // one for the d of all row blocks (WR*8 lanes, with a super-block's last stage)
  static constexpr int kPairJobs = WT * KC * 128 / 1024;
  static constexpr int kSmallJobs = kPairJobs + (kQ4 ? WR : 1);
};

// The weight side of one chunk: the MFMA operand(s) read from a stage, the
// MFMA(s) against the activation fragment, and the scale-carrying block dot J
// of output element i.
template <int TYPE>
struct WeightOps;

template <>
struct WeightOps<QMM_Q6_K> {
  struct A { v4i hi, lo; };
  struct D { v16i hi, lo; };
  static constexpr int kMfma = 2;
  __device__ static A load(const int8_t* frag, int lane) {
    return {*(const v4i*)(frag + lane * 16), *(const v4i*)(frag + 1024 + lane * 16)};
  }
  __device__ static D mma(const A& a, v4i bq) {
    const v16i zero = {};
    return {__builtin_amdgcn_mfma_i32_32x32x32_i8(a.hi, bq, zero, 0, 0, 0),
            __builtin_amdgcn_mfma_i32_32x32x32_i8(a.lo, bq, zero, 0, 0, 0)};
  }
  __device__ static void keep(D& d) { pin(d.hi); pin(d.lo); }
  // the scale-folded block dot J of output element i, as an f32 (exact: |J| < 2^24)
  __device__ static float val(const D& d, int i) { return (float)((d.hi[i] << 6) + d.lo[i]); }
};

// q4_K block dots come out of the matrix core biased: the accumulator input is
// the bit pattern of the f32 value kQ4Bias (1/(2 pi), encoded as an inline
// constant of the instruction, so it costs no register), and since the code dot
// |D| <= 32*15*127 = 60960 is far inside the 2291075 steps below and 6097533
// above it that its binade [1/8, 1/4) holds, the f32 value of the result's bits
// is kQ4Bias + D*2^-26 exactly.  Subtracting kQ4Bias is exact (both within a
// factor of two), so val() = D*2^-26 with one full-rate subtraction, written
// as -(kQ4Bias - x): the subtraction then takes kQ4Bias as an inline constant
// (x - kQ4Bias would need -1/(2 pi), a 32-bit literal in every instruction),
// and the negation folds into the scale FMA's operand (it cannot be folded back
// into x - kQ4Bias: the two differ in the sign of a zero result).
// The compiler encodes the splat as the inline constant only for an MFMA whose
// accumulator input is used by no other instruction of its basic block; an
// empty asm goto after each such MFMA ends its block without emitting an
// instruction (an always-taken uniform branch did the same for two scalar
// instructions per MFMA).  Shared, the splat is materialized in 16 registers,
// which the kernel does not have.
constexpr uint32_t kQ4BiasBits = 0x3E22F983u;

template <>
struct WeightOps<QMM_Q4_K> {
  struct A { v4i c; };
  struct D { v16i c; };
  static constexpr int kMfma = 1;
  __device__ static A load(const int8_t* frag, int lane) { return {*(const v4i*)(frag + lane * 16)}; }
  __device__ static D mma(const A& a, v4i bq) {
    const v16i bias = (v16i)(int)kQ4BiasBits;
    D r;
    r.c = __builtin_amdgcn_mfma_i32_32x32x32_i8(a.c, bq, bias, 0, 0, 0);
    asm goto("" :::: block_end);
  block_end:
    return r;
  }
  __device__ static void keep(D& d) { pin(d.c); }
  // D*2^-26 of output element i; the 6-bit scale is not in it but in the scale
  // product that multiplies it (scale_outer below)
  // (the whole vector is reinterpreted: hipcc's __builtin_bit_cast of one
  // element of an ext-vector reads element 0 whatever the index)
  __device__ static float val(const D& d, int i) {
    const v16f f = __builtin_bit_cast(v16f, d.c);
    return -(__builtin_bit_cast(float, kQ4BiasBits) - f[i]);
  }
};

// q4_K with the codes kept two per byte: a lane's 8 bytes hold its 16 codes,
// code i in the low nibble of byte i and code i+8 in the high one (i < 8); two
// masks and two shifts unpack them into the 16 code bytes the MFMA takes.
// Everything after the load is q4_K's.
template <>
struct WeightOps<QMM_Q4_K_PACKED> : WeightOps<QMM_Q4_K> {
  __device__ static A load(const int8_t* frag, int lane) {
    const uint2 p = *(const uint2*)(frag + lane * 8);
    const v4i c = {(int)(p.x & 0x0F0F0F0Fu), (int)(p.y & 0x0F0F0F0Fu), (int)((p.x >> 4) & 0x0F0F0F0Fu),
                   (int)((p.y >> 4) & 0x0F0F0F0Fu)};
    return {c};
  }
};

// q4_K: the scale of output element (row j, token t) of chunk c is
// d(j)*sc(j, c) * dh(t, c); d is applied once per super-block, and the outer
// product sc(j, c)*dh(t, c) of a row vector and a token vector -- both exact f16
// values, a 6-bit integer and the f16 activation scale -- comes from one f16
// MFMA (32x32x8) in the same output layout as the int8 MFMA's block dots.  A
// holds the stage's 4 scales of the lane's row (the same 4 on both lane halves,
// k = 4*half + chunk), B the chunk's dh in slot cc of both halves and zeros
// elsewhere, so each product is formed twice and added: 2*sc*dh, exact.  That
// 2 and the block dot's 2^-26 are undone by the plane's d*2^25.
// cc is the chunk's index in the stage (a constant once the loops are unrolled).
//   a_sc      the lane's 4 f16 scales (row lane & 31, the stage's chunks)
//   dh_bits   the chunk's (dh, s) pair of the lane's token (lane & 31)
__device__ __forceinline__ v16f scale_outer(v2i a_sc, uint32_t dh_bits, int cc) {
  typedef _Float16 v4h __attribute__((ext_vector_type(4)));
  // dh into the low (cc even) or high (cc odd) half of the word, zero elsewhere
  const uint32_t y = __builtin_amdgcn_perm(0u, dh_bits, cc % 2 == 0 ? 0x0C0C0100u : 0x01000C0Cu);
  const v2i b = {cc < 2 ? (int)y : 0, cc < 2 ? 0 : (int)y};
  const v16f zero = {};
  return __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(v4h, a_sc), __builtin_bit_cast(v4h, b), zero,
                                              0, 0, 0);
}

// Work-group index -> (row tile, token tile).  Work-groups are dispatched
// round-robin over the 8 XCDs (each with its own 4 MiB L2), so first every XCD
// gets a contiguous run of positions; positions then walk the tiles in groups of
// kGroupRows row tiles, row tile fastest, so the work-groups resident on one XCD
// at a time (32 or 128) form a block of 8 row tiles x 4 to 16 token tiles that
// share both their weight rows and their activations in that L2.
constexpr int kGroupRows = 8;

__host__ __device__ __forceinline__ int xcd_swizzle(int i, int n) {
  const int q = n / 8, r = n % 8;
  const int x = i % 8, slot = i / 8;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + slot;
}

__host__ __device__ __forceinline__ void tile_of(int pos, int row_tiles, int tok_tiles, int& rt, int& tt) {
  const int per_group = kGroupRows * tok_tiles;
  const int g = pos / per_group, idx = pos % per_group;
  const int left = row_tiles - g * kGroupRows;
  const int rows_here = left < kGroupRows ? left : kGroupRows;  // last group may be short
  rt = g * kGroupRows + idx % rows_here;
  tt = idx / rows_here;
}

// What work-group wg computes: a whole tile of the data-parallel part (the
// first dp_row_tiles * tok_tiles work-groups, walked as above), or one K slice
// of a tail tile -- the tail's work-groups take its tiles in order, split
// consecutive slices each, slice sl holding super-blocks
// [sl*nsb/split, (sl+1)*nsb/split).  tail: the work-group's index among the
// tail's (its partial tile's slot in the scratch), negative for a whole tile.
struct Work {
  int rt, tt, sb0, sb1, tail;
};
__host__ __device__ __forceinline__ Work work_of(int wg, int dp_row_tiles, int tok_tiles, int split, int nsb) {
  Work w;
  const int dp_tiles = dp_row_tiles * tok_tiles;
  w.tail = wg - dp_tiles;
  if (w.tail < 0) {
    tile_of(xcd_swizzle(wg, dp_tiles), dp_row_tiles, tok_tiles, w.rt, w.tt);
    w.sb0 = 0;
    w.sb1 = nsb;
  } else {
    const int u = w.tail / split, sl = w.tail % split;
    w.rt = dp_row_tiles + u / tok_tiles;
    w.tt = u % tok_tiles;
    w.sb0 = sl * nsb / split;
    w.sb1 = (sl + 1) * nsb / split;
  }
  return w;
}

// Output layout of a wave's 32 x 32 block: lane holds token (lane & 31) and,
// in acc[4*q + i], row 4*(lane >> 5) + 8*q + i.  store_quad writes the four
// rows of one q into out[t][od], masked at od and n_tok.
__device__ __forceinline__ void store_quad(float* __restrict__ out, float4 v, int rblock, int tblock,
                                           int lane, int q, int od, int n_tok, int vec_store) {
  const int tok = tblock * 32 + (lane & 31);
  if (tok >= n_tok) return;
  float* orow = out + (size_t)tok * od;
  const int j = rblock * 32 + 4 * (lane >> 5) + 8 * q;
  if (vec_store && j + 3 < od) {
    *(float4*)(orow + j) = v;
  } else {
    if (j < od) orow[j] = v.x;
    if (j + 1 < od) orow[j + 1] = v.y;
    if (j + 2 < od) orow[j + 2] = v.z;
    if (j + 3 < od) orow[j + 3] = v.w;
  }
}

// Store one wave's 32 x 32 block through LDS: the lane's 16 values go to the
// wave's 32 x 33 float region in [row][token] order (33: the reads below hit 32
// different banks) and come back with lane l holding row l % 32 of tokens
// 2k + l / 32, so each store instruction writes two runs of 32 consecutive
// floats of out, at any od and alignment, where store_block's lanes write
// 16-byte pieces of 32 different token rows (or 4-byte ones when od % 4 != 0).
//   lds   the wave's 32 * 33 floats, free for it to use
__device__ __forceinline__ void store_block_lds(float* __restrict__ out, const v16f& acc, float* lds, int rblock,
                                                int tblock, int lane, int od, int n_tok) {
  const int t = lane & 31, rb = 4 * (lane >> 5);
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) lds[(rb + 8 * q + i) * 33 + t] = acc[4 * q + i];
  const int r = lane & 31, j = rblock * 32 + r;
  if (j >= od) return;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int tl = 2 * k + (lane >> 5);
    const int tok = tblock * 32 + tl;
    const float v = lds[r * 33 + tl];
    if (tok < n_tok) out[(size_t)tok * od + j] = v;
  }
}

__device__ __forceinline__ void store_block(float* __restrict__ out, const v16f& acc, int rblock, int tblock,
                                            int lane, int od, int n_tok, int vec_store) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    store_quad(out, make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]), rblock, tblock,
               lane, q, od, n_tok, vec_store);
}

// Ragged second wave ("tail").  When the tiles fill the resident work-group
// slots once and a few more, the first wave's worth of row tiles run whole
// (data-parallel) and each of the remaining tail tiles is split along K into
// S slices of super-blocks, so the tail runs S times wider.  A slice writes its partial
// tile, in the work-group's register order, to a scratch buffer; the fixup
// kernel adds a tile's S partials in slice order and stores the tile.  The
// tail is whole row tiles at the end, so the rows before it keep exactly the
// summation order they have without a tail.
// Every launch shape runs 16 waves per CU, 4 per SIMD: at most 128 VGPRs.
template <int TYPE, int WR, int WT, int KC, int KS>
__global__ void __launch_bounds__(64 * WR * WT * KS) __attribute__((amdgpu_waves_per_eu(4, 4)))
mmq_kernel(const int8_t* __restrict__ wq, const float* __restrict__ wd,
           const uint8_t* __restrict__ wsm, const uint8_t* __restrict__ qq,
           const uint8_t* __restrict__ qs, int nchunk, int nsb, int od, int n_tok,
           int tok_tiles, int dp_row_tiles, int split, int vec_store, float* __restrict__ out,
           float* __restrict__ part) {
  using St = Stage<TYPE, WR, WT, KC>;
  using W = WeightOps<TYPE>;
  constexpr int kWaves = WR * WT;
  constexpr int kJobsA = WR * KC * kFragA<TYPE> / 1024, kJobsB = WT * KC;
  static_assert(KC == 2 || KC == 4 || KC == 8, "a stage is a quarter, half or a whole super-block");
  static_assert(KS == 1 || KS == 2, "one or two k-groups");
  static_assert((WT * KC * 128) % 1024 == 0, "whole pair jobs");
  static_assert((St::kQ4 ? __builtin_offsetof(St, rec) : __builtin_offsetof(St, d)) ==
                        __builtin_offsetof(St, s) + 1024 * St::kPairJobs &&
                    sizeof(St) == __builtin_offsetof(St, s) + 1024 * St::kPairJobs +
                                      (St::kQ4 ? 1024 * WR : 128 * WR),
                "the small region's jobs are contiguous 1 KiB units and end the stage");
  // the q4_K min term collects a super-block's 8 chunks over two stages
  constexpr bool kQ4 = is_q4k(TYPE);
  static_assert(!kQ4 || KC == 4, "q4_K stages are half super-blocks");
  // k-group 1's sums pass to k-group 0 through k-group 0's two stages
  static_assert(KS == 1 || 2 * sizeof(St) >= (size_t)kWaves * 16 * 64 * 4, "room to combine k-groups");
  __shared__ St stage_all[KS][2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int ks = wave_all / kWaves;      // k-group
  const int wave = wave_all % kWaves;    // wave within the k-group
  const int wr = wave / WT, wt = wave % WT;
  St* stage = stage_all[ks];
  // role: a whole tile of the data-parallel part, or one K slice of a tail tile
  const Work work = work_of((int)blockIdx.x, dp_row_tiles, tok_tiles, split, nsb);
  const int tail_idx = work.tail;  // >= 0: index into the partials
  const int rt = work.rt, tt = work.tt, sb0 = work.sb0, sb1 = work.sb1;
  const int rb0 = rt * WR, tb0 = tt * WT;
  // k-group ks owns super-blocks [sb0 + ks*n/KS, sb0 + (ks+1)*n/KS) of the n in
  // this work-group's range; the last group has the most, so every wave runs its
  // group's stages inside that many iterations.
  constexpr int kStagesPerSb = 8 / KC;
  const int nsb_here = sb1 - sb0;
  const int gbeg = (sb0 + ks * nsb_here / KS) * kStagesPerSb;
  const int nstages = (sb0 + (ks + 1) * nsb_here / KS) * kStagesPerSb - gbeg;
  const int niter = (nsb_here - (KS - 1) * nsb_here / KS) * kStagesPerSb;

  // Copy jobs of one stage (one wave instruction, 1 KiB each): the weight
  // fragments, then the code fragments, split into equal contiguous runs per
  // wave (a run stays inside one row / token block, so its source is one
  // uniform base plus immediate 1 KiB steps; with fewer weight jobs than waves,
  // the first waves take one each); then the small region in whole 1 KiB jobs
  // of one kind each (activation scale pairs, q4_K stage records, q6_K d), one
  // for each of the first waves.
  constexpr int kFrag = kFragA<TYPE>;
  constexpr int kPerRbA = KC * kFrag / 1024;  // weight jobs per row block and stage
  static_assert(kJobsA % kWaves == 0 || kJobsA < kWaves, "equal weight runs per wave");
  static_assert(kJobsB % kWaves == 0 || kJobsB < kWaves, "equal code runs per wave");
  constexpr int kRunA = kJobsA >= kWaves ? kJobsA / kWaves : 1;
  constexpr int kRunB = kJobsB >= kWaves ? kJobsB / kWaves : 1;
  static_assert(kPerRbA % kRunA == 0 && KC % kRunB == 0, "a run stays inside one block");
  static_assert(St::kSmallJobs <= kWaves, "one small-region job per wave at most");
  const bool has_a = kJobsA >= kWaves || wave < kJobsA;
  const bool has_b = kJobsB >= kWaves || wave < kJobsB;
  const int ka0 = wave * kRunA, kb0 = wave * kRunB;
  // wave-uniform sources (see copy16_run)
  const int8_t* srcA = wq + (size_t)(rb0 + ka0 / kPerRbA) * nchunk * kFrag + (ka0 % kPerRbA) * 1024 +
                      (size_t)gbeg * KC * kFrag;
  const uint8_t* srcB = qq + (size_t)(tb0 + kb0 / KC) * nchunk * 1024 + (kb0 % KC) * 1024 +
                        (size_t)gbeg * KC * 1024;
  const uint32_t lane_off = (uint32_t)lane * 16;
  // This wave's small-region job (a wave-uniform kind: wave < kSmallJobs),
  // as a scalar source at the k-group's first stage plus a lane offset:
  //   pair job k: the pairs of token blocks tb0 + (8/KC)*k + lane/(8*KC),
  //     KC*128 bytes each per stage;
  //   q4_K record job r: row block rb0 + r's stage records, 1 KiB per stage;
  //   q6_K d job: lanes 0..8*WR-1, row block rb0 + lane/8's d, 128 bytes per
  //     super-block.
  constexpr int kTokPerJob = 8 / KC;
  const bool pair_job = wave < St::kPairJobs;
  const uint8_t* small_src;
  uint32_t small_off;
  if (pair_job) {
    small_src = qs + ((size_t)(tb0 + wave * kTokPerJob) * nchunk + gbeg * KC) * 128;
    small_off = (uint32_t)(lane / (8 * KC)) * (uint32_t)nchunk * 128 + (uint32_t)(lane % (8 * KC)) * 16;
  } else if constexpr (kQ4) {
    small_src = wsm + ((size_t)(rb0 + wave - St::kPairJobs) * (nchunk / 4) + gbeg) * kQ4RecBytes;
    small_off = lane_off;
  } else {
    small_src = (const uint8_t*)wd + ((size_t)rb0 * nsb + gbeg / kStagesPerSb) * 128;
    small_off = (uint32_t)(lane / 8) * (uint32_t)nsb * 128 + (uint32_t)(lane % 8) * 16;
  }

  // This wave's copy jobs for one stage, numbered: its weight run, its code run,
  // its small-region job.  The jobs of stage g+1 are spread over the chunk steps
  // of stage g (one per step) rather than issued in one burst, so the copies'
  // LDS writes interleave with the steps' LDS reads instead of stalling them.
  // Every job is a run of whole-wave 1 KiB copies from a wave-uniform scalar
  // source plus a lane offset: the kind of job is uniform per wave and whether
  // it runs in a stage is known at compile time, so a copy costs no vector
  // instruction and no divergent branch (q6_K's d job masks its lanes past
  // 8*WR).
  constexpr int kWaveJobs = 3;
  const uint8_t* const srcA_u = (const uint8_t*)uniform_ptr(srcA);
  const uint8_t* const srcB_u = (const uint8_t*)uniform_ptr(srcB);
  const uint8_t* const small_u = (const uint8_t*)uniform_ptr(small_src);
  const uint32_t lds_k = __builtin_amdgcn_readfirstlane(lds_addr(stage));
  //   ends_sb  stage g is the last of its super-block (q6_K's d comes with it)
  auto issue_job = [&](int g, int buf, int j, bool ends_sb) __attribute__((always_inline)) {
    const uint32_t lds_buf = lds_k + (uint32_t)buf * (uint32_t)sizeof(St);
    if (j == 0) {
      if (has_a)
        copy16_run<kRunA>(srcA_u + (size_t)g * KC * kFrag, lane_off,
                          lds_buf + (uint32_t)__builtin_offsetof(St, a) + ka0 * 1024);
    } else if (j == 1) {
      if (has_b)
        copy16_run<kRunB>(srcB_u + (size_t)g * KC * 1024, lane_off,
                          lds_buf + (uint32_t)__builtin_offsetof(St, b) + kb0 * 1024);
    } else if (wave < St::kSmallJobs) {
      const uint32_t ls = lds_buf + (uint32_t)__builtin_offsetof(St, s) + wave * 1024;
      if (pair_job)
        copy16_run<1>(small_u + (size_t)g * KC * 128, small_off, ls);
      else if constexpr (kQ4)
        copy16_run<1>(small_u + (size_t)g * kQ4RecBytes, small_off, ls);
      else if (ends_sb && lane < 8 * WR)
        copy16_run<1>(small_u + (size_t)((g * KC) / 8) * 128, small_off, ls);
    }
  };
  auto issue_stage = [&](int g, int buf, bool ends_sb) __attribute__((always_inline)) {  // all at once
#pragma unroll
    for (int j = 0; j < kWaveJobs; ++j) issue_job(g, buf, j, ends_sb);
  };

  v16f acc, inner;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
  // q4_K min term of a super-block, sum over its chunks c of
  // min(row, c) * s(token, c), on one f16 MFMA (32x32x8) at its end (products
  // of a 6-bit integer and an f16 value: exact in f32), then times -dmin into
  // acc.  Lane half hh supplies chunks 4*hh..4*hh+3: the mins from the
  // super-block's last stage record (which holds all 8), the scaled sums (bs)
  // collected from the chunks' scale pairs as they pass, half hh of the lanes
  // during the super-block's stage hh.
  v2i bs = {};
  const bool lane_hi = lane >= 32;

  if (nstages > 0) issue_stage(0, 0, kStagesPerSb == 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // Super-blocks in turn, the stages of one unrolled, so where a super-block
  // starts and ends (first chunk: inner = dot * scale; last: apply d, and
  // q4_K's min term) is known at compile time.
  for (int sbi = 0; sbi < niter / kStagesPerSb; ++sbi) {
#pragma unroll
    for (int h = 0; h < kStagesPerSb; ++h) {
      const int g = sbi * kStagesPerSb + h;
      if (g < nstages) {  // uniform per k-group
        St& st = stage[g & 1];
        const bool starts_sb = h == 0;
        // Software pipeline over the KC chunks: step cc issues the MFMA(s) of
        // chunk cc+1 (operands read one step earlier), then the LDS reads of chunk
        // cc+2 and of chunk cc+1's activation scale, then the scale epilogue of
        // chunk cc on the vector ALU while the matrix core works.  Every LDS
        // value is consumed one step after its read, so a wait for it never
        // waits for the reads just issued.
        uint32_t dhr = st.s[wt][0][lane & 31], dhr_even = 0;
        v2i a_sc = {}, amin = {};
        if constexpr (kQ4) {
          if (h == kStagesPerSb - 1) amin = *(const v2i*)(&st.rec[wr].mn[lane >> 5][lane & 31][0]);
          a_sc = *(const v2i*)(&st.rec[wr].sc[lane & 31][0]);
        }
        typename W::A a0 = W::load(st.a[wr][0], lane);
        v4i bq0 = *(const v4i*)(st.b[wt][0] + lane * 16);
        typename W::A a1 = W::load(st.a[wr][1], lane);
        v4i bq1 = *(const v4i*)(st.b[wt][1] + lane * 16);
        typename W::D dj = W::mma(a0, bq0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int cc = 0; cc < KC; ++cc) {
          // the per-element scale of chunk cc.  q4_K: the scale products, first,
          // so they are ready for this step's epilogue; q6_K: dh, converted to
          // f32 once per chunk and kept in a register, so the 16 scale FMAs are
          // plain v_fma_f32, which issue at twice the rate of the mixed-precision
          // v_fma_mix_f32 the compiler would otherwise fold the f16 operand into
          v16f sd;
          float dh = 0.0f;
          if constexpr (kQ4) {
            sd = scale_outer(a_sc, dhr, cc);
            pin(sd);
          }
          typename W::D dj_next;
          if (cc + 1 < KC) {
            dj_next = W::mma(a1, bq1);
            W::keep(dj_next);
          }
          // stage (g+1)&1 was last read in iteration g-1, which every wave finished
          // before the barrier that ended it
          if (g + 1 < nstages) {
            constexpr int per = (kWaveJobs + KC - 1) / KC;
            const bool next_ends_sb = (h + 1) % kStagesPerSb == kStagesPerSb - 1;
#pragma unroll
            for (int q = 0; q < per; ++q)
              if (cc * per + q < kWaveJobs) issue_job(g + 1, (g + 1) & 1, cc * per + q, next_ends_sb);
          }
          typename W::A a2;
          v4i bq2;
          if (cc + 2 < KC) {
            a2 = W::load(st.a[wr][cc + 2], lane);
            bq2 = *(const v4i*)(st.b[wt][cc + 2] + lane * 16);
          }
          uint32_t dhr_next = 0;
          if (cc + 1 < KC) dhr_next = st.s[wt][cc + 1][lane & 31];
          if constexpr (kQ4) {
            if (cc & 1) {  // the scaled sums of chunks cc-1 and cc as an f16 pair
              const int sp = (int)__builtin_amdgcn_perm(dhr, dhr_even, 0x07060302u);
              if (lane_hi == (h == 1)) bs[cc >> 1] = sp;
            } else {
              dhr_even = dhr;
            }
          } else {
            dh = f16_bits_to_float(dhr & 0xFFFF);
            pin(dh);
          }
          // element i's scale: q4_K the outer product's, q6_K the token's dh
          auto scale = [&](int i) __attribute__((always_inline)) {
            if constexpr (kQ4) return sd[i];
            else return dh;
          };
          if (cc == 0 && starts_sb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) inner[i] = W::val(dj, i) * scale(i);
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) inner[i] = fmaf(W::val(dj, i), scale(i), inner[i]);
          }
          pin(inner);
          if (cc + 1 < KC) {
            dj = dj_next;
            a1 = a2;
            bq1 = bq2;
            dhr = dhr_next;
          }
          // order inside the step: MFMAs, stage copies, LDS reads, the vector epilogue
          // MFMA: q4_K's scale products of this chunk, then the next chunk's block dots
          __builtin_amdgcn_sched_group_barrier(0x008, W::kMfma + kQ4, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);         // VMEM (stage copies)
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);         // DS reads
          __builtin_amdgcn_sched_group_barrier(0x002, 72, 0);        // VALU
          __builtin_amdgcn_sched_barrier(0);
        }
        if (h == kStagesPerSb - 1) {  // end of a super-block: apply its d (q4_K: d*2^25)
          v16f mt;
          if constexpr (kQ4) {  // and q4_K's min term, times -dmin
            typedef _Float16 v4h __attribute__((ext_vector_type(4)));
            const v16f zero = {};
            mt = __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(v4h, amin), __builtin_bit_cast(v4h, bs),
                                                      zero, 0, 0, 0);
          }
          const float* dw;  // the row block's d (q4_K: d*2^25), then q4_K's -dmin
          if constexpr (kQ4) dw = st.rec[wr].d[0];
          else dw = st.d[wr];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 d4 = *(const float4*)(&dw[8 * q + 4 * (lane >> 5)]);
            acc[4 * q + 0] = fmaf(inner[4 * q + 0], d4.x, acc[4 * q + 0]);
            acc[4 * q + 1] = fmaf(inner[4 * q + 1], d4.y, acc[4 * q + 1]);
            acc[4 * q + 2] = fmaf(inner[4 * q + 2], d4.z, acc[4 * q + 2]);
            acc[4 * q + 3] = fmaf(inner[4 * q + 3], d4.w, acc[4 * q + 3]);
          }
          if constexpr (kQ4) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float4 m4 = *(const float4*)(&dw[32 + 8 * q + 4 * (lane >> 5)]);
              acc[4 * q + 0] = fmaf(mt[4 * q + 0], m4.x, acc[4 * q + 0]);
              acc[4 * q + 1] = fmaf(mt[4 * q + 1], m4.y, acc[4 * q + 1]);
              acc[4 * q + 2] = fmaf(mt[4 * q + 2], m4.z, acc[4 * q + 2]);
              acc[4 * q + 3] = fmaf(mt[4 * q + 3], m4.w, acc[4 * q + 3]);
            }
          }
        }
      }
      if (g + 1 < niter) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads for g+1 landed
        __syncthreads();                                   // everyone's landed; stage g is free
      }
    }
  }
  if (KS > 1) {  // add k-group 1's partial sums to k-group 0's, in that order
    __syncthreads();  // every wave is done with the stage buffers
    float* red = (float*)&stage_all[0][0] + wave * 1024 + lane;
    if (ks == 1) {
#pragma unroll
      for (int i = 0; i < 16; ++i) red[i * 64] = acc[i];
    }
    __syncthreads();
    if (ks == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] += red[i * 64];
    }
  }

  if (tail_idx < 0 && !vec_store) {
    // Without 16-byte stores (od % 4 != 0), through LDS: after the k-group
    // combine's region (kWaves x 4 KiB), or with one k-group once every wave
    // is done with the stage buffers.  od 4097 x 11008 at 509 tokens: 4-5%
    // faster.  With 16-byte stores it measured within 1% either way, and with
    // one k-group its barrier cost ~1% (q4_K 11008 x 4096, 3314 tokens), so
    // those stay direct.
    constexpr size_t kRed = KS > 1 ? (size_t)kWaves * 1024 : 0;
    static_assert((kRed + (size_t)kWaves * 32 * 33) * sizeof(float) <= KS * 2 * sizeof(St),
                  "room for the transposes after the combine's region");
    if (KS == 1) __syncthreads();
    if (ks != 0) return;
    store_block_lds(out, acc, (float*)stage_all + kRed + wave * 32 * 33, rb0 + wr, tb0 + wt, lane, od, n_tok);
    return;
  }
  if (ks != 0) return;
  if (tail_idx < 0) {
    store_block(out, acc, rb0 + wr, tb0 + wt, lane, od, n_tok, vec_store);
  } else {
    float* dst = part + ((size_t)tail_idx * kWaves + wave) * 1024 + lane;
#pragma unroll
    for (int i = 0; i < 16; ++i) dst[i * 64] = acc[i];
  }
}

// Adds each tail tile's `split` partials in slice order and stores the tile.
// One work-group per (tail tile, 32 x 32 block); thread (q, lane) sums the four
// values acc[4*q .. 4*q+3] of that lane over the slices.  The loads of up to
// kFixBatch slices are issued before their adds, so a tile split many ways (21
// slices for 4097 rows) waits for memory once per batch rather than once per
// slice; the adds keep slice order.
constexpr int kFixBatch = 8;

template <int WR, int WT>
__global__ void __launch_bounds__(256)
mmq_fixup_kernel(const float* __restrict__ part, int split, int dp_row_tiles, int tok_tiles, int od,
                 int n_tok, int vec_store, float* __restrict__ out) {
  constexpr int kWaves = WR * WT;
  constexpr size_t kSlice = (size_t)kWaves * 1024;  // floats per slice of one tile
  const int u = blockIdx.x / kWaves, w = blockIdx.x % kWaves;
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const float* src = part + ((size_t)u * split * kWaves + w) * 1024 + (4 * q) * 64 + lane;
  float4 v;
  for (int sl = 0; sl < split; sl += kFixBatch) {
    // a short last batch loads and adds only the slices that exist
    float4 t[kFixBatch];
#pragma unroll
    for (int b = 0; b < kFixBatch; ++b) {
      if (sl + b < split) {
        const float* p = src + (size_t)(sl + b) * kSlice;
        t[b] = make_float4(p[0], p[64], p[128], p[192]);
      }
    }
    if (sl == 0) v = t[0];
#pragma unroll
    for (int b = 0; b < kFixBatch; ++b) {
      if ((sl > 0 || b > 0) && sl + b < split) {
        v.x += t[b].x;
        v.y += t[b].y;
        v.z += t[b].z;
        v.w += t[b].w;
      }
    }
  }
  const int rt = dp_row_tiles + u / tok_tiles, tt = u % tok_tiles;
  store_quad(out, v, rt * WR + w / WT, tt * WT + w % WT, lane, q, od, n_tok, vec_store);
}

template <int TYPE, int WR, int WT, int KC, int KS>
static hipError_t launch_tiled(const Planes& p, const MmqPlan& plan, const uint8_t* qact, int64_t n_tok,
                               int64_t t_pad, float* out, float* part, hipStream_t s) {
  static_assert(kRowPad % (32 * WR) == 0 && kTokenPad % (32 * WT) == 0,
                "tiles must divide the row and token padding");
  const uint8_t* qs = qact + (size_t)t_pad * (size_t)p.id;
  const int vec_store = (p.od % 4 == 0) && ((uintptr_t)out % 16 == 0);
  const int64_t wgs = plan.work_groups;
  mmq_kernel<TYPE, WR, WT, KC, KS><<<dim3((unsigned)wgs), dim3(64 * WR * WT * KS), 0, s>>>(
      p.wq, p.wd, p.wsm, qact, qs, (int)p.nchunk, (int)p.nsb, (int)p.od, (int)n_tok, plan.tok_tiles,
      plan.dp_row_tiles, plan.split, vec_store, out, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.n_tail == 0) return e;
  mmq_fixup_kernel<WR, WT><<<dim3((unsigned)(plan.n_tail * WR * WT)), dim3(256), 0, s>>>(
      part, plan.split, plan.dp_row_tiles, plan.tok_tiles, (int)p.od, (int)n_tok, vec_store, out);
  return hipGetLastError();
}

// Tile geometry per launch (16 waves per CU in every shape):
//  * many tiles (at least four 64 x 64 tiles per CU, e.g. the 3314-token layer,
//    the 2048-token head): several work-groups per CU, so one group's barrier
//    wait is covered by the others.  q4_K: 2 x 2 waves (64 x 64 tiles), four
//    per CU, half-super-block stages (38 KiB of LDS, 114 VGPRs; packed codes
//    30 KiB, 112).  q6_K: 2 x 4 waves (64 rows x 128 tokens), two per CU,
//    half-super-block stages (68.5 KiB, 120 VGPRs): each weight fragment a
//    work-group copies serves four waves
//    instead of two, a third fewer copied bytes per output block, which is
//    what q6_K's 2-byte weights are short of (3-8% faster than 2 x 2 waves with
//    quarter stages; 4 x 4 and 4 x 2 waves were slower, and the 2 x 4 shape
//    was 4-9% slower for q4_K, whose copies are a quarter the size);
//  * few tiles (e.g. 512 tokens x 4096 rows = 256 64 x 128 tiles): 2 x 4 waves
//    (64 rows x 128 tokens) in two k-groups, half-super-block stages, 137 KiB
//    (q6_K), 112 KiB (q4_K) or 96 KiB (packed q4_K) of LDS, one work-group per
//    CU; the second k-group doubles the waves per CU.
// In all, a ragged second wave (tiles = slots + r with r <= slots / 2, the
// slots being the work-groups resident at once; e.g. 4097 rows x 512 tokens:
// 264 tiles on 256 CUs, 11008 rows x 512 tokens: 1376 tiles on 1024 slots) is
// split along K, and so is, with one or two work-groups per CU, a last wave of
// at most a quarter of the slots behind several full ones (the q6_K GEMMs of a
// layer at 3314 tokens).
// The switch point (about four 64 x 64 tiles per CU) was chosen by timing both
// on the 512-token shapes, the 3314-token layer shapes and the 2048-token head.
namespace {
// One launch shape: WR x WT waves per k-group, KS k-groups, stages of KC chunks,
// per_cu work-groups resident per CU (16 waves per CU in every shape).
struct Geometry {
  int wr, wt, ks, kc, per_cu;
};
constexpr Geometry kQ6Many{2, 4, 1, 4, 2};
constexpr Geometry kQ4Many{2, 2, 1, 4, 4};
constexpr Geometry kFew{2, 4, 2, 4, 1};
// a tail slice's partial tile fits the scratch's 64 KiB per CU in every shape
constexpr bool scratch_fits(const Geometry& g) {
  return g.per_cu * (32 * g.wr) * (32 * g.wt) * 4 <= 64 * 1024;
}
static_assert(scratch_fits(kQ6Many) && scratch_fits(kQ4Many) && scratch_fits(kFew), "scratch per CU");
constexpr bool sixteen_waves(const Geometry& g) { return g.per_cu * g.wr * g.wt * g.ks == 16; }
static_assert(sixteen_waves(kQ6Many) && sixteen_waves(kQ4Many) && sixteen_waves(kFew), "16 waves per CU");
Geometry geometry(int type, bool many) {
  return !many ? kFew : type == QMM_Q6_K ? kQ6Many : kQ4Many;
}
}  // namespace

MmqPlan plan_mmq(const Planes& p, int64_t n_tok, int num_cus) {
  MmqPlan plan{};
  const int64_t small_tiles = (p.od_pad / 64) * ((n_tok + 63) / 64);
  plan.many = small_tiles >= 4 * 256;
  const Geometry g = geometry(p.type, plan.many);
  // row tiles that hold at least one real row: the planes are padded to
  // kRowPad rows, but a tile of padding only would compute zeros
  plan.row_tiles = (int)((p.od + 32 * g.wr - 1) / (32 * g.wr));
  plan.tok_tiles = (int)((n_tok + 32 * g.wt - 1) / (32 * g.wt));
  plan.dp_row_tiles = plan.row_tiles;
  plan.split = 1;
  const int64_t tiles = (int64_t)plan.row_tiles * plan.tok_tiles;
  // work-groups resident at once
  const int64_t slots = (int64_t)num_cus * g.per_cu;
  // After at most one full wave; behind several, only for a tail of at most a
  // quarter of the slots with one or two work-groups per CU: there half the
  // CUs or more would idle through the last wave (q6_K 4096 x 11008 at 3314
  // tokens: 1664 tiles on 512 slots, 2.2% faster split).  Behind several waves with
  // four work-groups per CU (e.g. 3328 tiles on 1024 slots) the tail's
  // work-groups already overlap the last full wave's end, and the split
  // measured 0.5-1% slower there instead of 9% faster.  With no full wave (at
  // most half the slots filled, e.g. one GPU's 512-row share of a layer),
  // every tile is a tail tile.
  const int64_t last = num_cus > 0 ? tiles % slots : 0;  // tiles of a partial last wave
  const bool short_tail = tiles > 2 * slots && last > 0 && last * 4 <= slots && g.per_cu <= 2;
  if (num_cus > 0 && tiles != slots && (tiles < 2 * slots || short_tail)) {
    // the full wave stays data-parallel (whole row tiles), the row tiles after
    // it form the tail
    const int dp_rows = (int)((tiles / slots) * slots / plan.tok_tiles);
    const int n_tail = (plan.row_tiles - dp_rows) * plan.tok_tiles;  // > 0: tiles is no multiple of slots
    // at least one super-block per k-group in every slice: a k-group without
    // one would only wait
    const int split = n_tail > 0 ? (int)std::min<int64_t>(slots / n_tail, p.nsb / g.ks) : 1;
    if (split >= 2) {
      plan.dp_row_tiles = dp_rows;
      plan.n_tail = n_tail;
      plan.split = split;
      plan.scratch_bytes = (size_t)n_tail * split * (32 * g.wr) * (32 * g.wt) * sizeof(float);
    }
  }
  plan.work_groups = (int64_t)plan.dp_row_tiles * plan.tok_tiles + (int64_t)plan.n_tail * plan.split;
  plan.threads = 64 * g.wr * g.wt * g.ks;
  plan.tile_rows = 32 * g.wr;
  plan.tile_tokens = 32 * g.wt;
  plan.k_groups = g.ks;
  plan.per_cu = g.per_cu;
  return plan;
}

void plan_work(const MmqPlan& plan, int nsb, int64_t wg, int* rt, int* tt, int* sb0, int* sb1) {
  const Work w = work_of((int)wg, plan.dp_row_tiles, plan.tok_tiles, plan.split, nsb);
  *rt = w.rt;
  *tt = w.tt;
  *sb0 = w.sb0;
  *sb1 = w.sb1;
}

// n_tail * split work-groups, at most one per slot, each with one partial tile:
// at most 64 KiB per CU in every shape (scratch_fits).
size_t mmq_scratch_max_bytes(int num_cus) { return (size_t)num_cus * 64 * 1024; }

hipError_t launch_mmq(const Planes& p, const MmqPlan& plan, const uint8_t* qact, int64_t n_tok,
                      int64_t t_pad, float* out, float* part, hipStream_t s) {
  constexpr Geometry q6 = kQ6Many, q4 = kQ4Many, f = kFew;
  if (p.type == QMM_Q6_K)
    return plan.many ? launch_tiled<QMM_Q6_K, q6.wr, q6.wt, q6.kc, q6.ks>(p, plan, qact, n_tok, t_pad, out, part, s)
                     : launch_tiled<QMM_Q6_K, f.wr, f.wt, f.kc, f.ks>(p, plan, qact, n_tok, t_pad, out, part, s);
  if (p.type == QMM_Q4_K_PACKED)
    return plan.many ? launch_tiled<QMM_Q4_K_PACKED, q4.wr, q4.wt, q4.kc, q4.ks>(p, plan, qact, n_tok, t_pad, out,
                                                                               part, s)
                     : launch_tiled<QMM_Q4_K_PACKED, f.wr, f.wt, f.kc, f.ks>(p, plan, qact, n_tok, t_pad, out,
                                                                           part, s);
  return plan.many ? launch_tiled<QMM_Q4_K, q4.wr, q4.wt, q4.kc, q4.ks>(p, plan, qact, n_tok, t_pad, out, part, s)
                   : launch_tiled<QMM_Q4_K, f.wr, f.wt, f.kc, f.ks>(p, plan, qact, n_tok, t_pad, out, part, s);
}

// The tail partials of the allocation-free entry point (qmm_mmq_noalloc): one
// array per GPU, in the code object's zero-initialized device memory, so no
// call allocates.  Host code never passes the array's name to a kernel (there it
// is a host-side stand-in); it passes the device address hipGetSymbolAddress
// gives for the current device, looked up once per device.
static __device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];

hipError_t static_scratch(int device, float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[device] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[device] = (float*)p;
  }
  *ptr = addr[device];
  return hipSuccess;
}

}  // namespace qmm
