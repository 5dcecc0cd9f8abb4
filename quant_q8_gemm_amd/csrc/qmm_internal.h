// qmm_internal.h -- declarations shared by the library's host code and its HIP
// kernels (never installed, never seen by callers).
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace qmm {

// Device planes of one registered weight matrix (layout documented in
// qmm_repack.hip next to the repack kernel).
struct Planes {
  int type;          // QMM_Q4_K, QMM_Q4_K_PACKED or QMM_Q6_K
  int64_t od, id;    // logical shape
  int64_t od_pad;    // rows padded to kRowPad
  int64_t nsb;       // id / 256
  int64_t nchunk;    // id / 32
  int8_t* wq;        // weight fragments in MFMA order: q6_K folded hi/lo, q4_K codes
  float* wd;         // q6_K: d per (row, super-block); else nullptr
  uint8_t* wsm;      // q4_K: one 1 KiB record per (32-row block, 4-chunk stage) of the
                     // stage's scales and its super-block's mins, d*2^25 and -dmin; else nullptr
};

constexpr int kRowPad = 128;     // weight rows are padded to a multiple of this
constexpr int kTokenPad = 128;   // tokens are padded to a multiple of this
constexpr int kQ4CodeFrag = 1024; // q4_K code bytes per (32-row block, chunk): one code per byte
constexpr int kQ4PackedFrag = 512; // the same, packed: two codes per byte

// Both q4_K registrations share every plane but the codes'.
constexpr bool is_q4k(int type) { return type == 4 || type == 14; }  // QMM_Q4_K, QMM_Q4_K_PACKED

// q4_K's per-stage record: the 4 scales of each of the 32 rows (f16 integers,
// [row][chunk]), the 8 mins of the stage's super-block ([chunk/4][row][chunk%4],
// f16 integers) and its d*2^25 and -dmin ([part][row], f32) -- 1 KiB, one wave's
// direct-to-LDS copy.  Both stages of a super-block carry its mins and d.
constexpr int kQ4RecScOff = 0, kQ4RecMnOff = 256, kQ4RecDOff = 768, kQ4RecBytes = 1024;

// Byte sizes of the planes for a shape (all offsets 256-byte aligned).
size_t wq_bytes(int type, int64_t od_pad, int64_t id);
size_t wd_bytes(int type, int64_t od_pad, int64_t id);
size_t wsm_bytes(int type, int64_t od_pad, int64_t id);

// Kernel launchers: return the hipGetLastError() after the launch.
hipError_t launch_repack(const uint8_t* raw, const Planes& p, hipStream_t s);
hipError_t launch_quantize(const float* x, int64_t n_tok, int64_t t_pad, int64_t id,
                           uint8_t* qact, hipStream_t s);
// MMQ launch plan: tile geometry, and for a ragged last wave the K split of the
// tail tiles and the scratch they need (n_tail tiles x split partials).
struct MmqPlan {
  bool many;          // many tiles: the many-tile shapes, else 64 x 128 tiles in two k-groups
  int tile_rows, tile_tokens;  // output rows and tokens per tile
  int k_groups;       // wave groups per work-group, each over its share of a tile's super-blocks
  int per_cu;         // work-groups resident per compute unit
  int row_tiles, tok_tiles;
  int dp_row_tiles;   // row tiles computed whole
  int n_tail;         // tiles after them, each split along K
  int split;          // K slices per tail tile (1: no tail)
  size_t scratch_bytes;
  int64_t work_groups;  // of the MMQ launch (one-dimensional grid)
  int threads;          // per work-group
};
MmqPlan plan_mmq(const Planes& p, int64_t n_tok, int num_cus);
// What work-group wg (0 <= wg < plan.work_groups) of the plan's MMQ launch
// computes, by the kernel's own mapping: tile (rt, tt) over super-blocks
// [sb0, sb1) of nsb.
void plan_work(const MmqPlan& plan, int nsb, int64_t wg, int* rt, int* tt, int* sb0, int* sb1);
// Upper bound of MmqPlan::scratch_bytes on a device with num_cus compute units.
size_t mmq_scratch_max_bytes(int num_cus);
hipError_t launch_mmq(const Planes& p, const MmqPlan& plan, const uint8_t* qact, int64_t n_tok,
                      int64_t t_pad, float* out, float* part, hipStream_t s);
// The allocation-free entry point's tail scratch: a static device array of
// this many bytes per GPU (64 KiB per compute unit of a 256-CU MI355X).
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
// Its device address on `device`, which must be the current device; looked up
// on the first call for that device, without allocating.
hipError_t static_scratch(int device, float** ptr);

}  // namespace qmm
