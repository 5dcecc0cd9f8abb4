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
  int type;          // QMM_Q4_K or QMM_Q6_K
  int64_t od, id;    // logical shape
  int64_t od_pad;    // rows padded to kRowPad
  int64_t nsb;       // id / 256
  int64_t nchunk;    // id / 32
  int8_t* wq;        // folded int8 hi/lo planes, MFMA fragment order
  float* wd;         // d per (row, super-block)
  float* wm;         // -dmin*min per (row, chunk); q4_K only, else nullptr
};

constexpr int kRowPad = 128;     // weight rows are padded to a multiple of this
constexpr int kTokenPad = 128;   // tokens are padded to a multiple of this

// Byte sizes of the planes for a shape (all offsets 256-byte aligned).
size_t wq_bytes(int64_t od_pad, int64_t id);
size_t wd_bytes(int64_t od_pad, int64_t id);
size_t wm_bytes(int type, int64_t od_pad, int64_t id);

// Kernel launchers: return the hipGetLastError() after the launch.
hipError_t launch_repack(const uint8_t* raw, const Planes& p, hipStream_t s);
hipError_t launch_quantize(const float* x, int64_t n_tok, int64_t t_pad, int64_t id,
                           uint8_t* qact, hipStream_t s);
hipError_t launch_mmq(const Planes& p, const uint8_t* qact, int64_t n_tok, int64_t t_pad,
                      float* out, hipStream_t s);

}  // namespace qmm
