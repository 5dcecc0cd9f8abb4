// qmm_repack.hip -- registration-time repack of q6_K / q4_K blocks into the
// planes the MMQ streams (the once-per-weight expansion of the r56 and r58
// pages of the engineering log "minfer / cuda_optimization_steps": r56 sections
// 2.2-2.3, r58 section 3.2).  Instead of the pages' f32 d*scale pair plane the
// small integer group scales stay integers: q6_K's int8 scale of every 16
// weights is multiplied into the codes (exact) and the folded weight split into
// two int8 planes (hi = w >> 6, lo = w & 63), so one K=32 int8 MFMA per plane
// yields the block dot J = 64*J_hi + J_lo, and only the f16 d of the super-block
// stays a float.  q4_K's 4-bit codes become int8 bytes in MFMA fragment order;
// its 6-bit scales and mins become f16 integers (exact), the operands from which
// the GEMM's f16 matrix-core products form scale*dh and the min term; its d and
// dmin stay per super-block f32 values, applied once per super-block, so every
// stored value is exact whatever the spread of d and dmin along a row.  q4_K's
// scales, mins, d and dmin are grouped into one 1 KiB record per 32-row block
// and GEMM stage, which one wave copies to LDS with a single uniform load.
#include <algorithm>

#include "qmm_internal.h"
#include "qmm_common.h"

#include "../../include/qmm.h"

namespace qmm {

// ---------------------------------------------------------------------------
// Plane layout (all device, all library-owned; R = od_pad/32 row blocks):
//   wq  q6_K: int8 [R][nchunk][2 planes: hi, lo][2 k-halves][32 rows][16 bytes]
//             byte (row j, k) of plane p at
//             ((j/32*nchunk + k/32)*2 + p)*1024 + ((k%32)/16)*512 + (j%32)*16 + k%16
//             where the folded weight w = sc[k/16] * (code - 32) = hi*64 + lo,
//             w in [-4064, 4096], lo in [0, 63]
//       q4_K: int8 [R][nchunk][2 k-halves][32 rows][16 bytes]: the code of
//             (row j, k) in [0, 15] at byte
//             (j/32*nchunk + k/32)*1024 + ((k%32)/16)*512 + (j%32)*16 + k%16
//       q4_K packed: [R][nchunk][2 k-halves][32 rows][8 bytes]: the code of
//             (row j, k) in the low (k%16 < 8) or high (k%16 >= 8) nibble of
//             byte (j/32*nchunk + k/32)*512 + ((k%32)/16)*256 + (j%32)*8 + k%8
//             (one lane's 8 bytes unpack with two masks and two shifts into
//             its 16 code bytes)
//   wd  q6_K only: f32 [R][nsb][32 rows]  d of (row, super-block)
//   wsm q4_K only: [R][nchunk/4 stages][1024 bytes], one record per (32-row
//             block, stage of chunks 4g..4g+3), at byte (j/32*nchunk/4 + g)*1024:
//             +0    f16 [32 rows][4]: the 6-bit scale of (row j, chunk 4g + i)
//                   as an f16 integer at element (j%32)*4 + i (one 8-byte word
//                   per row: the A operand of the scale outer product)
//             +256  f16 [2][32 rows][4]: the 6-bit mins of the stage's
//                   super-block b = g/2, (row j, chunk 8b + 4h + i) at element
//                   (h*32 + j%32)*4 + i (lane half h of the min-term MFMA reads
//                   chunks 4h..4h+3 of its row as one 8-byte word)
//             +768  f32 [2][32 rows]: d*2^25 (part 0) and -dmin (part 1) of
//                   (row j, super-block b) at element part*32 + j%32 (both exact
//                   in f32; a zero is stored as +0)
//             the mins, d and dmin of super-block b are in both its records
// Rows od..od_pad-1 are zero in every plane.
// ---------------------------------------------------------------------------
size_t wq_bytes(int type, int64_t od_pad, int64_t id) {
  const size_t n = (size_t)od_pad * (size_t)id;
  return type == QMM_Q6_K ? n * 2 : type == QMM_Q4_K_PACKED ? n / 2 : n;
}
size_t wd_bytes(int type, int64_t od_pad, int64_t id) {
  return is_q4k(type) ? 0 : (size_t)od_pad * (size_t)(id / 256) * 4;
}
size_t wsm_bytes(int type, int64_t od_pad, int64_t id) {
  return is_q4k(type) ? (size_t)(od_pad / 32) * (size_t)(id / 128) * kQ4RecBytes : 0;
}

// q4_K: the 6-bit scale and min of sub-block cl of a 144-byte block (ggml's
// packing of the 12 bytes after d and dmin).
__device__ __forceinline__ void q4k_scale_min(const uint8_t* B, int cl, int& sc, int& mn) {
  const uint8_t* P = B + 4;
  if (cl < 4) {
    sc = P[cl] & 63;
    mn = P[cl + 4] & 63;
  } else {
    sc = (P[cl + 4] & 15) | ((P[cl - 4] >> 6) << 4);
    mn = (P[cl + 4] >> 4) | ((P[cl] >> 6) << 4);
  }
}

// q4_K: the values of (row jr of row block rb, chunk c) in the stage record of
// the chunk (its scale) and in both records of its super-block (its min; d25
// and ndmin, from the thread of the super-block's first chunk).
__device__ __forceinline__ void q4k_record(uint8_t* wsm, int rb, int nchunk, int c, int jr, uint16_t sc,
                                           uint16_t mn, float d25, float ndmin) {
  const int cl = c & 7;
  uint8_t* const rec0 = wsm + ((int64_t)rb * (nchunk / 4) + 2 * (c >> 3)) * kQ4RecBytes;
  uint8_t* const rec1 = rec0 + kQ4RecBytes;
  uint8_t* const rec = cl < 4 ? rec0 : rec1;
  ((uint16_t*)(rec + kQ4RecScOff))[jr * 4 + (cl & 3)] = sc;
  const int mi = ((cl >> 2) * 32 + jr) * 4 + (cl & 3);
  ((uint16_t*)(rec0 + kQ4RecMnOff))[mi] = mn;
  ((uint16_t*)(rec1 + kQ4RecMnOff))[mi] = mn;
  if (cl == 0) {
    for (uint8_t* r : {rec0, rec1}) {
      ((float*)(r + kQ4RecDOff))[jr] = d25;
      ((float*)(r + kQ4RecDOff))[32 + jr] = ndmin;
    }
  }
}

// One thread per (row j in [0, od_pad), chunk c, k-half h): 16 weights.
// One (row, 32-block, 16-weight half) of the planes: item gid.
__device__ __forceinline__ void repack_one(int64_t gid, const uint8_t* __restrict__ raw, int type, int od, int nsb,
                                           int nchunk, int8_t* __restrict__ wq, float* __restrict__ wd,
                                           uint8_t* __restrict__ wsm) {
  const int h = (int)(gid & 1);
  const int64_t rc = gid >> 1;
  const int c = (int)(rc % nchunk);
  const int j = (int)(rc / nchunk);
  const int rb = j >> 5, jr = j & 31;
  const int b = c >> 3, cl = c & 7;

  uint32_t hi[4] = {0, 0, 0, 0}, lo[4] = {0, 0, 0, 0};  // q6_K planes; q4_K codes in lo
  if (j < od) {
    if (type == QMM_Q6_K) {
      // 210-byte block: ql[128] | qh[64] | int8 scales[16] | f16 d (r56 section 1)
      const uint8_t* B = raw + ((int64_t)j * nsb + b) * 210;
      const int e0 = 32 * cl + 16 * h;          // first element inside the super-block
      const int half = e0 >> 7;                 // which 128-element half
      const int quarter = (e0 & 127) >> 5;      // which 32-element quarter of the half
      const int l0 = e0 & 31;
      const int sc = (int)(int8_t)B[192 + (e0 >> 4)];
      const uint8_t* ql = B + 64 * half + 32 * (quarter & 1);
      const uint8_t* qh = B + 128 + 32 * half;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int l = l0 + i;
        const int lowbits = quarter < 2 ? (ql[l] & 15) : (ql[l] >> 4);
        const int highbits = (qh[l] >> (2 * quarter)) & 3;
        const int w = sc * ((lowbits | (highbits << 4)) - 32);
        hi[i >> 2] |= (uint32_t)(uint8_t)(int8_t)(w >> 6) << (8 * (i & 3));
        lo[i >> 2] |= (uint32_t)(w & 63) << (8 * (i & 3));
      }
      if (h == 0 && cl == 0)
        wd[((int64_t)rb * nsb + b) * 32 + jr] = f16_bits_to_float(B[208] | (B[209] << 8));
    } else {
      // 144-byte block: f16 d | f16 dmin | 12 bytes of 6-bit scales/mins | qs[128]
      const uint8_t* B = raw + ((int64_t)j * nsb + b) * 144;
      int sc, mn;
      q4k_scale_min(B, cl, sc, mn);
      // 32-element sub-block cl: codes in qs[32*(cl/2) + 0..31], low nibble for
      // even sub-blocks, high nibble for odd ones
      const uint8_t* qs = B + 16 + 32 * (cl >> 1) + 16 * h;
      const int shift = (cl & 1) * 4;
#pragma unroll
      for (int i = 0; i < 16; ++i) lo[i >> 2] |= (uint32_t)((qs[i] >> shift) & 15) << (8 * (i & 3));
      if (h == 0) {
        // the scale and min as f16 integers (6 bits: exact); d and dmin once per
        // super-block, d times 2^25 (the GEMM's scale products and block dots
        // carry 2^-25 between them; a power of two, so the product stays exact)
        const float d = f16_bits_to_float(B[0] | (B[1] << 8)), dmin = f16_bits_to_float(B[2] | (B[3] << 8));
        q4k_record(wsm, rb, nchunk, c, jr, __builtin_bit_cast(uint16_t, (_Float16)sc),
                   __builtin_bit_cast(uint16_t, (_Float16)mn), ldexpf(d, 25) + 0.0f, -dmin + 0.0f);
      }
    }
  } else if (h == 0) {
    if (is_q4k(type))
      q4k_record(wsm, rb, nchunk, c, jr, 0, 0, 0.0f, 0.0f);
    else if (cl == 0)
      wd[((int64_t)rb * nsb + b) * 32 + jr] = 0.0f;
  }
  if (type == QMM_Q6_K) {
    int8_t* dst = wq + ((int64_t)rb * nchunk + c) * 2048 + h * 512 + jr * 16;
    *(uint4*)dst = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    *(uint4*)(dst + 1024) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  } else if (type == QMM_Q4_K_PACKED) {  // codes i and i+8 share byte i
    int8_t* dst = wq + ((int64_t)rb * nchunk + c) * kQ4PackedFrag + h * 256 + jr * 8;
    *(uint2*)dst = make_uint2(lo[0] | (lo[2] << 4), lo[1] | (lo[3] << 4));
  } else {
    int8_t* dst = wq + ((int64_t)rb * nchunk + c) * kQ4CodeFrag + h * 512 + jr * 16;
    *(uint4*)dst = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
}

// Items [0, total) over a grid of at most kRepackMaxBlocks work-groups (4M
// threads, eight times what the GPU holds at once), each thread striding by the
// grid's size: a launch stays far inside the 2^32 work-items one dispatch
// holds, whatever the matrix (2^37 items at the largest od and id), and every
// matrix above 4M items (e.g. a 32000 x 4096 output head: 8.2M) takes the
// stride.
constexpr int64_t kRepackMaxBlocks = 1 << 14;

__global__ void __launch_bounds__(256)
repack_kernel(const uint8_t* __restrict__ raw, int type, int od, int nsb, int nchunk,
              int64_t total, int8_t* __restrict__ wq, float* __restrict__ wd,
              uint8_t* __restrict__ wsm) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < total; gid += stride)
    repack_one(gid, raw, type, od, nsb, nchunk, wq, wd, wsm);
}

hipError_t launch_repack(const uint8_t* raw, const Planes& p, hipStream_t s) {
  const int64_t total = p.od_pad * p.nchunk * 2;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, kRepackMaxBlocks);
  repack_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
      raw, p.type, (int)p.od, (int)p.nsb, (int)p.nchunk, total, p.wq, p.wd, p.wsm);
  return hipGetLastError();
}

}  // namespace qmm
