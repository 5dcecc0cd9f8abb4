// qmm_repack.hip -- registration-time repack of q6_K / q4_K blocks into the
// planes the MMQ streams (the once-per-weight expansion of the r56 and r58
// pages of the engineering log "minfer / cuda_optimization_steps": r56 sections
// 2.2-2.3, r58 section 3.2).  Instead of the pages' f32 d*scale pair plane the
// small integer group scales stay integers: q6_K's int8 scale of every 16
// weights is multiplied into the codes (exact) and the folded weight split into
// two int8 planes (hi = w >> 6, lo = w & 63), so one K=32 int8 MFMA per plane
// yields the block dot J = 64*J_hi + J_lo, and only the f16 d of the super-block
// stays a float.  q4_K's 4-bit codes become int8 bytes in MFMA fragment order;
// its block scale d*sc and block min dmin*min (f16 times a 6-bit integer: 17
// significant bits, exact in f32) are stored, scaled by a power of two 2^e per
// row, as exact pairs of f16 values hi + lo -- the operands from which the GEMM's
// f16 matrix-core products form d*sc*dh and the min term; the GEMM multiplies
// its results by 2^-e once, at the store.
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
//   wd  q6_K: f32 [R][nsb][32 rows]  d of (row, super-block)
//       q4_K: f32 [R][32 rows]       2^-e of the row: e = 13 - floor(log2 M), M the
//             largest |d*sc| and |dmin*min| of the row (e = 0 if M = 0), so that
//             every scaled value is below 2^14 in magnitude
//   wmn f16   [R][nsb][2][2][32 rows][4]  q4_K only: -dmin*min*2^e of (row j,
//             chunk c) as hi + lo, hi = f16(v), lo = f16(v - hi), part p = 0 (hi)
//             or 1 (lo) at element (((j/32*nsb + c/8)*2 + p)*2 + (c%8)/4)*128
//             + (j%32)*4 + c%4: per part two halves of [32 rows][4 chunks], so
//             a lane half's 8-byte reads are consecutive
//   wsc f16   [R][nsb][2][2][32 rows][2][2]  q4_K only: d*sc*2^e of (row j,
//             chunk c) as the pair (hi, lo), at element
//             ((((j/32*nsb + c/8)*2 + (c%8)/4)*2 + (c%4)/2)*32 + j%32)*4
//             + (c%2)*2 + p: per stage of 4 chunks, lane half (c%4)/2 of a row
//             reads its two chunks' pairs as one 8-byte word
// Rows od..od_pad-1 are zero in every plane.
// ---------------------------------------------------------------------------
size_t wq_bytes(int type, int64_t od_pad, int64_t id) {
  return type == QMM_Q6_K ? (size_t)od_pad * (size_t)id * 2 : (size_t)od_pad * (size_t)id;
}
size_t wd_bytes(int type, int64_t od_pad, int64_t id) {
  return type == QMM_Q4_K ? (size_t)od_pad * 4 : (size_t)od_pad * (size_t)(id / 256) * 4;
}
size_t wmn_bytes(int type, int64_t od_pad, int64_t id) {
  return type == QMM_Q4_K ? (size_t)od_pad * (size_t)(id / 32) * 4 : 0;
}
size_t wdm_bytes(int, int64_t, int64_t) { return 0; }
size_t wsc_bytes(int type, int64_t od_pad, int64_t id) {
  return type == QMM_Q4_K ? (size_t)od_pad * (size_t)(id / 32) * 4 : 0;
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

// q4_K: one thread per row in [0, od_pad): wd[row] = 2^-e (1 for padding rows).
__global__ void __launch_bounds__(256)
q4k_row_scale_kernel(const uint8_t* __restrict__ raw, int od, int nsb, int od_pad, float* __restrict__ wd) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= od_pad) return;
  float m = 0.0f;
  if (j < od) {
    for (int b = 0; b < nsb; ++b) {
      const uint8_t* B = raw + ((int64_t)j * nsb + b) * 144;
      const float d = f16_bits_to_float(B[0] | (B[1] << 8)), dmin = f16_bits_to_float(B[2] | (B[3] << 8));
      for (int cl = 0; cl < 8; ++cl) {
        int sc, mn;
        q4k_scale_min(B, cl, sc, mn);
        m = fmaxf(m, fmaxf(fabsf(d * (float)sc), fabsf(dmin * (float)mn)));  // exact products
      }
    }
  }
  const int e = m > 0.0f ? 13 - ilogbf(m) : 0;
  wd[j] = ldexpf(1.0f, -e);
}

// v (exact in f32, at most 17 significant bits) as hi + lo, two f16 values; a
// zero part is stored as +0 (the + 0 maps -0 to +0), whatever the signs that
// formed it
__device__ __forceinline__ void split_f16(float v, uint16_t& hi, uint16_t& lo) {
  const _Float16 h = (_Float16)(v + 0.0f);
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, (_Float16)((v - (float)h) + 0.0f));
}

// One thread per (row j in [0, od_pad), chunk c, k-half h): 16 weights.
__global__ void __launch_bounds__(256)
repack_kernel(const uint8_t* __restrict__ raw, int type, int od, int nsb, int nchunk,
              int64_t total, int8_t* __restrict__ wq, float* __restrict__ wd,
              uint16_t* __restrict__ wmn, uint16_t* __restrict__ wsc) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
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
        // 2^e from the row's 2^-e (a power of two: exact); d*sc and dmin*min are
        // exact in f32, and so are their products with 2^e
        const float pe = 1.0f / wd[j];
        const float d = f16_bits_to_float(B[0] | (B[1] << 8)), dmin = f16_bits_to_float(B[2] | (B[3] << 8));
        uint16_t hi, lo;
        split_f16(d * (float)sc * pe, hi, lo);
        const int64_t si = ((((int64_t)rb * nsb + b) * 2 + (cl >> 2)) * 2 + ((cl & 3) >> 1)) * 32 + jr;
        wsc[si * 4 + (cl & 1) * 2] = hi;
        wsc[si * 4 + (cl & 1) * 2 + 1] = lo;
        split_f16(-(dmin * (float)mn) * pe, hi, lo);
        const int64_t mi = (((int64_t)rb * nsb + b) * 2) * 2 + (cl >> 2);
        wmn[mi * 128 + jr * 4 + (cl & 3)] = hi;
        wmn[(mi + 2) * 128 + jr * 4 + (cl & 3)] = lo;
      }
    }
  } else if (h == 0) {
    if (type == QMM_Q4_K) {
      const int64_t si = ((((int64_t)rb * nsb + b) * 2 + (cl >> 2)) * 2 + ((cl & 3) >> 1)) * 32 + jr;
      wsc[si * 4 + (cl & 1) * 2] = 0;
      wsc[si * 4 + (cl & 1) * 2 + 1] = 0;
      const int64_t mi = (((int64_t)rb * nsb + b) * 2) * 2 + (cl >> 2);
      wmn[mi * 128 + jr * 4 + (cl & 3)] = 0;
      wmn[(mi + 2) * 128 + jr * 4 + (cl & 3)] = 0;
    } else if (cl == 0) {
      wd[((int64_t)rb * nsb + b) * 32 + jr] = 0.0f;
    }
  }
  if (type == QMM_Q6_K) {
    int8_t* dst = wq + ((int64_t)rb * nchunk + c) * 2048 + h * 512 + jr * 16;
    *(uint4*)dst = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    *(uint4*)(dst + 1024) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  } else {
    int8_t* dst = wq + ((int64_t)rb * nchunk + c) * kQ4CodeFrag + h * 512 + jr * 16;
    *(uint4*)dst = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
}

hipError_t launch_repack(const uint8_t* raw, const Planes& p, hipStream_t s) {
  if (p.type == QMM_Q4_K) {  // the rows' 2^-e first: the repack reads it
    q4k_row_scale_kernel<<<dim3((unsigned)((p.od_pad + 255) / 256)), dim3(256), 0, s>>>(
        raw, (int)p.od, (int)p.nsb, (int)p.od_pad, p.wd);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  const int64_t total = p.od_pad * p.nchunk * 2;
  const int64_t blocks = (total + 255) / 256;
  repack_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
      raw, p.type, (int)p.od, (int)p.nsb, (int)p.nchunk, total, p.wq, p.wd, p.wmn, p.wsc);
  return hipGetLastError();
}

}  // namespace qmm
