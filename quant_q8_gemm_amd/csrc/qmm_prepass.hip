// qmm_prepass.hip -- the quantize-transpose prepass (r45 page, section 1.1):
// f32 activations -> q8 blocks of 32 with a (dh, s) scale pair, written in the
// MFMA fragment order the MMQ reads.
#include "qmm_internal.h"
#include "qmm_common.h"

#include "../../include/qmm.h"

namespace qmm {

// ---------------------------------------------------------------------------
// Quantize prepass.  Work-group = one 32-token block x kQuantChunks chunks;
// 8 lanes per (token, chunk), each lane holding 4 consecutive activations.
// A wave covers 8 consecutive tokens of one chunk, so its q bytes land as two
// contiguous 128-byte runs of the fragment and its scale pairs as 32 bytes.
// The kernel streams HBM: every lane issues all of its loads before the first
// wait, and the reductions over a (token, chunk)'s 8 lanes stay in registers
// (DPP moves).
// ---------------------------------------------------------------------------
constexpr int kQuantChunks = 2;

// DPP controls: swap neighbours in a quad, swap pairs in a quad, and mirror
// each half-row of 8 lanes (lane i <-> 7 - i).  After the two quad steps every
// lane of a quad holds the quad's result, so the mirror step combines the two
// quads of an aligned group of 8 lanes.
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror

template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}

// Maximum of non-negative finite floats over the 8 lanes, on their bit patterns
// (ordered like the values), so each step is one integer max.
__device__ __forceinline__ float max8(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  u = max(u, (uint32_t)dpp<kDppQuadXor1>((int)u));
  u = max(u, (uint32_t)dpp<kDppQuadXor2>((int)u));
  u = max(u, (uint32_t)dpp<kDppHalfMirror>((int)u));
  return __builtin_bit_cast(float, u);
}

__device__ __forceinline__ int sum8(int v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  return v + dpp<kDppHalfMirror>(v);
}

// q = clamp(rint(v / dh), -127, 127) where v / dh is the correctly rounded f32
// quotient (IEEE division) and rint rounds half to even.  The correctly rounded
// division costs about a dozen instructions, so the quotient is first formed as
// v * rcp(dh): with |v / dh| <= 127.1 (|v| <= amax, dh = f16(amax/127)) the
// reciprocal (1 ulp) and the product (0.5 ulp) put it within 2.3e-5 of the
// exact quotient, and the correctly rounded quotient is within 3.8e-6 of it.
// So unless the product lies within 1e-4 of a half-integer, both round to the
// same integer; when one of a lane's four products does, the lane divides all
// four exactly.  With dh == 0 the reciprocal is taken as 0, which gives q = 0.
__device__ __forceinline__ void quant4(const float4& v, float dhf, float inv, int q[4]) {
  const float r[4] = {v.x * inv, v.y * inv, v.z * inv, v.w * inv};
  float n[4], e[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    n[i] = __builtin_rintf(r[i]);
    e[i] = fabsf(r[i] - n[i]);
  }
  if (fmaxf(fmaxf(e[0], e[1]), fmaxf(e[2], e[3])) > 0.5f - 1e-4f) {
    n[0] = __builtin_rintf(v.x / dhf);
    n[1] = __builtin_rintf(v.y / dhf);
    n[2] = __builtin_rintf(v.z / dhf);
    n[3] = __builtin_rintf(v.w / dhf);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = (int)__builtin_amdgcn_fmed3f(n[i], -127.0f, 127.0f);
}

__global__ void __launch_bounds__(256)
quantize_kernel(const float* __restrict__ x, int n_tok, int id, int nchunk, int chunk_major,
                uint8_t* __restrict__ qq, uint8_t* __restrict__ qs) {
  const int tb = chunk_major ? blockIdx.y : blockIdx.x;
  const int c0 = (chunk_major ? blockIdx.x : blockIdx.y) * kQuantChunks;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tt = wave * 8 + (lane >> 3);
  const int sub = lane & 7;
  const int64_t t = (int64_t)tb * 32 + tt;
  const bool live = t < n_tok;
  const bool block_full = (int64_t)(tb + 1) * 32 <= n_tok;  // uniform: no lane past the end
  // Lanes past the last token read the last token's row (and chunks past the
  // end read the last chunk), so that every load is in bounds and issued
  // unconditionally; their values are replaced by zeros below.
  const float* xr = x + (live ? t : (int64_t)n_tok - 1) * id + 4 * sub;

  float4 v[kQuantChunks];
#pragma unroll
  for (int i = 0; i < kQuantChunks; ++i)
    v[i] = *(const float4*)(xr + 32 * min(c0 + i, nchunk - 1));
#pragma unroll
  for (int i = 0; i < kQuantChunks; ++i) {
    const int c = c0 + i;
    if (c >= nchunk) break;
    if (!block_full && !live) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    const float amax = max8(fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)),
                                  fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    const float d32 = amax / 127.0f;
    const _Float16 dh = (_Float16)d32;  // round to nearest even
    const float dhf = (float)dh;
    const float inv = dhf == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(dhf);
    int q[4];
    quant4(v[i], dhf, inv, q);
    const int S = sum8(q[0] + q[1] + q[2] + q[3]);
    const _Float16 sh = (_Float16)(dhf * (float)S);  // the product is exact in f32
    const uint32_t packed = (uint32_t)(q[0] & 255) | ((uint32_t)(q[1] & 255) << 8) |
                            ((uint32_t)(q[2] & 255) << 16) | ((uint32_t)(q[3] & 255) << 24);
    const int64_t frag = (int64_t)tb * nchunk + c;
    *(uint32_t*)(qq + frag * 1024 + (sub >> 2) * 512 + tt * 16 + (sub & 3) * 4) = packed;
    if (sub == 0)
      *(uint32_t*)(qs + frag * 128 + tt * 4) =
          (uint32_t)__builtin_bit_cast(uint16_t, dh) | ((uint32_t)__builtin_bit_cast(uint16_t, sh) << 16);
  }
}

hipError_t launch_quantize(const float* x, int64_t n_tok, int64_t t_pad, int64_t id,
                           uint8_t* qact, hipStream_t s) {
  const int64_t nchunk = id / 32;
  const unsigned n_tb = (unsigned)(t_pad / 32), n_cg = (unsigned)((nchunk + kQuantChunks - 1) / kQuantChunks);
  // Work-group order.  Many tokens: chunk groups fastest, so consecutive
  // work-groups read consecutive stretches of the same 32 rows (3314 x 4096:
  // 22% faster; with token blocks fastest the rows' power-of-two stride
  // concentrates the reads).  Few tokens: token blocks fastest (4-8% faster at
  // 512 and 2048 tokens).
  const int chunk_major = n_tb > 96;
  const dim3 grid = chunk_major ? dim3(n_cg, n_tb) : dim3(n_tb, n_cg);
  quantize_kernel<<<grid, dim3(256), 0, s>>>(x, (int)n_tok, (int)id, (int)nchunk, chunk_major, qact,
                                             qact + (size_t)t_pad * (size_t)id);
  return hipGetLastError();
}

}  // namespace qmm
