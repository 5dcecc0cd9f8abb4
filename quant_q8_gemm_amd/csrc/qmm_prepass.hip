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
// ---------------------------------------------------------------------------
constexpr int kQuantChunks = 4;

// q = clamp(rint(v / dh), -127, 127) where v / dh is the correctly rounded f32
// quotient (IEEE division) and rint rounds half to even.  The correctly rounded
// division costs about a dozen instructions, so the quotient is first formed as
// v * rcp(dh): with |v / dh| <= 127.1 (|v| <= amax, dh = f16(amax/127)) the
// reciprocal (1 ulp) and the product (0.5 ulp) put it within 2.3e-5 of the
// exact quotient, and the correctly rounded quotient is within 3.8e-6 of it.
// So unless the product lies within 1e-4 of a half-integer, both round to the
// same integer; in that rare case the quotient is divided exactly.
__device__ __forceinline__ int quant1(float v, float dhf, float inv) {
  if (dhf == 0.0f) return 0;
  const float r = v * inv;
  float n = __builtin_rintf(r);
  if (fabsf(r - n) > 0.5f - 1e-4f) n = __builtin_rintf(v / dhf);
  n = fminf(fmaxf(n, -127.0f), 127.0f);
  return (int)n;
}

__global__ void __launch_bounds__(256)
quantize_kernel(const float* __restrict__ x, int n_tok, int id, int nchunk,
                uint8_t* __restrict__ qq, uint8_t* __restrict__ qs) {
  const int tb = blockIdx.x;
  const int c0 = blockIdx.y * kQuantChunks;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tt = wave * 8 + (lane >> 3);
  const int sub = lane & 7;
  const int64_t t = (int64_t)tb * 32 + tt;
  const bool live = t < n_tok;
  const float* xr = x + t * id + 4 * sub;

  float4 v[kQuantChunks];
#pragma unroll
  for (int i = 0; i < kQuantChunks; ++i) {
    const int c = c0 + i;
    v[i] = (live && c < nchunk) ? *(const float4*)(xr + 32 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int i = 0; i < kQuantChunks; ++i) {
    const int c = c0 + i;
    if (c >= nchunk) break;
    float amax = fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w)));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    amax = fmaxf(amax, __shfl_xor(amax, 4));
    const float d32 = amax / 127.0f;
    const _Float16 dh = (_Float16)d32;  // round to nearest even
    const float dhf = (float)dh;
    const float inv = __builtin_amdgcn_rcpf(dhf);
    const int q0 = quant1(v[i].x, dhf, inv), q1 = quant1(v[i].y, dhf, inv);
    const int q2 = quant1(v[i].z, dhf, inv), q3 = quant1(v[i].w, dhf, inv);
    int S = q0 + q1 + q2 + q3;
    S += __shfl_xor(S, 1);
    S += __shfl_xor(S, 2);
    S += __shfl_xor(S, 4);
    const _Float16 sh = (_Float16)(dhf * (float)S);  // the product is exact in f32
    const uint32_t packed = (uint32_t)(q0 & 255) | ((uint32_t)(q1 & 255) << 8) |
                            ((uint32_t)(q2 & 255) << 16) | ((uint32_t)(q3 & 255) << 24);
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
  dim3 grid((unsigned)(t_pad / 32), (unsigned)((nchunk + kQuantChunks - 1) / kQuantChunks));
  quantize_kernel<<<grid, dim3(256), 0, s>>>(x, (int)n_tok, (int)id, (int)nchunk, qact,
                                             qact + (size_t)t_pad * (size_t)id);
  return hipGetLastError();
}

}  // namespace qmm
