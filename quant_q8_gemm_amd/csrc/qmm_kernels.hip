// qmm_kernels.hip -- HIP kernels for gfx950 (MI355X): registration repack,
// activation quantize prepass, and the q4_K / q6_K x q8 MMQ.
//
// Method (engineering log "minfer / cuda_optimization_steps", pages r45, r56,
// r58): activations are quantized by a prepass into q8 blocks of 32 with a
// (d, scaled sum) pair; weights are expanded once at registration into planes
// that the GEMM streams without arithmetic; the GEMM forms exact integer dots
// per 32-block on int8 matrix cores and applies the per-block scales in f32.
//
// MI355X design (differs from the pages' GB10 kernels on purpose):
//  * the d*scale pair plane of r56 section 2.2 becomes an integer fold: the
//    small integer scale of every 16/32-weight group is multiplied into the
//    weight codes at registration (exact), split into two int8 planes
//    (hi = w >> 6, lo = w & 63) so one K=32 int8 MFMA per plane yields the
//    scale-folded block dot J = 64*J_hi + J_lo exactly; only the f16 d of the
//    256-weight super-block stays a float, applied once per super-block;
//  * planes are stored in MFMA fragment order, so every lane's operand is one
//    contiguous 16-byte load and a wave's load is one contiguous 1 KiB;
//  * the q4_K min term sum_c dmin*min_c*s_c is a true small matrix product over
//    chunks; it runs on the f32 MFMA (32x32x2) instead of the vector ALU.
#include "qmm_internal.h"

#include "../../include/qmm.h"

namespace qmm {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// Plane layout (all device, all library-owned; R = od_pad/32 row blocks):
//   wq  int8  [R][nchunk][2 planes: hi, lo][2 k-halves][32 rows][16 bytes]
//             byte (row j, k) of plane p at
//             ((j/32*nchunk + k/32)*2 + p)*1024 + ((k%32)/16)*512 + (j%32)*16 + k%16
//             where the folded weight w = hi*64 + lo, lo in [0, 63]:
//               q6_K  w = sc[k/16] * (code - 32)      in [-4064, 4096]
//               q4_K  w = sc[k/32 % 8] * code         in [0, 945]
//   wd  f32   [R][nsb][32 rows]      d of (row, super-block)
//   wm  f32   [R][nchunk][32 rows]   -dmin*min of (row, chunk); q4_K only
// Rows od..od_pad-1 are zero in every plane.
// ---------------------------------------------------------------------------
size_t wq_bytes(int64_t od_pad, int64_t id) { return (size_t)od_pad * (size_t)id * 2; }
size_t wd_bytes(int64_t od_pad, int64_t id) { return (size_t)od_pad * (size_t)(id / 256) * 4; }
size_t wm_bytes(int type, int64_t od_pad, int64_t id) {
  return type == QMM_Q4_K ? (size_t)od_pad * (size_t)(id / 32) * 4 : 0;
}

__device__ __forceinline__ float f16_bits_to_float(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// One thread per (row j in [0, od_pad), chunk c, k-half h): 16 folded weights.
__global__ void __launch_bounds__(256)
repack_kernel(const uint8_t* __restrict__ raw, int type, int od, int nsb, int nchunk,
              int64_t total, int8_t* __restrict__ wq, float* __restrict__ wd,
              float* __restrict__ wm) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int h = (int)(gid & 1);
  const int64_t rc = gid >> 1;
  const int c = (int)(rc % nchunk);
  const int j = (int)(rc / nchunk);
  const int rb = j >> 5, jr = j & 31;
  const int b = c >> 3, cl = c & 7;

  uint32_t hi[4] = {0, 0, 0, 0}, lo[4] = {0, 0, 0, 0};
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
      const uint8_t* P = B + 4;
      int sc, mn;
      if (cl < 4) {
        sc = P[cl] & 63;
        mn = P[cl + 4] & 63;
      } else {
        sc = (P[cl + 4] & 15) | ((P[cl - 4] >> 6) << 4);
        mn = (P[cl + 4] >> 4) | ((P[cl] >> 6) << 4);
      }
      // 32-element sub-block cl: codes in qs[32*(cl/2) + 0..31], low nibble for
      // even sub-blocks, high nibble for odd ones
      const uint8_t* qs = B + 16 + 32 * (cl >> 1) + 16 * h;
      const int shift = (cl & 1) * 4;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int w = sc * ((qs[i] >> shift) & 15);
        hi[i >> 2] |= (uint32_t)(w >> 6) << (8 * (i & 3));
        lo[i >> 2] |= (uint32_t)(w & 63) << (8 * (i & 3));
      }
      if (h == 0) {
        const float dmin = f16_bits_to_float(B[2] | (B[3] << 8));
        wm[((int64_t)rb * nchunk + c) * 32 + jr] = -(dmin * (float)mn);
        if (cl == 0) wd[((int64_t)rb * nsb + b) * 32 + jr] = f16_bits_to_float(B[0] | (B[1] << 8));
      }
    }
  } else if (h == 0) {
    if (type == QMM_Q4_K) wm[((int64_t)rb * nchunk + c) * 32 + jr] = 0.0f;
    if (cl == 0) wd[((int64_t)rb * nsb + b) * 32 + jr] = 0.0f;
  }
  int8_t* dst = wq + ((int64_t)rb * nchunk + c) * 2048 + h * 512 + jr * 16;
  *(uint4*)dst = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  *(uint4*)(dst + 1024) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
}

hipError_t launch_repack(const uint8_t* raw, const Planes& p, hipStream_t s) {
  const int64_t total = p.od_pad * p.nchunk * 2;
  const int64_t blocks = (total + 255) / 256;
  repack_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
      raw, p.type, (int)p.od, (int)p.nsb, (int)p.nchunk, total, p.wq, p.wd, p.wm);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Quantize prepass.  Work-group = one 32-token block x kQuantChunks chunks;
// 8 lanes per (token, chunk), each lane holding 4 consecutive activations.
// A wave covers 8 consecutive tokens of one chunk, so its q bytes land as two
// contiguous 128-byte runs of the fragment and its scale pairs as 32 bytes.
// ---------------------------------------------------------------------------
constexpr int kQuantChunks = 8;

__device__ __forceinline__ int quant1(float v, float dhf) {
  if (dhf == 0.0f) return 0;
  float r = __builtin_rintf(v / dhf);  // IEEE division, round half to even
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
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
    const int q0 = quant1(v[i].x, dhf), q1 = quant1(v[i].y, dhf);
    const int q2 = quant1(v[i].z, dhf), q3 = quant1(v[i].w, dhf);
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

// ---------------------------------------------------------------------------
// MMQ.  Work-group = 4 waves in a 2 x 2 arrangement; each wave owns RB 32-row
// blocks x TB 32-token blocks of the output and streams every chunk of the
// inner dimension straight from the fragment-order planes into registers.
// MFMA orientation: A = weights (rows j), B = activations (columns t), so each
// lane's 16 outputs share one token: the activation scale dh is one register
// per chunk, and the super-block d is applied once per 8 chunks.
// ---------------------------------------------------------------------------
template <int TYPE, int RB, int TB>
__global__ void __launch_bounds__(256)
mmq_kernel(const int8_t* __restrict__ wq, const float* __restrict__ wd,
           const float* __restrict__ wm, const uint8_t* __restrict__ qq,
           const uint8_t* __restrict__ qs, int nchunk, int nsb, int od, int n_tok,
           int row_tiles, float* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rt = blockIdx.x % row_tiles;
  const int tt = blockIdx.x / row_tiles;
  const int rb0 = (rt * 2 + (wave >> 1)) * RB;
  const int tb0 = (tt * 2 + (wave & 1)) * TB;

  const int8_t* pa[RB];
  const float* pd[RB];
  const float* pm[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    pa[r] = wq + (size_t)(rb0 + r) * nchunk * 2048 + lane * 16;
    pd[r] = wd + (size_t)(rb0 + r) * nsb * 32 + 4 * (lane >> 5);
    pm[r] = TYPE == QMM_Q4_K ? wm + (size_t)(rb0 + r) * nchunk * 32 + lane : nullptr;
  }
  const uint8_t* pb[TB];
  const uint8_t* ps[TB];
  const uint8_t* pss[TB];
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    pb[t] = qq + (size_t)(tb0 + t) * nchunk * 1024 + lane * 16;
    ps[t] = qs + (size_t)(tb0 + t) * nchunk * 128 + (lane & 31) * 4;
    pss[t] = qs + (size_t)(tb0 + t) * nchunk * 128 + (lane >> 5) * 128 + (lane & 31) * 4 + 2;
  }

  v16f acc[RB][TB];
  v16f inner[RB][TB];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][t][i] = 0.0f;

  const v16i zero = {};
  for (int b = 0; b < nsb; ++b) {
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const size_t c = (size_t)b * 8 + cc;
      v4i ahi[RB], alo[RB], bq[TB];
      float dh[TB];
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        ahi[r] = *(const v4i*)(pa[r] + c * 2048);
        alo[r] = *(const v4i*)(pa[r] + c * 2048 + 1024);
      }
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        bq[t] = *(const v4i*)(pb[t] + c * 1024);
        dh[t] = f16_bits_to_float(*(const uint16_t*)(ps[t] + c * 128));
      }
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < TB; ++t) {
          const v16i jh = __builtin_amdgcn_mfma_i32_32x32x32_i8(ahi[r], bq[t], zero, 0, 0, 0);
          const v16i jl = __builtin_amdgcn_mfma_i32_32x32x32_i8(alo[r], bq[t], zero, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float f = (float)((jh[i] << 6) + jl[i]);
            inner[r][t][i] = cc == 0 ? f * dh[t] : fmaf(f, dh[t], inner[r][t][i]);
          }
        }
      if (TYPE == QMM_Q4_K && (cc & 1)) {
        float m[RB], sv[TB];
#pragma unroll
        for (int r = 0; r < RB; ++r) m[r] = pm[r][(c - 1) * 32];
#pragma unroll
        for (int t = 0; t < TB; ++t) sv[t] = f16_bits_to_float(*(const uint16_t*)(pss[t] + (c - 1) * 128));
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
          for (int t = 0; t < TB; ++t)
            acc[r][t] = __builtin_amdgcn_mfma_f32_32x32x2f32(m[r], sv[t], acc[r][t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      float d[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 d4 = *(const float4*)(pd[r] + (size_t)b * 32 + 8 * g);
        d[4 * g] = d4.x;
        d[4 * g + 1] = d4.y;
        d[4 * g + 2] = d4.z;
        d[4 * g + 3] = d4.w;
      }
#pragma unroll
      for (int t = 0; t < TB; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[r][t][i] = fmaf(inner[r][t][i], d[i], acc[r][t][i]);
    }
  }

#pragma unroll
  for (int t = 0; t < TB; ++t) {
    const int tok = (tb0 + t) * 32 + (lane & 31);
    if (tok >= n_tok) continue;
    float* orow = out + (size_t)tok * od;
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = (rb0 + r) * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        if (j < od) orow[j] = acc[r][t][i];
      }
  }
}

constexpr int kRB = 1;  // 32-row blocks per wave
constexpr int kTB = 2;  // 32-token blocks per wave

hipError_t launch_mmq(const Planes& p, const uint8_t* qact, int64_t n_tok, int64_t t_pad,
                      float* out, hipStream_t s) {
  const int row_tiles = (int)(p.od_pad / (64 * kRB));
  const int tok_tiles = (int)((n_tok + 64 * kTB - 1) / (64 * kTB));
  const uint8_t* qs = qact + (size_t)t_pad * (size_t)p.id;
  dim3 grid((unsigned)(row_tiles * tok_tiles)), block(256);
  if (p.type == QMM_Q6_K)
    mmq_kernel<QMM_Q6_K, kRB, kTB><<<grid, block, 0, s>>>(
        p.wq, p.wd, p.wm, qact, qs, (int)p.nchunk, (int)p.nsb, (int)p.od, (int)n_tok,
        row_tiles, out);
  else
    mmq_kernel<QMM_Q4_K, kRB, kTB><<<grid, block, 0, s>>>(
        p.wq, p.wd, p.wm, qact, qs, (int)p.nchunk, (int)p.nsb, (int)p.od, (int)n_tok,
        row_tiles, out);
  return hipGetLastError();
}

}  // namespace qmm
