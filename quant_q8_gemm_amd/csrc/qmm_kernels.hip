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

// Empty asm that claims to modify v: the value must be produced before this
// point and cannot be recomputed after it.  Emits no instruction; used to keep
// software-pipeline stages where they are written.
template <class T>
__device__ __forceinline__ void pin(T& v) {
  asm volatile("" : "+v"(v));
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
// MMQ.  Work-group = 8 waves (two per SIMD) on a 64-row x 128-token output tile:
// a 2 x 4 grid of 32 x 32 blocks, one block per wave.  The inner dimension is
// walked one 256-wide super-block at a time; each super-block's operands (both
// weight planes for the 2 row blocks, the q8 codes and scale pairs for the 4
// token blocks, d, and for q4_K the -dmin*min plane) are copied once per
// work-group into LDS and read from there by the waves that share them.  The
// LDS is double-buffered: the global loads for super-block b+1 are issued
// before super-block b is computed and written to the other buffer after it,
// so there is one barrier per super-block.
// MFMA orientation: A = weights (rows j), B = activations (columns t), so each
// lane's 16 outputs share one token: the activation scale dh is one register
// per chunk, and the super-block d is applied once per 8 chunks.
// ---------------------------------------------------------------------------
constexpr int kWavesR = 2;                 // row blocks per work-group
constexpr int kWavesT = 4;                 // token blocks per work-group
constexpr int kTileRows = 32 * kWavesR;    // 64
constexpr int kTileToks = 32 * kWavesT;    // 128
constexpr int kThreads = 64 * kWavesR * kWavesT;

struct alignas(16) Stage {
  int8_t a[kWavesR][8][2][1024];   // weight planes: [row block][chunk][hi, lo][fragment]
  int8_t b[kWavesT][8][1024];      // q8 codes: [token block][chunk][fragment]
  uint32_t s[kWavesT][8][32];      // (dh, s) pairs: [token block][chunk][token]
  float d[kWavesR][32];            // super-block d per row
  float m[kWavesR][8][32];         // -dmin*min per (chunk, row); q4_K only
};
static_assert(sizeof(Stage) % 16 == 0, "stage must be a whole number of 16-byte units");

// The staging code assigns whole 1 KiB fragments to waves; it is written for
// this geometry.
static_assert(kWavesR == 2 && kWavesT == 4, "staging assumes 2 row blocks x 4 token blocks");
static_assert(sizeof(((Stage*)0)->a) == 32 * 1024 && sizeof(((Stage*)0)->b) == 32 * 1024,
              "8 waves x 4 fragments of 1 KiB each for weights and codes");
static_assert(sizeof(((Stage*)0)->s) == 4 * 1024 && sizeof(((Stage*)0)->m) == 2 * 1024 &&
              sizeof(((Stage*)0)->d) == 256, "scale pairs, mins and d sizes");

// Work-group index -> (row tile, token tile).  Work-groups are dispatched
// round-robin over the 8 XCDs (each with its own L2); this map gives every XCD
// a contiguous run of tiles in row-major (row tile, token tile) order, so the
// work-groups that stream the same weight rows share one L2.
__device__ __forceinline__ int xcd_swizzle(int i, int n) {
  const int q = n / 8, r = n % 8;
  const int x = i % 8, slot = i / 8;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + slot;
}

template <int TYPE>
__global__ void __launch_bounds__(kThreads)
mmq_kernel(const int8_t* __restrict__ wq, const float* __restrict__ wd,
           const float* __restrict__ wm, const uint8_t* __restrict__ qq,
           const uint8_t* __restrict__ qs, int nchunk, int nsb, int od, int n_tok,
           int tok_tiles, int vec_store, float* __restrict__ out) {
  __shared__ Stage stage[2];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave / kWavesT, wt = wave % kWavesT;
  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int rt = tile / tok_tiles, tt = tile % tok_tiles;
  const int rb0 = rt * kWavesR, tb0 = tt * kWavesT;

  // Staging of super-block b into an LDS stage with direct global->LDS loads
  // (global_load_lds_dwordx4: lane l's 16 bytes land at the LDS base + 16*l, so
  // one wave instruction moves one 1 KiB fragment).  Per stage: 32 weight
  // fragments (2 row blocks x 8 chunks x hi/lo, 16 KiB contiguous per row block
  // in global memory), 32 code fragments (4 token blocks x 8 chunks, 8 KiB
  // contiguous per token block), 4 KiB of scale pairs, 1 KiB of -dmin*min per
  // row block (q4_K) and 128 bytes of d per row block.  Wave w moves weight
  // fragments 4w..4w+3 and code fragments 4w..4w+3; waves 0-3 the scale pairs
  // of token block w; waves 4-5 the -dmin*min of row block w-4; wave 6 the d.
  const size_t a_row = (size_t)nchunk * 2048, b_tok = (size_t)nchunk * 1024;
  const int8_t* ga = wq + (size_t)(rb0 + (4 * wave) / 16) * a_row + (size_t)((4 * wave) % 16) * 1024 + lane * 16;
  const uint8_t* gb = qq + (size_t)(tb0 + (4 * wave) / 8) * b_tok + (size_t)((4 * wave) % 8) * 1024 + lane * 16;
  const uint8_t* gs = qs + ((size_t)(tb0 + (wave & 3)) * nchunk) * 128 + lane * 16;
  const float* gm = TYPE == QMM_Q4_K ? wm + ((size_t)(rb0 + (wave & 1)) * nchunk) * 32 + lane * 4 : nullptr;
  const float* gd = wd + ((size_t)(rb0 + ((lane & 15) >> 3)) * nsb) * 32 + (lane & 7) * 4;

#define QMM_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define QMM_STAGE_LOADS(SB, ST)                                                                 \
  do {                                                                                         \
    const size_t sb = (size_t)(SB);                                                             \
    int8_t* la = &(ST).a[(4 * wave) / 16][0][0][0] + ((4 * wave) % 16) * 1024;                 \
    int8_t* lb = &(ST).b[(4 * wave) / 8][0][0] + ((4 * wave) % 8) * 1024;                      \
    _Pragma("unroll") for (int u = 0; u < 4; ++u) {                                            \
      __builtin_amdgcn_global_load_lds(ga + sb * 16384 + u * 1024, QMM_LDS(la + u * 1024), 16, 0, 0); \
      __builtin_amdgcn_global_load_lds(gb + sb * 8192 + u * 1024, QMM_LDS(lb + u * 1024), 16, 0, 0);  \
    }                                                                                          \
    if (wave < 4)                                                                              \
      __builtin_amdgcn_global_load_lds(gs + sb * 1024, QMM_LDS(&(ST).s[wave][0][0]), 16, 0, 0); \
    else if (TYPE == QMM_Q4_K && wave < 6)                                                     \
      __builtin_amdgcn_global_load_lds(gm + sb * 256, QMM_LDS(&(ST).m[wave - 4][0][0]), 16, 0, 0); \
    else if (wave == 6 && lane < 16)                                                           \
      __builtin_amdgcn_global_load_lds(gd + sb * 32, QMM_LDS(&(ST).d[0][0]), 16, 0, 0);        \
  } while (0)

  v16f acc, inner;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
  const v16i zero = {};

  QMM_STAGE_LOADS(0, stage[0]);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int b = 0; b < nsb; ++b) {
    const Stage& st = stage[b & 1];
    // stage (b+1)&1 was last read in iteration b-1, which every wave finished
    // before the barrier that ended it
    if (b + 1 < nsb) QMM_STAGE_LOADS(b + 1, stage[(b + 1) & 1]);
    // Software pipeline over the 8 chunks: step cc reads the LDS operands of
    // chunk cc+2, issues the two MFMAs of chunk cc+1, then runs the scale
    // epilogue of chunk cc on the vector ALU while the matrix core works.  The
    // scheduling-group barriers fix that order inside every step.
    v4i ahi0 = *(const v4i*)(st.a[wr][0][0] + lane * 16);
    v4i alo0 = *(const v4i*)(st.a[wr][0][1] + lane * 16);
    v4i bq0 = *(const v4i*)(st.b[wt][0] + lane * 16);
    v4i ahi1 = *(const v4i*)(st.a[wr][1][0] + lane * 16);
    v4i alo1 = *(const v4i*)(st.a[wr][1][1] + lane * 16);
    v4i bq1 = *(const v4i*)(st.b[wt][1] + lane * 16);
    v16i jh = __builtin_amdgcn_mfma_i32_32x32x32_i8(ahi0, bq0, zero, 0, 0, 0);
    v16i jl = __builtin_amdgcn_mfma_i32_32x32x32_i8(alo0, bq0, zero, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const float dh = f16_bits_to_float(st.s[wt][cc][lane & 31] & 0xFFFF);
      v4i ahi2, alo2, bq2;
      if (cc < 6) {
        ahi2 = *(const v4i*)(st.a[wr][cc + 2][0] + lane * 16);
        alo2 = *(const v4i*)(st.a[wr][cc + 2][1] + lane * 16);
        bq2 = *(const v4i*)(st.b[wt][cc + 2] + lane * 16);
      }
      v16i jh_next, jl_next;
      if (cc < 7) {
        jh_next = __builtin_amdgcn_mfma_i32_32x32x32_i8(ahi1, bq1, zero, 0, 0, 0);
        jl_next = __builtin_amdgcn_mfma_i32_32x32x32_i8(alo1, bq1, zero, 0, 0, 0);
        pin(jh_next);
        pin(jl_next);
      }
      if (TYPE == QMM_Q4_K && (cc & 1)) {
        const int ck = cc - 1 + (lane >> 5);
        const float mv = st.m[wr][ck][lane & 31];
        const float sv = f16_bits_to_float(st.s[wt][ck][lane & 31] >> 16);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(mv, sv, acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float f = (float)((jh[i] << 6) + jl[i]);
        inner[i] = cc == 0 ? f * dh : fmaf(f, dh, inner[i]);
      }
      pin(inner);
      if (cc < 7) {
        jh = jh_next;
        jl = jl_next;
        ahi1 = ahi2;
        alo1 = alo2;
        bq1 = bq2;
      }
      // order inside the step: LDS reads, then MFMAs, then the vector epilogue
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // DS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);  // VALU
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 d4 = *(const float4*)(&st.d[wr][8 * g + 4 * (lane >> 5)]);
      acc[4 * g + 0] = fmaf(inner[4 * g + 0], d4.x, acc[4 * g + 0]);
      acc[4 * g + 1] = fmaf(inner[4 * g + 1], d4.y, acc[4 * g + 1]);
      acc[4 * g + 2] = fmaf(inner[4 * g + 2], d4.z, acc[4 * g + 2]);
      acc[4 * g + 3] = fmaf(inner[4 * g + 3], d4.w, acc[4 * g + 3]);
    }
    if (b + 1 < nsb) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads for b+1 landed
      __syncthreads();                                   // everyone's landed; stage b is free
    }
  }

  const int tok = (tb0 + wt) * 32 + (lane & 31);
  if (tok < n_tok) {
    float* orow = out + (size_t)tok * od;
    const int jb = (rb0 + wr) * 32 + 4 * (lane >> 5);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int j = jb + 8 * g;
      if (vec_store && j + 3 < od) {
        *(float4*)(orow + j) = make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (j + i < od) orow[j + i] = acc[4 * g + i];
      }
    }
  }
}

#undef QMM_STAGE_LOADS
#undef QMM_LDS

hipError_t launch_mmq(const Planes& p, const uint8_t* qact, int64_t n_tok, int64_t t_pad,
                      float* out, hipStream_t s) {
  const int row_tiles = (int)(p.od_pad / kTileRows);
  const int tok_tiles = (int)((n_tok + kTileToks - 1) / kTileToks);
  const uint8_t* qs = qact + (size_t)t_pad * (size_t)p.id;
  const int vec_store = (p.od % 4 == 0) && ((uintptr_t)out % 16 == 0);
  dim3 grid((unsigned)(row_tiles * tok_tiles)), block(kThreads);
  if (p.type == QMM_Q6_K)
    mmq_kernel<QMM_Q6_K><<<grid, block, 0, s>>>(p.wq, p.wd, p.wm, qact, qs, (int)p.nchunk,
                                                 (int)p.nsb, (int)p.od, (int)n_tok, tok_tiles,
                                                 vec_store, out);
  else
    mmq_kernel<QMM_Q4_K><<<grid, block, 0, s>>>(p.wq, p.wd, p.wm, qact, qs, (int)p.nchunk,
                                                 (int)p.nsb, (int)p.od, (int)n_tok, tok_tiles,
                                                 vec_store, out);
  return hipGetLastError();
}

}  // namespace qmm
