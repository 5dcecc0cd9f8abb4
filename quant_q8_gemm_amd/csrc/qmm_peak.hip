// qmm_peak.hip -- calibration kernels for the rooflines that the benchmark
// reports next to the MMQ: the rate this GPU reaches on
//   kind 0: the int8 matrix core, back-to-back v_mfma_i32_32x32x32_i8 with
//           four independent accumulators per wave (no memory traffic);
//   kind 1: the vector ALU running the q6_K MMQ's per-block scale epilogue,
//           the same three instructions per (token, row, 32-block) -- combine
//           the two plane dots (v_lshl_add_u32), convert (v_cvt_f32_i32), scale
//           and accumulate with the activation scale held as f32 (v_fmac_f32)
//           -- on 16 elements per lane;
//   kind 2: the q4_K MMQ's epilogue over one 256-wide super-block (8 chunks):
//           per chunk and element, subtract the block dot from the accumulator
//           bias (v_sub_f32 with the bias as an inline constant), multiply the
//           negated difference by the element's own f32 scale product and
//           accumulate (v_fma_f32 with a negated operand); per super-block and
//           element, two more FMAs (apply d, add the min term times -dmin) --
//           2.25 instructions per (token, row, 32-block), on 16 elements per lane;
//   kind 3: the q4_K MMQ's whole chunk step without its memory traffic: the
//           MFMAs (the biased int8 block dot, the f16 scale outer product, per
//           super-block the f16 min term), the LDS reads of the operands and
//           the vector epilogue, software-pipelined as in the MMQ, over
//           LDS-resident operands, with no global copies and no barriers;
//   kind 4: the same for q6_K (two int8 plane dots, the three-instruction
//           epilogue, d per super-block);
//   kind 5: four independent int8 MFMAs and 64 independent v_fma_f32 per
//           iteration, and kind 6: the 64 FMAs alone -- with kind 0, whether
//           the matrix core and the vector ALU overlap (kind 5 near kind 0's
//           time) or add (near the sum of kinds 0 and 6).
// Work-group 0's first wave also records the shader clock (s_memtime) and the
// 100 MHz constant clock (s_memrealtime) across its run, so the caller can
// state the clock the rates were measured at.  These kernels are measurement
// infrastructure for the benchmark; they are not part of the libqmm ABI.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ void clock_start(uint64_t& t, uint64_t& r) {
  t = __builtin_amdgcn_s_memtime();
  r = __builtin_amdgcn_s_memrealtime();
}

__device__ __forceinline__ void clock_end(uint64_t t, uint64_t r, unsigned long long* clk) {
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clk[0] = t1 - t;
    clk[1] = r1 - r;
  }
}

__global__ void __launch_bounds__(256) peak_mfma_i8(int iters, unsigned long long* clk, int* sink) {
  const int lane = threadIdx.x & 63;
  const v4i a = {lane, lane * 3, lane * 5, lane * 7};
  const v4i b = {lane ^ 1, lane ^ 2, lane ^ 3, lane ^ 4};
  v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
  uint64_t t = 0, r = 0;
  clock_start(t, r);
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
  }
  clock_end(t, r, clk);
  int s = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] ^ c1[i] ^ c2[i] ^ c3[i];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ void __launch_bounds__(256) peak_epilogue(int iters, unsigned long long* clk, int* sink) {
  const int lane = threadIdx.x & 63;
  uint32_t hi[16], lo[16];
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    hi[i] = (uint32_t)(lane + i);
    lo[i] = (uint32_t)(lane * (i + 1));
    acc[i] = 0.0f;
  }
  const _Float16 dh = (_Float16)(1.0f / (float)(lane + 1));
  uint64_t t = 0, r = 0;
  clock_start(t, r);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      hi[i] = (hi[i] << 6) + lo[i];
      acc[i] = fmaf((float)(int)hi[i], (float)dh, acc[i]);
    }
  }
  clock_end(t, r, clk);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += acc[i];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = __builtin_bit_cast(int, s);
}

__global__ void __launch_bounds__(256) peak_epilogue_q4(int iters, unsigned long long* clk, int* sink) {
  const int lane = threadIdx.x & 63;
  float acc[16], inner[16], sc[16], d[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    acc[i] = 0.0f;
    inner[i] = (float)(lane + i);
    sc[i] = 0x1p-40f * (float)(lane + i + 1);  // in registers, as in the MMQ; keeps the values finite
    d[i] = 0x1p-20f * (float)(i + 1);
  }
  const float c0 = 0.15915494f;
  uint64_t t = 0, r = 0;
  clock_start(t, r);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
      for (int i = 0; i < 16; ++i)  // the "block dot" is inner's own value: it changes every step
        inner[i] = fmaf(-(c0 - inner[i]), sc[i], inner[i]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc[i] = fmaf(inner[i], d[i], acc[i]);
      acc[i] = fmaf(acc[i], sc[i], acc[i]);
    }
  }
  clock_end(t, r, clk);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += acc[i] + inner[i];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = __builtin_bit_cast(int, s);
}


constexpr uint32_t kBiasBits = 0x3E22F983u;  // 1/(2 pi): the q4_K MMQ's accumulator bias

template <class T>
__device__ __forceinline__ void pin(T& v) {
  asm volatile("" : "+v"(v));
}

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

// Operands of one chunk step as the MMQ holds them: the weight fragment(s)
// (q6_K: hi and lo planes), the activation fragment, and the block dots.
template <bool Q6>
struct ChunkOps {
  v4i a, a2;
  v16i d, d2;
};

// LDS image of one stage of four chunks for one wave (the MMQ's stage, less
// what other waves own): weight fragments [chunk][plane][1 KiB], activation
// fragments [chunk][1 KiB], (dh, s) pairs [chunk][32], the 4 scales [32][4]
// f16, the mins [2][32][4] f16, d and -dmin [2][32] f32.
struct alignas(16) CalStage {
  int8_t a[4][2][1024];
  int8_t b[4][1024];
  uint32_t s[4][32];
  uint16_t sc[32][4];
  uint16_t mn[2][32][4];
  float d[2][32];
};

// kind 3 (Q6 = false) and kind 4 (Q6 = true).  256 threads = 4 waves reading
// two shared stages (2 x 13.5 KiB of LDS, four work-groups per CU as in the
// q4_K MMQ), filled once; every iteration is one super-block: two stages of
// four chunk steps.
template <bool Q6>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4)))
peak_chunk(int iters, unsigned long long* clk, int* sink) {
  __shared__ CalStage st2[2];
  const int lane = threadIdx.x & 63;
  // codes 0..15 (q4_K) or -64..63 / 0..63 (q6_K), activations -64..63, dh = 1/64,
  // scales 1..4, d = 2^-20: finite values that change the sums every step
  const int tid = threadIdx.x;
  for (int b = 0; b < 2; ++b) {
    for (int i = tid; i < 2048; i += 256) ((uint32_t*)&st2[b].a[0][0][0])[i] = (i * 2654435761u) & 0x0F0F0F0Fu;
    for (int i = tid; i < 1024; i += 256) ((uint32_t*)&st2[b].b[0][0])[i] = (i * 40503u) & 0x3F3F3F3Fu;
    for (int i = tid; i < 128; i += 256) ((uint32_t*)&st2[b].s[0][0])[i] = 0x20002400u;  // dh = 2^-6, s = 2^-7
    for (int i = tid; i < 128; i += 256) ((uint16_t*)&st2[b].sc[0][0])[i] = (uint16_t)(0x3C00u + ((i & 3) << 10));
    for (int i = tid; i < 256; i += 256) ((uint16_t*)&st2[b].mn[0][0][0])[i] = 0x3C00u;
    for (int i = tid; i < 64; i += 256) ((float*)&st2[b].d[0][0])[i] = 0x1p-20f;
  }
  __syncthreads();
  v16f acc, inner;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    acc[i] = 0.0f;
    inner[i] = 0.0f;
  }
  v2i bs = {0, 0};
  uint64_t t = 0, r = 0;
  clock_start(t, r);
  auto mma = [&](const v4i& a, const v4i& a2, const v4i& bq) __attribute__((always_inline)) {
    ChunkOps<Q6> o;
    if constexpr (Q6) {
      const v16i z = {};
      o.d = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bq, z, 0, 0, 0);
      o.d2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a2, bq, z, 0, 0, 0);
    } else {  // the bias as the instruction's inline constant: the MFMA ends its block (see the MMQ)
      const v16i bias = (v16i)(int)kBiasBits;
      o.d = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bq, bias, 0, 0, 0);
      asm goto("" :::: block_end);
    block_end:;
    }
    return o;
  };
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const CalStage& st = st2[h];
      uint32_t dhr = st.s[0][lane & 31];
      v2i a_sc = {}, amin = {};
      if constexpr (!Q6) {
        if (h == 1) amin = *(const v2i*)(&st.mn[lane >> 5][lane & 31][0]);
        a_sc = *(const v2i*)(&st.sc[lane & 31][0]);
      }
      v4i a0 = *(const v4i*)(st.a[0][0] + lane * 16), a0b = {};
      if constexpr (Q6) a0b = *(const v4i*)(st.a[0][1] + lane * 16);
      v4i bq0 = *(const v4i*)(st.b[0] + lane * 16);
      v4i a1 = *(const v4i*)(st.a[1][0] + lane * 16), a1b = {};
      if constexpr (Q6) a1b = *(const v4i*)(st.a[1][1] + lane * 16);
      v4i bq1 = *(const v4i*)(st.b[1] + lane * 16);
      ChunkOps<Q6> dj = mma(a0, a0b, bq0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        v16f sd;
        float dh = 0.0f;
        if constexpr (!Q6) {
          const uint32_t y = __builtin_amdgcn_perm(0u, dhr, cc % 2 == 0 ? 0x0C0C0100u : 0x01000C0Cu);
          const v2i bb = {cc < 2 ? (int)y : 0, cc < 2 ? 0 : (int)y};
          const v16f zero = {};
          sd = __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(v4h, a_sc), __builtin_bit_cast(v4h, bb), zero,
                                                    0, 0, 0);
          pin(sd);
        }
        ChunkOps<Q6> dj_next;
        if (cc + 1 < 4) {
          dj_next = mma(a1, a1b, bq1);
          pin(dj_next.d);
          if constexpr (Q6) pin(dj_next.d2);
        }
        v4i a2 = {}, a2b = {}, bq2 = {};
        if (cc + 2 < 4) {
          a2 = *(const v4i*)(st.a[cc + 2][0] + lane * 16);
          if constexpr (Q6) a2b = *(const v4i*)(st.a[cc + 2][1] + lane * 16);
          bq2 = *(const v4i*)(st.b[cc + 2] + lane * 16);
        }
        uint32_t dhr_next = 0;
        if (cc + 1 < 4) dhr_next = st.s[cc + 1][lane & 31];
        if constexpr (!Q6) {
          if ((cc & 1) && (lane >= 32) == (h == 1)) bs[cc >> 1] = (int)__builtin_amdgcn_perm(dhr, dhr_next, 0x07060302u);
        } else {
          dh = (float)__builtin_bit_cast(_Float16, (uint16_t)(dhr & 0xFFFF));
          pin(dh);
        }
        const v16f df = __builtin_bit_cast(v16f, dj.d);
        if (cc == 0 && h == 0) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            if constexpr (Q6) inner[i] = (float)((dj.d[i] << 6) + dj.d2[i]) * dh;
            else inner[i] = -(__builtin_bit_cast(float, kBiasBits) - df[i]) * sd[i];
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            if constexpr (Q6) inner[i] = fmaf((float)((dj.d[i] << 6) + dj.d2[i]), dh, inner[i]);
            else inner[i] = fmaf(-(__builtin_bit_cast(float, kBiasBits) - df[i]), sd[i], inner[i]);
          }
        }
        pin(inner);
        if (cc + 1 < 4) {
          dj = dj_next;
          a1 = a2;
          a1b = a2b;
          bq1 = bq2;
          dhr = dhr_next;
        }
        __builtin_amdgcn_sched_group_barrier(0x008, Q6 ? 2 : 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 72, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (h == 1) {  // end of the super-block
        v16f mt = {};
        if constexpr (!Q6) {
          const v16f zero = {};
          mt = __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(v4h, amin), __builtin_bit_cast(v4h, bs), zero,
                                                    0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 d4 = *(const float4*)(&st.d[0][8 * q + 4 * (lane >> 5)]);
          acc[4 * q + 0] = fmaf(inner[4 * q + 0], d4.x, acc[4 * q + 0]);
          acc[4 * q + 1] = fmaf(inner[4 * q + 1], d4.y, acc[4 * q + 1]);
          acc[4 * q + 2] = fmaf(inner[4 * q + 2], d4.z, acc[4 * q + 2]);
          acc[4 * q + 3] = fmaf(inner[4 * q + 3], d4.w, acc[4 * q + 3]);
          if constexpr (!Q6) {
            const float4 m4 = *(const float4*)(&st.d[1][8 * q + 4 * (lane >> 5)]);
            acc[4 * q + 0] = fmaf(mt[4 * q + 0], m4.x, acc[4 * q + 0]);
            acc[4 * q + 1] = fmaf(mt[4 * q + 1], m4.y, acc[4 * q + 1]);
            acc[4 * q + 2] = fmaf(mt[4 * q + 2], m4.z, acc[4 * q + 2]);
            acc[4 * q + 3] = fmaf(mt[4 * q + 3], m4.w, acc[4 * q + 3]);
          }
        }
      }
    }
  }
  clock_end(t, r, clk);
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) sum += acc[i];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = __builtin_bit_cast(int, sum);
}

// kind 5 (WITH_MFMA) and kind 6: per iteration four independent int8 MFMAs
// (as kind 0) and 64 v_fma_f32 on 16 registers that the MFMAs do not touch.
template <bool WITH_MFMA>
__global__ void __launch_bounds__(256) peak_overlap(int iters, unsigned long long* clk, int* sink) {
  const int lane = threadIdx.x & 63;
  const v4i a = {lane, lane * 3, lane * 5, lane * 7};
  const v4i b = {lane ^ 1, lane ^ 2, lane ^ 3, lane ^ 4};
  v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = (float)(lane + i);
  const float m = 0.999f + 1e-6f * (float)lane;
  uint64_t t = 0, r = 0;
  clock_start(t, r);
  for (int it = 0; it < iters; ++it) {
    if constexpr (WITH_MFMA) {
      c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
    }
#pragma unroll
    for (int rep = 0; rep < 4; ++rep)
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = fmaf(x[i], m, 0.5f);
  }
  clock_end(t, r, clk);
  int s = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += (c0[i] ^ c1[i] ^ c2[i] ^ c3[i]) + __builtin_bit_cast(int, x[i]);
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

// Launches `grid` work-groups of 256 threads of calibration kernel `kind`
// (0: int8 MFMA, 1: q6_K scale epilogue, 2: q4_K scale epilogue, 3: q4_K chunk
// step, 4: q6_K chunk step, 5: MFMAs with independent FMAs, 6: the FMAs alone)
// for `iters` iterations on `stream`.
// clk: device uint64[2] (shader clocks, 100 MHz ticks of work-group 0's first
// wave); sink: device int32[grid * 256].  Each iteration is, per wave, 4 MFMAs
// of 32x32x32 (kinds 0 and 5), 16 epilogue elements per lane (kind 1), 8
// chunks of 16 epilogue elements per lane (kind 2), one super-block of 8 chunk
// steps of a 32 x 32 block (kinds 3 and 4), or 64 FMAs (kinds 5 and 6):
// 262144, 65536, 524288, 524288, 524288, 262144 or 0 int8-equivalent
// operations.  Returns 0 or the hipError_t of the launch.
extern "C" int qmm_peak_launch(int kind, int iters, int grid, void* clk, void* sink, void* stream) {
  if (kind < 0 || kind > 6 || iters < 1 || grid < 1 || !clk || !sink) return (int)hipErrorInvalidValue;
  hipStream_t s = (hipStream_t)stream;
  unsigned long long* c = (unsigned long long*)clk;
  int* k = (int*)sink;
  const dim3 g((unsigned)grid), b(256);
  switch (kind) {
    case 0: peak_mfma_i8<<<g, b, 0, s>>>(iters, c, k); break;
    case 1: peak_epilogue<<<g, b, 0, s>>>(iters, c, k); break;
    case 2: peak_epilogue_q4<<<g, b, 0, s>>>(iters, c, k); break;
    case 3: peak_chunk<false><<<g, b, 0, s>>>(iters, c, k); break;
    case 4: peak_chunk<true><<<g, b, 0, s>>>(iters, c, k); break;
    case 5: peak_overlap<true><<<g, b, 0, s>>>(iters, c, k); break;
    default: peak_overlap<false><<<g, b, 0, s>>>(iters, c, k); break;
  }
  return (int)hipGetLastError();
}
