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
//           per chunk and element, subtract the accumulator bias from the block
//           dot (v_add_f32 with a literal) and multiply by the element's own f32
//           scale product and accumulate (v_fmac_f32); per super-block and
//           element, two more FMAs (apply d, add the min term times -dmin) --
//           2.25 instructions per (token, row, 32-block), on 16 elements per lane.
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
        inner[i] = fmaf(inner[i] - c0, sc[i], inner[i]);
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

}  // namespace

// Launches `grid` work-groups of 256 threads of calibration kernel `kind`
// (0: int8 MFMA, 1: q6_K scale epilogue, 2: q4_K scale epilogue) for `iters`
// iterations on `stream`.
// clk: device uint64[2] (shader clocks, 100 MHz ticks of work-group 0's first
// wave); sink: device int32[grid * 256].  Each iteration is, per wave, 4 MFMAs
// of 32x32x32 (kind 0), 16 epilogue elements per lane (kind 1) or 8 chunks of
// 16 epilogue elements per lane (kind 2): 262144, 65536 or 524288
// int8-equivalent operations.  Returns 0 or the hipError_t of the launch.
extern "C" int qmm_peak_launch(int kind, int iters, int grid, void* clk, void* sink, void* stream) {
  if (kind < 0 || kind > 2 || iters < 1 || grid < 1 || !clk || !sink) return (int)hipErrorInvalidValue;
  hipStream_t s = (hipStream_t)stream;
  if (kind == 0)
    peak_mfma_i8<<<dim3((unsigned)grid), dim3(256), 0, s>>>(iters, (unsigned long long*)clk, (int*)sink);
  else if (kind == 1)
    peak_epilogue<<<dim3((unsigned)grid), dim3(256), 0, s>>>(iters, (unsigned long long*)clk, (int*)sink);
  else
    peak_epilogue_q4<<<dim3((unsigned)grid), dim3(256), 0, s>>>(iters, (unsigned long long*)clk, (int*)sink);
  return (int)hipGetLastError();
}
