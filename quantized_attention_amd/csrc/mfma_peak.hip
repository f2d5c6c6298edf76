// mfma_peak.hip -- a roofline diagnostic: the dense MFMA rate the device
// sustains and the shader clock it runs at meanwhile.
//
// The SageAttention2 detail page judges its kernels against the tensor cores'
// theoretical peak and the fraction of it they reach (its utilization
// discussion of the INT4 kernel).  The published MI355X peak assumes 2.4 GHz;
// under a dense MFMA load the clock can settle lower, so the attention
// kernel's fraction is also worth stating against what a plain MFMA loop
// sustains, at the clock it sustains it.
//
// Every wave issues `iters` rounds of four independent MFMAs (four
// accumulators: no instruction waits on the one before it) on operands held
// in registers: no memory traffic and no VALU work beyond the loop counter.
//   kind 0: v_mfma_i32_32x32x32_i8, the instruction of S = Q K^T
//           (32*32*32*2 = 65536 ops); every operand byte is 1, so each
//           accumulator element ends at 32 * iters.
//   kind 1: the scaled FP8 32x32x64 MFMA of P V with unit scales
//           (131072 flops); every operand byte is 1.0 in E4M3, so each
//           element ends at 64 * iters (exact in float32 below 2^24).
// Each lane stores the sum of its 64 accumulator elements (as integers), so
// the caller can check that every MFMA ran; lane 0 of each wave stores the
// shader clocks (clock64) and the constant-rate clocks (wall_clock64) its
// loop took.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

typedef int i32x4p __attribute__((ext_vector_type(4)));
typedef int i32x8p __attribute__((ext_vector_type(8)));
typedef int i32x16p __attribute__((ext_vector_type(16)));
typedef float f32x16p __attribute__((ext_vector_type(16)));

template <int KIND>
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, long long* __restrict__ clocks,
                                                        uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x % 64;
  const long long wave = (long long)blockIdx.x * 4 + threadIdx.x / 64;
  uint32_t s = 0;
  long long c0, c1, w0, w1;
  if constexpr (KIND == 0) {
    const i32x4p a = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    i32x16p acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][r] = 0;
    c0 = clock64();
    w0 = wall_clock64();
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, acc[j], 0, 0, 0);
    }
    c1 = clock64();
    w1 = wall_clock64();
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += (uint32_t)acc[j][r];
  } else {
    const int one = 0x38383838;   // four E4M3 1.0 codes
    const i32x8p a = {one, one, one, one, one, one, one, one};
    f32x16p acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
    c0 = clock64();
    w0 = wall_clock64();
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, acc[j], 0, 0, 0, 127, 0, 127);
    }
    c1 = clock64();
    w1 = wall_clock64();
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += (uint32_t)acc[j][r];
  }
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
  if (lane == 0) {
    clocks[2 * wave] = c1 - c0;
    clocks[2 * wave + 1] = w1 - w0;
  }
}

}  // namespace sage

hipError_t sage_launch_mfma_peak(int kind, int iters, int nwg, long long* clocks, uint32_t* sink,
                                 hipStream_t st) {
  using namespace sage;
  if (kind == 0)
    hipLaunchKernelGGL((mfma_peak_kernel<0>), dim3(nwg), dim3(256), 0, st, iters, clocks, sink);
  else if (kind == 1)
    hipLaunchKernelGGL((mfma_peak_kernel<1>), dim3(nwg), dim3(256), 0, st, iters, clocks, sink);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}
