// Measured MFMA ceiling: a register-only loop of v_mfma_f32_32x32x16_bf16
// (the instruction every GEMM and attention kernel of the step uses), with
// operands taken from a caller buffer so that their bit patterns (and with
// them the switching power that sets the clock) are those of real data.
// Each wave keeps eight independent accumulator chains in flight and
// rotates through eight A and eight B fragments (64 MFMAs per iteration);
// no memory traffic inside the loop. ops: 64 wave slots x 16 fragments x 64
// lanes x 8 bf16 (1 MiB). The sum of the accumulators is written out so nothing is
// optimized away.
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

__global__ __launch_bounds__(256) void mfma_loop_kernel(const bf16_t* ops, float* out, int iters) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * 4 + (threadIdx.x >> 6)) & 63;
  // 16 fragments of 8 bf16 per lane: 16 * 64 * 8 values per wave slot
  const u32x4* src = reinterpret_cast<const u32x4*>(ops) + (size_t)wave * 16 * 64;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = __builtin_bit_cast(bf16x8, src[i * 64 + lane]);
    b[i] = __builtin_bit_cast(bf16x8, src[(8 + i) * 64 + lane]);
  }
  f32x16 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  // 64 MFMAs per iteration; the operand rotation is unrolled so every
  // register index is a compile-time constant
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = mfma32(a[(c + j) & 7], b[(c + 3 * j) & 7], acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_loop(const uint16_t* ops, float* out, int blocks, int iters, hipStream_t s) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, s, ops, out, iters);
  return hipGetLastError();
}

}  // namespace dit
