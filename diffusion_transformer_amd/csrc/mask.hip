// Materializes the block-causal visibility exactly as the attention kernels
// apply it (test hook behind dit_debug_mask): per 128-query workgroup and
// 64-key tile, the same per-wave tile classification (skip / full /
// per-element) and the same row-limit predicate from common.h.
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int BQ = 128;
constexpr int BKV = 64;
constexpr int NT = 256;

__global__ __launch_bounds__(NT) void mask_kernel(const int32_t* limit, int S, uint8_t* mask) {
  __shared__ int red[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q_blk = blockIdx.x * BQ;
  const int lq = lane & 31, half = lane >> 5;
  const int qi = min(q_blk + wave * 32 + lq, S - 1);
  const bool q_valid = q_blk + wave * 32 + lq < S;
  const int lim = limit[qi];
  const int wlim_min = wave_min_i(lim), wlim_max = wave_max_i(lim);
  if (lane == 0) red[wave] = wlim_max;
  __syncthreads();
  const int blim_max = max(max(red[0], red[1]), max(red[2], red[3]));
  const int kv_end = min(S, blim_max + 1);
  const int kv0 = blockIdx.y * BKV;
  const bool loaded = kv0 < kv_end;
  const int cls = loaded ? tile_class<BKV>(kv0, wlim_min, wlim_max, S) : 0;
  if (!q_valid) return;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = kv0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (j >= S) continue;
      uint8_t vis = 0;
      if (cls == 1) vis = 1;
      else if (cls == 2) vis = key_visible(j, lim, S) ? 1 : 0;
      mask[(size_t)qi * S + j] = vis;
    }
}

}  // namespace

hipError_t launch_debug_mask(const int32_t* limit, int S, uint8_t* mask, hipStream_t s) {
  dim3 grid((S + BQ - 1) / BQ, (S + BKV - 1) / BKV);
  hipLaunchKernelGGL(mask_kernel, grid, dim3(NT), 0, s, limit, S, mask);
  return hipGetLastError();
}

}  // namespace dit
