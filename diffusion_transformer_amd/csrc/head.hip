// The two ends of the step, each one kernel on bf16 MFMA:
//  - img_in: h[i] = W_in · x[i], one latent cell (C = 64 channels, fp32) to
//    one H-wide token (fp32);
//  - the scale-only final AdaLN and proj_out: v[i] = W_out · (LN(h[i]) ·
//    (1 + scale_out)), H -> 64, fp32 out.
// Both are dense contractions with K or N of only 64, so the work per byte
// is low and the MFMA cost small; what they are built for is moving their
// bytes at HBM speed.
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

// ---------------------------------------------------------------------------
// img_in. The latents are fp32 and the weights bf16. Each fp32 latent is cut
// into three bf16 pieces by truncation, x = hi + mid + lo exactly (8
// significant bits each), so three bf16 MFMAs per block give the fp32
// product sum with fp32 accumulation (each bf16 x bf16 product is exact in
// fp32). A workgroup of 4 waves computes 64 tokens x 256 columns; wave w the
// 64 x 64 patch at column 64w, as 2 x 2 blocks of 32 x 32, K = 64 in 4 steps
// of 16. Operands come straight from global memory (the 16 KB of latents of
// a workgroup and the 32 KB of weight rows are cache hits for all but the
// first wave that touches them).
__device__ __forceinline__ void split3(const float (&x)[8], bf16x8& hi, bf16x8& mid, bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t b = __float_as_uint(x[j]);
    const float h = __uint_as_float(b & 0xFFFF0000u);
    const float r1 = x[j] - h;                           // exact
    const float m = __uint_as_float(__float_as_uint(r1) & 0xFFFF0000u);
    const float r2 = r1 - m;                             // exact, <= 8 significant bits
    hi[j] = __builtin_bit_cast(__bf16, (uint16_t)(b >> 16));
    mid[j] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(r1) >> 16));
    lo[j] = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(r2) >> 16));
    (void)m;
  }
}

__global__ __launch_bounds__(256) void img_in_kernel(const uint16_t* __restrict__ W,
                                                     const float* __restrict__ x, int n,
                                                     float* __restrict__ out, int ldo) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, lh = lane >> 5;
  const int t0 = blockIdx.y * 64;
  const int c0 = blockIdx.x * 256 + wave * 64;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // B fragments: lane supplies W[c0 + 32j + l32][16s + 8lh .. +7]
  bf16x8 wb[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      wb[j][s] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(W + (size_t)(c0 + 32 * j + l32) * 64 + 16 * s + 8 * lh));
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = t0 + 32 * i + l32;
    const bool ok = t < n;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float xv[8];
      if (ok) {
        const float4* xp = reinterpret_cast<const float4*>(x + (size_t)t * 64 + 16 * s + 8 * lh);
        const float4 a = xp[0], b = xp[1];
        xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w;
        xv[4] = b.x; xv[5] = b.y; xv[6] = b.z; xv[7] = b.w;
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) xv[j] = 0.f;
      }
      bf16x8 hi, mid, lo;
      split3(xv, hi, mid, lo);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[i][j] = mfma32(lo, wb[j][s], acc[i][j]);
        acc[i][j] = mfma32(mid, wb[j][s], acc[i][j]);
        acc[i][j] = mfma32(hi, wb[j][s], acc[i][j]);
      }
    }
  }
  // register r of lane l: row 8(r/4) + 4lh + r%4 of the block, column l32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = t0 + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
      if (t < n) {
        float* op = out + (size_t)t * ldo + c0 + l32;
        op[0] = acc[i][0][r];
        op[32] = acc[i][1][r];
      }
    }
}

// ---------------------------------------------------------------------------
// Scale-only final AdaLN + proj_out. A workgroup of 4 waves owns 16 rows:
//  1. wave w normalizes rows 4w..4w+3 (each row in registers between the
//     mean and the variance pass, the next row's loads in flight), scales by
//     (1 + scale_out) and stores it as bf16 in LDS (16 rows x H, 16-byte
//     chunks XOR-swizzled by the row so the fragment reads are conflict
//     free);
//  2. wave w multiplies the 16 rows by W_out over its quarter of H with
//     32x32x16 MFMAs (rows 16..31 of the A block are zero), two 32-column
//     blocks, the weight fragments read from global memory (W_out is 0.5 MB
//     and stays in cache);
//  3. the four partial 16 x 64 results are summed through LDS and written.
constexpr int FO_ROWS = 16;
constexpr int FO_MAXV = 16;   // float4 per lane per row: H <= 4096

__global__ __launch_bounds__(256) void final_out_kernel(const float* __restrict__ h, int ldh, int rows,
                                                        int H, const float* __restrict__ scale,
                                                        float eps, const uint16_t* __restrict__ W,
                                                        float* __restrict__ v) {
  __shared__ __align__(16) unsigned char fo_smem[FO_ROWS * FO_MAXV * 256 * 2 + 4 * FO_ROWS * 64 * 4];
  unsigned char* ys = fo_smem;                                   // [16][H] bf16, swizzled
  float* part = reinterpret_cast<float*>(fo_smem + FO_ROWS * FO_MAXV * 256 * 2);   // [4][16][64]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = blockIdx.x * FO_ROWS;
  const int nv = H >> 2;            // float4 per row
  const int rowb = H * 2;           // LDS bytes per row

  float4 sc[FO_MAXV];
#pragma unroll
  for (int i = 0; i < FO_MAXV; ++i) {
    const int c = lane + 64 * i;
    sc[i] = c < nv ? reinterpret_cast<const float4*>(scale)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float4 cur[FO_MAXV], nxt[FO_MAXV];
  auto load = [&](float4 (&dst)[FO_MAXV], int row) {
    const float4* hp = reinterpret_cast<const float4*>(h + (size_t)row * ldh);
#pragma unroll
    for (int i = 0; i < FO_MAXV; ++i) {
      const int c = lane + 64 * i;
      dst[i] = (row < rows && c < nv) ? hp[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  load(cur, r0 + 4 * wave);
#pragma unroll 1
  for (int rr = 0; rr < 4; ++rr) {
    const int lr = 4 * wave + rr;                 // local row
    if (rr < 3) load(nxt, r0 + lr + 1);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < FO_MAXV; ++i) s += (cur[i].x + cur[i].y) + (cur[i].z + cur[i].w);
    const float mean = wave_sum(s) / (float)H;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < FO_MAXV; ++i) {
      if (lane + 64 * i < nv) {
        const float a = cur[i].x - mean, b = cur[i].y - mean, c = cur[i].z - mean, d = cur[i].w - mean;
        q += (a * a + b * b) + (c * c + d * d);
      }
    }
    const float rstd = rsqrtf(wave_sum(q) / (float)H + eps);
#pragma unroll
    for (int i = 0; i < FO_MAXV; ++i) {
      const int c4 = lane + 64 * i;                // columns 4c4 .. 4c4+3
      if (c4 < nv) {
        u32x2 w;
        w.x = pack2bf((cur[i].x - mean) * rstd * (1.f + sc[i].x), (cur[i].y - mean) * rstd * (1.f + sc[i].y));
        w.y = pack2bf((cur[i].z - mean) * rstd * (1.f + sc[i].z), (cur[i].w - mean) * rstd * (1.f + sc[i].w));
        const int chunk = (c4 >> 1) ^ (lr & 15);   // 16-byte chunk, swizzled by the row
        *reinterpret_cast<u32x2*>(ys + lr * rowb + chunk * 16 + (c4 & 1) * 8) = w;
      }
    }
    if (rr < 3) {
#pragma unroll
      for (int i = 0; i < FO_MAXV; ++i) cur[i] = nxt[i];
    }
  }
  __syncthreads();

  // out[16 x 64] partial over k in [kq * wave, kq * (wave + 1))
  const int kq = H >> 2;
  const int l32 = lane & 31, lh = lane >> 5;
  f32x16 acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  const bf16x8 zero8 = {};
  const uint16_t* w0 = W + (size_t)l32 * H + 8 * lh;
  const uint16_t* w1 = W + (size_t)(32 + l32) * H + 8 * lh;
#pragma unroll 4
  for (int k = wave * kq; k < (wave + 1) * kq; k += 16) {
    const bf16x8 b0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(w0 + k));
    const bf16x8 b1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(w1 + k));
    bf16x8 a = zero8;
    if (l32 < FO_ROWS) {
      const int chunk = ((k + 8 * lh) >> 3) ^ l32;
      a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ys + l32 * rowb + chunk * 16));
    }
    acc[0] = mfma32(a, b0, acc[0]);
    acc[1] = mfma32(a, b1, acc[1]);
  }
  // rows 0..15 of a block sit in registers r < 8 (row 8(r/4) + 4lh + r%4)
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = 8 * (r >> 2) + 4 * lh + (r & 3);
      part[(wave * FO_ROWS + row) * 64 + 32 * j + l32] = acc[j][r];
    }
  __syncthreads();
  const int row = threadIdx.x >> 4, c = (threadIdx.x & 15) * 4;
  if (r0 + row < rows) {
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) {
      const float4 p = *reinterpret_cast<const float4*>(part + (wv * FO_ROWS + row) * 64 + c);
      o.x += p.x; o.y += p.y; o.z += p.z; o.w += p.w;
    }
    *reinterpret_cast<float4*>(v + (size_t)(r0 + row) * 64 + c) = o;
  }
}

}  // namespace

hipError_t launch_img_in(const uint16_t* W, const float* x, int n, int H, float* out, int ldo,
                         hipStream_t s) {
  if (n <= 0) return hipSuccess;
  dim3 grid(H / 256, (n + 63) / 64);
  hipLaunchKernelGGL(img_in_kernel, grid, dim3(256), 0, s, W, x, n, out, ldo);
  return hipGetLastError();
}

hipError_t launch_final_out(const float* h, int ldh, int rows, int H, const float* scale, float eps,
                            const uint16_t* W, float* v, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(final_out_kernel, dim3((rows + FO_ROWS - 1) / FO_ROWS), dim3(256), 0, s, h, ldh,
                     rows, H, scale, eps, W, v);
  return hipGetLastError();
}

}  // namespace dit
