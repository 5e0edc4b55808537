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
// fp32). The kernel is bound by writing its fp32 output. A workgroup of 4
// waves takes 64 tokens and IMG_CB blocks of 256 columns:
//  1. its 256 threads split the 64 x 64 latents once into three bf16 tiles
//     in LDS (128-byte token rows, 16-byte chunks XOR-swizzled by token%8);
//  2. for each 256-column block, wave w computes the 64 x 64 patch at
//     column 64w as two 32-token halves of 2 x 2 blocks of 32 x 32 (K = 64
//     in 4 steps of 16; A fragments from LDS, W fragments from global memory
//     (cache hits after the first wave), the next block's fetched while the
//     current one is multiplied), and writes each half row by row through
//     LDS; the stores of one half drain while the next half is computed.
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
  }
}

constexpr int IMG_LD = 68;   // floats per staged row (64 + 4 of padding)
constexpr int IMG_CB = 2;    // 256-column blocks per workgroup

__global__ __launch_bounds__(256) void img_in_kernel(const uint16_t* __restrict__ W,
                                                     const float* __restrict__ x, int n, int H,
                                                     float* __restrict__ out, int ldo) {
  __shared__ __align__(16) u32x4 img_split[3][64 * 8];       // [piece][token][chunk]: 24 KB
  __shared__ __align__(16) float img_smem[4 * 32 * IMG_LD];  // per-wave output staging: 34 KB
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, lh = lane >> 5;
  const int t0 = blockIdx.y * 64;
  const int ncb = H >> 8;
  const int cb0 = blockIdx.x * IMG_CB;

  // W fragments of a 256-column block: lane supplies W[c0 + 32j + l32][16s + 8lh .. +7]
  auto fetch_w = [&](bf16x8 (&wb)[2][4], int cb) {
    const int c0 = cb * 256 + wave * 64;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        wb[j][s] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(W + (size_t)(c0 + 32 * j + l32) * 64 + 16 * s + 8 * lh));
  };
  bf16x8 wa[2][4], wbn[2][4];
  fetch_w(wa, cb0);

  // 1. split: thread tid takes token tid/4, channels 16(tid%4) .. +15
  {
    const int tk = tid >> 2, ch0 = 16 * (tid & 3);
    const int t = t0 + tk;
    float v[16];
    if (t < n) {
      const float4* xp = reinterpret_cast<const float4*>(x + (size_t)t * 64 + ch0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 a = xp[q];
        v[4 * q] = a.x; v[4 * q + 1] = a.y; v[4 * q + 2] = a.z; v[4 * q + 3] = a.w;
      }
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = 0.f;
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      float xv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) xv[k] = v[8 * g + k];
      bf16x8 hi, mid, lo;
      split3(xv, hi, mid, lo);
      const int slot = tk * 8 + (((ch0 >> 3) + g) ^ (tk & 7));
      img_split[0][slot] = __builtin_bit_cast(u32x4, hi);
      img_split[1][slot] = __builtin_bit_cast(u32x4, mid);
      img_split[2][slot] = __builtin_bit_cast(u32x4, lo);
    }
  }
  __syncthreads();

  float* pt = img_smem + wave * 32 * IMG_LD;
  for (int cbi = 0; cbi < IMG_CB; ++cbi) {
    const int cb = cb0 + cbi;
    if (cb >= ncb) break;                               // workgroup-uniform
    const bool more = cbi + 1 < IMG_CB && cb + 1 < ncb;
    if (more) fetch_w(cbi & 1 ? wa : wbn, cb + 1);
    const bf16x8 (&wb)[2][4] = cbi & 1 ? wbn : wa;
    const int c0 = cb * 256 + wave * 64;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      f32x16 acc[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
      const int tk = 32 * i + l32;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int slot = tk * 8 + ((2 * s + lh) ^ (tk & 7));
        const bf16x8 hi = __builtin_bit_cast(bf16x8, img_split[0][slot]);
        const bf16x8 mid = __builtin_bit_cast(bf16x8, img_split[1][slot]);
        const bf16x8 lo = __builtin_bit_cast(bf16x8, img_split[2][slot]);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[j] = mfma32(lo, wb[j][s], acc[j]);
          acc[j] = mfma32(mid, wb[j][s], acc[j]);
          acc[j] = mfma32(hi, wb[j][s], acc[j]);
        }
      }
      // Register r of lane l holds row 8(r/4) + 4lh + r%4 of its block,
      // column l32. The wave's 32 x 64 half goes through LDS (rows padded to
      // 272 bytes) so that every store instruction writes four whole 256-byte
      // row segments.
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // the previous half's LDS reads are done
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          pt[(8 * (r >> 2) + 4 * lh + (r & 3)) * IMG_LD + 32 * j + l32] = acc[j][r];
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // the region is private to this wave
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int row = 4 * it + (lane >> 4);
        const int tr = t0 + 32 * i + row;
        const float4 v4 = *reinterpret_cast<const float4*>(pt + row * IMG_LD + 4 * (lane & 15));
        if (tr < n) *reinterpret_cast<float4*>(out + (size_t)tr * ldo + c0 + 4 * (lane & 15)) = v4;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Scale-only final AdaLN + proj_out. A workgroup of 4 waves owns 16 rows:
//  1. wave w normalizes rows 4w..4w+3 (each row in registers between the
//     mean and the variance pass, two rows' loads in flight), scales by
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

// HC: the width when known at compile time (4096, the production width: all
// the guards below fold away), 0 for any other supported width.
template <int HC>
__global__ __launch_bounds__(256) void final_out_kernel(const float* __restrict__ h, int ldh, int rows,
                                                        int H_, const float* __restrict__ scale,
                                                        float eps, const uint16_t* __restrict__ W,
                                                        float* __restrict__ v) {
  const int H = HC ? HC : H_;
  __shared__ __align__(16) unsigned char fo_smem[FO_ROWS * FO_MAXV * 256 * 2 + 4 * FO_ROWS * 64 * 4];
  unsigned char* ys = fo_smem;                                   // [16][H] bf16, swizzled
  float* part = reinterpret_cast<float*>(fo_smem + FO_ROWS * FO_MAXV * 256 * 2);   // [4][16][64]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = blockIdx.x * FO_ROWS;
  const int nv = H >> 2;            // float4 per row
  const int rowb = H * 2;           // LDS bytes per row
  constexpr uint32_t kOut = 0x80000000u;   // an offset past every resource: loads return 0

  // Every global load is a buffer load whose resource ends at the data's
  // end, so rows past `rows`, columns past H and K past this wave's range
  // read as zero without a branch.
  const __amdgpu_buffer_rsrc_t rh =
      make_rsrc(h + (size_t)r0 * ldh, (uint32_t)((size_t)min(rows - r0, FO_ROWS) * ldh * 4));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W, (uint32_t)(64u * (uint32_t)H * 2u));

  // W_out fragments of this wave's quarter of H, 16 K-steps (256 columns of
  // W) per chunk and two chunks in registers: the first is fetched before
  // the LayerNorm so its latency hides behind it, each next one while the
  // current one is multiplied.
  const int kq = H >> 2;
  const int kb = wave * kq, ke = kb + kq;
  const int l32 = lane & 31, lh = lane >> 5;
  const uint32_t wo0 = (uint32_t)(l32 * H + 8 * lh) * 2u, wo1 = (uint32_t)((32 + l32) * H + 8 * lh) * 2u;
  u32x4 bw0[2][16], bw1[2][16];
  auto fetch = [&](u32x4 (&b)[2][16], int k0) {
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int k = k0 + 16 * st;
      const bool in = k < ke;
      b[0][st] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, in ? wo0 + 2u * k : kOut, 0, 0));
      b[1][st] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, in ? wo1 + 2u * k : kOut, 0, 0));
    }
  };
  fetch(bw0, kb);
  __builtin_amdgcn_sched_barrier(0);

  float4 sc[FO_MAXV];
#pragma unroll
  for (int i = 0; i < FO_MAXV; ++i) {
    const int c = lane + 64 * i;
    sc[i] = c < nv ? reinterpret_cast<const float4*>(scale)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float4 ra[FO_MAXV], rb[FO_MAXV];
  auto load = [&](float4 (&dst)[FO_MAXV], int lr) {      // local row lr of this workgroup
#pragma unroll
    for (int i = 0; i < FO_MAXV; ++i) {
      const int c = lane + 64 * i;
      const uint32_t off = c < nv ? (uint32_t)(lr * ldh + 4 * c) * 4u : kOut;
      dst[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rh, off, 0, 0));
    }
  };
  auto norm_store = [&](const float4 (&x)[FO_MAXV], int lr) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < FO_MAXV; ++i) s += (x[i].x + x[i].y) + (x[i].z + x[i].w);
    const float mean = wave_sum(s) / (float)H;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < FO_MAXV; ++i) {
      const float m = lane + 64 * i < nv ? 1.f : 0.f;     // columns past H add nothing
      const float a = x[i].x - mean, b = x[i].y - mean, c = x[i].z - mean, d = x[i].w - mean;
      q += m * ((a * a + b * b) + (c * c + d * d));
    }
    const float rstd = rsqrtf(wave_sum(q) / (float)H + eps);
#pragma unroll
    for (int i = 0; i < FO_MAXV; ++i) {
      const int c4 = lane + 64 * i;                // columns 4c4 .. 4c4+3
      if (c4 < nv) {
        u32x2 w;
        w.x = pack2bf((x[i].x - mean) * rstd * (1.f + sc[i].x), (x[i].y - mean) * rstd * (1.f + sc[i].y));
        w.y = pack2bf((x[i].z - mean) * rstd * (1.f + sc[i].z), (x[i].w - mean) * rstd * (1.f + sc[i].w));
        const int chunk = (c4 >> 1) ^ (lr & 15);   // 16-byte chunk, swizzled by the row
        *reinterpret_cast<u32x2*>(ys + lr * rowb + chunk * 16 + (c4 & 1) * 8) = w;
      }
    }
  };
  // wave w: rows 4w .. 4w+3, two row buffers in turn. The scheduling
  // barriers keep each batch of loads where it is issued (ahead of the
  // arithmetic that hides it) instead of letting the compiler sink it.
  load(ra, 4 * wave);
  load(rb, 4 * wave + 1);
  __builtin_amdgcn_sched_barrier(0);
  norm_store(ra, 4 * wave);
  __builtin_amdgcn_sched_barrier(0);
  load(ra, 4 * wave + 2);
  __builtin_amdgcn_sched_barrier(0);
  norm_store(rb, 4 * wave + 1);
  __builtin_amdgcn_sched_barrier(0);
  load(rb, 4 * wave + 3);
  __builtin_amdgcn_sched_barrier(0);
  norm_store(ra, 4 * wave + 2);
  norm_store(rb, 4 * wave + 3);
  __syncthreads();

  // out[16 x 64] partial over k in [kb, ke)
  f32x16 acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  const int arow = l32 & 15;                       // lanes 16..31 read a row and zero it
  const bool areal = l32 < FO_ROWS;
  const int nsteps = kq >> 4;                      // 16-wide K steps of this wave
  auto compute = [&](const u32x4 (&b)[2][16], int c) {
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      if (16 * c + st < nsteps) {                  // wave-uniform
        const int k = kb + 16 * (16 * c + st);
        const int chunk = ((k + 8 * lh) >> 3) ^ arow;
        u32x4 av = *reinterpret_cast<const u32x4*>(ys + arow * rowb + chunk * 16);
        av = areal ? av : (u32x4){0u, 0u, 0u, 0u};
        const bf16x8 a = __builtin_bit_cast(bf16x8, av);
        acc[0] = mfma32(a, __builtin_bit_cast(bf16x8, b[0][st]), acc[0]);
        acc[1] = mfma32(a, __builtin_bit_cast(bf16x8, b[1][st]), acc[1]);
      }
    }
  };
  // kq <= 1024: at most 4 chunks of 16 steps
  if (nsteps > 16) fetch(bw1, kb + 256);
  __builtin_amdgcn_sched_barrier(0);
  compute(bw0, 0);
  if (nsteps > 16) {
    if (nsteps > 32) fetch(bw0, kb + 512);
    __builtin_amdgcn_sched_barrier(0);
    compute(bw1, 1);
  }
  if (nsteps > 32) {
    if (nsteps > 48) fetch(bw1, kb + 768);
    __builtin_amdgcn_sched_barrier(0);
    compute(bw0, 2);
  }
  if (nsteps > 48) compute(bw1, 3);
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
                         hipStream_t s, const LaunchEvents& ev) {
  if (n <= 0) {
    mark_empty(ev, s);
    return hipSuccess;
  }
  dim3 grid((H / 256 + IMG_CB - 1) / IMG_CB, (n + 63) / 64);
  launch_k(img_in_kernel, grid, dim3(256), s, ev.start, ev.stop, W, x, n, H, out, ldo);
  return hipGetLastError();
}

hipError_t launch_final_out(const float* h, int ldh, int rows, int H, const float* scale, float eps,
                            const uint16_t* W, float* v, hipStream_t s, const LaunchEvents& ev) {
  if (rows <= 0) {
    mark_empty(ev, s);
    return hipSuccess;
  }
  const dim3 grid((rows + FO_ROWS - 1) / FO_ROWS);
  if (H == 4096)
    launch_k(final_out_kernel<4096>, grid, dim3(256), s, ev.start, ev.stop, h, ldh, rows, H, scale, eps, W, v);
  else
    launch_k(final_out_kernel<0>, grid, dim3(256), s, ev.start, ev.stop, h, ldh, rows, H, scale, eps, W, v);
  return hipGetLastError();
}

}  // namespace dit
