// fp32 debug build (compiled only with -DDIT_F32 into libdit_f32.so): the
// step's GEMMs and attention as plain fp32 FMA kernels, so the whole step
// carries fp32 activations (weights stay bf16) and can be compared with the
// fp64 oracle at fp32 tolerance. Same entry points and orchestration as the
// production library; speed is not a goal here.
#include "common.h"
#include "kernels.h"

#ifndef DIT_F32
#error "debug_f32.hip is part of the fp32 debug build only"
#endif

namespace dit {

namespace {

// C[M,N] (or SwiGLU of two products) = A[M,K] (f32) · B[N,K]ᵀ (bf16).
// 64x64 output tile, 256 threads, 4x4 outputs per thread, K in chunks of 16.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g, int Nout) {
  constexpr int T = 64, KC = 16;
  constexpr bool SW = EPI == EPI_SWIGLU;
  __shared__ float As[KC][T + 1], Bs[KC][T + 1], Us[KC][T + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * T, n0 = blockIdx.x * T;
  float acc[4][4] = {}, accu[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += KC) {
    for (int q = threadIdx.x; q < T * KC; q += 256) {
      const int r = q / KC, c = q % KC;
      const int m = m0 + r, n = n0 + r;
      As[c][r] = m < g.M ? g.A[(size_t)m * g.lda + k0 + c] : 0.f;
      Bs[c][r] = bf2f(g.B[(size_t)n * g.ldb + k0 + c]);
      if (SW) Us[c][r] = bf2f(g.B2[(size_t)n * g.ldb + k0 + c]);
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      float a[4], b[4], u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[c][ty * 4 + i]; b[i] = Bs[c][tx * 4 + i]; }
      if (SW) {
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = Us[c][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
          if (SW) accu[i][j] = fmaf(a[i], u[j], accu[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= Nout) continue;
      const float v = acc[i][j];
      if (EPI == EPI_BF16) {
        reinterpret_cast<float*>(g.C)[(size_t)m * g.ldc + n] = v;
      } else if (EPI == EPI_F32) {
        reinterpret_cast<float*>(g.C)[(size_t)m * g.ldc + n] = v;
      } else if (EPI == EPI_RESID) {
        const float gt = (m < g.n_pre ? g.gate_0 : g.gate_t)[n];
        float* hp = g.Hres + (size_t)m * g.ldh + n;
        *hp = *hp + gt * v;
      } else {
        reinterpret_cast<float*>(g.C)[(size_t)m * g.ldc + n] = v / (1.f + expf(-v)) * accu[i][j];
      }
    }
  }
}

template <int EPI>
hipError_t run_f32(const GemmArgs& g, hipStream_t s) {
  const int Nout = EPI == EPI_SWIGLU ? g.N / 2 : g.N;
  dim3 grid((Nout + 63) / 64, (g.M + 63) / 64);
  hipLaunchKernelGGL((gemm_f32_kernel<EPI>), grid, dim3(256), 0, s, g, Nout);
  return hipGetLastError();
}

// One wave per (query, head); lane owns dims 2l, 2l+1. Online softmax in
// fp32 over the visible keys j <= limit[i] (and j < S).
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int qi = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int h = blockIdx.y;
  if (qi >= a.N) return;
  const float* q = a.q + (size_t)qi * a.q_stride + h * 128;
  const float q0 = q[2 * lane], q1 = q[2 * lane + 1];
  const float* kb = a.k + (size_t)h * a.cap * 128;
  const float* vb = a.vt + (size_t)h * 128 * a.cap;
  const int lim = a.limit[a.q_off + qi];
  const float scale = 0.08838834764831845f;   // 1/sqrt(128)
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int j = 0; j < a.S; ++j) {
    if (!key_visible(j, lim, a.S)) continue;
    const float s = wave_sum(q0 * kb[(size_t)j * 128 + 2 * lane] + q1 * kb[(size_t)j * 128 + 2 * lane + 1]) * scale;
    const float mn = fmaxf(m, s);
    const float alpha = expf(m - mn), p = expf(s - mn);
    l = l * alpha + p;
    o0 = o0 * alpha + p * vb[(size_t)(2 * lane) * a.cap + j];
    o1 = o1 * alpha + p * vb[(size_t)(2 * lane + 1) * a.cap + j];
    m = mn;
  }
  float* out = a.out + (size_t)qi * a.out_stride + h * 128;
  out[2 * lane] = o0 / l;
  out[2 * lane + 1] = o1 / l;
}

}  // namespace

bool gemm_shape_ok(int M, int N, int K, int epi) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 16) return false;
  return N % 64 == 0;
}

static hipError_t gemm_sequence(const GemmArgs& g, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_BF16: return run_f32<EPI_BF16>(g, s);
    case EPI_RESID: return run_f32<EPI_RESID>(g, s);
    case EPI_SWIGLU: return run_f32<EPI_SWIGLU>(g, s);
    case EPI_F32: return run_f32<EPI_F32>(g, s);
    case EPI_QKV: {   // plain GEMM, then the standalone norm / RoPE / cache kernel
      const hipError_t e = run_f32<EPI_BF16>(g, s);
      if (e != hipSuccess) return e;
      QkArgs q = g.qk;
      q.g_begin = q.q_row0;
      q.g_end = q.q_row0 + g.M;
      return launch_qknorm_rope(q, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(const GemmArgs& g, int epi, hipStream_t s, const LaunchEvents& ev) {
  if (ev.start) (void)hipEventRecord(ev.start, s);
  const hipError_t e = gemm_sequence(g, epi, s);
  if (ev.stop) (void)hipEventRecord(ev.stop, s);
  return e;
}

hipError_t launch_gemm_forced_split(const GemmArgs&, int, int, hipStream_t) { return hipErrorInvalidValue; }

hipError_t launch_attention(const AttnArgs& a, hipStream_t s, const LaunchEvents& ev) {
  dim3 grid((a.N + 3) / 4, a.nh);
  launch_k(attn_f32_kernel, grid, dim3(256), s, ev.start, ev.stop, a);
  return hipGetLastError();
}

hipError_t launch_attention_variant(const AttnArgs&, int, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace dit
