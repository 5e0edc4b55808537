// bf16 MFMA GEMM for gfx950: C = A·Bᵀ with A [M,K] and B [N,K] both
// K-contiguous (activations × nn.Linear weights), fp32 accumulation.
//
// Block tile BM×BN×64, WM×WN waves, each wave owns a (BM/WM)×(BN/WN) tile
// built from v_mfma_f32_32x32x16_bf16 blocks. Operand tiles are staged
// global -> registers -> LDS, double-buffered (one barrier per K step),
// with a 16-byte-chunk XOR swizzle (chunk ^ row%8) so that the 8 lanes an
// LDS read serves together hit 8 different bank groups.
//
// Tile order is XCD-aware: the hardware deals workgroups round-robin over
// the 8 XCDs, so block b is remapped to logical tile (b%8)*(n/8) + b/8,
// giving each XCD a contiguous run of logical tiles; logical tiles are then
// grouped GROUP_M tile-rows at a time so a run covers a compact M×N patch
// whose A and B panels stay in that XCD's L2.
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int BK = 64;
constexpr int GROUP_M = 4;

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(WM* WN * 64) void gemm_kernel(GemmArgs g) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int ACH = BM * BK / 8 / NT;   // 16-byte A chunks per thread per stage
  constexpr int BCH = BN * BK / 8 / NT;
  static_assert(ACH * NT * 8 == BM * BK && BCH * NT * 8 == BN * BK, "tile/thread mismatch");
  static_assert(EPI != EPI_SWIGLU || (FN % 2 == 0 && TN % 64 == 0), "SwiGLU pairs 32-col blocks");

  __shared__ u32x4 smem[2][(BM + BN) * BK / 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- tile coordinates (XCD-aware, grouped) ----
  const int ntm = (g.M + BM - 1) / BM;
  const int ntn = g.N / BN;
  const int nblk = ntm * ntn;
  int b = blockIdx.x;
  const int per = nblk >> 3;
  if (b < per * 8) b = (b & 7) * per + (b >> 3);
  const int in_group = GROUP_M * ntn;
  const int gid = b / in_group;
  const int first = gid * GROUP_M;
  const int gsz = min(ntm - first, GROUP_M);
  const int tm = first + (b % in_group) % gsz;
  const int tn = (b % in_group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  // ---- global source pointers for this thread's chunks ----
  const u32x4* asrc[ACH];
  int adst[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    int q = tid + i * NT;
    int row = q >> 3, c = q & 7;
    int gr = min(m0 + row, g.M - 1);
    asrc[i] = reinterpret_cast<const u32x4*>(g.A + (size_t)gr * g.lda + c * 8);
    adst[i] = row * 8 + (c ^ (row & 7));
  }
  const u32x4* bsrc[BCH];
  int bdst[BCH];
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    int q = tid + i * NT;
    int row = q >> 3, c = q & 7;
    int p = n0 + row;
    const uint16_t* base;
    if (EPI == EPI_SWIGLU) {
      // packed column p: 32-wide blocks alternate gate / up for the same
      // 32 features: block b2 = p/64, half s = (p/32)&1, feature 32*b2 + p%32
      int f = ((p >> 6) << 5) + (p & 31);
      base = (((p >> 5) & 1) ? g.B2 : g.B) + (size_t)f * g.ldb;
    } else {
      base = g.B + (size_t)p * g.ldb;
    }
    bsrc[i] = reinterpret_cast<const u32x4*>(base + c * 8);
    bdst[i] = BM * 8 + row * 8 + (c ^ (row & 7));
  }

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 ra[ACH], rb[BCH];
  const int nk = g.K / BK;

  // prologue: stage 0
#pragma unroll
  for (int i = 0; i < ACH; ++i) ra[i] = asrc[i][0];
#pragma unroll
  for (int i = 0; i < BCH; ++i) rb[i] = bsrc[i][0];
#pragma unroll
  for (int i = 0; i < ACH; ++i) smem[0][adst[i]] = ra[i];
#pragma unroll
  for (int i = 0; i < BCH; ++i) smem[0][bdst[i]] = rb[i];
  __syncthreads();

  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  const int sw = lane & 7;   // row % 8 of every row this lane reads

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int ko = (kt + 1) * (BK / 8);   // in 16-byte units
#pragma unroll
      for (int i = 0; i < ACH; ++i) ra[i] = asrc[i][ko];
#pragma unroll
      for (int i = 0; i < BCH; ++i) rb[i] = bsrc[i][ko];
    }
    const u32x4* As = smem[cur];
    const u32x4* Bs = smem[cur] + BM * 8;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int ch = (2 * s + lhalf) ^ sw;
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = __builtin_bit_cast(bf16x8, As[(wm * TM + i * 32 + lrow) * 8 + ch]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8, Bs[(wn * TN + j * 32 + lrow) * 8 + ch]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
    if (more) {
      u32x4* nxt = smem[cur ^ 1];
#pragma unroll
      for (int i = 0; i < ACH; ++i) nxt[adst[i]] = ra[i];
#pragma unroll
      for (int i = 0; i < BCH; ++i) nxt[bdst[i]] = rb[i];
    }
    __syncthreads();
  }

  // ---- epilogue ----
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * TM + i * 32 + 8 * (r >> 2) + 4 * lhalf + (r & 3);
      if (m >= g.M) continue;
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int j = 0; j < FN; j += 2) {
          const int n = n0 + wn * TN + j * 32;            // multiple of 64
          const int f = (n >> 1) + lrow;
          const float gv = acc[i][j][r], uv = acc[i][j + 1][r];
          const float sv = gv / (1.f + __expf(-gv));
          reinterpret_cast<bf16_t*>(g.C)[(size_t)m * g.ldc + f] = f2bf(sv * uv);
        }
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int n = n0 + wn * TN + j * 32 + lrow;
          const float v = acc[i][j][r];
          if (EPI == EPI_BF16) {
            reinterpret_cast<bf16_t*>(g.C)[(size_t)m * g.ldc + n] = f2bf(v);
          } else if (EPI == EPI_F32) {
            reinterpret_cast<float*>(g.C)[(size_t)m * g.ldc + n] = v;
          } else {
            const float gt = (m < g.n_pre ? g.gate_0 : g.gate_t)[n];
            float* hp = g.Hres + (size_t)m * g.ldh + n;
            *hp = *hp + tanhf(gt) * v;
          }
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int EPI>
hipError_t run(const GemmArgs& g, hipStream_t s) {
  const int nblk = ((g.M + BM - 1) / BM) * (g.N / BN);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI>), dim3(nblk), dim3(WM * WN * 64), 0, s, g);
  return hipGetLastError();
}

}  // namespace

bool gemm_shape_ok(int M, int N, int K, int epi) {
  if (M <= 0 || N <= 0 || K <= 0 || K % BK) return false;
  if (epi == EPI_F32) return N % 64 == 0;
  return N % 256 == 0;
}

hipError_t launch_gemm(const GemmArgs& g, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_BF16: return run<256, 256, 2, 4, EPI_BF16>(g, s);
    case EPI_RESID: return run<256, 256, 2, 4, EPI_RESID>(g, s);
    case EPI_SWIGLU: return run<256, 256, 2, 4, EPI_SWIGLU>(g, s);
    case EPI_F32: return run<64, 64, 2, 2, EPI_F32>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dit
