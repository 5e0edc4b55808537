// bf16 MFMA GEMMs for gfx950: C = A·Bᵀ with A [M,K] and B [N,K] both
// K-contiguous (activations × nn.Linear weights), fp32 accumulation, built
// from v_mfma_f32_32x32x16_bf16 blocks, with fused epilogues (bf16 store,
// fp32 store, gated fp32 residual update, SwiGLU).
//
// gemm_dma_kernel (the step's GEMMs): 256x256 block tile, 8 waves (2x4),
// K in stages of 32 held in a ring of four 32 KB LDS stages that are filled
// straight from global memory with buffer_load ... lds three stages ahead.
// gemm_kernel: register-staged variant (global -> VGPR -> LDS, two stages),
// used for the narrow proj_out GEMM (64x64 tiles) and kept as a reference.
//
// Both use an XCD-aware tile order: the hardware deals workgroups
// round-robin over the 8 XCDs, so block b is remapped to logical tile
// (b%8)*(n/8) + b/8, giving each XCD a contiguous run of logical tiles;
// logical tiles are then grouped GROUP_M tile-rows at a time so a run
// covers a compact M×N patch whose A and B panels stay in that XCD's L2.
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

  // ---- buffer resources (base at this tile's first row / feature) ----
  // Rows past M fall outside the A resource and read as zero. Thread t
  // loads 16-byte chunk c = t%8 of rows r0 + i*RPI (r0 = t/8, RPI = NT/8);
  // its lane offset is fixed, the row step i and the K position go into
  // the scalar offset, and the LDS slot of chunk i is a constant offset
  // (RPI is a multiple of 16, so the swizzle (row/2)%8 is the same for all i).
  constexpr int RPI = NT / 8;
  static_assert(RPI % 16 == 0, "swizzle must repeat across chunk passes");
  const int r0 = tid >> 3, c0 = tid & 7;
  const int sw0 = (r0 >> 1) & 7;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(
      g.A + (size_t)m0 * g.lda, (uint32_t)min((size_t)(g.M - m0) * g.lda * 2, (size_t)0xFFFFFFF0u));
  const uint32_t aoff = (uint32_t)((r0 * g.lda + c0 * 8) * 2);
  const uint32_t astep = (uint32_t)(RPI * g.lda * 2);
  const int adst = r0 * 8 + (c0 ^ sw0);
  // B: for SwiGLU the packed column p maps to feature 32*(p/64) + p%32 of
  // the gate matrix if (p/32) is even, else of the up matrix.
  __amdgpu_buffer_rsrc_t rB0, rB1;
  uint32_t boff, bstep;
  if (EPI == EPI_SWIGLU) {
    const size_t bytes = min((size_t)(BN / 2) * g.ldb * 2, (size_t)0xFFFFFFF0u);
    rB0 = make_rsrc(g.B + (size_t)(n0 >> 1) * g.ldb, (uint32_t)bytes);
    rB1 = make_rsrc(g.B2 + (size_t)(n0 >> 1) * g.ldb, (uint32_t)bytes);
    if (RPI >= 64) {
      // every chunk of this thread is in the same 32-row half: pick the
      // matrix once per wave (8 rows per wave never cross a 32-row block)
      const int sel = __builtin_amdgcn_readfirstlane((r0 >> 5) & 1);
      if (sel) rB0 = rB1;
      boff = (uint32_t)(((32 * (r0 >> 6) + (r0 & 31)) * g.ldb + c0 * 8) * 2);
      bstep = (uint32_t)((RPI / 2) * g.ldb * 2);
    } else {
      // RPI == 32: chunk i is gate for even i, up for odd i, row 32*(i/2) + r0
      boff = (uint32_t)((r0 * g.ldb + c0 * 8) * 2);
      bstep = (uint32_t)(32 * g.ldb * 2);
    }
  } else {
    rB0 = rB1 = make_rsrc(g.B + (size_t)n0 * g.ldb, (uint32_t)min((size_t)BN * g.ldb * 2, (size_t)0xFFFFFFF0u));
    boff = (uint32_t)((r0 * g.ldb + c0 * 8) * 2);
    bstep = (uint32_t)(RPI * g.ldb * 2);
  }
  const int bdst = BM * 8 + r0 * 8 + (c0 ^ sw0);

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = g.K / BK;
  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  const int sw = (lane >> 1) & 7;   // (row/2) % 8 of every row this lane reads

  // Two register staging sets: tile kt+1 sits in set (kt+1)&1 while the
  // loads of tile kt+2 go to set kt&1, so every global load has two K steps
  // of MFMA work to arrive before its ds_write.
  u32x4 ra[2][ACH], rb[2][BCH];
  auto gload = [&](int set, int kt) {
    const uint32_t ko = (uint32_t)(kt * BK * 2);   // bytes
#pragma unroll
    for (int i = 0; i < ACH; ++i)
      ra[set][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, aoff, ko + i * astep, 0));
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      if (EPI == EPI_SWIGLU && RPI < 64)
        rb[set][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
            (i & 1) ? rB1 : rB0, boff, ko + (i >> 1) * bstep, 0));
      else
        rb[set][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rB0, boff, ko + i * bstep, 0));
    }
  };
  auto lstore = [&](int set, int buf) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) smem[buf][adst + i * RPI * 8] = ra[set][i];
#pragma unroll
    for (int i = 0; i < BCH; ++i) smem[buf][bdst + i * RPI * 8] = rb[set][i];
  };
  // fragments of one 16-wide K slice, double-buffered in registers
  bf16x8 fa[2][FM], fb[2][FN];
  auto lread = [&](int fset, int buf, int s) {
    const u32x4* As = smem[buf];
    const u32x4* Bs = smem[buf] + BM * 8;
    const int ch = (2 * s + lhalf) ^ sw;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[fset][i] = __builtin_bit_cast(bf16x8, As[(wm * TM + i * 32 + lrow) * 8 + ch]);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb[fset][j] = __builtin_bit_cast(bf16x8, Bs[(wn * TN + j * 32 + lrow) * 8 + ch]);
  };
  auto mma = [&](int fset) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma32(fa[fset][i], fb[fset][j], acc[i][j]);
  };

  // prologue: tile 0 -> LDS buffer 0; tile 1 in flight in set 1
  gload(0, 0);
  gload(1, min(1, nk - 1));
  lstore(0, 0);
  lds_barrier();
  lread(0, 0, 0);

  // One K step of 64 = four 16-wide slices s = 0..3 on LDS buffer par:
  //  - tile kt+2 is requested into register set par (freed when tile kt
  //    was stored);
  //  - slice s+1 is read from LDS while the MFMAs of slice s run;
  //  - tile kt+1 (register set par^1, requested one step earlier) is
  //    stored to the other LDS buffer during slice 1;
  //  - the only barrier sits before slice 3, so the first slice of the next
  //    tile is read while slice 3 computes. Every read of a buffer is issued
  //    before the barrier that precedes the next store into it.
  // All memory operations in the loop are unconditional: past the end the
  // loads re-read the last tile and the store fills the idle LDS buffer,
  // which nothing reads again. This keeps the waitcnt analysis exact (the
  // LDS stores wait only for the older register set).
  auto step = [&](int kt, int par) {
    gload(par, min(kt + 2, nk - 1));
    __builtin_amdgcn_sched_barrier(0);   // keep the prefetch at the top
    lread(1, par, 1);
    mma(0);
    lread(0, par, 2);
    lstore(par ^ 1, par ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    mma(1);
    lread(1, par, 3);
    mma(0);
    lds_barrier();
    lread(0, par ^ 1, 0);
    mma(1);
  };
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(kt, 0);
    step(kt + 1, 1);
  }
  if (kt < nk) step(kt, 0);

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
            *hp = *hp + gt * v;
          }
        }
      }
    }
  }
}

// Epilogue shared by the direct-to-LDS kernels: wave (wm, wn) owns the
// TM x TN patch at (m0 + wm*TM, n0 + wn*TN) in FM x FN blocks of 32x32.
template <int FM, int FN, int TM, int TN, int EPI, bool SWAP>
__device__ __forceinline__ void store_tile(const GemmArgs& g, f32x16 (&acc)[FM][FN], int m0, int n0,
                                           int wm, int wn, int lrow, int lhalf) {
  if (!SWAP) {
    // accumulator register r of lane l holds C[8*(r/4) + 4*(l/32) + r%4][l%32]
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * TM + i * 32 + 8 * (r >> 2) + 4 * lhalf + (r & 3);
        if (m >= g.M) continue;
        if (EPI == EPI_SWIGLU) {
#pragma unroll
          for (int j = 0; j < FN; j += 2) {
            const int f = ((n0 + wn * TN + j * 32) >> 1) + lrow;
            const float gv = acc[i][j][r], uv = acc[i][j + 1][r];
            reinterpret_cast<bf16_t*>(g.C)[(size_t)m * g.ldc + f] = f2bf(gv / (1.f + __expf(-gv)) * uv);
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
              *hp = *hp + gt * v;
            }
          }
        }
      }
    }
    return;
  }
  // ---- epilogue: lane owns row m = .. + lrow, columns n0c + 8g + 4*lhalf + {0..3} ----
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * TM + i * 32 + lrow;
    if (m >= g.M) continue;
    if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int j = 0; j < FN; j += 2) {
        const int fbase = ((n0 + wn * TN + j * 32) >> 1);     // gate block j, up block j+1
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float gv = acc[i][j][4 * gq + e], uv = acc[i][j + 1][4 * gq + e];
            o[e] = gv / (1.f + __expf(-gv)) * uv;
          }
          u32x2 w;
          w.x = pack2bf(o[0], o[1]);
          w.y = pack2bf(o[2], o[3]);
          *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(g.C) + (size_t)m * g.ldc + fbase + 8 * gq + 4 * lhalf) = w;
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int n = n0 + wn * TN + j * 32 + 8 * gq + 4 * lhalf;
          float a4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) a4[e] = acc[i][j][4 * gq + e];
          if (EPI == EPI_BF16) {
            u32x2 w;
            w.x = pack2bf(a4[0], a4[1]);
            w.y = pack2bf(a4[2], a4[3]);
            *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(g.C) + (size_t)m * g.ldc + n) = w;
          } else if (EPI == EPI_F32) {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(g.C) + (size_t)m * g.ldc + n) =
                make_float4(a4[0], a4[1], a4[2], a4[3]);
          } else {
            const float4 gt = *reinterpret_cast<const float4*>((m < g.n_pre ? g.gate_0 : g.gate_t) + n);
            float4* hp = reinterpret_cast<float4*>(g.Hres + (size_t)m * g.ldh + n);
            float4 hv = *hp;
            hv.x += gt.x * a4[0];
            hv.y += gt.y * a4[1];
            hv.z += gt.z * a4[2];
            hv.w += gt.w * a4[3];
            *hp = hv;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Direct-to-LDS variant: BM = BN = 256, BK = 32, a ring of 4 LDS stages of
// 32 KB (separate arrays, so the compiler's LDS-DMA wait tracking can tell
// them apart). Tiles are fetched with buffer_load ... lds three stages ahead
// of their use, so no registers are spent on staging. Each LDS row holds 32
// bf16 of K (64 bytes = 4 chunks); chunk c of row r sits at c ^ ((r/4)%4),
// which spreads the 16 rows one ds_read_b128 phase touches over 16 distinct
// bank groups. One barrier per stage, placed after the first 16-wide slice
// so the next stage's first fragments are read while the second slice runs.
#define LDSP(p) ((__attribute__((address_space(3))) void*)(p))

template <int WM, int WN, int EPI, bool SWAP = true, int GM = GROUP_M>
__global__ __launch_bounds__(WM* WN * 64) void gemm_dma_kernel(GemmArgs g) {
  constexpr int BM = 256, BN = 256, DBK = 32;
  constexpr int NT = WM * WN * 64;
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int BLK = (BM + BN) / 16;          // 1 KB blocks (16 rows) per stage
  constexpr int CH = BLK / NW;                 // DMA instructions per wave per stage
  static_assert(CH * NW == BLK, "blocks per wave");
  static_assert(EPI != EPI_SWIGLU || (FN % 2 == 0 && TN % 64 == 0), "SwiGLU pairs 32-col blocks");
  constexpr int SW = (BM + BN) * DBK / 8;      // u32x4 per stage (2048)
  __shared__ u32x4 st0[SW], st1[SW], st2[SW], st3[SW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  const int ntm = (g.M + BM - 1) / BM;
  const int ntn = g.N / BN;
  const int nblk = ntm * ntn;
  int b = blockIdx.x;
  const int per = nblk >> 3;
  if (b < per * 8) b = (b & 7) * per + (b >> 3);
  const int in_group = GM * ntn;
  const int gid = b / in_group;
  const int first = gid * GM;
  const int gsz = min(ntm - first, GM);
  const int tm = first + (b % in_group) % gsz;
  const int tn = (b % in_group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  // lane part of every DMA: row l/4 of the 16-row block, logical chunk
  // (l%4) ^ ((l/16)%4) so the lane's 16 bytes land at physical slot l%4
  const int lr = lane >> 2;
  const int lc = (lane & 3) ^ ((lane >> 4) & 3);
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(
      g.A + (size_t)m0 * g.lda, (uint32_t)min((size_t)(g.M - m0) * g.lda * 2, (size_t)0xFFFFFFF0u));
  __amdgpu_buffer_rsrc_t rG, rU;
  if (EPI == EPI_SWIGLU) {
    const size_t bytes = min((size_t)(BN / 2) * g.ldb * 2, (size_t)0xFFFFFFF0u);
    rG = make_rsrc(g.B + (size_t)(n0 >> 1) * g.ldb, (uint32_t)bytes);
    rU = make_rsrc(g.B2 + (size_t)(n0 >> 1) * g.ldb, (uint32_t)bytes);
  } else {
    rG = rU = make_rsrc(g.B + (size_t)n0 * g.ldb, (uint32_t)min((size_t)BN * g.ldb * 2, (size_t)0xFFFFFFF0u));
  }
  const uint32_t aoff = (uint32_t)((lr * g.lda + lc * 8) * 2);
  const uint32_t boff = (uint32_t)((lr * g.ldb + lc * 8) * 2);
  const int nk = g.K / DBK;

  // DMA blocks: instruction j < CH/2 of a wave loads A block j*NW + wave;
  // instruction CH/2 + jj loads a 16-row B block whose gate/up choice is a
  // compile-time function of jj (B block bb = 4*q + 2*mat + half holds
  // features 32*q + 16*half + r of matrix mat).
  static_assert(BM == BN && CH % 2 == 0, "A and B blocks split evenly");
  constexpr int CHB = CH / 2;
  static_assert(NW * CHB == BN / 16 && (NW == 4 || NW == 8), "B block mapping");
  auto dma = [&](u32x4* stg, int kt) {
    const uint32_t ko = (uint32_t)(kt * DBK * 2);
#pragma unroll
    for (int j = 0; j < CHB; ++j) {
      const int blk = j * NW + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, LDSP(stg + blk * 64), 16, aoff,
                                               ko + (uint32_t)(blk * 16 * g.lda * 2), 0, 0);
    }
#pragma unroll
    for (int jj = 0; jj < CHB; ++jj) {
      int q, mat, hf;
      if (NW == 4) { q = wave; mat = jj >> 1; hf = jj & 1; }
      else { q = wave >> 1; mat = jj; hf = wave & 1; }
      const int bb = 4 * q + 2 * mat + hf;
      u32x4* dst = stg + (BM / 16 + bb) * 64;
      if (EPI == EPI_SWIGLU) {
        const uint32_t so = ko + (uint32_t)((32 * q + 16 * hf) * g.ldb * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(mat ? rU : rG, LDSP(dst), 16, boff, so, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rG, LDSP(dst), 16, boff,
                                                 ko + (uint32_t)(bb * 16 * g.ldb * 2), 0, 0);
      }
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int lrow = lane & 31, lhalf = lane >> 5;
  const int swz = (lrow >> 2) & 3;
  bf16x8 fa[2][FM], fb[2][FN];
  auto lread = [&](int fs, const u32x4* stg, int s) {
    const int ph = (2 * s + lhalf) ^ swz;
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[fs][i] = __builtin_bit_cast(bf16x8, stg[(wm * TM + i * 32 + lrow) * 4 + ph]);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[fs][j] = __builtin_bit_cast(bf16x8, stg[(BM + wn * TN + j * 32 + lrow) * 4 + ph]);
  };
  // Operands swapped (B fragment first): each 32x32 block is accumulated as
  // Cᵀ, so lane l holds row l%32 of the block and, in registers 4g..4g+3,
  // the four consecutive columns 8g + 4*(l/32) + {0..3} -> vector stores.
  auto mma = [&](int fs) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = SWAP ? mfma32(fb[fs][j], fa[fs][i], acc[i][j]) : mfma32(fa[fs][i], fb[fs][j], acc[i][j]);
  };
  // wait until this wave's DMA of the stage needed next has landed (the two
  // younger stages may stay in flight) and its LDS reads are done, then sync
  static_assert(2 * CH <= 63, "vmcnt range");
  auto stage_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * CH));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
  };

  // prologue: stages 0..2 in flight; wait for stage 0
  dma(st0, 0);
  dma(st1, min(1, nk - 1));
  dma(st2, min(2, nk - 1));
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * CH));
  __builtin_amdgcn_s_barrier();
  lread(0, st0, 0);

  // iteration on stage `cur`: DMA tile kt+3 into `fut` (freed at the last
  // barrier), slice 0, barrier (tile kt+1 visible), slice 1 while the next
  // stage's slice-0 fragments load.
  // Instruction order is pinned with sched_group_barrier: the fragment
  // reads for the next slice go out one per MFMA at the front of the
  // current slice's MFMAs (so they have the rest of the slice to land), and
  // the DMAs are spread over the remaining MFMAs.
  constexpr int NMF = FM * FN, NRD = FM + FN;
  // slice 0: reads paired with MFMAs first, then DMAs paired with the rest
  constexpr int P0 = NRD < NMF ? NRD : NMF;
  constexpr int P1 = (NMF - P0) < CH ? (NMF - P0) : CH;
  auto iter = [&](u32x4* cur, u32x4* nxt, u32x4* fut, int kt) {
    lread(1, cur, 1);
    dma(fut, min(kt + 3, nk - 1));
    mma(0);
#pragma unroll
    for (int k = 0; k < P0; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    }
    if (NRD > P0) __builtin_amdgcn_sched_group_barrier(0x100, NRD - P0, 0);
#pragma unroll
    for (int k = 0; k < P1; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read (LDS DMA)
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    if (CH > P1) __builtin_amdgcn_sched_group_barrier(0x020, CH - P1, 0);
    if (NMF > P0 + P1) __builtin_amdgcn_sched_group_barrier(0x008, NMF - P0 - P1, 0);
    stage_barrier();
    lread(0, nxt, 0);
    mma(1);
#pragma unroll
    for (int k = 0; k < P0; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    }
    if (NRD > P0) __builtin_amdgcn_sched_group_barrier(0x100, NRD - P0, 1);
    if (NMF > P0) __builtin_amdgcn_sched_group_barrier(0x008, NMF - P0, 1);
  };
  int kt = 0;
  for (; kt + 3 < nk; kt += 4) {
    iter(st0, st1, st3, kt);
    iter(st1, st2, st0, kt + 1);
    iter(st2, st3, st1, kt + 2);
    iter(st3, st0, st2, kt + 3);
  }
  if (kt < nk) iter(st0, st1, st3, kt);
  if (kt + 1 < nk) iter(st1, st2, st0, kt + 1);
  if (kt + 2 < nk) iter(st2, st3, st1, kt + 2);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // drain outstanding DMA before exit

  store_tile<FM, FN, TM, TN, EPI, SWAP>(g, acc, m0, n0, wm, wn, lrow, lhalf);
}

// Epilogue through LDS for the swapped layout (each 32x32 block accumulated
// as Cᵀ: lane l holds row l%32 and, in registers 4q..4q+3, the four
// consecutive columns 8q + 4*(l/32) + {0..3}). Storing that layout directly
// makes every store instruction touch 32 rows. Instead each wave stages its
// 128 x 128 patch (bf16; 128 x 64 after SwiGLU) row-major in its own LDS
// region, in 8-byte slots XOR-swizzled by the row so the writes of a half
// wave hit distinct banks, and then writes whole rows with 16-byte lanes.
// The caller guarantees every wave has finished reading the stage buffers.
template <int EPI>
__device__ __forceinline__ void store_tile_lds(const GemmArgs& g, f32x16 (&acc)[4][4], int m0, int n0,
                                               int wm, int wn, int lane, char* reg) {
  static_assert(EPI == EPI_BF16 || EPI == EPI_SWIGLU, "bf16 outputs only");
  constexpr int OUTC = EPI == EPI_SWIGLU ? 64 : 128;   // output columns of the patch
  constexpr int ROWB = OUTC * 2;                        // bytes per staged row
  constexpr int SLOTS = ROWB / 8;                       // 8-byte slots per row
  const int lrow = lane & 31, lhalf = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = i * 32 + lrow;
    char* rp = reg + row * ROWB;
    if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int j = 0; j < 4; j += 2)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float gv = acc[i][j][4 * q + e], uv = acc[i][j + 1][4 * q + e];
            o[e] = gv / (1.f + __expf(-gv)) * uv;
          }
          const int slot = (2 * ((j >> 1) * 4 + q) + lhalf) ^ (row & (SLOTS - 1));
          u32x2 w;
          w.x = pack2bf(o[0], o[1]);
          w.y = pack2bf(o[2], o[3]);
          *reinterpret_cast<u32x2*>(rp + slot * 8) = w;
        }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int slot = (2 * (4 * j + q) + lhalf) ^ (row & (SLOTS - 1));
          u32x2 w;
          w.x = pack2bf(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]);
          w.y = pack2bf(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          *reinterpret_cast<u32x2*>(rp + slot * 8) = w;
        }
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // the region is private to this wave
  // read back: a 16-byte chunk c of row R holds logical slots 2c, 2c+1, at
  // physical chunk c ^ ((R % SLOTS) / 2), halves exchanged when R is odd
  constexpr int CPR = ROWB / 16;           // chunks per row
  constexpr int RPI = 64 / CPR;            // rows per instruction
  const int cc = lane % CPR;
  bf16_t* C = reinterpret_cast<bf16_t*>(g.C);
  const int col0 = (EPI == EPI_SWIGLU ? (n0 >> 1) + wn * 64 : n0 + wn * 128) + 8 * cc;
#pragma unroll 4
  for (int q = 0; q < 128 / RPI; ++q) {
    const int R = q * RPI + lane / CPR;
    const int pc = cc ^ ((R & (SLOTS - 1)) >> 1);
    u32x4 v = *reinterpret_cast<const u32x4*>(reg + R * ROWB + pc * 16);
    if (R & 1) v = (u32x4){v.z, v.w, v.x, v.y};
    const int m = m0 + wm * 128 + R;
    if (m < g.M) *reinterpret_cast<u32x4*>(C + (size_t)m * g.ldc + col0) = v;
  }
}

// EPI_QKV epilogue. A wave's 128 x 128 patch is one head of q, k or v (the
// output columns are [q | k | v], 128 per head); the accumulators are
// rounded to bf16 exactly as EPI_BF16 stores them, so the norm sees the
// values the unfused path would have read back.
//  - q, k: the patch is staged row-major in LDS; the 16 lanes of a row (8
//    dims each) form the RMS over the head's 128 dims, apply (1 + w) and the
//    row token's 3D RoPE (interleaved pairs), and write q to its row of C
//    and k to its cache row;
//  - v: the patch is staged transposed (dim-major) and written to the
//    transposed cache, 16 lanes (256 bytes of consecutive tokens) per dim.
// Sum over the 16 lanes of a row (DPP: quad swaps, then half-row and row
// mirrors), the result in every lane.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);   // row_half_mirror
  v += dpp_f<0x140>(v);   // row_mirror
  return v;
}

__device__ __forceinline__ void store_tile_qkv(const GemmArgs& g, f32x16 (&acc)[4][4], int m0, int n0,
                                               int wm, int wn, int lane, char* reg) {
  constexpr int ROWB = 256;                 // bytes per staged row (128 bf16)
  constexpr int SLOTS = ROWB / 8;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const QkArgs& a = g.qk;
  const int c0 = n0 + wn * 128;
  const int sec = c0 / a.H;                  // 0 q, 1 k, 2 v (uniform over the wave)
  const int hh = (c0 - sec * a.H) >> 7;      // head
  const int rbase = m0 + wm * 128;           // local row of patch row 0
  const int cc = lane & 15;                  // 16-byte chunk of a staged row
  if (sec < 2) {
    // row-major staging, 8-byte slots XOR-swizzled by the row (as EPI_BF16)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = i * 32 + lrow;
      char* rp = reg + row * ROWB;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int slot = (2 * (4 * j + q) + lhalf) ^ (row & (SLOTS - 1));
          u32x2 w;
          w.x = pack2bf(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]);
          w.y = pack2bf(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          *reinterpret_cast<u32x2*>(rp + slot * 8) = w;
        }
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // the region is private to this wave
    const uint16_t* wv = sec == 0 ? a.wq : a.wk;
    float w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = 1.f + bf2f(wv[8 * cc + j]);
    bf16_t* C = reinterpret_cast<bf16_t*>(g.C);
    // RoPE tables of the lane's 32 rows (R = 4 it + lane/16), loaded up
    // front. Table row of token gq: gq itself before the prefix end P, else
    // P + (gq - P) % T_el (the latent's own layout row); it advances by 4
    // per row step and wraps by T_el.
    float4 cs[32], sn[32];
    {
      const int gq0 = a.q_row0 + rbase + (lane >> 4);
      int gl = (a.T_el > 0 && gq0 >= a.P) ? a.P + (gq0 - a.P) % a.T_el : gq0;
      // one subtraction per step wraps when T_el >= 4; tinier latents take
      // the modulo per row
      const bool tiny = a.T_el > 0 && a.T_el < 4;
      const int wrap = a.T_el > 0 ? a.P + a.T_el : 0x7FFFFFFF;
#pragma unroll
      for (int it = 0; it < 32; ++it) {
        const int m = rbase + it * 4 + (lane >> 4);
        int row = gl;
        if (tiny) {
          const int gq = gq0 + it * 4;
          row = gq >= a.P ? a.P + (gq - a.P) % a.T_el : gq;
        }
        row = m < g.M ? row : 0;                // rows past M read a valid row
        cs[it] = *reinterpret_cast<const float4*>(a.cosv + (size_t)row * 64 + 4 * cc);
        sn[it] = *reinterpret_cast<const float4*>(a.sinv + (size_t)row * 64 + 4 * cc);
        gl += 4;
        gl = gl >= wrap ? gl - a.T_el : gl;
      }
    }
#pragma unroll
    for (int it = 0; it < 32; ++it) {
      const int R = it * 4 + (lane >> 4);
      const int m = rbase + R;
      // chunk cc of row R (see store_tile_lds)
      const int pc = cc ^ ((R & (SLOTS - 1)) >> 1);
      u32x4 v = *reinterpret_cast<const u32x4*>(reg + R * ROWB + pc * 16);
      if (R & 1) v = (u32x4){v.z, v.w, v.x, v.y};
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
      float x[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = __uint_as_float(u[k] << 16);
        x[2 * k + 1] = __uint_as_float(u[k] & 0xFFFF0000u);
      }
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += x[j] * x[j];
      const float r = rsqrtf(row16_sum(ss) * (1.f / 128.f) + a.eps);
      const float c4[4] = {cs[it].x, cs[it].y, cs[it].z, cs[it].w};
      const float s4[4] = {sn[it].x, sn[it].y, sn[it].z, sn[it].w};
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float x0 = x[2 * k] * r * w[2 * k], x1 = x[2 * k + 1] * r * w[2 * k + 1];
        o[k] = pack2bf(x0 * c4[k] - x1 * s4[k], x0 * s4[k] + x1 * c4[k]);
      }
      const u32x4 ov = {o[0], o[1], o[2], o[3]};
      if (m < g.M) {
        if (sec == 0) *reinterpret_cast<u32x4*>(C + (size_t)m * g.ldc + c0 + 8 * cc) = ov;
        else *reinterpret_cast<u32x4*>(a.kc + ((size_t)hh * a.cap + a.q_row0 + m) * 128 + 8 * cc) = ov;
      }
    }
  } else {
    // transposed staging: dim row d (128 tokens, 256 bytes), 16-byte token
    // chunk c at c ^ (d % 16). A lane holds 4 consecutive dims of token t;
    // the pair of lanes with tokens t, t^1 swaps half of them, so that each
    // lane writes 2 dims x 2 tokens as two 4-byte words (the even-token lane
    // dims +0, +1, the odd-token lane dims +2, +3).
    const bool odd = lrow & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int te = i * 32 + (lrow & ~1);     // even token of the pair
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t p01 = pack2bf(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]);
          const uint32_t p23 = pack2bf(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          // quad_perm [1,0,3,2]: exchange with the neighbouring lane
          const uint32_t nb = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(odd ? p01 : p23), 0xB1, 0xF, 0xF,
                                                                    true);
          const uint32_t mine = odd ? p23 : p01;
          // words (token te, token te+1) for the lane's two dims
          const uint32_t lo = odd ? ((nb & 0xFFFFu) | (mine << 16)) : ((mine & 0xFFFFu) | (nb << 16));
          const uint32_t hi = odd ? ((nb >> 16) | (mine & 0xFFFF0000u)) : ((mine >> 16) | (nb & 0xFFFF0000u));
          const int d = j * 32 + 8 * q + 4 * lhalf + (odd ? 2 : 0);
          const int off = (((te >> 3) ^ (d & 15)) << 4) + (te & 7) * 2;
          *reinterpret_cast<uint32_t*>(reg + d * ROWB + off) = lo;
          *reinterpret_cast<uint32_t*>(reg + (d + 1) * ROWB + ((((te >> 3) ^ ((d + 1) & 15)) << 4) +
                                                                (te & 7) * 2)) = hi;
        }
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    act_t* vt = a.vtc + (size_t)hh * 128 * a.cap;
    const int g0 = a.q_row0 + rbase + 8 * cc;  // first token of the lane's chunk
    const int mv = rbase + 8 * cc;
    const bool full = mv + 8 <= g.M && (g0 & 7) == 0;
#pragma unroll 4
    for (int it = 0; it < 32; ++it) {
      const int d = it * 4 + (lane >> 4);
      const u32x4 v = *reinterpret_cast<const u32x4*>(reg + d * ROWB + ((cc ^ (d & 15)) << 4));
      act_t* dst = vt + (size_t)d * a.cap + g0;
      if (full) {
        *reinterpret_cast<u32x4*>(dst) = v;
      } else {
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (mv + j < g.M) dst[j] = (act_t)((j & 1) ? (u[j >> 1] >> 16) : (u[j >> 1] & 0xFFFF));
      }
    }
  }
}

// fp32 epilogue through LDS (swapped layout): Hres[m, n] += gate[n] *
// acc, fp32. The 128 x 128 fp32 patch of a wave (64 KB) is staged in two
// halves of 64 rows x 512 bytes, 16-byte chunks XOR-swizzled by the row;
// each half is then read back as whole rows (2 rows = 1 KB per instruction).
// All 32 Hres loads of a half are issued before any is used, so a wave keeps
// 32 KB of residual reads in flight.
// With PART, the patch is instead stored as fp32 partial sums of K split
// `split` into part[split][M][N] (no residual read).
template <bool PART>
__device__ __forceinline__ void store_tile_lds_f32(const GemmArgs& g, f32x16 (&acc)[4][4], int m0,
                                                   int n0, int wm, int wn, int lane, char* reg,
                                                   int split) {
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int cc = lane & 31;
  const int n = n0 + wn * 128 + 4 * cc;
  float4 gate_t = make_float4(0.f, 0.f, 0.f, 0.f), gate_0 = gate_t;
  if (!PART) {
    gate_t = *reinterpret_cast<const float4*>(g.gate_t + n);
    gate_0 = *reinterpret_cast<const float4*>(g.gate_0 + n);
  }
  float* out = PART ? g.part + (size_t)split * g.M * g.N : g.Hres;
  const int ldo = PART ? g.N : g.ldh;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int mb = m0 + wm * 128 + hf * 64 + (lane >> 5);
    float4 hv[32];
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const int m = mb + 2 * t;
      hv[t] = (!PART && m < g.M) ? *reinterpret_cast<const float4*>(g.Hres + (size_t)m * g.ldh + n)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = 2 * hf + ii;
      const int row = ii * 32 + lrow;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int k = (8 * j + 2 * q + lhalf) ^ (row & 31);
          *reinterpret_cast<float4*>(reg + row * 512 + k * 16) =
              make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        }
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const int R = 2 * t + (lane >> 5);
      const float4 a = *reinterpret_cast<const float4*>(reg + R * 512 + ((cc ^ (R & 31)) * 16));
      const int m = mb + 2 * t;
      float4 h = hv[t];
      if (PART) {
        h = a;
      } else {
        const float4 gt = m < g.n_pre ? gate_0 : gate_t;
        h.x += gt.x * a.x;
        h.y += gt.y * a.y;
        h.z += gt.z * a.z;
        h.w += gt.w * a.w;
      }
      if (m < g.M) *reinterpret_cast<float4*>(out + (size_t)m * ldo + n) = h;
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // reads done before the next half overwrites
  }
}

// ---------------------------------------------------------------------------
// One wave per SIMD: 4 waves (2x2) of 128x128 on the 256x256 block tile, K
// in stages of 64 (rows of 128 bytes), two 64 KB LDS stages. Per 16-wide K
// slice a wave reads 4 A + 4 B fragments for 16 MFMAs: two thirds of the
// LDS bytes per MFMA of a 128x64 wave tile; latency is hidden inside the
// wave by software pipelining instead of by a second wave.
//  - stage kt+1 is fetched into the other LDS stage during slice 0 of stage
//    kt (that stage was last read before the previous barrier);
//  - fragments of slice s+1 are read during the MFMAs of slice s;
//  - the one barrier per stage sits in the middle of slice 3, so the next
//    stage's slice-0 fragments load while the second half of slice 3 runs.
// LDS rows hold 64 bf16 of K (8 chunks of 16 B); chunk c of row r sits at
// c ^ ((r/2)%8), which puts the 16 rows one ds_read_b128 phase touches on
// all 64 banks exactly once.
template <int EPI, bool SWAP, bool PACKED = (EPI == EPI_SWIGLU)>
__global__ __launch_bounds__(256) void gemm_w4_kernel(GemmArgs g) {
  constexpr int BM = 256, BN = 256, SBK = 64;
  constexpr int WN = 2, TM = 128, TN = 128, FM = 4, FN = 4;
  constexpr int SW = (BM + BN) * SBK / 8;      // u32x4 per stage (64 KB)
  static_assert(EPI != EPI_SWIGLU || (FN % 2 == 0 && TN % 64 == 0), "SwiGLU pairs 32-col blocks");
  __shared__ u32x4 st0[SW], st1[SW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // Grid = tiles x splits (splits = 1 unless EPI_PART): block b works on
  // tile b % tiles over K range split * K/splits .. (split+1) * K/splits.
  const int ntm = (g.M + BM - 1) / BM;
  const int ntn = g.N / BN;
  const int ntiles = ntm * ntn;
  const int nblk = gridDim.x;
  int b = blockIdx.x;
  const int per = nblk >> 3;
  if (b < per * 8) b = (b & 7) * per + (b >> 3);
  const int split = EPI == EPI_PART ? b / ntiles : 0;
  b -= split * ntiles;
  const int in_group = GROUP_M * ntn;
  const int gid = b / in_group;
  const int first = gid * GROUP_M;
  const int gsz = min(ntm - first, GROUP_M);
  const int tm = first + (b % in_group) % gsz;
  const int tn = (b % in_group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;
  const int klen = EPI == EPI_PART ? g.K / g.splits : g.K;
  const int kbeg = split * klen;

  // DMA: an instruction moves an 8-row block (1 KB); lane l fills row l/8,
  // physical chunk l%8, which holds logical chunk (l%8) ^ ((row/2)%8). Wave
  // w moves blocks 4j + w (j = 0..7) of A and of B, whose row parity (and so
  // whose lane offsets) are the same for every j.
  const int lr = lane >> 3;
  const int lc = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(
      g.A + (size_t)m0 * g.lda, (uint32_t)min((size_t)(g.M - m0) * g.lda * 2, (size_t)0xFFFFFFF0u));
  __amdgpu_buffer_rsrc_t rG, rU;
  if (PACKED) {
    const size_t bytes = min((size_t)(BN / 2) * g.ldb * 2, (size_t)0xFFFFFFF0u);
    rG = make_rsrc(g.B + (size_t)(n0 >> 1) * g.ldb, (uint32_t)bytes);
    rU = make_rsrc(g.B2 + (size_t)(n0 >> 1) * g.ldb, (uint32_t)bytes);
  } else {
    rG = rU = make_rsrc(g.B + (size_t)n0 * g.ldb, (uint32_t)min((size_t)BN * g.ldb * 2, (size_t)0xFFFFFFF0u));
  }
  const uint32_t aoff = (uint32_t)((lr * g.lda + lc * 8) * 2);
  const uint32_t boff = (uint32_t)((lr * g.ldb + lc * 8) * 2);
  const int nk = klen / SBK;

  // B block bb = 4j + w holds packed columns 8bb .. 8bb+7. For SwiGLU the
  // packed column p is feature 32*(p/64) + p%32 of gate (p/32 even) or up
  // (p/32 odd): block 4j + w is rows 32*(j/2) + 8w .. +7 of matrix j%2.
  auto dma = [&](u32x4* stg, int kt) {
    const uint32_t ko = (uint32_t)((kbeg + kt * SBK) * 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int blk = 4 * j + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, LDSP(stg + blk * 64), 16, aoff,
                                               ko + (uint32_t)(blk * 8 * g.lda * 2), 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int bb = 4 * j + wave;
      u32x4* dst = stg + (BM / 8 + bb) * 64;
      if (PACKED) {
        const uint32_t so = ko + (uint32_t)((32 * (j >> 1) + 8 * wave) * g.ldb * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds((j & 1) ? rU : rG, LDSP(dst), 16, boff, so, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rG, LDSP(dst), 16, boff,
                                                 ko + (uint32_t)(bb * 8 * g.ldb * 2), 0, 0);
      }
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int lrow = lane & 31, lhalf = lane >> 5;
  const int swz = (lrow >> 1) & 7;
  bf16x8 fa[2][FM], fb[2][FN];
  auto lread = [&](int fs, const u32x4* stg, int s) {
    const int ph = (2 * s + lhalf) ^ swz;
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[fs][i] = __builtin_bit_cast(bf16x8, stg[(wm * TM + i * 32 + lrow) * 8 + ph]);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[fs][j] = __builtin_bit_cast(bf16x8, stg[(BM + wn * TN + j * 32 + lrow) * 8 + ph]);
  };
  auto mma = [&](int fs, int i0, int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = SWAP ? mfma32(fb[fs][j], fa[fs][i], acc[i][j]) : mfma32(fa[fs][i], fb[fs][j], acc[i][j]);
  };

  dma(st0, 0);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __builtin_amdgcn_s_barrier();
  lread(0, st0, 0);

  // Each slice is its own scheduling region (sched_barrier), inside which
  // the fragment reads / DMAs are paired one-to-one with the MFMAs.
  auto pair = [&](int n_ds, int n_vm) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k < n_ds) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // MFMA
      if (k < n_vm) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM (LDS DMA)
    }
  };
  auto iter = [&](const u32x4* cur, u32x4* nxt, int kt) {
    // slice 0: next slice's fragments and the whole next-stage DMA
    lread(1, cur, 1);
    dma(nxt, min(kt + 1, nk - 1));
    mma(0, 0, FM);
    pair(8, 16);
    __builtin_amdgcn_sched_barrier(0);
    lread(0, cur, 2);
    mma(1, 0, FM);
    pair(8, 0);
    __builtin_amdgcn_sched_barrier(0);
    lread(1, cur, 3);
    mma(0, 0, FM);
    pair(8, 0);
    __builtin_amdgcn_sched_barrier(0);
    // slice 3: half, barrier (next stage landed and visible), next stage's
    // slice-0 reads under the second half
    mma(1, 0, FM / 2);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    lds_barrier();
    lread(0, nxt, 0);
    mma(1, FM / 2, FM);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    iter(st0, st1, kt);
    iter(st1, st0, kt + 1);
  }
  if (kt < nk) iter(st0, st1, kt);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // drain the final (redundant) DMA before exit

  if (SWAP && EPI != EPI_F32) {
    lds_barrier();   // every wave is done with the stage buffers
    char* reg = reinterpret_cast<char*>((wave < 2 ? st0 : st1)) + (wave & 1) * 32768;
    if (EPI == EPI_RESID) store_tile_lds_f32<false>(g, acc, m0, n0, wm, wn, lane, reg, 0);
    else if (EPI == EPI_PART) store_tile_lds_f32<true>(g, acc, m0, n0, wm, wn, lane, reg, split);
    else if (EPI == EPI_QKV) store_tile_qkv(g, acc, m0, n0, wm, wn, lane, reg);
    else store_tile_lds<(EPI == EPI_SWIGLU ? EPI_SWIGLU : EPI_BF16)>(g, acc, m0, n0, wm, wn, lane, reg);
  } else {
    store_tile<FM, FN, TM, TN, EPI, SWAP>(g, acc, m0, n0, wm, wn, lrow, lhalf);
  }
}

template <int EPI, bool SWAP, bool PACKED = (EPI == EPI_SWIGLU)>
hipError_t run_w4(const GemmArgs& g, hipStream_t s) {
  const int nblk = ((g.M + 255) / 256) * (g.N / 256) * (EPI == EPI_PART ? g.splits : 1);
  hipLaunchKernelGGL((gemm_w4_kernel<EPI, SWAP, PACKED>), dim3(nblk), dim3(256), 0, s, g);
  return hipGetLastError();
}

// Sum of the K-split partial sums part[0..splits) of a (tail) GEMM, then the
// epilogue EPI on it. One thread per 4 consecutive output columns of a row.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g) {
  const int outc = EPI == EPI_SWIGLU ? g.N / 2 : g.N;
  const int per_row = outc / 4;
  const long long q = (long long)blockIdx.x * 256 + threadIdx.x;
  const int m = (int)(q / per_row);
  if (m >= g.M) return;
  const int c = (int)(q - (long long)m * per_row) * 4;
  const size_t MN = (size_t)g.M * g.N;
  auto sum4 = [&](int col) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sp = 0; sp < g.splits; ++sp) {
      const float4 v = *reinterpret_cast<const float4*>(g.part + sp * MN + (size_t)m * g.N + col);
      a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
    }
    return a;
  };
  if (EPI == EPI_SWIGLU) {
    // output feature c is packed column 64*(c/32) + c%32 (gate); up is 32 later
    const int pg = 64 * (c >> 5) + (c & 31);
    const float4 gv = sum4(pg), uv = sum4(pg + 32);
    const float o0 = gv.x / (1.f + __expf(-gv.x)) * uv.x, o1 = gv.y / (1.f + __expf(-gv.y)) * uv.y;
    const float o2 = gv.z / (1.f + __expf(-gv.z)) * uv.z, o3 = gv.w / (1.f + __expf(-gv.w)) * uv.w;
    u32x2 w;
    w.x = pack2bf(o0, o1);
    w.y = pack2bf(o2, o3);
    *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(g.C) + (size_t)m * g.ldc + c) = w;
  } else if (EPI == EPI_BF16) {
    const float4 a = sum4(c);
    u32x2 w;
    w.x = pack2bf(a.x, a.y);
    w.y = pack2bf(a.z, a.w);
    *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(g.C) + (size_t)m * g.ldc + c) = w;
  } else {
    const float4 a = sum4(c);
    const float4 gt = *reinterpret_cast<const float4*>((m < g.n_pre ? g.gate_0 : g.gate_t) + c);
    float4* hp = reinterpret_cast<float4*>(g.Hres + (size_t)m * g.ldh + c);
    float4 h = *hp;
    h.x += gt.x * a.x;
    h.y += gt.y * a.y;
    h.z += gt.z * a.z;
    h.w += gt.w * a.w;
    *hp = h;
  }
}

template <int EPI>
hipError_t run_reduce(const GemmArgs& g, hipStream_t s) {
  const long long n4 = (long long)g.M * ((EPI == EPI_SWIGLU ? g.N / 2 : g.N) / 4);
  hipLaunchKernelGGL((splitk_reduce_kernel<EPI>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, g);
  return hipGetLastError();
}

template <int EPI>
hipError_t run_main(const GemmArgs& g, hipStream_t s) { return run_w4<EPI, true>(g, s); }

hipError_t run_epi(const GemmArgs& g, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_BF16: return run_main<EPI_BF16>(g, s);
    case EPI_RESID: return run_main<EPI_RESID>(g, s);
    case EPI_SWIGLU: return run_main<EPI_SWIGLU>(g, s);
    case EPI_QKV: return run_main<EPI_QKV>(g, s);
  }
  return hipErrorInvalidValue;
}

// The last r row blocks (256 rows each) are computed as `splits` K-split
// GEMMs into g.part and reduced with the epilogue; the rows before them in
// one ordinary launch.
hipError_t launch_gemm_split(const GemmArgs& g, int epi, int r, int splits, hipStream_t s) {
  const int ntm = (g.M + 255) / 256;
  GemmArgs gm = g;
  gm.M = (ntm - r) * 256;
  if (gm.M > 0) {
    const hipError_t e = run_epi(gm, epi, s);
    if (e != hipSuccess) return e;
  }
  GemmArgs gt = g;
  gt.A = g.A + (size_t)gm.M * g.lda;
  gt.M = g.M - gm.M;
  if (g.C) gt.C = reinterpret_cast<bf16_t*>(g.C) + (size_t)gm.M * g.ldc;
  if (g.Hres) gt.Hres = g.Hres + (size_t)gm.M * g.ldh;
  gt.n_pre = g.n_pre - gm.M;
  gt.splits = splits;
  // the partial sums of a SwiGLU GEMM keep its packed gate/up columns
  hipError_t e = epi == EPI_SWIGLU ? run_w4<EPI_PART, true, true>(gt, s) : run_w4<EPI_PART, true, false>(gt, s);
  if (e != hipSuccess) return e;
  switch (epi) {
    case EPI_BF16: return run_reduce<EPI_BF16>(gt, s);
    case EPI_RESID: return run_reduce<EPI_RESID>(gt, s);
    case EPI_SWIGLU: return run_reduce<EPI_SWIGLU>(gt, s);
    case EPI_QKV: {
      // the reduced rows are stored as plain bf16 q|k|v, then normalized,
      // rotated and written to the cache by the standalone kernel
      e = run_reduce<EPI_BF16>(gt, s);
      if (e != hipSuccess) return e;
      QkArgs q = g.qk;
      q.g_begin = q.q_row0 + gm.M;
      q.g_end = q.q_row0 + g.M;
      return launch_qknorm_rope(q, s);
    }
  }
  return hipErrorInvalidValue;
}

template <int WM, int WN, int EPI, bool SWAP = true, int GM = GROUP_M>
hipError_t run_dma(const GemmArgs& g, hipStream_t s) {
  const int nblk = ((g.M + 255) / 256) * (g.N / 256);
  hipLaunchKernelGGL((gemm_dma_kernel<WM, WN, EPI, SWAP, GM>), dim3(nblk), dim3(WM * WN * 64), 0, s, g);
  return hipGetLastError();
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

hipError_t launch_gemm_variant(const GemmArgs& g, int variant, hipStream_t s) {
  switch (variant) {
    case 1: return run<256, 256, 2, 4, EPI_BF16>(g, s);        // register-staged, 2-stage LDS
    case 2: return run_dma<2, 4, EPI_BF16, true>(g, s);        // direct-to-LDS, swapped operands
    case 3: return run_dma<2, 2, EPI_BF16, false>(g, s);       // direct-to-LDS, 4 waves of 128x128
    case 4: return run_w4<EPI_BF16, false>(g, s);              // 4 waves of 128x128, K stages of 64
    case 5: return run_dma<2, 4, EPI_BF16, false>(g, s);       // 8 waves of 128x64
    case 6: {                                                  // split-K path for the last row block
      int sp = 1;
      while (sp < 4 && (g.K / 64) % (2 * sp) == 0) sp *= 2;
      return launch_gemm_split(g, EPI_BF16, 1, sp, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(const GemmArgs& g, int epi, hipStream_t s) {
  if (epi == EPI_F32) return run<64, 64, 2, 2, EPI_F32>(g, s);
  // One block tile per CU per round: when the tiles leave the last round
  // mostly idle and dropping the last r row blocks makes the rest whole
  // rounds, those r row blocks are spread over the idle CUs by splitting K.
  // A GEMM with less than one round of tiles is split whole (r = ntm).
  const int ntm = (g.M + 255) / 256, ntn = g.N / 256;
  constexpr int kRound = 256;
  if (g.part && (ntm * ntn) % kRound) {
    int r = ntm * ntn < kRound ? ntm : 0;
    for (int rr = 1; !r && rr < ntm && rr * ntn <= kRound; ++rr)
      if (((ntm - rr) * ntn) % kRound == 0) { r = rr; break; }
    int splits = 1;
    while (r && 2 * splits * r * ntn <= kRound && (g.K / 64) % (2 * splits) == 0 &&
           (size_t)(2 * splits) * g.N * (size_t)(g.M - (ntm - r) * 256) * 4 <= g.part_bytes)
      splits *= 2;
    if (r && splits > 1) return launch_gemm_split(g, epi, r, splits, s);
  }
  return run_epi(g, epi, s);
}

}  // namespace dit
