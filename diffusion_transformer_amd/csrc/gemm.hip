// bf16 MFMA GEMMs for gfx950: C = A·Bᵀ with A [M,K] and B [N,K] both
// K-contiguous (activations × nn.Linear weights), fp32 accumulation, built
// from v_mfma_f32_32x32x16_bf16 blocks, with fused epilogues (bf16 store,
// gated fp32 residual update, SwiGLU, QK-RMSNorm + RoPE + KV-cache write).
//
// gemm_w4_kernel (every GEMM of a layer): 256x256 block tile, 4 waves of
// 128x128, K in stages of 64 held in two 64 KB LDS stages that are filled
// straight from global memory with buffer_load ... lds one stage ahead.
//
// It uses an XCD-aware tile order: the hardware deals workgroups
// round-robin over the 8 XCDs, so block b is remapped to logical tile
// (b%8)*(n/8) + b/8, giving each XCD a contiguous run of logical tiles;
// logical tiles are then grouped GROUP_M tile-rows at a time so a run
// covers a compact M×N patch whose A and B panels stay in that XCD's L2.
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int BK = 64;
// Tile-rows per group: 4, or 8 for the long-K (K >= 8192) single-round
// down projection, where 8 x 4 tiles per XCD measured 2% faster than 4 x 8
// (4096 x 4096 x 16384: 0.451 -> 0.442 ms); the other layer shapes tie.
constexpr int GROUP_M = 4;
constexpr int GROUP_M_LONG_K = 8;

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
            o[e] = silu_f(gv) * uv;
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
  // The patch's rows through a buffer resource that ends after the last row
  // below M: stores of rows past M are dropped by the bounds check (the row
  // is in the checked per-lane offset), so no store sits behind a branch and
  // the LDS reads of several rows can be in flight at once.
  const int mrow0 = m0 + wm * 128;
  const bf16_t* cbase = reinterpret_cast<const bf16_t*>(g.C) + (size_t)mrow0 * g.ldc +
                        (EPI == EPI_SWIGLU ? (n0 >> 1) + wn * 64 : n0 + wn * 128);
  const uint32_t rowb = (uint32_t)g.ldc * 2u;
  const __amdgpu_buffer_rsrc_t rC = make_rsrc(
      uniform_ptr(cbase),
      (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)max(0, min(128, g.M - mrow0)) * rowb)));
#pragma unroll
  for (int q = 0; q < 128 / RPI; ++q) {
    const int R = q * RPI + lane / CPR;
    const int pc = cc ^ ((R & (SLOTS - 1)) >> 1);
    u32x4 v = *reinterpret_cast<const u32x4*>(reg + R * ROWB + pc * 16);
    if (R & 1) v = (u32x4){v.z, v.w, v.x, v.y};
    __builtin_amdgcn_raw_buffer_store_b128(v, rC, (int)((uint32_t)R * rowb + 16u * cc), 0, 0);
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
    // q rows go to C (row stride ldc), k rows to the head's cache rows
    // (stride 128). The buffer resource ends after the last row below M, so
    // stores of rows past M are dropped by the bounds check and the loop has
    // no per-row branch (the rows interleave freely).
    const bf16_t* dbase = sec == 0 ? C + (size_t)rbase * g.ldc + c0
                                   : a.kc + ((size_t)hh * a.cap + a.q_row0 + rbase) * 128;
    const uint32_t dstride = sec == 0 ? (uint32_t)g.ldc * 2u : 256u;
    const __amdgpu_buffer_rsrc_t rdst =
        make_rsrc(uniform_ptr(dbase), (uint32_t)__builtin_amdgcn_readfirstlane(
                                          (int)((uint32_t)max(0, min(128, g.M - rbase)) * dstride)));
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
      __builtin_amdgcn_raw_buffer_store_b128(ov, rdst, (int)((uint32_t)R * dstride + 16u * cc), 0, 0);
    }
  } else {
    // transposed staging: dim row d (128 tokens, 256 bytes), 16-byte token
    // chunk c at c ^ (d % 16). A lane holds 4 consecutive dims of token t;
    // the pair of lanes with tokens t, t^1 swaps half of them, so that each
    // lane writes 2 dims x 2 tokens as two 4-byte words (the even-token lane
    // dims +0, +1, the odd-token lane dims +2, +3).
    const bool odd = lrow & 1;
    // byte selectors of v_perm over {nb, mine}: the even lane keeps its own
    // low halves in the low half of each word, the odd lane in the high half
    const uint32_t sel_lo = odd ? 0x01000504u : 0x05040100u;
    const uint32_t sel_hi = odd ? 0x03020706u : 0x07060302u;
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
          const uint32_t lo = __builtin_amdgcn_perm(nb, mine, sel_lo);
          const uint32_t hi = __builtin_amdgcn_perm(nb, mine, sel_hi);
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
  // The patch's rows (residual or partial sums) through a buffer resource
  // that ends after the last row below M: rows past M read as zero and their
  // stores are dropped by the bounds check (the row is in the checked
  // per-lane offset), so no load or store sits behind a branch.
  const int mrow0 = m0 + wm * 128;
  const uint32_t rowb = (uint32_t)ldo * 4u;
  const __amdgpu_buffer_rsrc_t rO = make_rsrc(
      uniform_ptr(out + (size_t)mrow0 * ldo + n0 + wn * 128),
      (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)max(0, min(128, g.M - mrow0)) * rowb)));
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int mb = m0 + wm * 128 + hf * 64 + (lane >> 5);
    float4 hv[32];
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const uint32_t off = (uint32_t)(hf * 64 + 2 * t + (lane >> 5)) * rowb + 16u * cc;
      hv[t] = PART ? make_float4(0.f, 0.f, 0.f, 0.f)
                   : __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rO, (int)off, 0, 0));
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
      const uint32_t off = (uint32_t)(hf * 64 + R) * rowb + 16u * cc;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, h), rO, (int)off, 0, 0);
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
// PF > 0 (long K): each stage also prefetches, into L2, this workgroup's share
// of its XCD's A and B slices of stage kt + PF (three 1 KB blocks per wave,
// DMA'd into a small LDS sink nothing reads), and the stage-end wait leaves
// those three loads in flight (loads complete in issue order, so the stage's
// own DMAs, issued before them, have landed).
template <int EPI, bool PACKED = (EPI == EPI_SWIGLU), int PF = 0>
__global__ __launch_bounds__(256) void gemm_w4_kernel(GemmArgs g) {
  static_assert(EPI != EPI_F32, "no fp32-output GEMM in this library (proj_out is fused into the final AdaLN)");
  constexpr int BM = 256, BN = 256, SBK = 64;
  constexpr int WN = 2, TM = 128, TN = 128, FM = 4, FN = 4;
  constexpr int SW = (BM + BN) * SBK / 8;      // u32x4 per stage (64 KB)
  static_assert(EPI != EPI_SWIGLU || (FN % 2 == 0 && TN % 64 == 0), "SwiGLU pairs 32-col blocks");
  __shared__ u32x4 st0[SW], st1[SW];
  __shared__ u32x4 pf_sink[PF ? 4 * 64 : 1];

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
  const int gm = g.K >= 8192 ? GROUP_M_LONG_K : GROUP_M;
  const int in_group = gm * ntn;
  const int gid = b / in_group;
  const int first = gid * gm;
  const int gsz = min(ntm - first, gm);
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
  // The block row goes into the per-lane offset, which the bounds check
  // covers (rows of A past M read as zero without touching memory past A),
  // and the stage's K offset into the scalar one, the same for every DMA.
  auto dma = [&](u32x4* stg, int kt) {
    const uint32_t ko = (uint32_t)((kbeg + kt * SBK) * 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int blk = 4 * j + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, LDSP(stg + blk * 64), 16,
                                               aoff + (uint32_t)(blk * 8 * g.lda * 2), ko, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int bb = 4 * j + wave;
      u32x4* dst = stg + (BM / 8 + bb) * 64;
      if (PACKED) {
        const uint32_t ro = (uint32_t)((32 * (j >> 1) + 8 * wave) * g.ldb * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds((j & 1) ? rU : rG, LDSP(dst), 16, boff + ro, ko, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rG, LDSP(dst), 16, boff + (uint32_t)(bb * 8 * g.ldb * 2), ko,
                                                 0, 0);
      }
    }
  };

  // The XCD's tile block is gm tile-rows by 32/gm tile-columns (one round of
  // 32 tiles): the workgroup at local column c prefetches blocks of its A
  // slice, the one at local row r blocks of its B slice, so the 32 workgroups
  // cover the XCD's slices once.
  auto prefetch = [&](int kt) {
    const int lrow_t = (m0 / BM) % gm, lcol_t = (n0 / BN) % (32 / gm);
    const uint32_t ko = (uint32_t)((kbeg + kt * SBK) * 2);
    const int na = gm / 4, nb = 8 / gm;   // A and B blocks per wave (gm = 4 or 8)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (j < na) {
        const int blk = lcol_t * (4 * na) + wave * na + j;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, LDSP(pf_sink + wave * 64), 16,
                                                 aoff + (uint32_t)(blk * 8 * g.lda * 2), ko, 0, 0);
      }
      if (j < nb) {
        const int bb = lrow_t * (4 * nb) + wave * nb + j;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rG, LDSP(pf_sink + wave * 64), 16,
                                                 boff + (uint32_t)((PACKED ? (bb >> 1) : bb) * 8 * g.ldb * 2), ko,
                                                 0, 0);
      }
    }
  };

  f32x16 acc[FM][FN];

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
        acc[i][j] = mfma32(fb[fs][j], fa[fs][i], acc[i][j]);   // operands swapped: Cᵀ blocks
  };

  dma(st0, 0);
  // the 256 accumulator registers are cleared while the first stage is in
  // flight: the empty asm takes each cleared block as an accumulator-register
  // operand here, so the clearing cannot sink below the wait
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
      asm volatile("" : "+a"(acc[i][j]));
    }
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
    if constexpr (PF > 0) prefetch(min(kt + PF, nk - 1));
    mma(1, 0, FM);
    pair(8, PF ? 3 : 0);
    __builtin_amdgcn_sched_barrier(0);
    lread(1, cur, 3);
    mma(0, 0, FM);
    pair(8, 0);
    __builtin_amdgcn_sched_barrier(0);
    // slice 3: half, barrier (next stage landed and visible), next stage's
    // slice-0 reads under the second half
    mma(1, 0, FM / 2);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(PF ? 3 : 0));
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

  lds_barrier();   // every wave is done with the stage buffers
  char* reg = reinterpret_cast<char*>((wave < 2 ? st0 : st1)) + (wave & 1) * 32768;
  if (EPI == EPI_RESID) store_tile_lds_f32<false>(g, acc, m0, n0, wm, wn, lane, reg, 0);
  else if (EPI == EPI_PART) store_tile_lds_f32<true>(g, acc, m0, n0, wm, wn, lane, reg, split);
  else if (EPI == EPI_QKV) store_tile_qkv(g, acc, m0, n0, wm, wn, lane, reg);
  else store_tile_lds<(EPI == EPI_SWIGLU ? EPI_SWIGLU : EPI_BF16)>(g, acc, m0, n0, wm, wn, lane, reg);
}

// Persistent form of gemm_w4_kernel<EPI_SWIGLU> (the gate/up projection):
// the same tiles, main loop and epilogue, for whole rounds of tiles and an
// even number of K stages. The grid is one workgroup per CU, and each walks
// the tiles launch order would have dealt to its slot: virtual block
// b = blockIdx.x + r * gridDim.x for r = 0, 1, ..., so the same XCD works
// on the same logical tiles. The last K stage of a tile fetches the first
// stage of the next into st0 and the epilogue stages its 128 x 64 bf16
// patch per wave in st1 only, so a tile starts without waiting on memory
// and without a workgroup turnover.
__global__ __launch_bounds__(256) void gemm_w4p_swiglu_kernel(GemmArgs g) {
  constexpr int BM = 256, BN = 256, SBK = 64;
  constexpr int WN = 2, TM = 128, TN = 128, FM = 4, FN = 4;
  constexpr int SW = (BM + BN) * SBK / 8;      // u32x4 per stage (64 KB)
  __shared__ u32x4 st0[SW], st1[SW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  const int ntm = (g.M + BM - 1) / BM;
  const int ntn = g.N / BN;
  const int nblk = ntm * ntn;                  // virtual blocks = tiles
  const int per = nblk >> 3;
  const int gm = g.K >= 8192 ? GROUP_M_LONG_K : GROUP_M;
  const int in_group = gm * ntn;
  auto tile_of = [&](int b, int& m0_, int& n0_) {
    if (b < per * 8) b = (b & 7) * per + (b >> 3);
    const int first = (b / in_group) * gm;
    const int gsz = min(ntm - first, gm);
    m0_ = (first + (b % in_group) % gsz) * BM;
    n0_ = ((b % in_group) / gsz) * BN;
  };
  int vb = blockIdx.x;
  int m0, n0;
  tile_of(vb, m0, n0);
  const int nk = g.K / SBK;

  // DMA as in gemm_w4_kernel. `ln` is the lane id, made opaque again at the
  // start of every tile, so the per-lane offsets are derived per tile rather
  // than held in registers across the epilogue.
  int ln = lane;
  auto lane_off = [&](int ld) {
    const int lr = ln >> 3;
    const int lc = (ln & 7) ^ ((4 * (wave & 1) + (ln >> 4)) & 7);
    return (uint32_t)((lr * ld + lc * 8) * 2);
  };
  const uint32_t bbytes = (uint32_t)min((size_t)(BN / 2) * g.ldb * 2, (size_t)0xFFFFFFF0u);
  auto rsrc_a = [&](int m0_) {
    return make_rsrc(g.A + (size_t)m0_ * g.lda, (uint32_t)min((size_t)(g.M - m0_) * g.lda * 2, (size_t)0xFFFFFFF0u));
  };
  __amdgpu_buffer_rsrc_t rA = rsrc_a(m0);
  __amdgpu_buffer_rsrc_t rG = make_rsrc(g.B + (size_t)(n0 >> 1) * g.ldb, bbytes);
  __amdgpu_buffer_rsrc_t rU = make_rsrc(g.B2 + (size_t)(n0 >> 1) * g.ldb, bbytes);
  // ko: byte offset of the stage's first K column (the same for every DMA)
  auto dma = [&](u32x4* stg, uint32_t ko) {
    const uint32_t aoff = lane_off(g.lda), boff = lane_off(g.ldb);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int blk = 4 * j + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, LDSP(stg + blk * 64), 16,
                                               aoff + (uint32_t)(blk * 8 * g.lda * 2), ko, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4* dst = stg + (BM / 8 + 4 * j + wave) * 64;
      const uint32_t ro = (uint32_t)((32 * (j >> 1) + 8 * wave) * g.ldb * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds((j & 1) ? rU : rG, LDSP(dst), 16, boff + ro, ko, 0, 0);
    }
  };

  f32x16 acc[FM][FN];
  bf16x8 fa[2][FM], fb[2][FN];
  auto lread = [&](int fs, const u32x4* stg, int s) {
    const int lrow = ln & 31, lhalf = ln >> 5;
    const int ph = (2 * s + lhalf) ^ ((lrow >> 1) & 7);
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[fs][i] = __builtin_bit_cast(bf16x8, stg[(wm * TM + i * 32 + lrow) * 8 + ph]);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[fs][j] = __builtin_bit_cast(bf16x8, stg[(BM + wn * TN + j * 32 + lrow) * 8 + ph]);
  };
  // init: the tile's first MFMA on each block starts from zero (no clearing)
  auto mma = [&](int fs, int i0, int i1, bool init = false) {
#pragma unroll
    for (int i = i0; i < i1; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = mfma32(fb[fs][j], fa[fs][i], init ? f32x16{} : acc[i][j]);   // swapped: Cᵀ blocks
  };
  auto pair = [&](int n_ds, int n_vm) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k < n_ds) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // MFMA
      if (k < n_vm) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM (LDS DMA)
    }
  };
  // one K stage as in gemm_w4_kernel; its DMA fetches the stage at ko_dma.
  // `first`: the tile's first stage, whose slice 0 initializes every block.
  auto iter = [&](const u32x4* cur, u32x4* nxt, uint32_t ko_dma, bool first = false) {
    lread(1, cur, 1);
    dma(nxt, ko_dma);
    mma(0, 0, FM, first);
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
  auto ko = [&](int kt) { return (uint32_t)(kt * SBK * 2); };

  for (bool first_tile = true;; first_tile = false) {
    asm volatile("" : "+v"(ln));
    if (first_tile) dma(st0, 0);
    if (first_tile) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      __builtin_amdgcn_s_barrier();
    } else {
      // stage 0 landed before the previous tile's last barrier; this one
      // orders the previous epilogue's LDS reads before the DMA into st1
      lds_barrier();
    }
    lread(0, st0, 0);

    // nk is even: stage 0 is read from st0, the last stage (odd) from st1,
    // and the last stage's DMA fills st0 with the next tile's first stage
    // (or, with no next tile, repeats the last stage, never read)
    iter(st0, st1, ko(1), true);
    for (int kt = 1; kt + 2 < nk; kt += 2) {
      iter(st1, st0, ko(kt + 1));
      iter(st0, st1, ko(kt + 2));
    }
    const int vn = vb + (int)gridDim.x;
    const bool has_next = vn < nblk;
    int m0n = m0, n0n = n0;
    uint32_t ko_last = ko(nk - 1);
    if (has_next) {
      // the buffer resources switch to the next tile for the last DMA
      tile_of(vn, m0n, n0n);
      rA = rsrc_a(m0n);
      rG = make_rsrc(g.B + (size_t)(n0n >> 1) * g.ldb, bbytes);
      rU = make_rsrc(g.B2 + (size_t)(n0n >> 1) * g.ldb, bbytes);
      ko_last = 0;
    }
    iter(st1, st0, ko_last);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

    lds_barrier();   // every wave is done with the stage buffers
    // st0 holds the next tile's first stage: the patch goes to st1 only
    store_tile_lds<EPI_SWIGLU>(g, acc, m0, n0, wm, wn, lane, reinterpret_cast<char*>(st1) + wave * 16384);
    if (!has_next) break;
    vb = vn;
    m0 = m0n;
    n0 = n0n;
  }
}

template <int EPI, bool PACKED = (EPI == EPI_SWIGLU)>
hipError_t run_w4(const GemmArgs& g, hipStream_t s, const LaunchEvents& ev = {}) {
  const int nblk = ((g.M + 255) / 256) * (g.N / 256) * (EPI == EPI_PART ? g.splits : 1);
  if (EPI == EPI_SWIGLU) {
    // Persistent grid when the tiles are whole rounds of at least two (one
    // workgroup per CU, 8 XCDs) and the K stages are even in number (the
    // next tile's first stage then lands in st0).
    const int cus = device_cus();
    if (cus > 0 && cus % 8 == 0 && nblk % cus == 0 && nblk >= 2 * cus && (g.K / 64) % 2 == 0) {
      launch_k(gemm_w4p_swiglu_kernel, dim3(cus), dim3(256), s, ev.start, ev.stop, g);
      return hipGetLastError();
    }
  }
  if constexpr (EPI == EPI_RESID || EPI == EPI_BF16) {
    if (g.K >= 8192) {
      // Long K (the down projection, K = ffn): L2 prefetch two stages ahead.
      // Measured on 4096 x 16384 x 4096: 0.4405 -> 0.4278 ms; at K = 4096 it
      // slowed the QKV and O projections by 3.5-4.5%, so it stays off there.
      launch_k((gemm_w4_kernel<EPI, PACKED, 2>), dim3(nblk), dim3(256), s, ev.start, ev.stop, g);
      return hipGetLastError();
    }
  }
  launch_k((gemm_w4_kernel<EPI, PACKED>), dim3(nblk), dim3(256), s, ev.start, ev.stop, g);
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
    const float o0 = silu_f(gv.x) * uv.x, o1 = silu_f(gv.y) * uv.y;
    const float o2 = silu_f(gv.z) * uv.z, o3 = silu_f(gv.w) * uv.w;
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

hipError_t run_epi(const GemmArgs& g, int epi, hipStream_t s, const LaunchEvents& ev = {}) {
  switch (epi) {
    case EPI_BF16: return run_w4<EPI_BF16>(g, s, ev);
    case EPI_RESID: return run_w4<EPI_RESID>(g, s, ev);
    case EPI_SWIGLU: return run_w4<EPI_SWIGLU>(g, s, ev);
    case EPI_QKV: return run_w4<EPI_QKV>(g, s, ev);
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
  hipError_t e = epi == EPI_SWIGLU ? run_w4<EPI_PART, true>(gt, s) : run_w4<EPI_PART, false>(gt, s);
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

}  // namespace

bool gemm_shape_ok(int M, int N, int K, int epi) {
  if (M <= 0 || N <= 0 || K <= 0 || K % BK || epi == EPI_F32) return false;
  return N % 256 == 0;
}

hipError_t launch_gemm_forced_split(const GemmArgs& g, int epi, int splits, hipStream_t s) {
  return launch_gemm_split(g, epi, 1, splits, s);
}

hipError_t launch_gemm(const GemmArgs& g, int epi, hipStream_t s, const LaunchEvents& ev) {
  if (epi == EPI_F32) return hipErrorInvalidValue;
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
    if (r && splits > 1) {
      if (ev.start) (void)hipEventRecord(ev.start, s);
      const hipError_t e = launch_gemm_split(g, epi, r, splits, s);
      if (ev.stop) (void)hipEventRecord(ev.stop, s);
      return e;
    }
  }
  return run_epi(g, epi, s, ev);
}

}  // namespace dit
