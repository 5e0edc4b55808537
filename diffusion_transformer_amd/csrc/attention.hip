// Flash-style attention for head_dim 128 on gfx950 bf16 MFMA, with the
// block-causal mask in row-limit form (key j visible to query i iff
// j <= limit[i]); masked keys get exactly zero weight.
//
// Scores are computed transposed, Sᵀ = K·Qᵀ (32 keys × 32 queries
// per MFMA block), so each lane holds keys of ONE query and the row max/sum
// need in-lane work plus one exchange between the wave halves; the output is
// accumulated transposed as well, Oᵀ = Vᵀ·Pᵀ, which lets the probabilities
// feed the MFMA B operand straight from registers. V is kept transposed
// (dim-major) in the cache. Waves whose queries see none of a key tile skip
// its arithmetic; tiles past the workgroup's largest limit are never loaded.
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int D = 128;
constexpr int BKV = 64;

// ---------------------------------------------------------------------------
// attn2_kernel<NWV, QW, NST>: NWV waves, QW queries per wave, NST stages.
//  - each wave owns QW queries (QW/32 sub-blocks of 32) that share every K
//    and Vᵀ fragment read, halving LDS traffic per FLOP at QW = 64;
//  - K rows enter the score MFMA in the order π(i) = i with bits 2 and 3
//    swapped, so that for every 16-key chunk a lane half holds 8 CONTIGUOUS
//    keys of its query: the Vᵀ operand is then one 16-byte LDS read;
//  - K / Vᵀ tiles are fetched straight into LDS (buffer_load ... lds) into
//    a ring of 3 stages, two tiles ahead, one barrier per tile;
//  - the running max is only raised when a query's tile max exceeds it by
//    more than 2^8 (wave-uniform decision), so O and l are rescaled rarely;
//    probabilities stay below 2^8 and the final O/l is unchanged;
//  - optionally, the last (head, query block) units of the grid are split
//    over key ranges (AttnArgs::split_*): each piece writes its normalized
//    O and log2-sum-exp in fp32 and attn_combine_kernel merges them. With
//    every unit streaming the same keys (target rows of a cached step) this
//    turns a last, partly filled round of workgroups into a shorter one.

// max over the two 32-lane halves of the wave (v_permlane32_swap, no LDS)
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

__device__ __forceinline__ int perm23(int x) {   // swap bits 2 and 3
  return (x & ~0xC) | ((x & 4) << 1) | ((x & 8) >> 1);
}

template <int NWV, int QW, int NST>
__global__ __launch_bounds__(NWV * 64, (NWV == 4 && NST == 2) ? 2 : 1) void attn2_kernel(AttnArgs a) {
  constexpr int NSB = QW / 32;          // 32-query sub-blocks per wave
  constexpr int KAHEAD = 6;             // K fragment reads in flight
  constexpr int BQ2 = NWV * QW;
  constexpr int KT = BKV * 16;          // u32x4 per K tile (64 keys x 256 B)
  constexpr int VT = D * 8;             // u32x4 per Vᵀ tile (128 dims x 128 B)
  constexpr int DMA_PER_WAVE = 32 / NWV;   // 16 K + 16 Vᵀ 1-KB blocks per tile
  static_assert(32 % NWV == 0 && (DMA_PER_WAVE % 2) == 0, "DMA split");
  static_assert(NST == 2 || NST == 3, "ring of 2 or 3 stages");
  __shared__ u32x4 k0s[KT], k1s[KT], k2s[NST == 3 ? KT : 1];
  __shared__ u32x4 v0s[VT], v1s[VT], v2s[NST == 3 ? VT : 1];
  __shared__ int red[NWV];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroups are dealt to the 8 XCDs round-robin; renumber them so that
  // each XCD gets a contiguous run of (head, query block) pairs and its L2
  // serves the K/Vᵀ of a few heads instead of all of them.
  const int nqb = (a.N + BQ2 - 1) / BQ2;
  int bid = blockIdx.x, piece = -1;
  if (a.split_s > 1 && bid >= a.split_base) {
    // piece of a split unit: consecutive blocks are the key ranges of one unit
    piece = bid - a.split_base;
    bid = a.split_base + piece / a.split_s;
  } else {
    const int nwhole = a.split_s > 1 ? a.split_base : (int)gridDim.x;
    if ((nwhole & 7) == 0) bid = (bid & 7) * (nwhole >> 3) + (bid >> 3);
  }
  const int h = bid / nqb;
  const int qblk = a.rev_q ? nqb - 1 - (bid - h * nqb) : bid - h * nqb;
  const int lq = lane & 31, half = lane >> 5;
  // Target element of this workgroup's queries (one element per workgroup:
  // with several elements P and T_el are multiples of the query block): its
  // query rows and its cached keys past the prefix sit e*T_el rows further
  // than the logical rows of the layout.
  const int gq0 = a.q_off + qblk * BQ2;
  const int eoff = (a.T_el > 0 && gq0 >= a.P) ? (gq0 - a.P) / a.T_el * a.T_el : 0;

  int qi[NSB], lim[NSB];
  bool qv[NSB];
  int lmin = 1 << 30, lmax = -1;
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) {
    const int q = qblk * BQ2 + wave * QW + sb * 32 + lq;
    qv[sb] = q < a.N;
    qi[sb] = min(q, a.N - 1);
    lim[sb] = a.limit[a.q_off + qi[sb] - eoff];
    lmin = min(lmin, lim[sb]);
    lmax = max(lmax, lim[sb]);
  }
  const int wlim_min = __builtin_amdgcn_readfirstlane(wave_min_i(lmin));
  const int wlim_max = __builtin_amdgcn_readfirstlane(wave_max_i(lmax));
  if (lane == 0) red[wave] = wlim_max;
  __syncthreads();
  int blim_max = red[0];
#pragma unroll
  for (int w = 1; w < NWV; ++w) blim_max = max(blim_max, red[w]);
  const int kv_end = min(a.S, blim_max + 1);
  const int ntiles_all = (kv_end + BKV - 1) / BKV;
  // a piece j of a split unit takes key tiles [j*n/s, (j+1)*n/s)
  int ntiles = ntiles_all, kt0 = 0;
  if (piece >= 0) {
    const int j = piece % a.split_s;
    const int t_lo = j * ntiles_all / a.split_s;
    ntiles = (j + 1) * ntiles_all / a.split_s - t_lo;
    kt0 = t_lo * BKV;
  }

  bf16x8 qf[NSB][8];
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) {
    const u32x4* qp = reinterpret_cast<const u32x4*>(a.q + (size_t)qi[sb] * a.q_stride + h * D);
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[sb][s] = __builtin_bit_cast(bf16x8, qp[2 * s + half]);
  }

  // ---- DMA setup: wave w loads K blocks w, w+NWV, ... (4 keys each) and Vᵀ
  // blocks likewise (8 dims each); lane offsets bake in the swizzles ----
  const __amdgpu_buffer_rsrc_t rK = make_rsrc(a.k + (size_t)h * a.cap * D, (uint32_t)(a.cap * D * 2));
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(a.vt + (size_t)h * D * a.cap, (uint32_t)(a.cap * D * 2));
  // K block blk holds keys 4blk + l/16; lane writes physical chunk l%16 of
  // that row, which must hold logical chunk (l%16) ^ (row%16).
  uint32_t koff[4];
#pragma unroll
  for (int b4 = 0; b4 < 4; ++b4) {
    const int r = lane >> 4;
    const int c = (lane & 15) ^ ((4 * b4 + r) & 15);
    koff[b4] = (uint32_t)(r * 256 + c * 16);
  }
  // Vᵀ block blk holds dims 8blk + l/8; physical 16-byte chunk l%8 holds
  // logical chunk (l%8) ^ ((dim/2)%8).
  uint32_t voff[2];
#pragma unroll
  for (int b2 = 0; b2 < 2; ++b2) {
    const int r = lane >> 3;
    const int c = (lane & 7) ^ (((8 * b2 + r) >> 1) & 7);
    voff[b2] = (uint32_t)(r * a.cap * 2 + c * 16);
  }
  // tile of logical keys kv0 .. kv0+63 (P is a multiple of 64 whenever the
  // element offset is non-zero, so a tile never straddles the prefix end)
  auto dma = [&](u32x4* ks, u32x4* vs, int kv0) {
    const int kp = kv0 >= a.P ? kv0 + eoff : kv0;
#pragma unroll
    for (int j = 0; j < DMA_PER_WAVE / 2; ++j) {
      const int blk = j * NWV + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, LDSP(ks + blk * 64), 16, koff[blk & 3],
                                               (uint32_t)((kp + 4 * blk) * 256), 0, 0);
    }
#pragma unroll
    for (int j = 0; j < DMA_PER_WAVE / 2; ++j) {
      const int blk = j * NWV + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, LDSP(vs + blk * 64), 16, voff[blk & 1],
                                               (uint32_t)(8 * blk * a.cap * 2 + kp * 2), 0, 0);
    }
  };

  f32x16 oacc[NSB][4];
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[sb][j][r] = 0.f;
  float m_run[NSB], l_run[NSB];
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) { m_run[sb] = -INFINITY; l_run[sb] = 0.f; }
  const float sl2 = 1.4426950408889634f * 0.08838834764831845f;   // log2(e)/sqrt(128)

  // Scores, mask and online softmax of one key tile (K in ks): the bf16
  // probabilities go to pk; false when no query of the wave sees the tile.
  auto scores = [&](const u32x4* ks, int kv0, uint32_t (&pk)[NSB][2][8]) -> bool {
    const int cls = tile_class<BKV>(kv0, wlim_min, wlim_max, a.S);
    if (cls == 0) return false;
    f32x16 sacc[NSB][2];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[sb][kb][r] = 0.f;
    // Sᵀ = K·Qᵀ. All 16 K fragments are requested up front and consumed in
    // order, so LDS latency hides behind the MFMA chain (KAHEAD reads ahead).
    bf16x8 kf[8][2];
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = perm23(kb * 32 + lq);
        kf[s][kb] = __builtin_bit_cast(bf16x8, ks[row * 16 + ((2 * s + half) ^ (row & 15))]);
      }
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) sacc[sb][kb] = mfma32(kf[s][kb], qf[sb][s], sacc[sb][kb]);
    __builtin_amdgcn_sched_group_barrier(0x100, KAHEAD, 0);
#pragma unroll
    for (int i = 0; i < 16 - KAHEAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, NSB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, KAHEAD * NSB, 0);
    // masking only on tiles that straddle some query's limit (wave-uniform)
    if (cls == 2) {
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = kv0 + perm23(kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3));
            if (!key_visible(j, lim[sb], a.S)) sacc[sb][kb][r] = -INFINITY;
          }
    }
    // Scores stay unscaled; the softmax scale log2(e)/sqrt(d) > 0 commutes
    // with the max and is folded into the exponent: p = 2^(s*c - m).
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[sb][kb][r]);
      mt = half_max(mt) * sl2;
      // raise the running max only when some query of the wave needs it
      if (__builtin_amdgcn_ballot_w64(mt > m_run[sb] + 8.f)) {
        const float m_new = fmaxf(m_run[sb], mt);
        // a query that has seen no key yet keeps m = -inf and alpha = 1
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[sb] - m_new);
        m_run[sb] = m_new;
        l_run[sb] *= alpha;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[sb][j][r] *= alpha;
      }
      // (m = -inf: every score so far is -inf and every p below is 0; a key
      // range that starts past key 0 can have such queries)
      const float nm = m_run[sb] == -INFINITY ? 0.f : -m_run[sb];
      float ls = l_run[sb];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[sb][kb][r], sl2, nm));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[sb][kb][r + 1], sl2, nm));
          const uint32_t w = pack2bf(p0, p1);
          pk[sb][kb][r >> 1] = w;
          // the row sum takes the same bf16-rounded p the PV product uses
          ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), kOnes2, ls, false);
        }
      l_run[sb] = ls;
    }
    return true;
  };
  // Oᵀ += Vᵀ·Pᵀ for one key tile (Vᵀ in vs): chunk c = registers 8(c%2).. of
  // key block c/2, which (through π) are keys 16c + 8*half + {0..7} of this
  // lane's query
  auto pv = [&](const u32x4* vs, const uint32_t (&pk)[NSB][2][8]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8 pf[NSB];
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        u32x4 pb;
        pb.x = pk[sb][c >> 1][4 * (c & 1) + 0];
        pb.y = pk[sb][c >> 1][4 * (c & 1) + 1];
        pb.z = pk[sb][c >> 1][4 * (c & 1) + 2];
        pb.w = pk[sb][c >> 1][4 * (c & 1) + 3];
        pf[sb] = __builtin_bit_cast(bf16x8, pb);
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int e = db * 32 + lq;
        const bf16x8 vf = __builtin_bit_cast(bf16x8, vs[e * 8 + ((2 * c + half) ^ ((e >> 1) & 7))]);
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) oacc[sb][db] = mfma32(vf, pf[sb], oacc[sb][db]);
      }
    }
  };

  const int last = max(ntiles - 1, 0);
  if constexpr (NST == 3) {
    // ring of 3 stages: tile t lives in stage t%3; tiles t+1, t+2 in flight
    constexpr int PER_TILE = DMA_PER_WAVE;   // DMA instructions per wave per tile
    auto wait_barrier = [&]() {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(PER_TILE));   // tile t+1 landed, t+2 may fly
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_barrier();
    };
    if (ntiles > 0) {
      dma(k0s, v0s, kt0);
      dma(k1s, v1s, kt0 + min(1, last) * BKV);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(PER_TILE));
      __builtin_amdgcn_s_barrier();
    }
    // iteration on tile t in stage A: issue tile t+2 into stage C (its last
    // reader, tile t-1, finished before the previous barrier), compute, then
    // barrier so tile t+1 (stage B) is visible.
    auto iter = [&](u32x4* kA, u32x4* vA, u32x4* kC, u32x4* vC, int t) {
      dma(kC, vC, kt0 + min(t + 2, last) * BKV);
      uint32_t pk[NSB][2][8];
      if (scores(kA, kt0 + t * BKV, pk)) pv(vA, pk);
      wait_barrier();
    };
    int t = 0;
    for (; t + 2 < ntiles; t += 3) {
      iter(k0s, v0s, k2s, v2s, t);
      iter(k1s, v1s, k0s, v0s, t + 1);
      iter(k2s, v2s, k1s, v1s, t + 2);
    }
    if (t < ntiles) iter(k0s, v0s, k2s, v2s, t);
    if (t + 1 < ntiles) iter(k1s, v1s, k0s, v0s, t + 1);
  } else {
    // double buffer (64 KB, so two workgroups share a CU and their barriers
    // fall at different times): tile t+1 is fetched into the other stage,
    // whose previous tile was read before the last barrier
    if (ntiles > 0) {
      dma(k0s, v0s, kt0);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      __builtin_amdgcn_s_barrier();
    }
    auto iter = [&](u32x4* kA, u32x4* vA, u32x4* kB, u32x4* vB, int t) {
      dma(kB, vB, kt0 + min(t + 1, last) * BKV);
      uint32_t pk[NSB][2][8];
      if (scores(kA, kt0 + t * BKV, pk)) pv(vA, pk);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_barrier();
    };
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
      iter(k0s, v0s, k1s, v1s, t);
      iter(k1s, v1s, k0s, v0s, t + 1);
    }
    if (t < ntiles) iter(k0s, v0s, k1s, v1s, t);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

  if (piece >= 0) {
    // ---- split piece: normalized O and log2(sum 2^(s*c)) of its keys, fp32;
    // a piece that saw no key leaves O = 0 and -inf ----
    const int npieces = (int)gridDim.x - a.split_base;
    float* po = a.part + (size_t)piece * BQ2 * D;
    float* pl = a.part + (size_t)npieces * BQ2 * D + (size_t)piece * BQ2;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
      const float l_tot = l_run[sb] + __shfl_xor(l_run[sb], 32, 64);
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      const int rl = wave * QW + sb * 32 + lq;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = db * 32 + 8 * g + 4 * half;
          f32x4 w;
          w[0] = oacc[sb][db][4 * g + 0] * inv;
          w[1] = oacc[sb][db][4 * g + 1] * inv;
          w[2] = oacc[sb][db][4 * g + 2] * inv;
          w[3] = oacc[sb][db][4 * g + 3] * inv;
          *reinterpret_cast<f32x4*>(po + (size_t)rl * D + d0) = w;
        }
      if (half == 0) pl[rl] = l_tot > 0.f ? m_run[sb] + __log2f(l_tot) : -INFINITY;
    }
    return;
  }

  // ---- normalize and store O[query][dim] ----
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) {
    const float l_tot = l_run[sb] + __shfl_xor(l_run[sb], 32, 64);
    const float inv = 1.f / l_tot;
    if (qv[sb]) {
      uint16_t* op = a.out + (size_t)qi[sb] * a.out_stride + h * D;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = db * 32 + 8 * g + 4 * half;
          u32x2 w;
          w.x = pack2bf(oacc[sb][db][4 * g + 0] * inv, oacc[sb][db][4 * g + 1] * inv);
          w.y = pack2bf(oacc[sb][db][4 * g + 2] * inv, oacc[sb][db][4 * g + 3] * inv);
          *reinterpret_cast<u32x2*>(op + d0) = w;
        }
    }
  }
}

// ---------------------------------------------------------------------------
// attn3_kernel: the cached step's attention, software-pipelined inside each
// wave. Target rows of a cached step see every key, so no tile needs a mask
// (the launcher uses this kernel only when S is a multiple of 64).
// 8 waves of 32 queries (two per SIMD). For tile t a wave issues, in 32
// fixed slots, the score MFMAs of tile t+1 and the P·V MFMAs of tile t-1 on
// the matrix core, and the softmax of tile t (row max, lazy rescale
// decision, exponentials, bf16 packing, row sums) on the vector ALU; the
// three are independent, so the two units work at the same time. A raised
// running max rescales O after the P·V of tile t-1 has landed in it, which
// is the same product attn2_kernel forms (it rescales before the P·V of
// tile t), so per query the two kernels agree bit for bit.
// K and Vᵀ tiles come straight to LDS in rings of 4 stages each, K three
// tiles ahead of its score use and Vᵀ two tiles ahead of its P·V use; one
// barrier per tile.
__global__ __launch_bounds__(512, 1) void attn3_kernel(AttnArgs a) {
  constexpr int NWV = 8, BQ2 = 256;
  constexpr int KT = BKV * 16, VT = D * 8;
  constexpr int HALF = 16 / NWV;          // 1-KB DMA blocks per wave for one K (or Vᵀ) tile
  __shared__ u32x4 k0s[KT], k1s[KT], k2s[KT], k3s[KT];
  __shared__ u32x4 v0s[VT], v1s[VT], v2s[VT], v3s[VT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nqb = (a.N + BQ2 - 1) / BQ2;
  int bid = blockIdx.x, piece = -1;
  if (a.split_s > 1 && bid >= a.split_base) {
    piece = bid - a.split_base;
    bid = a.split_base + piece / a.split_s;
  } else {
    const int nwhole = a.split_s > 1 ? a.split_base : (int)gridDim.x;
    if ((nwhole & 7) == 0) bid = (bid & 7) * (nwhole >> 3) + (bid >> 3);
  }
  const int h = bid / nqb;
  const int qblk = bid - h * nqb;
  const int lq = lane & 31, half = lane >> 5;
  const int gq0 = a.q_off + qblk * BQ2;
  const int eoff = (a.T_el > 0 && gq0 >= a.P) ? (gq0 - a.P) / a.T_el * a.T_el : 0;
  const int q = qblk * BQ2 + wave * 32 + lq;
  const bool qvalid = q < a.N;
  const int qi = min(q, a.N - 1);
  // every target row of a cached step sees all S keys
  const int ntiles_all = a.S / BKV;
  int ntiles = ntiles_all, kt0 = 0;
  if (piece >= 0) {
    const int j = piece % a.split_s;
    const int t_lo = j * ntiles_all / a.split_s;
    ntiles = (j + 1) * ntiles_all / a.split_s - t_lo;
    kt0 = t_lo * BKV;
  }

  bf16x8 qf[8];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(a.q + (size_t)qi * a.q_stride + h * D);
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = __builtin_bit_cast(bf16x8, qp[2 * s + half]);
  }

  const __amdgpu_buffer_rsrc_t rK = make_rsrc(a.k + (size_t)h * a.cap * D, (uint32_t)(a.cap * D * 2));
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(a.vt + (size_t)h * D * a.cap, (uint32_t)(a.cap * D * 2));
  // the blocks a wave moves (wave, wave + 8) share their swizzle phase
  uint32_t koff, voff;
  {
    const int r = lane >> 4;
    koff = (uint32_t)(r * 256 + ((lane & 15) ^ ((4 * (wave & 3) + r) & 15)) * 16);
    const int rv = lane >> 3;
    voff = (uint32_t)(rv * a.cap * 2 + ((lane & 7) ^ (((8 * (wave & 1) + rv) >> 1) & 7)) * 16);
  }
  const int last = max(ntiles - 1, 0);
  auto key0 = [&](int t) {
    const int kv0 = kt0 + min(t, last) * BKV;
    return kv0 >= a.P ? kv0 + eoff : kv0;
  };
  auto dma_k = [&](u32x4* ks, int t) {
    const int kp = key0(t);
#pragma unroll
    for (int j = 0; j < HALF; ++j) {
      const int blk = j * NWV + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, LDSP(ks + blk * 64), 16, koff,
                                               (uint32_t)((kp + 4 * blk) * 256), 0, 0);
    }
  };
  auto dma_v = [&](u32x4* vs, int t) {
    const int kp = key0(t);
#pragma unroll
    for (int j = 0; j < HALF; ++j) {
      const int blk = j * NWV + wave;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, LDSP(vs + blk * 64), 16, voff,
                                               (uint32_t)(8 * blk * a.cap * 2 + kp * 2), 0, 0);
    }
  };

  f32x16 oacc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[j][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = 1.4426950408889634f * 0.08838834764831845f;   // log2(e)/sqrt(128)

  // Byte offsets of a lane's fragments within a K stage (K step s; key half
  // kb adds 8 KB) and a Vᵀ stage (key chunk c; dim block db adds 4 KB). They
  // are re-declared opaque at every tile so the compiler keeps these 12 and
  // folds stage and block into the instruction offsets, rather than holding
  // an address per stage.
  uint32_t ka[8], va[4];
  {
    const int row = perm23(lq);
#pragma unroll
    for (int s = 0; s < 8; ++s) ka[s] = (uint32_t)((row * 16 + ((2 * s + half) ^ (row & 15))) * 16);
#pragma unroll
    for (int c = 0; c < 4; ++c) va[c] = (uint32_t)((lq * 8 + ((2 * c + half) ^ ((lq >> 1) & 7))) * 16);
  }
  auto frag = [](const u32x4* stage, uint32_t off) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(stage) + off));
  };
  // score MFMAs of one 32-key half kb of a tile (a chain of 8 K steps)
  auto smfma = [&](const u32x4* ks, int kb, f32x16& sacc) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 kf = frag(ks, ka[s] + kb * 8192);
      sacc = s == 0 ? mfma32(kf, qf[s], f32x16{}) : mfma32(kf, qf[s], sacc);
    }
  };
  auto pv = [&](const u32x4* vs, const uint32_t (&pk)[2][8]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4 pb;
      pb.x = pk[c >> 1][4 * (c & 1) + 0];
      pb.y = pk[c >> 1][4 * (c & 1) + 1];
      pb.z = pk[c >> 1][4 * (c & 1) + 2];
      pb.w = pk[c >> 1][4 * (c & 1) + 3];
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pb);
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] = mfma32(frag(vs, va[c] + db * 4096), pf, oacc[db]);
    }
  };
  // Scores of the tile being softened: first key half in s0 (reused for the
  // next tile once its probabilities are out), second half alternating
  // between s1a and s1b so the next tile's can be formed meanwhile.
  f32x16 s0, s1a, s1b;
  uint32_t pA[2][8], pB[2][8];
  // Tile t: Kn is the K of tile t+1, Vp the Vᵀ of tile t-1 (P·V with pP);
  // s1c holds the second key half of tile t, s1n receives that of tile t+1;
  // pC receives tile t's probabilities. K of tile t+3 is fetched into kD
  // (the stage of tile t-1) and Vᵀ of tile t+2 into vD (that of tile t-2).
  //
  // The tile is issued as 32 slots, each one MFMA, the LDS read of the
  // fragment three slots ahead, and a planned share of the softmax:
  //   slots  0-15  P·V of tile t-1 (absent for the first tile),
  //   slots 16-23  scores of tile t+1, second key half (into s1n),
  //   slots 24-31  scores of tile t+1, first key half (into s0).
  // The softmax of tile t is 22 steps: the row max in 4 parts (A), the
  // rescale decision (B0: max over the wave halves and the ballot; B1: new
  // running max, factor, l), then 8 pairs of probabilities of each key
  // half (C on s0, D on s1c). C ends before slot 24 overwrites s0. A
  // scheduling barrier closes every slot, so the order is the one written.
  auto iter = [&](auto FIRST, const u32x4* Kn, const u32x4* Vp, u32x4* kD, u32x4* vD, int t,
                  const f32x16& s1c, f32x16& s1n, uint32_t (&pC)[2][8], const uint32_t (&pP)[2][8]) {
    constexpr bool first = decltype(FIRST)::value;
    constexpr int M0 = first ? 16 : 0;
#pragma unroll
    for (int s = 0; s < 8; ++s) asm volatile("" : "+v"(ka[s]));
#pragma unroll
    for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(va[c]));
    auto load = [&](int i) {
      if (i < 16) return frag(Vp, va[i >> 2] + (i & 3) * 4096);
      if (i < 24) return frag(Kn, ka[i - 16] + 8192);
      return frag(Kn, ka[i - 24]);
    };
    // slot of softmax step k (k < 6: A0-A3, B0, B1; then C0-C7, D0-D7)
    auto slot_of = [](int k) {
      if (first) return k < 6 ? 16 + k / 2 : k < 14 ? 19 + (k - 6) / 2 : 24 + (k - 14);
      return k < 6 ? k : 6 + ((k - 6) * 26) / 16;
    };
    float mt = -INFINITY, alpha = 1.f, nm = 0.f, ls = 0.f;
    bool up = false;
    auto pair = [&](const f32x16& sc, int j, uint32_t& w) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * j], sl2, nm));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[2 * j + 1], sl2, nm));
      w = pack2bf(p0, p1);
      ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), kOnes2, ls, false);
      asm volatile("" : "+v"(w), "+v"(ls));   // keep the pair in its slot
    };
    auto step = [&](int k) {
      if (k < 4) {
        const f32x16& sc = k < 2 ? s0 : s1c;
#pragma unroll
        for (int r = 0; r < 8; ++r) mt = fmaxf(mt, sc[8 * (k & 1) + r]);
        asm volatile("" : "+v"(mt));
      } else if (k == 4) {
        mt = half_max(mt) * sl2;
        up = __builtin_amdgcn_ballot_w64(mt > m_run + 8.f) != 0;
      } else if (k == 5) {
        const float m_new = fmaxf(m_run, mt);
        const float f = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        alpha = up ? f : 1.f;
        m_run = up ? m_new : m_run;
        ls = up ? l_run * f : l_run;
        nm = m_run == -INFINITY ? 0.f : -m_run;
        asm volatile("" : "+v"(alpha), "+v"(nm), "+v"(ls));
      } else if (k < 14) {
        pair(s0, k - 6, pC[0][k - 6]);
      } else {
        pair(s1c, k - 14, pC[1][k - 14]);
      }
    };
    dma_k(kD, t + 3);
    dma_v(vD, t + 2);
    bf16x8 fq[32];
#pragma unroll
    for (int i = M0; i < M0 + 3; ++i) fq[i] = load(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = M0; i < 32; ++i) {
      if (i + 3 < 32) fq[i + 3] = load(i + 3);
      if (i < 16) {
        const int c = i >> 2;
        u32x4 pb;
        pb.x = pP[c >> 1][4 * (c & 1) + 0];
        pb.y = pP[c >> 1][4 * (c & 1) + 1];
        pb.z = pP[c >> 1][4 * (c & 1) + 2];
        pb.w = pP[c >> 1][4 * (c & 1) + 3];
        oacc[i & 3] = mfma32(fq[i], __builtin_bit_cast(bf16x8, pb), oacc[i & 3]);
      } else if (i < 24) {
        s1n = i == 16 ? mfma32(fq[i], qf[0], f32x16{}) : mfma32(fq[i], qf[i - 16], s1n);
      } else {
        s0 = i == 24 ? mfma32(fq[i], qf[0], f32x16{}) : mfma32(fq[i], qf[i - 24], s0);
      }
#pragma unroll
      for (int k = 0; k < 22; ++k)
        if (slot_of(k) == i) step(k);
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run = ls;
    if (up) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[j][r] *= alpha;
    }
    __builtin_amdgcn_sched_barrier(0);
    // K of tile t+2 and Vᵀ of tile t landed (Vᵀ of t+1, K of t+3 and Vᵀ of
    // t+2 may still fly)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * HALF));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
  };

  if (ntiles > 0) {
    dma_k(k0s, 0);
    dma_k(k1s, 1);
    dma_k(k2s, 2);
    dma_v(v0s, 0);
    dma_v(v1s, 1);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * HALF));   // K of tiles 0 and 1 landed
    __builtin_amdgcn_s_barrier();
    smfma(k0s, 0, s0);
    smfma(k0s, 1, s1a);
    const std::false_type rest;
    iter(std::true_type(), k1s, v3s, k3s, v2s, 0, s1a, s1b, pA, pB);
    int t = 1;
    for (; t + 3 < ntiles; t += 4) {
      iter(rest, k2s, v0s, k0s, v3s, t, s1b, s1a, pB, pA);
      iter(rest, k3s, v1s, k1s, v0s, t + 1, s1a, s1b, pA, pB);
      iter(rest, k0s, v2s, k2s, v1s, t + 2, s1b, s1a, pB, pA);
      iter(rest, k1s, v3s, k3s, v2s, t + 3, s1a, s1b, pA, pB);
    }
    if (t < ntiles) iter(rest, k2s, v0s, k0s, v3s, t, s1b, s1a, pB, pA);
    if (t + 1 < ntiles) iter(rest, k3s, v1s, k1s, v0s, t + 1, s1a, s1b, pA, pB);
    if (t + 2 < ntiles) iter(rest, k0s, v2s, k2s, v1s, t + 2, s1b, s1a, pB, pA);
    // P·V of the last tile
    const int sl = last & 3;
    const u32x4* vl = sl == 0 ? v0s : sl == 1 ? v1s : sl == 2 ? v2s : v3s;
    if (last & 1) pv(vl, pB);
    else pv(vl, pA);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (piece >= 0) {
    const int npieces = (int)gridDim.x - a.split_base;
    float* po = a.part + (size_t)piece * BQ2 * D;
    float* pl = a.part + (size_t)npieces * BQ2 * D + (size_t)piece * BQ2;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int rl = wave * 32 + lq;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * half;
        f32x4 w;
        w[0] = oacc[db][4 * g + 0] * inv;
        w[1] = oacc[db][4 * g + 1] * inv;
        w[2] = oacc[db][4 * g + 2] * inv;
        w[3] = oacc[db][4 * g + 3] * inv;
        *reinterpret_cast<f32x4*>(po + (size_t)rl * D + d0) = w;
      }
    if (half == 0) pl[rl] = l_tot > 0.f ? m_run + __log2f(l_tot) : -INFINITY;
    return;
  }
  const float inv = 1.f / l_tot;
  if (qvalid) {
    uint16_t* op = a.out + (size_t)qi * a.out_stride + h * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * half;
        u32x2 w;
        w.x = pack2bf(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
        w.y = pack2bf(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(op + d0) = w;
      }
  }
}

// Merges the pieces of each split unit: with L = max_j lse_j, the output row
// is sum_j 2^(lse_j - L) O_j / sum_j 2^(lse_j - L) (the pieces' O_j are
// already normalized by their own sums). One thread per 4 dims of a row.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a, int bq) {
  const int rows_per_blk = 8;
  const int blks_per_unit = bq / rows_per_blk;
  const int ui = blockIdx.x / blks_per_unit;
  const int rl = (blockIdx.x - ui * blks_per_unit) * rows_per_blk + (threadIdx.x >> 5);
  const int d0 = (threadIdx.x & 31) * 4;
  const int nqb = (a.N + bq - 1) / bq;
  const int unit = a.split_base + ui;
  const int h = unit / nqb;
  const int qblk = a.rev_q ? nqb - 1 - (unit - h * nqb) : unit - h * nqb;
  const int q = qblk * bq + rl;
  if (q >= a.N) return;
  const int npieces = (int)gridDim.x / blks_per_unit * a.split_s;
  const float* lse = a.part + (size_t)npieces * bq * D;
  float lmax = -INFINITY;
  for (int j = 0; j < a.split_s; ++j) lmax = fmaxf(lmax, lse[(size_t)(ui * a.split_s + j) * bq + rl]);
  float acc[4] = {0.f, 0.f, 0.f, 0.f}, wsum = 0.f;
  if (lmax > -INFINITY) {
    for (int j = 0; j < a.split_s; ++j) {
      const int pc = ui * a.split_s + j;
      const float w = exp2f(lse[(size_t)pc * bq + rl] - lmax);
      const f32x4 o = *reinterpret_cast<const f32x4*>(a.part + ((size_t)pc * bq + rl) * D + d0);
      wsum += w;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += w * o[i];
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  u32x2 w;
  w.x = pack2bf(acc[0] * inv, acc[1] * inv);
  w.y = pack2bf(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<u32x2*>(a.out + (size_t)q * a.out_stride + h * D + d0) = w;
}

// The grid has units = query blocks x heads workgroups, `per_cu` of them
// resident per CU. With `split`, the units of a last, partly filled round
// are split over key ranges when that shortens the round (scratch allowing).
template <int NWV, int QW, int NST>
hipError_t run_attn2(const AttnArgs& a0, hipStream_t s, bool split, const LaunchEvents& ev = {}) {
  constexpr int BQ2 = NWV * QW;
  constexpr int per_cu = (NWV == 4 && NST == 2) ? 2 : 1;
  AttnArgs a = a0;
  const int units = ((a.N + BQ2 - 1) / BQ2) * a.nh;
  a.split_base = units; a.split_s = 1;
  if (split && a.part) {
    const int slots = device_cus() * per_cu;
    const int rem = slots > 0 ? units % slots : 0;
    if (rem > 0) {
      // pieces of the remaining units fill one round; each keeps >= 8 key tiles
      int sp = min(slots / rem, 8);
      sp = min(sp, ((a.S + BKV - 1) / BKV) / 8);
      const size_t need = (size_t)rem * sp * BQ2 * (D + 1) * sizeof(float);
      if (sp >= 2 && need <= a.part_bytes) { a.split_base = units - rem; a.split_s = sp; }
    }
  }
  const int nblk = a.split_s > 1 ? a.split_base + (units - a.split_base) * a.split_s : units;
  const bool comb = a.split_s > 1;
  launch_k((attn2_kernel<NWV, QW, NST>), dim3(nblk), dim3(NWV * 64), s, ev.start, comb ? nullptr : ev.stop, a);
  if (comb) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_k(attn_combine_kernel, dim3((units - a.split_base) * (BQ2 / 8)), dim3(256), s, nullptr, ev.stop,
             a, BQ2);
  }
  return hipGetLastError();
}

// The cached-step kernel: same grid and key split as attn2_kernel<8, 32, 3>.
hipError_t run_attn3(const AttnArgs& a0, hipStream_t s, bool split, const LaunchEvents& ev = {}) {
  constexpr int BQ2 = 256;
  AttnArgs a = a0;
  const int units = ((a.N + BQ2 - 1) / BQ2) * a.nh;
  a.split_base = units; a.split_s = 1;
  if (split && a.part) {
    const int slots = device_cus();
    const int rem = slots > 0 ? units % slots : 0;
    if (rem > 0) {
      int sp = min(slots / rem, 8);
      sp = min(sp, (a.S / BKV) / 8);
      const size_t need = (size_t)rem * sp * BQ2 * (D + 1) * sizeof(float);
      if (sp >= 2 && need <= a.part_bytes) { a.split_base = units - rem; a.split_s = sp; }
    }
  }
  const int nblk = a.split_s > 1 ? a.split_base + (units - a.split_base) * a.split_s : units;
  const bool comb = a.split_s > 1;
  launch_k(attn3_kernel, dim3(nblk), dim3(512), s, ev.start, comb ? nullptr : ev.stop, a);
  if (comb) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_k(attn_combine_kernel, dim3((units - a.split_base) * (BQ2 / 8)), dim3(256), s, nullptr, ev.stop,
             a, BQ2);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_variant(const AttnArgs& a, int variant, hipStream_t s) {
  // the pipelined kernel serves cached rows (every key visible) over whole 64-key tiles only
  if ((variant == 5 || variant == 6) && (a.q_off != a.P || a.S % BKV)) return hipErrorInvalidValue;
  switch (variant) {
    case 1: return run_attn2<8, 32, 3>(a, s, false);
    case 2: return run_attn2<4, 32, 2>(a, s, false);   // two workgroups per CU
    case 3: return run_attn2<8, 32, 3>(a, s, true);    // 1 with the last round split
    case 4: return run_attn2<4, 32, 2>(a, s, true);    // 2 with the last round split
    case 5: return run_attn3(a, s, false);              // pipelined, cached rows only
    case 6: return run_attn3(a, s, true);               // 5 with the last round split
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s, const LaunchEvents& ev) {
  // 256 queries per workgroup (8 waves, one workgroup per CU) unless that
  // leaves CUs idle, then 128-query workgroups two per CU. Target rows of a
  // cached step (q_off > 0) all stream the same keys, so a last, partly
  // filled round of workgroups is split over key ranges (measured on 32
  // heads: 9216 queries x 22016 keys 3.11 -> 2.86 ms, x 50688 keys 7.42 ->
  // 6.47 ms). The rows of an extract step differ in length; there the split
  // measured slower and is not used. Instead each head's query blocks are
  // dealt last block first: target rows (all keys) start first and the short
  // text / reference blocks fill the tail (22016 rows: 4.96 -> 4.57 ms).
  // Target rows of a cached step with S a multiple of 64 (no masked key
  // tile) go to the software-pipelined kernel, the same arithmetic per query
  // (measured on 32 heads: 4096 queries x 4352 keys 0.335 -> 0.273 ms,
  // 9216 x 22016 3.00 -> 2.80 ms).
  const long long blocks256 = (long long)((a.N + 255) / 256) * a.nh;
  const bool split = a.q_off > 0;
  AttnArgs b = a;
  b.rev_q = a.q_off == 0;
  if (blocks256 < 256) return run_attn2<4, 32, 2>(b, s, split, ev);
  if (a.q_off > 0 && a.q_off == a.P && a.S % BKV == 0) return run_attn3(b, s, split, ev);
  return run_attn2<8, 32, 3>(b, s, split, ev);
}


}  // namespace dit
