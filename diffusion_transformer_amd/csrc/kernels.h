// Internal launcher interface between the C ABI (dit_api.cpp) and the
// gfx950 kernels. Every launcher enqueues on `stream` and returns the
// hipGetLastError() of its launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

// Activation element type: bf16 bits in the production library, fp32 in
// the debug build compiled with -DDIT_F32 (weights stay bf16 in both).
#ifdef DIT_F32
typedef float act_t;
#else
typedef uint16_t act_t;
#endif

// Per-head QK-RMSNorm (1 + w) + 3D RoPE on q (in place) and k, and the K /
// Vᵀ cache writes for global tokens [g_begin, g_end); tokens >= S are
// zero-filled in the cache. qkv local row i holds global token q_row0 + i.
struct QkArgs {
  act_t* qkv; int ld;               // [rows, 3H]
  int q_row0;
  int g_begin, g_end, S, cap, nh, H;
  const uint16_t* wq; const uint16_t* wk;   // [128] bf16
  const float* cosv; const float* sinv;     // [S, 64]
  act_t* kc; act_t* vtc;                    // layer bases
  float eps;
  int P, T_el;   // rows >= P: RoPE of logical row P + (g - P) % T_el (T_el = 0: g)
};
hipError_t launch_qknorm_rope(const QkArgs& a, hipStream_t s);

enum GemmEpi {
  EPI_BF16 = 0,    // C (bf16) = A·Bᵀ
  EPI_F32 = 1,     // C (f32)  = A·Bᵀ
  EPI_RESID = 2,   // Hres (f32) += g[row] ⊙ A·Bᵀ, g = tanh(gate) chosen by the n_pre split
  EPI_SWIGLU = 3,  // C (bf16)[:, f] = SiLU(A·Gᵀ)[f] · (A·Uᵀ)[f]  (B = gate, B2 = up)
  EPI_PART = 4,    // internal: fp32 partial sums of one K split -> part[split][M][N]
  EPI_QKV = 5      // C = A·Bᵀ (bf16) with the QK-RMSNorm + RoPE + cache write of `qk` fused:
                   // q columns to C, k rows and transposed v to the cache
};

struct GemmArgs {
  const act_t* A; int lda;          // [M, K] activations
  const uint16_t* B; int ldb;       // [N, K] bf16 (gate for SwiGLU)
  const uint16_t* B2;               // up [N/2, K] for SwiGLU, else unused
  int M, N, K;                      // N = packed width (2F for SwiGLU)
  void* C; int ldc;                 // output (act_t, or f32 for EPI_F32)
  float* Hres; int ldh;             // residual stream for EPI_RESID
  const float* gate_t;              // [N] tanh(gate) of target / current-t tokens
  const float* gate_0;              // [N] tanh(gate) of prefix tokens (t = 0)
  int n_pre;                        // rows < n_pre use gate_0
  float* part; size_t part_bytes;   // scratch for split-K partial sums (may be null)
  int splits;                       // internal: K splits of an EPI_PART launch
  QkArgs qk;                        // EPI_QKV: norm weights, RoPE tables, cache, row mapping
};
// Bytes of split-K scratch the GEMM launcher can use: at most one round of
// 256 tiles of 256 x 256 fp32 partial sums. The step lends the same buffer
// to attention's key split (256 x 129 floats per piece).
constexpr size_t kGemmPartBytes = (size_t)256 * 256 * 256 * 4;

// Timing events of one launch sequence: `start` is taken when its first
// kernel starts and `stop` when its last one ends, by those kernels' own
// dispatch packets (a multi-kernel GEMM split records them into the stream
// around its kernels instead). Null events are not recorded.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
hipError_t launch_gemm(const GemmArgs& g, int epi, hipStream_t s, const LaunchEvents& ev = {});
// The last 256-row block (or the whole GEMM, if smaller) as `splits` K
// splits into g.part, reduced with the epilogue; the rows before it in one
// ordinary launch. The caller checks K / 64 % splits == 0 and the scratch.
hipError_t launch_gemm_forced_split(const GemmArgs& g, int epi, int splits, hipStream_t s);
bool gemm_shape_ok(int M, int N, int K, int epi);

struct AttnArgs {
  const act_t* q; int q_stride;     // local query rows 0..N-1, head h at column h*128
  int q_off;                        // global index of local row 0
  int N;
  const act_t* k;                   // K of this layer: [nh][cap][128]
  const act_t* vt;                  // Vᵀ of this layer: [nh][128][cap]
  int cap, S, nh;
  const int32_t* limit;             // [S]
  act_t* out; int out_stride;       // [N, nh*128]
  // Target latents sharing the prefix: global rows and cache keys >= P of
  // element e = (row - P) / T_el are that element's, its logical index is
  // row - e*T_el (layout tables and the mask describe one element). T_el = 0
  // or S - P: a single latent.
  int P, T_el;
  // Key-split scratch (fp32; null: no split) and, filled in by the launcher,
  // the first split unit and the pieces per split unit.
  float* part; size_t part_bytes;
  int split_base, split_s;
  int rev_q;                        // 1: a head's query blocks run last block first
};
hipError_t launch_attention(const AttnArgs& a, hipStream_t s, const LaunchEvents& ev = {});
hipError_t launch_attention_variant(const AttnArgs& a, int variant, hipStream_t s);
hipError_t launch_debug_mask(const int32_t* limit, int S, uint8_t* mask, hipStream_t s);

// LN(h)·(1 + scale[row]) -> act_t. rows < n_pre use scale_0, others scale_t.
hipError_t launch_ln_mod(const float* h, int ldh, int rows, int H, const float* scale_t,
                         const float* scale_0, int n_pre, float eps, act_t* out, int ldo,
                         hipStream_t s, const LaunchEvents& ev = {});


// Y[v][o] = W[o]·X[v] for v < nv (W bf16 [O, I]); optionally also writes
// silu(Y) to Ys.
hipError_t launch_gemv(const uint16_t* W, int O, int I, const float* X, int ldx, int nv,
                       float* Y, int ldy, float* Ys, hipStream_t s, const LaunchEvents& ev = {});
// [cos(t_v f_i), sin(t_v f_i)], f_i = base^(-2i/D), computed in double.
hipError_t launch_temb(float t0, float t1, int D, float base, float* out, hipStream_t s);
// z[r][c] = (z - mean[c]) / std[c] (inverse: z * std[c] + mean[c]), in place.
hipError_t launch_standardize(float* z, const float* mean, const float* std, long long rows,
                              int channels, int inverse, hipStream_t s);
// tanh of the gate sections of nv modulation rows [scale1 | gate1 | scale2 | gate2].
hipError_t launch_gate_tanh(float* mod, int H, int nv, hipStream_t s);
// hidden[i][n] = Σ_c W[n][c] x[i][c]; W bf16 [H, 64], x f32 [n, 64], fp32 out.
hipError_t launch_img_in(const uint16_t* W, const float* x, int n, int H, float* out, int ldo,
                         hipStream_t s, const LaunchEvents& ev = {});
// v[i] = W_out · (LN(h[i]) · (1 + scale)) for rows < rows: LN non-affine
// over H (<= 4096, % 256 == 0), the scaled row rounded to bf16, W_out bf16
// [64, H], v fp32 [rows, 64].
hipError_t launch_final_out(const float* h, int ldh, int rows, int H, const float* scale, float eps,
                            const uint16_t* W, float* v, hipStream_t s, const LaunchEvents& ev = {});
hipError_t launch_euler(float* x, const float* v, float dsig, long long n, hipStream_t s);
// dst = src, bytes % 16 == 0, 16-byte accesses.
hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t s);
// Register-only bf16 MFMA loop (measured ceiling): blocks x 4 waves x iters
// x 64 MFMAs of 32x32x16; ops 1 MiB of bf16 operands, out [blocks * 256].
hipError_t launch_mfma_loop(const uint16_t* ops, float* out, int blocks, int iters, hipStream_t s);

}  // namespace dit
