/*
 * dit.h — C ABI of the MI355X (gfx950) cached flow-matching DiT step.
 *
 * One denoising step of a single-stream Qwen-Image-2.1-style diffusion
 * transformer with a prefix KV cache, as described on the course pages
 * "Lab tổng hợp Qwen-Image-2.1 — chạy toàn trình 1A → 6B bằng NumPy"
 * (end-to-end lab, §3 Solution and §6 Glossary: extract / cached modes),
 * "3B · Causal condition (t=0 vs t) & shared modulation" (§1 Definition),
 * "6B · Scale-Only Final AdaLN, v_θ & 8-Step Euler" (§1 Definition) and the
 * lab index page's 1:1 mapping table (rows 3A, 3C, 4A, 5A, 6A, 6B).
 *
 * Conventions shared by every entry point:
 *  - Ownership: the caller allocates ALL device memory (weights, prefix
 *    hidden states, latents, velocity, KV cache, workspace, layout tables,
 *    and the scratch of the test hooks). Except for the small host-side
 *    model handle (and, while per-kernel timing is on, its HIP events), the
 *    library allocates nothing. Weight pointers are borrowed from
 *    dit_load_weights until dit_free; the caller keeps them alive and
 *    unchanged.
 *  - Threads: the weights are never written. A model handle's mutable
 *    host state is its registry of extracted caches (behind DIT_ERR_STATE)
 *    and its timing events; every call that reads or writes them takes a
 *    lock held by the handle, so calls on one handle from several threads
 *    are serialized on the host (the GPU work they enqueue is ordered only
 *    by the streams given). Steps that may run on the GPU at the same time
 *    need distinct workspaces and distinct caches. dit_free must not race
 *    with other calls on the handle.
 *  - Device pointers must be 16-byte aligned. bf16 tensors are raw
 *    bfloat16 bit patterns (uint16), row-major. Linear weights use the
 *    [out_features, in_features] layout: y = W x.
 *  - Streams: `stream` is a hipStream_t (NULL = the default stream). All
 *    device work is enqueued asynchronously on it; no call synchronizes.
 *  - Errors: every dit_status call validates its arguments on the host
 *    BEFORE enqueuing anything; on error nothing was enqueued, the status
 *    is returned and dit_last_error() (thread-local) holds a message.
 *    A failed kernel launch returns DIT_ERR_HIP. No C++ exception crosses
 *    the ABI.
 *  - Supported shapes on the GPU: head_dim 128, hidden = n_heads*128, a
 *    multiple of 256 and at most 4096, ffn a multiple of 128, latent 64,
 *    time_dim a multiple of 8 and at most 1024, rope_dims even and summing
 *    to 128.
 */
#ifndef DIT_H_
#define DIT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int dit_status;
enum {
  DIT_OK = 0,
  DIT_ERR_ARG = 1,         /* null pointer or out-of-range scalar          */
  DIT_ERR_SHAPE = 2,       /* dimensions the GPU path does not support     */
  DIT_ERR_LAYOUT = 3,      /* invalid token layout (see dit_build_layout)  */
  DIT_ERR_STATE = 4,       /* cached step on a cache never extracted       */
  DIT_ERR_WORKSPACE = 5,   /* workspace or cache buffer too small          */
  DIT_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed   */
  DIT_ERR_UNSUPPORTED = 7  /* valid request the library does not implement */
};

/* Step flags. */
enum {
  /* Prefix tokens read the current-t modulation row instead of the t = 0
   * row ("3B" page §4/Limits: with causal_condition off the prefix changes
   * every step and the cache is invalid). For the drift experiment only;
   * a cache extracted with this flag is refused by dit_step_cached. */
  DIT_FLAG_NO_CAUSAL_CONDITION = 1
};

/* Model dimensions. rope_base and eps: 10000 and 1e-6 as in the lab
 * script's configuration block. */
typedef struct dit_config {
  int hidden;       /* H  */
  int n_heads;      /* nh */
  int head_dim;     /* d (128) */
  int ffn;          /* F, SwiGLU inner width */
  int n_layers;     /* L  */
  int latent;       /* C (64) */
  int time_dim;     /* D_t, width of the sinusoidal timestep embedding */
  int rope_dims[3]; /* (frame, height, width) widths, even, sum = d */
  float rope_base;
  float eps;
} dit_config;

/* Device pointers to bf16 weights, [out, in] row-major, no biases.
 * Global: t1 [H, D_t], t2 [H, H] (timestep MLP, page 3B §1: sin-cos -> MLP);
 *         mod [4H, H] (shared SiLU -> Linear(H, 4H) giving
 *         [scale1, gate1, scale2, gate2], page 3B §1);
 *         so [H, H] (final AdaLN scale from the current-t embedding, page 6B §3);
 *         img_in [H, C]; proj_out [C, H] (page 6B §1: Linear(4096, 64)).
 * Per layer (host arrays of n_layers device pointers):
 *         qkv [3H, H] (q rows, then k, then v), q_norm [d], k_norm [d]
 *         (zero-centred QK-RMSNorm weights, used as 1 + w), o [H, H],
 *         gate [F, H], up [F, H], down [H, F] (SwiGLU, mapping row 5A). */
typedef struct dit_weights {
  const void* t1;
  const void* t2;
  const void* mod;
  const void* so;
  const void* img_in;
  const void* proj_out;
  const void* const* qkv;
  const void* const* q_norm;
  const void* const* k_norm;
  const void* const* o;
  const void* const* gate;
  const void* const* up;
  const void* const* down;
} dit_weights;

typedef struct dit_model dit_model; /* opaque host-side handle */

/* Device-side token layout of one joint sequence (built by dit_build_layout
 * on the host, copied to device memory by the caller).
 *   P prefix tokens (text and references) followed by T target tokens.
 *   d_row_limit [S] int32: largest key index visible to each query row.
 *   d_rope_cos, d_rope_sin [S, head_dim/2] float32: per-token, per-pair
 *   RoPE rotation.
 *   B: number of target latents denoised together against ONE shared prefix
 *   (independent requests or seeds; 0 or 1 = a single latent). Element b's
 *   target tokens are rows P + b*T .. P + (b+1)*T - 1 of every per-token
 *   tensor and of the KV cache; each sees the prefix and its own target
 *   block, never another element's (the layout tables describe one element:
 *   S = P + T entries). x and v_out are [B*T, C], the cache holds
 *   S_all = P + B*T keys, extract workspaces n_tokens = S_all, cached
 *   n_tokens = B*T. B > 1 needs P and T to be multiples of 256
 *   (DIT_ERR_SHAPE otherwise) and is not part of the fp32 debug build.
 *   S_all above 2^22 tokens is DIT_ERR_LAYOUT. */
typedef struct dit_seq {
  int P;
  int T;
  const int32_t* d_row_limit;
  const float* d_rope_cos;
  const float* d_rope_sin;
  int B;
} dit_seq;

/* Token layout from a segment list (host only, no device work).
 * Pages: "2A · 4× image-slot expansion & joint packing" §1 (order text ->
 * references -> target; image_ids -1 text, 0..K-1 references, K target;
 * row-major image cells), lab index mapping row 3A (text advances (c,c,c)
 * with c its index among text tokens; images at frame 0 on the zero-centred
 * grid r - n/2) and row 3C (key j visible to query i iff j <= i or both in
 * the same image block).
 *   seg_kind[n_seg]: 0 text (seg_rows tokens; seg_cols ignored),
 *                    1 reference image (seg_rows x seg_cols grid),
 *                    2 target image (exactly one, last).
 *   Outputs (host buffers, any may be NULL): image_ids [S], coords [S*3]
 *   (frame, height, width), row_limit [S], rope_cos / rope_sin
 *   [S * head_dim/2] (angles evaluated in double, stored as float),
 *   P_out, T_out.
 * Returns DIT_ERR_LAYOUT for an empty or misplaced target, a non-positive
 * segment size or S > 2^22 (4194304 tokens, the library's limit). With
 * contiguous segments the block-causal rule is exactly j <= row_limit[i];
 * the library relies on that. */
dit_status dit_build_layout(const dit_config* cfg, const int* seg_kind, const int* seg_rows,
                            const int* seg_cols, int n_seg, int32_t* image_ids,
                            int32_t* coords, int32_t* row_limit, float* rope_cos,
                            float* rope_sin, int* P_out, int* T_out);

/* Validate dimensions and borrow weight pointers (host only; no device
 * work). On success *out receives a new handle. */
dit_status dit_load_weights(const dit_config* cfg, const dit_weights* w, dit_model** out);
void dit_free(dit_model* m);

/* Bytes of workspace a step over up to n_tokens tokens needs (extract uses
 * n_tokens = S, cached n_tokens = T). */
size_t dit_workspace_bytes(const dit_model* m, int n_tokens);

/* Key capacity of a cache for S tokens (S rounded up to 128) and the cache
 * size in bytes. Cache layout, per layer l and head h (bf16):
 *   K  at  ((l*nh + h) * cap + j) * d + e          key j, dim e
 *   Vᵀ at  L*nh*cap*d + ((l*nh + h) * d + e) * cap + j
 * i.e. K is key-major and V is stored transposed (dim-major). Keys
 * S..cap-1 are zero-filled by dit_step_extract. */
int dit_kv_capacity(int S);
size_t dit_kv_cache_bytes(const dit_model* m, int S);

/* Step 1, extract (end-to-end lab §6 "kv_cache_mode"; page 3B §1):
 * runs all S = P + T tokens under the block-causal mask; prefix rows use
 * the t = 0 modulation row, target rows the row of t = 1000·sigma; writes
 * every layer's post-norm, post-RoPE K and raw V of all S tokens into
 * kv_cache (rows 0..P-1 persist for the cached steps) and v_out.
 *   prefix_hidden [P, H] f32 (device), x [T, C] f32 (device),
 *   kv_cache (device, >= dit_kv_cache_bytes(m, S)),
 *   v_out [T, C] f32 (device), workspace >= dit_workspace_bytes(m, S).
 * Full recompute at every step = calling this every step. */
dit_status dit_step_extract(dit_model* m, const dit_seq* seq, const float* prefix_hidden,
                            const float* x, float sigma, void* kv_cache, size_t kv_bytes,
                            float* v_out, void* workspace, size_t ws_bytes, int flags,
                            void* stream);

/* Steps 2..N, cached (end-to-end lab §6; mapping row 6A): only the T target
 * tokens are projected; every layer writes their K/V into cache rows
 * P..S-1 and attends over all S keys (cached prefix + fresh target).
 * Rows 0..P-1 are read, never written. Returns DIT_ERR_STATE unless
 * dit_step_extract (without DIT_FLAG_NO_CAUSAL_CONDITION) ran before on
 * this (model, kv_cache, P, T). workspace >= dit_workspace_bytes(m, T). */
dit_status dit_step_cached(dit_model* m, const dit_seq* seq, const float* x, float sigma,
                           void* kv_cache, size_t kv_bytes, float* v_out, void* workspace,
                           size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code recorded into a HIP
 * graph, tight serving loops, hosts that forbid allocation): dit_step_cached
 * with its workspace taken from a fixed device array the library holds, one
 * per GPU (DIT_NOALLOC_SCRATCH_BYTES, reserved on every GPU the library runs
 * on until the process ends). No allocation and no per-kernel timing happen
 * in this call. The array is shared by every call on that GPU and keeps the
 * last call's contents (nothing in it needs to start at zero); calls that
 * overlap on one GPU race. Workspace needs above the array's size (about
 * 2200 target rows at H = 4096, F = 16384) return DIT_ERR_WORKSPACE before
 * any device work; other arguments and errors as dit_step_cached. */
#define DIT_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
dit_status dit_step_cached_noalloc(dit_model* m, const dit_seq* seq, const float* x, float sigma,
                                   void* kv_cache, size_t kv_bytes, float* v_out, void* stream);

/* Flow-matching Euler update (page 6B §1/§6):
 * x[i] += (sigma_k1 - sigma_k) * v[i] for i < n, in float32, in place. */
dit_status euler_update(float* x, const float* v, float sigma_k, float sigma_k1, long long n,
                        void* stream);

/* Per-channel latent (un)standardization, in place, float32.
 * Page "1A · RGBA 64-Ch VAE & Unpatched Latents": each latent channel of a
 * reference image is standardized with its own statistics before img_in,
 * z_hat = (z - mean[c]) / std[c]; page 6B §1: after the last Euler step the
 * latent returns to the VAE's space, z = z_hat * std[c] + mean[c].
 *   z [rows, channels] f32 (device, in place), mean, std [channels] f32
 *   (device); inverse 0 = standardize, 1 = unstandardize; channels in
 *   1..1024. std entries are used as given (a zero std divides by zero). */
dit_status dit_latent_standardize(float* z, const float* mean, const float* std, long long rows,
                                  int channels, int inverse, void* stream);

/* img_in (end-to-end lab, block 1A: one latent cell -> one H-wide token):
 * hidden[i] = W_in · latents[i], latents [n, C] f32 -> hidden [n, H] f32.
 * Used to embed reference latents into prefix hidden states. */
dit_status dit_img_in(const dit_model* m, const float* latents, int n, float* hidden,
                      void* stream);

/* Test hook: writes mask[i*S + j] = 1 if the attention kernel treats key j
 * as visible to query i, else 0, for i, j < S (device u8 [S*S]). It uses
 * the attention kernel's own visibility predicate and tile classifier. */
dit_status dit_debug_mask(const dit_seq* seq, uint8_t* mask, void* stream);

/* Test hook: one attention layer call on explicit buffers.
 *   q [N, q_stride] bf16 with head h at columns h*128.., kv_cache layer 0
 *   of a cache with capacity dit_kv_capacity(S) for n_heads heads,
 *   queries are global rows q_off..q_off+N-1, out [N, n_heads*128] bf16.
 *   variant 0 = the launch the step makes (kernel shape, key split of a
 *   cached step's last round, longest-first order of an extract step);
 *   1 = 256-query workgroups (8 waves), 2 = 128-query workgroups (4 waves,
 *   two per CU), both in index order and unsplit; 3, 4 = 1, 2 with the last
 *   round of workgroups split over key ranges; 5 = the pipelined kernel of
 *   cached steps (8 waves of 32 queries; the softmax of key tile t runs
 *   under the score MFMAs of tile t+1 and the P·V of tile t-1; same
 *   arithmetic per query as 1; target rows only: q_off = P and S a multiple
 *   of 64, DIT_ERR_ARG otherwise), 6 = 5 with the last round split.
 *   scratch (device, caller-owned, may be NULL = no split) holds the split
 *   pieces: 256 * 129 * 4 bytes per piece at most; a launch whose pieces do
 *   not fit runs unsplit. Calls that overlap on one scratch race. */
dit_status dit_debug_attention(const dit_seq* seq, int n_heads, const void* q, int q_stride,
                               int q_off, int N, const void* kv_cache, void* out,
                               int variant, void* scratch, size_t scratch_bytes, void* stream);

/* Test hook: one GEMM of the step, with its fused epilogue, on explicit
 * device buffers: y = A · Bᵀ with A [M, K] and B [N, K] bf16 (K-contiguous,
 * the weights' nn.Linear layout), fp32 accumulation. Epilogues (the step's
 * use in brackets; mapping rows 4A and 5A of the lab index page):
 *   DIT_GEMM_BF16   C bf16 [M, N] = y.
 *   DIT_GEMM_RESID  h fp32 [M, N] += g[n] * y, g = gate_0 for rows < n_pre
 *                   and gate_t for the others, fp32 [N] each [O and down
 *                   projections: h += tanh(gate) * out].
 *   DIT_GEMM_SWIGLU C bf16 [M, N] = SiLU(A · Bᵀ) * (A · B2ᵀ) with B the gate
 *                   and B2 the up weights, both [N, K] [the SwiGLU MLP].
 *   DIT_GEMM_QKV    N = 3 * n_heads * 128 columns q | k | v, each head's
 *                   128 columns rounded to bf16, then q and k per head
 *                   RMSNorm (1 + w) with q_norm / k_norm (bf16 [128]) and
 *                   eps, and RoPE with the tables of token q_row0 + m
 *                   (rope_cos / rope_sin [S, 64]); q is written to C's q
 *                   columns (C bf16 [M, N]; its k and v columns are left
 *                   unspecified), k to K cache row q_row0 + m and v to
 *                   Vᵀ cache column q_row0 + m of layer 0 of kv_cache
 *                   (capacity dit_kv_capacity(S), dit_kv_capacity layout).
 * M > 0, N % 256 == 0, K % 64 == 0, else DIT_ERR_SHAPE.
 * splits: 0 = the step's rule (the last row blocks are split over K when
 * the tile count leaves a partly idle round and the partial sums fit the
 * scratch; none without scratch); 2 or 4 = always compute the last 256-row
 * block as that many K splits (needs K / 64 divisible by splits and
 * scratch_bytes >= splits * 256 * N * 4, doubled for DIT_GEMM_SWIGLU;
 * DIT_ERR_ARG otherwise). The scratch is caller-owned device memory. */
enum {
  DIT_GEMM_BF16 = 0,
  DIT_GEMM_RESID = 2,
  DIT_GEMM_SWIGLU = 3,
  DIT_GEMM_QKV = 5
};
typedef struct dit_gemm_desc {
  int epilogue;
  int M, N, K;
  const void* A;
  const void* B;
  const void* B2;           /* SWIGLU: up weights */
  void* C;
  float* h;                 /* RESID */
  const float* gate_t;      /* RESID */
  const float* gate_0;      /* RESID */
  int n_pre;                /* RESID */
  const void* q_norm;       /* QKV */
  const void* k_norm;       /* QKV */
  const float* rope_cos;    /* QKV */
  const float* rope_sin;    /* QKV */
  void* kv_cache;           /* QKV */
  int n_heads, S, q_row0;   /* QKV */
  float eps;                /* QKV */
  int splits;
  void* scratch;
  size_t scratch_bytes;
} dit_gemm_desc;
dit_status dit_debug_gemm(const dit_gemm_desc* d, void* stream);

/* Test hook: the step's scale-only final AdaLN + proj_out kernel on
 * explicit buffers (page 6B §1 and §3: v = W_out · (LN(h) · (1 + scale_out))
 * per target token; LN non-affine with population variance, eps inside the
 * root; the scaled row rounded to bf16 before the product, fp32 accumulation).
 *   h [rows, H] f32 (row stride ldh), scale_out [H] f32, w_out [64, H] bf16,
 *   v_out [rows, 64] f32 (all device). H must be the model widths the
 *   library supports (a multiple of 256, at most 4096). */
dit_status dit_debug_final_out(const float* h, int ldh, int rows, int H, const float* scale_out,
                               float eps, const void* w_out, float* v_out, void* stream);

/* Test hook: the step's GEMV kernel on explicit buffers, Y[v][o] = W[o] · X[v]
 * for v < nv: the timestep MLP's two linears, the shared modulation linear
 * and the final scale linear (page 3B §1; page 6B §3), fp32 accumulation of
 * bf16 weights times fp32 inputs. If Ys is not NULL it also receives
 * SiLU(Y) (the input of the next linear).
 *   W [O, I] bf16 row-major, X [nv, I] f32 (row stride ldx), Y and Ys
 *   [nv, O] f32 (row stride O), all device, 16-byte aligned. nv is 1 or 2,
 *   I a multiple of 8 and at most 4096, O > 0 and O·I·2 below 2^31 bytes
 *   (DIT_ERR_SHAPE otherwise). */
dit_status dit_debug_gemv(const void* W, int O, int I, const float* X, int ldx, int nv, float* Y,
                          float* Ys, void* stream);

/* Measurement hook: a device-to-device copy of `bytes` (a multiple of 16)
 * with 16-byte accesses, the HBM ceiling the bandwidth-bound kernels are
 * compared with. */
dit_status dit_debug_stream_copy(const void* src, void* dst, size_t bytes, void* stream);

/* Measurement hook: the bf16 MFMA ceiling the kernels run against. A
 * register-only loop of v_mfma_f32_32x32x16_bf16 (blocks workgroups of 4
 * waves, each wave iters x 64 MFMAs in 8 independent chains) on operands
 * read once from ops (device, 1 MiB of bf16: pass real-looking data, since
 * the operands' bit patterns set the power draw and with it the clock);
 * out (device, blocks * 256 floats) receives a checksum per thread.
 * Work per launch: blocks * 4 * iters * 64 * 32768 flop. blocks and iters
 * must be positive; not part of the fp32 debug build. */
dit_status dit_debug_mfma_loop(const void* ops, float* out, int blocks, int iters, void* stream);

/* Per-kernel timing over HIP events recorded on the step's stream around
 * every launch of one kernel class (0 = off). Enabling it adds an event
 * pair per launch. dit_profile_read returns the summed milliseconds and
 * the number of launches since the last read (it synchronizes the events)
 * and resets the totals. */
enum {
  DIT_PROF_OFF = 0,
  DIT_PROF_GEMM_QKV = 1,     /* includes the fused QK norm, RoPE and cache write */
  DIT_PROF_GEMM_O = 2,
  DIT_PROF_GEMM_GATEUP = 3,
  DIT_PROF_GEMM_DOWN = 4,
  DIT_PROF_ATTENTION = 5,
  DIT_PROF_LN = 6,
  DIT_PROF_QKNORM_ROPE = 7,  /* the standalone kernel: cache padding of an extract step */
  DIT_PROF_FINAL = 8,        /* scale-only final AdaLN + proj_out (one kernel) */
  DIT_PROF_IMG_IN = 9,
  DIT_PROF_GEMV = 10,        /* timestep MLP and final-scale GEMVs */
  DIT_PROF_GEMV_MOD = 11     /* the shared modulation GEMV, [4H, H] */
};
dit_status dit_profile_enable(dit_model* m, int kernel_class);
dit_status dit_profile_read(dit_model* m, double* total_ms, long long* launches);

const char* dit_last_error(void);
const char* dit_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DIT_H_ */
