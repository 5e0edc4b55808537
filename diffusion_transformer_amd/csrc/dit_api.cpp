// Host side of the C ABI declared in include/dit.h: validation, token
// layout, workspace plan, per-step kernel orchestration, the extract-state
// registry behind DIT_ERR_STATE and optional per-kernel event timing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dit.h"
#include "kernels.h"

using namespace dit;

namespace {

thread_local std::string g_err;

dit_status fail(dit_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

dit_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return DIT_OK;
  return fail(DIT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
// Longest joint sequence (all tokens, every target latent): the attention
// kernels address one head's K or Vᵀ block (capacity x 128 bf16) with 32-bit
// signed byte offsets, which holds up to 2^23 keys; 2^22 leaves a margin.
constexpr int kMaxTokens = 1 << 22;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct ExtractRecord {
  const void* kv;
  int P, T, B;
};

// Workspace of dit_step_cached_noalloc: one array per GPU, in the code
// object's own device memory (held by each GPU the library runs on until the
// process ends). Host code never uses this name as an address: the device
// address comes from hipGetSymbolAddress, once per device.
#ifndef DIT_F32
static __device__ __align__(256) unsigned char g_step_scratch[DIT_NOALLOC_SCRATCH_BYTES];
#endif

}  // namespace

struct dit_model {
  dit_config cfg;
  const void* t1; const void* t2; const void* mod; const void* so;
  const void* img_in; const void* proj_out;
  std::vector<const void*> qkv, qn, kn, o, gate, up, down;
  // Mutable host state, guarded by `mu`: the registry of extracted caches
  // and the timing events.
  std::mutex mu;
  std::vector<ExtractRecord> extracted;
  int prof_class = 0;
  std::vector<hipEvent_t> ev_start, ev_stop;
  size_t ev_used = 0;
};

namespace {

dit_status check_cfg(const dit_config* c) {
  if (!c) return fail(DIT_ERR_ARG, "config is NULL");
  if (c->hidden <= 0 || c->n_heads <= 0 || c->head_dim <= 0 || c->ffn <= 0 || c->n_layers <= 0 ||
      c->latent <= 0 || c->time_dim <= 0)
    return fail(DIT_ERR_ARG, "dimensions must be positive");
  if (c->head_dim != 128) return fail(DIT_ERR_SHAPE, "head_dim must be 128 (got %d)", c->head_dim);
  if (c->hidden != c->n_heads * c->head_dim)
    return fail(DIT_ERR_SHAPE, "hidden (%d) != n_heads*head_dim (%d)", c->hidden, c->n_heads * c->head_dim);
  if (c->hidden % 256 || c->hidden > 4096)
    return fail(DIT_ERR_SHAPE, "hidden must be a multiple of 256 and <= 4096 (got %d)", c->hidden);
  if (c->ffn % 128) return fail(DIT_ERR_SHAPE, "ffn must be a multiple of 128 (got %d)", c->ffn);
  if (c->latent != 64) return fail(DIT_ERR_SHAPE, "latent must be 64 (got %d)", c->latent);
  if (c->time_dim % 8 || c->time_dim > 1024)
    return fail(DIT_ERR_SHAPE, "time_dim must be a multiple of 8 and <= 1024 (got %d)", c->time_dim);
  int sum = 0;
  for (int a = 0; a < 3; ++a) {
    if (c->rope_dims[a] < 0 || c->rope_dims[a] % 2)
      return fail(DIT_ERR_SHAPE, "rope_dims[%d] must be even and >= 0", a);
    sum += c->rope_dims[a];
  }
  if (sum != c->head_dim) return fail(DIT_ERR_SHAPE, "rope_dims must sum to head_dim");
  if (!(c->rope_base > 1.f) || !(c->eps > 0.f)) return fail(DIT_ERR_ARG, "rope_base/eps out of range");
  return DIT_OK;
}

// Number of target latents sharing the prefix (B <= 1 means one).
inline int n_elem(const dit_seq* s) { return s->B > 1 ? s->B : 1; }
// Rows of every per-token tensor and keys of the cache: P + B*T.
inline int s_all(const dit_seq* s) { return s->P + n_elem(s) * s->T; }

dit_status check_seq(const dit_model* m, const dit_seq* s) {
  if (!s) return fail(DIT_ERR_ARG, "seq is NULL");
  if (s->P < 0 || s->T <= 0) return fail(DIT_ERR_LAYOUT, "need P >= 0 and T > 0 (P=%d T=%d)", s->P, s->T);
  if (s->B < 0) return fail(DIT_ERR_ARG, "negative batch %d", s->B);
  if ((long long)s->P + (long long)(s->B > 1 ? s->B : 1) * s->T > kMaxTokens)
    return fail(DIT_ERR_LAYOUT, "P + B*T exceeds %d tokens", kMaxTokens);
  if (s->B > 1) {
#ifdef DIT_F32
    return fail(DIT_ERR_UNSUPPORTED, "several target latents are not part of the fp32 debug build");
#endif
    if (s->P % 256 || s->T % 256)
      return fail(DIT_ERR_SHAPE, "several target latents need P and T multiples of 256 (P=%d T=%d)",
                  s->P, s->T);
  }
  if (!s->d_row_limit || !s->d_rope_cos || !s->d_rope_sin)
    return fail(DIT_ERR_ARG, "seq device tables are NULL");
  (void)m;
  return DIT_OK;
}

// Workspace plan for n tokens.
struct Plan {
  size_t mod, scale_out, temb_e, a1, a1s, temb, tembs, h, x, qkv, attn, ffn, part, total;
};
Plan plan(const dit_config& c, int n) {
  Plan p{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  const size_t H = c.hidden, F = c.ffn, N = (size_t)n;
  p.mod = take(2 * 4 * H * 4);
  p.scale_out = take(H * 4);
  p.temb_e = take(2 * (size_t)c.time_dim * 4);
  p.a1 = take(2 * H * 4);
  p.a1s = take(2 * H * 4);
  p.temb = take(2 * H * 4);
  p.tembs = take(2 * H * 4);
  p.h = take(N * H * 4);
  const size_t A = sizeof(act_t);
  p.x = take(N * H * A);
  p.qkv = take(N * 3 * H * A);
  p.attn = take(N * H * A);
  p.ffn = take(N * F * A);
  p.part = take(kGemmPartBytes);
  p.total = off;
  return p;
}

// Timing of one launch of a profiled kernel class: a pair of events that
// the launcher records on its kernels' dispatch packets (ev()), or, for the
// launchers that take no events, that are recorded into the stream around
// the launch (by_launch = false).
struct Timed {
  dit_model* m;
  int cls;
  hipStream_t s;
  bool on, by_launch;
  Timed(dit_model* m_, int cls_, hipStream_t s_, bool by_launch_ = true)
      : m(m_), cls(cls_), s(s_), on(m_ && m_->prof_class == cls_), by_launch(by_launch_) {
    if (!on) return;
    if (m->ev_used == m->ev_start.size()) {
      hipEvent_t a, b;
      if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) { on = false; return; }
      m->ev_start.push_back(a);
      m->ev_stop.push_back(b);
    }
    if (!by_launch) (void)hipEventRecord(m->ev_start[m->ev_used], s);
  }
  LaunchEvents ev() const {
    LaunchEvents e;
    if (on && by_launch) {
      e.start = m->ev_start[m->ev_used];
      e.stop = m->ev_stop[m->ev_used];
    }
    return e;
  }
  ~Timed() {
    if (!on) return;
    if (!by_launch) (void)hipEventRecord(m->ev_stop[m->ev_used], s);
    m->ev_used++;
  }
};

inline const uint16_t* U(const void* p) { return static_cast<const uint16_t*>(p); }

// One step over N tokens. extract: all S tokens (rows 0..P-1 prefix);
// cached: the T target tokens (global rows P..S-1).
dit_status run_step(dit_model* m, const dit_seq* seq, bool extract, const float* prefix,
                    const float* x, float sigma, void* kv, float* v_out, void* ws, int flags,
                    hipStream_t st, bool timing = true) {
  dit_model* const tmm = timing ? m : nullptr;   // per-kernel events only when timing
  const dit_config& c = m->cfg;
  const int H = c.hidden, F = c.ffn, nh = c.n_heads, L = c.n_layers;
  // S: one element's sequence (layout tables, mask); SA: all rows/keys with
  // the B target latents; TB: target rows of all elements
  const int P = seq->P, T = seq->T, S = P + T, SA = s_all(seq), TB = SA - P;
  const int cap = dit_kv_capacity(SA);
  const int N = extract ? SA : TB;
  const int n_pre = extract ? P : 0;
  const int q_row0 = extract ? 0 : P;
  const Plan pl = plan(c, N);
  char* w = static_cast<char*>(ws);
  float* mod = reinterpret_cast<float*>(w + pl.mod);
  float* scale_out = reinterpret_cast<float*>(w + pl.scale_out);
  float* te = reinterpret_cast<float*>(w + pl.temb_e);
  float* a1 = reinterpret_cast<float*>(w + pl.a1);
  float* a1s = reinterpret_cast<float*>(w + pl.a1s);
  float* tb = reinterpret_cast<float*>(w + pl.temb);
  float* tbs = reinterpret_cast<float*>(w + pl.tembs);
  float* hbuf = reinterpret_cast<float*>(w + pl.h);
  act_t* xb = reinterpret_cast<act_t*>(w + pl.x);
  act_t* qkv = reinterpret_cast<act_t*>(w + pl.qkv);
  act_t* att = reinterpret_cast<act_t*>(w + pl.attn);
  act_t* ffn = reinterpret_cast<act_t*>(w + pl.ffn);
  float* part = reinterpret_cast<float*>(w + pl.part);
  act_t* kbase = static_cast<act_t*>(kv);
  act_t* vbase = kbase + (size_t)L * nh * cap * 128;
  dit_status rc;
#define LAUNCH(expr, what) \
  do { if ((rc = hip_check((expr), what)) != DIT_OK) return rc; } while (0)

  // ---- conditioning: sinusoid(1000σ) -> MLP -> shared modulation rows ----
  // Row 0: current t; row 1: t = 0 (prefix rows), or t again without
  // causal conditioning. The cached step needs row 0 only.
  const float t = 1000.f * sigma;
  const int nv = extract ? 2 : 1;
  const float t_pre = (flags & DIT_FLAG_NO_CAUSAL_CONDITION) ? t : 0.f;
  LAUNCH(launch_temb(t, t_pre, c.time_dim, c.rope_base, te, st), "temb");
  {
    Timed tm(tmm, DIT_PROF_GEMV, st);
    LAUNCH(launch_gemv(U(m->t1), H, c.time_dim, te, c.time_dim, nv, a1, H, a1s, st, tm.ev()), "gemv t1");
  }
  {
    Timed tm(tmm, DIT_PROF_GEMV, st);
    LAUNCH(launch_gemv(U(m->t2), H, H, a1s, H, nv, tb, H, tbs, st, tm.ev()), "gemv t2");
  }
  {
    Timed tm(tmm, DIT_PROF_GEMV_MOD, st);
    LAUNCH(launch_gemv(U(m->mod), 4 * H, H, tbs, H, nv, mod, 4 * H, nullptr, st, tm.ev()), "gemv mod");
  }
  LAUNCH(launch_gate_tanh(mod, H, nv, st), "gate tanh");
  {
    Timed tm(tmm, DIT_PROF_GEMV, st);
    LAUNCH(launch_gemv(U(m->so), H, H, tbs, H, 1, scale_out, H, nullptr, st, tm.ev()), "gemv so");
  }
  const float* row_t = mod;
  const float* row_0 = extract ? mod + 4 * H : mod;

  // ---- residual stream init ----
  if (extract && P > 0)
    LAUNCH(hipMemcpyAsync(hbuf, prefix, (size_t)P * H * 4, hipMemcpyDeviceToDevice, st), "prefix copy");
  {
    Timed tm(tmm, DIT_PROF_IMG_IN, st);
    LAUNCH(launch_img_in(U(m->img_in), x, TB, H, hbuf + (size_t)n_pre * H, H, st, tm.ev()), "img_in");
  }

  for (int l = 0; l < L; ++l) {
    act_t* kl = kbase + (size_t)l * nh * cap * 128;
    act_t* vl = vbase + (size_t)l * nh * 128 * cap;
    {
      Timed tm(tmm, DIT_PROF_LN, st);
      LAUNCH(launch_ln_mod(hbuf, H, N, H, row_t, row_0, n_pre, c.eps, xb, H, st, tm.ev()), "ln1");
    }
    // QKV projection with the per-head QK-RMSNorm, RoPE and K / Vᵀ cache
    // writes of tokens q_row0 .. q_row0+N-1 fused into its epilogue
    QkArgs q{};
    q.qkv = qkv; q.ld = 3 * H; q.q_row0 = q_row0;
    q.g_begin = q_row0; q.g_end = q_row0 + N;
    q.S = SA; q.cap = cap; q.nh = nh; q.H = H; q.P = P; q.T_el = T;
    q.wq = U(m->qn[l]); q.wk = U(m->kn[l]);
    q.cosv = seq->d_rope_cos; q.sinv = seq->d_rope_sin;
    q.kc = kl; q.vtc = vl; q.eps = c.eps;
    {
      Timed tm(tmm, DIT_PROF_GEMM_QKV, st);
      GemmArgs g{};
      g.A = xb; g.lda = H; g.B = U(m->qkv[l]); g.ldb = H; g.M = N; g.N = 3 * H; g.K = H;
      g.C = qkv; g.ldc = 3 * H;
      g.part = part; g.part_bytes = kGemmPartBytes;
      g.qk = q;
      LAUNCH(launch_gemm(g, EPI_QKV, st, tm.ev()), "gemm qkv");
    }
    if (extract && cap > SA) {
      // cache keys SA .. cap-1 (capacity padding) are zero-filled
      Timed tm(tmm, DIT_PROF_QKNORM_ROPE, st, false);
      QkArgs z = q;
      z.g_begin = SA; z.g_end = cap;
      LAUNCH(launch_qknorm_rope(z, st), "cache padding");
    }
    {
      Timed tm(tmm, DIT_PROF_ATTENTION, st);
      AttnArgs a{};
      a.q = qkv; a.q_stride = 3 * H; a.q_off = q_row0; a.N = N;
      a.k = kl; a.vt = vl; a.cap = cap; a.S = S; a.nh = nh; a.limit = seq->d_row_limit;
      a.out = att; a.out_stride = H; a.P = P; a.T_el = T;
      a.part = part; a.part_bytes = kGemmPartBytes;   // free between the GEMMs
      LAUNCH(launch_attention(a, st, tm.ev()), "attention");
    }
    {
      Timed tm(tmm, DIT_PROF_GEMM_O, st);
      GemmArgs g{};
      g.A = att; g.lda = H; g.B = U(m->o[l]); g.ldb = H; g.M = N; g.N = H; g.K = H;
      g.Hres = hbuf; g.ldh = H; g.gate_t = row_t + H; g.gate_0 = row_0 + H; g.n_pre = n_pre;
      g.part = part; g.part_bytes = kGemmPartBytes;
      LAUNCH(launch_gemm(g, EPI_RESID, st, tm.ev()), "gemm o");
    }
    {
      Timed tm(tmm, DIT_PROF_LN, st);
      LAUNCH(launch_ln_mod(hbuf, H, N, H, row_t + 2 * H, row_0 + 2 * H, n_pre, c.eps, xb, H, st, tm.ev()), "ln2");
    }
    {
      Timed tm(tmm, DIT_PROF_GEMM_GATEUP, st);
      GemmArgs g{};
      g.A = xb; g.lda = H; g.B = U(m->gate[l]); g.B2 = U(m->up[l]); g.ldb = H;
      g.M = N; g.N = 2 * F; g.K = H; g.C = ffn; g.ldc = F;
      g.part = part; g.part_bytes = kGemmPartBytes;
      LAUNCH(launch_gemm(g, EPI_SWIGLU, st, tm.ev()), "gemm gate/up");
    }
    {
      Timed tm(tmm, DIT_PROF_GEMM_DOWN, st);
      GemmArgs g{};
      g.A = ffn; g.lda = F; g.B = U(m->down[l]); g.ldb = F; g.M = N; g.N = H; g.K = F;
      g.Hres = hbuf; g.ldh = H; g.gate_t = row_t + 3 * H; g.gate_0 = row_0 + 3 * H; g.n_pre = n_pre;
      g.part = part; g.part_bytes = kGemmPartBytes;
      LAUNCH(launch_gemm(g, EPI_RESID, st, tm.ev()), "gemm down");
    }
  }

  // ---- scale-only final AdaLN on target rows, proj_out -> v ----
#ifdef DIT_F32
  LAUNCH(launch_ln_mod(hbuf + (size_t)n_pre * H, H, TB, H, scale_out, scale_out, 0, c.eps, xb, H, st),
         "final ln");
  {
    GemmArgs g{};
    g.A = xb; g.lda = H; g.B = U(m->proj_out); g.ldb = H; g.M = TB; g.N = c.latent; g.K = H;
    g.C = v_out; g.ldc = c.latent;
    LAUNCH(launch_gemm(g, EPI_F32, st), "gemm proj_out");
  }
#else
  {
    Timed tm(tmm, DIT_PROF_FINAL, st);
    LAUNCH(launch_final_out(hbuf + (size_t)n_pre * H, H, TB, H, scale_out, c.eps, U(m->proj_out), v_out, st,
                            tm.ev()),
           "final adaln + proj_out");
  }
#endif
#undef LAUNCH
  return DIT_OK;
}

dit_status check_step_common(dit_model* m, const dit_seq* seq, const float* x, void* kv,
                             size_t kv_bytes, float* v_out, void* ws, size_t ws_bytes, int n) {
  if (!m) return fail(DIT_ERR_ARG, "model is NULL");
  dit_status rc = check_seq(m, seq);
  if (rc) return rc;
  if (!x || !kv || !v_out || !ws) return fail(DIT_ERR_ARG, "x, kv_cache, v_out and workspace must be non-NULL");
  const size_t need_kv = dit_kv_cache_bytes(m, s_all(seq));
  if (kv_bytes < need_kv)
    return fail(DIT_ERR_WORKSPACE, "kv_cache has %zu bytes, needs %zu", kv_bytes, need_kv);
  const size_t need_ws = dit_workspace_bytes(m, n);
  if (ws_bytes < need_ws)
    return fail(DIT_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need_ws);
  if ((reinterpret_cast<uintptr_t>(kv) | reinterpret_cast<uintptr_t>(ws) |
       reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(v_out)) & 15)
    return fail(DIT_ERR_ARG, "device buffers must be 16-byte aligned");
  return DIT_OK;
}

}  // namespace

extern "C" {

const char* dit_last_error(void) { return g_err.c_str(); }
#ifdef DIT_F32
const char* dit_version(void) { return "dit-gfx950 0.1 fp32-debug"; }
#else
const char* dit_version(void) { return "dit-gfx950 0.1"; }
#endif

int dit_kv_capacity(int S) { return S <= 0 ? 0 : (S + 127) / 128 * 128; }

size_t dit_kv_cache_bytes(const dit_model* m, int S) {
  if (!m || S <= 0) return 0;
  return (size_t)2 * m->cfg.n_layers * m->cfg.n_heads * (size_t)dit_kv_capacity(S) * m->cfg.head_dim *
         sizeof(act_t);
}

size_t dit_workspace_bytes(const dit_model* m, int n_tokens) {
  if (!m || n_tokens <= 0) return 0;
  return plan(m->cfg, n_tokens).total;
}

dit_status dit_build_layout(const dit_config* cfg, const int* seg_kind, const int* seg_rows,
                            const int* seg_cols, int n_seg, int32_t* image_ids, int32_t* coords,
                            int32_t* row_limit, float* rope_cos, float* rope_sin, int* P_out,
                            int* T_out) {
  dit_status rc = check_cfg(cfg);
  if (rc) return rc;
  if (!seg_kind || !seg_rows || !seg_cols || n_seg <= 0) return fail(DIT_ERR_ARG, "empty segment list");
  // validate: sizes positive, exactly one target and it is last
  long long S = 0;
  int n_target = 0;
  for (int i = 0; i < n_seg; ++i) {
    const int k = seg_kind[i];
    if (k < 0 || k > 2) return fail(DIT_ERR_LAYOUT, "segment %d: kind %d unknown", i, k);
    if (seg_rows[i] <= 0 || (k != 0 && seg_cols[i] <= 0))
      return fail(DIT_ERR_LAYOUT, "segment %d: non-positive size", i);
    S += (k == 0) ? seg_rows[i] : (long long)seg_rows[i] * seg_cols[i];
    if (k == 2) {
      ++n_target;
      if (i != n_seg - 1) return fail(DIT_ERR_LAYOUT, "the target image must be the last segment");
    }
    if (S > kMaxTokens) return fail(DIT_ERR_LAYOUT, "sequence longer than %d tokens", kMaxTokens);
  }
  if (n_target != 1) return fail(DIT_ERR_LAYOUT, "exactly one target segment is required");
  int n_ref = 0;
  for (int i = 0; i < n_seg; ++i) n_ref += seg_kind[i] == 1;
  const int Tt = seg_rows[n_seg - 1] * seg_cols[n_seg - 1];
  if (P_out) *P_out = (int)S - Tt;
  if (T_out) *T_out = Tt;

  // per-axis RoPE frequencies base^(-2j/d_a), pairs ordered axis by axis
  const int npair = cfg->head_dim / 2;
  std::vector<int> pair_axis(npair);
  std::vector<double> pair_freq(npair);
  {
    int m = 0;
    for (int a = 0; a < 3; ++a)
      for (int j = 0; j < cfg->rope_dims[a] / 2; ++j, ++m) {
        pair_axis[m] = a;
        pair_freq[m] = std::pow((double)cfg->rope_base, -2.0 * j / (double)cfg->rope_dims[a]);
      }
  }
  int i = 0, text_i = 0, ref_i = 0;
  for (int sgi = 0; sgi < n_seg; ++sgi) {
    const int k = seg_kind[sgi];
    const int rows = seg_rows[sgi], cols = (k == 0) ? 1 : seg_cols[sgi];
    const int cnt = (k == 0) ? rows : rows * cols;
    const int id = (k == 0) ? -1 : (k == 1 ? ref_i : n_ref);
    const int block_end = i + cnt - 1;
    for (int e = 0; e < cnt; ++e, ++i) {
      int cf, ch, cw;
      if (k == 0) { cf = ch = cw = text_i++; }
      else { cf = 0; ch = e / cols - rows / 2; cw = e % cols - cols / 2; }
      if (image_ids) image_ids[i] = id;
      if (coords) { coords[3 * i] = cf; coords[3 * i + 1] = ch; coords[3 * i + 2] = cw; }
      if (row_limit) row_limit[i] = (k == 0) ? i : block_end;
      if (rope_cos || rope_sin) {
        const int cc[3] = {cf, ch, cw};
        for (int m = 0; m < npair; ++m) {
          const double ang = (double)cc[pair_axis[m]] * pair_freq[m];
          if (rope_cos) rope_cos[(size_t)i * npair + m] = (float)std::cos(ang);
          if (rope_sin) rope_sin[(size_t)i * npair + m] = (float)std::sin(ang);
        }
      }
    }
    if (k == 1) ++ref_i;
  }
  return DIT_OK;
}

dit_status dit_load_weights(const dit_config* cfg, const dit_weights* w, dit_model** out) {
  dit_status rc = check_cfg(cfg);
  if (rc) return rc;
  if (!w || !out) return fail(DIT_ERR_ARG, "weights or out is NULL");
  if (!w->t1 || !w->t2 || !w->mod || !w->so || !w->img_in || !w->proj_out)
    return fail(DIT_ERR_ARG, "a global weight pointer is NULL");
  if (!w->qkv || !w->q_norm || !w->k_norm || !w->o || !w->gate || !w->up || !w->down)
    return fail(DIT_ERR_ARG, "a per-layer weight array is NULL");
  const void* g[] = {w->t1, w->t2, w->mod, w->so, w->img_in, w->proj_out};
  for (const void* p : g)
    if (reinterpret_cast<uintptr_t>(p) & 15) return fail(DIT_ERR_ARG, "weights must be 16-byte aligned");
  dit_model* m = new (std::nothrow) dit_model();
  if (!m) return fail(DIT_ERR_ARG, "out of host memory");
  m->cfg = *cfg;
  m->t1 = w->t1; m->t2 = w->t2; m->mod = w->mod; m->so = w->so; m->img_in = w->img_in;
  m->proj_out = w->proj_out;
  const int L = cfg->n_layers;
  for (int l = 0; l < L; ++l) {
    const void* p[] = {w->qkv[l], w->q_norm[l], w->k_norm[l], w->o[l], w->gate[l], w->up[l], w->down[l]};
    for (const void* q : p)
      if (!q || (reinterpret_cast<uintptr_t>(q) & 15)) {
        delete m;
        return fail(DIT_ERR_ARG, "layer %d: weight pointer NULL or not 16-byte aligned", l);
      }
    m->qkv.push_back(w->qkv[l]); m->qn.push_back(w->q_norm[l]); m->kn.push_back(w->k_norm[l]);
    m->o.push_back(w->o[l]); m->gate.push_back(w->gate[l]); m->up.push_back(w->up[l]);
    m->down.push_back(w->down[l]);
  }
  *out = m;
  return DIT_OK;
}

void dit_free(dit_model* m) {
  if (!m) return;
  for (auto e : m->ev_start) (void)hipEventDestroy(e);
  for (auto e : m->ev_stop) (void)hipEventDestroy(e);
  delete m;
}

dit_status dit_step_extract(dit_model* m, const dit_seq* seq, const float* prefix_hidden,
                            const float* x, float sigma, void* kv_cache, size_t kv_bytes,
                            float* v_out, void* workspace, size_t ws_bytes, int flags,
                            void* stream) {
  dit_status rc = check_step_common(m, seq, x, kv_cache, kv_bytes, v_out, workspace, ws_bytes,
                                    seq ? s_all(seq) : 0);
  if (rc) return rc;
  if (seq->P > 0 && !prefix_hidden) return fail(DIT_ERR_ARG, "prefix_hidden is NULL");
  if (flags & ~DIT_FLAG_NO_CAUSAL_CONDITION) return fail(DIT_ERR_ARG, "unknown flags 0x%x", flags);
  if (!std::isfinite(sigma)) return fail(DIT_ERR_ARG, "sigma is not finite");
  std::lock_guard<std::mutex> lock(m->mu);
  // forget any previous extract of this cache before overwriting it
  for (size_t i = 0; i < m->extracted.size(); ++i)
    if (m->extracted[i].kv == kv_cache) { m->extracted.erase(m->extracted.begin() + i); break; }
  rc = run_step(m, seq, true, prefix_hidden, x, sigma, kv_cache, v_out, workspace, flags,
                static_cast<hipStream_t>(stream));
  if (rc) return rc;
  if (!(flags & DIT_FLAG_NO_CAUSAL_CONDITION)) m->extracted.push_back({kv_cache, seq->P, seq->T, n_elem(seq)});
  return DIT_OK;
}

dit_status dit_step_cached(dit_model* m, const dit_seq* seq, const float* x, float sigma,
                           void* kv_cache, size_t kv_bytes, float* v_out, void* workspace,
                           size_t ws_bytes, void* stream) {
  dit_status rc = check_step_common(m, seq, x, kv_cache, kv_bytes, v_out, workspace, ws_bytes,
                                    seq ? s_all(seq) - seq->P : 0);
  if (rc) return rc;
  if (!std::isfinite(sigma)) return fail(DIT_ERR_ARG, "sigma is not finite");
  std::lock_guard<std::mutex> lock(m->mu);
  bool ok = false;
  for (const auto& r : m->extracted)
    if (r.kv == kv_cache && r.P == seq->P && r.T == seq->T && r.B == n_elem(seq)) ok = true;
  if (!ok)
    return fail(DIT_ERR_STATE,
                "no dit_step_extract with t=0 conditioning ran on this cache for P=%d T=%d B=%d",
                seq->P, seq->T, n_elem(seq));
  return run_step(m, seq, false, nullptr, x, sigma, kv_cache, v_out, workspace, 0,
                  static_cast<hipStream_t>(stream));
}

dit_status dit_step_cached_noalloc(dit_model* m, const dit_seq* seq, const float* x, float sigma,
                                   void* kv_cache, size_t kv_bytes, float* v_out, void* stream) {
  if (!m) return fail(DIT_ERR_ARG, "model is NULL");
  dit_status rc = check_seq(m, seq);
  if (rc) return rc;
  const int n = s_all(seq) - seq->P;
  const size_t need = dit_workspace_bytes(m, n);
  if (need > DIT_NOALLOC_SCRATCH_BYTES)
    return fail(DIT_ERR_WORKSPACE,
                "dit_step_cached_noalloc: %d target rows need %zu bytes of workspace, above the "
                "library's fixed %zu-byte device scratch (use dit_step_cached with a workspace)",
                n, need, (size_t)DIT_NOALLOC_SCRATCH_BYTES);
#ifdef DIT_F32
  (void)x; (void)sigma; (void)kv_cache; (void)kv_bytes; (void)v_out; (void)stream;
  return fail(DIT_ERR_UNSUPPORTED, "dit_step_cached_noalloc is not part of the fp32 debug build");
#else
  // device address of this GPU's scratch array, looked up once per device
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  rc = hip_check(hipGetDevice(&dev), "noalloc: device");
  if (rc) return rc;
  if (dev < 0 || dev >= 64) return fail(DIT_ERR_UNSUPPORTED, "device index %d", dev);
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
      void* p = nullptr;
      rc = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(g_step_scratch)), "noalloc: scratch address");
      if (rc) return rc;
      addr[dev] = p;
    }
    ws = addr[dev];
  }
  rc = check_step_common(m, seq, x, kv_cache, kv_bytes, v_out, ws, DIT_NOALLOC_SCRATCH_BYTES, n);
  if (rc) return rc;
  if (!std::isfinite(sigma)) return fail(DIT_ERR_ARG, "sigma is not finite");
  std::lock_guard<std::mutex> lock(m->mu);
  bool ok = false;
  for (const auto& r : m->extracted)
    if (r.kv == kv_cache && r.P == seq->P && r.T == seq->T && r.B == n_elem(seq)) ok = true;
  if (!ok)
    return fail(DIT_ERR_STATE,
                "no dit_step_extract with t=0 conditioning ran on this cache for P=%d T=%d B=%d",
                seq->P, seq->T, n_elem(seq));
  // nothing in the workspace has to start at zero: every region a step
  // reads is written earlier in the same step
  return run_step(m, seq, false, nullptr, x, sigma, kv_cache, v_out, ws, 0,
                  static_cast<hipStream_t>(stream), false);
#endif
}

dit_status euler_update(float* x, const float* v, float sigma_k, float sigma_k1, long long n,
                        void* stream) {
  if (!x || !v) return fail(DIT_ERR_ARG, "x or v is NULL");
  if (n < 0) return fail(DIT_ERR_ARG, "negative length");
  if (!std::isfinite(sigma_k) || !std::isfinite(sigma_k1)) return fail(DIT_ERR_ARG, "sigma is not finite");
  return hip_check(launch_euler(x, v, sigma_k1 - sigma_k, n, static_cast<hipStream_t>(stream)), "euler");
}

dit_status dit_latent_standardize(float* z, const float* mean, const float* std, long long rows,
                                  int channels, int inverse, void* stream) {
  if (!z || !mean || !std) return fail(DIT_ERR_ARG, "NULL argument");
  if (rows < 0 || channels < 1 || channels > 1024) return fail(DIT_ERR_ARG, "bad rows/channels");
  if (inverse != 0 && inverse != 1) return fail(DIT_ERR_ARG, "inverse must be 0 or 1");
  if ((channels & 3) == 0 &&
      ((reinterpret_cast<uintptr_t>(z) | reinterpret_cast<uintptr_t>(mean) | reinterpret_cast<uintptr_t>(std)) & 15))
    return fail(DIT_ERR_ARG, "z, mean and std must be 16-byte aligned");
  return hip_check(launch_standardize(z, mean, std, rows, channels, inverse, static_cast<hipStream_t>(stream)),
                   "standardize");
}

dit_status dit_img_in(const dit_model* m, const float* latents, int n, float* hidden, void* stream) {
  if (!m || !latents || !hidden) return fail(DIT_ERR_ARG, "NULL argument");
  if (n < 0) return fail(DIT_ERR_ARG, "negative token count");
  return hip_check(launch_img_in(U(m->img_in), latents, n, m->cfg.hidden, hidden, m->cfg.hidden,
                                 static_cast<hipStream_t>(stream)),
                   "img_in");
}

dit_status dit_debug_mask(const dit_seq* seq, uint8_t* mask, void* stream) {
  dit_status rc = check_seq(nullptr, seq);
  if (rc) return rc;
  if (!mask) return fail(DIT_ERR_ARG, "mask is NULL");
  return hip_check(launch_debug_mask(seq->d_row_limit, seq->P + seq->T, mask,
                                     static_cast<hipStream_t>(stream)),
                   "debug mask");
}

dit_status dit_debug_attention(const dit_seq* seq, int n_heads, const void* q, int q_stride,
                               int q_off, int N, const void* kv_cache, void* out, int variant,
                               void* scratch, size_t scratch_bytes, void* stream) {
  dit_status rc = check_seq(nullptr, seq);
  if (rc) return rc;
  const int S = seq->P + seq->T;
  if (!q || !kv_cache || !out) return fail(DIT_ERR_ARG, "NULL argument");
  if (n_heads <= 0 || N <= 0 || q_off < 0 || q_off + N > S || q_stride < n_heads * 128 || q_stride % 8)
    return fail(DIT_ERR_ARG, "bad attention shape");
  if (variant < 0 || variant > 6) return fail(DIT_ERR_ARG, "unknown attention variant %d", variant);
  if ((variant == 5 || variant == 6) && (q_off != seq->P || S % 64))
    return fail(DIT_ERR_ARG, "variants 5 and 6 take target rows (q_off = P) and S a multiple of 64");
  if (scratch && (reinterpret_cast<uintptr_t>(scratch) & 15))
    return fail(DIT_ERR_ARG, "scratch must be 16-byte aligned");
#ifdef DIT_F32
  (void)scratch_bytes; (void)stream;
  return fail(DIT_ERR_UNSUPPORTED, "dit_debug_attention is not part of the fp32 debug build");
#else
  const int cap = dit_kv_capacity(S);
  AttnArgs a{};
  a.q = static_cast<const act_t*>(q); a.q_stride = q_stride; a.q_off = q_off; a.N = N;
  a.k = static_cast<const act_t*>(kv_cache);
  a.vt = a.k + (size_t)n_heads * cap * 128;
  a.cap = cap; a.S = S; a.nh = n_heads; a.limit = seq->d_row_limit;
  a.out = static_cast<act_t*>(out); a.out_stride = n_heads * 128;
  a.P = seq->P; a.T_el = seq->T;
  a.part = scratch ? static_cast<float*>(scratch) : nullptr;
  a.part_bytes = scratch ? scratch_bytes : 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (variant == 0) return hip_check(launch_attention(a, st), "debug attention");
  return hip_check(launch_attention_variant(a, variant, st), "debug attention");
#endif
}

dit_status dit_debug_gemm(const dit_gemm_desc* d, void* stream) {
  if (!d) return fail(DIT_ERR_ARG, "descriptor is NULL");
  const int epi = d->epilogue;
  if (epi != DIT_GEMM_BF16 && epi != DIT_GEMM_RESID && epi != DIT_GEMM_SWIGLU && epi != DIT_GEMM_QKV)
    return fail(DIT_ERR_ARG, "unknown epilogue %d", epi);
  if (!d->A || !d->B) return fail(DIT_ERR_ARG, "A or B is NULL");
  if (epi == DIT_GEMM_RESID ? (!d->h || !d->gate_t || !d->gate_0) : !d->C)
    return fail(DIT_ERR_ARG, "output or gate pointer is NULL");
  if (epi == DIT_GEMM_SWIGLU && !d->B2) return fail(DIT_ERR_ARG, "SwiGLU needs B2 (up)");
  if (d->splits != 0 && d->splits != 2 && d->splits != 4) return fail(DIT_ERR_ARG, "splits must be 0, 2 or 4");
  const int N = epi == DIT_GEMM_SWIGLU ? 2 * d->N : d->N;   // packed gate/up width
  if (!gemm_shape_ok(d->M, N, d->K, EPI_BF16))
    return fail(DIT_ERR_SHAPE, "GEMM needs M > 0, N %% 256 == 0 and K %% 64 == 0");
  if (d->scratch && (reinterpret_cast<uintptr_t>(d->scratch) & 15))
    return fail(DIT_ERR_ARG, "scratch must be 16-byte aligned");
  const int tail = d->M - (d->M - 1) / 256 * 256;   // rows of the last 256-row block
  if (d->splits > 1) {
    if ((d->K / 64) % d->splits) return fail(DIT_ERR_ARG, "K / 64 must be divisible by splits");
    if (!d->scratch || d->scratch_bytes < (size_t)d->splits * tail * N * 4)
      return fail(DIT_ERR_ARG, "scratch below splits * rows * N * 4 bytes");
  }
#ifdef DIT_F32
  (void)stream; (void)tail;
  return fail(DIT_ERR_UNSUPPORTED, "dit_debug_gemm is not part of the fp32 debug build");
#else
  GemmArgs g{};
  g.A = static_cast<const act_t*>(d->A); g.lda = d->K;
  g.B = U(d->B); g.B2 = U(d->B2); g.ldb = d->K;
  g.M = d->M; g.N = N; g.K = d->K;
  g.C = d->C; g.ldc = d->N;
  g.Hres = d->h; g.ldh = d->N; g.gate_t = d->gate_t; g.gate_0 = d->gate_0; g.n_pre = d->n_pre;
  g.part = static_cast<float*>(d->scratch); g.part_bytes = d->scratch ? d->scratch_bytes : 0;
  int kepi = EPI_BF16;
  if (epi == DIT_GEMM_RESID) kepi = EPI_RESID;
  if (epi == DIT_GEMM_SWIGLU) kepi = EPI_SWIGLU;
  if (epi == DIT_GEMM_QKV) {
    kepi = EPI_QKV;
    const int nh = d->n_heads, H = nh * 128;
    if (nh <= 0 || d->N != 3 * H) return fail(DIT_ERR_SHAPE, "QKV needs N = 3 * n_heads * 128");
    if (!d->q_norm || !d->k_norm || !d->rope_cos || !d->rope_sin || !d->kv_cache)
      return fail(DIT_ERR_ARG, "QKV needs norm weights, RoPE tables and a cache");
    if (d->q_row0 < 0 || (long long)d->q_row0 + d->M > d->S || d->S > kMaxTokens)
      return fail(DIT_ERR_ARG, "rows q_row0 .. q_row0 + M - 1 must lie inside S");
    if (!(d->eps > 0.f)) return fail(DIT_ERR_ARG, "eps must be positive");
    const int cap = dit_kv_capacity(d->S);
    QkArgs& q = g.qk;
    q.qkv = static_cast<act_t*>(d->C); q.ld = d->N; q.q_row0 = d->q_row0;
    q.g_begin = d->q_row0; q.g_end = d->q_row0 + d->M;
    q.S = d->S; q.cap = cap; q.nh = nh; q.H = H; q.P = 0; q.T_el = 0;
    q.wq = U(d->q_norm); q.wk = U(d->k_norm);
    q.cosv = d->rope_cos; q.sinv = d->rope_sin;
    q.kc = static_cast<act_t*>(d->kv_cache);
    q.vtc = q.kc + (size_t)nh * cap * 128;
    q.eps = d->eps;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (d->splits > 1) return hip_check(launch_gemm_forced_split(g, kepi, d->splits, st), "debug gemm");
  return hip_check(launch_gemm(g, kepi, st), "debug gemm");
#endif
}

dit_status dit_debug_final_out(const float* h, int ldh, int rows, int H, const float* scale_out,
                               float eps, const void* w_out, float* v_out, void* stream) {
  if (!h || !scale_out || !w_out || !v_out) return fail(DIT_ERR_ARG, "NULL argument");
  if (rows < 0 || H <= 0 || H % 256 || H > 4096 || ldh < H || ldh % 4)
    return fail(DIT_ERR_SHAPE, "need H a multiple of 256, at most 4096, ldh >= H and a multiple of 4");
  if (!(eps > 0.f)) return fail(DIT_ERR_ARG, "eps must be positive");
  if ((reinterpret_cast<uintptr_t>(h) | reinterpret_cast<uintptr_t>(scale_out) |
       reinterpret_cast<uintptr_t>(w_out) | reinterpret_cast<uintptr_t>(v_out)) & 15)
    return fail(DIT_ERR_ARG, "buffers must be 16-byte aligned");
#ifdef DIT_F32
  (void)stream;
  return fail(DIT_ERR_UNSUPPORTED, "dit_debug_final_out is not part of the fp32 debug build");
#else
  return hip_check(launch_final_out(h, ldh, rows, H, scale_out, eps, U(w_out), v_out,
                                    static_cast<hipStream_t>(stream)),
                   "final out");
#endif
}

dit_status dit_debug_gemv(const void* W, int O, int I, const float* X, int ldx, int nv, float* Y,
                          float* Ys, void* stream) {
  if (!W || !X || !Y) return fail(DIT_ERR_ARG, "NULL argument");
  if (nv < 1 || nv > 2) return fail(DIT_ERR_ARG, "nv must be 1 or 2");
  if (O <= 0 || I <= 0 || I % 8 || I > 4096 || (size_t)O * I * 2 >= 0x80000000u || ldx < I || ldx % 4)
    return fail(DIT_ERR_SHAPE, "need O > 0, I a multiple of 8 and at most 4096, O*I*2 < 2^31, ldx >= I "
                               "and a multiple of 4");
  if ((reinterpret_cast<uintptr_t>(W) | reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(Y) |
       reinterpret_cast<uintptr_t>(Ys)) & 15)
    return fail(DIT_ERR_ARG, "buffers must be 16-byte aligned");
  return hip_check(launch_gemv(U(W), O, I, X, ldx, nv, Y, O, Ys, static_cast<hipStream_t>(stream)), "gemv");
}

dit_status dit_debug_stream_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return fail(DIT_ERR_ARG, "NULL argument");
  if (bytes % 16 || ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15))
    return fail(DIT_ERR_ARG, "bytes and pointers must be multiples of 16");
  return hip_check(launch_stream_copy(src, dst, bytes, static_cast<hipStream_t>(stream)), "copy");
}

dit_status dit_debug_mfma_loop(const void* ops, float* out, int blocks, int iters, void* stream) {
  if (!ops || !out) return fail(DIT_ERR_ARG, "NULL argument");
  if (blocks <= 0 || iters <= 0) return fail(DIT_ERR_ARG, "blocks and iters must be positive");
  if ((reinterpret_cast<uintptr_t>(ops) | reinterpret_cast<uintptr_t>(out)) & 15)
    return fail(DIT_ERR_ARG, "buffers must be 16-byte aligned");
#ifdef DIT_F32
  (void)stream;
  return fail(DIT_ERR_UNSUPPORTED, "dit_debug_mfma_loop is not part of the fp32 debug build");
#else
  return hip_check(launch_mfma_loop(static_cast<const uint16_t*>(ops), out, blocks, iters,
                                    static_cast<hipStream_t>(stream)),
                   "mfma loop");
#endif
}

dit_status dit_profile_enable(dit_model* m, int kernel_class) {
  if (!m) return fail(DIT_ERR_ARG, "model is NULL");
  if (kernel_class < DIT_PROF_OFF || kernel_class > DIT_PROF_GEMV_MOD)
    return fail(DIT_ERR_ARG, "unknown kernel class %d", kernel_class);
  std::lock_guard<std::mutex> lock(m->mu);
  m->prof_class = kernel_class;
  m->ev_used = 0;
  return DIT_OK;
}

dit_status dit_profile_read(dit_model* m, double* total_ms, long long* launches) {
  if (!m || !total_ms || !launches) return fail(DIT_ERR_ARG, "NULL argument");
  std::lock_guard<std::mutex> lock(m->mu);
  double tot = 0;
  for (size_t i = 0; i < m->ev_used; ++i) {
    hipError_t e = hipEventSynchronize(m->ev_stop[i]);
    if (e != hipSuccess) return hip_check(e, "event sync");
    float ms = 0;
    e = hipEventElapsedTime(&ms, m->ev_start[i], m->ev_stop[i]);
    if (e != hipSuccess) return hip_check(e, "event elapsed");
    tot += ms;
  }
  *total_ms = tot;
  *launches = (long long)m->ev_used;
  m->ev_used = 0;
  return DIT_OK;
}

}  // extern "C"
