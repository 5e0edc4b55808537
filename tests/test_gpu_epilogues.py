"""GPU parity of each shipped MFMA GEMM epilogue, element by element, through
the GEMM test hook: the same kernels the step launches (plain bf16 store,
fp32 store of proj_out, gated fp32 residual update, SwiGLU, and QK-RMSNorm
+ RoPE + KV-cache write), with and without the split-K path, against an
fp64 evaluation of the same bf16 operands.

Tolerances allow only what fp32 accumulation and the final rounding can
change: an absolute accumulation bound of 2^-20 * sum_k |a_k b_k| per dot
product (much more than fp32 summation of K <= 16384 terms in any order
reaches), and for bf16 outputs one bf16 ulp of the fp64 value. In addition
at least 99.5% of the bf16 outputs must equal the fp64 value rounded to
bf16 exactly (a dot product whose fp32 and fp64 values straddle a rounding
boundary is the only allowed difference)."""
import numpy as np
import pytest
import torch

from diffusion_transformer_amd import synth
from gpu_common import cache_views, i16_to_f32, say, split_cases

pytestmark = pytest.mark.gpu

L = pytest.importorskip("diffusion_transformer_amd._lib")

ACC = 2.0 ** -20     # accumulation bound per unit of sum |a b|


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def bf16_np(x):
    """fp64/fp32 numpy -> nearest bf16 (via fp32), as float64."""
    return synth.round_bf16(np.asarray(x, np.float32)).astype(np.float64)


def ulp_bf16(x):
    """One bf16 ulp at |x| (8 significant bits)."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def operands(M, N, K, seed, n_b=1):
    """A ~ N(0,1) and weights ~ N(0, 1/K), bf16, on the host (fp64 copies)
    and on the device."""
    g = torch.Generator().manual_seed(seed)
    A = torch.randn((M, K), generator=g).to(torch.bfloat16)
    Bs = [(torch.randn((N, K), generator=g) / np.sqrt(K)).to(torch.bfloat16) for _ in range(n_b)]
    return A, Bs


def host(t):
    return t.double().numpy()


def check_bf16(got, ref, bound, what):
    """got: bf16 values (float64), ref: fp64 values, bound: extra absolute
    bound per element."""
    err = np.abs(got - ref)
    assert np.all(err <= ulp_bf16(ref) + bound), \
        f"{what}: {(err > ulp_bf16(ref) + bound).sum()} elements beyond 1 ulp + bound"
    exact = float(np.mean(got == bf16_np(ref)))
    say(f"  {what}: {exact * 100:.3f}% equal to the rounded fp64 value")
    assert exact >= 0.995, (what, exact)


def scratch_for(splits, N, dev):
    return torch.empty(4 * 256 * N * 2, dtype=torch.float32, device=dev) if splits else None


SHAPES = [(700, 512, 512), (256, 256, 64), (37, 768, 1024)]


@pytest.mark.parametrize("M,N,K,splits", split_cases(SHAPES))
def test_bf16_epilogue(dev, M, N, K, splits):
    A, (B,) = operands(M, N, K, seed=M + N + K)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    say(f"bf16 epilogue M={M} N={N} K={K} splits={splits}")
    L.dit_debug_gemm("bf16", M, N, K, A.to(dev), B.to(dev), C, splits=splits,
                     scratch=scratch_for(splits, N, dev))
    torch.cuda.synchronize()
    a, b = host(A), host(B)
    check_bf16(host(C.cpu()), a @ b.T, ACC * (np.abs(a) @ np.abs(b).T), "C")


@pytest.mark.parametrize("rows,H", [(4096, 4096), (700, 4096), (37, 256), (1, 512), (16, 4096)])
def test_final_adaln_proj_out(dev, rows, H):
    """The step's last kernel: v = W_out (LN(h) (1 + scale_out)), LN
    non-affine with population variance and eps 1e-6, the scaled row rounded
    to bf16, fp32 accumulation over H. Against fp64; the bound allows the
    fp32 accumulation and, for the few elements whose fp32 normalized value
    lies within fp32 error of a bf16 rounding boundary, the other neighbour."""
    g = torch.Generator().manual_seed(rows + H)
    h = 3.0 * torch.randn((rows, H), generator=g) + 0.5
    sc = 0.3 * torch.randn(H, generator=g)
    W = (torch.randn((64, H), generator=g) / np.sqrt(H)).to(torch.bfloat16)
    v = torch.full((rows, 64), float("nan"), device=dev)
    say(f"final AdaLN + proj_out rows={rows} H={H}")
    L.dit_debug_final_out(h.to(dev), sc.to(dev), W.to(dev), v)
    torch.cuda.synchronize()
    hh = h.double().numpy()
    y = (hh - hh.mean(1, keepdims=True)) / np.sqrt(hh.var(1, keepdims=True) + 1e-6)
    y = y * (1.0 + sc.double().numpy())
    yb = bf16_np(y)
    w = host(W)
    ref = yb @ w.T
    near = ulp_bf16(y) / 2 - np.abs(y - yb) <= 4e-6 * np.abs(y) + 1e-7
    bound = ACC * (np.abs(yb) @ np.abs(w).T) + (near * ulp_bf16(y)) @ np.abs(w).T
    err = np.abs(v.cpu().double().numpy() - ref)
    say(f"  max err / bound {float((err / bound).max()):.3f}; {int(near.sum())} near-boundary inputs")
    assert np.all(err <= bound)


@pytest.mark.parametrize("O,I,nv,silu", [(16384, 4096, 2, False), (4096, 4096, 1, True), (4096, 256, 2, True),
                                         (37, 24, 1, False), (1001, 520, 2, True)])
def test_gemv_fp32_accumulation(dev, O, I, nv, silu):
    """The step's GEMV (timestep MLP, shared modulation, final scale): Y =
    W X for bf16 W and fp32 X, every output within the fp32 accumulation
    bound of the fp64 product, and SiLU(Y) where the MLP asks for it. The
    shapes are the modulation linear [16384 x 4096] on both timestep rows,
    the MLP's linears, and ragged ones (odd pair count, I not a multiple of
    the 512 values a wave covers per pass)."""
    g = torch.Generator().manual_seed(O + I + nv)
    W = (torch.randn((O, I), generator=g) / np.sqrt(I)).to(torch.bfloat16)
    X = torch.randn((nv, I), generator=g)
    Y = torch.empty((nv, O), dtype=torch.float32, device=dev)
    Ys = torch.empty((nv, O), dtype=torch.float32, device=dev) if silu else None
    say(f"gemv O={O} I={I} nv={nv} silu={silu}")
    L.dit_debug_gemv(W.to(dev), X.to(dev), Y, Ys)
    torch.cuda.synchronize()
    w, x = host(W), X.double().numpy()
    ref = x @ w.T
    bound = ACC * (np.abs(x) @ np.abs(w).T)
    err = np.abs(Y.cpu().double().numpy() - ref)
    assert np.all(err <= bound), float((err / np.maximum(bound, 1e-30)).max())
    if silu:
        sref = ref / (1.0 + np.exp(-ref))
        serr = np.abs(Ys.cpu().double().numpy() - sref)
        assert np.all(serr <= 1.1 * bound + 2e-6 * np.abs(sref) + 1e-7), float(serr.max())


@pytest.mark.parametrize("n", [4096, 700, 1])
def test_img_in_is_fp32_exact(dev, n):
    """img_in (fp32 latents, bf16 weights) through three bf16 MFMAs per block
    on an exact three-way split of each latent: every output within fp32
    accumulation error of the fp64 product."""
    H = 4096
    g = torch.Generator().manual_seed(n)
    x = torch.randn((n, 64), generator=g) * 2.0
    W = (torch.randn((H, 64), generator=g) / 8.0).to(torch.bfloat16)
    say(f"img_in n={n}")
    c = L.make_config(hidden=H, n_heads=32, head_dim=128, ffn=16384, n_layers=1)
    wd = {k: torch.zeros(8, dtype=torch.bfloat16, device=dev) for k in ("t1", "t2", "mod", "so", "proj_out")}
    wd["img_in"] = W.to(dev)
    for k in ("qkv", "q_norm", "k_norm", "o", "gate", "up", "down"):
        wd[k] = [torch.zeros(8, dtype=torch.bfloat16, device=dev)]
    m = L.dit_load_weights(c, wd)
    out = torch.full((n, H), float("nan"), device=dev)
    try:
        L.dit_img_in(m, x.to(dev).contiguous(), out)
        torch.cuda.synchronize()
    finally:
        L.dit_free(m)
    xx, w = x.double().numpy(), host(W)
    ref = xx @ w.T
    bound = ACC * (np.abs(xx) @ np.abs(w).T)
    err = np.abs(out.cpu().double().numpy() - ref)
    assert np.all(err <= bound), float((err / bound).max())


@pytest.mark.parametrize("M,N,K,n_pre,splits", split_cases([(700, 512, 512, 300), (256, 256, 64, 0),
                                                            (37, 768, 1024, 37), (256, 512, 16384, 100)]))
def test_residual_epilogue(dev, M, N, K, n_pre, splits):
    """h += g * (A Bᵀ), with g = gate_0 on rows < n_pre and gate_t after:
    the O and down projections' gated residual update, in fp32."""
    A, (B,) = operands(M, N, K, seed=5 * M + K)
    g = torch.Generator().manual_seed(M)
    h0 = torch.randn((M, N), generator=g)
    gt = torch.tanh(torch.randn(N, generator=g))
    g0 = torch.tanh(torch.randn(N, generator=g))
    h = h0.to(dev)
    say(f"residual epilogue M={M} N={N} K={K} n_pre={n_pre} splits={splits}")
    L.dit_debug_gemm("resid", M, N, K, A.to(dev), B.to(dev), h=h, gate_t=gt.to(dev),
                     gate_0=g0.to(dev), n_pre=n_pre, splits=splits, scratch=scratch_for(splits, N, dev))
    torch.cuda.synchronize()
    a, b = host(A), host(B)
    y = a @ b.T
    gate = np.where(np.arange(M)[:, None] < n_pre, g0.double().numpy()[None], gt.double().numpy()[None])
    ref = h0.double().numpy() + gate * y
    bound = (np.abs(gate) * ACC * (np.abs(a) @ np.abs(b).T) + 1e-5 * np.abs(gate * y)
             + 2.0 ** -23 * np.abs(ref))
    err = np.abs(h.cpu().double().numpy() - ref)
    assert np.all(err <= bound), (err / np.maximum(bound, 1e-30)).max()


@pytest.mark.parametrize("M,F,K,splits", split_cases([(700, 256, 512), (256, 512, 64), (37, 384, 1024),
                                                      (4096, 4096, 128)]) + [(2500, 16384, 128, 0)])
def test_swiglu_epilogue(dev, M, F, K, splits):
    """SiLU(A Gᵀ) * (A Uᵀ) with gate and up weights interleaved by the
    kernel's loader: the SwiGLU MLP's first GEMM. 4096 x 4096 x 128 (512
    tiles) and 2500 x 16384 x 128 (1280 tiles: ragged last row block, a last
    tile-row group two rows high) are whole rounds with an even number of K
    stages, which take the persistent grid (one workgroup per CU walking two
    or five tiles)."""
    A, (G, U) = operands(M, F, K, seed=7 * M + F, n_b=2)
    C = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
    say(f"swiglu epilogue M={M} F={F} K={K} splits={splits}")
    L.dit_debug_gemm("swiglu", M, F, K, A.to(dev), G.to(dev), C, B2=U.to(dev), splits=splits,
                     scratch=scratch_for(splits, 2 * F, dev))
    torch.cuda.synchronize()
    a, gw, uw = host(A), host(G), host(U)
    gv, uv = a @ gw.T, a @ uw.T
    sig = 1.0 / (1.0 + np.exp(-gv))
    ref = gv * sig * uv
    dg = ACC * (np.abs(a) @ np.abs(gw).T)
    du = ACC * (np.abs(a) @ np.abs(uw).T)
    # |d silu / dg| <= 1.1; the kernel's exp carries a few fp32 ulps
    bound = 1.1 * np.abs(uv) * dg + np.abs(gv * sig) * du + 1e-6 * np.abs(ref)
    check_bf16(host(C.cpu()), ref, bound, "SwiGLU")


def qkv_case(dev, M, nh, K, q_row0, S, splits, seed):
    H = nh * 128
    N = 3 * H
    A, (B,) = operands(M, N, K, seed=seed)
    g = torch.Generator().manual_seed(seed + 1)
    wq = (torch.randn(128, generator=g) / np.sqrt(128)).to(torch.bfloat16)
    wk = (torch.randn(128, generator=g) / np.sqrt(128)).to(torch.bfloat16)
    # RoPE tables of a real layout (512 text + 64 x 64 image, the first S rows)
    c = L.make_config(hidden=256, n_heads=2, head_dim=128, ffn=512, n_layers=1)
    lay = L.dit_build_layout(c, [("text", 512), ("target", 64, 64)])
    cos, sin = lay["rope_cos"][:S].copy(), lay["rope_sin"][:S].copy()
    cap = L.dit_kv_capacity(S)
    sentinel = 0x7E7E
    cache = torch.full((2 * nh * cap * 128,), sentinel, dtype=torch.int16, device=dev)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    eps = 1e-6
    L.dit_debug_gemm("qkv", M, N, K, A.to(dev), B.to(dev), C, q_norm=wq.to(dev), k_norm=wk.to(dev),
                     rope_cos=torch.from_numpy(cos).to(dev), rope_sin=torch.from_numpy(sin).to(dev),
                     kv_cache=cache, n_heads=nh, S=S, q_row0=q_row0, eps=eps, splits=splits,
                     scratch=scratch_for(splits, N, dev))
    torch.cuda.synchronize()
    a, b = host(A), host(B)
    y = a @ b.T
    acc_bound = ACC * (np.abs(a) @ np.abs(b).T)
    yb = bf16_np(y)          # the epilogue rounds the accumulators to bf16 first
    rows = np.arange(q_row0, q_row0 + M)
    cs, sn = cos[rows].astype(np.float64), sin[rows].astype(np.float64)
    kc, vt = cache_views(cache.cpu(), 1, nh, cap)
    out = {}
    for sec, w in ((0, wq), (1, wk)):
        x = yb[:, sec * H:(sec + 1) * H].reshape(M, nh, 128)
        xb = acc_bound[:, sec * H:(sec + 1) * H].reshape(M, nh, 128)
        r = 1.0 / np.sqrt(np.mean(x * x, axis=2, keepdims=True) + eps)
        xn = x * r * (1.0 + w.double().numpy())
        x0, x1 = xn[..., 0::2], xn[..., 1::2]
        ref = np.empty_like(xn)
        ref[..., 0::2] = x0 * cs[:, None] - x1 * sn[:, None]
        ref[..., 1::2] = x0 * sn[:, None] + x1 * cs[:, None]
        # An input whose fp32 accumulation lies on the other side of a bf16
        # rounding boundary than the fp64 value rounds to the neighbour, one
        # ulp away; that is possible only where the boundary (half an ulp
        # from the rounded value) is within the accumulation bound. Such an
        # input enters both outputs of its RoPE pair.
        yv = y[:, sec * H:(sec + 1) * H].reshape(M, nh, 128)
        near = ulp_bf16(x) / 2 - np.abs(yv - x) <= xb
        fl = np.where(near, ulp_bf16(x), 0.0) * r * np.abs(1.0 + w.double().numpy())
        f0, f1 = fl[..., 0::2], fl[..., 1::2]
        pair = np.empty_like(xn)
        pair[..., 0::2] = f0 * np.abs(cs[:, None]) + f1 * np.abs(sn[:, None])
        pair[..., 1::2] = f0 * np.abs(sn[:, None]) + f1 * np.abs(cs[:, None])
        # fp32 arithmetic of the norm and rotation, and the small change of
        # a row's RMS when one of its inputs flips
        bound = pair + 3e-4 * np.abs(ref) + 1e-6 * np.abs(xn).max(axis=2, keepdims=True)
        if sec == 0:
            got = host(C.cpu())[:, :H].reshape(M, nh, 128)
        else:
            got = i16_to_f32(kc[0, :, q_row0:q_row0 + M]).transpose(1, 0, 2).astype(np.float64)
        out[sec] = (got, ref, bound)
    check_bf16(out[0][0], out[0][1], out[0][2], "q")
    check_bf16(out[1][0], out[1][1], out[1][2], "k cache rows")
    vgot = i16_to_f32(vt[0, :, :, q_row0:q_row0 + M]).transpose(2, 0, 1).astype(np.float64)
    vref = y[:, 2 * H:].reshape(M, nh, 128)
    check_bf16(vgot, vref, acc_bound[:, 2 * H:].reshape(M, nh, 128), "v cache columns")
    # every other cache row / column still holds the sentinel
    kc16, vt16 = kc[0].numpy(), vt[0].numpy()
    keep = np.ones(cap, bool)
    keep[q_row0:q_row0 + M] = False
    assert np.all(kc16[:, keep] == sentinel) and np.all(vt16[:, :, keep] == sentinel)


@pytest.mark.parametrize("splits", [0, 2, 4])
@pytest.mark.parametrize("M,nh,K,q_row0,S", [(700, 2, 512, 512, 1300), (37, 2, 1024, 0, 37),
                                             (256, 4, 256, 256, 600)])
def test_qkv_epilogue(dev, M, nh, K, q_row0, S, splits):
    """The QKV projection with its fused per-head QK-RMSNorm (1 + w), 3D RoPE
    of each row's token, q written back and k / transposed v written to the
    cache rows of tokens q_row0.. (the split path sends its last row block
    through the reduction and the standalone norm / RoPE / cache kernel);
    cache rows of other tokens are untouched."""
    say(f"qkv epilogue M={M} nh={nh} K={K} rows {q_row0}.. of S={S} splits={splits}")
    qkv_case(dev, M, nh, K, q_row0, S, splits, seed=M + 17 * nh + K)


@pytest.mark.parametrize("epi", ["qkv", "swiglu", "resid_o", "resid_down"])
def test_full_size_step_gemms_sampled(dev, epi):
    """The step's four GEMMs at full width (4096 target rows, hidden 4096,
    32 heads, ffn 16384) through their epilogues; 64 sampled rows against
    fp64 (QKV: every column of those rows, and their cache rows)."""
    M, H, F = 4096, 4096, 16384
    rows = np.sort(np.random.default_rng(1).choice(M, 64, replace=False))
    say(f"full-size {epi} GEMM, {len(rows)} sampled rows")
    if epi == "qkv":
        nh, q_row0, S = 32, 256, 4352
        N, K = 3 * H, H
        A, (B,) = operands(M, N, K, seed=11)
        g = torch.Generator().manual_seed(12)
        wq = (torch.randn(128, generator=g) / np.sqrt(128)).to(torch.bfloat16)
        wk = (torch.randn(128, generator=g) / np.sqrt(128)).to(torch.bfloat16)
        c = L.make_config(hidden=256, n_heads=2, head_dim=128, ffn=512, n_layers=1)
        lay = L.dit_build_layout(c, [("text", 256), ("target", 64, 64)])
        cap = L.dit_kv_capacity(S)
        cache = torch.zeros((2 * nh * cap * 128,), dtype=torch.int16, device=dev)
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        L.dit_debug_gemm("qkv", M, N, K, A.to(dev), B.to(dev), C, q_norm=wq.to(dev), k_norm=wk.to(dev),
                         rope_cos=torch.from_numpy(lay["rope_cos"]).to(dev),
                         rope_sin=torch.from_numpy(lay["rope_sin"]).to(dev), kv_cache=cache,
                         n_heads=nh, S=S, q_row0=q_row0, eps=1e-6,
                         scratch=torch.empty(1 << 24, dtype=torch.float32, device=dev))
        torch.cuda.synchronize()
        a, b = host(A)[rows], host(B)
        y = a @ b.T
        yb = bf16_np(y)
        cs = lay["rope_cos"][q_row0 + rows].astype(np.float64)
        sn = lay["rope_sin"][q_row0 + rows].astype(np.float64)
        kc, vt = cache_views(cache.cpu(), 1, nh, cap)
        for sec, w in ((0, wq), (1, wk)):
            x = yb[:, sec * H:(sec + 1) * H].reshape(len(rows), nh, 128)
            r = 1.0 / np.sqrt(np.mean(x * x, axis=2, keepdims=True) + 1e-6)
            xn = x * r * (1.0 + w.double().numpy())
            ref = np.empty_like(xn)
            ref[..., 0::2] = xn[..., 0::2] * cs[:, None] - xn[..., 1::2] * sn[:, None]
            ref[..., 1::2] = xn[..., 0::2] * sn[:, None] + xn[..., 1::2] * cs[:, None]
            if sec == 0:
                got = host(C.cpu())[rows, :H].reshape(len(rows), nh, 128)
            else:
                got = i16_to_f32(kc[0][:, q_row0 + rows]).transpose(1, 0, 2).astype(np.float64)
            err = np.abs(got - ref)
            # one ulp of rounding plus an input rounding flip (one ulp of x)
            assert np.all(err <= 2 * ulp_bf16(ref) + 2 * ulp_bf16(np.abs(xn).max(axis=2, keepdims=True)))
            exact = float(np.mean(got == bf16_np(ref)))
            say(f"  {'q' if sec == 0 else 'k'}: {exact * 100:.3f}% equal to the rounded fp64 value")
            assert exact >= 0.995
        vgot = i16_to_f32(vt[0][:, :, q_row0 + rows]).transpose(2, 0, 1).astype(np.float64)
        check_bf16(vgot, y[:, 2 * H:].reshape(len(rows), nh, 128),
                   ACC * (np.abs(a) @ np.abs(b[2 * H:]).T).reshape(len(rows), nh, 128), "v")
        return
    if epi == "swiglu":
        A, (G, U) = operands(M, F, H, seed=13, n_b=2)
        C = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
        L.dit_debug_gemm("swiglu", M, F, H, A.to(dev), G.to(dev), C, B2=U.to(dev))
        torch.cuda.synchronize()
        a, gw, uw = host(A)[rows], host(G), host(U)
        gv, uv = a @ gw.T, a @ uw.T
        sig = 1.0 / (1.0 + np.exp(-gv))
        ref = gv * sig * uv
        bound = (1.1 * np.abs(uv) * ACC * (np.abs(a) @ np.abs(gw).T)
                 + np.abs(gv * sig) * ACC * (np.abs(a) @ np.abs(uw).T) + 1e-6 * np.abs(ref))
        check_bf16(host(C.cpu())[rows], ref, bound, "SwiGLU")
        return
    K = H if epi == "resid_o" else F
    A, (B,) = operands(M, H, K, seed=14 if epi == "resid_o" else 15)
    g = torch.Generator().manual_seed(16)
    h0 = torch.randn((M, H), generator=g)
    gt = torch.tanh(torch.randn(H, generator=g))
    h = h0.to(dev)
    L.dit_debug_gemm("resid", M, H, K, A.to(dev), B.to(dev), h=h, gate_t=gt.to(dev), gate_0=gt.to(dev),
                     n_pre=0, scratch=torch.empty(1 << 24, dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
    a, b = host(A)[rows], host(B)
    y = a @ b.T
    gg = gt.double().numpy()[None]
    ref = h0.double().numpy()[rows] + gg * y
    bound = (np.abs(gg) * ACC * (np.abs(a) @ np.abs(b).T) + 1e-5 * np.abs(gg * y) + 2.0 ** -23 * np.abs(ref))
    err = np.abs(h.cpu().double().numpy()[rows] - ref)
    assert np.all(err <= bound), (err / bound).max()
