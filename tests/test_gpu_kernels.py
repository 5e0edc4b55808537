"""GPU unit parity of individual kernels through the C ABI: the MFMA GEMM,
the attention kernel's mask and arithmetic, against the fp64 oracle or
exact integer arithmetic."""
import numpy as np
import pytest
import torch

import oracle as O
from diffusion_transformer_amd import synth
from gpu_common import cache_views, rel_err, say, seq_len, split_cases

pytestmark = pytest.mark.gpu

L = pytest.importorskip("diffusion_transformer_amd._lib")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.mark.parametrize("M,N,K,splits", split_cases([(32, 256, 64), (300, 512, 128), (257, 768, 256),
                                                      (600, 1024, 512)]))
def test_gemm_exact_small_integers(dev, M, N, K, splits):
    """Entries in {-1, 0, 1}: every partial sum is an integer of magnitude
    <= K <= 512, exact in fp32 and in the bf16 output, so the MFMA GEMM must
    match integer matrix multiplication bit for bit (checks the MFMA lane
    layout, the LDS swizzle, the tile order, the ragged M tail and, with
    ``splits``, the split-K partial sums and their reduction)."""
    say(f"gemm exact M={M} N={N} K={K} splits={splits}")
    g = torch.Generator().manual_seed(M * 7 + N + K)
    A = torch.randint(-1, 2, (M, K), generator=g).to(torch.float32)
    B = torch.randint(-1, 2, (N, K), generator=g).to(torch.float32)
    want = (A.to(torch.int64) @ B.to(torch.int64).T).to(torch.float32)
    Ad, Bd = A.to(dev, torch.bfloat16), B.to(dev, torch.bfloat16)
    Cd = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    scratch = torch.empty(4 * 256 * N, dtype=torch.float32, device=dev) if splits else None
    L.dit_debug_gemm("bf16", M, N, K, Ad, Bd, Cd, splits=splits, scratch=scratch)
    torch.cuda.synchronize()
    assert torch.equal(Cd.float().cpu(), want)


@pytest.mark.parametrize("M,N,K", [(512, 512, 16384), (4096, 4096, 16384)])
def test_long_k_gemm_exact_small_integers(dev, M, N, K):
    """The down projection's K (16384, 256 K stages): with entries in
    {-1, 0, 1} every partial sum is an integer below 2^24, exact in fp32, so
    the output is the integer product rounded once to bf16 (round to nearest
    even), bit for bit; at 4096 x 4096 a sample of rows is checked."""
    say(f"long-K gemm exact M={M} N={N} K={K}")
    g = torch.Generator().manual_seed(M + N + K)
    A = torch.randint(-1, 2, (M, K), generator=g).to(torch.float32)
    B = torch.randint(-1, 2, (N, K), generator=g).to(torch.float32)
    Ad, Bd = A.to(dev, torch.bfloat16), B.to(dev, torch.bfloat16)
    Cd = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    L.dit_debug_gemm("bf16", M, N, K, Ad, Bd, Cd)
    torch.cuda.synchronize()
    rows = torch.arange(M) if M <= 1024 else torch.from_numpy(
        np.sort(np.random.default_rng(3).choice(M, 96, replace=False)))
    want = (A[rows].to(torch.int64) @ B.to(torch.int64).T).to(torch.float32).to(torch.bfloat16)
    assert torch.equal(Cd.cpu()[rows].view(torch.int16), want.view(torch.int16))


def test_gemm_random_full_shape_sampled(dev):
    """QKV-shaped GEMM (4096 x 12288 x 4096) with N(0,1) bf16 inputs; sampled
    outputs against fp64 dot products of the same bf16 values."""
    M, N, K = 4096, 12288, 4096
    say(f"gemm random M={M} N={N} K={K}")
    g = torch.Generator(device=dev).manual_seed(5)
    A = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
    B = torch.randn((N, K), generator=g, device=dev).to(torch.bfloat16)
    Cd = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    L.dit_debug_gemm("bf16", M, N, K, A, B, Cd)
    torch.cuda.synchronize()
    rs = np.random.default_rng(0)
    rows = rs.choice(M, 64, replace=False)
    cols = rs.choice(N, 64, replace=False)
    Ah = A[rows].float().cpu().numpy().astype(np.float64)
    Bh = B[cols].float().cpu().numpy().astype(np.float64)
    ref = Ah @ Bh.T
    got = Cd[rows][:, cols].float().cpu().numpy()
    # bf16 output rounding (2^-9 relative) dominates
    assert np.abs(got - ref).max() <= 4e-3 * np.abs(ref).max() + 1e-2


LAYOUTS = {
    "c0w": [("text", 2), ("ref", 2, 2), ("text", 1), ("target", 2, 2)],
    "c1": synth.CONFIGS["c1"]["segments"],
    "c3": synth.CONFIGS["c3"]["segments"],
    **synth.RAGGED_LAYOUTS,
    "c4": synth.CONFIGS["c4"]["segments"],
    "c5": synth.CONFIGS["c5"]["segments"],
}


def layout_for(segments):
    c = L.make_config(hidden=256, n_heads=2, head_dim=128, ffn=512, n_layers=1)
    return L.dit_build_layout(c, segments)


@pytest.mark.parametrize("name", ["c0w", "c1", "c3", "ragged", "many_ragged", "c4", "c5"])
def test_attention_mask_bit_exact(dev, name):
    segs = LAYOUTS[name]
    lay = layout_for(segs)
    S = lay["P"] + lay["T"]
    say(f"mask {name} S={S}")
    lim = torch.from_numpy(lay["row_limit"]).to(dev)
    seq = L.make_seq(lay["P"], lay["T"], lim, lim, lim)
    mask = torch.full((S * S,), 7, dtype=torch.uint8, device=dev)
    L.dit_debug_mask(seq, mask)
    torch.cuda.synchronize()
    got = mask.view(S, S)
    ids = O.build_layout(segs).image_ids
    for r0 in range(0, S, 2048):
        rows = np.arange(r0, min(S, r0 + 2048))
        want = torch.from_numpy(O.block_causal_mask(ids, rows=rows).astype(np.uint8))
        assert torch.equal(got[r0:r0 + len(rows)].cpu(), want), f"rows {r0}.."


def fill_cache(dev, S, nh, seed):
    """Random K and V in the library's cache layout (layer 0 only); returns
    the cache and the bf16-exact float64 K, V [S, nh, 128] it holds."""
    cap = L.dit_kv_capacity(S)
    g = torch.Generator().manual_seed(seed)
    K = torch.randn((S, nh, 128), generator=g).to(torch.bfloat16)
    V = torch.randn((S, nh, 128), generator=g).to(torch.bfloat16)
    cache = torch.zeros(2 * nh * cap * 128, dtype=torch.int16)
    kv, vt = cache_views(cache, 1, nh, cap)
    kv[0, :, :S, :] = K.transpose(0, 1).view(torch.int16)
    vt[0, :, :, :S] = V.permute(1, 2, 0).view(torch.int16)
    return cache.to(dev), K.double().numpy(), V.double().numpy()


ATTN_VARIANTS = [0, 1, 2, 3, 4, 5, 6]


def variant_applies(variant, mode, S):
    """Variants 5 and 6 (the pipelined kernel of cached steps) take the
    target rows of a cached step with S a multiple of 64 only."""
    return variant < 5 or (mode == "cached" and S % 64 == 0)


def attn_scratch(dev):
    """Caller-owned key-split scratch of the attention test hook (64 MiB,
    the size the step lends it)."""
    return torch.empty(1 << 24, dtype=torch.float32, device=dev)


ATTN_CASES = [(name, mode, v)
              for name, mode in [("c0w", "extract"), ("c0w", "cached"), ("ragged", "extract"),
                                 ("ragged", "cached"), ("many_ragged", "extract"),
                                 ("many_ragged", "cached"), ("c1", "extract"), ("c1", "cached"),
                                 ("c3", "cached")]
              for v in ATTN_VARIANTS if variant_applies(v, mode, seq_len(LAYOUTS[name]))]


@pytest.mark.parametrize("name,mode,variant", ATTN_CASES)
def test_attention_matches_oracle(dev, name, mode, variant):
    nh = 2
    lay = layout_for(LAYOUTS[name])
    P, T = lay["P"], lay["T"]
    S = P + T
    assert S == seq_len(LAYOUTS[name]) and variant_applies(variant, mode, S)
    say(f"attention {name} {mode} S={S} variant={variant}")
    cache, K, V = fill_cache(dev, S, nh, seed=S)
    q_off, N = (0, S) if mode == "extract" else (P, T)
    g = torch.Generator().manual_seed(11)
    Q = torch.randn((N, nh, 128), generator=g).to(torch.bfloat16)
    lim = torch.from_numpy(lay["row_limit"]).to(dev)
    seq = L.make_seq(P, T, lim, lim, lim)
    out = torch.empty((N, nh * 128), dtype=torch.bfloat16, device=dev)
    Qd = Q.reshape(N, nh * 128).contiguous().to(dev)
    L.dit_debug_attention(seq, nh, Qd, nh * 128, q_off, N, cache, out, variant, attn_scratch(dev))
    torch.cuda.synchronize()
    ids = O.build_layout(LAYOUTS[name]).image_ids
    allowed = O.block_causal_mask(ids, rows=np.arange(q_off, q_off + N))
    ref = O.masked_attention(Q.double().numpy(), K, V, allowed)
    err = rel_err(out.float().cpu().numpy(), ref)
    say(f"  rel err {err:.3e}")
    assert err < 1e-2


@pytest.mark.parametrize("name", ["many_ragged", "c1", "c3"])
def test_attention_launch_choices_are_bitwise_neutral(dev, name):
    """The step's launcher only reorders work: in extract mode it deals query
    blocks last first (same output, bit for bit, as the unordered kernel), and
    in cached mode its key split of the last round is the forced-split
    variant's, bit for bit. With 2 heads every layout here runs the 4-wave
    kernel (variants 2 and 4)."""
    nh = 2
    lay = layout_for(LAYOUTS[name])
    P, T = lay["P"], lay["T"]
    S = P + T
    say(f"launcher order / split {name} S={S}")
    cache, _, _ = fill_cache(dev, S, nh, seed=S + 7)
    lim = torch.from_numpy(lay["row_limit"]).to(dev)
    seq = L.make_seq(P, T, lim, lim, lim)
    g = torch.Generator().manual_seed(13)
    scratch = attn_scratch(dev)
    for mode, other in (("extract", 2), ("cached", 4)):
        q_off, N = (0, S) if mode == "extract" else (P, T)
        Qd = torch.randn((N, nh * 128), generator=g).to(torch.bfloat16).to(dev)
        outs = []
        for variant in (0, other):
            out = torch.full((N, nh * 128), float("nan"), dtype=torch.bfloat16, device=dev)
            L.dit_debug_attention(seq, nh, Qd, nh * 128, q_off, N, cache, out, variant, scratch)
            outs.append(out)
        torch.cuda.synchronize()
        assert not torch.isnan(outs[0].float()).any(), mode
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), mode


def random_layout(seed):
    """Seeded random token layout: 1-10 text runs / reference images of
    mixed sizes in random order, then a target image (about 300-2500 tokens)."""
    r = np.random.default_rng(1000 + seed)
    segs = []
    for _ in range(int(r.integers(1, 11))):
        if r.random() < 0.4:
            segs.append(("text", int(r.integers(1, 80))))
        else:
            segs.append(("ref", int(r.integers(1, 24)), int(r.integers(1, 24))))
    segs.append(("target", int(r.integers(4, 30)), int(r.integers(4, 30))))
    return segs


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_attention_random_layouts(dev, seed):
    """Random layouts: the materialized mask is the oracle's rule bit for
    bit, and every attention variant matches the oracle in extract and
    cached mode."""
    nh = 2
    segs = random_layout(seed)
    lay = layout_for(segs)
    P, T = lay["P"], lay["T"]
    S = P + T
    say(f"random layout {seed}: {len(segs)} segments, P={P} T={T}")
    lim = torch.from_numpy(lay["row_limit"]).to(dev)
    seq = L.make_seq(P, T, lim, lim, lim)
    mask = torch.full((S * S,), 7, dtype=torch.uint8, device=dev)
    L.dit_debug_mask(seq, mask)
    torch.cuda.synchronize()
    ids = O.build_layout(segs).image_ids
    want = torch.from_numpy(O.block_causal_mask(ids).astype(np.uint8))
    assert torch.equal(mask.view(S, S).cpu(), want)
    cache, K, V = fill_cache(dev, S, nh, seed=S + seed)
    g = torch.Generator().manual_seed(seed)
    for mode in ("extract", "cached"):
        q_off, N = (0, S) if mode == "extract" else (P, T)
        Q = torch.randn((N, nh, 128), generator=g).to(torch.bfloat16)
        Qd = Q.reshape(N, nh * 128).contiguous().to(dev)
        allowed = O.block_causal_mask(ids, rows=np.arange(q_off, q_off + N))
        ref = O.masked_attention(Q.double().numpy(), K, V, allowed)
        for variant in ATTN_VARIANTS:
            if not variant_applies(variant, mode, S):
                continue
            out = torch.empty((N, nh * 128), dtype=torch.bfloat16, device=dev)
            L.dit_debug_attention(seq, nh, Qd, nh * 128, q_off, N, cache, out, variant,
                                  attn_scratch(dev))
            torch.cuda.synchronize()
            err = rel_err(out.float().cpu().numpy(), ref)
            assert err < 1e-2, (mode, variant, err)


@pytest.mark.parametrize("C", [64, 5])
def test_latent_standardize_matches_oracle(dev, C):
    """Per-channel standardize / unstandardize (pages 1A and 6B) on a ragged
    row count, against the oracle in fp64; C = 5 takes the scalar path."""
    rows = 4099
    say(f"latent standardize rows={rows} C={C}")
    mean, std = synth.latent_stats(C)
    z = (2.0 * np.random.default_rng(C).standard_normal((rows, C)) + 1.0).astype(np.float32)
    md, sd = torch.from_numpy(mean).to(dev), torch.from_numpy(std).to(dev)
    zd = torch.from_numpy(z).to(dev)
    L.dit_latent_standardize(zd, md, sd)
    torch.cuda.synchronize()
    ref = O.standardize(z, mean, std)
    assert rel_err(zd.cpu().numpy(), ref) < 1e-6
    L.dit_latent_standardize(zd, md, sd, inverse=True)
    torch.cuda.synchronize()
    assert rel_err(zd.cpu().numpy(), O.unstandardize(ref, mean, std)) < 1e-6


def rising_qk(kind, S, N, nh, seed):
    """Queries and keys whose scores drive the softmax's running max.
    "rising": every key is c*j*u + noise and every query 10*u + noise (u a
    unit direction per head), so scores climb about ten log2 units per 64-key
    tile and the running max must be raised on most tiles; "creeping": half
    that slope, so between raises the unnormalized weights reach up to 2^8;
    "q8" / "q32": N(0,1) keys with queries scaled 8x / 32x (peaked, random)."""
    g = np.random.default_rng(seed)
    u = g.standard_normal((nh, 128))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    if kind in ("rising", "creeping"):
        c = 0.12 if kind == "rising" else 0.06
        K = c * np.arange(S)[:, None, None] * u[None] + g.standard_normal((S, nh, 128))
        Q = 10.0 * u[None] + g.standard_normal((N, nh, 128))
    else:
        K = g.standard_normal((S, nh, 128))
        Q = (8.0 if kind == "q8" else 32.0) * g.standard_normal((N, nh, 128))
    return Q, K, g.standard_normal((S, nh, 128))


def running_max_events(Q, K, allowed, tile=64, jump=8.0):
    """Host-side count, in the kernel's exp2 domain (score * log2(e)/sqrt(d))
    and its key-tile order, of the tiles whose max exceeds the query's
    running max by more than ``jump`` (the kernel must raise its max and
    rescale O and l) and of those that exceed it by at most ``jump`` (the
    kernel keeps its max and the weights exceed 1)."""
    scale = np.log2(np.e) / np.sqrt(Q.shape[2])
    n_raise = n_over1 = 0
    for h in range(Q.shape[1]):
        s = (Q[:, h] @ K[:, h].T) * scale
        s = np.where(allowed, s, -np.inf)
        m = np.full(s.shape[0], -np.inf)
        for t0 in range(0, s.shape[1], tile):
            tm = s[:, t0:t0 + tile].max(axis=1)
            seen = np.isfinite(m) & np.isfinite(tm)
            n_raise += int((seen & (tm > m + jump)).sum())
            n_over1 += int((seen & (tm > m) & (tm <= m + jump)).sum())
            m = np.maximum(m, tm)
    return n_raise, n_over1


@pytest.mark.parametrize("kind", ["rising", "creeping", "q8", "q32"])
@pytest.mark.parametrize("name,mode", [("c1", "extract"), ("c1", "cached"),
                                       ("many_ragged", "extract"), ("many_ragged", "cached")])
def test_attention_running_max_raised_mid_stream(dev, name, mode, kind):
    """Scores that rise along the key sequence or are strongly peaked: the
    kernel's lazy running max is raised in the middle of the key stream (O and
    l rescaled) on many tiles, and on others the unnormalized weights exceed 1
    -- both counted on the host from the same inputs -- and every variant
    (split ones included) still matches the fp64 oracle."""
    nh = 2
    lay = layout_for(LAYOUTS[name])
    P, T = lay["P"], lay["T"]
    S = P + T
    q_off, N = (0, S) if mode == "extract" else (P, T)
    Q, K, V = rising_qk(kind, S, N, nh, seed=S + len(kind))
    Qb = torch.from_numpy(Q).to(torch.bfloat16)
    Kb = torch.from_numpy(K).to(torch.bfloat16)
    Vb = torch.from_numpy(V).to(torch.bfloat16)
    cap = L.dit_kv_capacity(S)
    cache = torch.zeros(2 * nh * cap * 128, dtype=torch.int16)
    kv, vt = cache_views(cache, 1, nh, cap)
    kv[0, :, :S, :] = Kb.transpose(0, 1).view(torch.int16)
    vt[0, :, :, :S] = Vb.permute(1, 2, 0).view(torch.int16)
    cache = cache.to(dev)
    ids = O.build_layout(LAYOUTS[name]).image_ids
    allowed = O.block_causal_mask(ids, rows=np.arange(q_off, q_off + N))
    Qh, Kh, Vh = Qb.double().numpy(), Kb.double().numpy(), Vb.double().numpy()
    n_raise, n_over1 = running_max_events(Qh, Kh, allowed)
    say(f"running max {kind} {name} {mode}: {n_raise} raises, {n_over1} tiles with weights > 1")
    if kind != "q32":
        assert n_over1 > 0
    assert n_raise > (N * nh if kind == "rising" else 0)
    ref = O.masked_attention(Qh, Kh, Vh, allowed)
    lim = torch.from_numpy(lay["row_limit"]).to(dev)
    seq = L.make_seq(P, T, lim, lim, lim)
    Qd = Qb.reshape(N, nh * 128).contiguous().to(dev)
    scratch = attn_scratch(dev)
    for variant in ATTN_VARIANTS:
        if not variant_applies(variant, mode, S):
            continue
        out = torch.empty((N, nh * 128), dtype=torch.bfloat16, device=dev)
        L.dit_debug_attention(seq, nh, Qd, nh * 128, q_off, N, cache, out, variant, scratch)
        torch.cuda.synchronize()
        err = rel_err(out.float().cpu().numpy(), ref)
        assert err < 1e-2, (variant, err)
    say(f"  last variant rel err {err:.2e}")


def cache_from(dev, K, V):
    """Layer-0 cache holding the bf16 roundings of K, V [S, nh, 128]."""
    S, nh = K.shape[0], K.shape[1]
    cap = L.dit_kv_capacity(S)
    cache = torch.zeros(2 * nh * cap * 128, dtype=torch.int16)
    kv, vt = cache_views(cache, 1, nh, cap)
    kv[0, :, :S, :] = torch.from_numpy(K).to(torch.bfloat16).transpose(0, 1).view(torch.int16)
    vt[0, :, :, :S] = torch.from_numpy(V).to(torch.bfloat16).permute(1, 2, 0).view(torch.int16)
    return cache.to(dev)


@pytest.mark.parametrize("kind", ["randn3", "rising", "q32"])
@pytest.mark.parametrize("name", ["c1", "c3"])
def test_pipelined_attention_is_bitwise_the_staged_kernel(dev, name, kind):
    """The cached-step kernel that overlaps the softmax of tile t with the
    score MFMAs of tile t+1 and the P·V of tile t-1 performs the same
    arithmetic per query as the staged 8-wave kernel, raised running maxima
    included (rising / peaked scores): bit-identical output unsplit
    (variants 1 and 5) and with the last round split over key ranges
    (variants 3 and 6)."""
    nh = 2
    lay = layout_for(LAYOUTS[name])
    P, T = lay["P"], lay["T"]
    S = P + T
    if kind == "randn3":
        g = np.random.default_rng(S)
        Q = 3.0 * g.standard_normal((T, nh, 128))
        K, V = g.standard_normal((S, nh, 128)), g.standard_normal((S, nh, 128))
    else:
        Q, K, V = rising_qk(kind, S, T, nh, seed=S + 5)
    cache = cache_from(dev, K, V)
    lim = torch.from_numpy(lay["row_limit"]).to(dev)
    seq = L.make_seq(P, T, lim, lim, lim)
    Qd = torch.from_numpy(Q).to(torch.bfloat16).reshape(T, nh * 128).contiguous().to(dev)
    say(f"pipelined attention {name} {kind} S={S}")
    scratch = attn_scratch(dev)
    for a, b in ((1, 5), (3, 6)):
        outs = []
        for variant in (a, b):
            out = torch.full((T, nh * 128), float("nan"), dtype=torch.bfloat16, device=dev)
            L.dit_debug_attention(seq, nh, Qd, nh * 128, P, T, cache, out, variant, scratch)
            outs.append(out)
        torch.cuda.synchronize()
        assert not torch.isnan(outs[0].float()).any()
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), (a, b)


def test_cached_launcher_takes_the_pipelined_kernel(dev):
    """At 16 heads the c3 target rows make 256 workgroups of 256 queries, so
    the step's launcher runs the pipelined kernel with its last-round key
    split: bit-identical to variant 6, and sampled rows match the fp64
    oracle."""
    nh = 16
    lay = layout_for(LAYOUTS["c3"])
    P, T = lay["P"], lay["T"]
    S = P + T
    g = np.random.default_rng(S + 16)
    Q = 2.0 * g.standard_normal((T, nh, 128))
    K, V = g.standard_normal((S, nh, 128)), g.standard_normal((S, nh, 128))
    cache = cache_from(dev, K, V)
    lim = torch.from_numpy(lay["row_limit"]).to(dev)
    seq = L.make_seq(P, T, lim, lim, lim)
    Qb = torch.from_numpy(Q).to(torch.bfloat16)
    Qd = Qb.reshape(T, nh * 128).contiguous().to(dev)
    say(f"cached launcher, c3 at {nh} heads")
    scratch = attn_scratch(dev)
    outs = []
    for variant in (0, 6):
        out = torch.full((T, nh * 128), float("nan"), dtype=torch.bfloat16, device=dev)
        L.dit_debug_attention(seq, nh, Qd, nh * 128, P, T, cache, out, variant, scratch)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    rows = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(3).choice(T, 30, replace=False)]))
    ids = O.build_layout(LAYOUTS["c3"]).image_ids
    allowed = O.block_causal_mask(ids, rows=P + rows)
    Kb = torch.from_numpy(K).to(torch.bfloat16).double().numpy()
    Vb = torch.from_numpy(V).to(torch.bfloat16).double().numpy()
    ref = O.masked_attention(Qb[rows].double().numpy(), Kb, Vb, allowed)
    got = outs[0].float().cpu().numpy()[rows]
    assert rel_err(got, ref) < 1e-2
