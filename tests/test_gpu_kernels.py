"""GPU unit parity of individual kernels through the C ABI: the MFMA GEMM,
the attention kernel's mask and arithmetic, against the fp64 oracle or
exact integer arithmetic."""
import numpy as np
import pytest
import torch

import oracle as O
from diffusion_transformer_amd import synth
from gpu_common import cache_views, rel_err, say

pytestmark = pytest.mark.gpu

L = pytest.importorskip("diffusion_transformer_amd._lib")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("M,N,K", [(32, 256, 64), (300, 512, 128), (257, 768, 256), (600, 1024, 512)])
def test_gemm_exact_small_integers(dev, M, N, K, variant):
    """Entries in {-1, 0, 1}: every partial sum is an integer of magnitude
    <= K <= 256, exact in fp32 and in the bf16 output, so the MFMA GEMM must
    match integer matrix multiplication bit for bit (checks the MFMA lane
    layout, the LDS swizzle, the tile order and the ragged M tail)."""
    say(f"gemm exact M={M} N={N} K={K} variant={variant}")
    g = torch.Generator().manual_seed(M * 7 + N + K)
    A = torch.randint(-1, 2, (M, K), generator=g).to(torch.float32)
    B = torch.randint(-1, 2, (N, K), generator=g).to(torch.float32)
    want = (A.to(torch.int64) @ B.to(torch.int64).T).to(torch.float32)
    Ad, Bd = A.to(dev, torch.bfloat16), B.to(dev, torch.bfloat16)
    Cd = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    L.dit_debug_gemm(Ad, Bd, Cd, M, N, K, variant)
    torch.cuda.synchronize()
    assert torch.equal(Cd.float().cpu(), want)


def test_gemm_random_full_shape_sampled(dev):
    """QKV-shaped GEMM (4096 x 12288 x 4096) with N(0,1) bf16 inputs; sampled
    outputs against fp64 dot products of the same bf16 values."""
    M, N, K = 4096, 12288, 4096
    say(f"gemm random M={M} N={N} K={K}")
    g = torch.Generator(device=dev).manual_seed(5)
    A = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
    B = torch.randn((N, K), generator=g, device=dev).to(torch.bfloat16)
    Cd = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    L.dit_debug_gemm(A, B, Cd, M, N, K)
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


@pytest.mark.parametrize("variant", [0, 1, 3, 4, 5, 6, 7])
@pytest.mark.parametrize("name,mode", [("c0w", "extract"), ("c0w", "cached"),
                                       ("ragged", "extract"), ("ragged", "cached"),
                                       ("many_ragged", "extract"), ("many_ragged", "cached"),
                                       ("c1", "extract"), ("c1", "cached"),
                                       ("c3", "cached")])
def test_attention_matches_oracle(dev, name, mode, variant):
    nh = 2
    lay = layout_for(LAYOUTS[name])
    P, T = lay["P"], lay["T"]
    S = P + T
    say(f"attention {name} {mode} S={S} variant={variant}")
    cache, K, V = fill_cache(dev, S, nh, seed=S)
    q_off, N = (0, S) if mode == "extract" else (P, T)
    g = torch.Generator().manual_seed(11)
    Q = torch.randn((N, nh, 128), generator=g).to(torch.bfloat16)
    lim = torch.from_numpy(lay["row_limit"]).to(dev)
    seq = L.make_seq(P, T, lim, lim, lim)
    out = torch.empty((N, nh * 128), dtype=torch.bfloat16, device=dev)
    Qd = Q.reshape(N, nh * 128).contiguous().to(dev)
    L.dit_debug_attention(seq, nh, Qd, nh * 128, q_off, N, cache, out, variant)
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
    kernel (variants 5 and 7)."""
    nh = 2
    lay = layout_for(LAYOUTS[name])
    P, T = lay["P"], lay["T"]
    S = P + T
    say(f"launcher order / split {name} S={S}")
    cache, _, _ = fill_cache(dev, S, nh, seed=S + 7)
    lim = torch.from_numpy(lay["row_limit"]).to(dev)
    seq = L.make_seq(P, T, lim, lim, lim)
    g = torch.Generator().manual_seed(13)
    for mode, other in (("extract", 5), ("cached", 7)):
        q_off, N = (0, S) if mode == "extract" else (P, T)
        Qd = torch.randn((N, nh * 128), generator=g).to(torch.bfloat16).to(dev)
        outs = []
        for variant in (0, other):
            out = torch.full((N, nh * 128), float("nan"), dtype=torch.bfloat16, device=dev)
            L.dit_debug_attention(seq, nh, Qd, nh * 128, q_off, N, cache, out, variant)
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
        for variant in (0, 1, 3, 4, 5, 6, 7):
            out = torch.empty((N, nh * 128), dtype=torch.bfloat16, device=dev)
            L.dit_debug_attention(seq, nh, Qd, nh * 128, q_off, N, cache, out, variant)
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
