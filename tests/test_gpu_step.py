"""GPU parity of the whole step (extract, cached, Euler) through the C ABI
against the fp64 oracle on the same seeded inputs, plus the cache
invariants the pages state, checked on the GPU path itself."""
import os

import numpy as np
import pytest
import torch

import oracle as O
from diffusion_transformer_amd import synth
from gpu_common import cache_views, i16_to_f32, rel_err, say, synth_weights_on_device
from oracle_inputs import dims_of, oracle_prefix

pytestmark = pytest.mark.gpu

L = pytest.importorskip("diffusion_transformer_amd._lib")
from diffusion_transformer_amd.runtime import DitRuntime  # noqa: E402

TOL_BF16 = 2e-2          # v_θ and final latent vs the oracle (bf16 path)
TOL_CACHED = 1e-2        # GPU cached vs GPU full recompute


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def build(name, dev, n_layers=None, seed=21):
    cfg = synth.config(name)
    if n_layers is not None:
        cfg["n_layers"] = n_layers
    W = synth.make_weights(cfg, seed=seed, workers=16)
    I = synth.make_inputs(cfg, seed=seed)
    rt = DitRuntime(cfg, W, device=dev)
    seq = rt.sequence(cfg["segments"])
    pre = rt.prefix_hidden(I)
    x0 = torch.from_numpy(I["x0"]).to(dev)
    return cfg, W, I, rt, seq, pre, x0


@pytest.mark.parametrize("name", ["c0w", "c1"])
def test_loop_matches_oracle(dev, name):
    cfg, W, I, rt, seq, pre, x0 = build(name, dev)
    sig = cfg["sigmas"]
    say(f"loop {name} P={seq.P} T={seq.T} L={cfg['n_layers']}")
    vs_c, xs_c = rt.run_loop(seq, pre, x0, sig, use_cache=True)
    vs_r, xs_r = rt.run_loop(seq, pre, x0, sig, use_cache=False)
    torch.cuda.synchronize()
    dims = dims_of(cfg)
    lay = O.build_layout(cfg["segments"])
    ref = O.run_loop(W, dims, lay, oracle_prefix(cfg, W, I), I["x0"], sig, use_cache=True)
    for k, r in enumerate(ref):
        e_v = rel_err(vs_c[k].cpu().numpy(), r["v"])
        e_x = rel_err(xs_c[k].cpu().numpy(), r["x_next"])
        e_cr = rel_err(vs_c[k].cpu().numpy(), vs_r[k].cpu().numpy())
        say(f"  step {k} {r['mode']}: v rel {e_v:.3e}  x rel {e_x:.3e}  cached-vs-recompute {e_cr:.3e}")
        assert e_v < TOL_BF16 and e_x < TOL_BF16
        assert e_cr < TOL_CACHED


@pytest.mark.parametrize("name", ["c2", "c3", "c4", "c5"])
def test_one_layer_full_token_counts_sampled(dev, name):
    """Real token counts of each workload with one layer: v_θ of 48 sampled
    target rows from extract (σ = 1) and from a cached step (σ = 0.978453, a
    fresh seeded latent) against the oracle's row-wise evaluation."""
    cfg, W, I, rt, seq, pre, x0 = build(name, dev, n_layers=1)
    say(f"one-layer {name} P={seq.P} T={seq.T}")
    cache = rt.alloc_cache(seq)
    ws = rt.alloc_workspace(seq.S)
    v = torch.empty_like(x0)
    rt.step_extract(seq, pre, x0, 1.0, cache, v, ws)
    x1 = synth._rng(99, "x_alt").standard_normal((seq.T, 64), dtype=np.float32)
    v1 = torch.empty_like(x0)
    rt.step_cached(seq, torch.from_numpy(x1).to(dev), 0.978453, cache, v1, ws)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(7).choice(seq.T, 48, replace=False))
    rows = np.unique(np.concatenate([[0, seq.T - 1], rows]))
    dims = dims_of(cfg)
    lay = O.build_layout(cfg["segments"])
    opre = oracle_prefix(cfg, W, I)
    r0 = O.cached_rows_one_layer(W, dims, lay, opre, I["x0"], 1.0, rows)
    r1 = O.cached_rows_one_layer(W, dims, lay, opre, x1, 0.978453, rows)
    e0 = rel_err(v.cpu().numpy()[rows], r0)
    e1 = rel_err(v1.cpu().numpy()[rows], r1)
    say(f"  extract rows rel {e0:.3e}  cached rows rel {e1:.3e}")
    assert e0 < TOL_BF16 and e1 < TOL_BF16


def random_full_width_layout(seed):
    """Seeded random layout at the real width: 1-4 text runs and 0-3
    reference images of mixed sizes in random order, then a target of
    46..64 x 46..64 tokens (enough 256-row blocks, with 32 heads, for the
    cached step's pipelined attention). Even seeds pad the first text run so S
    is a multiple of 64; odd seeds make it not one (staged kernel)."""
    r = np.random.default_rng(500 + seed)
    segs = [("text", int(r.integers(16, 300))) for _ in range(int(r.integers(1, 5)))]
    segs += [("ref", int(r.integers(8, 49)), int(r.integers(8, 49))) for _ in range(int(r.integers(0, 4)))]
    order = r.permutation(len(segs))
    segs = [segs[i] for i in order]
    segs.append(("target", int(r.integers(46, 65)), int(r.integers(46, 65))))
    S = sum(s[1] if s[0] == "text" else s[1] * s[2] for s in segs)
    i = next(k for k, s in enumerate(segs) if s[0] == "text")
    if seed % 2 == 0 and S % 64:
        segs[i] = ("text", segs[i][1] + 64 - S % 64)
    elif seed % 2 == 1 and S % 64 == 0:
        segs[i] = ("text", segs[i][1] + 1)
    return segs


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_layouts_one_layer_sampled(dev, seed):
    """Random full-width layouts (one layer, hidden 4096, 32 heads): v_θ of
    48 sampled target rows from extract and from a cached step against the
    oracle's row-wise evaluation, with S a multiple of 64 or not (the two
    attention kernels of cached steps)."""
    segs = random_full_width_layout(seed)
    cfg = synth.config("c1", segments=segs)
    W = synth.make_weights(cfg, seed=21, workers=16)
    I = synth.make_inputs(cfg, seed=21 + seed)
    rt = DitRuntime(cfg, W, device=dev)
    seq = rt.sequence(cfg["segments"])
    pre = rt.prefix_hidden(I)
    x0 = torch.from_numpy(I["x0"]).to(dev)
    say(f"random layout {seed}: {len(segs)} segments, P={seq.P} T={seq.T} S%64={seq.S % 64}")
    cache = rt.alloc_cache(seq)
    ws = rt.alloc_workspace(seq.S)
    v = torch.empty_like(x0)
    rt.step_extract(seq, pre, x0, 1.0, cache, v, ws)
    x1 = synth._rng(98 + seed, "x_alt").standard_normal((seq.T, 64), dtype=np.float32)
    v1 = torch.empty_like(x0)
    rt.step_cached(seq, torch.from_numpy(x1).to(dev), 0.978453, cache, v1, ws)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(8 + seed).choice(seq.T, 48, replace=False))
    rows = np.unique(np.concatenate([[0, seq.T - 1], rows]))
    dims = dims_of(cfg)
    lay = O.build_layout(cfg["segments"])
    opre = oracle_prefix(cfg, W, I)
    r0 = O.cached_rows_one_layer(W, dims, lay, opre, I["x0"], 1.0, rows)
    r1 = O.cached_rows_one_layer(W, dims, lay, opre, x1, 0.978453, rows)
    e0 = rel_err(v.cpu().numpy()[rows], r0)
    e1 = rel_err(v1.cpu().numpy()[rows], r1)
    say(f"  extract rows rel {e0:.3e}  cached rows rel {e1:.3e}")
    assert e0 < TOL_BF16 and e1 < TOL_BF16
    rt.close()


def nearest_rows(got, ref):
    """Index of the nearest ref row (squared distance) for every got row."""
    g = got.astype(np.float64)
    d2 = (g * g).sum(1)[:, None] + (ref * ref).sum(1)[None, :] - 2.0 * g @ ref.T
    return np.argmin(d2, axis=1)


def test_cache_rows_land_at_their_token_index(dev):
    """After extract, K cache row j of every head holds token j's post-norm,
    post-RoPE key (nearest oracle row is j itself, and values agree to bf16
    tolerance); V likewise; padding rows S..cap-1 are zero."""
    cfg, W, I, rt, seq, pre, x0 = build("c1", dev)
    cache = rt.alloc_cache(seq)
    cache.fill_(0x3F80)   # 1.0 everywhere before the step
    ws = rt.alloc_workspace(seq.S)
    v = torch.empty_like(x0)
    rt.step_extract(seq, pre, x0, 1.0, cache, v, ws)
    torch.cuda.synchronize()
    cap = L.dit_kv_capacity(seq.S)
    kc, vt = cache_views(cache, 1, 32, cap)
    lay = O.build_layout(cfg["segments"])
    e = O.forward_extract(W, dims_of(cfg), lay, oracle_prefix(cfg, W, I), I["x0"], 1.0)
    k_ref = e["k_all"][0]                               # [S, nh, d]
    v_ref = e["v_all"][0]
    for h in (0, 17, 31):
        kg = i16_to_f32(kc[0, h, :seq.S])               # [S, d]
        assert rel_err(kg, k_ref[:, h]) < TOL_BF16
        assert np.array_equal(nearest_rows(kg, k_ref[:, h]), np.arange(seq.S))
        vg = i16_to_f32(vt[0, h, :, :seq.S].T.contiguous())   # Vᵀ stored dim-major
        assert rel_err(vg, v_ref[:, h]) < TOL_BF16
        assert np.array_equal(nearest_rows(vg, v_ref[:, h]), np.arange(seq.S))
    assert int(kc[0, :, seq.S:].abs().sum()) == 0
    assert int(vt[0, :, :, seq.S:].abs().sum()) == 0


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def depth_golden(name, n_layers):
    """Stored oracle values of the 8-step Turbo loop of a deep model (written
    by ``tests/golden/make_depth_goldens.py``, which calls only the oracle and
    the seeded generators)."""
    path = os.path.join(GOLDEN, f"depth_{name}_L{n_layers}.npz")
    assert os.path.exists(path), f"missing {path}: run tests/golden/make_depth_goldens.py"
    g = np.load(path)
    return {k: g[k] for k in g.files}


def deep_runtime(name, n_layers, dev):
    """A runtime holding the seeded host weights of ``synth`` (the oracle's),
    drawn and uploaded layer by layer."""
    cfg = synth.config(name)
    cfg["n_layers"] = n_layers
    Wd, crcs, gcrc = synth_weights_on_device(cfg, dev)
    rt = DitRuntime(cfg, Wd, device=dev, on_device=True)
    I = synth.make_inputs(cfg)
    seq = rt.sequence(cfg["segments"])
    pre = rt.prefix_hidden(I)
    x0 = torch.from_numpy(I["x0"]).to(dev)
    return cfg, rt, seq, pre, x0, Wd, (crcs, gcrc)


@pytest.fixture(scope="module")
def c2_full(dev):
    """32-layer, 4096-wide text-to-image workload (256 text + 64x64 target)
    with the seeded host weights the oracle's stored values were made from."""
    say("c2 full depth: drawing 32 layers of seeded weights")
    cfg, rt, seq, pre, x0, Wd, crcs = deep_runtime("c2", 32, dev)
    yield cfg, rt, seq, pre, x0, crcs
    rt.close()
    del Wd
    torch.cuda.empty_cache()


def check_turbo_loop_against_golden(name, rt, seq, pre, x0, cfg, crcs):
    g = depth_golden(name, cfg["n_layers"])
    assert list(g["layer_crc"]) == list(crcs[0]) and int(g["global_crc"]) == crcs[1], \
        "the stored oracle values were made from other weights"
    sig = cfg["sigmas"]
    rows = g["rows"]
    vs, xs = rt.run_loop(seq, pre, x0, sig, use_cache=True)
    torch.cuda.synchronize()
    worst = 0.0
    for k in range(len(sig) - 1):
        v = vs[k].cpu().numpy()
        e_v = rel_err(v[rows], g["v"][k])
        e_max = abs(float(np.abs(v).max()) - g["v_absmax"][k]) / g["v_absmax"][k]
        e_xm = abs(float(xs[k].abs().max()) - g["x_absmax"][k]) / g["x_absmax"][k]
        say(f"  step {k} {'extract' if k == 0 else 'cached'}: v rel {e_v:.3e} on {len(rows)} rows, "
            f"max|v| rel {e_max:.1e}, max|x| rel {e_xm:.1e}")
        assert e_v < TOL_BF16 and e_max < TOL_BF16 and e_xm < TOL_BF16
        worst = max(worst, e_v)
    e_x = rel_err(xs[-1].cpu().numpy(), g["x_final"])
    say(f"  final latent (all {seq.T} rows) rel {e_x:.3e}; worst v step {worst:.3e}")
    assert e_x < TOL_BF16


@pytest.mark.timeout(900)
def test_full_depth_turbo_loop_matches_oracle(dev, c2_full):
    """The target configuration: the 32-layer, 4096-wide model over the whole
    8-step Turbo loop (extract, then seven cached steps) against the fp64
    oracle's stored values -- v_θ of every step on a seeded eighth of the
    target rows, max |v_θ| and max |x| over all rows, and the final latent
    on every row."""
    cfg, rt, seq, pre, x0, crcs = c2_full
    say("c2 full depth: 8-step Turbo loop vs the oracle")
    check_turbo_loop_against_golden("c2", rt, seq, pre, x0, cfg, crcs)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["c3", "c4"])
def test_two_layer_turbo_loop_matches_oracle(dev, name):
    """The editing (4352-row prefix) and multi-reference (12800-row prefix,
    96x96 target) workloads at full width with two layers, over all eight
    Turbo steps, against the oracle's stored values."""
    say(f"{name} two layers: 8-step Turbo loop vs the oracle")
    cfg, rt, seq, pre, x0, Wd, crcs = deep_runtime(name, 2, dev)
    check_turbo_loop_against_golden(name, rt, seq, pre, x0, cfg, crcs)
    rt.close()
    del Wd
    torch.cuda.empty_cache()


def test_full_depth_cached_matches_recompute(dev, c2_full):
    cfg, rt, seq, pre, x0, _ = c2_full
    say("c2 full depth: 8-step cached loop vs recompute")
    vs_c, xs_c = rt.run_loop(seq, pre, x0, cfg["sigmas"], use_cache=True)
    vs_r, xs_r = rt.run_loop(seq, pre, x0, cfg["sigmas"], use_cache=False)
    torch.cuda.synchronize()
    for k in range(len(vs_c)):
        assert torch.isfinite(vs_c[k]).all()
        e = rel_err(vs_c[k].cpu().numpy(), vs_r[k].cpu().numpy())
        say(f"  step {k}: cached vs recompute {e:.3e}")
        assert e < TOL_CACHED
    assert rel_err(xs_c[-1].cpu().numpy(), xs_r[-1].cpu().numpy()) < TOL_CACHED


def test_full_depth_cache_invariants(dev, c2_full):
    """Prefix K/V independent of σ and x; cached steps never write rows < P;
    the same cached step twice gives identical bits; without t = 0
    conditioning the prefix K/V change."""
    cfg, rt, seq, pre, x0, _ = c2_full
    say("c2 full depth: cache invariants")
    P, S = seq.P, seq.S
    cap = L.dit_kv_capacity(S)
    Lc = cfg["n_layers"]
    ws = rt.alloc_workspace(S)
    v = torch.empty_like(x0)
    c1 = rt.alloc_cache(seq)
    rt.step_extract(seq, pre, x0, 1.0, c1, v, ws)
    x1 = x0 + 0.37 * v
    c2 = rt.alloc_cache(seq)
    rt.step_extract(seq, pre, x1, 0.845148, c2, v, ws)
    torch.cuda.synchronize()
    k1, v1 = cache_views(c1, Lc, 32, cap)
    k2, v2 = cache_views(c2, Lc, 32, cap)
    assert torch.equal(k1[:, :, :P], k2[:, :, :P])
    assert torch.equal(v1[:, :, :, :P], v2[:, :, :, :P])
    # cached steps leave the prefix rows alone, and are deterministic
    before_k = k1[:, :, :P].clone()
    before_v = v1[:, :, :, :P].clone()
    wa = rt.alloc_workspace(seq.T)
    va, vb = torch.empty_like(x0), torch.empty_like(x0)
    rt.step_cached(seq, x1, 0.95418, c1, va, wa)
    rt.step_cached(seq, x1, 0.95418, c1, vb, wa)
    torch.cuda.synchronize()
    assert torch.equal(k1[:, :, :P], before_k) and torch.equal(v1[:, :, :, :P], before_v)
    assert torch.equal(va, vb)
    # drift without causal conditioning
    c3 = rt.alloc_cache(seq)
    c4 = rt.alloc_cache(seq)
    rt.step_extract(seq, pre, x0, 1.0, c3, v, ws, flags=L.DIT_FLAG_NO_CAUSAL_CONDITION)
    rt.step_extract(seq, pre, x1, 0.845148, c4, v, ws, flags=L.DIT_FLAG_NO_CAUSAL_CONDITION)
    torch.cuda.synchronize()
    k3, _ = cache_views(c3, Lc, 32, cap)
    k4, _ = cache_views(c4, Lc, 32, cap)
    for l in (0, Lc - 1):
        assert not torch.equal(k3[l, :, :P], k4[l, :, :P])
    with pytest.raises(L.DitError) as e:
        rt.step_cached(seq, x1, 0.95418, c3, va, wa)
    assert e.value.status == L.DIT_ERR_STATE


@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_full_depth_largest_workloads_cached_matches_recompute(dev, name):
    """The editing (4352-row prefix), multi-reference (12800-row prefix, 96x96
    target, 22016 keys, 11.6 GB of KV cache) and ten-reference (41472-row
    prefix, 50688 keys, 26.6 GB of KV cache) workloads at full depth: all
    eight Turbo steps, cached against full recompute, finite and within the
    cached-path bound."""
    from diffusion_transformer_amd.runtime import random_weights_device
    cfg = synth.config(name)
    Wd = random_weights_device(cfg, 21, dev)
    rt = DitRuntime(cfg, Wd, device=dev, on_device=True)
    I = synth.make_inputs(cfg)
    seq = rt.sequence(cfg["segments"])
    pre = rt.prefix_hidden(I)
    x0 = torch.from_numpy(I["x0"]).to(dev)
    sig = cfg["sigmas"]
    say(f"{name} full depth P={seq.P} T={seq.T}: 8-step cached loop vs recompute")
    vs_c, xs_c = rt.run_loop(seq, pre, x0, sig, use_cache=True)
    vs_r, xs_r = rt.run_loop(seq, pre, x0, sig, use_cache=False)
    torch.cuda.synchronize()
    for k in range(len(vs_c)):
        assert torch.isfinite(vs_c[k]).all()
        e = rel_err(vs_c[k].cpu().numpy(), vs_r[k].cpu().numpy())
        say(f"  step {k}: cached vs recompute {e:.3e}")
        assert e < TOL_CACHED
    assert rel_err(xs_c[-1].cpu().numpy(), xs_r[-1].cpu().numpy()) < TOL_CACHED
    rt.close()
    del Wd
    torch.cuda.empty_cache()


def test_batch_of_targets_shares_one_prefix(dev):
    """Three target latents denoised together against one shared prefix
    cache (512 text + 32x32 target, one layer): each element's v from the
    batched extract and cached steps equals the same element run alone, the
    shared prefix K/V rows are identical to a single run's and each
    element's target K rows sit at P + b*T; the middle element's cached rows
    also match the oracle."""
    cfg, W, I, rt, seq1, pre, x0 = build("c1", dev)
    B, P, T = 3, seq1.P, seq1.T
    seqb = rt.sequence(cfg["segments"], batch=B)
    say(f"batch of {B} targets sharing P={P} (T={T})")
    rng = [synth._rng(100 + b, "x_batch") for b in range(B)]
    xs = [x0] + [torch.from_numpy(rng[b].standard_normal((T, 64), dtype=np.float32)).to(dev)
                 for b in range(1, B)]
    x2 = [torch.from_numpy(rng[b].standard_normal((T, 64), dtype=np.float32)).to(dev)
          for b in range(B)]
    cb, wb = rt.alloc_cache(seqb), rt.alloc_workspace(seqb.S_all)
    xb, x2b = torch.cat(xs).contiguous(), torch.cat(x2).contiguous()
    vb, vbc = torch.empty_like(xb), torch.empty_like(xb)
    rt.step_extract(seqb, pre, xb, 1.0, cb, vb, wb)
    rt.step_cached(seqb, x2b, 0.978453, cb, vbc, wb)
    torch.cuda.synchronize()
    Lc, nh = cfg["n_layers"], cfg["n_heads"]
    kb, _ = cache_views(cb, Lc, nh, L.dit_kv_capacity(seqb.S_all))
    for b in range(B):
        c1, w1 = rt.alloc_cache(seq1), rt.alloc_workspace(seq1.S)
        v1, v1c = torch.empty_like(x0), torch.empty_like(x0)
        rt.step_extract(seq1, pre, xs[b], 1.0, c1, v1, w1)
        k_after_extract = cache_views(c1, Lc, nh, L.dit_kv_capacity(seq1.S))[0].clone()
        rt.step_cached(seq1, x2[b], 0.978453, c1, v1c, w1)
        torch.cuda.synchronize()
        k1, _ = cache_views(c1, Lc, nh, L.dit_kv_capacity(seq1.S))
        ex = rel_err(vb[b * T:(b + 1) * T].cpu().numpy(), v1.cpu().numpy())
        ec = rel_err(vbc[b * T:(b + 1) * T].cpu().numpy(), v1c.cpu().numpy())
        say(f"  element {b}: extract vs alone {ex:.2e}, cached vs alone {ec:.2e}")
        assert ex < TOL_CACHED and ec < TOL_CACHED
        assert torch.equal(kb[:, :, :P], k_after_extract[:, :, :P])
        # the batched cache holds the cached step's target K of element b
        et = rel_err(i16_to_f32(kb[:, :, P + b * T:P + (b + 1) * T]), i16_to_f32(k1[:, :, P:P + T]))
        assert et < TOL_CACHED
    rows = np.sort(np.random.default_rng(5).choice(T, 32, replace=False))
    r1 = O.cached_rows_one_layer(W, dims_of(cfg), O.build_layout(cfg["segments"]),
                                 oracle_prefix(cfg, W, I), x2[1].cpu().numpy(), 0.978453, rows)
    e = rel_err(vbc[T:2 * T].cpu().numpy()[rows], r1)
    say(f"  element 1 cached rows vs oracle {e:.2e}")
    assert e < TOL_BF16


def test_prefix_front_end_and_unstandardized_output(dev):
    """Reference latents given in VAE space are standardized per channel on
    the GPU before img_in (page 1A): the prefix equals the one built from the
    standardized latents. After a short loop the final latent is returned to
    VAE space (page 6B) and matches the oracle's unstandardized latent."""
    cfg, W, I, rt, seq, pre, x0 = build("c0w", dev)
    mean, std = synth.latent_stats(cfg["latent"])
    md, sd = torch.from_numpy(mean).to(dev), torch.from_numpy(std).to(dev)
    cfg1, W1, I1, rt1, seq1, pre1, _ = build("c3", dev, n_layers=1)
    raw = O.unstandardize(I1["ref_latents"], mean, std).astype(np.float32)
    say(f"c3 prefix from {raw.shape[0]} raw reference latents")
    pre_raw = rt1.prefix_hidden(I1, raw_latents=torch.from_numpy(raw), stats=(md, sd))
    torch.cuda.synchronize()
    assert rel_err(pre_raw.cpu().numpy(), pre1.cpu().numpy()) < 1e-5
    rt1.close()
    say("c0w loop, final latent unstandardized")
    sig = cfg["sigmas"]
    vs, xs = rt.run_loop(seq, pre, x0, sig, use_cache=True)
    xf = rt.standardize(xs[-1].clone(), (md, sd), inverse=True)
    torch.cuda.synchronize()
    ref = O.run_loop(W, dims_of(cfg), O.build_layout(cfg["segments"]), oracle_prefix(cfg, W, I),
                     I["x0"], sig, use_cache=True)
    e = rel_err(xf.cpu().numpy(), O.unstandardize(ref[-1]["x_next"], mean, std))
    say(f"  unstandardized final latent vs oracle {e:.2e}")
    assert e < TOL_BF16


@pytest.mark.parametrize("mode", ["linear12", "no_causal"])
def test_general_schedules_and_no_causal_condition(dev, mode):
    """The GPU loop over a 12-step linear schedule (cached after step 1), and
    the loop without t = 0 conditioning (every step recomputes, page 3B §4),
    against the oracle's loops: v and the latent after every step."""
    cfg, W, I, rt, seq, pre, x0 = build("c0w", dev)
    if mode == "linear12":
        sig, use_cache, cc = tuple(float(s) for s in np.linspace(1.0, 0.0, 13)), True, True
    else:
        sig, use_cache, cc = cfg["sigmas"], False, False
    say(f"c0w loop {mode}: {len(sig) - 1} steps")
    vs, xs = rt.run_loop(seq, pre, x0, sig, use_cache=use_cache, causal_condition=cc)
    torch.cuda.synchronize()
    ref = O.run_loop(W, dims_of(cfg), O.build_layout(cfg["segments"]), oracle_prefix(cfg, W, I),
                     I["x0"], sig, use_cache=use_cache, causal_condition=cc)
    for k, r in enumerate(ref):
        ev = rel_err(vs[k].cpu().numpy(), r["v"])
        ex = rel_err(xs[k].cpu().numpy(), r["x_next"])
        assert ev < TOL_BF16 and ex < TOL_BF16, (k, ev, ex)
    say(f"  last step: v {ev:.2e}, x {ex:.2e}")


def test_cached_step_graph_replays_match_eager(dev):
    """The cached Euler step recorded into a HIP graph: every replay (with
    eager work and synchronizations between replays) gives the eager step's
    v and x bit for bit."""
    cfg, W, I, rt, seq, pre, x0 = build("c1", dev)
    sig = cfg["sigmas"]
    cache = rt.alloc_cache(seq)
    ws = rt.alloc_workspace(seq.S_all)
    v = torch.empty_like(x0)
    rt.step_extract(seq, pre, x0.clone(), sig[0], cache, v, ws)
    xe, ve = x0.clone(), torch.empty_like(x0)
    rt.step_cached(seq, xe, sig[1], cache, ve, ws)
    L.euler_update(xe, ve, sig[1], sig[2])
    torch.cuda.synchronize()
    xg, vg = x0.clone(), torch.empty_like(x0)
    g = rt.cached_step_graph(seq, xg, sig[1], sig[2], cache, vg, ws)
    say("c1 cached step graph: 3 replays")
    for r in range(3):
        xg.copy_(x0)
        vg.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(vg, ve), r
        assert torch.equal(xg, xe), r
        assert float((xe * 2).sum()) != 0.0   # eager work between replays


@pytest.mark.parametrize("tgt", [(4, 4), (20, 20)])
def test_loop_without_prefix(dev, tgt):
    """A layout with no text and no reference (P = 0): the extract step and
    the cached steps see only the target tokens, and match the oracle."""
    cfg = synth.config("c0w", segments=[("target", *tgt)])
    W = synth.make_weights(cfg)
    I = synth.make_inputs(cfg)
    rt = DitRuntime(cfg, W, device=dev)
    seq = rt.sequence(cfg["segments"])
    assert seq.P == 0
    pre = rt.prefix_hidden(I)
    x0 = torch.from_numpy(I["x0"]).to(dev)
    sig = cfg["sigmas"]
    say(f"no prefix: target {tgt}, T={seq.T}")
    vs, xs = rt.run_loop(seq, pre, x0, sig, use_cache=True)
    torch.cuda.synchronize()
    ref = O.run_loop(W, dims_of(cfg), O.build_layout(cfg["segments"]), oracle_prefix(cfg, W, I),
                     I["x0"], sig, use_cache=True)
    for k, r in enumerate(ref):
        e_v = rel_err(vs[k].cpu().numpy(), r["v"])
        say(f"  step {k} {r['mode']}: v rel {e_v:.3e}")
        assert e_v < TOL_BF16
    rt.close()


@pytest.mark.parametrize("segs", [
    [("text", 1), ("target", 1, 1)],
    [("target", 1, 1)],
    [("ref", 1, 1), ("target", 1, 7)],
    [("text", 3), ("ref", 5, 1), ("target", 3, 1)],
], ids=["text1-target1x1", "target1x1", "ref1x1-target1x7", "strips"])
def test_degenerate_layouts(dev, segs):
    """Single-token and one-row / one-column images: every GEMM, the
    attention and the elementwise kernels run on one-token or one-strip
    inputs, and the 3-step loop matches the oracle."""
    cfg = synth.config("c0w", segments=segs)
    W = synth.make_weights(cfg)
    I = synth.make_inputs(cfg)
    rt = DitRuntime(cfg, W, device=dev)
    seq = rt.sequence(cfg["segments"])
    pre = rt.prefix_hidden(I)
    x0 = torch.from_numpy(I["x0"]).to(dev)
    sig = cfg["sigmas"]
    say(f"degenerate layout {segs}: P={seq.P} T={seq.T}")
    vs, xs = rt.run_loop(seq, pre, x0, sig, use_cache=True)
    torch.cuda.synchronize()
    ref = O.run_loop(W, dims_of(cfg), O.build_layout(cfg["segments"]), oracle_prefix(cfg, W, I),
                     I["x0"], sig, use_cache=True)
    for k, r in enumerate(ref):
        e_v = rel_err(vs[k].cpu().numpy(), r["v"])
        e_x = rel_err(xs[k].cpu().numpy(), r["x_next"])
        say(f"  step {k} {r['mode']}: v rel {e_v:.3e}  x rel {e_x:.3e}")
        assert e_v < TOL_BF16 and e_x < TOL_BF16
    rt.close()


def test_peaked_attention_loop_matches_oracle(dev):
    """Peaked attention inside the step: QK-RMSNorm weights near 1.5 (so
    1 + w is about 2.5 and every score is about six times larger) on a
    344-token layout with six key tiles, through the 3-step loop against the
    oracle on the same weights."""
    segs = [("text", 100), ("ref", 10, 10), ("target", 12, 12)]
    cfg = synth.config("c0w", segments=segs)
    W = synth.make_weights(cfg)
    g = np.random.default_rng(31)
    for layer in W["layers"]:
        for k in ("q_norm", "k_norm"):
            layer[k] = synth.round_bf16((1.5 + 0.1 * g.standard_normal(128)).astype(np.float32))
    I = synth.make_inputs(cfg)
    rt = DitRuntime(cfg, W, device=dev)
    seq = rt.sequence(cfg["segments"])
    pre = rt.prefix_hidden(I)
    x0 = torch.from_numpy(I["x0"]).to(dev)
    sig = cfg["sigmas"]
    say(f"peaked attention: P={seq.P} T={seq.T}")
    vs, xs = rt.run_loop(seq, pre, x0, sig, use_cache=True)
    torch.cuda.synchronize()
    ref = O.run_loop(W, dims_of(cfg), O.build_layout(segs), oracle_prefix(cfg, W, I), I["x0"], sig,
                     use_cache=True)
    for k, r in enumerate(ref):
        e_v = rel_err(vs[k].cpu().numpy(), r["v"])
        e_x = rel_err(xs[k].cpu().numpy(), r["x_next"])
        say(f"  step {k} {r['mode']}: v rel {e_v:.3e}  x rel {e_x:.3e}")
        assert e_v < TOL_BF16 and e_x < TOL_BF16
    rt.close()


@pytest.mark.parametrize("name", ["c0w", "c1"])
def test_per_kernel_timing_hooks(dev, name):
    """dit_profile_enable / dit_profile_read for every kernel class: one
    extract plus one cached step record one event pair per launch of that
    class (on the kernel's own dispatch packet, or around a multi-kernel
    split-K sequence), each with a positive duration that fits in the two
    steps, and the outputs are bitwise those of an untimed run."""
    cfg, W, I, rt, seq, pre, x0 = build(name, dev)
    nl = cfg["n_layers"]
    sig = cfg["sigmas"]
    cache = rt.alloc_cache(seq)
    ws = rt.alloc_workspace(seq.S_all)
    pad = L.dit_kv_capacity(seq.S_all) > seq.S_all
    per_step = {"gemm_qkv": nl, "gemm_o": nl, "gemm_gateup": nl, "gemm_down": nl, "attention": nl,
                "ln": 2 * nl, "final": 1, "img_in": 1, "gemv": 3, "gemv_mod": 1}

    def two_steps(cls):
        L.dit_profile_enable(rt.model, cls)
        x = x0.clone()
        v0, v1 = torch.empty_like(x), torch.empty_like(x)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        rt.step_extract(seq, pre, x, sig[0], cache, v0, ws)
        rt.step_cached(seq, x, sig[1], cache, v1, ws)
        b.record()
        torch.cuda.synchronize()
        ms, n = L.dit_profile_read(rt.model)
        L.dit_profile_enable(rt.model, "off")
        return v0, v1, ms, n, a.elapsed_time(b)

    ref0, ref1, ms, n, _ = two_steps("off")
    assert n == 0 and ms == 0.0
    for cls in list(L.PROF)[1:]:
        v0, v1, ms, n, wall = two_steps(cls)
        want = 2 * per_step.get(cls, 0) + (nl if cls == "qknorm_rope" and pad else 0)
        say(f"{name} {cls}: {n} launches, {ms:.4f} ms of {wall:.3f} ms")
        assert n == want, (cls, n, want)
        if n:
            assert 0.0 < ms < wall, (cls, ms, wall)
        assert torch.equal(v0, ref0) and torch.equal(v1, ref1), cls
