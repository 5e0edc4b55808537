"""GPU parity of the fp32 debug build (libdit_f32.so: fp32 activations,
KV cache and attention, bf16 weights) against the fp64 oracle at fp32
tolerance: v_θ and the latent after every step within 1e-5 (max relative
error over the tensor)."""
import numpy as np
import pytest
import torch

import oracle as O
from diffusion_transformer_amd import synth
from gpu_common import rel_err, say
from oracle_inputs import dims_of, oracle_prefix

pytestmark = pytest.mark.gpu

L = pytest.importorskip("diffusion_transformer_amd._lib")
from diffusion_transformer_amd.runtime import DitRuntime  # noqa: E402

TOL_F32 = 1e-5


@pytest.fixture(scope="module")
def f32():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api = L.load_f32()
    assert "fp32-debug" in api.dit_version()
    return api


@pytest.mark.parametrize("name", ["c0w", "c1"])
def test_f32_debug_loop_matches_oracle(f32, name):
    dev = torch.device("cuda:0")
    cfg = synth.config(name)
    W = synth.make_weights(cfg)
    I = synth.make_inputs(cfg)
    rt = DitRuntime(cfg, W, device=dev, api=f32)
    seq = rt.sequence(cfg["segments"])
    pre = rt.prefix_hidden(I)
    x0 = torch.from_numpy(I["x0"]).to(dev)
    sig = cfg["sigmas"]
    say(f"fp32 debug loop {name}")
    vs, xs = rt.run_loop(seq, pre, x0, sig, use_cache=True)
    vr, _ = rt.run_loop(seq, pre, x0, sig, use_cache=False)
    torch.cuda.synchronize()
    ref = O.run_loop(W, dims_of(cfg), O.build_layout(cfg["segments"]), oracle_prefix(cfg, W, I),
                     I["x0"], sig, use_cache=True)
    for k, r in enumerate(ref):
        ev = rel_err(vs[k].cpu().numpy(), r["v"])
        ex = rel_err(xs[k].cpu().numpy(), r["x_next"])
        ec = rel_err(vs[k].cpu().numpy(), vr[k].cpu().numpy())
        say(f"  step {k} {r['mode']}: v {ev:.2e}  x {ex:.2e}  cached-vs-recompute {ec:.2e}")
        assert ev < TOL_F32 and ex < TOL_F32 and ec < TOL_F32
    rt.close()
