"""The allocation-free cached step (dit_step_cached_noalloc, workspace in the
library's fixed device array) against dit_step_cached with a caller
workspace: three calls in a row, each with a smaller layout than the one
before (the first large enough, 256 workgroups of 256 target queries, for
the pipelined attention kernel), all bit for bit equal to the ordinary entry
point; sizes above the array are refused before any device work."""
import numpy as np
import pytest
import torch

from diffusion_transformer_amd import synth
from gpu_common import say

pytestmark = pytest.mark.gpu

L = pytest.importorskip("diffusion_transformer_amd._lib")
from diffusion_transformer_amd.runtime import DitRuntime  # noqa: E402


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def test_noalloc_cached_step_matches_cached_step(dev):
    cfg = synth.config("c1")                      # one layer, hidden 4096, 32 heads, ffn 16384
    W = synth.make_weights(cfg, workers=16)
    rt = DitRuntime(cfg, W, device=dev)
    layouts = [[("text", 512), ("target", 32, 64)], cfg["segments"],
               [("text", 128), ("ref", 8, 8), ("target", 16, 16)]]
    prev_T = None
    for call, segs in enumerate(layouts):
        c = synth.config("c1", segments=segs)
        I = synth.make_inputs(c, seed=40 + call)
        seq = rt.sequence(segs)
        if prev_T is not None:
            assert seq.T < prev_T                   # the second call is smaller
        prev_T = seq.T
        say(f"noalloc call {call}: P={seq.P} T={seq.T}")
        pre = rt.prefix_hidden(I)
        x0 = torch.from_numpy(I["x0"]).to(dev)
        cache = rt.alloc_cache(seq)
        ws = rt.alloc_workspace(seq.S_all)
        v = torch.empty_like(x0)
        rt.step_extract(seq, pre, x0, 1.0, cache, v, ws)
        x1 = x0 + 0.02 * v
        va = torch.full_like(x0, float("nan"))
        vb = torch.full_like(x0, float("nan"))
        L.dit_step_cached(rt.model, seq.c, x1, 0.978453, cache, va, ws)
        L.dit_step_cached_noalloc(rt.model, seq.c, x1, 0.978453, cache, vb)
        torch.cuda.synchronize()
        assert torch.isfinite(va).all()
        assert torch.equal(va, vb), float((va - vb).abs().max())
    # a workspace need above the fixed array is refused on the host
    big = rt.sequence([("text", 16), ("target", 64, 64)])
    need = L.dit_workspace_bytes(rt.model, big.T)
    assert need > 256 << 20
    xb = torch.zeros((big.T, 64), device=dev)
    with pytest.raises(L.DitError) as e:
        L.dit_step_cached_noalloc(rt.model, big.c, xb, 0.5, torch.empty(16, device=dev), xb)
    assert e.value.status == L.DIT_ERR_WORKSPACE
    rt.close()
