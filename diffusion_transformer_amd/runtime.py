"""Torch plumbing around the C ABI: device memory for weights, layout
tables, KV cache, workspace and latents, and the sampler loop (step 1
extract, steps 2..N cached, Euler after each step). PyTorch only allocates
and holds memory here; every computation is a call into ``libdit.so``."""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as L

LAYER_KEYS = ("qkv", "q_norm", "k_norm", "o", "gate", "up", "down")
GLOBAL_KEYS = ("t1", "t2", "mod", "so", "img_in", "proj_out")


def to_device_bf16(a, device):
    """bf16-exact float32 numpy array (or torch tensor) -> contiguous bf16 device tensor."""
    if isinstance(a, torch.Tensor):
        return a.to(device=device, dtype=torch.bfloat16).contiguous()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(
        device=device).to(torch.bfloat16).contiguous()


def upload_weights(W: dict, device) -> dict:
    out = {k: to_device_bf16(W[k], device) for k in GLOBAL_KEYS}
    for k in LAYER_KEYS:
        out[k] = [to_device_bf16(layer[k], device) for layer in W["layers"]]
    return out


def random_weights_device(cfg: dict, seed: int, device, n_layers=None) -> dict:
    """Seeded N(0, 1/fan_in) bf16 weights drawn directly on the GPU with
    torch's generator (for full-size throughput runs, where host generation
    of 17 GB would dominate). Same shapes as synth.make_weights."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    H, d, F, C, Dt = cfg["hidden"], cfg["head_dim"], cfg["ffn"], cfg["latent"], cfg["time_dim"]
    Lc = cfg["n_layers"] if n_layers is None else n_layers

    def n(shape, fan_in):
        t = torch.empty(shape, device=device, dtype=torch.float32)
        t.normal_(0.0, 1.0 / float(np.sqrt(fan_in)), generator=g)
        return t.to(torch.bfloat16)

    out = {"t1": n((H, Dt), Dt), "t2": n((H, H), H), "mod": n((4 * H, H), H),
           "so": n((H, H), H), "img_in": n((H, C), C), "proj_out": n((C, H), H)}
    for k in LAYER_KEYS:
        out[k] = []
    for _ in range(Lc):
        out["qkv"].append(n((3 * H, H), H))
        out["q_norm"].append(n((d,), d))
        out["k_norm"].append(n((d,), d))
        out["o"].append(n((H, H), H))
        out["gate"].append(n((F, H), H))
        out["up"].append(n((F, H), H))
        out["down"].append(n((H, F), F))
    return out


class Sequence:
    """Device copy of one token layout plus its C struct. ``batch`` target
    latents share the prefix: x and v hold batch*T rows, the cache
    S_all = P + batch*T keys."""

    def __init__(self, cfg_c, segments, device, api=L, batch=1):
        lay = api.dit_build_layout(cfg_c, segments)
        self.host = lay
        self.P, self.T = lay["P"], lay["T"]
        self.S = self.P + self.T
        self.B = batch
        self.S_all = self.P + batch * self.T
        self.row_limit = torch.from_numpy(lay["row_limit"]).to(device)
        self.rope_cos = torch.from_numpy(lay["rope_cos"]).to(device)
        self.rope_sin = torch.from_numpy(lay["rope_sin"]).to(device)
        self.c = api.make_seq(self.P, self.T, self.row_limit, self.rope_cos, self.rope_sin, batch)


class DitRuntime:
    """``api``: the binding of the library to use (default: the production
    bf16 library; ``_lib.load_f32()`` for the fp32 debug build)."""

    def __init__(self, cfg: dict, weights: dict, device="cuda", on_device=False, api=None):
        self.L = api if api is not None else L
        self.cfg = cfg
        self.device = torch.device(device)
        self.c = self.L.make_config(**{k: cfg[k] for k in ("hidden", "n_heads", "head_dim", "ffn",
                                                      "n_layers", "latent", "time_dim",
                                                      "rope_dims")})
        self.w = weights if on_device else upload_weights(weights, self.device)
        self.model = self.L.dit_load_weights(self.c, self.w)

    def close(self):
        if self.model:
            self.L.dit_free(self.model)
            self.model = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def sequence(self, segments, batch=1) -> Sequence:
        return Sequence(self.c, segments, self.device, self.L, batch)

    def alloc_cache(self, seq: Sequence) -> torch.Tensor:
        nbytes = self.L.dit_kv_cache_bytes(self.model, seq.S_all)
        return torch.empty(nbytes // 2, dtype=torch.int16, device=self.device)

    def alloc_workspace(self, n_tokens: int) -> torch.Tensor:
        nbytes = self.L.dit_workspace_bytes(self.model, n_tokens)
        return torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=self.device)

    def img_in(self, latents: torch.Tensor) -> torch.Tensor:
        out = torch.empty((latents.shape[0], self.cfg["hidden"]), dtype=torch.float32,
                          device=self.device)
        if latents.shape[0]:
            self.L.dit_img_in(self.model, latents.contiguous(), out)
        return out

    def standardize(self, z: torch.Tensor, stats, inverse=False) -> torch.Tensor:
        """Per-channel latent (un)standardization on the GPU, in place;
        ``stats`` = (mean [C], std [C]) device float32 tensors."""
        self.L.dit_latent_standardize(z, stats[0], stats[1], inverse)
        return z

    def prefix_hidden(self, inputs: dict, raw_latents=None, stats=None) -> torch.Tensor:
        """Prefix rows in sequence order: text hidden states as given,
        reference tokens drawn directly or embedded from latents by img_in.
        With ``raw_latents`` [n_ref, C] (VAE space) and ``stats`` the
        reference latents are standardized on the GPU first (page 1A)."""
        kind = torch.from_numpy(inputs["prefix_kind"].astype(np.int64)).to(self.device)
        text = torch.from_numpy(inputs["text_hidden"]).to(self.device)
        if raw_latents is not None:
            z = raw_latents.to(self.device, torch.float32).contiguous().clone()
            ref = self.img_in(self.standardize(z, stats))
        elif "ref_hidden" in inputs:
            ref = torch.from_numpy(inputs["ref_hidden"]).to(self.device)
        else:
            ref = self.img_in(torch.from_numpy(inputs["ref_latents"]).to(self.device))
        out = torch.empty((kind.numel(), self.cfg["hidden"]), dtype=torch.float32, device=self.device)
        out[kind == 0] = text
        out[kind == 1] = ref
        return out

    def step_extract(self, seq, prefix, x, sigma, cache, v, ws, flags=0, stream=None):
        self.L.dit_step_extract(self.model, seq.c, prefix, x, sigma, cache, v, ws, flags, stream)

    def step_cached(self, seq, x, sigma, cache, v, ws, stream=None):
        self.L.dit_step_cached(self.model, seq.c, x, sigma, cache, v, ws, stream)

    def cached_step_graph(self, seq, x, sigma, sigma_next, cache, v, ws):
        """Record one cached Euler step -- dit_step_cached(x, sigma) into v,
        then euler_update(x, v, sigma, sigma_next) in place -- into a HIP
        graph and return it; graph.replay() re-issues exactly those launches
        on the current stream (same buffers, same sigmas) without per-launch
        host work. The step must be valid when recorded (an extract into
        `cache` before), and the buffers must outlive the graph."""
        import torch
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=side):
            self.step_cached(seq, x, sigma, cache, v, ws)
            self.L.euler_update(x, v, sigma, sigma_next)
        torch.cuda.current_stream().wait_stream(side)
        return g

    def run_loop(self, seq, prefix, x0, sigmas, use_cache=True, causal_condition=True):
        """Sampler loop over any decreasing sigma schedule; returns (list of v
        per step, list of x after each step). Without causal conditioning
        every step recomputes (the prefix follows t, so no cache)."""
        if not causal_condition and use_cache:
            raise ValueError("without causal conditioning the prefix cache is invalid")
        flags = 0 if causal_condition else self.L.DIT_FLAG_NO_CAUSAL_CONDITION
        x = x0.clone().contiguous()
        cache = self.alloc_cache(seq)
        ws = self.alloc_workspace(seq.S_all)
        vs, xs = [], []
        for k in range(len(sigmas) - 1):
            v = torch.empty_like(x)
            if k == 0 or not use_cache:
                self.step_extract(seq, prefix, x, sigmas[k], cache, v, ws, flags=flags)
            else:
                self.step_cached(seq, x, sigmas[k], cache, v, ws)
            vs.append(v)
            self.L.euler_update(x, v, sigmas[k], sigmas[k + 1])
            xs.append(x.clone())
        return vs, xs
