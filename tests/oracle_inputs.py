"""Glue between the seeded workload descriptions and the fp64 oracle
(test infrastructure)."""
import numpy as np

import oracle as O
from diffusion_transformer_amd import synth


def dims_of(cfg, n_layers=None):
    return O.DitDims(hidden=cfg["hidden"], n_heads=cfg["n_heads"], head_dim=cfg["head_dim"],
                     ffn=cfg["ffn"], n_layers=cfg["n_layers"] if n_layers is None else n_layers,
                     latent=cfg["latent"], time_dim=cfg["time_dim"],
                     rope_dims=tuple(cfg["rope_dims"]))


def oracle_prefix(cfg, W, inputs):
    """Prefix hidden rows in sequence order; reference rows embedded with the
    oracle's own fp64 img_in when the config draws latents."""
    kind = inputs["prefix_kind"]
    if "ref_hidden" in inputs:
        ref = inputs["ref_hidden"].astype(np.float64)
    else:
        ref = inputs["ref_latents"].astype(np.float64) @ np.asarray(W["img_in"], np.float64).T
    out = np.empty((len(kind), cfg["hidden"]))
    out[kind == 0] = inputs["text_hidden"]
    out[kind == 1] = ref
    return out


def setup(name, n_layers=None, seed=21, **over):
    cfg = synth.config(name, **over)
    if n_layers is not None:
        cfg["n_layers"] = n_layers
    W = synth.make_weights(cfg, seed=seed)
    I = synth.make_inputs(cfg, seed=seed)
    dims = dims_of(cfg)
    lay = O.build_layout(cfg["segments"])
    pre = oracle_prefix(cfg, W, I)
    return cfg, W, I, dims, lay, pre
