"""Seeded synthetic workloads: configuration descriptions, weights and inputs.

This module holds no arithmetic of the method. It only describes the
workloads (dimensions, token segments, sigma schedules) and draws seeded
random numbers; both the HIP path and the fp64 oracle receive exactly the
arrays produced here.

Recipe (the same for every configuration):
- Weights are drawn N(0, 1/fan_in) in float32 (fan_in = input features of a
  Linear; norm vectors use their own length), then rounded to bfloat16
  (round-to-nearest-even); the arrays returned are float32 holding those
  bf16-exact values. Every named tensor has its own stream
  ``SeedSequence(seed, spawn_key=(crc32(name),))``.
- Text prefix hidden states and reference/target latents are N(0, 1)
  float32, each from its own named stream.
"""
from __future__ import annotations

import zlib

import numpy as np

# 8-step Turbo sigma table (page "6B · Scale-Only Final AdaLN ...", §1/§6).
TURBO_SIGMAS = (1.0, 0.978453, 0.95418, 0.926626, 0.89508, 0.845148,
                0.704534, 0.414568, 0.0)

_BIG = dict(hidden=4096, n_heads=32, head_dim=128, ffn=16384, latent=64,
            time_dim=256, rope_dims=(16, 56, 56))

# Workloads. "segments": ("text", n) | ("ref", h, w) | ("target", h, w).
CONFIGS = {
    # Lab-scale toy: 11 tokens, 7 prefix + 4 target; fp64 oracle only.
    # Its 7 prefix hidden states are drawn N(0,1) directly ("prefix_direct").
    "c0": dict(hidden=8, n_heads=2, head_dim=4, ffn=16, n_layers=2, latent=64,
               time_dim=8, rope_dims=(0, 2, 2), prefix_direct=True,
               segments=[("text", 2), ("ref", 2, 2), ("text", 1), ("target", 2, 2)],
               sigmas=(1.0, 0.85, 0.45, 0.0)),
    # GPU-shaped twin of the toy: same 11-token layout, head_dim 128.
    "c0w": dict(hidden=256, n_heads=2, head_dim=128, ffn=512, n_layers=2, latent=64,
                time_dim=256, rope_dims=(16, 56, 56), prefix_direct=True,
                segments=[("text", 2), ("ref", 2, 2), ("text", 1), ("target", 2, 2)],
                sigmas=(1.0, 0.85, 0.45, 0.0)),
    # One layer, 512 text + 32x32 target; extract at 1.0, cached at 0.978453.
    "c1": dict(_BIG, n_layers=1,
               segments=[("text", 512), ("target", 32, 32)],
               sigmas=(1.0, 0.978453, 0.95418)),
    # Text-to-image: 256 text + 64x64 target, 32 layers, 8 Turbo steps.
    "c2": dict(_BIG, n_layers=32,
               segments=[("text", 256), ("target", 64, 64)],
               sigmas=TURBO_SIGMAS),
    # Editing: 256 text + one 64x64 reference + 64x64 target.
    "c3": dict(_BIG, n_layers=32,
               segments=[("text", 256), ("ref", 64, 64), ("target", 64, 64)],
               sigmas=TURBO_SIGMAS),
    # Multi-reference: 512 text + three 64x64 references + 96x96 target.
    "c4": dict(_BIG, n_layers=32,
               segments=[("text", 512), ("ref", 64, 64), ("ref", 64, 64),
                         ("ref", 64, 64), ("target", 96, 96)],
               sigmas=TURBO_SIGMAS),
    # Many references: 512 text + ten 64x64 references + 96x96 target
    # (41472 prefix tokens, 50688 in all; 26.6 GB of KV cache).
    "c5": dict(_BIG, n_layers=32,
               segments=[("text", 512)] + [("ref", 64, 64)] * 10 + [("target", 96, 96)],
               sigmas=TURBO_SIGMAS),
}

# Token layouts (segments only) whose block edges fall off the 64/128/256
# tile boundaries, for mask and attention tests.
RAGGED_LAYOUTS = {
    "ragged": [("text", 37), ("ref", 5, 7), ("text", 3), ("ref", 3, 3), ("target", 9, 11)],
    # ten references of mixed shapes (one a single cell), text between some
    "many_ragged": [("text", 61), ("ref", 9, 13), ("ref", 16, 16), ("text", 5), ("ref", 5, 40),
                    ("ref", 1, 1), ("ref", 33, 7), ("ref", 12, 12), ("text", 2), ("ref", 20, 3),
                    ("ref", 8, 8), ("ref", 3, 50), ("ref", 17, 17), ("target", 19, 23)],
}


def config(name: str, **overrides) -> dict:
    c = dict(CONFIGS[name])
    c.update(overrides)
    c["name"] = name
    return c


def token_counts(cfg: dict):
    """(P, T, S) implied by the segment list (plain counting)."""
    n = 0
    T = 0
    for seg in cfg["segments"]:
        cnt = seg[1] if seg[0] == "text" else seg[1] * seg[2]
        n += cnt
        if seg[0] == "target":
            T = cnt
    return n - T, T, n


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(zlib.crc32(name.encode()),)))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32."""
    return _round_bf16_inplace(np.array(x, dtype=np.float32, copy=True))


def _round_bf16_inplace(a: np.ndarray) -> np.ndarray:
    """Round an owned, contiguous float32 array to bfloat16 in place (ties to
    even): add 0x7FFF plus the kept part's lowest bit, then clear the low 16
    bits."""
    b = a.view(np.uint32)
    keep_lsb = b >> np.uint32(16)
    keep_lsb &= np.uint32(1)
    keep_lsb += np.uint32(0x7FFF)
    b += keep_lsb
    b &= np.uint32(0xFFFF0000)
    return a


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-exact."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (b >> np.uint32(16)).astype(np.uint16)


def _normal(seed, name, shape, fan_in):
    g = _rng(seed, name)
    a = g.standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(1.0 / np.sqrt(fan_in))
    return _round_bf16_inplace(a)


def _global_specs(cfg: dict):
    H, C, Dt = cfg["hidden"], cfg["latent"], cfg["time_dim"]
    return [("t1", "t1", (H, Dt), Dt), ("t2", "t2", (H, H), H), ("mod", "mod", (4 * H, H), H),
            ("so", "so", (H, H), H), ("img_in", "img_in", (H, C), C),
            ("proj_out", "proj_out", (C, H), H)]


def _layer_specs(cfg: dict, l: int):
    H, d, F = cfg["hidden"], cfg["head_dim"], cfg["ffn"]
    return [("qkv", f"l{l}.qkv", (3 * H, H), H), ("q_norm", f"l{l}.q_norm", (d,), d),
            ("k_norm", f"l{l}.k_norm", (d,), d), ("o", f"l{l}.o", (H, H), H),
            ("gate", f"l{l}.gate", (F, H), H), ("up", f"l{l}.up", (F, H), H),
            ("down", f"l{l}.down", (H, F), F)]


def global_weights(cfg: dict, seed: int = 21) -> dict:
    """The weights shared by all layers (see ``make_weights``)."""
    return {key: _normal(seed, name, shape, fan) for key, name, shape, fan in _global_specs(cfg)}


def layer_weights(cfg: dict, l: int, seed: int = 21, workers: int = 1) -> dict:
    """Layer ``l``'s weights (see ``make_weights``); each tensor has its own
    named stream, so the values do not depend on ``workers`` or on which
    other layers are drawn."""
    return layers_weights(cfg, [l], seed, workers)[0]


def layers_weights(cfg: dict, layers, seed: int = 21, workers: int = 1) -> list:
    """Weights of the given layers, drawn by up to ``workers`` threads (one
    tensor per task; NumPy's generators release the GIL while filling)."""
    jobs = [(i, key, name, shape, fan) for i, l in enumerate(layers)
            for key, name, shape, fan in _layer_specs(cfg, l)]
    out = [dict() for _ in layers]
    if workers <= 1:
        for i, key, name, shape, fan in jobs:
            out[i][key] = _normal(seed, name, shape, fan)
        return out
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=workers) as ex:
        futs = [(i, key, ex.submit(_normal, seed, name, shape, fan))
                for i, key, name, shape, fan in jobs]
        for i, key, f in futs:
            out[i][key] = f.result()
    return out


def make_weights(cfg: dict, seed: int = 21, n_layers: int | None = None,
                 workers: int = 1) -> dict:
    """All weights in nn.Linear layout [out, in], bf16-exact float32.

    Global: t1 [H, D_t], t2 [H, H], mod [4H, H], so [H, H], img_in [H, C],
    proj_out [C, H]. Per layer: qkv [3H, H] (q rows, then k, then v),
    q_norm [d], k_norm [d], o [H, H], gate [F, H], up [F, H], down [H, F].
    """
    L = cfg["n_layers"] if n_layers is None else n_layers
    W = global_weights(cfg, seed)
    W["layers"] = layers_weights(cfg, range(L), seed, workers)
    return W


def bits_crc(bits: dict) -> int:
    """CRC-32 of a dict of bf16 bit-pattern arrays, in key order (a
    fingerprint to tell whether stored expected values were made from the
    same weights)."""
    c = 0
    for k in sorted(bits):
        c = zlib.crc32(np.ascontiguousarray(bits[k]).tobytes(), c)
    return c


def weights_crc(tensors: dict) -> int:
    """``bits_crc`` of bf16-exact float32 weights."""
    return bits_crc({k: bf16_bits(v) for k, v in tensors.items()})


def make_inputs(cfg: dict, seed: int = 21) -> dict:
    """Seeded N(0,1) float32 inputs.

    ``text_hidden`` [n_text, H]; ``x0`` [T, C] (initial target latent);
    for reference tokens either ``ref_hidden`` [n_ref, H] drawn directly
    (configs with ``prefix_direct``) or ``ref_latents`` [n_ref, C] that the
    caller embeds with img_in. ``prefix_kind`` gives each prefix row's origin
    in sequence order (0 text, 1 reference).
    """
    H, C = cfg["hidden"], cfg["latent"]
    n_text = sum(s[1] for s in cfg["segments"] if s[0] == "text")
    n_ref = sum(s[1] * s[2] for s in cfg["segments"] if s[0] == "ref")
    T = sum(s[1] * s[2] for s in cfg["segments"] if s[0] == "target")
    kind = []
    for s in cfg["segments"]:
        if s[0] == "text":
            kind += [0] * s[1]
        elif s[0] == "ref":
            kind += [1] * (s[1] * s[2])
    out = {
        "text_hidden": _rng(seed, "prefix").standard_normal((n_text, H), dtype=np.float32),
        "x0": _rng(seed, "x0").standard_normal((T, C), dtype=np.float32),
        "prefix_kind": np.asarray(kind, dtype=np.int8),
    }
    if cfg.get("prefix_direct"):
        out["ref_hidden"] = _rng(seed, "ref_hidden").standard_normal((n_ref, H), dtype=np.float32)
    else:
        out["ref_latents"] = _rng(seed, "ref_latents").standard_normal((n_ref, C), dtype=np.float32)
    return out


def latent_stats(C: int = 64, seed: int = 21):
    """Synthetic per-channel VAE latent statistics (mean [C], std [C]) standing
    in for a checkpoint's: mean N(0, 0.5²), std exp(N(0, 0.3²)), float32."""
    mean = (0.5 * _rng(seed, "latents_mean").standard_normal(C)).astype(np.float32)
    std = np.exp(0.3 * _rng(seed, "latents_std").standard_normal(C)).astype(np.float32)
    return mean, std


def interleave_prefix(kind: np.ndarray, text_rows: np.ndarray, ref_rows: np.ndarray) -> np.ndarray:
    """Place text rows and reference rows in sequence order (row copies only)."""
    out = np.empty((len(kind), text_rows.shape[1]), dtype=np.float32)
    out[kind == 0] = text_rows
    out[kind == 1] = ref_rows
    return out
