"""Helpers shared by the GPU parity tests (test infrastructure)."""
import sys

import numpy as np

import oracle as O
from diffusion_transformer_amd import synth


def rel_err(got, ref):
    """max |got - ref| / max |ref| over the whole tensor."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def bf16_round_np(a):
    return synth.round_bf16(np.asarray(a, np.float32))


def cache_views(cache_i16, L, nh, cap, d=128):
    """(K [L, nh, cap, d], Vt [L, nh, d, cap]) int16 views of a cache buffer."""
    k = cache_i16[: L * nh * cap * d].view(L, nh, cap, d)
    v = cache_i16[L * nh * cap * d: 2 * L * nh * cap * d].view(L, nh, d, cap)
    return k, v


def i16_to_f32(t):
    """bf16 bits held in an int16 tensor -> float32 numpy."""
    a = t.cpu().numpy().astype(np.int16).view(np.uint16).astype(np.uint32) << 16
    return a.view(np.float32)


def synth_weights_on_device(cfg, dev, seed=21, workers=16, n_layers=None):
    """The seeded host weights of ``synth`` (the ones the oracle and the
    stored expected values use), drawn layer by layer on ``workers`` threads
    and uploaded as bf16 without keeping the host copies. Returns
    (device weight dict for ``DitRuntime(on_device=True)``, per-layer CRC-32
    of the bf16 bits, CRC-32 of the shared weights)."""
    from concurrent.futures import ThreadPoolExecutor

    import torch
    from diffusion_transformer_amd.runtime import GLOBAL_KEYS, LAYER_KEYS

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    Lc = cfg["n_layers"] if n_layers is None else n_layers
    G = synth.global_weights(cfg, seed)
    gbits = {k: synth.bf16_bits(v) for k, v in G.items()}
    out = {k: up(gbits[k]) for k in GLOBAL_KEYS}
    for k in LAYER_KEYS:
        out[k] = []

    def one(l):
        bits = {k: synth.bf16_bits(v) for k, v in synth.layer_weights(cfg, l, seed).items()}
        return bits, synth.bits_crc(bits)

    crcs = []
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for l0 in range(0, Lc, workers):
            for bits, crc in ex.map(one, range(l0, min(Lc, l0 + workers))):
                crcs.append(crc)
                for k in LAYER_KEYS:
                    out[k].append(up(bits[k]))
            say(f"  weights of layers < {min(Lc, l0 + workers)} drawn and uploaded")
    return out, crcs, synth.bits_crc(gbits)


def split_cases(shapes, splits=(0, 2, 4)):
    """(shape..., splits) cases the split-K path takes: no split, or a split
    count that divides the K / 64 stages (K is each shape's third entry)."""
    return [(*s, k) for s in shapes for k in splits if k == 0 or (s[2] // 64) % k == 0]


def seq_len(segments):
    """Tokens of a layout: ("text", n) counts n, ("ref" | "target", h, w)
    counts h * w."""
    return sum(s[1] if s[0] == "text" else s[1] * s[2] for s in segments)
