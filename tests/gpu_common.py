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
