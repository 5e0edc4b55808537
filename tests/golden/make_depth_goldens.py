"""Writes the stored expected values of the deep-model parity tests
(``depth_<workload>_L<layers>.npz`` beside this file).

It calls only the fp64 oracle (``oracle/``) and the seeded generators
(``diffusion_transformer_amd.synth``, through ``tests/oracle_inputs.py``):
for each job it draws the workload's weights and inputs, runs the oracle's
sampler loop over the 8-step Turbo schedule (step 1 extract, steps 2..8
cached against the prefix K/V of step 1) and stores

- ``rows``: the sampled target rows (a seeded eighth of them, plus the first
  and the last row);
- ``v``: v_θ of every step on those rows, float32 [steps, rows, C];
- ``v_absmax``: max |v_θ| of every step over all target rows (float64);
- ``x_final``: the latent after the last Euler step, all rows, float32;
- ``x_absmax``: max |x| of the latent after every step (float64);
- ``layer_crc`` / ``global_crc``: CRC-32 of each layer's and of the shared
  bf16 weights, so a test can tell that it drew the same weights;
- ``meta``: a JSON string with the workload, depth, seed and sigmas.

The deep model's weights are held as bf16 bit patterns (17.2 GB for the
32-layer model) and handed to the oracle one layer at a time.

Usage: ``python tests/golden/make_depth_goldens.py c2 c3 c4`` (each name may
carry its depth as ``c3:2``; the defaults are c2 at 32 layers, c3 and c4 at
2 layers).
"""
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
TESTS = os.path.dirname(HERE)
ROOT = os.path.dirname(TESTS)
for p in (ROOT, TESTS):
    if p not in sys.path:
        sys.path.insert(0, p)

import oracle as O  # noqa: E402
from diffusion_transformer_amd import synth  # noqa: E402
from oracle_inputs import dims_of, oracle_prefix  # noqa: E402

DEFAULT_DEPTH = {"c2": 32, "c3": 2, "c4": 2}
SEED = 21
ROW_SEED = 8


def golden_path(name: str, n_layers: int) -> str:
    return os.path.join(HERE, f"depth_{name}_L{n_layers}.npz")


def sample_rows(T: int) -> np.ndarray:
    rows = np.random.default_rng(ROW_SEED).choice(T, T // 8, replace=False)
    return np.unique(np.concatenate([[0, T - 1], rows]))


def _bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def make(name: str, n_layers: int, workers: int = 8) -> str:
    t0 = time.time()
    cfg = synth.config(name)
    cfg["n_layers"] = n_layers
    W = synth.global_weights(cfg, SEED)
    store, crcs = [], []
    for l0 in range(0, n_layers, 4):
        chunk = synth.layers_weights(cfg, range(l0, min(n_layers, l0 + 4)), SEED, workers)
        for Lw in chunk:
            crcs.append(synth.weights_crc(Lw))
            store.append({k: synth.bf16_bits(v) for k, v in Lw.items()})
        print(f"[{name}] weights of layers < {l0 + len(chunk)} drawn ({time.time() - t0:.0f} s)",
              flush=True)
    W["layers"] = lambda l: {k: _bits_to_f32(b) for k, b in store[l].items()}
    I = synth.make_inputs(cfg, SEED)
    dims = dims_of(cfg)
    lay = O.build_layout(cfg["segments"])
    pre = oracle_prefix(cfg, W, I)
    sig = cfg["sigmas"]
    rows = sample_rows(lay.T)
    x = np.asarray(I["x0"], np.float64)
    cache = None
    v_rows, v_max, x_max = [], [], []
    for k in range(len(sig) - 1):
        if k == 0:
            out = O.forward_extract(W, dims, lay, pre, x, sig[k])
            cache = out["cache"]
        else:
            out = O.forward_cached(W, dims, lay, cache, x, sig[k])
        x = O.euler_step(x, out["v"], sig[k], sig[k + 1])
        v_rows.append(out["v"][rows])
        v_max.append(np.abs(out["v"]).max())
        x_max.append(np.abs(x).max())
        print(f"[{name}] step {k} ({'extract' if k == 0 else 'cached'}) done, "
              f"max|v| {v_max[-1]:.4f} ({time.time() - t0:.0f} s)", flush=True)
    meta = {"workload": name, "n_layers": n_layers, "seed": SEED, "sigmas": list(sig),
            "row_seed": ROW_SEED, "P": lay.P, "T": lay.T,
            "loop": "step 1 extract, steps 2.. cached (oracle.forward_extract / forward_cached), "
                    "Euler after every step",
            "seconds": round(time.time() - t0, 1)}
    path = golden_path(name, n_layers)
    np.savez_compressed(path, rows=rows, v=np.asarray(v_rows, np.float32),
                        v_absmax=np.asarray(v_max), x_final=x.astype(np.float32),
                        x_absmax=np.asarray(x_max),
                        layer_crc=np.asarray(crcs, np.uint32),
                        global_crc=np.uint32(synth.weights_crc(
                            {k: v for k, v in W.items() if k != "layers"})),
                        meta=np.asarray(json.dumps(meta)))
    print(f"[{name}] wrote {path} in {time.time() - t0:.0f} s", flush=True)
    return path


if __name__ == "__main__":
    for arg in (sys.argv[1:] or ["c3", "c4", "c2"]):
        nm, _, depth = arg.partition(":")
        make(nm, int(depth) if depth else DEFAULT_DEPTH[nm])
