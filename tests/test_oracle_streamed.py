"""The oracle with its per-layer weights supplied on demand (a callable, as
the deep-model stored values are made) computes bit for bit what it computes
from a list of layers; and the seeded generators the GPU tests and the bench
draw from agree with the printed schedule and with themselves."""
import json
import os

import numpy as np
import pytest

import oracle as O
from diffusion_transformer_amd import synth
from oracle_inputs import setup

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "lab_toy.json")))


@pytest.mark.parametrize("name", ["c0w", "c1"])
def test_layer_streamed_weights_are_bitwise_the_same(name):
    cfg, W, I, dims, lay, pre = setup(name)
    sig = cfg["sigmas"] if name == "c0w" else cfg["sigmas"][:3]
    calls = []

    def layer(l):
        calls.append(l)
        return W["layers"][l]
    Ws = dict(W, layers=layer)
    a = O.run_loop(W, dims, lay, pre, I["x0"], sig, use_cache=True)
    b = O.run_loop(Ws, dims, lay, pre, I["x0"], sig, use_cache=True)
    for ra, rb in zip(a, b):
        assert np.array_equal(ra["v"], rb["v"]) and np.array_equal(ra["x_next"], rb["x_next"])
    assert calls == list(range(dims.n_layers)) * (len(sig) - 1)


def test_synth_turbo_sigmas_are_the_printed_table():
    """The schedule every GPU test and the bench use is the page's table."""
    assert list(synth.TURBO_SIGMAS) == GOLD["turbo_sigmas"]["value"]
    assert synth.CONFIGS["c2"]["sigmas"] == synth.TURBO_SIGMAS


def test_per_layer_draws_match_whole_model_draws():
    cfg = synth.config("c0w")
    W = synth.make_weights(cfg)
    par = synth.make_weights(cfg, workers=4)
    one = synth.layer_weights(cfg, 1)
    for k, v in one.items():
        assert np.array_equal(v, W["layers"][1][k]) and np.array_equal(v, par["layers"][1][k])
    assert synth.weights_crc(W["layers"][0]) == synth.weights_crc(par["layers"][0])
    assert synth.weights_crc(W["layers"][0]) != synth.weights_crc(W["layers"][1])


def test_round_bf16_ties_to_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 1.0 + 2 ** -8 + 2 ** -20,
                  3.0e38, 0.0], np.float32)
    want = np.array([1.0, 1.0 + 2 ** -6, -1.0, 1.0 + 2 ** -7, 226.0 * 2.0 ** 120, 0.0], np.float32)
    assert np.array_equal(synth.round_bf16(x), want)
