"""Oracle pins: the invariants the pages state for the cached step, on the
lab-scale toy (c0) and its head_dim-128 twin (c0w), in float64."""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from oracle_inputs import setup

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "lab_toy.json")))


@pytest.fixture(scope="module", params=["c0", "c0w"])
def case(request):
    return setup(request.param)


def test_cached_equals_recompute(case):
    cfg, W, I, dims, lay, pre = case
    sig = cfg["sigmas"]
    a = O.run_loop(W, dims, lay, pre, I["x0"], sig, use_cache=True)
    b = O.run_loop(W, dims, lay, pre, I["x0"], sig, use_cache=False)
    assert [r["mode"] for r in a] == ["extract"] + ["cached"] * (len(sig) - 2)
    assert all(r["mode"] == "extract" for r in b)
    thr = GOLD["cached_vs_recompute_threshold"]["value"]
    for ra, rb in zip(a, b):
        dv = np.abs(ra["v"] - rb["v"]).max()
        assert dv < 1e-13 < thr
    assert np.abs(a[-1]["x_next"] - b[-1]["x_next"]).max() < 1e-13


def test_prefix_kv_independent_of_sigma(case):
    cfg, W, I, dims, lay, pre = case
    x0 = I["x0"]
    e1 = O.forward_extract(W, dims, lay, pre, x0, 1.0)
    x1 = O.euler_step(x0, e1["v"], 1.0, cfg["sigmas"][1])
    e2 = O.forward_extract(W, dims, lay, pre, x1, cfg["sigmas"][1])
    for (k1, v1), (k2, v2) in zip(e1["cache"], e2["cache"]):
        assert k1.shape == (lay.P, dims.n_heads, dims.head_dim)
        assert np.abs(k1 - k2).max() <= 1e-15
        assert np.abs(v1 - v2).max() <= 1e-15


def test_prefix_kv_drifts_without_causal_condition(case):
    cfg, W, I, dims, lay, pre = case
    x0 = I["x0"]
    e1 = O.forward_extract(W, dims, lay, pre, x0, 1.0, causal_condition=False)
    x1 = O.euler_step(x0, e1["v"], 1.0, cfg["sigmas"][1])
    e2 = O.forward_extract(W, dims, lay, pre, x1, cfg["sigmas"][1], causal_condition=False)
    for (k1, _), (k2, _) in zip(e1["cache"], e2["cache"]):
        assert np.abs(k1 - k2).max() > 1e-6


def test_isolation(case):
    cfg, W, I, dims, lay, pre = case
    base = O.forward_extract(W, dims, lay, pre, I["x0"], 1.0)["h_final"]
    pt = O.forward_extract(W, dims, lay, pre, I["x0"], 1.0, perturb=[(7, 0, 0.5)])["h_final"]
    leak = np.abs(pt - base)[:7].max()
    assert leak == GOLD["prefix_leak_on_target_perturb"]["value"]
    assert np.abs(pt - base)[7:].max() > 0
    pr = O.forward_extract(W, dims, lay, pre, I["x0"], 1.0, perturb=[(5, 0, 0.5)])["h_final"]
    d = np.abs(pr - base).max(axis=1)
    assert (d[2:6] > 0).all()               # the reference block is bidirectional
    assert d[0] == 0.0 and d[1] == 0.0      # earlier text is causal


def test_velocity_depends_on_sigma(case):
    cfg, W, I, dims, lay, pre = case
    vs = [O.forward_extract(W, dims, lay, pre, I["x0"], s)["v"] for s in (1.0, 0.85, 0.45)]
    assert np.abs(vs[0] - vs[1]).max() > 1e-6
    assert np.abs(vs[1] - vs[2]).max() > 1e-6
    assert np.abs(vs[0] - vs[2]).max() > 1e-6


def test_t0_row_fixed_and_rows_differ_only_for_targets(case):
    cfg, W, I, dims, lay, pre = case
    c1 = O.conditioning(W, dims, 1.0)
    c2 = O.conditioning(W, dims, 0.85)
    assert np.abs(c1["row_0"] - c2["row_0"]).max() == GOLD["t0_row_step_diff"]["value"]
    assert np.abs(c1["row_t"] - c2["row_t"]).max() > 0
    assert c1["row_t"].shape == (4 * dims.hidden,)


def test_modulation_parameter_count():
    H = 4096
    assert H * (4 * H) == GOLD["modulation_params_h4096"]["value"]
    from diffusion_transformer_amd import synth
    c = synth.config("c1")
    assert (4 * c["hidden"], c["hidden"]) == (16384, 4096)


def test_token_counts(case):
    cfg, W, I, dims, lay, pre = case
    e = O.forward_extract(W, dims, lay, pre, I["x0"], 1.0)
    assert e["h_final"].shape[0] == GOLD["tokens_per_step_lab"]["extract"]
    assert e["v"].shape[0] == GOLD["tokens_per_step_lab"]["cached"]


def test_zero_gates_reduce_to_closed_form(case):
    """With the gate rows of the shared modulation zeroed, tanh(0) = 0 turns
    every block into the identity on the residual stream, so v_θ equals
    (LN(x W_inᵀ)·(1+scale_out)) W_outᵀ. Evaluated here with torch routines."""
    cfg, W, I, dims, lay, pre = case
    H = dims.hidden
    W2 = dict(W)
    mod = np.array(W["mod"], dtype=np.float64)
    mod[H:2 * H] = 0.0
    mod[3 * H:4 * H] = 0.0
    W2["mod"] = mod
    v = O.forward_extract(W2, dims, lay, pre, I["x0"], 0.85)["v"]
    te = torch.from_numpy(O.timestep_embedding(850.0, dims.time_dim))
    f = lambda n: torch.from_numpy(np.asarray(W[n], np.float64))
    temb = F.linear(F.silu(F.linear(te, f("t1"))), f("t2"))
    sc = F.linear(F.silu(temb), f("so"))
    h = F.linear(torch.from_numpy(I["x0"].astype(np.float64)), f("img_in"))
    want = F.linear(F.layer_norm(h, (H,), eps=1e-6) * (1 + sc), f("proj_out")).numpy()
    assert np.abs(v - want).max() < 1e-12


def test_cached_rows_one_layer_agrees():
    cfg, W, I, dims, lay, pre = setup("c0w", n_layers=1)
    e = O.forward_extract(W, dims, lay, pre, I["x0"], 1.0)
    c = O.forward_cached(W, dims, lay, e["cache"], I["x0"], 0.85)
    rows = [0, 2, 3]
    r = O.cached_rows_one_layer(W, dims, lay, pre, I["x0"], 0.85, rows)
    assert np.abs(r - c["v"][rows]).max() < 1e-13
