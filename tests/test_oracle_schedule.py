"""Oracle pins: the Turbo schedule, t = 1000σ and the Euler update."""
import json
import os

import numpy as np

import oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "lab_toy.json")))


def test_turbo_table_and_deltas():
    s = np.array(O.TURBO_SIGMAS)
    assert s.tolist() == GOLD["turbo_sigmas"]["value"]
    d = s[:-1] - s[1:]
    assert np.abs(d - np.array(GOLD["turbo_delta_sigma_abs"]["value"])).max() < 5e-7
    assert abs(d.sum() - GOLD["turbo_delta_sigma_abs"]["sum"]) < 1e-12


def test_t_is_1000_sigma():
    W = {"t1": np.zeros((8, 8)), "t2": np.zeros((8, 8)), "mod": np.zeros((32, 8)),
         "so": np.zeros((8, 8))}
    dims = O.DitDims(hidden=8, n_heads=2, head_dim=4, ffn=16, n_layers=2, time_dim=8,
                     rope_dims=(0, 2, 2))
    g = GOLD["lab_sigmas_and_t"]
    for s, t in zip(g["sigmas"], g["t"]):
        assert O.conditioning(W, dims, s)["t"] == t


def test_euler_closed_forms():
    rng = np.random.default_rng(3)
    x0 = rng.standard_normal((4, 64))
    v = rng.standard_normal((4, 64))
    x = x0.copy()
    for k in range(8):
        x = O.euler_step(x, v, O.TURBO_SIGMAS[k], O.TURBO_SIGMAS[k + 1])
    # constant velocity: the deltas sum to sigma_N - sigma_0 = -1
    assert np.abs(x - (x0 - v)).max() < 1e-14
    assert np.array_equal(O.euler_step(x0, np.zeros_like(x0), 1.0, 0.5), x0)
    one = O.euler_step(x0, v, 0.85, 0.45)
    assert np.abs(one - (x0 - 0.4 * v)).max() < 1e-15


def _toy():
    import numpy as np
    from oracle_inputs import setup
    cfg, W, I, dims, lay, pre = setup("c0")
    return W, dims, lay, pre, I["x0"], np


def test_general_schedule_loop():
    """A 12-step linear schedule (not Turbo): the cached loop equals full
    recompute to fp64 rounding (the pages' 2.22e-16 agreement, here at every
    step), and the latent is x0 plus the sum of Δσ·v over the steps."""
    W, dims, lay, pre, x0, np = _toy()
    sig = tuple(np.linspace(1.0, 0.0, 13))
    rc = O.run_loop(W, dims, lay, pre, x0, sig, use_cache=True)
    rr = O.run_loop(W, dims, lay, pre, x0, sig, use_cache=False)
    assert [r["mode"] for r in rc] == ["extract"] + ["cached"] * 11
    for a, b in zip(rc, rr):
        assert np.max(np.abs(a["v"] - b["v"])) < 1e-12
    total = np.asarray(x0, np.float64) + sum((sig[k + 1] - sig[k]) * rc[k]["v"] for k in range(12))
    assert np.max(np.abs(rc[-1]["x_next"] - total)) < 1e-12


def test_loop_without_causal_conditioning():
    """[3B] §4: without t = 0 conditioning the prefix follows t, so the
    cached loop is refused; at t = 0 (σ = 0) both conditionings coincide
    exactly, and at σ = 1 they differ."""
    W, dims, lay, pre, x0, np = _toy()
    import pytest
    with pytest.raises(ValueError):
        O.run_loop(W, dims, lay, pre, x0, (1.0, 0.5), use_cache=True, causal_condition=False)
    a = O.run_loop(W, dims, lay, pre, x0, (0.0, -0.25), use_cache=False, causal_condition=False)
    b = O.run_loop(W, dims, lay, pre, x0, (0.0, -0.25), use_cache=False, causal_condition=True)
    assert np.array_equal(a[0]["v"], b[0]["v"])
    c = O.run_loop(W, dims, lay, pre, x0, (1.0, 0.5), use_cache=False, causal_condition=False)
    d = O.run_loop(W, dims, lay, pre, x0, (1.0, 0.5), use_cache=False, causal_condition=True)
    assert np.max(np.abs(c[0]["v"] - d[0]["v"])) > 1e-6
