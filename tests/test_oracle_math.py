"""Oracle pins: the primitive operations against independent library
routines (torch CPU float64) and closed forms."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O

rng = np.random.default_rng(1234)


def t64(a):
    return torch.from_numpy(np.asarray(a, np.float64))


def test_layernorm_matches_torch():
    x = rng.standard_normal((5, 37)) * 3 + 1.5
    want = F.layer_norm(t64(x), (37,), eps=1e-6).numpy()
    assert np.abs(O.layernorm(x, 1e-6) - want).max() < 1e-13


def test_rmsnorm_matches_torch():
    x = rng.standard_normal((4, 3, 128))
    w = rng.standard_normal(128) * 0.1
    want = F.rms_norm(t64(x), (128,), weight=t64(1.0 + w), eps=1e-6).numpy()
    assert np.abs(O.rmsnorm(x, w, 1e-6) - want).max() < 1e-13


def test_silu_matches_torch():
    x = rng.standard_normal(1000) * 6
    assert np.abs(O.silu(x) - F.silu(t64(x)).numpy()).max() < 1e-14


@pytest.mark.parametrize("ids", [[-1, -1, 0, 0, 0, 0, -1, 1, 1, 1, 1],
                                 [-1] * 5 + [0] * 9 + [-1] * 3 + [1] * 16])
def test_masked_attention_matches_sdpa(ids):
    S, nh, d = len(ids), 3, 16
    q, k, v = (rng.standard_normal((S, nh, d)) for _ in range(3))
    allowed = O.block_causal_mask(ids)
    got = O.masked_attention(q, k, v, allowed, row_block=4)
    want = F.scaled_dot_product_attention(
        t64(q).transpose(0, 1), t64(k).transpose(0, 1), t64(v).transpose(0, 1),
        attn_mask=torch.from_numpy(allowed)).transpose(0, 1).reshape(S, nh * d).numpy()
    assert np.abs(got - want).max() < 1e-13


def test_masked_keys_get_exactly_zero_weight():
    # value rows of masked keys are huge; they must not leak at all
    ids = [-1, -1, 0, 0, -1]
    S, nh, d = 5, 1, 4
    q = rng.standard_normal((S, nh, d))
    k = rng.standard_normal((S, nh, d))
    v = np.zeros((S, nh, d))
    v[4] = 1e30                      # key 4 is visible only to query 4
    out = O.masked_attention(q, k, v, O.block_causal_mask(ids))
    assert np.all(out[:4] == 0.0)


def test_rope_identity_at_zero_and_norm_preserving():
    dims = O.DitDims(hidden=256, n_heads=2, head_dim=128, ffn=8, n_layers=1)
    x = rng.standard_normal((6, 2, 128))
    ang0 = O.rope_angles(np.zeros((6, 3)), dims)
    assert np.array_equal(O.rope_rotate(x, ang0), x)
    coords = rng.integers(-40, 40, size=(6, 3))
    y = O.rope_rotate(x, O.rope_angles(coords, dims))
    # each interleaved pair keeps its length
    assert np.allclose(y[..., 0::2] ** 2 + y[..., 1::2] ** 2,
                       x[..., 0::2] ** 2 + x[..., 1::2] ** 2, atol=1e-12)


def test_rope_equals_complex_multiplication():
    """Pair (x0, x1) as the complex number x0 + i x1, multiplied by e^{iθ}."""
    dims = O.DitDims(hidden=256, n_heads=2, head_dim=128, ffn=8, n_layers=1)
    x = rng.standard_normal((7, 2, 128))
    coords = rng.integers(-30, 30, size=(7, 3))
    ang = O.rope_angles(coords, dims)
    z = torch.view_as_complex(t64(x).reshape(7, 2, 64, 2).contiguous())
    rot = torch.polar(torch.ones_like(t64(ang)), t64(ang))[:, None, :]
    want = torch.view_as_real(z * rot).reshape(7, 2, 128).numpy()
    assert np.abs(O.rope_rotate(x, ang) - want).max() < 1e-12


def test_rope_relative_position():
    """<R(a)q, R(b)k> depends on a and b only through a - b (per axis)."""
    dims = O.DitDims(hidden=256, n_heads=2, head_dim=128, ffn=8, n_layers=1)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    a = np.array([[3, -7, 11]])
    b = np.array([[1, 5, -2]])
    shift = np.array([[9, -4, 6]])

    def dot(pa, pb):
        return float(np.sum(O.rope_rotate(q, O.rope_angles(pa, dims)) *
                            O.rope_rotate(k, O.rope_angles(pb, dims))))
    assert abs(dot(a, b) - dot(a + shift, b + shift)) < 1e-12
    assert abs(dot(a, b) - dot(a - b, np.zeros((1, 3)))) < 1e-12


def test_rope_axis_split_lab_toy_and_production():
    # toy dims (0, 2, 2): pair 0 turns by the row coordinate, pair 1 by the
    # column coordinate, both at frequency base^0 = 1
    toy = O.DitDims(hidden=8, n_heads=2, head_dim=4, ffn=16, n_layers=2, rope_dims=(0, 2, 2))
    ang = O.rope_angles(np.array([[5, -1, 2]]), toy)
    assert ang.tolist() == [[-1.0, 2.0]]
    # production split (16, 56, 56): the first pair of each axis turns by the
    # raw coordinate (frame pair 0, height pair 8, width pair 36); the
    # frequencies inside an axis follow the standard RoPE base^(-2j/d_axis)
    prod = O.DitDims(hidden=4096, n_heads=32, head_dim=128, ffn=8, n_layers=1)
    ang = O.rope_angles(np.array([[3.0, 5.0, 7.0]]), prod)[0]
    assert ang.shape == (64,)
    assert ang[0] == 3.0 and ang[8] == 5.0 and ang[36] == 7.0
    assert math.isclose(ang[1], 3.0 * 10000 ** (-2 / 16), rel_tol=1e-15)
    assert math.isclose(ang[35], 5.0 * 10000 ** (-54 / 56), rel_tol=1e-15)
    assert math.isclose(ang[63], 7.0 * 10000 ** (-54 / 56), rel_tol=1e-15)


def test_timestep_embedding_closed_forms():
    e0 = O.timestep_embedding(0.0, 8)
    assert e0.tolist() == [1, 1, 1, 1, 0, 0, 0, 0]          # cosine half first
    e = O.timestep_embedding(850.0, 256)
    assert abs(np.sum(e ** 2) - 128.0) < 1e-10
    # first frequency is 1: entries cos(t), sin(t)
    assert e[0] == math.cos(850.0) and e[128] == math.sin(850.0)


def test_standardize_closed_forms_and_inverse():
    """[1A] standardize and [6B] unstandardize: the channel mean maps to 0 and
    mean + std to 1, channels are independent, and the two are inverses;
    checked against hand values, not by re-running the formula."""
    mean = np.array([0.5, -2.0, 0.0, 3.0])
    std = np.array([2.0, 0.25, 1.0, 4.0])
    np.testing.assert_array_equal(O.standardize(mean[None, :], mean, std), np.zeros((1, 4)))
    np.testing.assert_array_equal(O.standardize((mean + std)[None, :], mean, std), np.ones((1, 4)))
    z = np.array([[1.5, -1.5, 7.0, -1.0]])
    np.testing.assert_allclose(O.standardize(z, mean, std), [[0.5, 2.0, 7.0, -1.0]])
    np.testing.assert_allclose(O.unstandardize([[0.5, 2.0, 7.0, -1.0]], mean, std), z)
    rng = np.random.default_rng(1)
    zz = rng.standard_normal((9, 4)) * 3
    np.testing.assert_allclose(O.unstandardize(O.standardize(zz, mean, std), mean, std), zz,
                               rtol=0, atol=1e-12)
    # changing one channel of the input changes only that channel
    z2 = zz.copy()
    z2[:, 2] += 1.0
    d = O.standardize(z2, mean, std) - O.standardize(zz, mean, std)
    assert np.all(d[:, [0, 1, 3]] == 0) and np.allclose(d[:, 2], 1.0)
