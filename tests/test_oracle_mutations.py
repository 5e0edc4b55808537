"""The oracle's pins catch planted mistakes: each test plants one plausible
slip in the oracle (on the CPU, by patching one of its functions or handing
it a transposed operand) and checks that the independent torch composition
of the step then disagrees with it, while it agrees without the slip."""
import numpy as np
import pytest

import oracle as O
import oracle.dit_oracle as DO
from oracle_inputs import setup
from test_oracle_torch_composition import torch_forward


def _gap(W_oracle, W_ref, name="c0w", sigma=0.85):
    cfg, W, I, dims, lay, pre = setup(name)
    got = O.forward_extract(W_oracle(W), dims, lay, pre, I["x0"], sigma)["v"]
    want = torch_forward(W_ref(W), dims, lay.image_ids, lay.coords, lay.target_mask, pre, I["x0"],
                         sigma)
    return np.abs(got - want).max() / np.abs(want).max()


def same(W):
    return W


def test_unplanted_oracle_agrees():
    assert _gap(same, same) < 1e-12


def test_transposed_output_projection_is_caught():
    def transposed_o(W):
        W2 = dict(W)
        W2["layers"] = [dict(L, o=np.ascontiguousarray(np.asarray(L["o"]).T)) for L in W["layers"]]
        return W2
    assert _gap(transposed_o, same) > 1e-3


def test_rope_sign_is_caught(monkeypatch):
    good = DO.rope_rotate
    monkeypatch.setattr(DO, "rope_rotate", lambda x, ang: good(x, -np.asarray(ang)))
    assert _gap(same, same) > 1e-3


@pytest.mark.parametrize("order", [(1, 0, 2, 3), (2, 1, 0, 3), (0, 3, 2, 1)],
                         ids=["scale1<->gate1", "scale1<->scale2", "gate1<->gate2"])
def test_modulation_chunk_order_is_caught(monkeypatch, order):
    good = DO._split_rows

    def swapped(row, H):
        parts = good(row, H)
        return tuple(parts[i] for i in order)
    monkeypatch.setattr(DO, "_split_rows", swapped)
    assert _gap(same, same) > 1e-3


def test_timestep_frequency_is_caught(monkeypatch):
    good = DO.timestep_embedding
    monkeypatch.setattr(DO, "timestep_embedding",
                        lambda t, D, base=10000.0: good(t, D, base * 2.0))
    assert _gap(same, same) > 1e-6


def test_mask_rule_is_caught(monkeypatch):
    """A mask that lets text see the whole image block after it (the
    bidirectional rule applied to text tokens too) is caught."""
    def leaky(image_ids, rows=None):
        ids = np.asarray(image_ids)
        S = len(ids)
        qi = np.arange(S) if rows is None else np.asarray(rows)
        kj = np.arange(S)
        return (qi[:, None] >= kj[None, :]) | (ids[qi][:, None] == ids[None, :])
    monkeypatch.setattr(DO, "block_causal_mask", leaky)
    assert _gap(same, same) > 1e-6
