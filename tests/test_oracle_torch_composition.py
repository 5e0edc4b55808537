"""Oracle pin: the whole extract/cached step against a second, independent
composition of torch library routines (F.linear, F.layer_norm, F.rms_norm,
complex-multiplication RoPE, F.scaled_dot_product_attention with a boolean
mask, F.silu), float64 on the CPU. It catches transposed operands, wrong
head splits, a wrong RoPE sign and misplaced modulation chunks, which the
invariant tests cannot see."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from oracle_inputs import setup


def torch_forward(W, dims, ids, coords, target_mask, pre, x, sigma):
    H, nh, d = dims.hidden, dims.n_heads, dims.head_dim
    f = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    half = dims.time_dim // 2
    t = 1000.0 * sigma
    fr = torch.exp(-np.log(dims.rope_base) * torch.arange(half, dtype=torch.float64) * 2 / dims.time_dim)
    emb = lambda tv: torch.cat([torch.cos(tv * fr), torch.sin(tv * fr)])
    temb = lambda tv: F.linear(F.silu(F.linear(emb(tv), f(W["t1"]))), f(W["t2"]))
    mod_t = F.linear(F.silu(temb(t)), f(W["mod"])).reshape(4, H)
    mod_0 = F.linear(F.silu(temb(0.0)), f(W["mod"])).reshape(4, H)
    sel = torch.from_numpy(np.asarray(target_mask))[:, None, None]
    mods = torch.where(sel, mod_t[None], mod_0[None])           # [S, 4, H]
    h = torch.cat([f(pre), F.linear(f(x), f(W["img_in"]))])
    S = h.shape[0]
    # RoPE angles per axis: theta_j = base^(-2j/d_axis), pairs axis by axis
    freqs = [dims.rope_base ** (-torch.arange(0, da, 2, dtype=torch.float64) / da)
             for da in dims.rope_dims]
    c = f(coords)
    ang = torch.cat([c[:, a:a + 1] * freqs[a][None, :] for a in range(3)], dim=1)
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]          # [S, 1, d/2]

    def rope(z):
        zc = torch.view_as_complex(z.reshape(S, nh, d // 2, 2).contiguous())
        return torch.view_as_real(zc * rot).reshape(S, nh, d)

    ids_t = torch.from_numpy(np.asarray(ids))
    i = torch.arange(S)
    mask = (i[:, None] >= i[None, :]) | ((ids_t[:, None] == ids_t[None, :]) & (ids_t[:, None] >= 0))
    for L in W["layers"]:
        x1 = F.layer_norm(h, (H,), eps=dims.eps) * (1 + mods[:, 0])
        q, k, v = F.linear(x1, f(L["qkv"])).split(H, dim=-1)
        q = rope(F.rms_norm(q.reshape(S, nh, d), (d,), weight=1 + f(L["q_norm"]), eps=dims.eps))
        k = rope(F.rms_norm(k.reshape(S, nh, d), (d,), weight=1 + f(L["k_norm"]), eps=dims.eps))
        v = v.reshape(S, nh, d)
        o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1),
                                           v.transpose(0, 1), attn_mask=mask)
        o = o.transpose(0, 1).reshape(S, H)
        h = h + torch.tanh(mods[:, 1]) * F.linear(o, f(L["o"]))
        x2 = F.layer_norm(h, (H,), eps=dims.eps) * (1 + mods[:, 2])
        m = F.linear(F.silu(F.linear(x2, f(L["gate"]))) * F.linear(x2, f(L["up"])), f(L["down"]))
        h = h + torch.tanh(mods[:, 3]) * m
    so = F.linear(F.silu(temb(t)), f(W["so"]))
    P = int((~torch.from_numpy(np.asarray(target_mask))).sum())
    return F.linear(F.layer_norm(h[P:], (H,), eps=dims.eps) * (1 + so), f(W["proj_out"])).numpy()


@pytest.mark.parametrize("name", ["c0", "c0w"])
@pytest.mark.parametrize("sigma", [1.0, 0.45])
def test_extract_matches_torch_composition(name, sigma):
    cfg, W, I, dims, lay, pre = setup(name)
    got = O.forward_extract(W, dims, lay, pre, I["x0"], sigma)["v"]
    want = torch_forward(W, dims, lay.image_ids, lay.coords, lay.target_mask, pre, I["x0"], sigma)
    scale = np.abs(want).max()
    assert np.abs(got - want).max() / scale < 1e-12


def test_cached_matches_torch_composition():
    cfg, W, I, dims, lay, pre = setup("c0w")
    e = O.forward_extract(W, dims, lay, pre, I["x0"], 1.0)
    x1 = O.euler_step(I["x0"], e["v"], 1.0, 0.85)
    got = O.forward_cached(W, dims, lay, e["cache"], x1, 0.85)["v"]
    want = torch_forward(W, dims, lay.image_ids, lay.coords, lay.target_mask, pre, x1, 0.85)
    assert np.abs(got - want).max() / np.abs(want).max() < 1e-12
