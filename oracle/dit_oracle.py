"""Plain fp64 NumPy oracle of one flow-matching denoising step of a
single-stream Qwen-Image-2.1-style DiT with a prefix KV cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): used by ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg, never by
the product path. It shares no code, table or helper with the HIP library.

Sources (five course pages on Qwen-Image-2.1, cited by page title and section):
  [LAB]   "Lab tổng hợp Qwen-Image-2.1 — chạy toàn trình 1A → 6B bằng NumPy"
          (end-to-end lab page): §3 Solution, §4 Profiling, §6 Glossary.
  [6B]    "6B · Scale-Only Final AdaLN, velocity v_θ & 8-Step Euler":
          §1 Definition, §4 Profiling, §6 Glossary.
  [3B]    "3B · Causal condition (t=0 vs t) & shared modulation":
          §1 Definition, §2 Flow, §3 Solution, §6 Glossary.
  [2A]    "2A · 4× image-slot expansion & joint sequence packing": §1, §2.
  [1A]    "1A · RGBA 64-Ch VAE & Unpatched Latents" (the end-to-end lab's first
          diagram step: per-channel standardization before img_in).
  [INDEX] "Bài Lab tổng hợp — Qwen-Image-2.1 Architecture" (lab index page):
          the 1:1 mapping table (rows 3A, 3B, 3C, 4A, 5A, 6A, 6B) and the
          script qwen-image-21.py, cited by its banner blocks
          ([3A] RoPE, [3B] timestep/modulation, [3C] mask, the math helpers,
          the transformer's full and cached layer functions, the scheduler).

All arithmetic is float64. Where the pages leave a step open, the reading
taken is stated at the function (and collected in the design notes). Every
function is pinned by a test in ``tests/test_oracle_*.py`` against something
other than itself (printed values, closed forms, invariants, independent
library routines); no function here is "parity unpinned" except the exact
v_θ values of the large synthetic configurations, which no page prints and
which are pinned only through those invariants.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "TURBO_SIGMAS", "DitDims", "Layout", "build_layout", "block_causal_mask",
    "row_limits", "rope_angles", "timestep_embedding", "conditioning",
    "layernorm", "rmsnorm", "silu", "rope_rotate", "masked_attention",
    "forward_extract", "forward_cached", "euler_step", "run_loop",
    "cached_rows_one_layer", "standardize", "unstandardize",
]

# [6B] §1 Definition / §6 Glossary: the 8-step Turbo sigma table (9 marks).
TURBO_SIGMAS = (1.0, 0.978453, 0.95418, 0.926626, 0.89508, 0.845148,
                0.704534, 0.414568, 0.0)


@dataclass(frozen=True)
class DitDims:
    """Model dimensions. eps and the RoPE/time base follow the lab script's
    configuration block ([INDEX] script, constants EPS_NORM and ROPE_BASE)."""
    hidden: int
    n_heads: int
    head_dim: int
    ffn: int
    n_layers: int
    latent: int = 64
    time_dim: int = 256
    rope_dims: tuple = (16, 56, 56)
    rope_base: float = 10000.0
    eps: float = 1e-6


@dataclass
class Layout:
    image_ids: np.ndarray          # int [S]; -1 text, 0..K-1 refs, K target
    target_mask: np.ndarray        # bool [S]
    coords: np.ndarray             # int [S, 3] (frame, height, width)
    P: int
    T: int
    S: int
    segments: list = field(default_factory=list)


def build_layout(segments) -> Layout:
    """Token metadata of the joint sequence.

    [2A] §1/§2: the joint sequence is text -> reference images -> target
    image; ``image_ids`` is -1 for text, 0..K-1 for the references in order,
    K for the image being generated, and ``target_token_mask`` is True only
    on the target block. Image cells are laid out row-major.
    [INDEX] mapping row 3A and [LAB] §3: text tokens advance all three axes
    together, (0,0,0) -> (1,1,1) -> (2,2,2), counting text tokens only; every
    image is pinned to frame 0 with a zero-centred grid, which for a 2x2 grid
    is (-1,-1), (-1,0), (0,-1), (0,0), i.e. offset ``r - n//2``.

    ``segments`` is a list of ("text", n), ("ref", h, w), ("target", h, w);
    exactly one "target", and it must be last.
    """
    ids, coords, tmask = [], [], []
    text_i = 0
    n_ref = 0
    kinds = [s[0] for s in segments]
    if kinds.count("target") != 1 or kinds[-1] != "target":
        raise ValueError("exactly one target segment, placed last")
    for seg in segments:
        kind = seg[0]
        if kind == "text":
            for _ in range(int(seg[1])):
                ids.append(-1)
                coords.append((text_i, text_i, text_i))
                tmask.append(False)
                text_i += 1
        elif kind in ("ref", "target"):
            h, w = int(seg[1]), int(seg[2])
            img_id = n_ref if kind == "ref" else sum(1 for s in segments if s[0] == "ref")
            for r in range(h):
                for q in range(w):
                    ids.append(img_id)
                    coords.append((0, r - h // 2, q - w // 2))
                    tmask.append(kind == "target")
            if kind == "ref":
                n_ref += 1
        else:
            raise ValueError(f"unknown segment {seg!r}")
    ids = np.asarray(ids, dtype=np.int64)
    tm = np.asarray(tmask, dtype=bool)
    T = int(tm.sum())
    S = len(ids)
    return Layout(image_ids=ids, target_mask=tm,
                  coords=np.asarray(coords, dtype=np.int64),
                  P=S - T, T=T, S=S, segments=list(segments))


def block_causal_mask(image_ids, rows=None) -> np.ndarray:
    """[INDEX] mapping row 3C and script block [3C]: key j is visible to
    query i iff i >= j, or both tokens carry the same image id and it is >= 0.
    Evaluated as that pairwise rule for every (i, j) (no block structure is
    assumed). ``rows``: optional query indices (default: all S)."""
    ids = np.asarray(image_ids)
    S = len(ids)
    qi = np.arange(S) if rows is None else np.asarray(rows)
    kj = np.arange(S)
    causal = qi[:, None] >= kj[None, :]
    same = (ids[qi][:, None] >= 0) & (ids[qi][:, None] == ids[None, :])
    return causal | same


def row_limits(image_ids, rows=None, chunk: int = 1024) -> np.ndarray:
    """Largest visible key index per query row under the block-causal rule,
    read off the pairwise mask (the last True in each row), for all rows or
    the given ``rows``. The mask is formed ``chunk`` query rows at a time
    only to bound memory."""
    ids = np.asarray(image_ids)
    S = len(ids)
    qi = np.arange(S) if rows is None else np.asarray(rows)
    out = np.empty(len(qi), dtype=np.int64)
    for r0 in range(0, len(qi), chunk):
        m = block_causal_mask(ids, rows=qi[r0:r0 + chunk])
        out[r0:r0 + m.shape[0]] = S - 1 - np.argmax(m[:, ::-1], axis=1)
    return out


def rope_angles(coords, dims: DitDims) -> np.ndarray:
    """3D axial RoPE angles, one per rotated pair, shape [S, head_dim/2].

    [INDEX] script block [3A] and its note that production splits head_dim
    128 as (16, 56, 56) over (frame, height, width): pairs are taken axis by
    axis in that order. Reading (the pages give only the split): within an
    axis of width d_a, pair j turns by coordinate * base^(-2j/d_a), the
    standard per-axis RoPE frequency with the pages' base 10000.
    """
    coords = np.asarray(coords, dtype=np.float64)
    if sum(dims.rope_dims) != dims.head_dim:
        raise ValueError("rope_dims must sum to head_dim")
    cols = []
    for axis, d_a in enumerate(dims.rope_dims):
        if d_a % 2:
            raise ValueError("each rope axis width must be even")
        for j in range(d_a // 2):
            freq = dims.rope_base ** (-2.0 * j / d_a)
            cols.append(coords[:, axis] * freq)
    return np.stack(cols, axis=1) if cols else np.zeros((len(coords), 0))


def rope_rotate(x, angles):
    """Rotate interleaved pairs (2m, 2m+1) of the last axis by angles[..., m]:
    (x0 c - x1 s, x0 s + x1 c). [INDEX] script block [3A], rope rotation of
    heads. ``x``: [N, nh, d]; ``angles``: [N, d/2]."""
    c = np.cos(angles)[:, None, :]
    s = np.sin(angles)[:, None, :]
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def timestep_embedding(t: float, time_dim: int, base: float = 10000.0):
    """[3B] §1/§6: the timestep 1000·σ becomes a sin-cos vector; the lab's
    [3B] block orders it cosine first. With K = time_dim/2 angular
    frequencies ω_i = base^(-i/K), i < K, the vector is
    [cos(t ω_0) .. cos(t ω_{K-1}), sin(t ω_0) .. sin(t ω_{K-1})],
    taken here as the real and imaginary parts of exp(i t ω)."""
    half = time_dim // 2
    omega = np.exp(-np.log(base) * np.arange(half, dtype=np.float64) / half)
    rot = np.exp(1j * (float(t) * omega))
    return np.hstack((rot.real, rot.imag))


def silu(x):
    """x·sigmoid(x) ([INDEX] script, math helpers)."""
    return x / (1.0 + np.exp(-x))


def layernorm(x, eps: float = 1e-6):
    """Non-affine LayerNorm over the last axis: (x - E[x]) · (Var[x] + ε)^(-1/2)
    with the population (1/n) variance ([INDEX] script, math helpers)."""
    centred = x - np.mean(x, axis=-1, keepdims=True)
    inv_sd = 1.0 / np.sqrt(np.var(x, axis=-1, keepdims=True) + eps)
    return centred * inv_sd


def rmsnorm(x, w, eps: float = 1e-6):
    """Zero-centred RMSNorm over the last axis (length d):
    x · (‖x‖²/d + ε)^(-1/2) · (1 + w) ([INDEX] script, math helpers; used per
    head as QK-RMSNorm, mapping row 4A)."""
    d = x.shape[-1]
    sq = np.linalg.norm(x, axis=-1, keepdims=True) ** 2
    return (x * (1.0 / np.sqrt(sq / d + eps))) * (1.0 + w)


def conditioning(W, dims: DitDims, sigma: float, causal_condition: bool = True):
    """Timestep embedding and the two shared modulation rows.

    [3B] §1: t = 1000·σ goes through a sin-cos embedding and an MLP to a
    hidden-width vector; with causal_condition two rows are formed, one at
    t = 0 (for prefix tokens) and one at the current t (for target tokens);
    one shared SiLU -> Linear(H, 4H) turns each row into
    [scale1, gate1, scale2, gate2], read by every block.
    [6B] §3: the final AdaLN's scale comes from the same current-t row.

    Readings: the embedding MLP is Linear(D_t, H) -> SiLU -> Linear(H, H);
    the final scale is a separate SiLU -> Linear(H, H) of the same t
    embedding; no biases. With causal_condition False both rows use t.
    Returns dict(row_t, row_0 [4H], scale_out [H]).
    """
    t = 1000.0 * float(sigma)

    def temb(tv):
        e = timestep_embedding(tv, dims.time_dim, dims.rope_base)
        return W["t2"] @ silu(W["t1"] @ e)

    te_t = temb(t)
    te_0 = temb(0.0) if causal_condition else te_t
    row_t = W["mod"] @ silu(te_t)
    row_0 = W["mod"] @ silu(te_0)
    scale_out = W["so"] @ silu(te_t)
    return {"row_t": row_t, "row_0": row_0, "scale_out": scale_out, "t": t}


def _split_rows(row, H):
    # [3B] §1 and §2: chunk order [scale1, gate1, scale2, gate2].
    return row[0:H], row[H:2 * H], row[2 * H:3 * H], row[3 * H:4 * H]


def masked_attention(q, k, v, allowed, row_block: int = 128):
    """softmax(q kᵀ/√d) v per head with masked keys excluded.

    [INDEX] script, the full layer function: scores scaled by 1/√head_dim,
    masked entries pushed to -1e9 before a max-subtracted softmax, so masked
    weights are exactly 0 in fp64 (every row keeps at least its own key).
    Here masked scores are -inf, which gives the same exact zeros.
    ``q``: [Nq, nh, d], ``k``/``v``: [Nk, nh, d], ``allowed``: bool [Nq, Nk].
    Returns [Nq, nh*d]. Query rows are processed ``row_block`` at a time
    (each row's softmax is independent, so this changes no arithmetic).
    """
    Nq, nh, d = q.shape
    out = np.empty((Nq, nh, d))
    kh = k.transpose(1, 2, 0)            # [nh, d, Nk]
    vh = v.transpose(1, 0, 2)            # [nh, Nk, d]
    scale = 1.0 / math.sqrt(d)
    for r0 in range(0, Nq, row_block):
        r1 = min(Nq, r0 + row_block)
        qh = q[r0:r1].transpose(1, 0, 2)                 # [nh, b, d]
        s = np.matmul(qh, kh) * scale                    # [nh, b, Nk]
        s = np.where(allowed[None, r0:r1, :], s, -np.inf)
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=-1, keepdims=True)
        out[r0:r1] = np.matmul(p, vh).transpose(1, 0, 2)
    return out.reshape(Nq, nh * d)


def _layer(h, scale1, gate1, scale2, gate2, L, dims, angles, allowed,
           k_prefix=None, v_prefix=None):
    """One single-stream block on the rows of ``h``.

    [INDEX] mapping rows 4A and 5A, and the script's full/cached layer
    functions: LN(h)·(1+scale1) -> shared QKV projection -> per-head
    QK-RMSNorm (1+w) -> 3D RoPE -> masked SDPA -> W_O -> h += tanh(gate1)·out;
    LN(h)·(1+scale2) -> SwiGLU (SiLU(x W_g) ⊙ x W_u) W_d -> h += tanh(gate2)·ffn.
    Reading (page 3B §1, spec wording): four modulation chunks, no
    shift. ``scale*``/``gate*`` are per-row arrays [N, H].
    If ``k_prefix``/``v_prefix`` are given (cached mode, page [LAB] §6
    kv_cache_mode), the fresh K/V rows are appended after them.
    Returns (h_new, k_rows, v_rows) where k_rows/v_rows are this call's own
    post-norm, post-RoPE K and raw V rows [N, nh, d].
    """
    N, H = h.shape
    nh, d = dims.n_heads, dims.head_dim
    x1 = layernorm(h, dims.eps) * (1.0 + scale1)
    qkv = x1 @ L["qkv"].T                                  # [N, 3H]
    q = qkv[:, 0:H].reshape(N, nh, d)
    k = qkv[:, H:2 * H].reshape(N, nh, d)
    v = qkv[:, 2 * H:3 * H].reshape(N, nh, d)
    q = rope_rotate(rmsnorm(q, L["q_norm"], dims.eps), angles)
    k = rope_rotate(rmsnorm(k, L["k_norm"], dims.eps), angles)
    if k_prefix is not None:
        k_all = np.concatenate([k_prefix, k], axis=0)
        v_all = np.concatenate([v_prefix, v], axis=0)
    else:
        k_all, v_all = k, v
    o = masked_attention(q, k_all, v_all, allowed)
    h = h + np.tanh(gate1) * (o @ L["o"].T)
    x2 = layernorm(h, dims.eps) * (1.0 + scale2)
    m = (silu(x2 @ L["gate"].T) * (x2 @ L["up"].T)) @ L["down"].T
    h = h + np.tanh(gate2) * m
    return h, k, v


def _output(h_tgt, cond, W, dims):
    """[6B] §1/§6: scale-only final AdaLN LN(h)·(1+scale_out), then
    proj_out Linear(H, C) gives v_θ per target token."""
    return (layernorm(h_tgt, dims.eps) * (1.0 + cond["scale_out"])) @ W["proj_out"].T


class _F64Layers:
    """The per-layer weights of ``W["layers"]`` read one layer at a time and
    converted to float64 when a layer is used. ``W["layers"]`` may be a list
    of per-layer dicts or a callable ``l -> dict`` that supplies layer l on
    demand, so a deep model's weights need not all be held in float64 at
    once; the arithmetic is the same either way."""

    def __init__(self, layers):
        self._src = layers

    def __getitem__(self, l):
        L = self._src(l) if callable(self._src) else self._src[l]
        return {k: np.asarray(v, dtype=np.float64) for k, v in L.items()}


def _f64(W):
    out = {k: np.asarray(v, dtype=np.float64) for k, v in W.items() if k != "layers"}
    out["layers"] = _F64Layers(W["layers"])
    return out


def forward_extract(W, dims: DitDims, layout: Layout, prefix_hidden, x, sigma,
                    causal_condition: bool = True, perturb=None, n_layers=None):
    """Step 1 (extract): all S = P + T tokens, block-causal mask, prefix rows
    read the t = 0 modulation row, target rows the current-t row; stores the
    prefix K (post-norm, post-RoPE) and raw V of every layer.

    [LAB] §3/§6 (kv_cache_mode extract) and [3B] §1 (row selection by
    target_token_mask). ``perturb``: optional list of (token, dim, delta)
    added to the joint input (the lab's isolation experiment, [INDEX]
    mapping row 3C). Returns dict(v, cache=[(K [P,nh,d], V [P,nh,d])],
    k_all=[K [S,nh,d]], v_all=[V [S,nh,d]], h_final [S,H], cond).
    """
    W = _f64(W)
    Lc = dims.n_layers if n_layers is None else n_layers
    H, P, T, S = dims.hidden, layout.P, layout.T, layout.S
    cond = conditioning(W, dims, sigma, causal_condition)
    h_tgt = np.asarray(x, dtype=np.float64) @ W["img_in"].T        # [T, H]
    h = np.concatenate([np.asarray(prefix_hidden, dtype=np.float64), h_tgt], axis=0)
    if perturb:
        for (i, dd, delta) in perturb:
            h[i, dd] += delta
    # [3B] _select_modulation_rows: mask False -> t=0 row, True -> t row.
    rows = np.where(layout.target_mask[:, None], cond["row_t"][None, :],
                    cond["row_0"][None, :])
    s1, g1, s2, g2 = _split_rows(rows.T, H)
    s1, g1, s2, g2 = s1.T, g1.T, s2.T, g2.T
    angles = rope_angles(layout.coords, dims)
    allowed = block_causal_mask(layout.image_ids)
    cache, k_all, v_all = [], [], []
    for l in range(Lc):
        h, k, v = _layer(h, s1, g1, s2, g2, W["layers"][l], dims, angles, allowed)
        cache.append((k[:P].copy(), v[:P].copy()))
        k_all.append(k)
        v_all.append(v)
    vel = _output(h[P:], cond, W, dims)
    return {"v": vel, "cache": cache, "k_all": k_all, "v_all": v_all, "h_final": h, "cond": cond}


def forward_cached(W, dims: DitDims, layout: Layout, cache, x, sigma, n_layers=None):
    """Steps 2..N (cached): only the T target tokens are projected; each
    layer attends against [cached prefix K/V ; fresh target K/V]. Every
    target query sees all S keys under the block-causal rule (the target
    block is last), so the mask rows P..S-1 are all True.
    [LAB] §3/§6 (kv_cache_mode cached) and [INDEX] mapping row 6A."""
    W = _f64(W)
    Lc = dims.n_layers if n_layers is None else n_layers
    H, P = dims.hidden, layout.P
    cond = conditioning(W, dims, sigma, True)
    h = np.asarray(x, dtype=np.float64) @ W["img_in"].T
    s1, g1, s2, g2 = _split_rows(cond["row_t"], H)
    angles = rope_angles(layout.coords[P:], dims)
    allowed = block_causal_mask(layout.image_ids, rows=np.arange(P, layout.S))
    for l in range(Lc):
        kp, vp = cache[l]
        h, _, _ = _layer(h, s1[None], g1[None], s2[None], g2[None],
                         W["layers"][l], dims, angles, allowed,
                         k_prefix=np.asarray(kp, np.float64),
                         v_prefix=np.asarray(vp, np.float64))
    return {"v": _output(h, cond, W, dims), "cond": cond}


def standardize(z, mean, std):
    """[1A] and the [INDEX] script's helper of that name: each of the C
    latent channels is standardized with its own statistics before img_in,
    ẑ = (z − mean_c) / std_c. z [n, C], mean and std [C]."""
    z = np.asarray(z, np.float64)
    return (z - np.asarray(mean, np.float64)) / np.asarray(std, np.float64)


def unstandardize(z_std, mean, std):
    """[6B] §1 Definition: after the last Euler step the latent returns to the
    VAE's space, z = ẑ·std_c + mean_c per channel (the inverse of [1A])."""
    return np.asarray(z_std, np.float64) * np.asarray(std, np.float64) + np.asarray(mean, np.float64)


def euler_step(x, v, sigma_k, sigma_k1):
    """[6B] §1/§6: x_{k+1} = x_k + (σ_{k+1} − σ_k)·v_θ."""
    return np.asarray(x, np.float64) + (float(sigma_k1) - float(sigma_k)) * np.asarray(v, np.float64)


def run_loop(W, dims, layout, prefix_hidden, x0, sigmas=TURBO_SIGMAS, use_cache=True,
             n_layers=None, causal_condition=True):
    """The sampler loop: step 1 extract, steps 2..N cached (use_cache=True),
    or extract at every step (full recompute). [LAB] §4 Profiling and the
    [INDEX] script's pipeline driver. Any decreasing sigma list is a schedule
    ([6B] §1: Turbo fixes 8 steps; more steps are the general case). With
    causal_condition False ([3B] §4 Limits) the prefix follows t, its K/V
    change every step, so the cache is invalid and every step recomputes.
    Returns list of dict(v, x_next, mode)."""
    if not causal_condition and use_cache:
        raise ValueError("without causal conditioning the prefix cache is invalid")
    x = np.asarray(x0, np.float64)
    cache = None
    recs = []
    for k in range(len(sigmas) - 1):
        if k == 0 or not use_cache:
            out = forward_extract(W, dims, layout, prefix_hidden, x, sigmas[k],
                                  causal_condition=causal_condition, n_layers=n_layers)
            if cache is None:
                cache = out["cache"]
            mode = "extract"
        else:
            out = forward_cached(W, dims, layout, cache, x, sigmas[k], n_layers=n_layers)
            mode = "cached"
        xn = euler_step(x, out["v"], sigmas[k], sigmas[k + 1])
        recs.append({"v": out["v"], "x_next": xn, "mode": mode, "sigma": sigmas[k]})
        x = xn
    return recs


def cached_rows_one_layer(W, dims: DitDims, layout: Layout, prefix_hidden, x, sigma,
                          rows, mode="cached"):
    """v_θ of selected target rows for a ONE-layer model, computed row by row.

    With one layer, the prefix cache is the layer-0 K/V of the prefix input
    (no attention is needed to form it), and a target row's output depends on
    the other tokens only through layer-0 K/V. So the K/V of all S tokens are
    formed once and the rest (attention, W_O, SwiGLU, final AdaLN, proj_out)
    is evaluated only for ``rows`` (indices into the T target tokens).
    Same arithmetic as ``forward_extract``/``forward_cached`` with
    n_layers = 1; in exact arithmetic both modes give the same target rows.
    """
    W = _f64(W)
    H, P, S = dims.hidden, layout.P, layout.S
    nh, d = dims.n_heads, dims.head_dim
    cond = conditioning(W, dims, sigma, True)
    L = W["layers"][0]
    h_tgt = np.asarray(x, np.float64) @ W["img_in"].T
    h = np.concatenate([np.asarray(prefix_hidden, np.float64), h_tgt], axis=0)
    rows_mod = np.where(layout.target_mask[:, None], cond["row_t"][None, :],
                        cond["row_0"][None, :])
    scale1 = rows_mod[:, 0:H]
    x1 = layernorm(h, dims.eps) * (1.0 + scale1)
    ang = rope_angles(layout.coords, dims)
    kv = x1 @ L["qkv"][H:3 * H].T
    k = rope_rotate(rmsnorm(kv[:, :H].reshape(S, nh, d), L["k_norm"], dims.eps), ang)
    v = kv[:, H:].reshape(S, nh, d)
    sel = P + np.asarray(rows)
    q = (x1[sel] @ L["qkv"][0:H].T).reshape(len(sel), nh, d)
    q = rope_rotate(rmsnorm(q, L["q_norm"], dims.eps), ang[sel])
    allowed = block_causal_mask(layout.image_ids, rows=sel)
    o = masked_attention(q, k, v, allowed)
    s1, g1, s2, g2 = _split_rows(cond["row_t"], H)
    hs = h[sel] + np.tanh(g1) * (o @ L["o"].T)
    x2 = layernorm(hs, dims.eps) * (1.0 + s2)
    m = (silu(x2 @ L["gate"].T) * (x2 @ L["up"].T)) @ L["down"].T
    hs = hs + np.tanh(g2) * m
    return _output(hs, cond, W, dims)
