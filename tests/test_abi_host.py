"""C ABI checks that need no GPU: the library loads, exports every entry
point include/dit.h declares, builds layouts identical to the oracle's, and
rejects bad arguments on the host before any device work."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle as O
from diffusion_transformer_amd import _lib as L
from diffusion_transformer_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "dit.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"^\s*#.*$", "", src, flags=re.M)       # preprocessor lines
    return sorted(set(re.findall(r"\b(\w+)\s*\([^;{]*\)\s*;", src)) - {"if", "for", "while"})


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert len(names) >= 17
    lib = C.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTS)


def cfg_c(name):
    c = synth.config(name)
    return c, L.make_config(**{k: c[k] for k in ("hidden", "n_heads", "head_dim", "ffn",
                                                  "n_layers", "latent", "time_dim", "rope_dims")})


@pytest.mark.parametrize("name", ["c0w", "c1", "c2", "c3", "c4", "c5", "ragged", "many_ragged"])
def test_layout_matches_oracle(name):
    if name in synth.RAGGED_LAYOUTS:
        cfg, c = cfg_c("c1")
        cfg = dict(cfg, segments=synth.RAGGED_LAYOUTS[name])
    else:
        cfg, c = cfg_c(name)
    lay = L.dit_build_layout(c, cfg["segments"])
    ol = O.build_layout(cfg["segments"])
    assert (lay["P"], lay["T"]) == (ol.P, ol.T)
    assert np.array_equal(lay["image_ids"], ol.image_ids)
    assert np.array_equal(lay["coords"], ol.coords)
    S = ol.S
    rows = np.arange(S)
    if S > 20000:
        # the pairwise read-off on every row next to a block edge and 4000 random rows
        edges = np.nonzero(np.diff(ol.image_ids))[0]
        near = np.clip(np.concatenate([edges - 1, edges, edges + 1, edges + 2]), 0, S - 1)
        rows = np.unique(np.concatenate([near, [0, S - 1], np.random.default_rng(5).choice(S, 4000)]))
    assert np.array_equal(lay["row_limit"][rows], O.row_limits(ol.image_ids, rows=rows))
    dims = O.DitDims(hidden=cfg["hidden"], n_heads=cfg["n_heads"], head_dim=128, ffn=cfg["ffn"],
                     n_layers=1, rope_dims=tuple(cfg["rope_dims"]))
    ang = O.rope_angles(ol.coords, dims)
    assert np.abs(lay["rope_cos"] - np.cos(ang)).max() < 1e-7
    assert np.abs(lay["rope_sin"] - np.sin(ang)).max() < 1e-7


def test_layout_errors():
    _, c = cfg_c("c1")
    with pytest.raises(L.DitError) as e:
        L.dit_build_layout(c, [("target", 2, 2), ("text", 3)])
    assert e.value.status == L.DIT_ERR_LAYOUT
    with pytest.raises(L.DitError) as e:
        L.dit_build_layout(c, [("text", 3), ("ref", 0, 2), ("target", 2, 2)])
    assert e.value.status == L.DIT_ERR_LAYOUT
    with pytest.raises(L.DitError) as e:
        L.dit_build_layout(c, [("text", 3), ("target", 2, 2), ("target", 2, 2)])
    assert e.value.status == L.DIT_ERR_LAYOUT
    # the library's sequence limit: 2^22 tokens in all (ten 700x700 references exceed it)
    with pytest.raises(L.DitError) as e:
        L.dit_build_layout(c, [("text", 512)] + [("ref", 700, 700)] * 10 + [("target", 96, 96)])
    assert e.value.status == L.DIT_ERR_LAYOUT


FAKE = 1 << 20   # 16-byte aligned stand-in pointer; never dereferenced on these paths


def fake_weights(nl):
    arr = (C.c_void_p * nl)(*([FAKE] * nl))
    p = C.cast(arr, C.POINTER(C.c_void_p))
    return L.dit_weights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, p, p, p, p, p, p, p), arr


def load(c, api=L):
    w, keep = fake_weights(c.n_layers)
    h = C.c_void_p()
    st = api._lib.dit_load_weights(C.byref(c), C.byref(w), C.byref(h))
    return st, h.value


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, L.DIT_ERR_SHAPE), ("hidden", 4000, L.DIT_ERR_SHAPE),
    ("latent", 32, L.DIT_ERR_SHAPE), ("ffn", 100, L.DIT_ERR_SHAPE), ("n_layers", 0, L.DIT_ERR_ARG)])
def test_load_weights_validation(field, value, status):
    _, c = cfg_c("c1")
    setattr(c, field, value)
    st, h = load(c)
    assert st == status and h is None
    assert L.dit_last_error()


def test_rope_dims_must_sum_to_head_dim():
    _, c = cfg_c("c1")
    c.rope_dims[:] = [16, 56, 54]
    assert load(c)[0] == L.DIT_ERR_SHAPE


def test_null_weight_pointer_rejected():
    _, c = cfg_c("c0w")
    w, keep = fake_weights(c.n_layers)
    w.mod = None
    h = C.c_void_p()
    assert L._lib.dit_load_weights(C.byref(c), C.byref(w), C.byref(h)) == L.DIT_ERR_ARG


def test_step_state_and_workspace_errors():
    cfg, c = cfg_c("c0w")
    st, m = load(c)
    assert st == L.DIT_OK
    try:
        seq = L.dit_seq(7, 4, FAKE, FAKE, FAKE)
        kvb = L.dit_kv_cache_bytes(m, 11)
        wsb = L.dit_workspace_bytes(m, 11)
        assert kvb == 2 * 2 * 2 * 128 * 128 * 2     # L * {K,V} * nh * cap(128) * d * bf16
        assert L.dit_kv_capacity(11) == 128 and L.dit_kv_capacity(128) == 128
        assert L.dit_kv_capacity(129) == 256
        # cached before any extract
        r = L._lib.dit_step_cached(m, C.byref(seq), FAKE, 0.85, FAKE, kvb, FAKE, FAKE, wsb, None)
        assert r == L.DIT_ERR_STATE
        # short workspace / cache
        r = L._lib.dit_step_extract(m, C.byref(seq), FAKE, FAKE, 1.0, FAKE, kvb, FAKE, FAKE,
                                    wsb - 1, 0, None)
        assert r == L.DIT_ERR_WORKSPACE
        r = L._lib.dit_step_extract(m, C.byref(seq), FAKE, FAKE, 1.0, FAKE, kvb - 2, FAKE, FAKE,
                                    wsb, 0, None)
        assert r == L.DIT_ERR_WORKSPACE
        # null pointers, bad flags, bad sigma, bad layout counts
        r = L._lib.dit_step_extract(m, C.byref(seq), FAKE, None, 1.0, FAKE, kvb, FAKE, FAKE, wsb, 0, None)
        assert r == L.DIT_ERR_ARG
        r = L._lib.dit_step_extract(m, C.byref(seq), FAKE, FAKE, 1.0, FAKE, kvb, FAKE, FAKE, wsb, 8, None)
        assert r == L.DIT_ERR_ARG
        r = L._lib.dit_step_extract(m, C.byref(seq), FAKE, FAKE, float("nan"), FAKE, kvb, FAKE,
                                    FAKE, wsb, 0, None)
        assert r == L.DIT_ERR_ARG
        bad = L.dit_seq(7, 0, FAKE, FAKE, FAKE)
        r = L._lib.dit_step_extract(m, C.byref(bad), FAKE, FAKE, 1.0, FAKE, kvb, FAKE, FAKE, wsb, 0, None)
        assert r == L.DIT_ERR_LAYOUT
        r = L._lib.dit_step_extract(m, C.byref(seq), FAKE, FAKE + 4, 1.0, FAKE, kvb, FAKE, FAKE,
                                    wsb, 0, None)
        assert r == L.DIT_ERR_ARG            # misaligned
        assert L._lib.euler_update(None, FAKE, 1.0, 0.5, 4, None) == L.DIT_ERR_ARG
        d = L.dit_gemm_desc(epilogue=0, M=10, N=100, K=64, A=FAKE, B=FAKE, C=FAKE)
        assert L._lib.dit_debug_gemm(C.byref(d), None) == L.DIT_ERR_SHAPE
        assert L._lib.dit_profile_enable(m, 99) == L.DIT_ERR_ARG
    finally:
        L.dit_free(m)


def test_batch_of_targets_validation():
    """Several target latents sharing one prefix: the cache and workspace
    cover P + B*T rows, B > 1 needs P and T multiples of 256, and a cached
    step needs an extract of the same batch."""
    cfg, c = cfg_c("c1")
    st, m = load(c)
    assert st == L.DIT_OK
    try:
        P, T, B = 512, 1024, 3
        seq = L.dit_seq(P, T, FAKE, FAKE, FAKE, B)
        kvb = L.dit_kv_cache_bytes(m, P + B * T)
        ws_x, ws_c = L.dit_workspace_bytes(m, P + B * T), L.dit_workspace_bytes(m, B * T)
        # a cache sized for one latent is too small for three
        r = L._lib.dit_step_extract(m, C.byref(seq), FAKE, FAKE, 1.0, FAKE,
                                    L.dit_kv_cache_bytes(m, P + T), FAKE, FAKE, ws_x, 0, None)
        assert r == L.DIT_ERR_WORKSPACE
        r = L._lib.dit_step_extract(m, C.byref(seq), FAKE, FAKE, 1.0, FAKE, kvb, FAKE, FAKE,
                                    ws_c, 0, None)
        assert r == L.DIT_ERR_WORKSPACE          # extract needs the P + B*T workspace
        r = L._lib.dit_step_cached(m, C.byref(seq), FAKE, 0.9, FAKE, kvb, FAKE, FAKE, ws_c, None)
        assert r == L.DIT_ERR_STATE
        for bad in (L.dit_seq(500, T, FAKE, FAKE, FAKE, 2), L.dit_seq(P, 1000, FAKE, FAKE, FAKE, 2)):
            r = L._lib.dit_step_extract(m, C.byref(bad), FAKE, FAKE, 1.0, FAKE, kvb, FAKE, FAKE,
                                        ws_x, 0, None)
            assert r == L.DIT_ERR_SHAPE
        neg = L.dit_seq(P, T, FAKE, FAKE, FAKE, -1)
        r = L._lib.dit_step_extract(m, C.byref(neg), FAKE, FAKE, 1.0, FAKE, kvb, FAKE, FAKE, ws_x, 0, None)
        assert r == L.DIT_ERR_ARG
        # P + B*T beyond 2^22 tokens is refused before any size check
        long_seq = L.dit_seq(1 << 21, 1 << 20, FAKE, FAKE, FAKE, 3)
        r = L._lib.dit_step_extract(m, C.byref(long_seq), FAKE, FAKE, 1.0, FAKE, 1 << 60, FAKE,
                                    FAKE, 1 << 60, 0, None)
        assert r == L.DIT_ERR_LAYOUT
    finally:
        L.dit_free(m)
    # the fp32 debug build refuses several latents
    f32 = L.load_f32()
    st, m = load(c, api=f32)
    assert st == L.DIT_OK
    try:
        seq = L.dit_seq(512, 1024, FAKE, FAKE, FAKE, 2)
        r = f32._lib.dit_step_extract(m, C.byref(seq), FAKE, FAKE, 1.0, FAKE, 1 << 40, FAKE,
                                      FAKE, 1 << 40, 0, None)
        assert r == L.DIT_ERR_UNSUPPORTED
    finally:
        f32.dit_free(m)


def test_workspace_grows_with_tokens():
    cfg, c = cfg_c("c1")
    st, m = load(c)
    try:
        a, b = L.dit_workspace_bytes(m, 1024), L.dit_workspace_bytes(m, 1536)
        assert 0 < a < b
        # activations: f32 residual + bf16 (x, qkv, attn, ffn) per token
        per_tok = 4096 * 4 + 4096 * 2 + 3 * 4096 * 2 + 4096 * 2 + 16384 * 2
        assert abs((b - a) - 512 * per_tok) < 64 * 256
    finally:
        L.dit_free(m)


def test_one_hip_runtime_per_process():
    """The binding opens the library after torch, so both share torch's HIP
    runtime (a second runtime in the process cannot see the device once the
    first one holds it, and torch's streams would be foreign to it)."""
    import subprocess
    import sys
    code = ("import diffusion_transformer_amd._lib\n"
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         check=True).stdout.strip().splitlines()[-1]
    assert out.count("libamdhip64") == 1, out


# Random token layouts: text runs and reference images in any order, then
# one target image; every output of the C layout builder must equal the
# oracle's plain construction (ids, coordinates, row limits read off the
# pairwise mask, RoPE tables).
try:
    from hypothesis import given, settings, strategies as st
except ImportError:   # pragma: no cover
    given = None

if given is not None:
    _seg = st.one_of(st.tuples(st.just("text"), st.integers(1, 40)),
                     st.tuples(st.just("ref"), st.integers(1, 12), st.integers(1, 12)))

    @settings(max_examples=60, deadline=None)
    @given(st.lists(_seg, min_size=0, max_size=12),
           st.tuples(st.just("target"), st.integers(1, 12), st.integers(1, 12)))
    def test_random_layouts_match_oracle(prefix, target):
        segs = list(prefix) + [target]
        _, c = cfg_c("c1")
        lay = L.dit_build_layout(c, segs)
        ol = O.build_layout(segs)
        assert (lay["P"], lay["T"]) == (ol.P, ol.T)
        assert np.array_equal(lay["image_ids"], ol.image_ids)
        assert np.array_equal(lay["coords"], ol.coords)
        assert np.array_equal(lay["row_limit"], O.row_limits(ol.image_ids))
        dims = O.DitDims(hidden=4096, n_heads=32, head_dim=128, ffn=16384, n_layers=1)
        ang = O.rope_angles(ol.coords, dims)
        assert np.abs(lay["rope_cos"] - np.cos(ang)).max() < 1e-7
        assert np.abs(lay["rope_sin"] - np.sin(ang)).max() < 1e-7


def test_debug_gemm_descriptor_validation():
    """The GEMM test hook rejects on the host: unknown epilogues, missing
    operands, unsupported shapes, a forced split without enough scratch or
    with K not divisible into the splits, and a QKV width that is not three
    heads' worth."""
    def st(**kw):
        base = dict(epilogue=0, M=300, N=512, K=256, A=FAKE, B=FAKE, C=FAKE)
        base.update(kw)
        return L._lib.dit_debug_gemm(C.byref(L.dit_gemm_desc(**base)), None)

    assert st(epilogue=4) == L.DIT_ERR_ARG            # the internal partial-sum epilogue
    assert st(epilogue=9) == L.DIT_ERR_ARG
    assert st(A=None) == L.DIT_ERR_ARG
    assert st(epilogue=2, C=None) == L.DIT_ERR_ARG    # residual needs h and both gates
    assert st(epilogue=3) == L.DIT_ERR_ARG            # SwiGLU needs the up weights
    assert st(K=100) == L.DIT_ERR_SHAPE
    assert st(epilogue=1) == L.DIT_ERR_ARG            # no fp32-output GEMM (proj_out is fused)
    assert st(splits=3) == L.DIT_ERR_ARG
    assert st(splits=2) == L.DIT_ERR_ARG              # no scratch
    need = 2 * (300 - 256) * 512 * 4
    assert st(splits=2, scratch=FAKE, scratch_bytes=need - 1) == L.DIT_ERR_ARG
    assert st(splits=4, K=192, scratch=FAKE, scratch_bytes=1 << 30) == L.DIT_ERR_ARG
    assert st(epilogue=5, N=768, n_heads=1, q_norm=FAKE, k_norm=FAKE, rope_cos=FAKE,
              rope_sin=FAKE, kv_cache=FAKE, S=300, eps=1e-6) == L.DIT_ERR_SHAPE
    assert st(epilogue=5, N=768, n_heads=2, q_norm=FAKE, k_norm=FAKE, rope_cos=FAKE,
              rope_sin=FAKE, kv_cache=FAKE, S=299, eps=1e-6) == L.DIT_ERR_ARG   # rows past S
    assert st(epilogue=5, N=768, n_heads=2, S=300, eps=1e-6) == L.DIT_ERR_ARG  # no tables


def test_debug_attention_validation():
    seq = L.dit_seq(7, 4, FAKE, FAKE, FAKE)

    def st(variant=0, scratch=None, N=4, q_off=7):
        return L._lib.dit_debug_attention(C.byref(seq), 2, FAKE, 256, q_off, N, FAKE, FAKE,
                                          variant, scratch, 1 << 20, None)

    assert st(variant=7) == L.DIT_ERR_ARG             # no such variant
    assert st(variant=5) == L.DIT_ERR_ARG             # pipelined kernel: S = 11 not a multiple of 64
    assert st(variant=6, N=11, q_off=0) == L.DIT_ERR_ARG   # ... and target rows only
    assert st(scratch=FAKE + 4) == L.DIT_ERR_ARG
    assert st(N=5) == L.DIT_ERR_ARG                   # rows past S


def test_host_tensor_checks_in_the_binding():
    """The binding checks on the host what the C ABI cannot see: the step's
    x / v / prefix tensors must be contiguous float32 device tensors of the
    sizes the call reads and writes (here CPU tensors are refused)."""
    import torch
    cfg, c = cfg_c("c0w")
    W = {k: FAKE for k in ("t1", "t2", "mod", "so", "img_in", "proj_out")}
    for k in ("qkv", "q_norm", "k_norm", "o", "gate", "up", "down"):
        W[k] = [FAKE] * cfg["n_layers"]
    m = L.dit_load_weights(c, W)
    try:
        seq = L.dit_seq(7, 4, FAKE, FAKE, FAKE)
        x = torch.zeros((4, 64))
        with pytest.raises(L.DitError) as e:
            L.dit_step_cached(m, seq, x, 0.5, FAKE, x, FAKE)
        assert e.value.status == L.DIT_ERR_ARG and "x" in str(e.value)
        with pytest.raises(L.DitError):
            L.dit_step_extract(m, seq, torch.zeros((7, 256)), x, 1.0, FAKE, x, FAKE)
        with pytest.raises(L.DitError):
            L.euler_update(x, x, 1.0, 0.5)
    finally:
        L.dit_free(m)


def test_model_handle_calls_from_many_threads():
    """Calls on one handle from several threads are serialized by the
    handle's lock: concurrent cached-step requests (refused: nothing was
    extracted) and timing-state calls neither crash nor change each other's
    answers."""
    import threading
    cfg, c = cfg_c("c0w")
    st, m = load(c)
    assert st == L.DIT_OK
    seq = L.dit_seq(7, 4, FAKE, FAKE, FAKE)
    kvb, wsb = L.dit_kv_cache_bytes(m, 11), L.dit_workspace_bytes(m, 4)
    bad = []

    def work(i):
        for _ in range(300):
            r = L._lib.dit_step_cached(m, C.byref(seq), FAKE, 0.85, FAKE, kvb, FAKE, FAKE, wsb, None)
            if r != L.DIT_ERR_STATE:
                bad.append(("cached", r))
            if L._lib.dit_profile_enable(m, 1 + i % 7) != L.DIT_OK:
                bad.append("enable")
            ms, n = C.c_double(), C.c_longlong()
            if L._lib.dit_profile_read(m, C.byref(ms), C.byref(n)) != L.DIT_OK or n.value != 0:
                bad.append("read")

    try:
        th = [threading.Thread(target=work, args=(i,)) for i in range(8)]
        for t in th:
            t.start()
        for t in th:
            t.join()
        assert not bad, bad[:5]
    finally:
        L.dit_free(m)


def test_noalloc_step_refuses_sizes_above_its_array():
    """The allocation-free cached step refuses, on the host and before any
    device work, a target row count whose workspace exceeds the library's
    fixed device array (c1's dimensions: 4096 target rows need about 360 MB);
    null arguments are refused too."""
    cfg, c = cfg_c("c1")
    st, m = load(c)
    assert st == L.DIT_OK
    try:
        big = L.dit_seq(16, 4096, FAKE, FAKE, FAKE)
        assert L.dit_workspace_bytes(m, 4096) > 256 << 20
        r = L._lib.dit_step_cached_noalloc(m, C.byref(big), FAKE, 0.5, FAKE, 1 << 40, FAKE, None)
        assert r == L.DIT_ERR_WORKSPACE
        assert "fixed" in L.dit_last_error()
        assert L._lib.dit_step_cached_noalloc(None, C.byref(big), FAKE, 0.5, FAKE, 1 << 40, FAKE,
                                              None) == L.DIT_ERR_ARG
    finally:
        L.dit_free(m)


def test_measurement_and_final_hooks_validation():
    f = L._lib.dit_debug_final_out
    assert f(None, 4096, 10, 4096, FAKE, 1e-6, FAKE, FAKE, None) == L.DIT_ERR_ARG
    assert f(FAKE, 4096, 10, 4000, FAKE, 1e-6, FAKE, FAKE, None) == L.DIT_ERR_SHAPE
    assert f(FAKE, 4096, 10, 8192, FAKE, 1e-6, FAKE, FAKE, None) == L.DIT_ERR_SHAPE
    assert f(FAKE, 100, 10, 256, FAKE, 1e-6, FAKE, FAKE, None) == L.DIT_ERR_SHAPE      # ldh < H
    assert f(FAKE, 4096, 10, 4096, FAKE, 0.0, FAKE, FAKE, None) == L.DIT_ERR_ARG
    assert L._lib.dit_debug_stream_copy(FAKE, FAKE, 24, None) == L.DIT_ERR_ARG
    assert L._lib.dit_debug_mfma_loop(FAKE, FAKE, 0, 10, None) == L.DIT_ERR_ARG


def test_gemv_hook_validation():
    f = L._lib.dit_debug_gemv
    assert f(None, 16, 64, FAKE, 64, 1, FAKE, None, None) == L.DIT_ERR_ARG
    assert f(FAKE, 16, 64, FAKE, 64, 3, FAKE, None, None) == L.DIT_ERR_ARG        # nv
    assert f(FAKE, 16, 60, FAKE, 64, 1, FAKE, None, None) == L.DIT_ERR_SHAPE      # I % 8
    assert f(FAKE, 16, 8192, FAKE, 8192, 1, FAKE, None, None) == L.DIT_ERR_SHAPE  # I > 4096
    assert f(FAKE, 0, 64, FAKE, 64, 1, FAKE, None, None) == L.DIT_ERR_SHAPE       # O
    assert f(FAKE, 16, 64, FAKE, 32, 1, FAKE, None, None) == L.DIT_ERR_SHAPE      # ldx < I
    assert f(FAKE, 1 << 20, 4096, FAKE, 4096, 1, FAKE, None, None) == L.DIT_ERR_SHAPE   # 8 GiB of W
    assert "I a multiple of 8" in L.dit_last_error()
