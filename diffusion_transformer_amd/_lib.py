"""ctypes binding of ``libdit.so`` (include/dit.h), one Python function per C
entry point with the same name. Argument marshalling only: torch tensors
are passed as raw device pointers, every computation happens in the HIP
library. Importing this module raises if the library is not built.

torch is imported before the library is opened on purpose: torch ships its
own HIP runtime (soname libamdhip64.so.7) and the library must bind to that
same instance, so that torch's device pointers and stream handles are valid
inside it. Opened first, the library would pull in the system runtime and
torch would then load a second one next to it."""
from __future__ import annotations

import ctypes as C
import ctypes as C_  # for wrappers whose arguments shadow C
import os

import numpy as np
import torch  # noqa: F401  (see above: one HIP runtime per process)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdit.so")

DIT_OK, DIT_ERR_ARG, DIT_ERR_SHAPE, DIT_ERR_LAYOUT, DIT_ERR_STATE, DIT_ERR_WORKSPACE, \
    DIT_ERR_HIP, DIT_ERR_UNSUPPORTED = range(8)
DIT_FLAG_NO_CAUSAL_CONDITION = 1
PROF = {"off": 0, "gemm_qkv": 1, "gemm_o": 2, "gemm_gateup": 3, "gemm_down": 4,
        "attention": 5, "ln": 6, "qknorm_rope": 7, "final": 8, "img_in": 9, "gemv": 10,
        "gemv_mod": 11}
SEG_TEXT, SEG_REF, SEG_TARGET = 0, 1, 2

EXPORTS = ["dit_build_layout", "dit_load_weights", "dit_free", "dit_workspace_bytes",
           "dit_kv_capacity", "dit_kv_cache_bytes", "dit_step_extract", "dit_step_cached",
           "dit_step_cached_noalloc",
           "euler_update", "dit_img_in", "dit_latent_standardize", "dit_debug_mask", "dit_debug_attention",
           "dit_debug_gemm", "dit_debug_final_out", "dit_debug_gemv", "dit_debug_stream_copy", "dit_debug_mfma_loop",
           "dit_profile_enable", "dit_profile_read",
           "dit_last_error",
           "dit_version"]


class DitError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"dit status {status}: {msg}")
        self.status = status


class dit_config(C.Structure):
    _fields_ = [("hidden", C.c_int), ("n_heads", C.c_int), ("head_dim", C.c_int),
                ("ffn", C.c_int), ("n_layers", C.c_int), ("latent", C.c_int),
                ("time_dim", C.c_int), ("rope_dims", C.c_int * 3),
                ("rope_base", C.c_float), ("eps", C.c_float)]


class dit_weights(C.Structure):
    _fields_ = [("t1", C.c_void_p), ("t2", C.c_void_p), ("mod", C.c_void_p), ("so", C.c_void_p),
                ("img_in", C.c_void_p), ("proj_out", C.c_void_p),
                ("qkv", C.POINTER(C.c_void_p)), ("q_norm", C.POINTER(C.c_void_p)),
                ("k_norm", C.POINTER(C.c_void_p)), ("o", C.POINTER(C.c_void_p)),
                ("gate", C.POINTER(C.c_void_p)), ("up", C.POINTER(C.c_void_p)),
                ("down", C.POINTER(C.c_void_p))]


class dit_seq(C.Structure):
    _fields_ = [("P", C.c_int), ("T", C.c_int), ("d_row_limit", C.c_void_p),
                ("d_rope_cos", C.c_void_p), ("d_rope_sin", C.c_void_p), ("B", C.c_int)]


class dit_gemm_desc(C.Structure):
    _fields_ = [("epilogue", C.c_int), ("M", C.c_int), ("N", C.c_int), ("K", C.c_int),
                ("A", C.c_void_p), ("B", C.c_void_p), ("B2", C.c_void_p), ("C", C.c_void_p),
                ("h", C.c_void_p), ("gate_t", C.c_void_p), ("gate_0", C.c_void_p),
                ("n_pre", C.c_int), ("q_norm", C.c_void_p), ("k_norm", C.c_void_p),
                ("rope_cos", C.c_void_p), ("rope_sin", C.c_void_p), ("kv_cache", C.c_void_p),
                ("n_heads", C.c_int), ("S", C.c_int), ("q_row0", C.c_int), ("eps", C.c_float),
                ("splits", C.c_int), ("scratch", C.c_void_p), ("scratch_bytes", C.c_size_t)]


DIT_GEMM = {"bf16": 0, "resid": 2, "swiglu": 3, "qkv": 5}


def _load(path=None):
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() "
                          "or python diffusion_transformer_amd/build.py")
    lib = C.CDLL(path)
    vp, i, f, sz, ll = C.c_void_p, C.c_int, C.c_float, C.c_size_t, C.c_longlong
    P = C.POINTER
    sig = {
        "dit_build_layout": (i, [P(dit_config), P(i), P(i), P(i), i, vp, vp, vp, vp, vp, P(i), P(i)]),
        "dit_load_weights": (i, [P(dit_config), P(dit_weights), P(vp)]),
        "dit_free": (None, [vp]),
        "dit_workspace_bytes": (sz, [vp, i]),
        "dit_kv_capacity": (i, [i]),
        "dit_kv_cache_bytes": (sz, [vp, i]),
        "dit_step_extract": (i, [vp, P(dit_seq), vp, vp, f, vp, sz, vp, vp, sz, i, vp]),
        "dit_step_cached": (i, [vp, P(dit_seq), vp, f, vp, sz, vp, vp, sz, vp]),
        "dit_step_cached_noalloc": (i, [vp, P(dit_seq), vp, f, vp, sz, vp, vp]),
        "euler_update": (i, [vp, vp, f, f, ll, vp]),
        "dit_img_in": (i, [vp, vp, i, vp, vp]),
        "dit_latent_standardize": (i, [vp, vp, vp, ll, i, i, vp]),
        "dit_debug_mask": (i, [P(dit_seq), vp, vp]),
        "dit_debug_attention": (i, [P(dit_seq), i, vp, i, i, i, vp, vp, i, vp, sz, vp]),
        "dit_debug_gemm": (i, [P(dit_gemm_desc), vp]),
        "dit_debug_mfma_loop": (i, [vp, vp, i, i, vp]),
        "dit_debug_final_out": (i, [vp, i, i, i, vp, f, vp, vp, vp]),
        "dit_debug_gemv": (i, [vp, i, i, vp, i, i, vp, vp, vp]),
        "dit_debug_stream_copy": (i, [vp, vp, sz, vp]),
        "dit_profile_enable": (i, [vp, i]),
        "dit_profile_read": (i, [vp, P(C.c_double), P(ll)]),
        "dit_last_error": (C.c_char_p, []),
        "dit_version": (C.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def _ptr(t):
    """Device (or host) pointer of a torch tensor / numpy array, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if hasattr(t, "data_ptr"):
        if not t.is_contiguous():
            raise ValueError("tensor must be contiguous")
        return t.data_ptr()
    return t.ctypes.data


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_config(hidden, n_heads, head_dim, ffn, n_layers, latent=64, time_dim=256,
                rope_dims=(16, 56, 56), rope_base=10000.0, eps=1e-6, **_ignored) -> dit_config:
    c = dit_config()
    c.hidden, c.n_heads, c.head_dim, c.ffn = hidden, n_heads, head_dim, ffn
    c.n_layers, c.latent, c.time_dim = n_layers, latent, time_dim
    c.rope_dims[:] = list(rope_dims)
    c.rope_base, c.eps = rope_base, eps
    return c


def _make_api(_lib):
    """All wrappers bound to one loaded library (the production libdit.so
    or the fp32 debug build libdit_f32.so)."""

    def _check(st):
        if st != DIT_OK:
            raise DitError(st, _lib.dit_last_error().decode())

    def dit_version() -> str:
        return _lib.dit_version().decode()

    def dit_last_error() -> str:
        return _lib.dit_last_error().decode()

    def dit_build_layout(cfg: dit_config, segments):
        """segments: ("text", n) | ("ref", h, w) | ("target", h, w). Returns a
        dict of host numpy arrays (image_ids, coords, row_limit, rope_cos,
        rope_sin) and P, T."""
        kind = {"text": SEG_TEXT, "ref": SEG_REF, "target": SEG_TARGET}
        n = len(segments)
        k = (C.c_int * n)(*[kind[s[0]] for s in segments])
        r = (C.c_int * n)(*[int(s[1]) for s in segments])
        c = (C.c_int * n)(*[int(s[2]) if len(s) > 2 else 0 for s in segments])
        P, T = C.c_int(), C.c_int()
        _check(_lib.dit_build_layout(C.byref(cfg), k, r, c, n, None, None, None, None, None,
                                     C.byref(P), C.byref(T)))
        S = P.value + T.value
        half = cfg.head_dim // 2
        out = {"image_ids": np.empty(S, np.int32), "coords": np.empty((S, 3), np.int32),
               "row_limit": np.empty(S, np.int32), "rope_cos": np.empty((S, half), np.float32),
               "rope_sin": np.empty((S, half), np.float32)}
        _check(_lib.dit_build_layout(C.byref(cfg), k, r, c, n, _ptr(out["image_ids"]),
                                     _ptr(out["coords"]), _ptr(out["row_limit"]),
                                     _ptr(out["rope_cos"]), _ptr(out["rope_sin"]),
                                     C.byref(P), C.byref(T)))
        out["P"], out["T"] = P.value, T.value
        return out

    def dit_load_weights(cfg: dit_config, w: dict):
        """w: dict of device tensors (bf16 bits) t1, t2, mod, so, img_in, proj_out
        and per-layer lists qkv, q_norm, k_norm, o, gate, up, down. Returns an
        opaque handle (an int); the tensors must outlive it."""
        L = cfg.n_layers
        arrs = {}
        for name in ("qkv", "q_norm", "k_norm", "o", "gate", "up", "down"):
            arrs[name] = (C.c_void_p * L)(*[_ptr(t) for t in w[name]])
        ws = dit_weights(_ptr(w["t1"]), _ptr(w["t2"]), _ptr(w["mod"]), _ptr(w["so"]),
                         _ptr(w["img_in"]), _ptr(w["proj_out"]),
                         *[C.cast(arrs[n], C.POINTER(C.c_void_p)) for n in
                           ("qkv", "q_norm", "k_norm", "o", "gate", "up", "down")])
        h = C.c_void_p()
        _check(_lib.dit_load_weights(C.byref(cfg), C.byref(ws), C.byref(h)))
        _dims[h.value] = (cfg.hidden, cfg.latent)
        return h.value

    def dit_free(model):
        _dims.pop(model, None)
        _lib.dit_free(model)

    def dit_workspace_bytes(model, n_tokens: int) -> int:
        return _lib.dit_workspace_bytes(model, n_tokens)

    def dit_kv_capacity(S: int) -> int:
        return _lib.dit_kv_capacity(S)

    def dit_kv_cache_bytes(model, S: int) -> int:
        return _lib.dit_kv_cache_bytes(model, S)

    def make_seq(P, T, row_limit, rope_cos, rope_sin, B=1) -> dit_seq:
        """B target latents share the prefix (rows P + b*T .. of x, v, cache)."""
        return dit_seq(P, T, _ptr(row_limit), _ptr(rope_cos), _ptr(rope_sin), B)

    def _nbytes(t):
        return t.numel() * t.element_size()

    _dims = {}   # model handle -> (hidden, latent), for the host-side tensor checks

    def _need(t, what, numel, dtype=None):
        """The C ABI cannot see tensor sizes: check on the host that a tensor
        handed to a step is a contiguous float32 device tensor of the size
        the call will read or write."""
        dtype = torch.float32 if dtype is None else dtype
        ok = (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == dtype and t.is_contiguous()
              and t.numel() == numel)
        if not ok:
            desc = (f"{tuple(t.shape)} {t.dtype} on {t.device}, contiguous={t.is_contiguous()}"
                    if isinstance(t, torch.Tensor) else type(t).__name__)
            raise DitError(DIT_ERR_ARG, f"{what}: need a contiguous {dtype} device tensor of "
                                        f"{numel} elements, got {desc}")

    def _step_tensors(model, seq, x, v_out, prefix_hidden=None, extract=False):
        if model not in _dims:
            raise DitError(DIT_ERR_ARG, "model handle is not loaded")
        H, Cl = _dims[model]
        rows = max(int(seq.B), 1) * int(seq.T)
        _need(x, "x", rows * Cl)
        _need(v_out, "v_out", rows * Cl)
        if extract and (prefix_hidden is not None or seq.P > 0):
            _need(prefix_hidden, "prefix_hidden", int(seq.P) * H)

    def dit_step_extract(model, seq: dit_seq, prefix_hidden, x, sigma, kv_cache, v_out, workspace,
                         flags=0, stream=None):
        _step_tensors(model, seq, x, v_out, prefix_hidden, extract=True)
        _check(_lib.dit_step_extract(model, C.byref(seq), _ptr(prefix_hidden), _ptr(x), float(sigma),
                                     _ptr(kv_cache), _nbytes(kv_cache), _ptr(v_out), _ptr(workspace),
                                     _nbytes(workspace), int(flags), _stream(stream)))

    def dit_step_cached(model, seq: dit_seq, x, sigma, kv_cache, v_out, workspace, stream=None):
        _step_tensors(model, seq, x, v_out)
        _check(_lib.dit_step_cached(model, C.byref(seq), _ptr(x), float(sigma), _ptr(kv_cache),
                                    _nbytes(kv_cache), _ptr(v_out), _ptr(workspace),
                                    _nbytes(workspace), _stream(stream)))

    def dit_step_cached_noalloc(model, seq: dit_seq, x, sigma, kv_cache, v_out, stream=None):
        _step_tensors(model, seq, x, v_out)
        _check(_lib.dit_step_cached_noalloc(model, C.byref(seq), _ptr(x), float(sigma), _ptr(kv_cache),
                                            _nbytes(kv_cache), _ptr(v_out), _stream(stream)))

    def euler_update(x, v, sigma_k, sigma_k1, n=None, stream=None):
        n = x.numel() if n is None else int(n)
        for t, what in ((x, "x"), (v, "v")):
            if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == torch.float32
                    and t.is_contiguous() and t.numel() >= n):
                raise DitError(DIT_ERR_ARG, f"euler_update: {what} must be a contiguous float32 "
                                            f"device tensor of at least {n} elements")
        _check(_lib.euler_update(_ptr(x), _ptr(v), float(sigma_k), float(sigma_k1), int(n),
                                 _stream(stream)))

    def dit_img_in(model, latents, hidden, stream=None):
        _check(_lib.dit_img_in(model, _ptr(latents), int(latents.shape[0]), _ptr(hidden),
                               _stream(stream)))

    def dit_latent_standardize(z, mean, std, inverse=False, stream=None):
        """In place on a contiguous float32 [rows, C] device tensor."""
        _check(_lib.dit_latent_standardize(_ptr(z), _ptr(mean), _ptr(std), int(z.shape[0]),
                                           int(z.shape[1]), int(bool(inverse)), _stream(stream)))

    def dit_debug_mask(seq: dit_seq, mask, stream=None):
        _check(_lib.dit_debug_mask(C.byref(seq), _ptr(mask), _stream(stream)))

    def dit_debug_attention(seq: dit_seq, n_heads, q, q_stride, q_off, N, kv_cache, out, variant=0,
                            scratch=None, stream=None):
        _check(_lib.dit_debug_attention(C.byref(seq), int(n_heads), _ptr(q), int(q_stride), int(q_off),
                                        int(N), _ptr(kv_cache), _ptr(out), int(variant), _ptr(scratch),
                                        _nbytes(scratch) if scratch is not None else 0,
                                        _stream(stream)))

    def dit_debug_gemm(epilogue, M, N, K, A, B, C=None, B2=None, h=None, gate_t=None, gate_0=None,
                       n_pre=0, q_norm=None, k_norm=None, rope_cos=None, rope_sin=None,
                       kv_cache=None, n_heads=0, S=0, q_row0=0, eps=1e-6, splits=0, scratch=None,
                       stream=None):
        """``epilogue``: one of DIT_GEMM's names or values (see dit_gemm_desc)."""
        d = dit_gemm_desc()
        d.epilogue = DIT_GEMM.get(epilogue, epilogue) if isinstance(epilogue, str) else int(epilogue)
        d.M, d.N, d.K = int(M), int(N), int(K)
        d.A, d.B, d.B2, d.C = _ptr(A), _ptr(B), _ptr(B2), _ptr(C)
        d.h, d.gate_t, d.gate_0, d.n_pre = _ptr(h), _ptr(gate_t), _ptr(gate_0), int(n_pre)
        d.q_norm, d.k_norm, d.rope_cos, d.rope_sin = _ptr(q_norm), _ptr(k_norm), _ptr(rope_cos), \
            _ptr(rope_sin)
        d.kv_cache, d.n_heads, d.S, d.q_row0, d.eps = _ptr(kv_cache), int(n_heads), int(S), \
            int(q_row0), float(eps)
        d.splits = int(splits)
        d.scratch = _ptr(scratch)
        d.scratch_bytes = _nbytes(scratch) if scratch is not None else 0
        _check(_lib.dit_debug_gemm(C_.byref(d), _stream(stream)))

    def dit_debug_final_out(h, scale_out, w_out, v_out, eps=1e-6, stream=None):
        """h [rows, H] f32, scale_out [H] f32, w_out [64, H] bf16, v_out [rows, 64] f32."""
        _check(_lib.dit_debug_final_out(_ptr(h), int(h.shape[1]), int(h.shape[0]), int(h.shape[1]),
                                        _ptr(scale_out), float(eps), _ptr(w_out), _ptr(v_out),
                                        _stream(stream)))

    def dit_debug_gemv(W, X, Y, Ys=None, stream=None):
        """W [O, I] bf16, X [nv, I] f32, Y (and Ys) [nv, O] f32; all contiguous device tensors."""
        O_, I_ = int(W.shape[0]), int(W.shape[1])
        _check(_lib.dit_debug_gemv(_ptr(W), O_, I_, _ptr(X), I_, int(X.shape[0]), _ptr(Y), _ptr(Ys),
                                   _stream(stream)))

    def dit_debug_stream_copy(src, dst, stream=None):
        _check(_lib.dit_debug_stream_copy(_ptr(src), _ptr(dst), _nbytes(src), _stream(stream)))

    def dit_debug_mfma_loop(ops, out, blocks, iters, stream=None):
        _check(_lib.dit_debug_mfma_loop(_ptr(ops), _ptr(out), int(blocks), int(iters),
                                        _stream(stream)))

    def dit_profile_enable(model, kernel_class):
        if isinstance(kernel_class, str):
            kernel_class = PROF[kernel_class]
        _check(_lib.dit_profile_enable(model, int(kernel_class)))

    def dit_profile_read(model):
        ms, n = C.c_double(), C.c_longlong()
        _check(_lib.dit_profile_read(model, C.byref(ms), C.byref(n)))
        return ms.value, n.value

    return {k: v for k, v in locals().items() if k.startswith(("dit_", "euler_", "make_seq"))}


def _bind(path):
    import types
    lib = _load(path)
    ns = types.SimpleNamespace(**_make_api(lib))
    ns._lib = lib
    ns.make_config = make_config
    ns.DitError = DitError
    for k in ("DIT_OK", "DIT_ERR_ARG", "DIT_ERR_SHAPE", "DIT_ERR_LAYOUT", "DIT_ERR_STATE",
              "DIT_ERR_WORKSPACE", "DIT_ERR_HIP", "DIT_ERR_UNSUPPORTED", "DIT_FLAG_NO_CAUSAL_CONDITION",
              "PROF", "DIT_GEMM", "dit_seq", "dit_config", "dit_weights", "dit_gemm_desc"):
        setattr(ns, k, globals()[k])
    return ns


_default = _bind(LIB_PATH)
_lib = _default._lib
globals().update({k: v for k, v in vars(_default).items() if k.startswith(("dit_", "euler_", "make_seq"))})

LIB_F32_PATH = os.path.join(_PKG, "libdit_f32.so")


def load_f32():
    """The same API bound to the fp32 debug build (libdit_f32.so)."""
    return _bind(LIB_F32_PATH)
