"""Python binding of the Gemma decoder-attention library (libgemma_attn.so, gfx950).

Argument marshalling only: tensors are checked for dtype, device, shape and
contiguity, then their device pointers and the current HIP stream are passed
to the C ABI declared in ``include/gemma_attn.h``.  Every step of the
computation runs in the library's HIP kernels; there is no fallback, and a
missing library raises.

Tensor conventions (torch, on the GPU):
  q [B,S,Hq,D], k and v [B,S,Hkv,D], caches [B,Smax,Hkv,D]: torch.bfloat16
  norm weights [D]: torch.float32;  pos0, ctx_len [B]: torch.int32
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
# GEMMA_ATTN_LIBRARY selects another build of the same library by path (the
# tests use it for the LDS-poisoning debug build, libgemma_attn_ldsnan.so).
LIB_PATH = os.environ.get("GEMMA_ATTN_LIBRARY") or os.path.join(_HERE, "libgemma_attn.so")

GA_OK, GA_ERR_INVALID_ARG, GA_ERR_UNSUPPORTED, GA_ERR_WORKSPACE, GA_ERR_HIP, GA_ERR_SCRATCH_LIMIT = 0, 1, 2, 3, 4, 5


class GemmaAttnError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {_strerror(code)} (code {code})")
        self.code = code


class CConfig(ctypes.Structure):
    """Mirror of ``gemma_attn_config``."""

    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("num_global_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("global_head_dim", ctypes.c_int32),
        ("sliding_window", ctypes.c_int32),
        ("sliding_window_pattern", ctypes.c_int32),
        ("k_eq_v", ctypes.c_int32),
        ("norm_weight_offset", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("rope_local_theta", ctypes.c_double),
        ("partial_rotary_factor", ctypes.c_double),
        ("attn_logit_softcapping", ctypes.c_double),
        ("query_pre_attn_scalar", ctypes.c_double),
        ("norm_eps", ctypes.c_double),
        ("rope_scaling_factor", ctypes.c_double),
    ]


class CLayer(ctypes.Structure):
    """Mirror of ``gemma_attn_layer``."""

    _fields_ = [
        ("is_global", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("rotary_dim", ctypes.c_int32),
        ("k_eq_v", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("theta", ctypes.c_double),
        ("scale", ctypes.c_double),
        ("softcap", ctypes.c_double),
        ("pos_div", ctypes.c_double),
    ]


@dataclass
class Config:
    """The pages' attention knobs (same names and meanings as the C struct)."""

    num_heads: int
    num_kv_heads: int
    head_dim: int
    num_global_kv_heads: int = 0
    global_head_dim: int = 0
    sliding_window: int = 0
    sliding_window_pattern: int = 1
    rope_theta: float = 10000.0
    rope_local_theta: float = 0.0
    partial_rotary_factor: float = 1.0
    attn_logit_softcapping: float = 0.0
    query_pre_attn_scalar: float = 0.0
    k_eq_v: bool = False
    norm_eps: float = 1e-6
    norm_weight_offset: int = 0
    rope_scaling_factor: float = 0.0

    def to_c(self) -> CConfig:
        return CConfig(
            num_heads=int(self.num_heads), num_kv_heads=int(self.num_kv_heads),
            num_global_kv_heads=int(self.num_global_kv_heads), head_dim=int(self.head_dim),
            global_head_dim=int(self.global_head_dim), sliding_window=int(self.sliding_window),
            sliding_window_pattern=int(self.sliding_window_pattern), k_eq_v=int(bool(self.k_eq_v)),
            norm_weight_offset=int(self.norm_weight_offset), reserved=0,
            rope_theta=float(self.rope_theta), rope_local_theta=float(self.rope_local_theta),
            partial_rotary_factor=float(self.partial_rotary_factor),
            attn_logit_softcapping=float(self.attn_logit_softcapping),
            query_pre_attn_scalar=float(self.query_pre_attn_scalar), norm_eps=float(self.norm_eps),
            rope_scaling_factor=float(self.rope_scaling_factor or 0.0))

    @classmethod
    def from_any(cls, obj) -> "Config":
        if isinstance(obj, Config):
            return obj
        if isinstance(obj, dict):
            return cls(**obj)
        return cls(**{f: getattr(obj, f) for f in cls.__dataclass_fields__ if hasattr(obj, f)})


_lib = None
_VP = ctypes.c_void_p


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the built library (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m decoder_attention_amd.build`")
    # torch ships its own HIP runtime under the soname the library links
    # against.  Loaded first, the library would pull in the system runtime and
    # torch would then load its own beside it: two runtimes in one process,
    # and the library's launches on torch's streams fail.  With torch loaded
    # first, the library binds to torch's runtime.
    import torch  # noqa: F401

    lib = ctypes.CDLL(p)
    i32, cfgp = ctypes.c_int32, ctypes.POINTER(CConfig)
    lib.gemma_attn_resolve_layer.argtypes = [cfgp, i32, ctypes.POINTER(CLayer)]
    lib.gemma_attn_resolve_layer.restype = ctypes.c_int
    lib.gemma_attn_strerror.argtypes = [ctypes.c_int]
    lib.gemma_attn_strerror.restype = ctypes.c_char_p
    lib.gemma_qk_prologue.argtypes = [cfgp, i32, i32, i32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]
    lib.gemma_qk_prologue.restype = ctypes.c_int
    lib.gemma_attn_prefill.argtypes = [cfgp, i32, i32, i32, _VP, _VP, _VP, _VP, _VP, _VP]
    lib.gemma_attn_prefill.restype = ctypes.c_int
    lib.gemma_attn_decode_workspace_size.argtypes = [cfgp, i32, i32, i32]
    lib.gemma_attn_decode_workspace_size.restype = ctypes.c_size_t
    lib.gemma_attn_decode.argtypes = [cfgp, i32, i32, i32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]
    lib.gemma_attn_decode.restype = ctypes.c_int
    lib.gemma_attn_decode_multi.argtypes = [cfgp, i32, i32, i32, i32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                            ctypes.c_size_t, _VP]
    lib.gemma_attn_decode_multi.restype = ctypes.c_int
    lib.gemma_attn_decode_multi_noalloc.argtypes = [cfgp, i32, i32, i32, i32, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                                    _VP]
    lib.gemma_attn_decode_multi_noalloc.restype = ctypes.c_int
    lib.gemma_attn_decode_multi_workspace_size.argtypes = [cfgp, i32, i32, i32, i32]
    lib.gemma_attn_decode_multi_workspace_size.restype = ctypes.c_size_t
    lib.gemma_qk_prologue_cache.argtypes = [cfgp, i32, i32, i32, i32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]
    lib.gemma_qk_prologue_cache.restype = ctypes.c_int
    lib.gemma_attn_decode_int8.argtypes = [cfgp, i32, i32, i32, i32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                           _VP, ctypes.c_size_t, _VP]
    lib.gemma_attn_prefill_ragged.argtypes = [cfgp, i32, i32, i32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]
    lib.gemma_attn_prefill_ragged.restype = ctypes.c_int
    lib.gemma_attn_prefill_qrope.argtypes = [cfgp, i32, i32, i32, _VP, _VP, _VP, _VP, _VP, _VP, _VP]
    lib.gemma_attn_prefill_qrope.restype = ctypes.c_int
    lib.gemma_attn_decode_int8.restype = ctypes.c_int
    lib.gemma_qk_prologue_cache_int8.argtypes = [cfgp, i32, i32, i32, i32] + [_VP] * 12
    lib.gemma_qk_prologue_cache_int8.restype = ctypes.c_int
    lib.gemma_kv_quantize_int8.argtypes = [i32, i32, i32, i32, i32, _VP, _VP, _VP, _VP, _VP]
    lib.gemma_kv_quantize_int8.restype = ctypes.c_int
    _lib = lib
    return lib


def _strerror(code: int) -> str:
    try:
        return load().gemma_attn_strerror(int(code)).decode()
    except Exception:  # pragma: no cover
        return "error"


def _check(rc: int, what: str) -> None:
    if rc != GA_OK:
        raise GemmaAttnError(rc, what)


def resolve_layer(cfg, layer_idx: int) -> dict:
    c = Config.from_any(cfg).to_c()
    out = CLayer()
    _check(load().gemma_attn_resolve_layer(ctypes.byref(c), int(layer_idx), ctypes.byref(out)), "resolve_layer")
    return {f: getattr(out, f) for f, _ in CLayer._fields_ if f != "reserved"}


# ----------------------------------------------------------------------------- tensor helpers
def _ptr(t, dtype=None, name="tensor"):
    import torch

    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream):
    import torch

    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _expect(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


# ----------------------------------------------------------------------------- entry points
def qk_prologue(cfg, layer_idx, q, k=None, q_out=None, k_out=None, q_norm_w=None, k_norm_w=None,
                pos0=None, stream=None):
    """gemma_qk_prologue; returns (q_out, k_out).  Pass q_out=q for in place; q=None processes the keys
    only (q_out is then None)."""
    import torch

    cfg = Config.from_any(cfg)
    L = resolve_layer(cfg, layer_idx)
    if q is None and k is None:
        raise ValueError("qk_prologue needs q or k")
    B, S = (q if q is not None else k).shape[:2]
    if q is not None:
        _expect(q, (B, S, cfg.num_heads, L["head_dim"]), "q")
    if k is not None:
        _expect(k, (B, S, L["num_kv_heads"], L["head_dim"]), "k")
    if q is None:
        q_out = None
    elif q_out is None:
        q_out = torch.empty_like(q)
    if q is not None:
        _expect(q_out, tuple(q.shape), "q_out")
    if k is not None and k_out is None:
        k_out = torch.empty_like(k)
    if k is not None:
        _expect(k_out, tuple(k.shape), "k_out")
    for w, n in ((q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w")):
        if w is not None:
            _expect(w, (L["head_dim"],), n)
    if pos0 is not None:
        _expect(pos0, (B,), "pos0")
    bf = torch.bfloat16
    rc = load().gemma_qk_prologue(
        ctypes.byref(cfg.to_c()), int(layer_idx), B, S, _ptr(q, bf, "q"), _ptr(k, bf, "k"),
        _ptr(q_out, bf, "q_out") if q is not None else None, _ptr(k_out, bf, "k_out") if k is not None else None,
        _ptr(q_norm_w, torch.float32, "q_norm_w"), _ptr(k_norm_w, torch.float32, "k_norm_w"),
        _ptr(pos0, torch.int32, "pos0"), _stream(stream))
    _check(rc, "gemma_qk_prologue")
    return q_out, k_out


def attn_prefill(cfg, layer_idx, q, k, v=None, out=None, lse=None, want_lse=False, stream=None, seq_start=None,
                 seq_end=None):
    """gemma_attn_prefill (gemma_attn_prefill_ragged when seq_start or seq_end [B] int32 is given: sequence b
    keeps rows [start, end)); returns out, or (out, lse) when an lse buffer is asked for."""
    import torch

    cfg = Config.from_any(cfg)
    L = resolve_layer(cfg, layer_idx)
    B, S = q.shape[0], q.shape[1]
    _expect(q, (B, S, cfg.num_heads, L["head_dim"]), "q")
    _expect(k, (B, S, L["num_kv_heads"], L["head_dim"]), "k")
    if v is not None and not L["k_eq_v"]:
        _expect(v, (B, S, L["num_kv_heads"], L["head_dim"]), "v")
    if out is None:
        out = torch.empty_like(q)
    _expect(out, tuple(q.shape), "out")
    if want_lse and lse is None:
        lse = torch.empty((B, cfg.num_heads, S), dtype=torch.float32, device=q.device)
    if lse is not None:
        _expect(lse, (B, cfg.num_heads, S), "lse")
    bf = torch.bfloat16
    args = (ctypes.byref(cfg.to_c()), int(layer_idx), B, S, _ptr(q, bf, "q"), _ptr(k, bf, "k"),
            None if L["k_eq_v"] else _ptr(v, bf, "v"), _ptr(out, bf, "out"), _ptr(lse, torch.float32, "lse"))
    if seq_start is None and seq_end is None:
        _check(load().gemma_attn_prefill(*args, _stream(stream)), "gemma_attn_prefill")
    else:
        for t, n in ((seq_start, "seq_start"), (seq_end, "seq_end")):
            if t is not None:
                _expect(t, (B,), n)
        rc = load().gemma_attn_prefill_ragged(*args, _ptr(seq_start, torch.int32, "seq_start"),
                                              _ptr(seq_end, torch.int32, "seq_end"), _stream(stream))
        _check(rc, "gemma_attn_prefill_ragged")
    return (out, lse) if lse is not None else out


def attn_prefill_qrope(cfg, layer_idx, q_raw, k, v=None, pos0=None, out=None, lse=None, want_lse=False,
                       stream=None):
    """gemma_attn_prefill_qrope: q_raw [B,S,Hq,D] before rotary (rotated inside the attention kernel), k already
    processed (qk_prologue with q=None); returns out, or (out, lse) when an lse buffer is asked for."""
    import torch

    cfg = Config.from_any(cfg)
    L = resolve_layer(cfg, layer_idx)
    B, S = q_raw.shape[0], q_raw.shape[1]
    _expect(q_raw, (B, S, cfg.num_heads, L["head_dim"]), "q_raw")
    _expect(k, (B, S, L["num_kv_heads"], L["head_dim"]), "k")
    if v is not None and not L["k_eq_v"]:
        _expect(v, (B, S, L["num_kv_heads"], L["head_dim"]), "v")
    if pos0 is not None:
        _expect(pos0, (B,), "pos0")
    if out is None:
        out = torch.empty_like(q_raw)
    _expect(out, tuple(q_raw.shape), "out")
    if want_lse and lse is None:
        lse = torch.empty((B, cfg.num_heads, S), dtype=torch.float32, device=q_raw.device)
    if lse is not None:
        _expect(lse, (B, cfg.num_heads, S), "lse")
    bf = torch.bfloat16
    rc = load().gemma_attn_prefill_qrope(
        ctypes.byref(cfg.to_c()), int(layer_idx), B, S, _ptr(q_raw, bf, "q_raw"), _ptr(k, bf, "k"),
        None if L["k_eq_v"] else _ptr(v, bf, "v"), _ptr(pos0, torch.int32, "pos0"), _ptr(out, bf, "out"),
        _ptr(lse, torch.float32, "lse"), _stream(stream))
    _check(rc, "gemma_attn_prefill_qrope")
    return (out, lse) if lse is not None else out


def decode_workspace_size(cfg, layer_idx, batch, max_ctx) -> int:
    cfg = Config.from_any(cfg)
    return int(load().gemma_attn_decode_workspace_size(ctypes.byref(cfg.to_c()), int(layer_idx), int(batch),
                                                       int(max_ctx)))


def attn_decode(cfg, layer_idx, q, k_cache, v_cache, ctx_len, out=None, lse=None, want_lse=False,
                workspace=None, stream=None):
    """gemma_attn_decode; q [B,Hq,D]; returns out, or (out, lse)."""
    import torch

    cfg = Config.from_any(cfg)
    L = resolve_layer(cfg, layer_idx)
    B, Smax = k_cache.shape[0], k_cache.shape[1]
    _expect(q, (B, cfg.num_heads, L["head_dim"]), "q")
    _expect(k_cache, (B, Smax, L["num_kv_heads"], L["head_dim"]), "k_cache")
    if v_cache is not None and not L["k_eq_v"]:
        _expect(v_cache, (B, Smax, L["num_kv_heads"], L["head_dim"]), "v_cache")
    _expect(ctx_len, (B,), "ctx_len")
    if out is None:
        out = torch.empty_like(q)
    _expect(out, tuple(q.shape), "out")
    if want_lse and lse is None:
        lse = torch.empty((B, cfg.num_heads), dtype=torch.float32, device=q.device)
    if lse is not None:
        _expect(lse, (B, cfg.num_heads), "lse")
    need = decode_workspace_size(cfg, layer_idx, B, Smax)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    bf = torch.bfloat16
    rc = load().gemma_attn_decode(
        ctypes.byref(cfg.to_c()), int(layer_idx), B, Smax, _ptr(q, bf, "q"), _ptr(k_cache, bf, "k_cache"),
        None if L["k_eq_v"] else _ptr(v_cache, bf, "v_cache"), _ptr(ctx_len, torch.int32, "ctx_len"),
        _ptr(out, bf, "out"), _ptr(lse, torch.float32, "lse"), _ptr(workspace, None, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "gemma_attn_decode")
    return (out, lse) if lse is not None else out


def decode_multi_workspace_size(cfg, layer_idx, batch, q_len, max_ctx) -> int:
    cfg = Config.from_any(cfg)
    return int(load().gemma_attn_decode_multi_workspace_size(ctypes.byref(cfg.to_c()), int(layer_idx), int(batch),
                                                             int(q_len), int(max_ctx)))


def attn_decode_multi(cfg, layer_idx, q, k_cache, v_cache, ctx_len, out=None, lse=None, want_lse=False,
                      workspace=None, stream=None, kv_start=None):
    """gemma_attn_decode_multi; q [B,L,Hq,D]; returns out [B,L,Hq,D], or (out, lse [B,Hq,L])."""
    import torch

    cfg = Config.from_any(cfg)
    L = resolve_layer(cfg, layer_idx)
    B, Lq = q.shape[0], q.shape[1]
    Smax = k_cache.shape[1]
    _expect(q, (B, Lq, cfg.num_heads, L["head_dim"]), "q")
    _expect(k_cache, (B, Smax, L["num_kv_heads"], L["head_dim"]), "k_cache")
    if v_cache is not None and not L["k_eq_v"]:
        _expect(v_cache, (B, Smax, L["num_kv_heads"], L["head_dim"]), "v_cache")
    _expect(ctx_len, (B,), "ctx_len")
    if kv_start is not None:
        _expect(kv_start, (B,), "kv_start")
    if out is None:
        out = torch.empty_like(q)
    _expect(out, tuple(q.shape), "out")
    if want_lse and lse is None:
        lse = torch.empty((B, cfg.num_heads, Lq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _expect(lse, (B, cfg.num_heads, Lq), "lse")
    need = decode_multi_workspace_size(cfg, layer_idx, B, Lq, Smax)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    bf = torch.bfloat16
    rc = load().gemma_attn_decode_multi(
        ctypes.byref(cfg.to_c()), int(layer_idx), B, Lq, Smax, _ptr(q, bf, "q"), _ptr(k_cache, bf, "k_cache"),
        None if L["k_eq_v"] else _ptr(v_cache, bf, "v_cache"), _ptr(ctx_len, torch.int32, "ctx_len"),
        _ptr(kv_start, torch.int32, "kv_start"), _ptr(out, bf, "out"), _ptr(lse, torch.float32, "lse"),
        _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "gemma_attn_decode_multi")
    return (out, lse) if lse is not None else out


def attn_decode_multi_noalloc(cfg, layer_idx, q, k_cache, v_cache, ctx_len, out, lse=None, stream=None,
                              kv_start=None):
    """gemma_attn_decode_multi_noalloc: decode_multi with the library's own fixed scratch array as workspace;
    the caller passes every output (nothing is allocated here either).  Calls overlapping on one GPU race.
    Returns out, or (out, lse) when lse is given."""
    import torch

    cfg = Config.from_any(cfg)
    L = resolve_layer(cfg, layer_idx)
    B, Lq = q.shape[0], q.shape[1]
    Smax = k_cache.shape[1]
    _expect(q, (B, Lq, cfg.num_heads, L["head_dim"]), "q")
    _expect(k_cache, (B, Smax, L["num_kv_heads"], L["head_dim"]), "k_cache")
    if v_cache is not None and not L["k_eq_v"]:
        _expect(v_cache, (B, Smax, L["num_kv_heads"], L["head_dim"]), "v_cache")
    _expect(ctx_len, (B,), "ctx_len")
    if kv_start is not None:
        _expect(kv_start, (B,), "kv_start")
    _expect(out, tuple(q.shape), "out")
    if lse is not None:
        _expect(lse, (B, cfg.num_heads, Lq), "lse")
    bf = torch.bfloat16
    rc = load().gemma_attn_decode_multi_noalloc(
        ctypes.byref(cfg.to_c()), int(layer_idx), B, Lq, Smax, _ptr(q, bf, "q"), _ptr(k_cache, bf, "k_cache"),
        None if L["k_eq_v"] else _ptr(v_cache, bf, "v_cache"), _ptr(ctx_len, torch.int32, "ctx_len"),
        _ptr(kv_start, torch.int32, "kv_start"), _ptr(out, bf, "out"), _ptr(lse, torch.float32, "lse"),
        _stream(stream))
    _check(rc, "gemma_attn_decode_multi_noalloc")
    return (out, lse) if lse is not None else out


def qk_prologue_cache(cfg, layer_idx, q, k, v, k_cache, v_cache, ctx_len, q_out=None, q_norm_w=None, k_norm_w=None,
                      stream=None):
    """gemma_qk_prologue_cache: q [B,L,Hq,D] -> q_out; k (normed, rotated) and v (copied) appended to the
    caches at rows ctx_len[b] - L + s.  Returns q_out."""
    import torch

    cfg = Config.from_any(cfg)
    L = resolve_layer(cfg, layer_idx)
    B, Lq = q.shape[0], q.shape[1]
    Smax = k_cache.shape[1]
    D, Hkv = L["head_dim"], L["num_kv_heads"]
    _expect(q, (B, Lq, cfg.num_heads, D), "q")
    _expect(k, (B, Lq, Hkv, D), "k")
    _expect(k_cache, (B, Smax, Hkv, D), "k_cache")
    if not L["k_eq_v"]:
        _expect(v, (B, Lq, Hkv, D), "v")
        _expect(v_cache, (B, Smax, Hkv, D), "v_cache")
    _expect(ctx_len, (B,), "ctx_len")
    if q_out is None:
        q_out = torch.empty_like(q)
    _expect(q_out, tuple(q.shape), "q_out")
    bf = torch.bfloat16
    rc = load().gemma_qk_prologue_cache(
        ctypes.byref(cfg.to_c()), int(layer_idx), B, Lq, Smax, _ptr(q, bf, "q"), _ptr(k, bf, "k"),
        None if L["k_eq_v"] else _ptr(v, bf, "v"), _ptr(q_out, bf, "q_out"), _ptr(k_cache, bf, "k_cache"),
        None if L["k_eq_v"] else _ptr(v_cache, bf, "v_cache"), _ptr(q_norm_w, torch.float32, "q_norm_w"),
        _ptr(k_norm_w, torch.float32, "k_norm_w"), _ptr(ctx_len, torch.int32, "ctx_len"), _stream(stream))
    _check(rc, "gemma_qk_prologue_cache")
    return q_out


# ----------------------------------------------------------------------------- int8 KV cache
# codes [B,Smax,Hkv,D] torch.int8; scales [B,Hkv,Smax] torch.float32 (one per token and head).
def attn_decode_int8(cfg, layer_idx, q, k_codes, k_scales, v_codes, v_scales, ctx_len, out=None, lse=None,
                     want_lse=False, workspace=None, stream=None, kv_start=None):
    """gemma_attn_decode_int8; q [B,L,Hq,D]; returns out [B,L,Hq,D], or (out, lse [B,Hq,L])."""
    import torch

    cfg = Config.from_any(cfg)
    L = resolve_layer(cfg, layer_idx)
    B, Lq = q.shape[0], q.shape[1]
    Smax = k_codes.shape[1]
    D, Hkv = L["head_dim"], L["num_kv_heads"]
    _expect(q, (B, Lq, cfg.num_heads, D), "q")
    _expect(k_codes, (B, Smax, Hkv, D), "k_codes")
    _expect(k_scales, (B, Hkv, Smax), "k_scales")
    if not L["k_eq_v"]:
        _expect(v_codes, (B, Smax, Hkv, D), "v_codes")
        _expect(v_scales, (B, Hkv, Smax), "v_scales")
    _expect(ctx_len, (B,), "ctx_len")
    if kv_start is not None:
        _expect(kv_start, (B,), "kv_start")
    if out is None:
        out = torch.empty_like(q)
    _expect(out, tuple(q.shape), "out")
    if want_lse and lse is None:
        lse = torch.empty((B, cfg.num_heads, Lq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _expect(lse, (B, cfg.num_heads, Lq), "lse")
    need = decode_multi_workspace_size(cfg, layer_idx, B, Lq, Smax)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    kv = not L["k_eq_v"]
    rc = load().gemma_attn_decode_int8(
        ctypes.byref(cfg.to_c()), int(layer_idx), B, Lq, Smax, _ptr(q, torch.bfloat16, "q"),
        _ptr(k_codes, torch.int8, "k_codes"), _ptr(k_scales, torch.float32, "k_scales"),
        _ptr(v_codes, torch.int8, "v_codes") if kv else None, _ptr(v_scales, torch.float32, "v_scales") if kv else None,
        _ptr(ctx_len, torch.int32, "ctx_len"), _ptr(kv_start, torch.int32, "kv_start"),
        _ptr(out, torch.bfloat16, "out"), _ptr(lse, torch.float32, "lse"),
        _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, "gemma_attn_decode_int8")
    return (out, lse) if lse is not None else out


def qk_prologue_cache_int8(cfg, layer_idx, q, k, v, k_codes, k_scales, v_codes, v_scales, ctx_len, q_out=None,
                           q_norm_w=None, k_norm_w=None, stream=None):
    """gemma_qk_prologue_cache_int8: like qk_prologue_cache, appending to an int8 cache.  Returns q_out."""
    import torch

    cfg = Config.from_any(cfg)
    L = resolve_layer(cfg, layer_idx)
    B, Lq = q.shape[0], q.shape[1]
    Smax = k_codes.shape[1]
    D, Hkv = L["head_dim"], L["num_kv_heads"]
    _expect(q, (B, Lq, cfg.num_heads, D), "q")
    _expect(k, (B, Lq, Hkv, D), "k")
    _expect(k_codes, (B, Smax, Hkv, D), "k_codes")
    _expect(k_scales, (B, Hkv, Smax), "k_scales")
    kv = not L["k_eq_v"]
    if kv:
        _expect(v, (B, Lq, Hkv, D), "v")
        _expect(v_codes, (B, Smax, Hkv, D), "v_codes")
        _expect(v_scales, (B, Hkv, Smax), "v_scales")
    _expect(ctx_len, (B,), "ctx_len")
    if q_out is None:
        q_out = torch.empty_like(q)
    _expect(q_out, tuple(q.shape), "q_out")
    bf = torch.bfloat16
    rc = load().gemma_qk_prologue_cache_int8(
        ctypes.byref(cfg.to_c()), int(layer_idx), B, Lq, Smax, _ptr(q, bf, "q"), _ptr(k, bf, "k"),
        _ptr(v, bf, "v") if kv else None, _ptr(q_out, bf, "q_out"), _ptr(k_codes, torch.int8, "k_codes"),
        _ptr(k_scales, torch.float32, "k_scales"), _ptr(v_codes, torch.int8, "v_codes") if kv else None,
        _ptr(v_scales, torch.float32, "v_scales") if kv else None, _ptr(q_norm_w, torch.float32, "q_norm_w"),
        _ptr(k_norm_w, torch.float32, "k_norm_w"), _ptr(ctx_len, torch.int32, "ctx_len"), _stream(stream))
    _check(rc, "gemma_qk_prologue_cache_int8")
    return q_out


def kv_quantize_int8(x, codes, scales, pos0=None, stream=None):
    """gemma_kv_quantize_int8: rows x [B,S,Hkv,D] bf16 into codes [B,Smax,Hkv,D] / scales [B,Hkv,Smax]
    at rows pos0[b] + s."""
    import torch

    B, S, Hkv, D = x.shape
    Smax = codes.shape[1]
    _expect(codes, (B, Smax, Hkv, D), "codes")
    _expect(scales, (B, Hkv, Smax), "scales")
    if pos0 is not None:
        _expect(pos0, (B,), "pos0")
    rc = load().gemma_kv_quantize_int8(B, S, Hkv, D, Smax, _ptr(x, torch.bfloat16, "x"),
                                       _ptr(pos0, torch.int32, "pos0"), _ptr(codes, torch.int8, "codes"),
                                       _ptr(scales, torch.float32, "scales"), _stream(stream))
    _check(rc, "gemma_kv_quantize_int8")
