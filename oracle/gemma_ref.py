"""Plain fp64 definition of one Gemma attention layer (TEST INFRASTRUCTURE ONLY).

What is computed, step by step, for one layer ``layer_idx`` of a model whose
attention knobs are a :class:`GemmaAttnConfig`:

0. resolve the layer: local (sliding window) or global, and with it the window,
   rotary base, KV-head count, head width and keys-as-values flag;
1. QK-norm: RMSNorm over each head vector of q and k (optional);
2. rotary position embedding on the first ``rotary_dim`` dims of each head of
   q and k, the rest passed through;
3. values: the processed keys when keys-as-values is on, else the given v;
4. scores ``q.k * query_pre_attn_scalar**-0.5`` per query head against its KV
   head (contiguous GQA groups);
5. tanh soft-cap ``cap * tanh(s / cap)`` when a cap is set;
6. causal mask, plus the sliding window on local layers;
7. softmax over the allowed keys (two-pass: max, then normalised exponentials);
8. output = probabilities times values; log-sum-exp per row on request.

Everything is numpy float64.  Inputs are the bf16 values the GPU receives,
widened exactly.  Rows are independent; :func:`prefill` batches rows of one
(batch, KV head) pair into blocks only to call the library matmul once per
block, which changes no sum's order within a row.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class GemmaAttnConfig:
    """The pages' attention knobs (argument tables of Gemma/Gemma2/Gemma3/Gemma4Model).

    ``num_global_kv_heads`` and ``global_head_dim`` are the Gemma 4 table's
    global-layer values; 0 means "same as the local value".
    ``sliding_window`` <= 0 means every layer is global.
    ``sliding_window_pattern`` N >= 1: one global layer every N layers.
    ``rope_local_theta`` <= 0 means the local layers use ``rope_theta``.
    ``attn_logit_softcapping`` <= 0 disables the cap.
    ``query_pre_attn_scalar`` <= 0 means the layer's head width.
    ``norm_weight_offset`` 1 multiplies by (1 + w) (Gemma 1-3), 0 by w (Gemma 4).
    ``rope_scaling_factor`` > 0: global layers divide positions by it; <= 0: off.
    """

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


def resolve_layer(cfg: GemmaAttnConfig, layer_idx: int) -> dict:
    """Per-layer values.

    Which layer is global: the Gemma 3 table describes ``sliding_window_pattern``
    as one global layer every N (five local to one global at N=6); the Gemma 2
    introduction says every other layer is local.  Reading: the local layers come
    first in each period, so layer ``l`` is global iff ``(l + 1) % N == 0``.
    A non-positive window means no local layers.  Local layers take
    ``rope_local_theta`` (Gemma 3 "Dual RoPE bases"); global layers take the
    global KV-head count, global head width and keys-as-values flag (Gemma 4
    table and "K=V global MQA").
    """
    if layer_idx < 0:
        raise ValueError("layer_idx must be >= 0")
    n = int(cfg.sliding_window_pattern)
    is_global = cfg.sliding_window <= 0 or (n >= 1 and (layer_idx + 1) % n == 0)
    if is_global:
        window = 0
        theta = float(cfg.rope_theta)
        hkv = cfg.num_global_kv_heads if cfg.num_global_kv_heads > 0 else cfg.num_kv_heads
        dim = cfg.global_head_dim if cfg.global_head_dim > 0 else cfg.head_dim
        kv_eq = bool(cfg.k_eq_v)
    else:
        window = int(cfg.sliding_window)
        theta = float(cfg.rope_local_theta) if cfg.rope_local_theta > 0 else float(cfg.rope_theta)
        hkv = cfg.num_kv_heads
        dim = cfg.head_dim
        kv_eq = False
    if hkv <= 0 or cfg.num_heads % hkv != 0:
        raise ValueError("num_heads must be a multiple of the KV-head count")
    rotary_dim = 2 * int(math.floor(float(cfg.partial_rotary_factor) * dim / 2.0))
    factor = float(getattr(cfg, "rope_scaling_factor", 0.0) or 0.0)
    pos_div = factor if (is_global and factor > 0) else 1.0
    qpas = float(cfg.query_pre_attn_scalar) if cfg.query_pre_attn_scalar > 0 else float(dim)
    return dict(
        is_global=bool(is_global),
        window=window,
        theta=theta,
        num_kv_heads=int(hkv),
        head_dim=int(dim),
        group=cfg.num_heads // hkv,
        rotary_dim=rotary_dim,
        k_eq_v=kv_eq,
        scale=qpas ** -0.5,
        softcap=float(cfg.attn_logit_softcapping) if cfg.attn_logit_softcapping > 0 else 0.0,
        pos_div=pos_div,
    )


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float, offset: int) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * (w + offset).

    The Gemma 4 page ("Plain-weight RMSNorm") uses w directly; Gemma 1-3 scale
    by 1 + w.  QK-norm applies it to each head vector of q and k (atlas summary:
    RMSNorm pre/post-norm with QK-norm).
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * (np.asarray(w, dtype=np.float64) + float(offset))


def rotary_inv_freq(theta: float, rotary_dim: int) -> np.ndarray:
    """Angular frequencies omega_i = theta^(-2i/r), i in [0, r/2)."""
    i = np.arange(rotary_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / float(rotary_dim))


def rotary(x: np.ndarray, positions: np.ndarray, theta: float, rotary_dim: int) -> np.ndarray:
    """Rotate the first ``rotary_dim`` dims of every head vector; pass the rest.

    ``x`` is [B, S, H, D]; ``positions`` is [B, S].  Pairs are (i, i + r/2)
    ("rotate half"), each turned by the angle p * omega_i.  The Gemma 4 page
    ("Zero-pad partial rope") rotates only ``partial_rotary_factor`` of each head
    and passes the remainder through; reading: the rotated part is the first r
    dims, contiguous.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    half = rotary_dim // 2
    if half == 0:
        return out
    omega = rotary_inv_freq(theta, rotary_dim)
    phi = np.asarray(positions, dtype=np.float64)[:, :, None, None] * omega  # [B,S,1,half]
    c, s = np.cos(phi), np.sin(phi)
    a = x[..., :half]
    b = x[..., half:rotary_dim]
    out[..., :half] = a * c - b * s
    out[..., half:rotary_dim] = b * c + a * s
    return out


def rotary_zero_pad(x: np.ndarray, positions: np.ndarray, theta: float, rotary_dim: int) -> np.ndarray:
    """The other reading of partial rotary: a zero-padded frequency vector.

    The Gemma 4 page ("Zero-pad partial rope") can also be read as rotating
    every head vector over its full width D in rotate-half pairs (j, j + D/2),
    with the frequencies of a full-width rotary, theta^(-2j/D), kept for the
    first r/2 pairs and set to zero (no rotation) for the rest; r is the same
    ``rotary_dim`` as in :func:`rotary`.  The rotated dims are then
    [0, r/2) and [D/2, D/2 + r/2) instead of [0, r).  At r = D the two readings
    are the same function.  ``x`` is [B, S, H, D], ``positions`` [B, S].
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    D = x.shape[-1]
    half = D // 2
    n_rot = rotary_dim // 2
    if n_rot == 0:
        return out
    j = np.arange(half, dtype=np.float64)
    omega = np.where(j < n_rot, np.power(float(theta), -2.0 * j / float(D)), 0.0)
    phi = np.asarray(positions, dtype=np.float64)[:, :, None, None] * omega  # [B,S,1,D/2]
    c, s = np.cos(phi), np.sin(phi)
    a = x[..., :half]
    b = x[..., half:2 * half]
    out[..., :half] = a * c - b * s
    out[..., half:2 * half] = b * c + a * s
    return out


ROTARY_LAYOUTS = ("first", "zero_pad")


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (8 significant bits, ties to even), returned as fp64.

    The library's activations are bf16, so the processed q and k cross the
    boundary between the prologue and the attention as bf16; an end-to-end
    comparison applies this rounding to the oracle's own prologue output.
    Written from the definition: x = m * 2^(e-7) with e = floor(log2|x|) and m
    rounded half-to-even.  Normal range only (bf16 shares fp32's exponents).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    ax = np.abs(x[nz])
    e = np.floor(np.log2(ax))
    # log2 can land one off for values a hair below a power of two
    e = np.where(2.0 ** e > ax, e - 1, e)
    e = np.where(2.0 ** (e + 1) <= ax, e + 1, e)
    ulp = 2.0 ** (e - 7)
    out[nz] = np.sign(x[nz]) * np.rint(ax / ulp) * ulp
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out


def softcap(s: np.ndarray, cap: float) -> np.ndarray:
    """Gemma 2 attention-logit soft cap: cap * tanh(s / cap); cap <= 0 is off."""
    if cap <= 0:
        return s
    return cap * np.tanh(s / cap)


def allowed(i: np.ndarray, j: np.ndarray, window: int) -> np.ndarray:
    """Causal mask with an optional sliding window.

    Reading of "local attention span" W: a query at position i sees keys j with
    j <= i and i - j < W, i.e. exactly W keys including itself.  W = 0: no window.
    """
    i = np.asarray(i)
    j = np.asarray(j)
    ok = j <= i
    if window > 0:
        ok &= (i - j) < window
    return ok


def prologue(cfg, layer_idx, q, k=None, q_norm_w=None, k_norm_w=None, pos0=None, rotary_layout="first"):
    """QK-norm then rotary on q [B,S,Hq,D] and k [B,S,Hkv,D]; returns fp64 arrays.

    Positions are ``pos0[b] + s`` (``pos0`` defaults to zeros), divided by the
    layer's ``pos_div`` (rope scaling).  The norm is applied only when its
    weight is given.  Values are never normed or rotated.  ``rotary_layout``
    picks the reading of partial rotary: "first" (the first r dims, the
    library's reading; :func:`rotary`) or "zero_pad" (:func:`rotary_zero_pad`).
    """
    if rotary_layout not in ROTARY_LAYOUTS:
        raise ValueError(f"rotary_layout must be one of {ROTARY_LAYOUTS}")
    rot = rotary if rotary_layout == "first" else rotary_zero_pad
    L = resolve_layer(cfg, layer_idx)
    q = np.asarray(q, dtype=np.float64)
    B, S = q.shape[0], q.shape[1]
    p0 = np.zeros(B, dtype=np.int64) if pos0 is None else np.asarray(pos0, dtype=np.int64)
    positions = p0[:, None] + np.arange(S, dtype=np.int64)[None, :]
    if L["pos_div"] != 1.0:
        positions = positions.astype(np.float64) / L["pos_div"]

    def one(x, w):
        if w is not None:
            x = rms_norm(x, w, cfg.norm_eps, cfg.norm_weight_offset)
        return rot(x, positions, L["theta"], L["rotary_dim"])

    qo = one(q, q_norm_w)
    ko = None if k is None else one(np.asarray(k, dtype=np.float64), k_norm_w)
    return qo, ko


def _workers() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _rows_block(qb, keys, vals, i_pos, j_pos, L):
    """Attention for a block of independent query rows against one KV head.

    qb [g, n, D]; keys/vals [m, D]; i_pos [n] query positions; j_pos [m] key
    positions.  Returns out [g, n, D] and lse [g, n] (natural log).
    """
    s = np.matmul(qb, keys.T) * L["scale"]                      # step 4
    s = softcap(s, L["softcap"])                                 # step 5
    ok = allowed(i_pos[:, None], j_pos[None, :], L["window"])    # step 6
    s = np.where(ok[None, :, :], s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)                        # step 7, pass 1
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe)                                       # step 7, pass 2
    tot = np.sum(e, axis=-1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(tot > 0, e / tot, 0.0)
        lse = np.where(tot[..., 0] > 0, m_safe[..., 0] + np.log(tot[..., 0]), -np.inf)
    return np.matmul(p, vals), lse                               # step 8


def prefill(cfg, layer_idx, q, k, v=None, block_rows: int = 256, threads: int | None = None):
    """Causal (optionally windowed) attention over prologue outputs.

    q [B,S,Hq,D], k [B,S,Hkv,D], v [B,S,Hkv,D] (ignored with keys-as-values,
    the k_eq_v flag of the Gemma 4 page's Gemma4Model table, under which one
    projection serves for keys and values on global layers; reading: the
    value tensor is the processed key tensor).  Query and key
    positions are 0..S-1.  Returns out [B,S,Hq,D] and lse [B,Hq,S], fp64.
    """
    L = resolve_layer(cfg, layer_idx)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    vv = k if L["k_eq_v"] else np.asarray(v, dtype=np.float64)
    B, S, Hq, D = q.shape
    Hkv, g, W = L["num_kv_heads"], L["group"], L["window"]
    out = np.zeros((B, S, Hq, vv.shape[-1]))
    lse = np.full((B, Hq, S), -np.inf)
    units = [(b, h, i0) for b in range(B) for h in range(Hkv) for i0 in range(0, S, block_rows)]

    def run(u):
        b, h, i0 = u
        i1 = min(S, i0 + block_rows)
        lo = max(0, i0 - W + 1) if W > 0 else 0
        heads = slice(h * g, (h + 1) * g)                         # contiguous GQA group
        qb = np.transpose(q[b, i0:i1, heads, :], (1, 0, 2))       # [g, n, D]
        o, l = _rows_block(qb, k[b, lo:i1, h, :], vv[b, lo:i1, h, :],
                           np.arange(i0, i1), np.arange(lo, i1), L)
        out[b, i0:i1, heads, :] = np.transpose(o, (1, 0, 2))
        lse[b, heads, i0:i1] = l

    n = threads or _workers()
    if n > 1 and len(units) > 1:
        with ThreadPoolExecutor(n) as ex:
            list(ex.map(run, units))
    else:
        for u in units:
            run(u)
    return out, lse


def prefill_ragged(cfg, layer_idx, q, k, v, seq_start, seq_end):
    """Prefill of a padded batch: sequence b keeps rows [start_b, end_b).

    The Gemma pages' generate() takes an attention_mask (batch, seq) with 1 =
    keep and 0 = padding.  Reading: padding is contiguous at the ends (left
    padding for batched generation, right padding for ragged lengths), so the
    mask is the range [start_b, end_b); padded tokens are neither queries nor
    keys.  The mask is positional (i - j), so attention over the kept rows is
    the plain prefill of the slice; padded rows give out = 0, lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    B, S, Hq, D = q.shape
    k = np.asarray(k, dtype=np.float64)
    L = resolve_layer(cfg, layer_idx)
    vv = k if L["k_eq_v"] else np.asarray(v, dtype=np.float64)
    out = np.zeros((B, S, Hq, vv.shape[-1]))
    lse = np.full((B, Hq, S), -np.inf)
    for b in range(B):
        lo = min(max(int(seq_start[b]), 0), S)
        hi = min(max(int(seq_end[b]), lo), S)
        if hi == lo:
            continue
        o, l = prefill(cfg, layer_idx, q[b:b + 1, lo:hi], k[b:b + 1, lo:hi], None if L["k_eq_v"] else vv[b:b + 1, lo:hi])
        out[b, lo:hi] = o[0]
        lse[b, :, lo:hi] = l[0]
    return out, lse


def prefill_rows(cfg, layer_idx, q_rows, k, v, rows):
    """Attention for a sample of query rows only.

    ``rows`` is a list of (b, head, i); ``q_rows`` [len(rows), D] holds the
    processed query vectors of those rows; k, v are full [B,S,Hkv,D] tensors
    (v ignored with keys-as-values).  Returns out [n, D] and lse [n].
    """
    L = resolve_layer(cfg, layer_idx)
    k = np.asarray(k, dtype=np.float64)
    vv = k if L["k_eq_v"] else np.asarray(v, dtype=np.float64)
    W, g = L["window"], L["group"]
    outs, lses = [], []
    for r, (b, hq, i) in enumerate(rows):
        h = hq // g
        lo = max(0, i - W + 1) if W > 0 else 0
        o, l = _rows_block(np.asarray(q_rows[r], dtype=np.float64)[None, None, :],
                           k[b, lo:i + 1, h, :], vv[b, lo:i + 1, h, :],
                           np.array([i]), np.arange(lo, i + 1), L)
        outs.append(o[0, 0])
        lses.append(l[0, 0])
    return np.array(outs), np.array(lses)


def decode(cfg, layer_idx, q, k_cache, v_cache, ctx_len, batches=None):
    """One query token per sequence against a contiguous KV cache.

    q [B,Hq,D] is the processed query at position ctx_b - 1; the cache
    [B,Smax,Hkv,D] holds processed keys (and values) for positions
    0..Smax-1, including the current token (reading).  Allowed keys are
    j in [0, ctx_b) with ctx_b - 1 - j < W on local layers.  ctx_b = 0 gives
    out = 0 and lse = -inf.  ``batches`` restricts the work to some sequences
    (others are left zero / -inf).  Returns out [B,Hq,D], lse [B,Hq].
    """
    L = resolve_layer(cfg, layer_idx)
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    g, W = L["group"], L["window"]
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in (range(B) if batches is None else batches):
        c = int(ctx_len[b])
        if c <= 0:
            continue
        t = c - 1
        lo = max(0, c - W) if W > 0 else 0
        for h in range(L["num_kv_heads"]):
            keys = np.asarray(k_cache[b, lo:c, h, :], dtype=np.float64)
            vals = keys if L["k_eq_v"] else np.asarray(v_cache[b, lo:c, h, :], dtype=np.float64)
            qb = q[b, h * g:(h + 1) * g, :][:, None, :]            # [g, 1, D]
            o, l = _rows_block(qb, keys, vals, np.array([t]), np.arange(lo, c), L)
            out[b, h * g:(h + 1) * g, :] = o[:, 0, :]
            lse[b, h * g:(h + 1) * g] = l[:, 0]
    return out, lse


def decode_multi(cfg, layer_idx, q, k_cache, v_cache, ctx_len, kv_start=None):
    """Several new tokens per sequence against a contiguous cache.

    q [B,L,Hq,D] holds the processed queries of the tokens at positions
    ctx_b - L + t (reading: the cache already holds the new tokens, as in
    single-token decode).  Token t at position i sees cache rows j with
    0 <= j <= i and, on local layers, i - j < W -- the prefill mask.  A token
    with i < 0 sees nothing (out 0, lse -inf).  ``kv_start`` [B] (optional)
    drops the cache rows before it: the left padding of a padded prefill.
    Returns out [B,L,Hq,D] and lse [B,Hq,L].
    """
    Lr = resolve_layer(cfg, layer_idx)
    q = np.asarray(q, dtype=np.float64)
    B, Lq, Hq, D = q.shape
    g, W = Lr["group"], Lr["window"]
    out = np.zeros((B, Lq, Hq, D))
    lse = np.full((B, Hq, Lq), -np.inf)
    for b in range(B):
        c = int(ctx_len[b])
        first = 0 if kv_start is None else max(0, int(kv_start[b]))
        for t in range(Lq):
            i = c - Lq + t
            if i < 0:
                continue
            lo = max(0, i - W + 1) if W > 0 else 0
            lo = max(lo, first)
            if lo > i:
                continue
            for h in range(Lr["num_kv_heads"]):
                keys = np.asarray(k_cache[b, lo:i + 1, h, :], dtype=np.float64)
                vals = keys if Lr["k_eq_v"] else np.asarray(v_cache[b, lo:i + 1, h, :], dtype=np.float64)
                qb = q[b, t, h * g:(h + 1) * g, :][:, None, :]
                o, l = _rows_block(qb, keys, vals, np.array([i]), np.arange(lo, i + 1), Lr)
                out[b, t, h * g:(h + 1) * g, :] = o[:, 0, :]
                lse[b, h * g:(h + 1) * g, t] = l[:, 0]
    return out, lse


def quantize_int8(x):
    """Symmetric int8 quantization of each vector along the last axis.

    The "google-gemma-4" atlas summary ("Training" section, efficiency entry)
    says int8 KV caching is offered and gives no format.  Reading: one fp32
    scale per (token, KV head) vector, s = max|x| / 127, codes
    c = round-half-even(x / s) in [-127, 127]; an all-zero vector has s = 0 and
    codes 0.  The decision is taken in fp32 (IEEE division), the precision of
    the bf16 activations' arithmetic, so both sides reach the same integers.
    Returns (codes int8 [..., D], scales fp32 [...]).
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        c = np.rint(np.divide(x, safe[..., None], dtype=np.float32))
    c = np.where(s[..., None] > 0, c, 0.0)
    return np.clip(c, -127, 127).astype(np.int8), s


def dequantize_int8(codes, scales):
    """codes * scale per vector, exact in fp64 (a 7-bit integer times an fp32)."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[..., None]


def decode_int8(cfg, layer_idx, q, k_codes, k_scales, v_codes, v_scales, ctx_len, kv_start=None):
    """Decode (any number of new tokens) against an int8 cache.

    Cache codes [B,Smax,Hkv,D] int8 with scales [B,Hkv,Smax] fp32 (one per
    token and head).  The attention is the one of ``decode_multi`` on the
    dequantized cache; values are ignored on keys-as-values layers.  q
    [B,L,Hq,D].  Returns out [B,L,Hq,D] and lse [B,Hq,L].
    """
    L = resolve_layer(cfg, layer_idx)
    kd = dequantize_int8(k_codes, np.swapaxes(np.asarray(k_scales), 1, 2))
    vd = kd if L["k_eq_v"] else dequantize_int8(v_codes, np.swapaxes(np.asarray(v_scales), 1, 2))
    return decode_multi(cfg, layer_idx, q, kd, vd, ctx_len, kv_start)


def prefill_flops(cfg, layer_idx, batch: int, seq: int) -> int:
    """Algorithmic prefill work: 4*D FLOPs per allowed (query head, key) pair."""
    L = resolve_layer(cfg, layer_idx)
    W, S = L["window"], int(seq)
    if W <= 0 or W >= S:
        n = S * (S + 1) // 2
    else:
        n = W * (W + 1) // 2 + (S - W) * W
    return 4 * L["head_dim"] * int(batch) * cfg.num_heads * n


def decode_kv_bytes(cfg, layer_idx, ctx_len, int8: bool = False) -> int:
    """Algorithmic decode bytes: every allowed cache element read once (bf16,
    or int8 codes plus one fp32 scale per token and head)."""
    L = resolve_layer(cfg, layer_idx)
    W = L["window"]
    c = np.asarray(ctx_len, dtype=np.int64)
    span = np.minimum(c, W) if W > 0 else c
    row = L["head_dim"] + 4 if int8 else L["head_dim"] * 2
    per_tok = L["num_kv_heads"] * row * (1 if L["k_eq_v"] else 2)
    return int(np.sum(np.maximum(span, 0)) * per_tok)
