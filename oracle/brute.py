"""Scalar pure-Python twin of the oracle, for tiny inputs (TEST INFRASTRUCTURE ONLY).

Written independently of ``gemma_ref`` (no shared helper): the layer kind is
found by walking the layer stack, rotary uses complex multiplication, sums use
``math.fsum`` and every query row builds its own list of visible keys.  It is
slow on purpose and only meant for shapes of a few dozen positions.

Inputs are nested Python lists (or anything indexable) of floats:
q[b][s][h][d], k[b][s][hk][d], v likewise; returns (out[b][s][h][d], lse[b][h][s]).
"""
from __future__ import annotations

import cmath
import math


def layer_kind(pattern: int, window: int, layer_idx: int) -> str:
    """Walk the stack: every ``pattern``-th layer (counting from 1) is global."""
    if window <= 0:
        return "global"
    kind = "local"
    since_global = 0
    for _ in range(layer_idx + 1):
        since_global += 1
        if pattern >= 1 and since_global == pattern:
            kind = "global"
            since_global = 0
        else:
            kind = "local"
    return kind


def _norm(vec, w, eps, offset):
    n = len(vec)
    mean_sq = math.fsum(x * x for x in vec) / n
    inv = 1.0 / math.sqrt(mean_sq + eps)
    return [vec[d] * inv * (w[d] + offset) for d in range(n)]


def _rope(vec, pos, theta, r):
    out = list(vec)
    half = r // 2
    for i in range(half):
        freq = theta ** (-(2.0 * i) / r)
        z = complex(vec[i], vec[i + half]) * cmath.exp(1j * pos * freq)
        out[i], out[i + half] = z.real, z.imag
    return out


def _rope_zero_pad(vec, pos, theta, r):
    """Zero-padded frequencies over the whole width: pair (j, j + D/2) turns
    by pos * theta^(-2j/D) for j < r/2 and stays put for larger j."""
    out = list(vec)
    n = len(vec)
    for j in range(n // 2):
        if j >= r // 2:
            continue
        z = complex(vec[j], vec[j + n // 2]) * cmath.exp(1j * pos * theta ** (-(2.0 * j) / n))
        out[j], out[j + n // 2] = z.real, z.imag
    return out


def brute_layer(p: dict, layer_idx, q, k, v=None, q_norm_w=None, k_norm_w=None, pos0=None, keep=None):
    """Whole layer (QK-norm, rotary, attention) for tiny shapes.

    ``p`` uses the pages' knob names (same meaning as the oracle's config).
    ``keep`` (optional, [B][S] of 0/1) is an attention mask: a position with 0
    is neither a query (its output row is 0, lse -inf) nor a key.
    ``p["rotary_layout"]`` "zero_pad" takes the zero-padded reading of partial
    rotary (default "first": the first r dims).
    """
    rope = _rope_zero_pad if p.get("rotary_layout", "first") == "zero_pad" else _rope
    kind = layer_kind(p.get("sliding_window_pattern", 1), p.get("sliding_window", 0), layer_idx)
    pos_div = 1.0
    if kind == "global":
        W = 0
        theta = p["rope_theta"]
        if (p.get("rope_scaling_factor") or 0) > 0:
            pos_div = float(p["rope_scaling_factor"])
        hkv = p.get("num_global_kv_heads") or p["num_kv_heads"]
        D = p.get("global_head_dim") or p["head_dim"]
        tied = bool(p.get("k_eq_v", False))
    else:
        W = p["sliding_window"]
        theta = p.get("rope_local_theta") or p["rope_theta"]
        hkv = p["num_kv_heads"]
        D = p["head_dim"]
        tied = False
    Hq = p["num_heads"]
    r = 2 * int(p.get("partial_rotary_factor", 1.0) * D / 2.0)
    qpas = p.get("query_pre_attn_scalar") or D
    cap = p.get("attn_logit_softcapping") or 0.0
    eps = p.get("norm_eps", 1e-6)
    off = p.get("norm_weight_offset", 0)
    kv_of = []
    for kvh in range(hkv):
        kv_of += [kvh] * (Hq // hkv)

    B, S = len(q), len(q[0])
    out = [[[[0.0] * D for _ in range(Hq)] for _ in range(S)] for _ in range(B)]
    lse = [[[float("-inf")] * S for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        base = 0 if pos0 is None else int(pos0[b])

        def prep(vec, w, s):
            vec = [float(x) for x in vec]
            if w is not None:
                vec = _norm(vec, w, eps, off)
            return rope(vec, (base + s) / pos_div, theta, r)

        kk = [[prep(k[b][s][h], k_norm_w, s) for h in range(hkv)] for s in range(S)]
        vv = kk if tied else [[[float(x) for x in v[b][s][h]] for h in range(hkv)] for s in range(S)]
        for s in range(S):
            if keep is not None and not keep[b][s]:
                continue
            lo = 0 if W == 0 else max(0, s - W + 1)
            visible = [j for j in range(lo, s + 1) if keep is None or keep[b][j]]
            for h in range(Hq):
                qq = prep(q[b][s][h], q_norm_w, s)
                kh = kv_of[h]
                logits = []
                for j in visible:
                    x = math.fsum(qq[d] * kk[j][kh][d] for d in range(D)) / math.sqrt(qpas)
                    if cap > 0:
                        x = cap * math.tanh(x / cap)
                    logits.append(x)
                top = max(logits)
                w = [math.exp(x - top) for x in logits]
                tot = math.fsum(w)
                for d in range(D):
                    out[b][s][h][d] = math.fsum(w[n] * vv[j][kh][d] for n, j in enumerate(visible)) / tot
                lse[b][h][s] = top + math.log(tot)
    return out, lse
