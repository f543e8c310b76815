"""Pins for the fp64 oracle (CPU only).

The oracle is checked against things other than itself: an independent scalar
brute force on tiny inputs, closed forms, invariants the mathematics fixes, and
torch's own scaled_dot_product_attention (fp64, CPU) where the method reduces
to plain causal or windowed softmax attention.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import gemma_ref as R
from oracle.brute import brute_layer, layer_kind
from synth import bf16_bits_to_f64, normal_bf16, norm_weight

TOL = 1e-12


def _cfg_dict(cfg):
    return {f: getattr(cfg, f) for f in cfg.__dataclass_fields__}


def _inputs(seed, B, S, Hq, Hkv, D, qscale=1.0):
    q = bf16_bits_to_f64(normal_bf16(seed, (B, S, Hq, D), scale=qscale))
    k = bf16_bits_to_f64(normal_bf16(seed + 1, (B, S, Hkv, D)))
    v = bf16_bits_to_f64(normal_bf16(seed + 2, (B, S, Hkv, D)))
    return q, k, v


# --------------------------------------------------------------------------- brute force
_COMBOS = list(itertools.product(
    [(4, 4, 8), (4, 2, 8), (4, 1, 16)],        # (Hq, Hkv, D)
    [0, 1, 3, 40],                              # window (0 => global)
    [0.0, 2.5],                                 # softcap
    [1.0, 0.5, 0.0],                            # partial rotary factor
    [None, 0, 1],                               # QK-norm: off / offset 0 / offset 1
))


@pytest.mark.parametrize("combo", _COMBOS[::3] + [_COMBOS[-1]])
def test_oracle_matches_brute_force(combo):
    (Hq, Hkv, D), W, cap, f, norm = combo
    cfg = R.GemmaAttnConfig(num_heads=Hq, num_kv_heads=Hkv, head_dim=D, sliding_window=W,
                            sliding_window_pattern=0, rope_theta=1e4, partial_rotary_factor=f,
                            attn_logit_softcapping=cap, query_pre_attn_scalar=6.0 if cap else 0.0,
                            norm_weight_offset=norm or 0)
    B, S = 2, 11
    q, k, v = _inputs(7, B, S, Hq, Hkv, D, qscale=3.0)
    qw = norm_weight(3, D) if norm is not None else None
    kw = norm_weight(4, D) if norm is not None else None
    pos0 = np.array([0, 5])
    qt, kt = R.prologue(cfg, 0, q, k, qw, kw, pos0)
    o, l = R.prefill(cfg, 0, qt, kt, v, block_rows=4)
    ob, lb = brute_layer(_cfg_dict(cfg), 0, q.tolist(), k.tolist(), v.tolist(),
                         None if qw is None else qw.tolist(), None if kw is None else kw.tolist(), pos0.tolist())
    assert np.abs(o - np.array(ob)).max() < TOL
    assert np.abs(l - np.array(lb)).max() < TOL


@pytest.mark.parametrize("layer", [0, 1, 2, 5])
def test_oracle_matches_brute_force_layer_stack(layer):
    """Dual bases, wider global heads, global KV heads and keys-as-values."""
    cfg = R.GemmaAttnConfig(num_heads=4, num_kv_heads=2, head_dim=8, num_global_kv_heads=1,
                            global_head_dim=16, sliding_window=4, sliding_window_pattern=3,
                            rope_theta=1e6, rope_local_theta=1e4, partial_rotary_factor=0.25,
                            k_eq_v=True, norm_weight_offset=0)
    Lr = R.resolve_layer(cfg, layer)
    assert Lr["is_global"] == (layer_kind(3, 4, layer) == "global")
    D, Hkv = Lr["head_dim"], Lr["num_kv_heads"]
    B, S = 1, 13
    q, k, v = _inputs(11, B, S, 4, Hkv, D, qscale=2.0)
    qw, kw = norm_weight(5, D), norm_weight(6, D)
    qt, kt = R.prologue(cfg, layer, q, k, qw, kw)
    o, l = R.prefill(cfg, layer, qt, kt, v, block_rows=5)
    ob, lb = brute_layer(_cfg_dict(cfg), layer, q.tolist(), k.tolist(), v.tolist(), qw.tolist(), kw.tolist())
    assert np.abs(o - np.array(ob)).max() < TOL
    assert np.abs(l - np.array(lb)).max() < TOL


# --------------------------------------------------------------------------- closed forms
def test_rotary_closed_form():
    # one pair, frequency theta^0 = 1: (1, 0) at position p turns to (cos p, sin p)
    x = np.zeros((1, 3, 1, 2))
    x[..., 0] = 1.0
    y = R.rotary(x, np.array([[0, 1, 7]]), 1e4, 2)
    for s, p in enumerate([0, 1, 7]):
        assert abs(y[0, s, 0, 0] - math.cos(p)) < 1e-15
        assert abs(y[0, s, 0, 1] - math.sin(p)) < 1e-15
    # second pair of r=4 turns at theta^(-1/2): 1e4 -> 0.01 rad per position
    assert abs(R.rotary_inv_freq(1e4, 4)[1] - 0.01) < 1e-18
    x = np.zeros((1, 1, 1, 6))
    x[0, 0, 0, 1] = 2.0
    x[0, 0, 0, 4:] = [5.0, -6.0]  # pass-through dims
    y = R.rotary(x, np.array([[100]]), 1e4, 4)
    assert abs(y[0, 0, 0, 1] - 2 * math.cos(1.0)) < 1e-14
    assert abs(y[0, 0, 0, 3] - 2 * math.sin(1.0)) < 1e-14
    assert y[0, 0, 0, 4] == 5.0 and y[0, 0, 0, 5] == -6.0


def test_rotary_invariants():
    rng = np.random.default_rng(0)
    D, r = 16, 8
    q = rng.standard_normal((1, 1, 1, D))
    k = rng.standard_normal((1, 1, 1, D))
    # position 0 is the identity
    assert np.array_equal(R.rotary(q, np.array([[0]]), 1e4, r), q)
    # each rotated pair keeps its norm
    y = R.rotary(q, np.array([[12345]]), 1e4, r)
    for i in range(r // 2):
        assert abs(math.hypot(y[..., i].item(), y[..., i + r // 2].item())
                   - math.hypot(q[..., i].item(), q[..., i + r // 2].item())) < 1e-12
    # the score depends only on the offset m - n
    def dot(m, n):
        return float(np.sum(R.rotary(q, np.array([[m]]), 1e4, r) * R.rotary(k, np.array([[n]]), 1e4, r)))
    assert abs(dot(10, 3) - dot(1007, 1000)) < 1e-11
    assert abs(dot(3, 10) - dot(50, 57)) < 1e-11


def test_rms_norm_closed_form():
    x = np.full((1, 8), 3.0)
    eps = 1e-6
    y = R.rms_norm(x, np.ones(8), eps, 0)
    assert np.allclose(y, 3.0 / math.sqrt(9.0 + eps), rtol=0, atol=1e-15)
    y1 = R.rms_norm(x, np.zeros(8), eps, 1)          # (1 + w) with w = 0 is the same
    assert np.array_equal(y, y1)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 32))
    y = R.rms_norm(x, np.ones(32), eps, 0)
    ms = np.mean(x * x, axis=-1)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), np.sqrt(ms / (ms + eps)), rtol=1e-14)
    w = rng.standard_normal(32)
    assert np.allclose(R.rms_norm(x, w, eps, 0) * (w + 1), R.rms_norm(x, w, eps, 1) * w, rtol=1e-12, atol=1e-13)


def test_softcap_properties():
    s = np.linspace(-400, 400, 4001)
    c = R.softcap(s, 50.0)
    assert np.all(np.diff(c) > 0)                     # monotone
    assert np.all(np.abs(c) < 50.0)                   # bounded by the cap
    assert np.array_equal(R.softcap(-s, 50.0), -c)    # odd
    assert np.allclose(R.softcap(s[1900:2100], 1e9), s[1900:2100], rtol=1e-12)  # identity as cap -> inf
    assert np.array_equal(R.softcap(s, 0.0), s)       # off
    assert abs(R.softcap(np.array([50.0]), 50.0)[0] - 50.0 * math.tanh(1.0)) < 1e-13


# --------------------------------------------------------------------------- invariants
def _small_cfg(**kw):
    base = dict(num_heads=4, num_kv_heads=2, head_dim=16, sliding_window=0, sliding_window_pattern=0,
                rope_theta=1e4, attn_logit_softcapping=0.0)
    base.update(kw)
    return R.GemmaAttnConfig(**base)


@pytest.mark.parametrize("W,cap", [(0, 0.0), (5, 0.0), (5, 20.0), (1, 0.0)])
def test_rows_sum_to_one_and_mask(W, cap):
    cfg = _small_cfg(sliding_window=W, attn_logit_softcapping=cap)
    B, S, D = 1, 16, 16
    q, k, _ = _inputs(21, B, S, 4, 2, D, qscale=4.0)
    # V = identity over positions (D = S) turns the output into the probability matrix
    v = np.zeros((B, S, 2, S))
    for j in range(S):
        v[0, j, :, j] = 1.0
    o, _ = R.prefill(cfg, 0, q, k, v)
    P = o[0, :, 0, :]
    assert np.allclose(P.sum(axis=-1), 1.0, atol=1e-14)
    ii, jj = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
    forbidden = (jj > ii) | ((ii - jj) >= W if W > 0 else False)
    assert np.all(P[forbidden] == 0.0)
    assert np.all(P[~forbidden] > 0.0)
    ones, _ = R.prefill(cfg, 0, q, k, np.ones((B, S, 2, 3)))
    assert np.allclose(ones, 1.0, atol=1e-14)


def test_window_at_least_seq_is_global():
    B, S = 2, 20
    q, k, v = _inputs(31, B, S, 4, 2, 16)
    og, lg = R.prefill(_small_cfg(), 0, q, k, v, block_rows=7)
    for W in (S, S + 9):
        ow, lw = R.prefill(_small_cfg(sliding_window=W), 0, q, k, v, block_rows=7)
        assert np.array_equal(og, ow) and np.array_equal(lg, lw)


def test_partial_factor_zero_is_position_free():
    cfg = _small_cfg(partial_rotary_factor=0.0, sliding_window=6)
    q, k, v = _inputs(41, 2, 12, 4, 2, 16)
    a = R.prologue(cfg, 0, q, k, pos0=np.array([0, 0]))
    b = R.prologue(cfg, 0, q, k, pos0=np.array([977, 31]))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(a[0], q)


def test_keys_as_values_equals_explicit_copy():
    cfg_t = R.GemmaAttnConfig(num_heads=4, num_kv_heads=1, head_dim=16, k_eq_v=True, sliding_window=0)
    cfg_f = R.GemmaAttnConfig(num_heads=4, num_kv_heads=1, head_dim=16, k_eq_v=False, sliding_window=0)
    q, k, v = _inputs(51, 1, 14, 4, 1, 16)
    qt, kt = R.prologue(cfg_t, 0, q, k, norm_weight(1, 16), norm_weight(2, 16))
    a = R.prefill(cfg_t, 0, qt, kt, v)            # v ignored
    b = R.prefill(cfg_f, 0, qt, kt, kt.copy())    # explicit copy of the processed keys
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_integer_facts():
    """Row 0 sees only key 0; W=1 sees only itself; q=0 gives uniform weights."""
    B, S, D = 1, 10, 16
    q, k, v = _inputs(61, B, S, 4, 2, D)
    o, _ = R.prefill(_small_cfg(sliding_window=3), 0, q, k, v)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0]) and np.array_equal(o[0, 0, 3], v[0, 0, 1])
    o1, l1 = R.prefill(_small_cfg(sliding_window=1), 0, q, k, v)
    assert np.array_equal(o1[0, :, 0], v[0, :, 0]) and np.array_equal(o1[0, :, 2], v[0, :, 1])
    for W in (0, 4):
        oz, lz = R.prefill(_small_cfg(sliding_window=W, attn_logit_softcapping=30.0), 0, np.zeros_like(q), k, v)
        for i in range(S):
            lo = max(0, i - W + 1) if W else 0
            cnt = i - lo + 1
            assert abs(lz[0, 0, i] - math.log(cnt)) < 1e-14
            assert np.allclose(oz[0, i, 1], v[0, lo:i + 1, 0].mean(axis=0), atol=1e-15)


def test_prefill_rows_and_decode_agree_with_prefill():
    for W, tied in [(0, False), (4, False), (0, True)]:
        cfg = _small_cfg(sliding_window=W, k_eq_v=tied, attn_logit_softcapping=10.0)
        B, S = 2, 15
        q, k, v = _inputs(71, B, S, 4, 2, 16, qscale=2.0)
        o, l = R.prefill(cfg, 0, q, k, v)
        rows = [(0, 3, 14), (1, 0, 0), (1, 2, 9)]
        orr, lrr = R.prefill_rows(cfg, 0, np.array([q[b, i, h] for b, h, i in rows]), k, v, rows)
        for n, (b, h, i) in enumerate(rows):
            assert np.abs(orr[n] - o[b, i, h]).max() < 1e-14 and abs(lrr[n] - l[b, h, i]) < 1e-14
        # decode of the last row: cache = the keys/values, ctx = S, NaN beyond ctx never read
        ctx = np.array([S, 9])
        kc = np.concatenate([k, np.full((B, 5, 2, 16), np.nan)], axis=1)
        vc = np.concatenate([v, np.full((B, 5, 2, 16), np.nan)], axis=1)
        kc[1, 9:] = np.nan
        vc[1, 9:] = np.nan
        qd = np.stack([q[0, S - 1], q[1, 8]])
        od, ld = R.decode(cfg, 0, qd, kc, vc, ctx)
        assert np.abs(od[0] - o[0, S - 1]).max() < 1e-14 and np.abs(ld[0] - l[0, :, S - 1]).max() < 1e-14
        assert np.abs(od[1] - o[1, 8]).max() < 1e-14 and np.abs(ld[1] - l[1, :, 8]).max() < 1e-14
    od, ld = R.decode(_small_cfg(), 0, np.ones((1, 4, 16)), np.ones((1, 4, 2, 16)), np.ones((1, 4, 2, 16)), [0])
    assert np.all(od == 0) and np.all(np.isneginf(ld))


# --------------------------------------------------------------------------- library routine
@pytest.mark.parametrize("W,g", [(0, 1), (0, 4), (6, 2), (1, 1)])
def test_attention_matches_torch_sdpa(W, g):
    """No cap: the attention part is plain masked softmax attention."""
    import torch
    import torch.nn.functional as F

    Hkv, D, B, S = 2, 16, 2, 23
    Hq = g * Hkv
    cfg = R.GemmaAttnConfig(num_heads=Hq, num_kv_heads=Hkv, head_dim=D, sliding_window=W,
                            sliding_window_pattern=0, query_pre_attn_scalar=7.0)
    q, k, v = _inputs(81, B, S, Hq, Hkv, D, qscale=3.0)
    o, _ = R.prefill(cfg, 0, q, k, v, block_rows=8)
    tq = torch.tensor(q).permute(0, 2, 1, 3)
    tk = torch.tensor(k).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    tv = torch.tensor(v).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    if W == 0:
        ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=7.0 ** -0.5)
    else:
        i = torch.arange(S)[:, None]
        j = torch.arange(S)[None, :]
        mask = (j <= i) & (i - j < W)
        ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=7.0 ** -0.5)
    assert np.abs(ref.permute(0, 2, 1, 3).numpy() - o).max() < 1e-12


# --------------------------------------------------------------------------- work counts
@pytest.mark.parametrize("S,W", [(9, 0), (9, 3), (9, 9), (9, 20), (1, 1)])
def test_work_counts_by_enumeration(S, W):
    cfg = _small_cfg(sliding_window=W)
    pairs = sum(1 for i in range(S) for j in range(S) if j <= i and (W == 0 or i - j < W))
    assert R.prefill_flops(cfg, 0, 3, S) == 4 * 16 * 3 * 4 * pairs
    ctx = [0, 1, 5, 9]
    span = sum(min(c, W) if W else c for c in ctx)
    assert R.decode_kv_bytes(cfg, 0, ctx) == span * 2 * 16 * 2 * 2


def test_round_bf16_closed_forms_and_bits():
    from synth import bf16_bits_to_f64, f32_to_bf16_bits

    # ties go to the even neighbour; 8 significant bits
    assert R.round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert R.round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    assert R.round_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1 + 2.0 ** -7
    assert R.round_bf16(np.array([-3.0, 0.0, 2.0 ** -100]))[1] == 0.0
    assert R.round_bf16(np.array([255.5]))[0] == 256.0 and R.round_bf16(np.array([254.5]))[0] == 254.0
    # agrees with bit-level round-to-nearest-even of fp32 values (fp32 -> bf16 is a single rounding)
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    assert np.array_equal(R.round_bf16(x.astype(np.float64)), bf16_bits_to_f64(f32_to_bf16_bits(x)))


@pytest.mark.parametrize("W,tied", [(0, False), (5, False), (0, True)])
def test_decode_multi_equals_prefill_tail_and_decode(W, tied):
    cfg = _small_cfg(sliding_window=W, k_eq_v=tied, attn_logit_softcapping=7.0)
    B, S, Lq = 2, 17, 6
    q, k, v = _inputs(91, B, S, 4, 2, 16, qscale=2.0)
    o, l = R.prefill(cfg, 0, q, k, v)
    # caches longer than the context, poisoned past it
    kc = np.concatenate([k, np.full((B, 4, 2, 16), np.nan)], axis=1)
    vc = np.concatenate([v, np.full((B, 4, 2, 16), np.nan)], axis=1)
    om, lm = R.decode_multi(cfg, 0, q[:, S - Lq:], kc, vc, [S, S])
    assert np.abs(om - o[:, S - Lq:]).max() < 1e-13
    assert np.abs(lm - l[:, :, S - Lq:]).max() < 1e-13
    o1, l1 = R.decode_multi(cfg, 0, q[:, S - 1:], kc, vc, [S, 9])
    od, ld = R.decode(cfg, 0, np.stack([q[0, S - 1], q[1, S - 1]]), kc, vc, [S, 9])
    assert np.array_equal(o1[:, 0], od) and np.array_equal(l1[:, :, 0], ld)
    # more new tokens than context: early tokens see nothing
    oz, lz = R.decode_multi(cfg, 0, q[:, :3], kc, vc, [2, 2])
    assert np.all(oz[:, 0] == 0) and np.all(np.isneginf(lz[:, :, 0]))


# --------------------------------------------------------------------------- rope scaling
def _scaled_cfg(factor, **kw):
    base = dict(num_heads=4, num_kv_heads=2, head_dim=8, num_global_kv_heads=1, global_head_dim=16,
                sliding_window=4, sliding_window_pattern=3, rope_theta=1e4, rope_local_theta=1e3,
                partial_rotary_factor=0.5, norm_weight_offset=0, rope_scaling_factor=factor)
    base.update(kw)
    return R.GemmaAttnConfig(**base)


@pytest.mark.parametrize("layer", [0, 2])
def test_rope_scaling_matches_brute_force(layer):
    cfg = _scaled_cfg(4.0)
    Lr = R.resolve_layer(cfg, layer)
    assert Lr["pos_div"] == (4.0 if Lr["is_global"] else 1.0)
    D, Hkv = Lr["head_dim"], Lr["num_kv_heads"]
    q, k, v = _inputs(13, 2, 9, 4, Hkv, D, qscale=2.0)
    pos0 = np.array([3, 1001])
    qt, kt = R.prologue(cfg, layer, q, k, pos0=pos0)
    o, l = R.prefill(cfg, layer, qt, kt, v)
    ob, lb = brute_layer(_cfg_dict(cfg), layer, q.tolist(), k.tolist(), v.tolist(), pos0=pos0.tolist())
    assert np.abs(o - np.array(ob)).max() < TOL
    assert np.abs(l - np.array(lb)).max() < TOL


def test_rope_scaling_divides_global_positions_only():
    """Closed form: with factor f, global position f*m rotates like position m
    without scaling (exactly, f a power of two); local layers ignore f."""
    q, k, _ = _inputs(17, 2, 6, 4, 1, 16)
    f = 8.0
    m = np.array([5, 123])
    qs, ks = R.prologue(_scaled_cfg(f), 2, q, k, pos0=(m * 8))
    q0, k0 = R.prologue(_scaled_cfg(0.0), 2, q, k, pos0=m)
    # positions (8m + s) / 8 = m + s/8: compare at s = 0 only, where they coincide
    assert np.array_equal(qs[:, 0], q0[:, 0]) and np.array_equal(ks[:, 0], k0[:, 0])
    ql, kl = _inputs(19, 2, 6, 4, 2, 8)[:2]
    a = R.prologue(_scaled_cfg(f), 0, ql, kl, pos0=m)
    b = R.prologue(_scaled_cfg(0.0), 0, ql, kl, pos0=m)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # and scaling changes the global rotation elsewhere
    assert not np.allclose(qs[:, 1:], R.prologue(_scaled_cfg(0.0), 2, q, k, pos0=(m * 8))[0][:, 1:])


def test_rope_scaling_mutants_are_caught(monkeypatch):
    orig = R.resolve_layer

    def on_local_layers_too(cfg, layer_idx):
        L = dict(orig(cfg, layer_idx))
        L["pos_div"] = float(cfg.rope_scaling_factor)
        return L

    def multiplied(cfg, layer_idx):
        L = dict(orig(cfg, layer_idx))
        if L["pos_div"] != 1.0:
            L["pos_div"] = 1.0 / L["pos_div"]
        return L

    for mutant, layer in ((on_local_layers_too, 0), (multiplied, 2)):
        monkeypatch.setattr(R, "resolve_layer", mutant)
        with pytest.raises(AssertionError):
            test_rope_scaling_matches_brute_force(layer)
        monkeypatch.setattr(R, "resolve_layer", orig)


# --------------------------------------------------------------------------- padded (ragged) prefill
_RAGGED_RANGES = [(3, 11), (0, 7), (2, 10), (5, 5), (0, 11)]     # left pad, right pad, both, empty, none


@pytest.mark.parametrize("W,cap,tied", [(0, 0.0, False), (4, 3.0, False), (0, 0.0, True)])
def test_prefill_ragged_matches_brute_force_mask(W, cap, tied):
    cfg = R.GemmaAttnConfig(num_heads=4, num_kv_heads=2 if not tied else 1, head_dim=8, global_head_dim=8,
                            sliding_window=W, sliding_window_pattern=0 if W else 1, attn_logit_softcapping=cap,
                            k_eq_v=tied, rope_theta=1e4)
    L = R.resolve_layer(cfg, 0)
    B, S = len(_RAGGED_RANGES), 11
    q, k, v = _inputs(23, B, S, 4, L["num_kv_heads"], 8, qscale=2.0)
    start = np.array([a for a, _ in _RAGGED_RANGES])
    end = np.array([b for _, b in _RAGGED_RANGES])
    pos0 = -start                                     # kept tokens start at position 0
    qt, kt = R.prologue(cfg, 0, q, k, pos0=pos0)
    o, l = R.prefill_ragged(cfg, 0, qt, kt, v, start, end)
    keep = [[1 if a <= s < b else 0 for s in range(S)] for a, b in _RAGGED_RANGES]
    ob, lb = brute_layer(_cfg_dict(cfg), 0, q.tolist(), k.tolist(), v.tolist(), pos0=pos0.tolist(), keep=keep)
    assert np.abs(o - np.array(ob)).max() < TOL
    fin = np.isfinite(np.array(lb))
    assert np.array_equal(np.isfinite(l), fin)
    assert np.abs(l[fin] - np.array(lb)[fin]).max() < TOL
    for bi, (a, b_) in enumerate(_RAGGED_RANGES):     # padded rows are exactly zero
        assert np.all(o[bi, :a] == 0) and np.all(o[bi, b_:] == 0)


def test_prefill_ragged_unpadded_is_prefill_and_left_pad_is_shift_invariant():
    cfg = _small_cfg(sliding_window=5, attn_logit_softcapping=4.0)
    q, k, v = _inputs(29, 2, 14, 4, 2, 16)
    o, l = R.prefill(cfg, 0, q, k, v)
    og, lg = R.prefill_ragged(cfg, 0, q, k, v, [0, 0], [14, 14])
    assert np.array_equal(o, og) and np.array_equal(l, lg)
    # left padding by 4: the kept rows equal the unpadded prefill of the same tokens
    pad = np.zeros((2, 4) + q.shape[2:])
    padk = np.zeros((2, 4) + k.shape[2:])
    o2, _ = R.prefill_ragged(cfg, 0, np.concatenate([pad, q], 1), np.concatenate([padk, k], 1),
                             np.concatenate([padk, v], 1), [4, 4], [18, 18])
    assert np.array_equal(o2[:, 4:], o) and np.all(o2[:, :4] == 0)


def test_decode_after_left_padded_prefill_uses_kv_start():
    cfg = _small_cfg(sliding_window=0)
    B, S = 2, 12
    q, k, v = _inputs(31, B, S, 4, 2, 16, qscale=2.0)
    start = np.array([3, 0])
    o, l = R.prefill_ragged(cfg, 0, q, k, v, start, [S, S])
    od, ld = R.decode_multi(cfg, 0, q[:, S - 2:], k, v, [S, S], kv_start=start)
    assert np.abs(od - o[:, S - 2:]).max() < 1e-13 and np.abs(ld - l[:, :, S - 2:]).max() < 1e-13
    # without kv_start the padded rows would be attended
    ow, _ = R.decode_multi(cfg, 0, q[:, S - 2:], k, v, [S, S])
    assert np.abs(ow[0] - o[0, S - 2:]).max() > 1e-6


def test_ragged_mutant_is_caught(monkeypatch):
    orig = R.prefill_ragged

    def keys_not_masked(cfg, layer_idx, q, k, v, seq_start, seq_end):
        out, lse = R.prefill(cfg, layer_idx, q, k, v)
        for b in range(len(seq_start)):
            out[b, :seq_start[b]] = 0
            out[b, seq_end[b]:] = 0
            lse[b, :, :seq_start[b]] = -np.inf
            lse[b, :, seq_end[b]:] = -np.inf
        return out, lse

    monkeypatch.setattr(R, "prefill_ragged", keys_not_masked)
    with pytest.raises(AssertionError):
        test_prefill_ragged_matches_brute_force_mask(0, 0.0, False)
    monkeypatch.setattr(R, "prefill_ragged", orig)


# --------------------------------------------------------------------------- the zero-pad rotary reading
# The Gemma 4 page's "Zero-pad partial rope" has two plain readings (the
# library takes the first): rotate the first r dims in pairs (i, i + r/2) at
# theta^(-2i/r), or rotate the full width in pairs (j, j + D/2) at the
# full-width frequencies theta^(-2j/D) with all but the first r/2 set to 0.
@pytest.mark.parametrize("layer,f", [(0, 0.25), (0, 0.5), (2, 0.25), (2, 0.75), (0, 1.0), (2, 0.0)])
def test_zero_pad_rotary_matches_brute_force(layer, f):
    cfg = R.GemmaAttnConfig(num_heads=4, num_kv_heads=2, head_dim=8, num_global_kv_heads=1,
                            global_head_dim=16, sliding_window=4, sliding_window_pattern=3,
                            rope_theta=1e6, rope_local_theta=1e4, partial_rotary_factor=f,
                            k_eq_v=True, norm_weight_offset=0, attn_logit_softcapping=3.0)
    Lr = R.resolve_layer(cfg, layer)
    D, Hkv = Lr["head_dim"], Lr["num_kv_heads"]
    B, S = 2, 9
    q, k, v = _inputs(19, B, S, 4, Hkv, D, qscale=2.0)
    qw, kw = norm_weight(7, D), norm_weight(8, D)
    pos0 = np.array([3, 1000])
    qt, kt = R.prologue(cfg, layer, q, k, qw, kw, pos0, rotary_layout="zero_pad")
    o, l = R.prefill(cfg, layer, qt, kt, v, block_rows=4)
    p = _cfg_dict(cfg) | dict(rotary_layout="zero_pad")
    ob, lb = brute_layer(p, layer, q.tolist(), k.tolist(), v.tolist(), qw.tolist(), kw.tolist(), pos0.tolist())
    assert np.abs(o - np.array(ob)).max() < TOL
    assert np.abs(l - np.array(lb)).max() < TOL


def test_zero_pad_rotary_closed_forms():
    D, r, theta = 16, 4, 1e4
    x = bf16_bits_to_f64(normal_bf16(41, (1, 3, 2, D)))
    pos = np.array([[0, 7, 300]])
    y = R.rotary_zero_pad(x, pos, theta, r)
    # position 0 is the identity; only dims [0, r/2) and [D/2, D/2 + r/2) move
    assert np.array_equal(y[:, 0], x[:, 0])
    moved = np.any(y != x, axis=(0, 1, 2))
    assert moved.tolist() == [d < r // 2 or D // 2 <= d < D // 2 + r // 2 for d in range(D)]
    # each pair (j, j + D/2) keeps its norm; pair 0 turns by p (frequency 1),
    # pair 1 by p * theta^(-2/D)
    a, b = x[..., :D // 2], x[..., D // 2:]
    ya, yb = y[..., :D // 2], y[..., D // 2:]
    assert np.abs(np.hypot(ya, yb) - np.hypot(a, b)).max() < 1e-12
    e = np.zeros((1, 1, 1, D))
    e[..., 1] = 1.0
    z = R.rotary_zero_pad(e, np.array([[5]]), theta, r)
    w = 5.0 * theta ** (-2.0 / D)
    assert abs(z[0, 0, 0, 1] - math.cos(w)) < 1e-15 and abs(z[0, 0, 0, 1 + D // 2] - math.sin(w)) < 1e-15


def test_rotary_readings_agree_at_full_width_and_differ_when_partial():
    x = bf16_bits_to_f64(normal_bf16(42, (2, 5, 3, 32)))
    pos = np.array([[0, 1, 2, 3, 4], [9, 10, 11, 12, 13]])
    assert np.array_equal(R.rotary(x, pos, 1e6, 32), R.rotary_zero_pad(x, pos, 1e6, 32))
    for r in (2, 8, 16, 30):
        a, b = R.rotary(x, pos, 1e6, r), R.rotary_zero_pad(x, pos, 1e6, r)
        assert np.abs(a - b).max() > 1e-3, r
    # the difference reaches the attention output of a partial layer (the
    # Gemma-4-shaped global layer: r = 128 of 512)
    cfg = R.GemmaAttnConfig(num_heads=2, num_kv_heads=1, head_dim=512, partial_rotary_factor=0.25, k_eq_v=True)
    q, k, _ = _inputs(43, 1, 24, 2, 1, 512)
    o1, _ = R.prefill(cfg, 0, *R.prologue(cfg, 0, q, k, pos0=[100]))
    o2, _ = R.prefill(cfg, 0, *R.prologue(cfg, 0, q, k, pos0=[100], rotary_layout="zero_pad"))
    assert np.abs(o1 - o2).max() > 1e-3


def test_zero_pad_mutant_is_caught(monkeypatch):
    """Frequencies over r instead of D (the first reading's) fail the brute force."""
    def wrong(x, positions, theta, rotary_dim):
        x = np.asarray(x, dtype=np.float64)
        out = x.copy()
        D = x.shape[-1]
        j = np.arange(D // 2, dtype=np.float64)
        omega = np.where(j < rotary_dim // 2, np.power(theta, -2.0 * j / rotary_dim), 0.0)
        phi = np.asarray(positions, dtype=np.float64)[:, :, None, None] * omega
        a, b = x[..., :D // 2], x[..., D // 2:]
        out[..., :D // 2] = a * np.cos(phi) - b * np.sin(phi)
        out[..., D // 2:] = b * np.cos(phi) + a * np.sin(phi)
        return out

    cfg = R.GemmaAttnConfig(num_heads=2, num_kv_heads=1, head_dim=16, partial_rotary_factor=0.5)
    q, k, v = _inputs(44, 1, 7, 2, 1, 16)
    p = _cfg_dict(cfg) | dict(rotary_layout="zero_pad")
    ob, _ = brute_layer(p, 0, q.tolist(), k.tolist(), v.tolist(), pos0=[50])
    o, _ = R.prefill(cfg, 0, *R.prologue(cfg, 0, q, k, pos0=[50], rotary_layout="zero_pad"), v)
    assert np.abs(o - np.array(ob)).max() < TOL
    monkeypatch.setattr(R, "rotary_zero_pad", wrong)
    om, _ = R.prefill(cfg, 0, *R.prologue(cfg, 0, q, k, pos0=[50], rotary_layout="zero_pad"), v)
    assert np.abs(om - np.array(ob)).max() > 1e-3
