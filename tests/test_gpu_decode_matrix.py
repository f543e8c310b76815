"""GPU parity of every decode instantiation the library advertises.

gemma_attn_decode_multi and gemma_attn_decode_int8 take head width D in
{64, 256, 512} and group size g in {1, 2, 4, 8, 16}, with or without keys as
values, with or without the logit soft cap, on local (window) and global
layers, for any number of new tokens.  The matrix below runs each of those
combinations at 1, 4 and 13 new tokens, which between them reach every
kernel form the host plan picks:
  * one 16-column block per workgroup (few query columns per KV head);
  * four column blocks sharing one tile stream (bf16, D >= 256, >= 3 blocks);
  * the 32-key tile kernel (bf16 keys-as-values at D = 512, >= 48 columns);
  * the int8 kernel (codes + per-(token, head) scales);
and both split modes: the balanced key line (a workgroup's range may cross
sequences) and, in the batched cases at the end, one workgroup per sequence.
The group size 8 with one KV head at D = 256 is the multi-query layout of the
Gemma page's GemmaModel table (8 heads, 1 KV head).

Every cache row a sequence may not read holds bf16 NaN (int8: a NaN scale),
so a stray read turns its output non-finite.  Outputs are held to max-abs
2e-2 / mean-abs 2e-3 against the fp64 oracle, lse likewise; tokens with no
visible key must give exactly 0 and -inf.
"""
import itertools

import numpy as np
import pytest

from oracle import gemma_ref as R
from synth import BF16_NAN, bf16_bits_to_f64, ctx_lengths, normal_bf16
from tests.gpu_util import assert_close, from_dev_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

# (D, g, keys-as-values, window); keys as values only on global layers (window 0)
SHAPES = [(D, g, kv, W) for D, g, kv, W in itertools.product([64, 256, 512], [1, 2, 4, 8, 16], [False, True], [0, 45])
          if not (kv and W)]
MATRIX = [(D, g, kv, W, cap, ql) for (D, g, kv, W), cap, ql in itertools.product(SHAPES, [0.0, 50.0], [1, 4, 13])]


def _ids(c):
    D, g, kv, W, cap, ql = c
    return f"D{D}-g{g}-{'keqv' if kv else 'kv'}-W{W}-cap{int(cap)}-L{ql}"


def _config(D, g, keqv, W, cap, hkv):
    # one layer, local when W > 0 (pattern 0: every layer local), else global
    return dict(num_heads=g * hkv, num_kv_heads=hkv, head_dim=D, sliding_window=W, sliding_window_pattern=0,
                attn_logit_softcapping=cap, k_eq_v=keqv)


def _contexts(seed, B, Smax, q_len):
    ctx = ctx_lengths(seed, B, 1, Smax)
    ctx[0] = 1                              # a single visible row for the last token
    ctx[1] = Smax                           # the whole cache
    if B > 2:
        ctx[2] = max(1, q_len - 2)          # fewer keys than new tokens: early tokens see nothing
    return ctx


def _poison(cache, ctx, W, q_len, kv_start=None):
    """NaN in every row outside [lo, ctx) of each sequence (lo from the window of the first new token)."""
    for b in range(cache.shape[0]):
        lo = max(0, int(ctx[b]) - (W + q_len - 1)) if W else 0
        if kv_start is not None:
            lo = max(lo, int(kv_start[b]))
        cache[b, :lo] = BF16_NAN
        cache[b, ctx[b]:] = BF16_NAN


def _check(name, out, lse, ro, rl, ctx, q_len):
    o, l = from_dev_f64(out), from_dev_f64(lse)
    assert_close(o, ro, what=name)
    seen = np.isfinite(rl)
    assert np.array_equal(np.isfinite(l), seen), name + ": rows with / without visible keys differ"
    assert_close(l[seen], rl[seen], what=name + " lse")
    for b in range(len(ctx)):
        for t in range(q_len):
            if ctx[b] - q_len + t < 0:
                assert np.all(o[b, t] == 0.0) and np.all(np.isneginf(l[b, :, t])), (name, b, t)


def _run_bf16(ga, D, g, keqv, W, cap, q_len, B, Smax, hkv, seed, kv_start=None, empty=()):
    import torch

    kw = _config(D, g, keqv, W, cap, hkv)
    cfg = R.GemmaAttnConfig(**kw)
    name = _ids((D, g, keqv, W, cap, q_len)) + f"-B{B}"
    ctx = _contexts(seed, B, Smax, q_len)
    ctx[list(empty)] = 0                    # sequences with nothing to read
    print(f"[decode matrix] {name} ctx={ctx[:6].tolist()}", flush=True)
    kc = normal_bf16(seed + 1, (B, Smax, hkv, D))
    vc = normal_bf16(seed + 2, (B, Smax, hkv, D))
    _poison(kc, ctx, W, q_len, kv_start)
    _poison(vc, ctx, W, q_len, kv_start)
    q = normal_bf16(seed + 3, (B, q_len, g * hkv, D), scale=2.0)
    ks = None if kv_start is None else to_dev(kv_start)
    out, lse = ga.attn_decode_multi(kw, 0, to_dev_bf16(q), to_dev_bf16(kc), None if keqv else to_dev_bf16(vc),
                                    to_dev(ctx), want_lse=True, kv_start=ks)
    torch.cuda.synchronize()
    ro, rl = R.decode_multi(cfg, 0, bf16_bits_to_f64(q), bf16_bits_to_f64(kc), bf16_bits_to_f64(vc), ctx, kv_start)
    _check(name, out, lse, ro, rl, ctx, q_len)


def _run_int8(ga, D, g, keqv, W, cap, q_len, B, Smax, hkv, seed, empty=()):
    import torch

    kw = _config(D, g, keqv, W, cap, hkv)
    cfg = R.GemmaAttnConfig(**kw)
    name = "int8-" + _ids((D, g, keqv, W, cap, q_len)) + f"-B{B}"
    ctx = _contexts(seed, B, Smax, q_len)
    ctx[list(empty)] = 0                    # sequences with nothing to read
    print(f"[decode matrix] {name} ctx={ctx[:6].tolist()}", flush=True)
    kc, ks = R.quantize_int8(bf16_bits_to_f64(normal_bf16(seed + 1, (B, Smax, hkv, D))).astype(np.float32))
    vc, vs = R.quantize_int8(bf16_bits_to_f64(normal_bf16(seed + 2, (B, Smax, hkv, D))).astype(np.float32))
    ks, vs = np.ascontiguousarray(np.swapaxes(ks, 1, 2)), np.ascontiguousarray(np.swapaxes(vs, 1, 2))
    for b in range(B):                     # a NaN scale on every row the kernel must not read
        lo = max(0, int(ctx[b]) - (W + q_len - 1)) if W else 0
        for s_ in (ks, vs):
            s_[b, :, :lo] = np.nan
            s_[b, :, ctx[b]:] = np.nan
    q = normal_bf16(seed + 3, (B, q_len, g * hkv, D), scale=2.0)
    out, lse = ga.attn_decode_int8(kw, 0, to_dev_bf16(q), to_dev(kc), to_dev(ks),
                                   None if keqv else to_dev(vc), None if keqv else to_dev(vs), to_dev(ctx),
                                   want_lse=True)
    torch.cuda.synchronize()
    ro, rl = R.decode_int8(cfg, 0, bf16_bits_to_f64(q), kc, ks, vc, vs, ctx)
    _check(name, out, lse, ro, rl, ctx, q_len)


@pytest.mark.parametrize("D,g,keqv,W,cap,q_len", MATRIX, ids=[_ids(c) for c in MATRIX])
def test_decode_bf16_instantiations(gpu, D, g, keqv, W, cap, q_len):
    hkv = 2 if g <= 4 else 1
    _run_bf16(gpu, D, g, keqv, W, cap, q_len, B=3, Smax=150, hkv=hkv, seed=4000 + D + 10 * g + q_len)


@pytest.mark.parametrize("D,g,keqv,W,cap,q_len", MATRIX, ids=[_ids(c) for c in MATRIX])
def test_decode_int8_instantiations(gpu, D, g, keqv, W, cap, q_len):
    hkv = 2 if g <= 4 else 1
    _run_int8(gpu, D, g, keqv, W, cap, q_len, B=3, Smax=150, hkv=hkv, seed=5000 + D + 10 * g + q_len)


# Enough sequences times KV heads to fill a round of workgroups with short
# (windowed) spans: the plan then gives every sequence one workgroup of its own.
PER_SEQ = [(256, 2, False, 45, 0.0, 1, 8), (256, 2, False, 45, 50.0, 4, 8), (64, 1, False, 30, 0.0, 1, 16),
           (64, 4, False, 30, 50.0, 4, 16), (512, 2, False, 40, 0.0, 1, 8)]


@pytest.mark.parametrize("D,g,keqv,W,cap,q_len,hkv", PER_SEQ,
                         ids=[_ids(c[:6]) + f"-hkv{c[6]}" for c in PER_SEQ])
def test_decode_one_workgroup_per_sequence(gpu, D, g, keqv, W, cap, q_len, hkv):
    # 72 sequences x 8 or 16 KV heads (one column block each) reach the 512 or
    # 1024 workgroups of one round on 256 CUs, and every span is under 8K keys
    B, Smax = 72, 120
    _run_bf16(gpu, D, g, keqv, W, cap, q_len, B=B, Smax=Smax, hkv=hkv, seed=6000 + D + q_len)
    _run_int8(gpu, D, g, keqv, W, cap, q_len, B=B, Smax=Smax, hkv=hkv, seed=6100 + D + q_len)


@pytest.mark.parametrize("D,g,keqv,W,q_len", [(256, 2, False, 45, 1), (256, 2, False, 45, 4), (64, 4, False, 30, 4),
                                               (512, 2, False, 40, 1)])
def test_decode_one_workgroup_per_sequence_empty(gpu, D, g, keqv, W, q_len):
    """One workgroup per sequence writes its sequence's output itself (width <= 256) or its
    partial (width 512): sequences with no readable row (ctx 0, or kv_start at ctx) get zeros
    and lse -inf, and their neighbours are unaffected."""
    hkv = 8 if D != 64 else 16
    B, Smax = 72, 120
    kv_start = np.zeros(B, dtype=np.int32)
    ctx = _contexts(6200 + D + q_len, B, Smax, q_len)
    for b in (5, 40, 71):                   # kv_start at ctx: nothing readable
        kv_start[b] = ctx[b]
    _run_bf16(gpu, D, g, keqv, W, 0.0, q_len, B=B, Smax=Smax, hkv=hkv, seed=6200 + D + q_len, kv_start=kv_start,
              empty=(3, 4, 70))
    _run_int8(gpu, D, g, keqv, W, 50.0, q_len, B=B, Smax=Smax, hkv=hkv, seed=6300 + D + q_len, empty=(0, 3, 71))


@pytest.mark.parametrize("D,g,keqv,W", [(256, 2, False, 45), (512, 16, True, 0), (64, 4, False, 0)])
def test_decode_kv_start_matrix(gpu, D, g, keqv, W):
    """Rows before kv_start[b] are never read (NaN there), on each kernel form."""
    hkv = 2 if g <= 4 else 1
    B, Smax = 4, 150
    kv_start = np.array([0, 37, 149, 10], dtype=np.int32)
    for q_len in (1, 4, 13):
        _run_bf16(gpu, D, g, keqv, W, 0.0, q_len, B=B, Smax=Smax, hkv=hkv, seed=7000 + D + q_len, kv_start=kv_start)
