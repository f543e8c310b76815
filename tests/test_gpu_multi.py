"""GPU parity of the multi-token entry points against the fp64 oracle.

gemma_attn_decode_multi (several new tokens per sequence against the cache:
chunked prefill, draft verification) and gemma_qk_prologue_cache (the
prologue that appends the new keys and values to the cache).  Same bar as the
single-token path: attention outputs max-abs 2e-2 / mean-abs 2e-3, the cache
rows bitwise equal to what the row-mode prologue writes, untouched rows
bitwise untouched.
"""
import numpy as np
import pytest

from oracle import gemma_ref as R
from synth import BF16_NAN, bf16_bits_to_f64, ctx_lengths, normal_bf16, norm_weight
from tests.gpu_util import assert_close, from_dev_bf16_bits, from_dev_f64, to_dev, to_dev_bf16
from tests.test_gpu_parity import GEMMA2, GEMMA3, GEMMA4, TINY

pytestmark = pytest.mark.gpu

MULTI = [
    ("gemma4_local_q4", GEMMA4 | dict(sliding_window=1024), 0, 4),
    ("gemma4_global_keqv_q3", GEMMA4, 5, 3),
    # many columns per KV head at width 512 (the 32-key tile kernel): a capped
    # variant with a partly filled second column group, and four column groups
    ("gemma4_global_keqv_cap_q5", GEMMA4 | dict(attn_logit_softcapping=30.0), 5, 5),
    ("gemma4_global_keqv_q16", GEMMA4, 5, 16),
    ("gemma2_local_cap_q8", GEMMA2, 0, 8),
    ("gemma2_global_cap_q5", GEMMA2, 1, 5),
    ("gemma3_local_mqa_q16", GEMMA3, 0, 16),
    ("tiny_mqa_q7", TINY, 0, 7),
]


@pytest.mark.parametrize("name,kw,layer,q_len", MULTI, ids=[m[0] for m in MULTI])
def test_decode_multi_vs_oracle_with_sentinels(gpu, name, kw, layer, q_len):
    ga = gpu
    import torch

    cfg = R.GemmaAttnConfig(**kw)
    L = R.resolve_layer(cfg, layer)
    B, Smax = 5, 2500
    D, Hkv, Hq, W = L["head_dim"], L["num_kv_heads"], cfg.num_heads, L["window"]
    ctx = ctx_lengths(2234 + q_len, B, 1, Smax)
    ctx[0], ctx[1], ctx[2] = 1, Smax, max(1, q_len - 2)    # fewer keys than new tokens in rows 0 and 2
    print(f"[decode_multi] {name} q_len={q_len} ctx={ctx.tolist()}", flush=True)
    kc = normal_bf16(2300, (B, Smax, Hkv, D))
    vc = normal_bf16(2301, (B, Smax, Hkv, D))
    for b in range(B):                     # poison every row the kernel must not read
        lo = max(0, ctx[b] - (W + q_len - 1)) if W else 0
        for c in (kc, vc):
            c[b, :lo] = BF16_NAN
            c[b, ctx[b]:] = BF16_NAN
    q = normal_bf16(2302, (B, q_len, Hq, D), scale=2.0)
    out, lse = ga.attn_decode_multi(kw, layer, to_dev_bf16(q), to_dev_bf16(kc),
                                    None if L["k_eq_v"] else to_dev_bf16(vc), to_dev(ctx), want_lse=True)
    torch.cuda.synchronize()
    ro, rl = R.decode_multi(cfg, layer, bf16_bits_to_f64(q), bf16_bits_to_f64(kc), bf16_bits_to_f64(vc), ctx)
    assert_close(from_dev_f64(out), ro, what=name)
    got_l = from_dev_f64(lse)
    seen = np.isfinite(rl)
    assert np.array_equal(np.isfinite(got_l), seen)
    assert_close(got_l[seen], rl[seen], what=name + " lse")
    # integer facts: a token with no visible key gives exactly 0 / -inf; the
    # first token of sequence 0 sees only cache row 0 and returns it exactly
    o = from_dev_f64(out)
    l = from_dev_f64(lse)
    for b in range(B):
        for t in range(q_len):
            if ctx[b] - q_len + t < 0:
                assert np.all(o[b, t] == 0.0) and np.all(np.isneginf(l[b, :, t])), (b, t)
            else:
                assert np.all(np.isfinite(l[b, :, t])), (b, t)
    ob = from_dev_bf16_bits(out)
    vals = kc if L["k_eq_v"] else vc
    for h in range(Hq):
        assert np.array_equal(ob[0, q_len - 1, h], vals[0, 0, h // L["group"]])


@pytest.mark.parametrize("kw,layer", [(GEMMA2, 0), (GEMMA4, 5), (TINY, 0)])
def test_decode_multi_one_token_is_decode(gpu, kw, layer):
    """q_len = 1 is bitwise the single-token decode entry point."""
    ga = gpu
    import torch

    cfg = R.GemmaAttnConfig(**kw)
    L = R.resolve_layer(cfg, layer)
    B, Smax = 3, 1700
    D, Hkv, Hq = L["head_dim"], L["num_kv_heads"], cfg.num_heads
    ctx = to_dev(np.array([1700, 5, 333], dtype=np.int32))
    kc = to_dev_bf16(normal_bf16(2400, (B, Smax, Hkv, D)))
    vc = to_dev_bf16(normal_bf16(2401, (B, Smax, Hkv, D)))
    q = normal_bf16(2402, (B, Hq, D))
    o1, l1 = ga.attn_decode(kw, layer, to_dev_bf16(q), kc, vc, ctx, want_lse=True)
    o2, l2 = ga.attn_decode_multi(kw, layer, to_dev_bf16(q.reshape(B, 1, Hq, D)), kc, vc, ctx, want_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev_bf16_bits(o1), from_dev_bf16_bits(o2).reshape(B, Hq, D))
    assert np.array_equal(from_dev_f64(l1), from_dev_f64(l2).reshape(B, Hq))


PRO_CACHE = [
    ("gemma2_local", GEMMA2, 0, 0),
    ("gemma3_global_norm1", GEMMA3, 5, 1),
    ("gemma4_local_partial", GEMMA4, 0, 0),
    ("gemma4_global_keqv", GEMMA4, 5, 0),
]


@pytest.mark.parametrize("name,kw,layer,offset", PRO_CACHE, ids=[p[0] for p in PRO_CACHE])
def test_prologue_cache_append(gpu, name, kw, layer, offset):
    """Cache rows ctx-L..ctx-1 get exactly the row-mode prologue's keys and the
    raw values; every other cache row keeps its sentinel bits."""
    ga = gpu
    import torch

    kw = kw | dict(norm_weight_offset=offset)
    cfg = R.GemmaAttnConfig(**kw)
    L = R.resolve_layer(cfg, layer)
    B, Lq, Smax = 4, 6, 40
    D, Hkv, Hq = L["head_dim"], L["num_kv_heads"], cfg.num_heads
    ctx = np.array([6, 40, 3, 23], dtype=np.int32)   # sequence 2: three new tokens fall before row 0
    print(f"[prologue_cache] {name} ctx={ctx.tolist()}", flush=True)
    q = normal_bf16(2500, (B, Lq, Hq, D))
    k = normal_bf16(2501, (B, Lq, Hkv, D))
    v = normal_bf16(2502, (B, Lq, Hkv, D))
    qw, kwt = norm_weight(2503, D), norm_weight(2504, D)
    kc0 = normal_bf16(2505, (B, Smax, Hkv, D))
    vc0 = normal_bf16(2506, (B, Smax, Hkv, D))
    kc, vc = to_dev_bf16(kc0), to_dev_bf16(vc0)
    q_out = ga.qk_prologue_cache(kw, layer, to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), kc,
                                 None if L["k_eq_v"] else vc, to_dev(ctx), q_norm_w=to_dev(qw), k_norm_w=to_dev(kwt))
    # the row-mode prologue at positions pos0 = ctx - L
    pos0 = (ctx - Lq).astype(np.int32)
    q_ref, k_ref = ga.qk_prologue(kw, layer, to_dev_bf16(q), to_dev_bf16(k), q_norm_w=to_dev(qw),
                                  k_norm_w=to_dev(kwt), pos0=to_dev(pos0))
    torch.cuda.synchronize()
    assert np.array_equal(from_dev_bf16_bits(q_out), from_dev_bf16_bits(q_ref))
    kcb, vcb, krb = from_dev_bf16_bits(kc), from_dev_bf16_bits(vc), from_dev_bf16_bits(k_ref)
    for b in range(B):
        for s in range(Smax):
            t = s - (int(ctx[b]) - Lq)
            if 0 <= t < Lq:
                assert np.array_equal(kcb[b, s], krb[b, t]), (b, s)
                if not L["k_eq_v"]:
                    assert np.array_equal(vcb[b, s], v[b, t]), (b, s)
                else:
                    assert np.array_equal(vcb[b, s], vc0[b, s]), (b, s)
            else:
                assert np.array_equal(kcb[b, s], kc0[b, s]), (b, s)
                assert np.array_equal(vcb[b, s], vc0[b, s]), (b, s)


@pytest.mark.parametrize("kw,layer,chunk", [(GEMMA2, 0, 96), (GEMMA2, 1, 128), (GEMMA4, 5, 100),
                                            (GEMMA4, 0, 64), (GEMMA3, 0, 33)])
def test_chunked_prefill_through_the_cache(gpu, kw, layer, chunk):
    """A prompt fed in chunks (prologue_cache, then decode_multi per chunk)
    matches the oracle's prologue + whole-prompt prefill."""
    ga = gpu
    import torch

    cfg = R.GemmaAttnConfig(**kw)
    L = R.resolve_layer(cfg, layer)
    B, S = 2, 460
    D, Hkv, Hq = L["head_dim"], L["num_kv_heads"], cfg.num_heads
    q = normal_bf16(2600, (B, S, Hq, D))
    k = normal_bf16(2601, (B, S, Hkv, D))
    v = normal_bf16(2602, (B, S, Hkv, D))
    qw, kwt = norm_weight(2603, D), norm_weight(2604, D)
    print(f"[chunked] layer={layer} D={D} chunk={chunk}", flush=True)
    kc = torch.full((B, S, Hkv, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    outs = []
    for s0 in range(0, S, chunk):
        s1 = min(S, s0 + chunk)
        ctx = to_dev(np.full(B, s1, dtype=np.int32))
        qc = ga.qk_prologue_cache(kw, layer, to_dev_bf16(np.ascontiguousarray(q[:, s0:s1])),
                                  to_dev_bf16(np.ascontiguousarray(k[:, s0:s1])),
                                  to_dev_bf16(np.ascontiguousarray(v[:, s0:s1])), kc,
                                  None if L["k_eq_v"] else vc, ctx, q_norm_w=to_dev(qw), k_norm_w=to_dev(kwt))
        outs.append(ga.attn_decode_multi(kw, layer, qc, kc, None if L["k_eq_v"] else vc, ctx))
    torch.cuda.synchronize()
    got = np.concatenate([from_dev_f64(o) for o in outs], axis=1)
    qp, kp = R.prologue(cfg, layer, bf16_bits_to_f64(q), bf16_bits_to_f64(k), qw, kwt)
    qp, kp = R.round_bf16(qp), R.round_bf16(kp)
    ro, _ = R.prefill(cfg, layer, qp, kp, bf16_bits_to_f64(v))
    assert_close(got, ro, what=f"chunked layer {layer}")
