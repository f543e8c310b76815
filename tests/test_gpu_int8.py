"""GPU parity of the int8 KV-cache path against the oracle.

The quantizer is an integer decision taken in fp32 on both sides, so codes
and scales are compared bit for bit.  int8 decode is compared with the
oracle's decode on the dequantized cache at the attention tolerance (max-abs
2e-2, mean-abs 2e-3).  Scales outside each sequence's readable rows are NaN:
a value row read by mistake turns the output NaN through the value scale.
"""
import numpy as np
import pytest

from oracle import gemma_ref as R
from synth import bf16_bits_to_f64, ctx_lengths, normal_bf16, norm_weight
from tests.gpu_util import assert_close, from_dev_bf16_bits, from_dev_f64, to_dev, to_dev_bf16
from tests.test_gpu_parity import GEMMA2, GEMMA3, GEMMA4, TINY

pytestmark = pytest.mark.gpu


def _rows(seed, shape):
    """bf16 rows of mixed magnitudes, a few all-zero and a few exact c * 2^k rows."""
    x = bf16_bits_to_f64(normal_bf16(seed, shape)).astype(np.float32)
    rng = np.random.default_rng(seed)
    mag = np.exp2(rng.integers(-12, 8, size=shape[:-1])).astype(np.float32)
    x = x * mag[..., None]
    flat = x.reshape(-1, shape[-1])
    flat[::17] = 0.0
    ci = rng.integers(-127, 128, size=(flat[3::29].shape[0], shape[-1]))
    ci[:, 0] = 127
    flat[3::29] = ci * np.float32(2.0 ** -5)
    return x


def _bf16_bits(x32):
    return (np.asarray(x32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("D,Hkv", [(64, 1), (256, 8), (512, 1), (8, 3)])
def test_quantize_bit_exact_and_placed(gpu, D, Hkv):
    ga = gpu
    import torch

    B, S, Smax = 3, 37, 50
    x = _rows(3100 + D, (B, S, Hkv, D))
    assert np.array_equal(bf16_bits_to_f64(_bf16_bits(x)).astype(np.float32), x)   # x is bf16-exact
    pos0 = np.array([0, 20, -5], dtype=np.int32)            # sequence 1 runs past the cache, 2 starts before it
    print(f"[quantize] D={D} Hkv={Hkv} pos0={pos0.tolist()}", flush=True)
    codes = torch.full((B, Smax, Hkv, D), 0x55, dtype=torch.int8, device="cuda")
    scales = torch.full((B, Hkv, Smax), float("nan"), dtype=torch.float32, device="cuda")
    ga.kv_quantize_int8(to_dev_bf16(_bf16_bits(x)), codes, scales, pos0=to_dev(pos0))
    torch.cuda.synchronize()
    c = codes.cpu().numpy()
    s = scales.cpu().numpy()
    rc, rs = R.quantize_int8(x)                              # [B,S,Hkv,D], [B,S,Hkv]
    for b in range(B):
        for p in range(Smax):
            t = p - pos0[b]
            if 0 <= t < S:
                assert np.array_equal(c[b, p], rc[b, t]), (b, p)
                assert np.array_equal(s[b, :, p].view(np.uint32), rs[b, t].view(np.uint32)), (b, p)
            else:
                assert np.all(c[b, p] == 0x55) and np.all(np.isnan(s[b, :, p])), (b, p)


INT8 = [
    ("gemma4_local_q1", GEMMA4 | dict(sliding_window=1024), 0, 1),
    ("gemma4_local_q4", GEMMA4 | dict(sliding_window=1024), 0, 4),
    ("gemma4_global_keqv_q1", GEMMA4, 5, 1),
    ("gemma4_global_keqv_q3", GEMMA4, 5, 3),
    ("gemma2_local_cap_q2", GEMMA2, 0, 2),
    ("gemma2_global_cap_q1", GEMMA2, 1, 1),
    ("gemma3_local_mqa_q16", GEMMA3, 0, 16),
    ("tiny_mqa_q5", TINY, 0, 5),
]


@pytest.mark.parametrize("name,kw,layer,q_len", INT8, ids=[m[0] for m in INT8])
def test_decode_int8_vs_oracle_with_sentinels(gpu, name, kw, layer, q_len):
    ga = gpu
    import torch

    cfg = R.GemmaAttnConfig(**kw)
    L = R.resolve_layer(cfg, layer)
    B, Smax = 5, 2600
    D, Hkv, Hq, W = L["head_dim"], L["num_kv_heads"], cfg.num_heads, L["window"]
    ctx = ctx_lengths(3234 + q_len, B, 1, Smax)
    ctx[0], ctx[1], ctx[2] = 1, Smax, max(1, q_len - 1)
    print(f"[decode_int8] {name} q_len={q_len} ctx={ctx.tolist()}", flush=True)
    kx = bf16_bits_to_f64(normal_bf16(3300, (B, Smax, Hkv, D))).astype(np.float32)
    vx = bf16_bits_to_f64(normal_bf16(3301, (B, Smax, Hkv, D))).astype(np.float32)
    kc, ks = R.quantize_int8(kx)
    vc, vs = R.quantize_int8(vx)
    ks, vs = np.ascontiguousarray(np.swapaxes(ks, 1, 2)), np.ascontiguousarray(np.swapaxes(vs, 1, 2))
    for b in range(B):                     # scales of every row the kernel must not read are NaN
        lo = max(0, ctx[b] - (W + q_len - 1)) if W else 0
        for s_ in (ks, vs):
            s_[b, :, :lo] = np.nan
            s_[b, :, ctx[b]:] = np.nan
    q = normal_bf16(3302, (B, q_len, Hq, D), scale=2.0)
    out, lse = ga.attn_decode_int8(kw, layer, to_dev_bf16(q), to_dev(kc), to_dev(ks), to_dev(vc), to_dev(vs),
                                   to_dev(ctx), want_lse=True)
    torch.cuda.synchronize()
    ro, rl = R.decode_int8(cfg, layer, bf16_bits_to_f64(q), kc, ks, vc, vs, ctx)
    assert_close(from_dev_f64(out), ro, what=name)
    got_l = from_dev_f64(lse)
    seen = np.isfinite(rl)
    assert np.array_equal(np.isfinite(got_l), seen)
    assert_close(got_l[seen], rl[seen], what=name + " lse")
    o = from_dev_f64(out)
    for t in range(q_len):                 # tokens before position 0 see nothing
        if ctx[0] - q_len + t < 0:
            assert np.all(o[0, t] == 0.0)


@pytest.mark.parametrize("kw,layer", [(GEMMA2, 0), (GEMMA4, 5), (TINY, 0)])
def test_decode_int8_exact_cache_matches_bf16_decode(gpu, kw, layer):
    """Codes with power-of-two scales dequantize to bf16 values exactly, so the
    int8 path and the bf16 path see the same cache."""
    ga = gpu
    import torch

    cfg = R.GemmaAttnConfig(**kw)
    L = R.resolve_layer(cfg, layer)
    B, Smax, Lq = 3, 1500, 2
    D, Hkv, Hq = L["head_dim"], L["num_kv_heads"], cfg.num_heads
    rng = np.random.default_rng(3400)

    def cache():
        ci = rng.integers(-127, 128, size=(B, Smax, Hkv, D))
        ci[..., 0] = 127
        return (ci * np.exp2(rng.integers(-13, -8, size=(B, Smax, Hkv)))[..., None]).astype(np.float32)   # |x| < 0.5

    kx, vx = cache(), cache()
    kc, ks = R.quantize_int8(kx)
    vc, vs = R.quantize_int8(vx)
    ks, vs = np.ascontiguousarray(np.swapaxes(ks, 1, 2)), np.ascontiguousarray(np.swapaxes(vs, 1, 2))
    ctx = to_dev(np.array([1500, 700, 33], dtype=np.int32))
    q = to_dev_bf16(normal_bf16(3401, (B, Lq, Hq, D)))
    o8 = ga.attn_decode_int8(kw, layer, q, to_dev(kc), to_dev(ks), to_dev(vc), to_dev(vs), ctx)
    o16 = ga.attn_decode_multi(kw, layer, q, to_dev_bf16(_bf16_bits(kx)), to_dev_bf16(_bf16_bits(vx)), ctx)
    torch.cuda.synchronize()
    assert_close(from_dev_f64(o8), from_dev_f64(o16), max_abs=1e-2, mean_abs=1e-3, what="int8 vs bf16")


@pytest.mark.parametrize("kw,layer", [(GEMMA2, 0), (GEMMA4, 0), (GEMMA3, 0), (TINY, 0)])
def test_decode_int8_uniform_values_are_exact(gpu, kw, layer):
    """The output is a convex combination of value rows, so whatever the scores:
    value codes all equal to c with unit scales give c, and one value row
    repeated over every key gives that row.  The kernel's value product carries
    1152 * sum(p * vs), removed after the product; the product and the separate
    sum round differently in fp32, which leaves at most a few 1152 * 2^-24 of
    the value scale (1 here): within 2^-10, and nonzero codes round back to the
    exact bf16 integer.  A wrong offset term misses by hundreds."""
    ga = gpu
    import torch

    cfg = R.GemmaAttnConfig(**kw)
    L = R.resolve_layer(cfg, layer)
    B, Smax = 3, 300
    D, Hkv, Hq = L["head_dim"], L["num_kv_heads"], cfg.num_heads
    rng = np.random.default_rng(3450)
    kc = to_dev(rng.integers(-127, 128, size=(B, Smax, Hkv, D)).astype(np.int8))
    ks = to_dev(np.full((B, Hkv, Smax), 0.02, dtype=np.float32))
    vs = to_dev(np.ones((B, Hkv, Smax), dtype=np.float32))
    q = to_dev_bf16(normal_bf16(3451, (B, 1, Hq, D), scale=3.0))
    for ctx_list in ([300, 1, 33], [2, 17, 299]):
        ctx = to_dev(np.array(ctx_list, dtype=np.int32))
        for c in (0, 1, -7, 127, -127):
            vc = to_dev(np.full((B, Smax, Hkv, D), c, dtype=np.int8))
            o = ga.attn_decode_int8(kw, layer, q, kc, ks, vc, vs, ctx)
            torch.cuda.synchronize()
            got = from_dev_f64(o)
            assert np.all(np.abs(got - c) <= 2.0 ** -10), (ctx_list, c, np.max(np.abs(got - c)))
            if c != 0:
                assert np.all(got == c), (ctx_list, c)
        row = rng.integers(-127, 128, size=(Hkv, D)).astype(np.int8)
        vc = to_dev(np.ascontiguousarray(np.broadcast_to(row, (B, Smax, Hkv, D))))
        o = from_dev_f64(ga.attn_decode_int8(kw, layer, q, kc, ks, vc, vs, ctx))
        torch.cuda.synchronize()
        for h in range(Hq):
            want = row[h // L["group"]].astype(np.float64)
            assert np.all(np.abs(o[:, :, h] - want) <= 2.0 ** -10), (ctx_list, h)
            assert np.all((o[:, :, h] == want) | (want == 0)), (ctx_list, h)


PRO8 = [("gemma2_local", GEMMA2, 0), ("gemma3_global", GEMMA3, 5), ("gemma4_local", GEMMA4, 0),
        ("gemma4_global_keqv", GEMMA4, 5)]


@pytest.mark.parametrize("name,kw,layer", PRO8, ids=[p[0] for p in PRO8])
def test_prologue_cache_int8(gpu, name, kw, layer):
    """The fused append equals the bf16 append followed by the quantizer, bit
    for bit; against the oracle's prologue the codes are within one step
    (the two bf16 roundings may differ by an ulp); other rows are untouched."""
    ga = gpu
    import torch

    cfg = R.GemmaAttnConfig(**kw)
    L = R.resolve_layer(cfg, layer)
    B, Lq, Smax = 3, 5, 24
    D, Hkv, Hq = L["head_dim"], L["num_kv_heads"], cfg.num_heads
    ctx = np.array([5, 24, 2], dtype=np.int32)
    print(f"[prologue_cache_int8] {name} ctx={ctx.tolist()}", flush=True)
    q = normal_bf16(3500, (B, Lq, Hq, D))
    k = normal_bf16(3501, (B, Lq, Hkv, D))
    v = normal_bf16(3502, (B, Lq, Hkv, D))
    qw, kwt = norm_weight(3503, D), norm_weight(3504, D)
    kc = torch.full((B, Smax, Hkv, D), 0x55, dtype=torch.int8, device="cuda")
    ks = torch.full((B, Hkv, Smax), float("nan"), dtype=torch.float32, device="cuda")
    vc, vs = kc.clone(), ks.clone()
    kvl = not L["k_eq_v"]
    q_out = ga.qk_prologue_cache_int8(kw, layer, to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), kc, ks,
                                      vc if kvl else None, vs if kvl else None, to_dev(ctx), q_norm_w=to_dev(qw),
                                      k_norm_w=to_dev(kwt))
    # unfused: bf16 append into a scratch cache, then the quantizer on the new rows
    kb = torch.zeros((B, Smax, Hkv, D), dtype=torch.bfloat16, device="cuda")
    vb = torch.zeros_like(kb)
    q_ref = ga.qk_prologue_cache(kw, layer, to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), kb, vb if kvl else None,
                                 to_dev(ctx), q_norm_w=to_dev(qw), k_norm_w=to_dev(kwt))
    torch.cuda.synchronize()
    assert np.array_equal(from_dev_bf16_bits(q_out), from_dev_bf16_bits(q_ref))
    c8, s8 = kc.cpu().numpy(), ks.cpu().numpy()
    kbn = from_dev_bf16_bits(kb)
    # the rows the fused call wrote, quantized by the oracle from the bf16 append's rows
    rc, rs = R.quantize_int8(bf16_bits_to_f64(kbn).astype(np.float32))
    qp = R.round_bf16(R.prologue(cfg, layer, bf16_bits_to_f64(q), bf16_bits_to_f64(k), qw, kwt,
                                 pos0=(ctx - Lq))[1])
    oc, _ = R.quantize_int8(qp.astype(np.float32))
    for b in range(B):
        for p in range(Smax):
            t = p - (int(ctx[b]) - Lq)
            if 0 <= t < Lq:
                assert np.array_equal(c8[b, p], rc[b, p]), (b, p)
                assert np.array_equal(s8[b, :, p].view(np.uint32), rs[b, p].view(np.uint32)), (b, p)
                assert np.max(np.abs(c8[b, p].astype(int) - oc[b, t].astype(int))) <= 1, (b, p)
            else:
                assert np.all(c8[b, p] == 0x55) and np.all(np.isnan(s8[b, :, p])), (b, p)
    if kvl:
        vcn, vsn = vc.cpu().numpy(), vs.cpu().numpy()
        rvc, rvs = R.quantize_int8(bf16_bits_to_f64(v).astype(np.float32))
        for b in range(B):
            for t in range(Lq):
                p = int(ctx[b]) - Lq + t
                if 0 <= p < Smax:
                    assert np.array_equal(vcn[b, p], rvc[b, t]), (b, p)
                    assert np.array_equal(vsn[b, :, p].view(np.uint32), rvs[b, t].view(np.uint32)), (b, p)
