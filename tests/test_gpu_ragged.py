"""GPU parity of padded (ragged) prefill and of decode from a first kept row.

Every padded row of q, k and v holds bf16 NaN: a padded key or value row read
by mistake turns real rows NaN (a masked probability is 0 and 0 * NaN is
NaN), and padded output rows must come back exactly zero.
"""
import numpy as np
import pytest

from oracle import gemma_ref as R
from synth import BF16_NAN, bf16_bits_to_f64, normal_bf16
from tests.gpu_util import assert_close, from_dev_bf16_bits, from_dev_f64, to_dev, to_dev_bf16
from tests.test_gpu_parity import GEMMA2, GEMMA3, GEMMA4, TINY

pytestmark = pytest.mark.gpu

RAG = [
    ("gemma2_local_cap", GEMMA2, 0),
    ("gemma2_global_cap", GEMMA2, 1),
    ("gemma3_local_mqa", GEMMA3, 0),
    ("gemma4_global_keqv_d512", GEMMA4, 5),
    ("gemma4_local", GEMMA4, 0),
    ("tiny_mqa_d64", TINY, 0),
]


def _ranges(S):
    # left pad, right pad (ragged length), both, empty, none, one kept row
    return np.array([[37, S], [0, S - 100], [50, S - 13], [S // 2, S // 2], [0, S], [S - 1, S]], dtype=np.int32)


@pytest.mark.parametrize("name,kw,layer", RAG, ids=[r[0] for r in RAG])
def test_prefill_ragged_vs_oracle_with_nan_padding(gpu, name, kw, layer):
    ga = gpu
    import torch

    cfg = R.GemmaAttnConfig(**kw)
    L = R.resolve_layer(cfg, layer)
    S = 700
    rng = _ranges(S)
    B = len(rng)
    D, Hkv, Hq = L["head_dim"], L["num_kv_heads"], cfg.num_heads
    print(f"[ragged] {name} ranges={rng.tolist()}", flush=True)
    q = normal_bf16(5000, (B, S, Hq, D), scale=2.0)
    k = normal_bf16(5001, (B, S, Hkv, D))
    v = normal_bf16(5002, (B, S, Hkv, D))
    for b, (lo, hi) in enumerate(rng):
        for t in (q, k, v):
            t[b, :lo] = BF16_NAN
            t[b, hi:] = BF16_NAN
    out, lse = ga.attn_prefill(kw, layer, to_dev_bf16(q), to_dev_bf16(k), None if L["k_eq_v"] else to_dev_bf16(v),
                               want_lse=True, seq_start=to_dev(rng[:, 0].copy()), seq_end=to_dev(rng[:, 1].copy()))
    torch.cuda.synchronize()
    qf, kf, vf = (np.nan_to_num(bf16_bits_to_f64(t)) for t in (q, k, v))
    ro, rl = R.prefill_ragged(cfg, layer, qf, kf, vf, rng[:, 0], rng[:, 1])
    got = from_dev_f64(out)
    assert_close(got, ro, what=name)
    gl = from_dev_f64(lse)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(gl), fin)
    assert_close(gl[fin], rl[fin], what=name + " lse")
    bits = from_dev_bf16_bits(out)
    for b, (lo, hi) in enumerate(rng):
        assert np.all(bits[b, :lo] == 0) and np.all(bits[b, hi:] == 0), b


def test_prefill_ragged_full_ranges_equal_prefill(gpu):
    ga = gpu
    import torch

    for kw, layer in ((GEMMA2, 0), (GEMMA4, 5)):
        L = R.resolve_layer(R.GemmaAttnConfig(**kw), layer)
        B, S = 2, 333
        q = to_dev_bf16(normal_bf16(5100, (B, S, kw["num_heads"], L["head_dim"])))
        k = to_dev_bf16(normal_bf16(5101, (B, S, L["num_kv_heads"], L["head_dim"])))
        v = to_dev_bf16(normal_bf16(5102, (B, S, L["num_kv_heads"], L["head_dim"])))
        o1 = ga.attn_prefill(kw, layer, q, k, v)
        o2 = ga.attn_prefill(kw, layer, q, k, v, seq_start=to_dev(np.zeros(B, np.int32)),
                             seq_end=to_dev(np.full(B, S, np.int32)))
        torch.cuda.synchronize()
        assert np.array_equal(from_dev_bf16_bits(o1), from_dev_bf16_bits(o2))


@pytest.mark.parametrize("kw,layer,int8", [(GEMMA2, 1, False), (GEMMA4, 5, False), (GEMMA4, 0, True)])
def test_decode_after_left_padded_prefill(gpu, kw, layer, int8):
    """Decode with kv_start over a left-padded cache equals the padded
    prefill's last rows (oracle), and never reads the padded rows."""
    ga = gpu
    import torch

    cfg = R.GemmaAttnConfig(**kw)
    L = R.resolve_layer(cfg, layer)
    B, S, Lq = 3, 600, 3
    D, Hkv, Hq = L["head_dim"], L["num_kv_heads"], cfg.num_heads
    start = np.array([100, 0, 599], dtype=np.int32)
    print(f"[decode kv_start] layer={layer} int8={int8} start={start.tolist()}", flush=True)
    q = normal_bf16(5200, (B, S, Hq, D), scale=2.0)
    k = normal_bf16(5201, (B, S, Hkv, D))
    v = normal_bf16(5202, (B, S, Hkv, D))
    ctx = np.full(B, S, dtype=np.int32)
    qn = np.ascontiguousarray(q[:, S - Lq:])
    if int8:
        kx = bf16_bits_to_f64(k).astype(np.float32)
        vx = bf16_bits_to_f64(v).astype(np.float32)
        kc, ks = R.quantize_int8(kx)
        vc, vs = R.quantize_int8(vx)
        ks, vs = np.ascontiguousarray(np.swapaxes(ks, 1, 2)), np.ascontiguousarray(np.swapaxes(vs, 1, 2))
        for b in range(B):
            ks[b, :, :start[b]] = np.nan
            vs[b, :, :start[b]] = np.nan
        out = ga.attn_decode_int8(kw, layer, to_dev_bf16(qn), to_dev(kc), to_dev(ks), to_dev(vc), to_dev(vs),
                                  to_dev(ctx), kv_start=to_dev(start))
        torch.cuda.synchronize()
        ro, _ = R.decode_int8(cfg, layer, bf16_bits_to_f64(qn), kc, np.nan_to_num(ks), vc, np.nan_to_num(vs), ctx,
                              kv_start=start)
    else:
        for b in range(B):
            k[b, :start[b]] = BF16_NAN
            v[b, :start[b]] = BF16_NAN
        out = ga.attn_decode_multi(kw, layer, to_dev_bf16(qn), to_dev_bf16(k),
                                   None if L["k_eq_v"] else to_dev_bf16(v), to_dev(ctx), kv_start=to_dev(start))
        torch.cuda.synchronize()
        kf, vf = np.nan_to_num(bf16_bits_to_f64(k)), np.nan_to_num(bf16_bits_to_f64(v))
        ro, _ = R.decode_multi(cfg, layer, bf16_bits_to_f64(qn), kf, vf, ctx, kv_start=start)
        rp, _ = R.prefill_ragged(cfg, layer, bf16_bits_to_f64(q), kf, vf, start, ctx)
        assert np.abs(ro - rp[:, S - Lq:]).max() < 1e-12
    got = from_dev_f64(out)
    assert_close(got, ro, what=f"layer {layer}")
    assert np.all(got[2, :2] == 0)          # sequence 2 keeps only its last row
