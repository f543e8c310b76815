"""GPU parity of the fused query rotary (gemma_attn_prefill_qrope).

The attention kernel takes the queries before rotary and turns them itself
(the prologue's rotate-half pairs, angle (p / pos_div) * theta^(-2i/D)), so
the prologue only processes the keys.  Checked against the fp64 oracle
(prologue, then prefill) at the attention tolerance, and against the unfused
path (prologue of q and k, then gemma_attn_prefill) bit for bit: the kernel
turns the query with the prologue's own arithmetic.  A keys-only prologue
must equal the keys of the full prologue bit for bit.
Cases cover g = 1, 2, 4, 8 and 16, the soft-capped local (four-wave) and
global (eight-wave) forms and an uncapped one, ragged tails, first positions
up to 2^30, a single token, rope scaling, and rows whose capped logits all lie
far below the cap (the fixed-maximum pass and its workgroup recompute).
"""
import numpy as np
import pytest

from oracle import gemma_ref as R
from synth import bf16_bits_to_f64, f32_to_bf16_bits, normal_bf16
from tests.gpu_util import assert_close, from_dev_bf16_bits, from_dev_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

GEMMA2 = dict(num_heads=8, num_kv_heads=4, head_dim=256, sliding_window=300, sliding_window_pattern=2,
              rope_theta=1e4, attn_logit_softcapping=50.0, query_pre_attn_scalar=256.0)
_GLOBAL = dict(head_dim=256, sliding_window=0, sliding_window_pattern=1)

# name, config, layer, batch, seq, pos0 (None: zeros), query scale
CASES = [
    ("g2_local_w300", GEMMA2, 0, 2, 450, None, 1.0),
    ("g2_global_wide", GEMMA2, 1, 2, 450, [0, 100000], 1.0),
    ("g2_global_scaled4", GEMMA2 | dict(rope_scaling_factor=4.0), 1, 1, 333, [77], 2.0),
    ("g1_nocap", dict(num_heads=2, num_kv_heads=2, rope_theta=1e4) | _GLOBAL, 0, 2, 163, [5, 9], 2.0),
    ("g4_cap_global", dict(num_heads=8, num_kv_heads=2, rope_theta=1e6, attn_logit_softcapping=30.0) | _GLOBAL,
     0, 1, 290, [31337], 1.0),
    ("g8_local_w100", dict(num_heads=16, num_kv_heads=2, head_dim=256, sliding_window=100, sliding_window_pattern=0,
                           rope_theta=1e4, attn_logit_softcapping=50.0), 0, 1, 257, [3], 1.0),
    ("g16_window_large_pos", dict(num_heads=16, num_kv_heads=1, head_dim=256, sliding_window=64,
                                  sliding_window_pattern=0, rope_theta=1e6), 0, 1, 200, [123456], 1.0),
    # one token; one block with a ragged tail; positions near 2^30 (the fp64 angle's fraction)
    ("g2_one_token", GEMMA2, 1, 3, 1, [0, 7, 1 << 20], 1.0),
    ("g2_one_block_ragged", GEMMA2, 0, 2, 33, [1 << 30, 5], 1.0),
]


@pytest.mark.parametrize("name,kw,layer,B,S,pos0,qscale", CASES, ids=[c[0] for c in CASES])
def test_fused_query_rotary_matches_oracle_and_unfused(gpu, name, kw, layer, B, S, pos0, qscale):
    ga = gpu
    import torch

    cfg = R.GemmaAttnConfig(**kw)
    L = R.resolve_layer(cfg, layer)
    D, Hkv, Hq = L["head_dim"], L["num_kv_heads"], cfg.num_heads
    seed = 4200 + 17 * layer + S
    q = normal_bf16(seed, (B, S, Hq, D), scale=qscale)
    k = normal_bf16(seed + 1, (B, S, Hkv, D))
    v = normal_bf16(seed + 2, (B, S, Hkv, D))
    print(f"[qrope] {name} layer={layer} B={B} S={S} g={L['group']} window={L['window']} pos0={pos0}", flush=True)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    p0 = None if pos0 is None else np.asarray(pos0, dtype=np.int32)
    p0d = None if p0 is None else to_dev(p0)

    _, k_only = ga.qk_prologue(kw, layer, None, kd, pos0=p0d)
    qt, kt = ga.qk_prologue(kw, layer, qd, kd, pos0=p0d)
    out_f, lse_f = ga.attn_prefill_qrope(kw, layer, qd, k_only, vd, pos0=p0d, want_lse=True)
    out_u, lse_u = ga.attn_prefill(kw, layer, qt, kt, vd, want_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev_bf16_bits(k_only), from_dev_bf16_bits(kt)), "keys-only prologue differs"
    assert np.array_equal(from_dev_bf16_bits(qd), q), "the fused call wrote its query input"

    rq, rk = R.prologue(cfg, layer, bf16_bits_to_f64(q), bf16_bits_to_f64(k), pos0=p0)
    ro, rl = R.prefill(cfg, layer, R.round_bf16(rq), R.round_bf16(rk), bf16_bits_to_f64(v))
    mx, mn = assert_close(from_dev_f64(out_f), ro, what=name + " fused out")
    assert_close(from_dev_f64(lse_f), rl, what=name + " fused lse")
    print(f"[qrope] {name}: vs oracle max {mx:.2e} mean {mn:.2e}", flush=True)
    assert np.array_equal(from_dev_bf16_bits(out_f), from_dev_bf16_bits(out_u)), "fused and unfused outputs differ"
    assert np.array_equal(from_dev_f64(lse_f), from_dev_f64(lse_u)), "fused and unfused lse differ"


def test_fused_query_rotary_is_deterministic(gpu):
    ga = gpu
    import torch

    kw, layer, B, S = GEMMA2, 1, 1, 200
    q = to_dev_bf16(normal_bf16(91, (B, S, 8, 256)))
    k = to_dev_bf16(normal_bf16(92, (B, S, 4, 256)))
    v = to_dev_bf16(normal_bf16(93, (B, S, 4, 256)))
    _, kt = ga.qk_prologue(kw, layer, None, k)
    a = ga.attn_prefill_qrope(kw, layer, q, kt, v)
    b = ga.attn_prefill_qrope(kw, layer, q, kt, v)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev_bf16_bits(a), from_dev_bf16_bits(b))


@pytest.mark.parametrize("kw,layer,why", [
    (dict(num_heads=8, num_kv_heads=1, head_dim=512, k_eq_v=True) | dict(sliding_window=0), 0, "width 512"),
    (dict(num_heads=4, num_kv_heads=1, head_dim=64, sliding_window=0), 0, "width 64"),
    (dict(num_heads=8, num_kv_heads=4, head_dim=256, partial_rotary_factor=0.5, sliding_window=0), 0, "partial rotary"),
    (dict(num_heads=8, num_kv_heads=4, head_dim=256, k_eq_v=True, sliding_window=0), 0, "keys as values"),
])
def test_fused_query_rotary_refuses_other_layers(gpu, kw, layer, why):
    ga = gpu
    import torch

    L = R.resolve_layer(R.GemmaAttnConfig(**kw), layer)
    D, Hkv, Hq = L["head_dim"], L["num_kv_heads"], kw["num_heads"]
    q = torch.zeros((1, 8, Hq, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 8, Hkv, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ga.GemmaAttnError) as e:
        ga.attn_prefill_qrope(kw, layer, q, k, k)
    assert e.value.code == ga.GA_ERR_UNSUPPORTED, why


@pytest.mark.parametrize("layer", [0, 1], ids=["local_4wave", "global_8wave"])
def test_fused_query_rotary_capped_rows_far_below_cap(gpu, layer):
    """The fused kernels' fixed-maximum pass and its workgroup recompute: rows
    whose every capped logit lies near -cap sit beside ordinary rows.  Keys
    and the far rows' queries live on the slowest-turning rotary pairs, so the
    rotation keeps the far scores near -1.3 cap / scale over the sequence."""
    ga = gpu
    import torch

    kw = GEMMA2
    cfg = R.GemmaAttnConfig(**kw)
    L = R.resolve_layer(cfg, layer)
    D, Hkv, Hq = L["head_dim"], L["num_kv_heads"], cfg.num_heads
    B, S = 1, 700
    slow = np.zeros(D)
    slow[D // 2 - 16:D // 2] = 1.0
    slow[D - 16:] = 1.0
    k0 = bf16_bits_to_f64(normal_bf16(920, (1, D)))[0] * slow
    noise = bf16_bits_to_f64(normal_bf16(921, (B, S, Hkv, D)))
    k = R.round_bf16(k0[None, None, None, :] + 0.02 * noise * slow)
    v = bf16_bits_to_f64(normal_bf16(922, (B, S, Hkv, D)))
    q = bf16_bits_to_f64(normal_bf16(923, (B, S, Hq, D)))
    c = 1.3 * kw["attn_logit_softcapping"] / (float(k0 @ k0) * L["scale"])
    far = np.zeros((B, S), dtype=bool)
    far[0, 200:264] = True
    far[0, 3::41] = True
    q = np.where(far[:, :, None, None], R.round_bf16(-c * k0)[None, None, None, :], q)
    bits = lambda x: f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    qd, kd, vd = to_dev_bf16(bits(q)), to_dev_bf16(bits(k)), to_dev_bf16(bits(v))
    print(f"[qrope-far] layer={layer} far rows {int(far.sum())}", flush=True)
    _, k_only = ga.qk_prologue(kw, layer, None, kd)
    qt, kt = ga.qk_prologue(kw, layer, qd, kd)
    out_f, lse_f = ga.attn_prefill_qrope(kw, layer, qd, k_only, vd, want_lse=True)
    out_u, lse_u = ga.attn_prefill(kw, layer, qt, kt, vd, want_lse=True)
    torch.cuda.synchronize()
    rq, rk = R.prologue(cfg, layer, q, k)
    ro, rl = R.prefill(cfg, layer, R.round_bf16(rq), R.round_bf16(rk), v)
    assert np.all(rl[0][:, far[0]] < -0.7 * kw["attn_logit_softcapping"] + np.log(S))   # the rows are far
    assert_close(from_dev_f64(out_f), ro, what="fused far out")
    assert_close(from_dev_f64(lse_f), rl, what="fused far lse")
    assert np.array_equal(from_dev_bf16_bits(out_f), from_dev_bf16_bits(out_u)), "fused and unfused outputs differ"
    assert np.array_equal(from_dev_f64(lse_f), from_dev_f64(lse_u)), "fused and unfused lse differ"
