"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances: attention outputs max-abs 2e-2 and mean-abs 2e-3 on unit-scale
outputs; prologue outputs within one bf16 ulp of the fp64 value; integer
facts (mask, window, GQA map, decode range) bit-exact.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import gemma_ref as R
from synth import BF16_NAN, bf16_bits_to_f64, ctx_lengths, f32_to_bf16_bits, normal_bf16, norm_weight
from tests.gpu_util import (assert_close, assert_within_one_ulp, from_dev_bf16_bits, from_dev_f64, to_dev,
                            to_dev_bf16)

pytestmark = pytest.mark.gpu

GEMMA2 = dict(num_heads=8, num_kv_heads=4, head_dim=256, sliding_window=300, sliding_window_pattern=2,
              rope_theta=1e4, attn_logit_softcapping=50.0, query_pre_attn_scalar=256.0)
GEMMA3 = dict(num_heads=4, num_kv_heads=1, head_dim=256, sliding_window=128, sliding_window_pattern=6,
              rope_theta=1e6, rope_local_theta=1e4, query_pre_attn_scalar=256.0, norm_weight_offset=1)
GEMMA4 = dict(num_heads=16, num_kv_heads=8, num_global_kv_heads=1, head_dim=256, global_head_dim=512,
              sliding_window=200, sliding_window_pattern=6, rope_theta=1e6, rope_local_theta=1e4,
              partial_rotary_factor=0.25, k_eq_v=True, norm_weight_offset=0)
TINY = dict(num_heads=4, num_kv_heads=1, head_dim=64, sliding_window=64, sliding_window_pattern=0,
            rope_theta=1e4, attn_logit_softcapping=50.0, query_pre_attn_scalar=64.0)


def _cfgs(kw):
    return R.GemmaAttnConfig(**kw), kw


def _layer_inputs(kw, layer, B, S, seed, qscale=1.0, with_norm=False):
    cfg = R.GemmaAttnConfig(**kw)
    L = R.resolve_layer(cfg, layer)
    D, Hkv, Hq = L["head_dim"], L["num_kv_heads"], cfg.num_heads
    q = normal_bf16(seed, (B, S, Hq, D), scale=qscale)
    k = normal_bf16(seed + 1, (B, S, Hkv, D))
    v = normal_bf16(seed + 2, (B, S, Hkv, D))
    qw = norm_weight(seed + 3, D) if with_norm else None
    kw_ = norm_weight(seed + 4, D) if with_norm else None
    return cfg, L, q, k, v, qw, kw_


# ----------------------------------------------------------------------------- end to end
E2E = [
    ("tiny_local", TINY, 0, 1, 256, False),
    ("gemma2_local", GEMMA2, 0, 2, 1000, False),
    ("gemma2_global", GEMMA2, 1, 2, 1000, False),
    ("gemma3_local_qknorm", GEMMA3, 0, 1, 777, True),
    ("gemma3_global_qknorm", GEMMA3, 5, 1, 777, True),
    ("gemma4_global_keqv_partial", GEMMA4, 5, 1, 600, True),
    ("gemma4_local_partial", GEMMA4, 0, 2, 450, True),
]


@pytest.mark.parametrize("name,kw,layer,B,S,norm", E2E, ids=[e[0] for e in E2E])
def test_end_to_end_layer(gpu, name, kw, layer, B, S, norm):
    ga = gpu
    cfg, L, q, k, v, qw, kw_ = _layer_inputs(kw, layer, B, S, seed=100 + layer, with_norm=norm)
    print(f"[e2e] {name} layer={layer} B={B} S={S} D={L['head_dim']} g={L['group']}", flush=True)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    qwd = to_dev(qw) if norm else None
    kwd = to_dev(kw_) if norm else None
    qt, kt = ga.qk_prologue(kw, layer, qd, kd, q_norm_w=qwd, k_norm_w=kwd)
    out, lse = ga.attn_prefill(kw, layer, qt, kt, None if L["k_eq_v"] else vd, want_lse=True)
    import torch

    torch.cuda.synchronize()
    rq, rk = R.prologue(cfg, layer, bf16_bits_to_f64(q), bf16_bits_to_f64(k), qw, kw_)
    # the processed q and k cross the library boundary as bf16
    ro, rl = R.prefill(cfg, layer, R.round_bf16(rq), R.round_bf16(rk), bf16_bits_to_f64(v))
    mx, mn = assert_close(from_dev_f64(out), ro, what=name)
    assert_close(from_dev_f64(lse), rl, max_abs=2e-2, mean_abs=2e-3, what=name + " lse")
    rms = float(np.sqrt(np.mean((from_dev_f64(out) - ro) ** 2)) / np.sqrt(np.mean(ro ** 2)))
    print(f"[e2e] {name}: max-abs {mx:.2e} mean-abs {mn:.2e} rms-rel {rms:.2e}", flush=True)


# ----------------------------------------------------------------------------- prologue only
_WIDE = dict(sliding_window=0, sliding_window_pattern=1, rope_theta=1e4)
PRO = [
    ("d64_full", TINY, 0, None, [0], 67),
    ("d256_norm1", GEMMA3, 0, 1, [0, 70000], 67),
    ("d512_partial_norm0", GEMMA4, 5, 0, [3, 65535], 67),
    ("d256_partial_local", GEMMA4, 1, 0, [0, 12345], 67),
    ("d256_global_rope_scaled8", GEMMA3 | dict(rope_scaling_factor=8.0), 5, 1, [5, 98765], 67),
    ("d512_global_rope_scaled3", GEMMA4 | dict(rope_scaling_factor=3.0), 5, 0, [0, 200001], 67),
    ("d256_local_ignores_scaling", GEMMA3 | dict(rope_scaling_factor=8.0), 0, 1, [7, 4321], 67),
    # rotary widths whose partner distance r/16 is not a power of two (LDS exchange), a
    # half-width r/2 that is not a multiple of 8 (lanes straddling the rotary edge)
    ("d128_rotary48_lds", dict(num_heads=6, num_kv_heads=2, head_dim=128, partial_rotary_factor=0.375) | _WIDE,
     0, 0, [0, 9, 400], 67),
    ("d64_rotary18_lds_nonorm", dict(num_heads=3, num_kv_heads=1, head_dim=64, partial_rotary_factor=0.3) | _WIDE,
     0, None, [2, 0, 77, 5], 67),
    # more (token, head) rows per token than one work item holds
    ("d512_40heads", dict(num_heads=32, num_kv_heads=8, head_dim=512) | _WIDE, 0, 0, [0, 3000], 67),
    # one new token per sequence (decode), many sequences per work item
    ("d64_seq1", TINY, 0, None, list(range(0, 70 * 37, 37)), 1),
    ("d256_seq3", GEMMA2, 0, None, list(range(11, 40 * 101, 101)), 3),
]


@pytest.mark.parametrize("name,kw,layer,offset,pos0,S", PRO, ids=[p[0] for p in PRO])
def test_prologue_within_one_ulp(gpu, name, kw, layer, offset, pos0, S):
    ga = gpu
    kw = dict(kw)
    if offset is not None:
        kw["norm_weight_offset"] = offset
    B = len(pos0)
    cfg, L, q, k, _, qw, kw_ = _layer_inputs(kw, layer, B, S, seed=300, with_norm=offset is not None)
    print(f"[prologue] {name} B={B} S={S} D={L['head_dim']} r={L['rotary_dim']}", flush=True)
    p0 = np.array(pos0, dtype=np.int32)
    qt, kt = ga.qk_prologue(kw, layer, to_dev_bf16(q), to_dev_bf16(k),
                            q_norm_w=None if qw is None else to_dev(qw),
                            k_norm_w=None if kw_ is None else to_dev(kw_), pos0=to_dev(p0))
    rq, rk = R.prologue(cfg, layer, bf16_bits_to_f64(q), bf16_bits_to_f64(k), qw, kw_, p0)
    assert_within_one_ulp(from_dev_f64(qt), rq, what=name + " q")
    assert_within_one_ulp(from_dev_f64(kt), rk, what=name + " k")


def test_prologue_in_place_and_queries_only(gpu):
    ga = gpu
    cfg, L, q, k, _, qw, kw_ = _layer_inputs(GEMMA3, 0, 2, 40, seed=310, with_norm=True)
    qd, kd = to_dev_bf16(q), to_dev_bf16(k)
    a_q, a_k = ga.qk_prologue(GEMMA3, 0, qd, kd, q_norm_w=to_dev(qw), k_norm_w=to_dev(kw_))
    ga.qk_prologue(GEMMA3, 0, qd, kd, q_out=qd, k_out=kd, q_norm_w=to_dev(qw), k_norm_w=to_dev(kw_))
    b_q, _ = ga.qk_prologue(GEMMA3, 0, to_dev_bf16(q), None, q_norm_w=to_dev(qw))
    assert np.array_equal(from_dev_bf16_bits(a_q), from_dev_bf16_bits(qd))
    assert np.array_equal(from_dev_bf16_bits(a_k), from_dev_bf16_bits(kd))
    assert np.array_equal(from_dev_bf16_bits(a_q), from_dev_bf16_bits(b_q))


# ----------------------------------------------------------------------------- attention only, all instantiations
MATRIX = [(D, g, kv, cap, W) for D, g, kv, cap, W in itertools.product(
    [64, 256, 512], [1, 2, 4, 8, 16], [False, True], [0.0, 50.0], [0, 45]) if not (kv and W)]


@pytest.mark.parametrize("D,g,keqv,cap,W", MATRIX)
def test_prefill_instantiations(gpu, D, g, keqv, cap, W):
    ga = gpu
    Hkv = 2 if g <= 4 else 1
    kw = dict(num_heads=g * Hkv, num_kv_heads=Hkv, head_dim=D, sliding_window=W, sliding_window_pattern=0,
              attn_logit_softcapping=cap, k_eq_v=keqv)
    cfg = R.GemmaAttnConfig(**kw)
    B, S = 2, 163
    print(f"[prefill] D={D} g={g} keqv={keqv} cap={cap} W={W}", flush=True)
    q = normal_bf16(500, (B, S, g * Hkv, D), scale=2.0)
    k = normal_bf16(501, (B, S, Hkv, D))
    v = normal_bf16(502, (B, S, Hkv, D))
    out, lse = ga.attn_prefill(kw, 0, to_dev_bf16(q), to_dev_bf16(k), None if keqv else to_dev_bf16(v), want_lse=True)
    ro, rl = R.prefill(cfg, 0, bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v))
    assert_close(from_dev_f64(out), ro, what=f"D{D} g{g}")
    assert_close(from_dev_f64(lse), rl, what=f"D{D} g{g} lse")


@pytest.mark.parametrize("D,g,keqv,cap,S", [(64, 1, False, 0.0, 163), (64, 4, True, 50.0, 163), (256, 2, False, 50.0, 163),
                                             (256, 16, True, 0.0, 97), (512, 16, True, 0.0, 163),
                                             (512, 2, False, 50.0, 1), (256, 4, False, 0.0, 1)])
def test_prefill_writes_only_its_output(gpu, D, g, keqv, cap, S):
    """The output goes into a view of a larger buffer whose guard regions hold a
    sentinel pattern: every guard byte stays unchanged (the last block runs past
    S, so its columns beyond the sequence must not be written), and the view
    matches a plain call bit for bit."""
    import torch

    ga = gpu
    Hkv = 2 if g <= 4 else 1
    kw = dict(num_heads=g * Hkv, num_kv_heads=Hkv, head_dim=D, sliding_window=0, sliding_window_pattern=0,
              attn_logit_softcapping=cap, k_eq_v=keqv)
    B = 2
    print(f"[prefill guard] D={D} g={g} keqv={keqv} S={S}", flush=True)
    q = to_dev_bf16(normal_bf16(510, (B, S, g * Hkv, D)))
    k = to_dev_bf16(normal_bf16(511, (B, S, Hkv, D)))
    v = None if keqv else to_dev_bf16(normal_bf16(512, (B, S, Hkv, D)))
    n = B * S * g * Hkv * D
    guard = 8192                                          # elements; keeps the view 16-byte aligned
    big = torch.full((n + 2 * guard,), 0x5A5A, dtype=torch.int16, device="cuda")
    out = big[guard:guard + n].view(torch.bfloat16).view(B, S, g * Hkv, D)
    ga.attn_prefill(kw, 0, q, k, v, out=out)
    ref = ga.attn_prefill(kw, 0, q, k, v)
    torch.cuda.synchronize()
    host = big.cpu().numpy()
    assert (host[:guard] == 0x5A5A).all() and (host[guard + n:] == 0x5A5A).all(), "a guard element was written"
    assert np.array_equal(host[guard:guard + n], from_dev_bf16_bits(ref).reshape(-1).view(np.int16))


@pytest.mark.parametrize("g", [1, 2, 4, 16])
def test_prefill_eight_and_four_wave_forms_agree(gpu, g):
    """A soft-capped layer of width 256 whose window reaches the whole sequence
    (W = S) runs the eight-wave form; W = S - 1 runs the four-wave form and
    masks only key 0 for the last row.  Every column visits the same tiles in
    the same key order in both, so all other rows agree bit for bit."""
    ga = gpu
    Hkv = 2 if g <= 4 else 1
    B, S, D = 2, 300, 256
    print(f"[prefill forms] g={g} S={S}", flush=True)
    q = to_dev_bf16(normal_bf16(520, (B, S, g * Hkv, D), scale=2.0))
    k = to_dev_bf16(normal_bf16(521, (B, S, Hkv, D)))
    v = to_dev_bf16(normal_bf16(522, (B, S, Hkv, D)))
    outs = []
    for W in (S, S - 1):
        kw = dict(num_heads=g * Hkv, num_kv_heads=Hkv, head_dim=D, sliding_window=W, sliding_window_pattern=0,
                  attn_logit_softcapping=50.0)
        outs.append(ga.attn_prefill(kw, 0, q, k, v, want_lse=True))
    (o8, l8), (o4, l4) = outs
    a8, a4 = from_dev_bf16_bits(o8), from_dev_bf16_bits(o4)
    assert np.array_equal(a8[:, :S - 1], a4[:, :S - 1])
    assert not np.array_equal(a8[:, S - 1], a4[:, S - 1])     # key 0 is masked only in the windowed form
    lw8, lw4 = from_dev_f64(l8), from_dev_f64(l4)
    assert np.array_equal(lw8[:, :, :S - 1], lw4[:, :, :S - 1])


@pytest.mark.parametrize("scale", [8.0, 32.0])
@pytest.mark.parametrize("kw,layer", [(GEMMA2, 0), (GEMMA2, 1), (GEMMA4, 5)])
def test_prefill_peaked(gpu, kw, layer, scale):
    """Large logits reach the soft cap's nonlinear range and give sharp maxima."""
    ga = gpu
    cfg, L, q, k, v, _, _ = _layer_inputs(kw, layer, 1, 333, seed=600, qscale=scale)
    print(f"[peaked] layer={layer} scale={scale}", flush=True)
    out = ga.attn_prefill(kw, layer, to_dev_bf16(q), to_dev_bf16(k), None if L["k_eq_v"] else to_dev_bf16(v))
    ro, _ = R.prefill(cfg, layer, bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v))
    assert_close(from_dev_f64(out), ro, what=f"peaked x{scale}")


# Soft-capped layers first run with the cap as a fixed softmax maximum (every
# capped logit lies below it).  A row whose logits all lie far below the cap
# would put its probabilities near the bottom of the fp32/bf16 range, so the
# workgroup holding it recomputes with a running maximum.  These rows sit next
# to ordinary ones, in the same workgroups and in others.
FAR = [("gemma2_local_4wave", GEMMA2, 0, 2), ("gemma2_global_8wave", GEMMA2, 1, 1), ("tiny_d64", TINY, 0, 1),
       # a cap above 96 log2 units keeps the running maximum from the start
       ("gemma2_local_cap120", GEMMA2 | dict(attn_logit_softcapping=120.0), 0, 1)]


@pytest.mark.parametrize("name,kw,layer,B", FAR, ids=[f[0] for f in FAR])
def test_prefill_capped_rows_far_below_cap(gpu, name, kw, layer, B):
    ga = gpu
    cfg = R.GemmaAttnConfig(**kw)
    L = R.resolve_layer(cfg, layer)
    D, Hkv, Hq = L["head_dim"], L["num_kv_heads"], cfg.num_heads
    S = 700
    # keys close to one direction k0; far rows ask for -c k0, which puts
    # score * scale / cap near -1.3 (capped logits near -0.86 cap) for every key
    k0 = bf16_bits_to_f64(normal_bf16(910, (1, D)))[0]
    noise = bf16_bits_to_f64(normal_bf16(911, (B, S, Hkv, D)))
    k = R.round_bf16(k0[None, None, None, :] + 0.05 * noise)
    v = bf16_bits_to_f64(normal_bf16(912, (B, S, Hkv, D)))
    q = bf16_bits_to_f64(normal_bf16(913, (B, S, Hq, D)))
    c = 1.3 * kw["attn_logit_softcapping"] / (float(k0 @ k0) * L["scale"])
    far = np.zeros((B, S), dtype=bool)
    far[0, 100:164] = True          # a whole query block
    far[:, 5::37] = True            # scattered rows beside ordinary ones
    q = np.where(far[:, :, None, None], R.round_bf16(-c * k0)[None, None, None, :], q)
    print(f"[far] {name} layer={layer} D={D} g={L['group']} far rows {int(far.sum())}", flush=True)
    ro, rl = R.prefill(cfg, layer, q, k, v)
    for b in range(B):   # the rows are far below the cap
        assert np.all(rl[b][:, far[b]] < -0.7 * kw["attn_logit_softcapping"] + np.log(S))
    out, lse = ga.attn_prefill(kw, layer, to_dev_bf16(_bits(q)), to_dev_bf16(_bits(k)),
                               None if L["k_eq_v"] else to_dev_bf16(_bits(v)), want_lse=True)
    assert_close(from_dev_f64(out), ro, what=name)
    assert_close(from_dev_f64(lse), rl, max_abs=2e-2, mean_abs=2e-3, what=name + " lse")


def _bits(x):
    """bf16 bit patterns of values that are already bf16-exact."""
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


# ----------------------------------------------------------------------------- integer facts, bit-exact
@pytest.mark.parametrize("D,g,W", [(64, 4, 64), (256, 2, 100), (512, 16, 0), (256, 1, 1)])
def test_prefill_integer_facts(gpu, D, g, W):
    """q = 0: every allowed key weighs exactly 1, so lse = ln(count) and the
    output is the exact mean; V constant per KV head (distinct powers of two)
    pins the head map; W = 1 returns v itself; row 0 returns v_0."""
    ga = gpu
    import torch

    Hkv = 2
    kw = dict(num_heads=g * Hkv, num_kv_heads=Hkv, head_dim=D, sliding_window=W, sliding_window_pattern=0,
              attn_logit_softcapping=50.0)
    B, S = 1, 150
    q = torch.zeros((B, S, g * Hkv, D), dtype=torch.bfloat16, device="cuda")
    k = to_dev_bf16(normal_bf16(700, (B, S, Hkv, D)))
    vc = torch.empty((B, S, Hkv, D), dtype=torch.bfloat16, device="cuda")
    vc[:, :, 0] = 0.25
    vc[:, :, 1] = 4.0
    out, lse = ga.attn_prefill(kw, 0, q, k, vc, want_lse=True)
    o = from_dev_f64(out)
    assert np.all(o[:, :, :g] == 0.25) and np.all(o[:, :, g:] == 4.0)
    cnt = np.array([i - (max(0, i - W + 1) if W else 0) + 1 for i in range(S)], dtype=np.float64)
    l = from_dev_f64(lse)[0]
    assert np.all(np.rint(np.exp(l)) == cnt[None, :])
    assert np.abs(l - np.log(cnt)[None, :]).max() < 1e-5
    # a random V: row 0 is v_0 bitwise; W = 1 gives v_i bitwise
    v = normal_bf16(701, (B, S, Hkv, D))
    qn = to_dev_bf16(normal_bf16(702, (B, S, g * Hkv, D)))
    out = ga.attn_prefill(kw, 0, qn, k, to_dev_bf16(v))
    ob = from_dev_bf16_bits(out)
    assert np.array_equal(ob[0, 0, :g], np.broadcast_to(v[0, 0, 0], (g, D)))
    if W == 1:
        for hq in range(g * Hkv):
            assert np.array_equal(ob[0, :, hq], v[0, :, hq // g])


# Short windows (at most 1/8 of the sequence): the XCDs sharing a (sequence, KV
# head) pair take contiguous runs of its query blocks, the last run ending in
# padding blocks, and every block past the first window visits its key tiles in
# the shared rotated order.  (B, Hkv) give 1 or 2 pairs (8 or 4 XCDs per pair).
RUNS = [(1, 1, 2, 256, 2100, 200, 0.0), (2, 1, 4, 256, 1700, 160, 50.0), (1, 2, 8, 256, 2500, 300, 0.0),
        (1, 1, 4, 64, 3000, 96, 50.0), (2, 1, 2, 512, 1300, 150, 0.0)]


@pytest.mark.parametrize("B,Hkv,g,D,S,W,cap", RUNS, ids=[f"B{r[0]}-Hkv{r[1]}-g{r[2]}-D{r[3]}-S{r[4]}-W{r[5]}"
                                                         for r in RUNS])
def test_prefill_short_window_block_runs(gpu, B, Hkv, g, D, S, W, cap):
    ga = gpu
    kw = dict(num_heads=g * Hkv, num_kv_heads=Hkv, head_dim=D, sliding_window=W, sliding_window_pattern=0,
              attn_logit_softcapping=cap)
    cfg = R.GemmaAttnConfig(**kw)
    print(f"[prefill runs] B={B} Hkv={Hkv} g={g} D={D} S={S} W={W}", flush=True)
    q = normal_bf16(830, (B, S, g * Hkv, D), scale=2.0)
    k = normal_bf16(831, (B, S, Hkv, D))
    v = normal_bf16(832, (B, S, Hkv, D))
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    out, lse = ga.attn_prefill(kw, 0, qd, kd, vd, want_lse=True)
    again = ga.attn_prefill(kw, 0, qd, kd, vd)
    ro, rl = R.prefill(cfg, 0, bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v))
    assert_close(from_dev_f64(out), ro, what="short-window runs")
    assert_close(from_dev_f64(lse), rl, what="short-window runs lse")
    assert np.array_equal(from_dev_bf16_bits(out), from_dev_bf16_bits(again))


def test_prefill_deterministic(gpu):
    ga = gpu
    cfg, L, q, k, v, _, _ = _layer_inputs(GEMMA2, 0, 2, 700, seed=800)
    a = ga.attn_prefill(GEMMA2, 0, to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v))
    b = ga.attn_prefill(GEMMA2, 0, to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v))
    assert np.array_equal(from_dev_bf16_bits(a), from_dev_bf16_bits(b))


def test_keys_as_values_equals_explicit_copy(gpu):
    ga = gpu
    kw = dict(GEMMA4)
    cfg, L, q, k, _, _, _ = _layer_inputs(kw, 5, 1, 300, seed=900)
    a = ga.attn_prefill(kw, 5, to_dev_bf16(q), to_dev_bf16(k), None)
    kw2 = dict(kw, k_eq_v=False)
    b = ga.attn_prefill(kw2, 5, to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(k.copy()))
    assert np.array_equal(from_dev_bf16_bits(a), from_dev_bf16_bits(b))


# ----------------------------------------------------------------------------- decode
DEC = [
    ("gemma4_local", GEMMA4 | dict(sliding_window=1024), 0),
    ("gemma4_global_keqv", GEMMA4, 5),
    ("gemma2_local_cap", GEMMA2, 0),
    ("tiny_mqa", TINY, 0),
]


@pytest.mark.parametrize("name,kw,layer", DEC, ids=[d[0] for d in DEC])
def test_decode_vs_oracle_with_sentinels(gpu, name, kw, layer):
    ga = gpu
    import torch

    cfg = R.GemmaAttnConfig(**kw)
    L = R.resolve_layer(cfg, layer)
    B, Smax = 6, 3000
    D, Hkv, Hq = L["head_dim"], L["num_kv_heads"], cfg.num_heads
    ctx = ctx_lengths(1234, B, 1, Smax)
    ctx[0], ctx[1] = 1, Smax
    print(f"[decode] {name} ctx={ctx.tolist()}", flush=True)
    kc = normal_bf16(1300, (B, Smax, Hkv, D))
    vc = normal_bf16(1301, (B, Smax, Hkv, D))
    W = L["window"]
    for b in range(B):                     # poison every row the kernel must not read
        lo = max(0, ctx[b] - W) if W else 0
        kc[b, :lo] = BF16_NAN
        kc[b, ctx[b]:] = BF16_NAN
        vc[b, :lo] = BF16_NAN
        vc[b, ctx[b]:] = BF16_NAN
    q = normal_bf16(1302, (B, Hq, D), scale=2.0)
    out, lse = ga.attn_decode(kw, layer, to_dev_bf16(q), to_dev_bf16(kc), None if L["k_eq_v"] else to_dev_bf16(vc),
                              to_dev(ctx), want_lse=True)
    torch.cuda.synchronize()
    ro, rl = R.decode(cfg, layer, bf16_bits_to_f64(q), bf16_bits_to_f64(kc), bf16_bits_to_f64(vc), ctx)
    assert_close(from_dev_f64(out), ro, what=name)
    assert_close(from_dev_f64(lse), rl, what=name + " lse")
    # ctx = 1: the single visible row is returned exactly
    ob = from_dev_bf16_bits(out)
    for hq in range(Hq):
        assert np.array_equal(ob[0, hq], (kc if L["k_eq_v"] else vc)[0, 0, hq // L["group"]])


def test_decode_matches_prefill_rows(gpu):
    """decode at ctx = p + 1 equals prefill row p of the same keys (within tolerance)."""
    ga = gpu
    import torch

    kw = GEMMA2
    cfg = R.GemmaAttnConfig(**kw)
    for layer in (0, 1):
        L = R.resolve_layer(cfg, layer)
        B, S = 2, 900
        q = normal_bf16(1400, (B, S, 8, 256))
        k = normal_bf16(1401, (B, S, 4, 256))
        v = normal_bf16(1402, (B, S, 4, 256))
        full = from_dev_f64(ga.attn_prefill(kw, layer, to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)))
        for p in (0, 299, 300, 899):
            ctx = np.array([p + 1, p + 1], dtype=np.int32)
            out = ga.attn_decode(kw, layer, to_dev_bf16(np.ascontiguousarray(q[:, p])), to_dev_bf16(k),
                                 to_dev_bf16(v), to_dev(ctx))
            torch.cuda.synchronize()
            assert_close(from_dev_f64(out), full[:, p], max_abs=1e-2, mean_abs=1e-3, what=f"row {p}")


def test_decode_zero_context(gpu):
    ga = gpu
    kw = TINY
    q = to_dev_bf16(normal_bf16(1500, (2, 4, 64)))
    kc = to_dev_bf16(normal_bf16(1501, (2, 16, 1, 64)))
    out, lse = ga.attn_decode(kw, 0, q, kc, kc, to_dev(np.array([0, 3], dtype=np.int32)), want_lse=True)
    o, l = from_dev_f64(out), from_dev_f64(lse)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(l[0])) and np.all(np.isfinite(l[1]))
