"""Pins of the oracle's int8 KV-cache functions (quantize, dequantize, decode).

Checked against what the mathematics fixes, not against the code itself:
exactly representable rows, powers of two, the half-ulp error bound, the
round-to-nearest choice checked in exact rational arithmetic, and decode on a
cache whose dequantization is exact.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import gemma_ref as R
from synth import bf16_bits_to_f64, normal_bf16


def test_integer_rows_are_their_own_codes():
    rng = np.random.default_rng(1)
    x = rng.integers(-127, 128, size=(5, 3, 64)).astype(np.float32)
    x[..., 7] = 127.0                      # every row reaches the code range's end
    x[1, 2, 7] = -127.0
    x[1, 2, 8] = 100.0
    c, s = R.quantize_int8(x)
    assert c.dtype == np.int8 and s.dtype == np.float32 and s.shape == (5, 3)
    assert np.array_equal(c.astype(np.float32), x)
    assert np.all(s == 1.0)


@pytest.mark.parametrize("k", [-20, -3, 0, 5])
def test_power_of_two_scaled_rows(k):
    rng = np.random.default_rng(100 + k)
    ci = rng.integers(-127, 128, size=(4, 32))
    ci[:, 0] = np.where(rng.random(4) < 0.5, 127, -127)
    x = (ci * 2.0 ** k).astype(np.float32)
    c, s = R.quantize_int8(x)
    assert np.array_equal(c.astype(np.int64), ci)
    assert np.all(s == np.float32(2.0 ** k))
    assert np.array_equal(R.dequantize_int8(c, s), x.astype(np.float64))


def test_zero_and_single_element_rows():
    x = np.zeros((3, 16), dtype=np.float32)
    x[1, 4] = -0.37
    x[2, 15] = 1e-30
    c, s = R.quantize_int8(x)
    assert s[0] == 0 and np.all(c[0] == 0)
    assert c[1, 4] == -127 and np.all(np.delete(c[1], 4) == 0)
    assert c[2, 15] == 127 and s[2] > 0


def _nearest_exact(x: float, s: float) -> tuple[int, Fraction]:
    """Round x / s to the nearest integer in exact rational arithmetic."""
    r = Fraction(x) / Fraction(s)
    n = round(r)                           # Fraction rounds half to even
    return n, abs(r - n)


@pytest.mark.parametrize("scale", [1e-3, 1.0, 37.0])
def test_codes_are_the_nearest_integer_in_exact_arithmetic(scale):
    x = (bf16_bits_to_f64(normal_bf16(3, (40, 64))) * scale).astype(np.float32)
    x[5] = 0.0
    c, s = R.quantize_int8(x)
    checked = 0
    for i in range(x.shape[0]):
        amax = float(np.max(np.abs(x[i])))
        if amax == 0:
            assert s[i] == 0 and np.all(c[i] == 0)
            continue
        assert s[i] == np.float32(amax / 127.0) or abs(float(s[i]) - amax / 127.0) <= amax / 127.0 * 2 ** -23
        for d in range(x.shape[1]):
            n, dist = _nearest_exact(float(x[i, d]), float(s[i]))
            # the fp32 quotient can only move the choice when the exact quotient sits at a half
            if abs(dist - Fraction(1, 2)) > Fraction(1, 1 << 16):
                assert int(c[i, d]) == max(-127, min(127, n)), (i, d)
                checked += 1
        err = np.abs(x[i].astype(np.float64) - c[i].astype(np.float64) * float(s[i]))
        assert np.all(err <= float(s[i]) * (0.5 + 2 ** -16))
        assert np.max(np.abs(c[i].astype(np.int64))) == 127
    assert checked > 2000


def test_decode_int8_on_an_exactly_representable_cache():
    """Rows c * 2^k dequantize exactly, so int8 decode equals bf16-free decode."""
    cfg = R.GemmaAttnConfig(num_heads=4, num_kv_heads=2, head_dim=16, sliding_window=6,
                            sliding_window_pattern=0, attn_logit_softcapping=5.0)
    B, Smax, Hkv, D, Lq = 2, 13, 2, 16, 3
    rng = np.random.default_rng(4)

    def cache(seed):
        ci = rng.integers(-127, 128, size=(B, Smax, Hkv, D))
        ci[..., 0] = 127
        k = rng.integers(-9, 3, size=(B, Smax, Hkv))            # a different power of two per row and head
        return (ci * np.exp2(k)[..., None]).astype(np.float32)

    kx, vx = cache(5), cache(6)
    kc, ks = R.quantize_int8(kx)
    vc, vs = R.quantize_int8(vx)
    ks_t, vs_t = np.swapaxes(ks, 1, 2).copy(), np.swapaxes(vs, 1, 2).copy()   # [B,Hkv,Smax]
    q = rng.standard_normal((B, Lq, 4, D))
    ctx = np.array([13, 4])
    o8, l8 = R.decode_int8(cfg, 0, q, kc, ks_t, vc, vs_t, ctx)
    o, l = R.decode_multi(cfg, 0, q, kx.astype(np.float64), vx.astype(np.float64), ctx)
    assert np.array_equal(o8, o) and np.array_equal(l8, l)
    # keys as values: the value codes are ignored
    cfg2 = R.GemmaAttnConfig(num_heads=4, num_kv_heads=1, head_dim=16, global_head_dim=16, sliding_window=0,
                             sliding_window_pattern=1, k_eq_v=True)
    o8, _ = R.decode_int8(cfg2, 0, q, kc[:, :, :1], ks_t[:, :1], None, None, ctx)
    o, _ = R.decode_multi(cfg2, 0, q, kx[:, :, :1].astype(np.float64), None, ctx)
    assert np.array_equal(o8, o)


def test_decode_int8_bytes():
    cfg = R.GemmaAttnConfig(num_heads=16, num_kv_heads=8, head_dim=256, sliding_window=1024,
                            sliding_window_pattern=0)
    # two tokens: spans 1024 and 7 rows; each row is 8 heads x (256 codes + 4 scale bytes), K and V
    assert R.decode_kv_bytes(cfg, 0, [5000, 7], int8=True) == (1024 + 7) * 8 * 260 * 2
    assert R.decode_kv_bytes(cfg, 0, [5000, 7]) == (1024 + 7) * 8 * 512 * 2


# --------------------------------------------------------------------------- planted mistakes
_orig_quantize = R.quantize_int8


def _q_truncate(x):
    x = np.asarray(x, dtype=np.float32)
    s = (np.max(np.abs(x), axis=-1) / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, 1.0).astype(np.float32)
    return np.trunc(x / safe[..., None]).astype(np.int8), s


def _q_divide_by_128(x):
    x = np.asarray(x, dtype=np.float32)
    s = (np.max(np.abs(x), axis=-1) / np.float32(128.0)).astype(np.float32)
    safe = np.where(s > 0, s, 1.0).astype(np.float32)
    return np.clip(np.rint(x / safe[..., None]), -127, 127).astype(np.int8), s


def _q_mean_abs(x):
    x = np.asarray(x, dtype=np.float32)
    s = (np.mean(np.abs(x), axis=-1) / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, 1.0).astype(np.float32)
    return np.clip(np.rint(x / safe[..., None]), -127, 127).astype(np.int8), s


@pytest.mark.parametrize("mutant", [_q_truncate, _q_divide_by_128, _q_mean_abs])
def test_pins_catch_planted_quantizer_mistakes(monkeypatch, mutant):
    monkeypatch.setattr(R, "quantize_int8", mutant)
    caught = 0
    for pin in (lambda: test_power_of_two_scaled_rows(-3),
                lambda: test_codes_are_the_nearest_integer_in_exact_arithmetic(1.0)):
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1


def test_pins_catch_untransposed_scales(monkeypatch):
    orig = R.decode_int8

    def wrong_layout(cfg, layer_idx, q, k_codes, k_scales, v_codes, v_scales, ctx_len):
        L = R.resolve_layer(cfg, layer_idx)
        ks = np.asarray(k_scales).reshape(k_codes.shape[:3])          # reads [B,Hkv,Smax] as [B,Smax,Hkv]
        kd = R.dequantize_int8(k_codes, ks)
        vd = kd if L["k_eq_v"] else R.dequantize_int8(v_codes, np.asarray(v_scales).reshape(v_codes.shape[:3]))
        return R.decode_multi(cfg, layer_idx, q, kd, vd, ctx_len)

    monkeypatch.setattr(R, "decode_int8", wrong_layout)
    with pytest.raises(AssertionError):
        test_decode_int8_on_an_exactly_representable_cache()
    monkeypatch.setattr(R, "decode_int8", orig)
