"""Plant plausible mistakes in the oracle (CPU only) and check the brute force catches each.

Each mutant replaces one oracle step with a wrong variant that a careless
reading of the pages could produce; the scalar brute force must disagree.
"""
import numpy as np
import pytest

from oracle import gemma_ref as R
from oracle.brute import brute_layer
from synth import bf16_bits_to_f64, normal_bf16, norm_weight

_orig_rotary = R.rotary
_orig_allowed = R.allowed
_orig_softcap = R.softcap
_orig_rms = R.rms_norm
_orig_resolve = R.resolve_layer


def _rotary_sign(x, positions, theta, r):
    return _orig_rotary(x, -np.asarray(positions), theta, r)


def _rotary_interleaved(x, positions, theta, r):
    x = np.asarray(x, dtype=np.float64)
    perm = list(range(0, r, 2)) + list(range(1, r, 2)) + list(range(r, x.shape[-1]))
    inv = np.argsort(perm)
    return _orig_rotary(x[..., perm], positions, theta, r)[..., inv]


def _window_plus_one(i, j, window):
    return _orig_allowed(i, j, window + 1 if window > 0 else 0)


def _softcap_unscaled(s, cap):
    return cap * np.tanh(s) if cap > 0 else s


def _norm_no_offset(x, w, eps, offset):
    return _orig_rms(x, w, eps, 0)


def _scale_linear(cfg, layer_idx):
    L = dict(_orig_resolve(cfg, layer_idx))
    L["scale"] = L["scale"] ** 2
    return L


def _theta_swapped(cfg, layer_idx):
    L = dict(_orig_resolve(cfg, layer_idx))
    L["theta"] = cfg.rope_theta if not L["is_global"] else L["theta"]
    return L


MUTANTS = {
    "rotary_sign": ("rotary", _rotary_sign),
    "rotary_interleaved_pairs": ("rotary", _rotary_interleaved),
    "window_off_by_one": ("allowed", _window_plus_one),
    "softcap_unscaled": ("softcap", _softcap_unscaled),
    "norm_offset_dropped": ("rms_norm", _norm_no_offset),
    "scale_not_sqrt": ("resolve_layer", _scale_linear),
    "local_uses_global_theta": ("resolve_layer", _theta_swapped),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(R, attr, fn)
    cfg = R.GemmaAttnConfig(num_heads=4, num_kv_heads=2, head_dim=8, sliding_window=4, sliding_window_pattern=2,
                            rope_theta=1e6, rope_local_theta=1e4, attn_logit_softcapping=3.0,
                            query_pre_attn_scalar=5.0, norm_weight_offset=1)
    B, S, D = 1, 10, 8
    q = bf16_bits_to_f64(normal_bf16(5, (B, S, 4, D), scale=2.0))
    k = bf16_bits_to_f64(normal_bf16(6, (B, S, 2, D)))
    v = bf16_bits_to_f64(normal_bf16(7, (B, S, 2, D)))
    qw, kw = norm_weight(8, D), norm_weight(9, D)
    qt, kt = R.prologue(cfg, 0, q, k, qw, kw)
    o, _ = R.prefill(cfg, 0, qt, kt, v)
    p = {f: getattr(cfg, f) for f in cfg.__dataclass_fields__}
    ob, _ = brute_layer(p, 0, q.tolist(), k.tolist(), v.tolist(), qw.tolist(), kw.tolist())
    assert np.abs(o - np.array(ob)).max() > 1e-6
