"""The C-ABI library on the CPU: it loads, exports every declared entry point,
matches the C struct layouts, resolves layers exactly like the oracle and
rejects bad arguments before any HIP call."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import gemma_ref as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemma_attn.h")


@pytest.fixture(scope="module")
def ga():
    import decoder_attention_amd as ga

    if not os.path.exists(ga.LIB_PATH):
        pytest.skip("library not built (python -m decoder_attention_amd.build)")
    ga.load()
    return ga


def _declared_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(gemma_\w+)\s*\(", txt, flags=re.M)))


def test_exports_every_declared_symbol(ga):
    names = _declared_functions()
    assert set(names) == {"gemma_attn_resolve_layer", "gemma_qk_prologue", "gemma_attn_prefill",
                          "gemma_attn_decode_workspace_size", "gemma_attn_decode", "gemma_attn_strerror",
                          "gemma_attn_decode_multi", "gemma_attn_decode_multi_workspace_size",
                          "gemma_qk_prologue_cache", "gemma_attn_decode_int8", "gemma_qk_prologue_cache_int8",
                          "gemma_kv_quantize_int8", "gemma_attn_prefill_ragged", "gemma_attn_decode_multi_noalloc",
                          "gemma_attn_prefill_qrope"}
    lib = ctypes.CDLL(ga.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_load_before_torch_keeps_one_hip_runtime(ga):
    """torch bundles a HIP runtime under the soname the library links against.
    load() called before anything imported torch must still leave a single
    runtime in the process (two runtimes make the library's launches on
    torch's streams fail)."""
    import sys

    code = ("import decoder_attention_amd as ga; ga.load(); "
            "print(len(set(l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l)))")
    out = subprocess.check_output([sys.executable, "-c", code], cwd=ROOT, text=True)
    assert out.strip().splitlines()[-1] == "1"


def test_lds_poisoning_debug_build_exports_the_same_symbols():
    """The debug build (every kernel's LDS filled with NaN bytes before use)
    is the same library: the same entry points, loadable on the CPU."""
    from decoder_attention_amd import build as b

    if not os.path.exists(b.LIB_LDSNAN):
        pytest.skip("debug build not built (python -m decoder_attention_amd.build)")
    lib = ctypes.CDLL(b.LIB_LDSNAN)
    for n in _declared_functions():
        assert hasattr(lib, n), n


def test_struct_layout_matches_c(tmp_path):
    src = tmp_path / "sz.c"
    src.write_text('#include "gemma_attn.h"\n#include <stdio.h>\n#include <stddef.h>\n'
                   'int main(void){printf("%zu %zu %zu %zu %zu %zu %zu\\n", sizeof(gemma_attn_config), sizeof(gemma_attn_layer),'
                   ' offsetof(gemma_attn_config, rope_theta), offsetof(gemma_attn_config, norm_eps),'
                   ' offsetof(gemma_attn_layer, softcap), offsetof(gemma_attn_config, rope_scaling_factor),'
                   ' offsetof(gemma_attn_layer, pos_div)); return 0;}\n')
    exe = tmp_path / "sz"
    subprocess.check_call(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)])
    got = [int(x) for x in subprocess.check_output([str(exe)]).split()]
    import decoder_attention_amd as ga

    assert got == [ctypes.sizeof(ga.CConfig), ctypes.sizeof(ga.CLayer), ga.CConfig.rope_theta.offset,
                   ga.CConfig.norm_eps.offset, ga.CLayer.softcap.offset, ga.CConfig.rope_scaling_factor.offset,
                   ga.CLayer.pos_div.offset]


CFGS = [
    dict(num_heads=16, num_kv_heads=8, num_global_kv_heads=1, head_dim=256, global_head_dim=512, sliding_window=1024,
         sliding_window_pattern=6, rope_theta=1e6, rope_local_theta=1e4, partial_rotary_factor=0.25, k_eq_v=True),
    dict(num_heads=8, num_kv_heads=4, head_dim=256, sliding_window=4096, sliding_window_pattern=2,
         query_pre_attn_scalar=256.0, attn_logit_softcapping=50.0),
    dict(num_heads=4, num_kv_heads=1, head_dim=256, sliding_window=512, sliding_window_pattern=6, rope_theta=1e6,
         rope_local_theta=1e4, norm_weight_offset=1),
    dict(num_heads=8, num_kv_heads=1, head_dim=256, sliding_window=0),
    dict(num_heads=6, num_kv_heads=3, head_dim=64, sliding_window=7, sliding_window_pattern=0,
         partial_rotary_factor=0.3),
    dict(num_heads=6, num_kv_heads=3, head_dim=96, sliding_window=7, sliding_window_pattern=1,
         partial_rotary_factor=0.7, query_pre_attn_scalar=10.0),
    dict(num_heads=4, num_kv_heads=1, head_dim=256, sliding_window=512, sliding_window_pattern=6, rope_theta=1e6,
         rope_local_theta=1e4, rope_scaling_factor=8.0),
]


@pytest.mark.parametrize("kw", CFGS)
def test_resolve_layer_matches_oracle(ga, kw):
    cfg = R.GemmaAttnConfig(**kw)
    for layer in range(64):
        a = ga.resolve_layer(kw, layer)
        b = R.resolve_layer(cfg, layer)
        for key in ("is_global", "window", "num_kv_heads", "head_dim", "group", "rotary_dim", "k_eq_v", "theta",
                    "scale", "softcap", "pos_div"):
            assert a[key] == b[key], (layer, key, a[key], b[key])


BAD = [
    dict(num_heads=6, num_kv_heads=4, head_dim=64),                        # Hq % Hkv
    dict(num_heads=8, num_kv_heads=4, head_dim=64, num_global_kv_heads=3),  # Hq % Hkv(global)
    dict(num_heads=8, num_kv_heads=4, head_dim=0),
    dict(num_heads=8, num_kv_heads=4, head_dim=64, partial_rotary_factor=1.5),
    dict(num_heads=8, num_kv_heads=4, head_dim=64, partial_rotary_factor=float("nan")),
    dict(num_heads=8, num_kv_heads=4, head_dim=64, rope_theta=0.0),
    dict(num_heads=8, num_kv_heads=4, head_dim=64, norm_eps=0.0),
    dict(num_heads=8, num_kv_heads=4, head_dim=64, norm_weight_offset=2),
    dict(num_heads=8, num_kv_heads=4, head_dim=64, attn_logit_softcapping=float("inf")),
    dict(num_heads=8, num_kv_heads=4, head_dim=64, rope_scaling_factor=float("nan")),
]


@pytest.mark.parametrize("kw", BAD)
def test_invalid_configs_rejected(ga, kw):
    with pytest.raises(ga.GemmaAttnError) as e:
        ga.resolve_layer(kw, 0)
    assert e.value.code == ga.GA_ERR_INVALID_ARG


def test_argument_errors_before_any_launch(ga):
    """Every check runs on the host; none of these calls reaches HIP."""
    lib = ga.load()
    good = ga.Config(num_heads=8, num_kv_heads=4, head_dim=256).to_c()
    ref = ctypes.byref
    fake = ctypes.c_void_p(1 << 20)        # 16-byte aligned, never dereferenced
    odd = ctypes.c_void_p((1 << 20) + 2)
    assert lib.gemma_attn_prefill(ref(good), -1, 1, 8, fake, fake, fake, fake, None, None) == ga.GA_ERR_INVALID_ARG
    assert lib.gemma_attn_prefill(ref(good), 0, -1, 8, fake, fake, fake, fake, None, None) == ga.GA_ERR_INVALID_ARG
    assert lib.gemma_attn_prefill(ref(good), 0, 1, 8, None, fake, fake, fake, None, None) == ga.GA_ERR_INVALID_ARG
    assert lib.gemma_attn_prefill(ref(good), 0, 1, 8, odd, fake, fake, fake, None, None) == ga.GA_ERR_INVALID_ARG
    assert lib.gemma_attn_prefill(ref(good), 0, 1, 8, fake, fake, None, fake, None, None) == ga.GA_ERR_INVALID_ARG
    assert lib.gemma_attn_prefill(ref(good), 0, 0, 8, None, None, None, None, None, None) == ga.GA_OK
    unsup = ga.Config(num_heads=8, num_kv_heads=4, head_dim=128).to_c()
    assert lib.gemma_attn_prefill(ref(unsup), 0, 1, 8, fake, fake, fake, fake, None, None) == ga.GA_ERR_UNSUPPORTED
    g32 = ga.Config(num_heads=32, num_kv_heads=1, head_dim=256).to_c()
    assert lib.gemma_attn_prefill(ref(g32), 0, 1, 8, fake, fake, fake, fake, None, None) == ga.GA_ERR_UNSUPPORTED
    pro = ga.Config(num_heads=8, num_kv_heads=4, head_dim=96).to_c()
    assert lib.gemma_qk_prologue(ref(pro), 0, 1, 8, fake, fake, fake, fake, None, None, None, None) == ga.GA_ERR_UNSUPPORTED
    assert lib.gemma_qk_prologue(ref(good), 0, 1, 8, fake, fake, fake, None, None, None, None, None) == ga.GA_ERR_INVALID_ARG
    # keys only needs k; neither q nor k is an error
    assert lib.gemma_qk_prologue(ref(good), 0, 1, 8, None, None, None, None, None, None, None, None) == ga.GA_ERR_INVALID_ARG
    assert lib.gemma_qk_prologue(ref(good), 0, 1, 8, None, fake, None, None, None, None, None, None) == ga.GA_ERR_INVALID_ARG
    # the fused query rotary: width 256, separate values, full-width rotary only
    QR = lib.gemma_attn_prefill_qrope
    assert QR(ref(good), 0, 1, 8, None, fake, fake, None, fake, None, None) == ga.GA_ERR_INVALID_ARG
    assert QR(ref(good), 0, 0, 8, None, None, None, None, None, None, None) == ga.GA_OK
    for bad in (ga.Config(num_heads=4, num_kv_heads=1, head_dim=64),
                ga.Config(num_heads=8, num_kv_heads=1, head_dim=512, k_eq_v=True),
                ga.Config(num_heads=8, num_kv_heads=4, head_dim=256, k_eq_v=True),
                ga.Config(num_heads=8, num_kv_heads=4, head_dim=256, partial_rotary_factor=0.5)):
        assert QR(ref(bad.to_c()), 0, 1, 8, fake, fake, fake, None, fake, None, None) == ga.GA_ERR_UNSUPPORTED
    keqv = ga.Config(num_heads=8, num_kv_heads=1, head_dim=512, k_eq_v=True).to_c()
    need = lib.gemma_attn_decode_workspace_size(ref(keqv), 0, 4, 1000)
    assert need > 0
    assert lib.gemma_attn_decode(ref(keqv), 0, 4, 1000, fake, fake, None, fake, fake, None, fake, need - 1,
                                 None) == ga.GA_ERR_WORKSPACE
    assert lib.gemma_attn_decode(ref(keqv), 0, 4, 1000, fake, fake, None, fake, fake, None, None, need,
                                 None) == ga.GA_ERR_WORKSPACE
    assert lib.gemma_attn_decode(ref(good), 0, 4, 1000, fake, fake, None, fake, fake, None, fake, 1 << 30,
                                 None) == ga.GA_ERR_INVALID_ARG   # v_cache missing without keys-as-values
    assert lib.gemma_attn_decode(ref(keqv), 0, 4, 0, fake, fake, None, fake, fake, None, fake, need,
                                 None) == ga.GA_ERR_INVALID_ARG
    assert lib.gemma_attn_decode_workspace_size(ref(keqv), 0, 4, 0) == 0
    assert ga.load().gemma_attn_strerror(ga.GA_ERR_WORKSPACE).decode().startswith("decode workspace")


def _decode_ws_bytes(B, q_len, Hq, D, n_wg):
    """The documented layout: int64 prefix [B+1], int32 lo [B], then fp32 o, m, l for n_wg + B slots."""
    up = lambda x: (x + 255) // 256 * 256
    rows = (n_wg + B) * q_len * Hq
    return up((B + 1) * 8) + up(B * 4 + 4) + up(rows * D * 4) + 2 * up(rows * 4)


@pytest.mark.parametrize("W,max_ctx,B", [(1024, 65536, 64), (0, 65536, 64), (0, 100, 1), (4096, 3000, 2), (0, 1, 1)])
def test_decode_workspace_covers_every_split(ga, W, max_ctx, B):
    kw = dict(num_heads=16, num_kv_heads=8, head_dim=256, sliding_window=W, sliding_window_pattern=0)
    need = ga.decode_workspace_size(kw, 0, B, max_ctx)
    # 8 KV heads x 1 column block = 8 grid rows; D = 256 with separate K and V: a 64 KB ring, two
    # workgroups per CU -> 512 // 8 = 64 per row, kept within [line/16384, line/256] keys
    span = min(W, max_ctx) if W else max_ctx
    line = B * span
    n_wg = max(1, min(max(512 // 8, -(-line // 16384)), -(-line // 256)))
    if B * 8 >= 512 and span <= 8192:
        n_wg = B                                        # one workgroup per sequence and row
    assert need == _decode_ws_bytes(B, 1, 16, 256, n_wg)


def test_multi_token_entry_points_reject_bad_arguments(ga):
    lib, ref, fake = ga.load(), ctypes.byref, ctypes.c_void_p(1 << 20)
    keqv = ga.Config(num_heads=8, num_kv_heads=1, head_dim=512, k_eq_v=True).to_c()
    good = ga.Config(num_heads=8, num_kv_heads=4, head_dim=256).to_c()
    need = lib.gemma_attn_decode_multi_workspace_size(ref(keqv), 0, 4, 5, 1000)
    assert need > lib.gemma_attn_decode_workspace_size(ref(keqv), 0, 4, 1000) > 0
    assert lib.gemma_attn_decode_multi_workspace_size(ref(keqv), 0, 4, 1, 1000) == \
        lib.gemma_attn_decode_workspace_size(ref(keqv), 0, 4, 1000)
    for q_len, max_ctx in [(0, 1000), (1001, 1000), (-1, 1000), (1, 0)]:
        assert lib.gemma_attn_decode_multi_workspace_size(ref(keqv), 0, 4, q_len, max_ctx) == 0
        assert lib.gemma_attn_decode_multi(ref(keqv), 0, 4, q_len, max_ctx, fake, fake, None, fake, None, fake, None,
                                           fake, 1 << 30, None) == ga.GA_ERR_INVALID_ARG
    assert lib.gemma_attn_decode_multi(ref(keqv), 0, 4, 5, 1000, fake, fake, None, fake, None, fake, None, fake,
                                       need - 1, None) == ga.GA_ERR_WORKSPACE
    assert lib.gemma_attn_decode_multi(ref(good), 0, 4, 5, 1000, fake, fake, None, fake, None, fake, None, fake,
                                       1 << 30, None) == ga.GA_ERR_INVALID_ARG   # v_cache missing
    assert lib.gemma_attn_decode_multi(ref(keqv), 0, 4, 5, 1000, fake, fake, None, None, None, fake, None, fake,
                                       1 << 30, None) == ga.GA_ERR_INVALID_ARG   # ctx_len missing
    # too many 16-column blocks for the grid
    g16 = ga.Config(num_heads=16 * 4096, num_kv_heads=4096, head_dim=64).to_c()
    assert lib.gemma_attn_decode_multi(ref(g16), 0, 1, 300, 1000, fake, fake, fake, fake, None, fake, None, fake,
                                       1 << 40, None) == ga.GA_ERR_UNSUPPORTED
    # prologue with cache append
    P = lib.gemma_qk_prologue_cache
    assert P(ref(good), 0, 2, 4, 3, fake, fake, fake, fake, fake, fake, None, None, fake, None) == ga.GA_ERR_INVALID_ARG
    assert P(ref(good), 0, 2, 4, 16, fake, fake, None, fake, fake, fake, None, None, fake, None) == ga.GA_ERR_INVALID_ARG
    assert P(ref(good), 0, 2, 4, 16, fake, fake, fake, fake, fake, fake, None, None, None, None) == ga.GA_ERR_INVALID_ARG
    assert P(ref(good), 0, 0, 4, 16, None, None, None, None, None, None, None, None, None, None) == ga.GA_OK
    odd = ga.Config(num_heads=8, num_kv_heads=4, head_dim=96).to_c()
    assert P(ref(odd), 0, 2, 4, 16, fake, fake, fake, fake, fake, fake, None, None, fake, None) == ga.GA_ERR_UNSUPPORTED
    # keys-as-values: no value tensors needed
    assert P(ref(keqv), 0, 0, 4, 16, fake, fake, None, fake, fake, None, None, None, fake, None) == ga.GA_OK


@pytest.mark.parametrize("W,max_ctx,B,q_len", [(1024, 65536, 8, 16), (0, 4096, 2, 7), (100, 3000, 3, 64),
                                               (0, 64, 1, 64)])
def test_decode_multi_workspace_covers_every_split(ga, W, max_ctx, B, q_len):
    kw = dict(num_heads=16, num_kv_heads=8, head_dim=256, sliding_window=W, sliding_window_pattern=0)
    need = ga.decode_multi_workspace_size(kw, 0, B, q_len, max_ctx)
    span = min(W + q_len - 1, max_ctx) if W else max_ctx
    rows = 8 * -(-2 * q_len // 16)                      # KV heads x 16-column blocks (g = 2)
    line = B * span
    n_wg = max(1, min(max(512 // rows, -(-line // 16384)), -(-line // 256)))
    if B * rows >= 512 and span <= 8192:
        n_wg = B
    assert need == _decode_ws_bytes(B, q_len, 16, 256, n_wg)


def test_int8_entry_points_reject_bad_arguments(ga):
    lib, ref, fake = ga.load(), ctypes.byref, ctypes.c_void_p(1 << 20)
    good = ga.Config(num_heads=8, num_kv_heads=4, head_dim=256).to_c()
    keqv = ga.Config(num_heads=8, num_kv_heads=1, head_dim=512, k_eq_v=True).to_c()
    need = lib.gemma_attn_decode_multi_workspace_size(ref(good), 0, 2, 3, 100)
    D8 = lib.gemma_attn_decode_int8
    assert D8(ref(good), 0, 2, 3, 100, fake, fake, None, fake, fake, fake, None, fake, None, fake, need,
              None) == ga.GA_ERR_INVALID_ARG                                  # key scales missing
    assert D8(ref(good), 0, 2, 3, 100, fake, fake, fake, fake, None, fake, None, fake, None, fake, need,
              None) == ga.GA_ERR_INVALID_ARG                                  # value scales missing
    assert D8(ref(good), 0, 2, 3, 100, fake, fake, fake, fake, fake, fake, None, fake, None, fake, need - 1,
              None) == ga.GA_ERR_WORKSPACE
    assert D8(ref(keqv), 0, 0, 3, 100, None, None, fake, None, None, None, None, None, None, None, 0, None) == ga.GA_OK
    P8 = lib.gemma_qk_prologue_cache_int8
    assert P8(ref(good), 0, 2, 4, 16, fake, fake, fake, fake, fake, None, fake, fake, None, None, fake,
              None) == ga.GA_ERR_INVALID_ARG                                  # key scales missing
    assert P8(ref(good), 0, 2, 4, 16, fake, fake, None, fake, fake, fake, fake, fake, None, None, fake,
              None) == ga.GA_ERR_INVALID_ARG                                  # values missing
    assert P8(ref(good), 0, 2, 17, 16, fake, fake, fake, fake, fake, fake, fake, fake, None, None, fake,
              None) == ga.GA_ERR_INVALID_ARG                                  # q_len > max_ctx
    Q = lib.gemma_kv_quantize_int8
    assert Q(2, 4, 1, 96, 16, fake, None, fake, fake, None) == ga.GA_ERR_UNSUPPORTED
    assert Q(2, 4, 0, 64, 16, fake, None, fake, fake, None) == ga.GA_ERR_INVALID_ARG
    assert Q(2, 4, 1, 64, 16, fake, None, fake, None, None) == ga.GA_ERR_INVALID_ARG
    assert Q(0, 4, 1, 64, 16, None, None, None, None, None) == ga.GA_OK


@pytest.mark.parametrize("q_len", [1, 2, 3, 4, 5, 16])
def test_decode_workspace_follows_the_kernel_choice(ga, q_len):
    """Keys as values at head width 512 (an MQA global layer, g = 16): with 48 or more query columns the
    32-key tile kernel runs, 64 columns per workgroup and two workgroups per CU; otherwise the split
    kernel, 16-column blocks and four workgroups per CU (a 32 KB ring).  The workspace holds one partial
    per (workgroup + sequence, token, head) of the chosen plan."""
    kw = dict(num_heads=16, num_kv_heads=1, head_dim=512, k_eq_v=True, sliding_window=0, sliding_window_pattern=1)
    B, max_ctx = 64, 65536
    need = ga.decode_multi_workspace_size(kw, 0, B, q_len, max_ctx)
    cols = 16 * q_len
    if cols >= 48:
        rows, per_cu = -(-cols // 64), 2
    else:
        rows, per_cu = -(-cols // 16), 4
    line = B * max_ctx
    n_wg = max(1, min(max(256 * per_cu // rows, -(-line // 16384)), -(-line // 256)))
    assert need == _decode_ws_bytes(B, q_len, 16, 512, n_wg)


# ----------------------------------------------------------------------------- binding: output shapes
_G4 = dict(num_heads=16, num_kv_heads=8, num_global_kv_heads=1, head_dim=256, global_head_dim=512,
           sliding_window=64, sliding_window_pattern=6, partial_rotary_factor=0.25, k_eq_v=True)


def _bad_output_calls(ga):
    """(name, call) pairs whose one wrongly shaped output must be refused.

    The tensors live on the CPU: the binding checks every shape before it
    takes a device pointer, so a refusal here happens before any launch."""
    import torch

    bf, B, S, L, Smax = torch.bfloat16, 2, 5, 3, 40
    e = lambda *s, dt=bf: torch.empty(s, dtype=dt)            # noqa: E731
    i32 = torch.int32
    q, k = e(B, S, 16, 256), e(B, S, 8, 256)
    qd, kc = e(B, 16, 512), e(B, Smax, 1, 512)
    qm = e(B, L, 16, 512)
    ctx = e(B, dt=i32)
    codes, scales = e(B, Smax, 1, 512, dt=torch.int8), e(B, 1, Smax, dt=torch.float32)
    kcl, vcl = e(B, Smax, 8, 256), e(B, Smax, 8, 256)
    return [
        ("prologue q_out", lambda: ga.qk_prologue(_G4, 0, q, k, q_out=e(B, S, 16, 128))),
        ("prologue k_out", lambda: ga.qk_prologue(_G4, 0, q, k, k_out=e(B, S - 1, 8, 256))),
        ("prefill out", lambda: ga.attn_prefill(_G4, 0, q, k, k, out=e(B, S, 8, 256))),
        ("prefill lse", lambda: ga.attn_prefill(_G4, 0, q, k, k, lse=e(B, 16, S - 1, dt=torch.float32))),
        ("decode out", lambda: ga.attn_decode(_G4, 5, qd, kc, None, ctx, out=e(B, 16, 256))),
        ("decode lse", lambda: ga.attn_decode(_G4, 5, qd, kc, None, ctx, lse=e(B, 8, dt=torch.float32))),
        ("decode_multi out", lambda: ga.attn_decode_multi(_G4, 5, qm, kc, None, ctx, out=e(B, L - 1, 16, 512))),
        ("decode_multi lse", lambda: ga.attn_decode_multi(_G4, 5, qm, kc, None, ctx,
                                                          lse=e(B, 16, L + 1, dt=torch.float32))),
        ("decode_multi kv_start", lambda: ga.attn_decode_multi(_G4, 5, qm, kc, None, ctx, kv_start=e(B + 1, dt=i32))),
        ("decode_int8 out", lambda: ga.attn_decode_int8(_G4, 5, qm, codes, scales, None, None, ctx,
                                                        out=e(B, L, 16, 256))),
        ("decode_int8 lse", lambda: ga.attn_decode_int8(_G4, 5, qm, codes, scales, None, None, ctx,
                                                        lse=e(B, 16, dt=torch.float32))),
        ("prologue_cache q_out", lambda: ga.qk_prologue_cache(_G4, 0, e(B, L, 16, 256), e(B, L, 8, 256),
                                                              e(B, L, 8, 256), kcl, vcl, ctx,
                                                              q_out=e(B, L, 8, 256))),
        ("prologue_cache_int8 q_out", lambda: ga.qk_prologue_cache_int8(_G4, 5, qm, e(B, L, 1, 512), None, codes,
                                                                        scales, None, None, ctx,
                                                                        q_out=e(B, L, 16, 511))),
    ]


def test_binding_refuses_wrongly_shaped_outputs(ga):
    for name, call in _bad_output_calls(ga):
        with pytest.raises(ValueError, match="has shape"):
            call()


def test_noalloc_refuses_shapes_beyond_its_scratch(ga):
    """64 sequences of up to 65536 keys at head width 512 with 16 new tokens need
    about 160 MiB of split partials, more than the 80 MiB scratch array: refused
    on the host with its own error, before anything is enqueued (the pointers
    here are never dereferenced)."""
    cfg = ga.Config(**_G4).to_c()
    fake = ctypes.c_void_p(0x10000)
    lib = ga.load()
    need = lib.gemma_attn_decode_multi_workspace_size(ctypes.byref(cfg), 5, 64, 16, 65536)
    assert need > 80 << 20
    rc = lib.gemma_attn_decode_multi_noalloc(ctypes.byref(cfg), 5, 64, 16, 65536, fake, fake, None, fake, None, fake,
                                             None, None)
    assert rc == ga.GA_ERR_SCRATCH_LIMIT
    assert b"scratch" in lib.gemma_attn_strerror(rc)
    # argument errors still come first
    assert lib.gemma_attn_decode_multi_noalloc(ctypes.byref(cfg), 5, 64, 16, 65536, None, fake, None, fake, None, fake,
                                               None, None) == ga.GA_ERR_INVALID_ARG
