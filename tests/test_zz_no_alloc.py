"""The allocation-free decode entry point through the C ABI (GPU).

gemma_attn_decode_multi_noalloc takes its split-KV workspace from the
library's fixed device array instead of an argument.  Its outputs and lse
must equal those of gemma_attn_decode_multi (with an allocated workspace)
bit for bit, call after call: the array keeps the previous call's contents,
so a larger call, then a smaller one, then the larger one again must each
still match.  The outputs are also held to the oracle at the attention
tolerance, and every cache row a sequence may not read is NaN.
"""
import numpy as np
import pytest

from oracle import gemma_ref as R
from synth import BF16_NAN, bf16_bits_to_f64, ctx_lengths, normal_bf16
from tests.gpu_util import assert_close, from_dev_bf16_bits, from_dev_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

G4 = dict(num_heads=16, num_kv_heads=8, num_global_kv_heads=1, head_dim=256, global_head_dim=512,
          sliding_window=1024, sliding_window_pattern=6, rope_theta=1e6, rope_local_theta=1e4,
          partial_rotary_factor=0.25, k_eq_v=True)
G2 = dict(num_heads=8, num_kv_heads=4, head_dim=256, sliding_window=300, sliding_window_pattern=2,
          attn_logit_softcapping=50.0, query_pre_attn_scalar=256.0)

# (name, config, layer, batch, cache rows, new tokens): a large call (global layer, balanced
# key line, 32-key tile kernel), then a smaller one (local layer, fewer sequences and rows)
CALLS = [("gemma4_global_q4", G4, 5, 8, 3000, 4), ("gemma2_local_q1", G2, 0, 3, 700, 1),
         ("gemma4_global_q4_again", G4, 5, 8, 3000, 4), ("gemma4_local_q2", G4, 0, 2, 1500, 2)]


def _inputs(kw, layer, B, Smax, q_len, seed):
    cfg = R.GemmaAttnConfig(**kw)
    L = R.resolve_layer(cfg, layer)
    D, Hkv, Hq, W = L["head_dim"], L["num_kv_heads"], cfg.num_heads, L["window"]
    ctx = ctx_lengths(seed, B, 1, Smax)
    ctx[0], ctx[-1] = Smax, max(1, q_len - 1)
    kc = normal_bf16(seed + 1, (B, Smax, Hkv, D))
    vc = normal_bf16(seed + 2, (B, Smax, Hkv, D))
    for b in range(B):
        lo = max(0, int(ctx[b]) - (W + q_len - 1)) if W else 0
        for c in (kc, vc):
            c[b, :lo] = BF16_NAN
            c[b, ctx[b]:] = BF16_NAN
    q = normal_bf16(seed + 3, (B, q_len, Hq, D), scale=2.0)
    return cfg, L, ctx, q, kc, vc


def test_noalloc_matches_decode_multi_call_after_call(gpu):
    ga = gpu
    import torch

    for i, (name, kw, layer, B, Smax, q_len) in enumerate(CALLS):
        seed = 9100 + 10 * (i % 2)
        cfg, L, ctx, q, kc, vc = _inputs(kw, layer, B, Smax, q_len, seed)
        print(f"[noalloc] {name}: B={B} Smax={Smax} q_len={q_len} ctx={ctx.tolist()}", flush=True)
        qd, kd, cd = to_dev_bf16(q), to_dev_bf16(kc), to_dev(ctx)
        vd = None if L["k_eq_v"] else to_dev_bf16(vc)
        ref, ref_l = ga.attn_decode_multi(kw, layer, qd, kd, vd, cd, want_lse=True)
        out = torch.full_like(qd, float("nan"))
        lse = torch.full((B, cfg.num_heads, q_len), float("nan"), dtype=torch.float32, device="cuda")
        ga.attn_decode_multi_noalloc(kw, layer, qd, kd, vd, cd, out, lse)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev_bf16_bits(out), from_dev_bf16_bits(ref)), name
        assert np.array_equal(lse.cpu().numpy().view(np.uint32), ref_l.cpu().numpy().view(np.uint32)), name
        ro, rl = R.decode_multi(cfg, layer, bf16_bits_to_f64(q), bf16_bits_to_f64(kc), bf16_bits_to_f64(vc), ctx)
        assert_close(from_dev_f64(out), ro, what=name)
        seen = np.isfinite(rl)
        assert np.array_equal(np.isfinite(from_dev_f64(lse)), seen), name
        assert_close(from_dev_f64(lse)[seen], rl[seen], what=name + " lse")
