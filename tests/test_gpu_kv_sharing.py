"""Cross-layer KV sharing on the GPU path.

The "google-gemma-4" atlas summary says KV caches are shared across layers
(20/35 and 18/42 of the layers on the small models).  The library keeps no
per-layer state: a layer that shares reads the owning layer's cache by being
handed the same pointers, and the decode kernels only read the caches.  These
tests append once (owning layer), decode several layers against the one
cache, compare each with the oracle, and check the cache bits are unchanged.
"""
import numpy as np
import pytest

from oracle import gemma_ref as R
from synth import bf16_bits_to_f64, normal_bf16, norm_weight
from tests.gpu_util import assert_close, from_dev_bf16_bits, from_dev_f64, to_dev, to_dev_bf16
from tests.test_gpu_parity import GEMMA4

pytestmark = pytest.mark.gpu

# Gemma-4-shaped: layers 0-4 local (16/8 heads, D256), layer 5 global K=V (D512)
SHARED = GEMMA4 | dict(sliding_window=64)


@pytest.mark.parametrize("owner,sharers,int8", [(0, (1, 3), False), (5, (11,), False), (0, (2,), True)])
def test_layers_share_one_cache(gpu, owner, sharers, int8):
    ga = gpu
    import torch

    cfg = R.GemmaAttnConfig(**SHARED)
    L = R.resolve_layer(cfg, owner)
    for s_ in sharers:                                  # only layers of the same geometry can share
        Ls = R.resolve_layer(cfg, s_)
        assert (Ls["num_kv_heads"], Ls["head_dim"], Ls["k_eq_v"]) == (L["num_kv_heads"], L["head_dim"], L["k_eq_v"])
    B, S, Smax, Lq = 2, 150, 200, 3
    D, Hkv, Hq = L["head_dim"], L["num_kv_heads"], cfg.num_heads
    print(f"[kv_sharing] owner={owner} sharers={sharers} int8={int8}", flush=True)
    k = normal_bf16(4000 + owner, (B, S, Hkv, D))
    v = normal_bf16(4001 + owner, (B, S, Hkv, D))
    kn = norm_weight(4002, D)
    ctx = np.array([S, S - 40], dtype=np.int32)
    kvl = not L["k_eq_v"]
    # the owning layer appends its keys and values for positions 0..ctx-1 (its queries are discarded here)
    q0 = to_dev_bf16(normal_bf16(4003, (B, S, Hq, D)))
    ctx_full = to_dev(np.full(B, S, dtype=np.int32))
    if int8:
        kc = torch.zeros((B, Smax, Hkv, D), dtype=torch.int8, device="cuda")
        ks = torch.zeros((B, Hkv, Smax), dtype=torch.float32, device="cuda")
        vc, vs = torch.zeros_like(kc), torch.zeros_like(ks)
        ga.qk_prologue_cache_int8(SHARED, owner, q0, to_dev_bf16(k), to_dev_bf16(v), kc, ks, vc if kvl else None,
                                  vs if kvl else None, ctx_full, k_norm_w=to_dev(kn))
        before = [t.cpu().numpy().copy() for t in (kc, ks, vc, vs)]
    else:
        kc = torch.zeros((B, Smax, Hkv, D), dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        ga.qk_prologue_cache(SHARED, owner, q0, to_dev_bf16(k), to_dev_bf16(v), kc, vc if kvl else None, ctx_full,
                             k_norm_w=to_dev(kn))
        before = [from_dev_bf16_bits(t).copy() for t in (kc, vc)]
    torch.cuda.synchronize()
    for layer in (owner,) + tuple(sharers):
        q = normal_bf16(4100 + layer, (B, Lq, Hq, D), scale=2.0)
        if int8:
            out = ga.attn_decode_int8(SHARED, layer, to_dev_bf16(q), kc, ks, vc, vs, to_dev(ctx))
            torch.cuda.synchronize()
            kk = (kc.cpu().numpy(), ks.cpu().numpy(), vc.cpu().numpy(), vs.cpu().numpy())
            ro, _ = R.decode_int8(cfg, layer, bf16_bits_to_f64(q), *kk, ctx)
        else:
            out = ga.attn_decode_multi(SHARED, layer, to_dev_bf16(q), kc, vc if kvl else None, to_dev(ctx))
            torch.cuda.synchronize()
            ro, _ = R.decode_multi(cfg, layer, bf16_bits_to_f64(q), bf16_bits_to_f64(from_dev_bf16_bits(kc)),
                                   bf16_bits_to_f64(from_dev_bf16_bits(vc)), ctx)
        assert_close(from_dev_f64(out), ro, what=f"layer {layer}")
    after = ([t.cpu().numpy() for t in (kc, ks, vc, vs)] if int8 else [from_dev_bf16_bits(t) for t in (kc, vc)])
    for a, b in zip(before, after):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
