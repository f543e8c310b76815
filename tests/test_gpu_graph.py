"""Decode inside a captured HIP graph (GPU).

Callers that cannot allocate device memory during a step (graph capture,
tight serving loops) take gemma_attn_decode_multi_noalloc; callers that
allocate once take gemma_attn_decode_multi with a workspace allocated before
capture.  Both enqueue only kernels on the caller's stream (no memset, no
allocation, no host synchronisation), so a step captured once can be replayed.
Every replay must equal the eager call on the inputs the captured tensors
hold at replay time, bit for bit: three replays, with other eager decode work
and host synchronisations between them, and with new query values and new
context lengths copied into the captured inputs before the later replays.
"""
import numpy as np
import pytest

from synth import BF16_NAN, ctx_lengths, normal_bf16
from tests.gpu_util import from_dev_bf16_bits, from_dev_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

G4 = dict(num_heads=16, num_kv_heads=8, num_global_kv_heads=1, head_dim=256, global_head_dim=512,
          sliding_window=1024, sliding_window_pattern=6, rope_theta=1e6, rope_local_theta=1e4,
          partial_rotary_factor=0.25, k_eq_v=True)

# (layer, batch, cache rows, new tokens): the global layer's balanced key line
# with the tile kernel (4 tokens) and the split kernel (1 token), and the local
# layer with one workgroup per sequence (72 sequences x 8 KV heads).
CASES = [(5, 8, 3000, 4), (5, 8, 3000, 1), (0, 72, 1200, 1)]


def _caches(layer, B, Smax, seed):
    import decoder_attention_amd as ga

    L = ga.resolve_layer(G4, layer)
    D, Hkv = L["head_dim"], L["num_kv_heads"]
    kc = normal_bf16(seed + 1, (B, Smax, Hkv, D))
    vc = normal_bf16(seed + 2, (B, Smax, Hkv, D))
    kc[:, Smax - 7:] = BF16_NAN     # rows no context below reaches
    vc[:, Smax - 7:] = BF16_NAN
    return L, to_dev_bf16(kc), (None if L["k_eq_v"] else to_dev_bf16(vc))


@pytest.mark.parametrize("noalloc", [True, False], ids=["noalloc", "workspace"])
@pytest.mark.parametrize("layer,B,Smax,q_len", CASES, ids=[f"L{c[0]}-B{c[1]}-q{c[3]}" for c in CASES])
def test_decode_graph_replays_equal_eager(gpu, layer, B, Smax, q_len, noalloc):
    ga = gpu
    import torch

    seed = 9700 + layer + q_len
    L, kd, vd = _caches(layer, B, Smax, seed)
    D, Hq = L["head_dim"], G4["num_heads"]
    print(f"[graph] layer {layer} B={B} Smax={Smax} q_len={q_len} noalloc={noalloc}", flush=True)
    inputs = [(normal_bf16(seed + 10 + i, (B, q_len, Hq, D), scale=2.0),
               np.minimum(ctx_lengths(seed + 20 + i, B, 1, Smax - 7), Smax - 7).astype(np.int32)) for i in range(3)]
    q_cap = to_dev_bf16(inputs[0][0])
    c_cap = to_dev(inputs[0][1])
    out_cap = torch.empty_like(q_cap)
    lse_cap = torch.empty((B, Hq, q_len), dtype=torch.float32, device="cuda")
    ws = torch.empty(ga.decode_multi_workspace_size(G4, layer, B, q_len, Smax), dtype=torch.uint8, device="cuda")

    def call(q, c, out, lse, stream=None):
        if noalloc:
            ga.attn_decode_multi_noalloc(G4, layer, q, kd, vd, c, out, lse=lse, stream=stream)
        else:
            ga.attn_decode_multi(G4, layer, q, kd, vd, c, out=out, lse=lse, workspace=ws, stream=stream)

    # warm up on a side stream, then capture one call
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(q_cap, c_cap, out_cap, lse_cap)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(q_cap, c_cap, out_cap, lse_cap)
    torch.cuda.synchronize()

    # other eager decode work between replays (it also rewrites the library's scratch array)
    other_q = to_dev_bf16(normal_bf16(seed + 30, (B, q_len, Hq, D)))
    other_c = to_dev(np.full(B, Smax // 2, dtype=np.int32))
    for i, (qh, ch) in enumerate(inputs):
        if i > 0:
            q_cap.copy_(to_dev_bf16(qh))
            c_cap.copy_(to_dev(ch))
        graph.replay()
        torch.cuda.synchronize()
        got, got_l = from_dev_bf16_bits(out_cap).copy(), from_dev_f64(lse_cap).copy()
        ref = torch.empty_like(q_cap)
        ref_l = torch.empty_like(lse_cap)
        call(to_dev_bf16(qh), to_dev(ch), ref, ref_l)
        torch.cuda.synchronize()
        assert np.array_equal(got, from_dev_bf16_bits(ref)), f"replay {i}: outputs differ from the eager call"
        assert np.array_equal(got_l, from_dev_f64(ref_l), equal_nan=True), f"replay {i}: lse differs"
        assert np.isfinite(from_dev_f64(ref)).all(), f"replay {i}: a NaN row was read"
        o2 = torch.empty_like(other_q)
        call(other_q, other_c, o2, None)
        torch.cuda.synchronize()
