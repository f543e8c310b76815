"""GPU parity at the benchmark's own sizes and launches, on every output.

The inputs are the benchmark's seeded tensors (bench.py builds them, the
same calls launch the kernels), so every launch shape timed there is also
checked here:
  * prefill: the Gemma-2-2B-shaped pair (B2 S8192), the Gemma-3-1B-shaped
    local (window 512) and global layers (B4 S16384, QK-norm 1+w) and the
    Gemma-4-12B-shaped global layer (B1 S32768, D512, keys as values);
  * decode: the Gemma-4-12B-shaped step over 64 ragged contexts of up to
    65536 rows (local layer window 1024, global layer D512), one new token,
    four new tokens, and the int8 cache.
The pair's timed form (keys-only prologue, query rotary in the prefill
kernel) must equal prologue + prefill bit for bit.
The oracle recomputes every output: the prologue of the whole q and k
tensors, then the attention of every query row (prefill) or of every
sequence (decode).  Outputs and lse are held to the attention tolerance
(max-abs 2e-2, mean-abs 2e-3), prologue outputs to one bf16 ulp, int8 codes
and scales bit for bit.  Decode caches are NaN outside the rows a sequence
may read, so a stray read shows as a non-finite output anywhere in the batch.
The oracle runs in a pool of host threads with the BLAS library held to one
thread per worker.
"""
import os

import numpy as np
import pytest

import bench
from oracle import gemma_ref as R
from synth import bf16_bits_to_f64, normal_bf16_row, seed_for
from tests.gpu_util import assert_close, assert_within_one_ulp, from_dev_f64, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

PREFILL = [(f"{name}_layer{layer}", name, layer)
           for name, (_, _, layers, _, _, _) in bench.PREFILL_WORKLOADS.items() for layer in layers]


def _one_blas_thread():
    from threadpoolctl import threadpool_limits

    return threadpool_limits(limits=1)


def _threads():
    return min(16, len(os.sched_getaffinity(0)))


def _chunks(S):
    n = _threads()
    step = max(1, -(-S // n))
    return [(s0, min(S, s0 + step)) for s0 in range(0, S, step)]


def _prologue_rows(cfg, layer, q, k, qw, kw):
    """The oracle's prologue of [B,S,H,D] tensors, in position chunks on host
    threads (a chunk starting at s0 takes positions s0, s0 + 1, ...)."""
    from concurrent.futures import ThreadPoolExecutor

    B, S = q.shape[0], q.shape[1]
    rq = np.empty(q.shape)
    rk = np.empty(k.shape)

    def run(c):
        s0, s1 = c
        a, b = R.prologue(cfg, layer, bf16_bits_to_f64(q[:, s0:s1]), bf16_bits_to_f64(k[:, s0:s1]), qw, kw,
                          pos0=[s0] * B)
        rq[:, s0:s1] = a
        rk[:, s0:s1] = b

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(run, _chunks(S)))
    return rq, rk


def _rowwise(fn, x, *more):
    """fn applied to position chunks of [B,S,...] arrays on host threads (fn is row-wise)."""
    from concurrent.futures import ThreadPoolExecutor

    chunks = _chunks(x.shape[1])
    with ThreadPoolExecutor(_threads()) as ex:
        return list(ex.map(lambda c: fn(x[:, c[0]:c[1]], *(m[:, c[0]:c[1]] for m in more)), chunks)), chunks


def _round_bf16(x):
    parts, chunks = _rowwise(R.round_bf16, x)
    out = np.empty(x.shape)
    for (s0, s1), p in zip(chunks, parts):
        out[:, s0:s1] = p
    return out


def _within_one_ulp(got, ref, what):
    _rowwise(lambda a, b: assert_within_one_ulp(a, b, what=what), got, ref)


@pytest.mark.parametrize("case,workload,layer", PREFILL, ids=[p[0] for p in PREFILL])
def test_prefill_full_size_every_row(gpu, case, workload, layer):
    ga = gpu
    import torch

    cfg_id, kw, _, B, S, norm = bench.PREFILL_WORKLOADS[workload]
    cfg = R.GemmaAttnConfig(**kw)
    L = R.resolve_layer(cfg, layer)
    W = L["window"]
    print(f"[fullsize] {case}: B={B} S={S} D={L['head_dim']} window={W}", flush=True)
    h = bench.layer_inputs(cfg_id, kw, layer, B, S, norm)
    t = bench.layer_tensors(cfg_id, kw, layer, B, S, norm, host=h)
    bench.run_layer_step(ga, kw, layer, t)                 # prologue, then prefill
    out2, lse = ga.attn_prefill(kw, layer, t["qt"], t["kt"], t["v"], want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), t["out"].view(torch.int16)), "lse request changed the output"
    del out2
    if workload == "gemma2_pair":
        # the timed form of this workload: keys-only prologue, query rotary in the prefill kernel
        _, k_only = ga.qk_prologue(kw, layer, None, t["k"])
        fused = ga.attn_prefill_qrope(kw, layer, t["q"], k_only, t["v"])
        torch.cuda.synchronize()
        assert torch.equal(k_only.view(torch.int16), t["kt"].view(torch.int16)), "keys-only prologue differs"
        assert torch.equal(fused.view(torch.int16), t["out"].view(torch.int16)), "fused form differs"
        del k_only, fused
    got_q = from_dev_f64(t["qt"])
    got_k = from_dev_f64(t["kt"])
    got_o = from_dev_f64(t["out"])
    got_l = from_dev_f64(lse)
    del t, lse
    torch.cuda.empty_cache()

    # oracle: the prologue of the whole tensors (positions 0..S-1), then every row's attention
    ref_q, ref_k = _prologue_rows(cfg, layer, h["q"], h["k"], h["qw"], h["kw"])
    _within_one_ulp(got_q, ref_q, what=case + " q")
    _within_one_ulp(got_k, ref_k, what=case + " k")
    del got_q, got_k
    v = None if L["k_eq_v"] else bf16_bits_to_f64(h["v"])
    del h
    # the processed q and k cross the library boundary as bf16
    rq, rk = _round_bf16(ref_q), _round_bf16(ref_k)
    del ref_q, ref_k
    block = 64 if L["head_dim"] > 256 or S > 16384 else 256     # bounds the oracle's score blocks
    with _one_blas_thread():
        ro, rl = R.prefill(cfg, layer, rq, rk, v, block_rows=block, threads=_threads())
    del rq, rk, v
    mx, mn = assert_close(got_o, ro, what=case)
    assert_close(got_l, rl, what=case + " lse")
    print(f"[fullsize] {case}: {got_o.shape[0] * got_o.shape[1] * got_o.shape[2]} rows, max-abs {mx:.2e} "
          f"mean-abs {mn:.2e}", flush=True)


class _Spans:
    """Read-only stand-in for a [B', Smax, Hkv, D] cache of which only the
    rows [lo_b, hi_b) of each sequence exist (the rows the decode step may
    read); reading any other row fails."""

    def __init__(self, spans, rows):
        self.spans, self.rows = spans, rows

    def __getitem__(self, idx):
        b, s, h, d = idx
        lo, hi = self.spans[b]
        assert s.step is None and lo <= s.start <= s.stop <= hi, (b, s, (lo, hi))
        return self.rows[b][s.start - lo:s.stop - lo, h, d]


def _decode_oracle_caches(layer, ctx, sel):
    """The selected sequences' cache rows, drawn on the host from the same
    seeded streams that fill the device caches: (spans, bf16 bits per tensor)."""
    from concurrent.futures import ThreadPoolExecutor

    L = R.resolve_layer(R.GemmaAttnConfig(**bench.GEMMA4_12B), layer)
    Hkv, D, W = L["num_kv_heads"], L["head_dim"], L["window"]
    spans = [bench.decode_span(ctx[b], W) for b in sel]
    bits = {}
    for tensor in (("k",) if L["k_eq_v"] else ("k", "v")):
        seed = seed_for(5, layer, tensor)
        with ThreadPoolExecutor(min(16, len(os.sched_getaffinity(0)))) as ex:
            bits[tensor] = list(ex.map(lambda a: normal_bf16_row(seed, int(a[0]), (a[1][1] - a[1][0], Hkv, D)),
                                       zip(sel, spans)))
    return spans, bits


@pytest.mark.parametrize("layer", [0, 5], ids=["local_w1024", "global_keqv_d512"])
def test_decode_full_size_every_sequence(gpu, layer):
    ga = gpu
    import torch

    kw = bench.GEMMA4_12B
    cfg = R.GemmaAttnConfig(**kw)
    L = R.resolve_layer(cfg, layer)
    B, Smax, D, Lq = bench.DECODE_B, bench.DECODE_SMAX, L["head_dim"], bench.DECODE_MULTI
    ctx = bench.decode_contexts()
    sel = list(range(B))
    print(f"[fullsize] decode layer {layer}: B={B} Smax={Smax} D={D} ctx {ctx.min()}..{ctx.max()}", flush=True)

    # the timed launches, in the timed configuration
    kc, vc = bench.decode_caches(ga, layer, ctx)
    ctx_d = torch.from_numpy(ctx).cuda()
    q_bits = bench.decode_query(layer)
    q = to_dev(q_bits.view(np.int16)).view(torch.bfloat16)
    qt = torch.empty_like(q)
    out = torch.empty((B, 16, D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ga.decode_workspace_size(kw, layer, B, Smax), dtype=torch.uint8, device="cuda")
    ga.qk_prologue(kw, layer, q, None, q_out=qt, pos0=to_dev((ctx - 1).astype(np.int32)))
    ga.attn_decode(kw, layer, qt.view(B, 16, D), kc, vc, ctx_d, out=out, workspace=ws)
    out_l, lse = ga.attn_decode(kw, layer, qt.view(B, 16, D), kc, vc, ctx_d, want_lse=True, workspace=ws)
    qm_bits = bench.decode_query(layer, multi=True)
    qm = to_dev(qm_bits.view(np.int16)).view(torch.bfloat16)
    wsm = torch.empty(ga.decode_multi_workspace_size(kw, layer, B, Lq, Smax), dtype=torch.uint8, device="cuda")
    outm = ga.attn_decode_multi(kw, layer, qm, kc, vc, ctx_d, workspace=wsm)
    (kq, ksq), (vq, vsq) = bench.decode_int8_caches(ga, layer, kc, vc, ctx)
    out8 = ga.attn_decode_int8(kw, layer, qt.view(B, 1, 16, D), kq, ksq, vq, vsq, ctx_d, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out_l.view(torch.int16), out.view(torch.int16)), "lse request changed the output"
    for name, o in (("q1", out), ("q4", outm), ("int8", out8)):
        assert bool(torch.isfinite(o.float()).all()), f"decode {name}: non-finite output (a row outside a span was read)"
    sel_d = torch.tensor(sel, device="cuda")
    got = dict(q=from_dev_f64(qt[sel_d]), q1=from_dev_f64(out[sel_d]), lse=from_dev_f64(lse[sel_d]),
               q4=from_dev_f64(outm[sel_d]), int8=from_dev_f64(out8[sel_d]))
    spans = [bench.decode_span(ctx[b], L["window"]) for b in sel]
    got_codes = [([c[b, lo:hi].cpu().numpy() for b, (lo, hi) in zip(sel, spans)],
                  [np.ascontiguousarray(s[b, :, lo:hi].cpu().numpy().T) for b, (lo, hi) in zip(sel, spans)])
                 for c, s in ((kq, ksq), (vq, vsq)) if c is not None]
    del kc, vc, kq, ksq, vq, vsq, out, out_l, outm, out8, ws, wsm
    torch.cuda.empty_cache()

    o_spans, bits = _decode_oracle_caches(layer, ctx, sel)
    assert o_spans == spans
    f64 = {t: [bf16_bits_to_f64(x) for x in xs] for t, xs in bits.items()}
    kc_o = _Spans(spans, f64["k"])
    vc_o = None if L["k_eq_v"] else _Spans(spans, f64["v"])
    ctx_s = ctx[sel]

    # one new token: the prologue rotates q at position ctx - 1
    rq = R.prologue(cfg, layer, bf16_bits_to_f64(q_bits[sel]), pos0=ctx_s - 1)[0]       # [n,1,16,D]
    assert_within_one_ulp(got["q"], rq, what=f"decode layer {layer} q")
    rq = R.round_bf16(rq)
    ro, rl = R.decode(cfg, layer, rq[:, 0], kc_o, vc_o, ctx_s)
    mx, mn = assert_close(got["q1"], ro, what=f"decode layer {layer} q1")
    assert_close(got["lse"], rl, what=f"decode layer {layer} lse")
    print(f"[fullsize] decode layer {layer} q1: max-abs {mx:.2e} mean-abs {mn:.2e}", flush=True)

    # four new tokens at positions ctx - 4 .. ctx - 1 (queries taken as processed)
    rm, _ = R.decode_multi(cfg, layer, bf16_bits_to_f64(qm_bits[sel]), kc_o, vc_o, ctx_s)
    mx, mn = assert_close(got["q4"], rm, what=f"decode layer {layer} q4")
    print(f"[fullsize] decode layer {layer} q4: max-abs {mx:.2e} mean-abs {mn:.2e}", flush=True)

    # int8 cache: codes and scales bit for bit over each span, then attention
    # over the oracle's own dequantized codes
    deq = {}
    for (codes, scales), t in zip(got_codes, ("k", "v")):
        deq[t] = []
        for j, (lo, hi) in enumerate(spans):
            rc, rs = R.quantize_int8(f64[t][j].astype(np.float32))        # bf16 values are exact in fp32
            assert np.array_equal(codes[j], rc), f"int8 codes, layer {layer} {t} seq {sel[j]}"
            assert np.array_equal(scales[j].view(np.uint32), rs.view(np.uint32)), \
                f"int8 scales, layer {layer} {t} seq {sel[j]}"
            deq[t].append(R.dequantize_int8(rc, rs))
    k8 = _Spans(spans, deq["k"])
    v8 = None if L["k_eq_v"] else _Spans(spans, deq["v"])
    r8, _ = R.decode_multi(cfg, layer, rq, k8, v8, ctx_s)
    mx, mn = assert_close(got["int8"], r8, what=f"decode layer {layer} int8")
    print(f"[fullsize] decode layer {layer} int8: max-abs {mx:.2e} mean-abs {mn:.2e}", flush=True)
