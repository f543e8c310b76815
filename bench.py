"""Throughput of the Gemma decoder-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu-baseline]

One step = one pass of the hot path over the Gemma-2-2B-shaped layer pair
(B=2, S=8192, 8 query heads, 4 KV heads, head width 256, logit soft cap 50,
query_pre_attn_scalar 256, RoPE base 1e4): QK-norm/rotary and prefill
attention of the local layer (window 4096) and of the global layer.  The
Gemma 2 layers have no query norm, so the step takes the fused form: the
prologue processes the keys and the prefill kernel rotates the queries as it
loads them (gemma_attn_prefill_qrope, bit-identical to prologue + prefill).
``value`` is the step's unmasked attention FLOPs (4*D per allowed query-key
pair) divided by the step time, in TFLOP/s, with every input already resident
in HBM.  The K timed steps run back to back with events only before the first
and after the last; the per-kernel launch times below come from a second pass
of K steps with an event pair around every launch.  ``step_forms`` also times
the prologue-then-prefill form over K steps.

The same JSON line also carries
  * ``roofline``: the prefill kernel's algorithmic FLOPs per launch over its
    average launch time (HIP events on the launch stream), against the bf16
    dense MFMA peak of 2.5 PFLOP/s;
  * ``decode``: the Gemma-4-12B-shaped decode step (64 sequences, contexts
    drawn from U[512, 65536]; local layer 16/8 heads D256 window 1024 and
    global layer 16/1 heads D512 keys-as-values), in GB/s of KV read against
    8 TB/s HBM; also 4 new tokens per sequence (``*_q4``) and the same cache
    stored as int8 codes with per-(token, head) scales (``*_int8``);
  * ``prefill_configs``: the Gemma-3-1B-shaped 6-layer stack and the
    Gemma-4-12B-shaped global layer (TFLOP/s per layer);
  * ``prologue_ms`` / ``prologue_gbs`` (and the same per prefill config): the
    QK prologue's time and its rate over the bytes it must move (k, and q
    outside the fused pair, read and written once), as it is HBM-bound;
  * ``cpu_baseline``: the fp64 oracle timed on the host's cores over a
    bounded sample of the same workload (``value``), and beside it over
    samples of the Gemma-3 stack, the Gemma-4 global layer and the decode
    step (``configs``), with the CPU model and the threads used.
Every ``roofline`` block (the pair's, one per layer in ``prefill_configs``,
and the decode one) divides the kernel's algorithmic work per launch by its
mean launch time from HIP events recorded on the launch stream around its
launches (``timing`` says which); ``traffic`` is the HBM bytes per launch
from the committed rocprofv3 counter summary under ``profiles/`` while the
kernel source still hashes to the value recorded there, else null.
``measured_ceiling`` holds what library code reaches on the same GPU in the
same run (bf16 GEMMs through torch.matmul, a device-to-device copy); each
MFMA-bound roofline block adds ``frac_of_measured``, its achieved rate over
the GEMM figure, beside ``frac`` against the published peak.
All inputs are seeded synthetic tensors (N(0,1) drawn in fp32, rounded to
bf16); no trained weights or datasets are involved.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0
HBM_PEAK_GBS = 8000.0

GEMMA2_PAIR = dict(num_heads=8, num_kv_heads=4, head_dim=256, sliding_window=4096, sliding_window_pattern=2,
                   rope_theta=1e4, attn_logit_softcapping=50.0, query_pre_attn_scalar=256.0)
GEMMA3_STACK = dict(num_heads=4, num_kv_heads=1, head_dim=256, sliding_window=512, sliding_window_pattern=6,
                    rope_theta=1e6, rope_local_theta=1e4, query_pre_attn_scalar=256.0, norm_weight_offset=1)
GEMMA4_12B = dict(num_heads=16, num_kv_heads=8, num_global_kv_heads=1, head_dim=256, global_head_dim=512,
                  sliding_window=1024, sliding_window_pattern=6, rope_theta=1e6, rope_local_theta=1e4,
                  partial_rotary_factor=0.25, k_eq_v=True, norm_weight_offset=0)

# Prefill workloads: name -> (seed family, config, timed layers, batch, sequence length, QK-norm).
PREFILL_WORKLOADS = {
    "gemma2_pair": (2, GEMMA2_PAIR, (0, 1), 2, 8192, False),
    "gemma3_stack": (3, GEMMA3_STACK, (0, 5), 4, 16384, True),
    "gemma4_global": (4, GEMMA4_12B, (5,), 1, 32768, True),
}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


TIMING = "HIP events on the launch stream around each timed launch; mean over the timed launches"


def measured_traffic(kernel_source: str, summary: str):
    """The JSON block of a committed rocprofv3 counter summary, or None when the
    kernel source has changed since the counters were taken."""
    import hashlib
    import re

    try:
        text = open(os.path.join(ROOT, "profiles", summary)).read()
        block = json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))
        src = hashlib.sha256(open(os.path.join(ROOT, kernel_source), "rb").read()).hexdigest()
    except (OSError, AttributeError, ValueError):
        return None
    if block.get("source_sha256") != src:
        return None
    return block


def traffic_of(kernel_source: str, summary: str, key: str):
    """HBM bytes per launch of one workload from a counter summary (None if absent or stale)."""
    block = measured_traffic(kernel_source, summary)
    if block is None:
        return None
    v = block.get("hbm_bytes_per_launch", {}).get(key)
    return None if v is None else int(v)


def mfma_roofline(flops: int, ms: float, kernel: str, traffic=None) -> dict:
    achieved = flops / (ms * 1e-3) / 1e12
    return dict(bound="mfma", achieved=round(achieved, 2), peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                frac=round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), traffic=traffic, kernel=kernel,
                flops_per_launch=int(flops), avg_launch_ms=round(ms, 4), timing=TIMING)


def _flops(kw, layer, B, S) -> int:
    """4*D per allowed (query head, key) pair; window W sees exactly W keys."""
    import decoder_attention_amd as ga

    L = ga.resolve_layer(kw, layer)
    W = L["window"]
    n = S * (S + 1) // 2 if (W <= 0 or W >= S) else W * (W + 1) // 2 + (S - W) * W
    return 4 * L["head_dim"] * B * kw["num_heads"] * n


def _dev_bf16(bits):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def layer_inputs(cfg_id, kw, layer, B, S, with_norm):
    """Host inputs of one prefill layer of a benchmark workload: raw bf16 bits
    of q [B,S,Hq,D], k and v [B,S,Hkv,D] (v None with keys-as-values), and the
    fp32 QK-norm weights [D] (None without QK-norm)."""
    import decoder_attention_amd as ga
    from synth import normal_bf16, norm_weight, seed_for

    L = ga.resolve_layer(kw, layer)
    D, Hkv, Hq = L["head_dim"], L["num_kv_heads"], kw["num_heads"]
    h = dict(L=L)
    h["q"] = normal_bf16(seed_for(cfg_id, layer, "q"), (B, S, Hq, D))
    h["k"] = normal_bf16(seed_for(cfg_id, layer, "k"), (B, S, Hkv, D))
    h["v"] = None if L["k_eq_v"] else normal_bf16(seed_for(cfg_id, layer, "v"), (B, S, Hkv, D))
    h["qw"] = norm_weight(seed_for(cfg_id, layer, "q_norm_w"), D) if with_norm else None
    h["kw"] = norm_weight(seed_for(cfg_id, layer, "k_norm_w"), D) if with_norm else None
    return h


def layer_tensors(cfg_id, kw, layer, B, S, with_norm, host=None):
    """Device tensors of one prefill layer (from ``host``, else freshly drawn)."""
    import torch

    h = host if host is not None else layer_inputs(cfg_id, kw, layer, B, S, with_norm)
    t = dict(L=h["L"])
    for name in ("q", "k", "v"):
        t[name] = None if h[name] is None else _dev_bf16(h[name])
    for name in ("qw", "kw"):
        t[name] = None if h[name] is None else torch.from_numpy(h[name]).cuda()
    t["qt"] = torch_empty_like(t["q"])
    t["kt"] = torch_empty_like(t["k"])
    t["out"] = torch_empty_like(t["q"])
    return t


def torch_empty_like(x):
    import torch

    return torch.empty_like(x)


class Timer:
    """HIP events around launches on the current stream."""

    def __init__(self):
        self.pairs = {}

    def start(self, name):
        import torch

        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.setdefault(name, []).append([e, None])

    def stop(self, name):
        import torch

        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs[name][-1][1] = e

    def ms(self, name):
        return [a.elapsed_time(b) for a, b in self.pairs.get(name, [])]


def run_layer_step(ga, kw, layer, t, timer=None, tag="", fused=False):
    """One layer of the hot path.  fused: the prologue processes the keys only and the prefill kernel rotates
    the queries as it loads them (gemma_attn_prefill_qrope; layers without a query norm)."""
    if timer:
        timer.start(f"prologue{tag}")
    if fused:
        ga.qk_prologue(kw, layer, None, t["k"], k_out=t["kt"], k_norm_w=t["kw"])
    else:
        ga.qk_prologue(kw, layer, t["q"], t["k"], q_out=t["qt"], k_out=t["kt"], q_norm_w=t["qw"], k_norm_w=t["kw"])
    if timer:
        timer.stop(f"prologue{tag}")
        timer.start(f"prefill{tag}")
    if fused:
        ga.attn_prefill_qrope(kw, layer, t["q"], t["kt"], t["v"], out=t["out"])
    else:
        ga.attn_prefill(kw, layer, t["qt"], t["kt"], t["v"], out=t["out"])
    if timer:
        timer.stop(f"prefill{tag}")


def _prologue_bytes(kw, layer, B, S, keys_only=False) -> int:
    """Bytes the QK prologue must move: q (unless keys only) and k read once and written once (bf16)."""
    import decoder_attention_amd as ga

    L = ga.resolve_layer(kw, layer)
    heads = (0 if keys_only else kw["num_heads"]) + L["num_kv_heads"]
    return 2 * 2 * B * S * heads * L["head_dim"]


def _pair_traffic():
    """Mean HBM bytes per launch of the pair's prefill kernel (counter summary), or None."""
    t = measured_traffic("decoder_attention_amd/csrc/prefill.hip", "prefill_gemma2_pair_hbm_traffic.md")
    return None if t is None else t["hbm_bytes_mean"]


def bench_pair(ga, steps, warmup):
    import torch

    cfg_id, kw, _, B, S, norm = PREFILL_WORKLOADS["gemma2_pair"]
    layers = {layer: layer_tensors(cfg_id, kw, layer, B, S, norm) for layer in (0, 1)}
    flops = {layer: _flops(kw, layer, B, S) for layer in (0, 1)}
    for _ in range(warmup):
        for fused in (True, False):
            for layer in (0, 1):
                run_layer_step(ga, kw, layer, layers[layer], fused=fused)
    torch.cuda.synchronize()

    def timed(fused):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps):
            for layer in (0, 1):
                run_layer_step(ga, kw, layer, layers[layer], fused=fused)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    # The timed steps carry no events between their launches (an event record
    # between two kernels idles the GPU for a few microseconds); the launch
    # times per kernel come from a second, instrumented pass of as many steps.
    # The step is the fused form (keys-only prologue, query rotary in the
    # prefill kernel); the prologue-then-prefill form is timed after it for
    # comparison.
    t0 = time.perf_counter()
    step_ms = timed(True)
    wall = time.perf_counter() - t0
    unfused_ms = timed(False)
    timer = Timer()
    for _ in range(steps):
        for layer in (0, 1):
            run_layer_step(ga, kw, layer, layers[layer], timer, tag=str(layer), fused=True)
    torch.cuda.synchronize()
    pre = {layer: float(np.mean(timer.ms(f"prefill{layer}"))) for layer in (0, 1)}
    pro = {layer: float(np.mean(timer.ms(f"prologue{layer}"))) for layer in (0, 1)}
    total_flops = flops[0] + flops[1]
    achieved = total_flops / ((pre[0] + pre[1]) * 1e-3) / 1e12
    return dict(
        step_ms=step_ms, wall_s=wall, total_flops=total_flops,
        value=total_flops / (step_ms * 1e-3) / 1e12,
        step_forms={
            "fused_query_rotary": dict(ms=round(step_ms, 4), tflops=round(total_flops / (step_ms * 1e-3) / 1e12, 2)),
            "prologue_then_prefill": dict(ms=round(unfused_ms, 4),
                                          tflops=round(total_flops / (unfused_ms * 1e-3) / 1e12, 2))},
        prefill_ms={"local_w4096": pre[0], "global": pre[1]},
        prologue_ms={"local_w4096": pro[0], "global": pro[1]},
        prologue_gbs={name: round(_prologue_bytes(kw, layer, B, S, keys_only=True) / (pro[layer] * 1e-3) / 1e9, 1)
                      for layer, name in ((0, "local_w4096"), (1, "global"))},
        prefill_tflops={"local_w4096": flops[0] / (pre[0] * 1e-3) / 1e12, "global": flops[1] / (pre[1] * 1e-3) / 1e12},
        roofline=dict(bound="mfma", achieved=round(achieved, 2), peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                      frac=round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), traffic=_pair_traffic(),
                      kernel="prefill_kernel<256,2,false,true,WIDE,true> (query rotary in the kernel): local "
                             "WIDE=false (4 waves), global WIDE=true (8)",
                      flops_per_launch={"local_w4096": flops[0], "global": flops[1]},
                      avg_launch_ms={"local_w4096": round(pre[0], 4), "global": round(pre[1], 4)},
                      timing="HIP events on the launch stream around each launch of an instrumented pass of as many "
                             "steps, run after the timed ones; mean over those launches; achieved = both layers' FLOPs "
                             "over their summed mean launch times"),
        layers=layers,
    )


# Kernel forms the host picks for the prefill workloads (for the roofline blocks).
PREFILL_KERNEL = {
    ("gemma3_stack", 0): "prefill_kernel<256,4,false,false,false> (4 waves)",
    ("gemma3_stack", 5): "prefill_kernel<256,4,false,false,false> (4 waves)",
    ("gemma4_global", 5): "prefill_kernel<512,16,true,false,false> (4 waves, D split in pairs)",
}


def bench_prefill_layer(ga, workload, layer, reps=10, traffic_key=None):
    import torch

    cfg_id, kw, _, B, S, with_norm = PREFILL_WORKLOADS[workload]
    t = layer_tensors(cfg_id, kw, layer, B, S, with_norm)
    # Warm up for about 100 ms of this layer's launches (at least two), so the
    # timed launches start from a settled clock.
    w = Timer()
    for _ in range(2):
        w.start("x")
        run_layer_step(ga, kw, layer, t)
        w.stop("x")
    torch.cuda.synchronize()
    for _ in range(min(200, int(100.0 / max(float(np.mean(w.ms("x"))), 1e-3)))):
        run_layer_step(ga, kw, layer, t)
    timer = Timer()
    for _ in range(reps):
        run_layer_step(ga, kw, layer, t, timer)
    torch.cuda.synchronize()
    ms = float(np.mean(timer.ms("prefill")))
    pro_ms = float(np.mean(timer.ms("prologue")))
    f = _flops(kw, layer, B, S)
    del t
    torch.cuda.empty_cache()
    traffic = None
    if traffic_key:
        traffic = traffic_of("decoder_attention_amd/csrc/prefill.hip", "prefill_gemma3_gemma4_hbm_traffic.md",
                             traffic_key)
    return dict(prefill_ms=round(ms, 4), tflops=round(f / (ms * 1e-3) / 1e12, 2),
                prologue_ms=round(pro_ms, 4),
                prologue_gbs=round(_prologue_bytes(kw, layer, B, S) / (pro_ms * 1e-3) / 1e9, 1), flops=f,
                roofline=mfma_roofline(f, ms, PREFILL_KERNEL[(workload, layer)], traffic))


DECODE_B, DECODE_SMAX, DECODE_MULTI = 64, 65536, 4


def decode_contexts():
    """The 64 ragged context lengths of the Gemma-4-12B decode workload."""
    from synth import ctx_lengths, seed_for

    return ctx_lengths(seed_for(5, 0, "ctx"), DECODE_B, 512, DECODE_SMAX)


def decode_span(c, W):
    """Cache rows [lo, c) that the decode steps of a sequence with context c
    read: on a local layer the window of the first of the DECODE_MULTI new
    tokens, on a global layer all c rows."""
    return (max(0, int(c) - W - (DECODE_MULTI - 1)) if W else 0, int(c))


def decode_caches(ga, layer, ctx):
    """bf16 caches [B, Smax, Hkv, D] of one layer of the decode workload: the
    rows of each sequence's span drawn from its own seeded stream, every other
    row NaN.  Returns (k_cache, v_cache or None with keys-as-values)."""
    import torch

    from synth import BF16_NAN, normal_bf16_row, seed_for

    B, Smax = DECODE_B, DECODE_SMAX
    L = ga.resolve_layer(GEMMA4_12B, layer)
    D, Hkv, W = L["head_dim"], L["num_kv_heads"], L["window"]
    nan = torch.tensor(int(np.int16(BF16_NAN.view(np.int16))), dtype=torch.int16)
    spans = [decode_span(ctx[b], W) for b in range(B)]
    caches = []
    for tensor in (("k",) if L["k_eq_v"] else ("k", "v")):
        c = torch.full((B, Smax, Hkv, D), nan.item(), dtype=torch.int16, device="cuda")
        seed = seed_for(5, layer, tensor)
        with ThreadPoolExecutor(min(16, len(os.sched_getaffinity(0)))) as ex:
            rows = list(ex.map(lambda b: normal_bf16_row(seed, b, (spans[b][1] - spans[b][0], Hkv, D)), range(B)))
        for b in range(B):
            c[b, spans[b][0]:spans[b][1]] = torch.from_numpy(rows[b].view(np.int16)).cuda()
        del rows
        caches.append(c.view(torch.bfloat16))
    return caches[0], (None if L["k_eq_v"] else caches[1])


def decode_int8_caches(ga, layer, kc, vc, ctx):
    """The same spans quantized on the device: (codes int8 [B, Smax, Hkv, D],
    scales fp32 [B, Hkv, Smax]) per cache, zero codes and NaN scales elsewhere."""
    import torch

    B, Smax = DECODE_B, DECODE_SMAX
    L = ga.resolve_layer(GEMMA4_12B, layer)
    D, Hkv, W = L["head_dim"], L["num_kv_heads"], L["window"]
    res = []
    for c in ((kc,) if vc is None else (kc, vc)):
        cc = torch.zeros((B, Smax, Hkv, D), dtype=torch.int8, device="cuda")
        sc = torch.full((B, Hkv, Smax), float("nan"), dtype=torch.float32, device="cuda")
        for b in range(B):
            lo, hi = decode_span(ctx[b], W)
            p0 = torch.tensor([lo], dtype=torch.int32, device="cuda")
            ga.kv_quantize_int8(c[b:b + 1, lo:hi], cc[b:b + 1], sc[b:b + 1], pos0=p0)
        res.append((cc, sc))
    return res[0], (None, None) if vc is None else res[1]


def decode_query(layer, multi=False):
    """Raw bf16 bits of the decode workload's queries: [B, 1, 16, D] for the
    one-token step (rotated by the prologue at position ctx - 1), else
    [B, DECODE_MULTI, 16, D], taken as already processed."""
    import decoder_attention_amd as ga
    from synth import normal_bf16, seed_for

    D = ga.resolve_layer(GEMMA4_12B, layer)["head_dim"]
    if multi:
        return normal_bf16(seed_for(5, layer, "q") + 7, (DECODE_B, DECODE_MULTI, 16, D))
    return normal_bf16(seed_for(5, layer, "q"), (DECODE_B, 1, 16, D))


DECODE_KERNEL = {
    "local_w1024": "decode_split_kernel<256,2,false,false,1> (one workgroup per sequence, which writes the output)",
    "local_w1024_q4": "decode_split_kernel<256,2,false,false,1> (one workgroup per sequence, which writes the output)",
    "local_w1024_int8": "decode_split_i8_kernel<256,2,false,false> (one workgroup per sequence, which writes the output)",
    "global_keqv": "decode_plan_kernel + decode_split_kernel<512,16,true,false,1> + decode_combine_kernel<512>",
    "global_keqv_q4": "decode_plan_kernel + decode_tile_kernel<16,false> + decode_combine_kernel<512>",
    "global_keqv_int8": "decode_plan_kernel + decode_split_i8_kernel<512,16,true,false> + decode_combine_kernel<512>",
}


def hbm_roofline(nbytes: int, ms: float, case: str) -> dict:
    achieved = nbytes / (ms * 1e-3) / 1e9
    traffic = traffic_of("decoder_attention_amd/csrc/decode.hip", "decode_hbm_traffic.md", case)
    return dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic, kernel=DECODE_KERNEL[case],
                bytes_per_launch=int(nbytes), avg_launch_ms=round(ms, 4),
                timing=TIMING + " (the whole decode call: every kernel it launches)")


# Untimed calls before each decode case: the multi-token tile kernel and the
# int8 kernel take a few dozen calls to settle (20-call rounds right after two
# warm-up calls measured 488, 472, 467, 458 us on the 4-token global layer).
DECODE_WARMUP = 60


def bench_decode(ga, reps=20, warm=DECODE_WARMUP):
    """Gemma-4-12B decode step: one local and one global layer over 64 ragged contexts.

    Every timed call follows a 1 GiB read that evicts the previous call's lines
    from the last-level cache: in a model each layer's cache was last read a
    whole step earlier, while here the same cache is read call after call (the
    local layer's 0.54 GB would otherwise partly stay cached)."""
    import torch

    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
    flush_out = torch.empty((), dtype=torch.float32, device="cuda")

    def cold():
        torch.sum(flush_buf, dim=0, out=flush_out)

    B, Smax = DECODE_B, DECODE_SMAX
    ctx = decode_contexts()
    ctx_d = torch.from_numpy(ctx).cuda()
    p32 = torch.from_numpy(ctx - 1).to(torch.int32).cuda()
    res = {}
    for layer, name in ((0, "local_w1024"), (5, "global_keqv")):
        L = ga.resolve_layer(GEMMA4_12B, layer)
        D, Hkv, W = L["head_dim"], L["num_kv_heads"], L["window"]
        kc, vc = decode_caches(ga, layer, ctx)
        q = _dev_bf16(decode_query(layer))
        qt = torch.empty_like(q)
        out = torch.empty((B, 16, D), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(ga.decode_workspace_size(GEMMA4_12B, layer, B, Smax), dtype=torch.uint8, device="cuda")
        for _ in range(warm):
            ga.qk_prologue(GEMMA4_12B, layer, q, None, q_out=qt, pos0=p32)
            ga.attn_decode(GEMMA4_12B, layer, qt.view(B, 16, D), kc, vc, ctx_d, out=out, workspace=ws)
        timer = Timer()
        for _ in range(reps):
            cold()
            timer.start("prologue")
            ga.qk_prologue(GEMMA4_12B, layer, q, None, q_out=qt, pos0=p32)
            timer.stop("prologue")
            timer.start("decode")
            ga.attn_decode(GEMMA4_12B, layer, qt.view(B, 16, D), kc, vc, ctx_d, out=out, workspace=ws)
            timer.stop("decode")
        torch.cuda.synchronize()
        span = np.minimum(ctx, W) if W else ctx
        nbytes = int(span.sum()) * Hkv * D * 2 * (1 if L["k_eq_v"] else 2)
        ms = float(np.mean(timer.ms("decode")))
        res[name] = dict(decode_ms=round(ms, 4), kv_bytes=nbytes, gbs=round(nbytes / (ms * 1e-3) / 1e9, 1),
                         frac=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         prologue_ms=round(float(np.mean(timer.ms("prologue"))), 4),
                         roofline=hbm_roofline(nbytes, ms, name))

        # Several new tokens per sequence (draft verification): the same cache
        # rows plus the DECODE_MULTI - 1 extra rows the first token's window adds.
        Lq = DECODE_MULTI
        qm = _dev_bf16(decode_query(layer, multi=True))
        outm = torch.empty_like(qm)
        wsm = torch.empty(ga.decode_multi_workspace_size(GEMMA4_12B, layer, B, Lq, Smax), dtype=torch.uint8,
                          device="cuda")
        for _ in range(warm):
            ga.attn_decode_multi(GEMMA4_12B, layer, qm, kc, vc, ctx_d, out=outm, workspace=wsm)
        tm = Timer()
        for _ in range(reps):
            cold()
            tm.start("m")
            ga.attn_decode_multi(GEMMA4_12B, layer, qm, kc, vc, ctx_d, out=outm, workspace=wsm)
            tm.stop("m")
        torch.cuda.synchronize()
        span_m = np.minimum(ctx, W + Lq - 1) if W else ctx
        nb_m = int(span_m.sum()) * Hkv * D * 2 * (1 if L["k_eq_v"] else 2)
        ms_m = float(np.mean(tm.ms("m")))
        res[name + "_q4"] = dict(decode_ms=round(ms_m, 4), kv_bytes=nb_m, gbs=round(nb_m / (ms_m * 1e-3) / 1e9, 1),
                                 frac=round(nb_m / (ms_m * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                 roofline=hbm_roofline(nb_m, ms_m, name + "_q4"))
        del qm, outm, wsm

        # int8 cache: the same rows quantized on the device (codes + one fp32
        # scale per token and head); algorithmic bytes = codes + scales read.
        (kq, ksq), (vq, vsq) = decode_int8_caches(ga, layer, kc, vc, ctx)
        q1 = qt.view(B, 1, 16, D)
        out1 = out.view(B, 1, 16, D)
        for _ in range(warm):
            ga.attn_decode_int8(GEMMA4_12B, layer, q1, kq, ksq, vq, vsq, ctx_d, out=out1, workspace=ws)
        t8 = Timer()
        for _ in range(reps):
            cold()
            t8.start("d8")
            ga.attn_decode_int8(GEMMA4_12B, layer, q1, kq, ksq, vq, vsq, ctx_d, out=out1, workspace=ws)
            t8.stop("d8")
        torch.cuda.synchronize()
        nb8 = int(span.sum()) * Hkv * (D + 4) * (1 if L["k_eq_v"] else 2)
        ms8 = float(np.mean(t8.ms("d8")))
        res[name + "_int8"] = dict(decode_ms=round(ms8, 4), kv_bytes=nb8, gbs=round(nb8 / (ms8 * 1e-3) / 1e9, 1),
                                   frac=round(nb8 / (ms8 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                   speedup_vs_bf16=round(ms / ms8, 3),
                                   roofline=hbm_roofline(nb8, ms8, name + "_int8"))
        del kq, ksq, vq, vsq, kc, vc
        torch.cuda.empty_cache()
    tot_bytes = 5 * res["local_w1024"]["kv_bytes"] + res["global_keqv"]["kv_bytes"]
    tot_ms = 5 * res["local_w1024"]["decode_ms"] + res["global_keqv"]["decode_ms"]
    res["stack_5local_1global"] = dict(ms=round(tot_ms, 4), gbs=round(tot_bytes / (tot_ms * 1e-3) / 1e9, 1))
    res["roofline"] = res["global_keqv"]["roofline"]
    return res


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


class _SpanCache:
    """[B', Smax, Hkv, D] view of per-sequence cache rows [lo_b, hi_b) (the rows a decode step reads)."""

    def __init__(self, spans, rows):
        self.spans, self.rows = spans, rows

    def __getitem__(self, idx):
        b, s, h, d = idx
        lo, hi = self.spans[b]
        assert s.step is None and lo <= s.start <= s.stop <= hi
        return self.rows[b][s.start - lo:s.stop - lo, h, d]


def cpu_baseline():
    """The fp64 oracle as it stands, on the host's cores, with BLAS held to one
    thread per worker (threadpoolctl is required: without it the workers'
    BLAS calls would oversubscribe the cores and the figure would mean
    nothing).  ``value``: both layers of the Gemma-2-2B pair, whole.  Beside
    it (``configs``): the Gemma-3-1B local and global layers, whole; the
    Gemma-4-12B global layer on its first 8192 positions (a causal prefix is
    a complete problem of its own); the Gemma-4-12B decode step on every
    eighth of its 64 sequences (GB/s over those sequences' KV bytes).  Only
    the oracle's attention (and, for prefill, its prologue) is timed; drawing
    the inputs is not."""
    from threadpoolctl import threadpool_limits

    from oracle import gemma_ref as R
    from synth import bf16_bits_to_f64, normal_bf16, norm_weight, normal_bf16_row, seed_for

    threads = len(os.sched_getaffinity(0))

    def prefill_sample(workload, layer, s_sample):
        cfg_id, kw, _, B, S, with_norm = PREFILL_WORKLOADS[workload]
        cfg = R.GemmaAttnConfig(**kw)
        L = R.resolve_layer(cfg, layer)
        D, Hkv, Hq = L["head_dim"], L["num_kv_heads"], cfg.num_heads
        q = bf16_bits_to_f64(normal_bf16(seed_for(cfg_id, layer, "q"), (B, S, Hq, D))[:, :s_sample])
        k = bf16_bits_to_f64(normal_bf16(seed_for(cfg_id, layer, "k"), (B, S, Hkv, D))[:, :s_sample])
        v = None if L["k_eq_v"] else bf16_bits_to_f64(
            normal_bf16(seed_for(cfg_id, layer, "v"), (B, S, Hkv, D))[:, :s_sample])
        qw = norm_weight(seed_for(cfg_id, layer, "q_norm_w"), D) if with_norm else None
        kw_ = norm_weight(seed_for(cfg_id, layer, "k_norm_w"), D) if with_norm else None
        t0 = time.perf_counter()
        with threadpool_limits(limits=1):
            qt, kt = R.prologue(cfg, layer, q, k, qw, kw_)
            R.prefill(cfg, layer, qt, kt, v, block_rows=64 if D > 256 else 256, threads=threads)
        dt = time.perf_counter() - t0
        f = R.prefill_flops(cfg, layer, B, s_sample)
        return f, dt

    pf, pt = 0, 0.0
    for layer in (0, 1):
        f, dt = prefill_sample("gemma2_pair", layer, 8192)
        pf += f
        pt += dt
    configs = {}
    for name, (wl, layer, s_sample) in {"gemma3_1b_local_w512": ("gemma3_stack", 0, 16384),
                                          "gemma3_1b_global": ("gemma3_stack", 5, 16384),
                                          "gemma4_12b_global_keqv_d512": ("gemma4_global", 5, 8192)}.items():
        f, dt = prefill_sample(wl, layer, s_sample)
        S = PREFILL_WORKLOADS[wl][4]
        configs[name] = dict(value=round(f / dt / 1e12, 5), unit="TFLOP/s", seconds=round(dt, 2), flops=f,
                             sample=f"first {s_sample} of {S} positions, every sequence and head")

    # decode: every eighth sequence of the Gemma-4-12B step, both layers
    cfg = R.GemmaAttnConfig(**GEMMA4_12B)
    ctx = decode_contexts()
    sel = list(range(0, DECODE_B, 8))
    for layer, name in ((0, "decode_local_w1024"), (5, "decode_global_keqv")):
        L = R.resolve_layer(cfg, layer)
        D, Hkv, W = L["head_dim"], L["num_kv_heads"], L["window"]
        spans = [decode_span(ctx[b], W) for b in sel]
        caches = []
        for tensor in (("k",) if L["k_eq_v"] else ("k", "v")):
            seed = seed_for(5, layer, tensor)
            caches.append(_SpanCache(spans, [bf16_bits_to_f64(normal_bf16_row(seed, b, (hi - lo, Hkv, D)))
                                             for b, (lo, hi) in zip(sel, spans)]))
        kc = caches[0]
        vc = None if L["k_eq_v"] else caches[1]
        cs = ctx[sel]
        q = R.prologue(cfg, layer, bf16_bits_to_f64(decode_query(layer)[sel]), pos0=cs - 1)[0][:, 0]
        t0 = time.perf_counter()
        R.decode(cfg, layer, q, kc, vc, cs)
        dt = time.perf_counter() - t0
        nbytes = R.decode_kv_bytes(cfg, layer, cs)
        configs[name] = dict(value=round(nbytes / dt / 1e9, 3), unit="GB/s", seconds=round(dt, 2), kv_bytes=nbytes,
                             sample=f"sequences {sel} of {DECODE_B} (one new token each)")
    return dict(value=round(pf / pt / 1e12, 5), unit="TFLOP/s", cores=threads, kind="oracle",
                sample=f"both layers of the Gemma-2-2B pair, all 8192 positions of both sequences "
                       f"({pf:.3e} unmasked FLOPs in {pt:.1f} s, fp64 numpy)",
                cpu_model=_cpu_model(), configs=configs)


def measured_ceilings() -> dict:
    """What library code reaches on this GPU: bf16 GEMMs through torch.matmul
    (hipBLASLt; the best of two sizes) and a device-to-device copy.  Context
    for the roofline fractions, which stay against the published peaks."""
    import torch

    def timed(fn, warm=10, reps=10):
        for _ in range(warm):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in ev:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))

    gemm = {}
    for n in (8192, 16384):
        a = torch.randn((n, n), device="cuda").to(torch.bfloat16)
        b = torch.randn((n, n), device="cuda").to(torch.bfloat16)
        c = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
        gemm[n] = 2 * n ** 3 / (timed(lambda: torch.matmul(a, b, out=c)) * 1e-3) / 1e12
        del a, b, c
    best = max(gemm, key=gemm.get)
    x = torch.empty(1 << 29, dtype=torch.float32, device="cuda")   # 2 GiB
    x.fill_(1.0)
    y = torch.empty_like(x)
    copy_ms = timed(lambda: y.copy_(x))
    del x, y
    torch.cuda.empty_cache()
    return dict(
        mfma_bf16_gemm=dict(value=round(gemm[best], 1), unit="TFLOP/s",
                            how=f"torch.matmul bf16 {best}^3 (hipBLASLt), median of 10 after 10 warm-up; "
                                + ", ".join(f"{n}^3: {v:.1f}" for n, v in gemm.items())),
        hbm_copy=dict(value=round(2 * (2 << 30) / (copy_ms * 1e-3) / 1e9, 1), unit="GB/s",
                      how="2 GiB device-to-device copy, bytes read + written, median of 10"))


def _with_measured(roof: dict, ceil: dict) -> dict:
    """MFMA-bound blocks gain frac_of_measured (over the library GEMM); a copy is
    no ceiling for a read-only stream, so HBM-bound blocks stay as they are."""
    if roof.get("bound") != "mfma":
        return roof
    return dict(roof, frac_of_measured=round(roof["achieved"] / ceil["mfma_bf16_gemm"]["value"], 4))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="skip decode and the other prefill configs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true", help="also run a 1 GiB device copy (counter scale)")
    ap.add_argument("--workload", default="all", choices=["all", "pair", "gemma3", "gemma4", "decode"],
                    help="restrict to one workload (for profiling); the JSON line is printed for 'all'/'pair' only")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported (the attention path is "
              "single-GPU; multi-GPU sharding is a design note)", file=sys.stderr)
        sys.exit(2)
    import torch

    import decoder_attention_amd as ga

    torch.cuda.set_device(0)
    ga.load()
    if a.calibrate_copy:
        # three 1 GiB device copies: a known byte count for scaling the HBM counters
        x = torch.empty(1 << 29, dtype=torch.int16, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        del x, y
        torch.cuda.empty_cache()
    if a.workload in ("gemma3", "gemma4", "decode"):
        out = {}
        if a.workload == "gemma3":
            for layer, name in ((0, "gemma3_1b_local_w512"), (5, "gemma3_1b_global")):
                out[name] = bench_prefill_layer(ga, "gemma3_stack", layer, reps=a.steps, traffic_key=name)
        elif a.workload == "gemma4":
            out["gemma4_12b_global_keqv_d512"] = bench_prefill_layer(ga, "gemma4_global", 5, reps=a.steps,
                                                                     traffic_key="gemma4_12b_global_keqv_d512")
        else:
            out["decode"] = bench_decode(ga, reps=a.steps)
        print(json.dumps({"workload": a.workload, **out}), flush=True)
        return
    log("[bench] gemma2 pair: generating inputs")
    pair = bench_pair(ga, a.steps, a.warmup)
    log(f"[bench] gemma2 pair: {pair['value']:.1f} TFLOP/s, step {pair['step_ms']:.3f} ms")
    del pair["layers"]
    torch.cuda.empty_cache()
    line = {
        "metric": "prefill attn TFLOP/s (unmasked FLOPs, % MFMA peak); decode KV GB/s (% HBM peak)",
        "value": round(pair["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(pair["step_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) fp32 rounded to bf16; no weights)",
        "config": {"workload": "Gemma-2-2B-shaped layer pair: QK prologue (keys) + prefill attention with the "
                               "query rotary in the kernel, of one local (window 4096) and one global layer; "
                               "B2 S8192 Hq8 Hkv4 D256, softcap 50, qpas 256, RoPE 1e4",
                   "batch": 2, "seq_len": 8192, "num_heads": 8, "num_kv_heads": 4, "head_dim": 256,
                   "flops_per_step": pair["total_flops"]},
        "roofline": pair["roofline"],
        "prefill_ms": pair["prefill_ms"],
        "prologue_ms": pair["prologue_ms"],
        "prologue_gbs": pair["prologue_gbs"],
        "prefill_tflops": {k: round(v, 2) for k, v in pair["prefill_tflops"].items()},
        "step_forms": pair["step_forms"],
    }
    if not a.no_extra and a.workload == "all":
        log("[bench] gemma3 stack / gemma4 global prefill")
        cfgs = {}
        for layer, name in ((0, "gemma3_1b_local_w512"), (5, "gemma3_1b_global")):
            cfgs[name] = bench_prefill_layer(ga, "gemma3_stack", layer, traffic_key=name)
        s3 = cfgs["gemma3_1b_local_w512"]
        g3 = cfgs["gemma3_1b_global"]
        stack_f = 5 * s3["flops"] + g3["flops"]
        stack_ms = 5 * s3["prefill_ms"] + g3["prefill_ms"]
        cfgs["gemma3_1b_stack_5local_1global"] = dict(prefill_ms=round(stack_ms, 4),
                                                       tflops=round(stack_f / (stack_ms * 1e-3) / 1e12, 2))
        cfgs["gemma4_12b_global_keqv_d512"] = bench_prefill_layer(ga, "gemma4_global", 5, reps=5,
                                                                  traffic_key="gemma4_12b_global_keqv_d512")
        line["prefill_configs"] = cfgs
        log(f"[bench] prefill configs: {json.dumps(cfgs)}")
        log("[bench] gemma4 decode: building caches")
        line["decode"] = bench_decode(ga)
        log(f"[bench] decode: {json.dumps(line['decode'])}")
    if a.workload == "all" and not a.no_extra:
        log("[bench] measured ceilings (library GEMM, device copy)")
        ceil = measured_ceilings()
        line["measured_ceiling"] = ceil
        line["roofline"] = _with_measured(line["roofline"], ceil)
        for blk in list(line.get("prefill_configs", {}).values()) + list(line.get("decode", {}).values()):
            if isinstance(blk, dict) and "roofline" in blk:
                blk["roofline"] = _with_measured(blk["roofline"], ceil)
        if "decode" in line:
            line["decode"]["roofline"] = line["decode"]["global_keqv"]["roofline"]
        log(f"[bench] measured ceilings: {json.dumps(ceil)}")
    if not a.no_cpu_baseline and a.workload == "all":
        log("[bench] cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
