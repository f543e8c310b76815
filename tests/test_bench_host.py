"""The benchmark's host-side contract (CPU, no GPU touched).

- `bench.py --gpus N` with N > 1 refuses with a message and exit status 2
  before touching a device;
- the algorithmic work it divides by is the oracle's: prefill FLOPs per layer
  (4*D per allowed query-key pair, checked against the figures the survey
  derives for each workload) and decode KV bytes (each cache element read
  once; codes plus scales for int8);
- the committed rocprofv3 summaries that `bench.py` reads `traffic` from carry a
  JSON block with a source hash and one positive byte count per workload key
  it asks for.
"""
import json
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import bench
from oracle import gemma_ref as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("workload,layer,expected", [
    ("gemma2_pair", 0, 4.124e11), ("gemma2_pair", 1, 5.498e11),
    ("gemma3_stack", 0, 1.353e11), ("gemma3_stack", 5, 2.199e12), ("gemma4_global", 5, 1.759e13)])
def test_prefill_flops_match_the_oracle(workload, layer, expected):
    cfg_id, kw, _, B, S, _ = bench.PREFILL_WORKLOADS[workload]
    got = bench._flops(kw, layer, B, S)
    assert got == R.prefill_flops(R.GemmaAttnConfig(**kw), layer, B, S)
    assert abs(got - expected) / expected < 1e-3


def test_decode_bytes_match_the_oracle():
    ctx = bench.decode_contexts()
    assert len(ctx) == bench.DECODE_B and ctx.min() >= 512 and ctx.max() <= bench.DECODE_SMAX
    cfg = R.GemmaAttnConfig(**bench.GEMMA4_12B)
    for layer in (0, 5):
        L = R.resolve_layer(cfg, layer)
        D, Hkv, W = L["head_dim"], L["num_kv_heads"], L["window"]
        span = np.minimum(ctx, W) if W else ctx
        bf16 = int(span.sum()) * Hkv * D * 2 * (1 if L["k_eq_v"] else 2)
        int8 = int(span.sum()) * Hkv * (D + 4) * (1 if L["k_eq_v"] else 2)
        assert bf16 == R.decode_kv_bytes(cfg, layer, ctx)
        assert int8 == R.decode_kv_bytes(cfg, layer, ctx, int8=True)
        # the 4-token span reaches back to the first new token's window
        for c in ctx[:8]:
            lo, hi = bench.decode_span(c, W)
            assert hi == c and (lo == 0 if not W else lo == max(0, c - W - bench.DECODE_MULTI + 1))


@pytest.mark.parametrize("summary,keys", [
    ("prefill_gemma2_pair_hbm_traffic.md", ["local_w4096", "global"]),
    ("prefill_gemma3_gemma4_hbm_traffic.md", ["gemma3_1b_local_w512", "gemma3_1b_global",
                                              "gemma4_12b_global_keqv_d512"]),
    ("decode_hbm_traffic.md", list(bench.DECODE_KERNEL))])
def test_traffic_summaries_carry_what_bench_reads(summary, keys):
    text = open(os.path.join(ROOT, "profiles", summary)).read()
    block = json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))
    assert re.fullmatch(r"[0-9a-f]{64}", block["source_sha256"])
    assert 1.9 < block["fetch_scale"] < 2.1 and 0.9 < block["write_scale"] < 1.1
    for k in keys:
        assert int(block["hbm_bytes_per_launch"][k]) > 0, k
    assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text
