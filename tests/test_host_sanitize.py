"""The library's host logic under the address and undefined-behaviour sanitizers (CPU).

``tests/host/host_logic_check.cpp`` links the plain C++ host logic
(``host_logic.cpp``: config validation, layer resolution, decode plan and
workspace layout) with ASan and UBSan, no HIP involved, and runs it over
configurations that include edge values: the largest and negative integers,
NaN and infinite doubles, empty batches, one-row caches, more new tokens
than cache rows, devices with few CUs.  Any sanitizer report aborts the run.
Every layer the driver resolves is compared with the oracle's resolution,
value for value, and invalid configurations must be refused.
"""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import gemma_ref as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decoder_attention_amd", "csrc")
INT_MAX = 2 ** 31 - 1

FIELDS = ["num_heads", "num_kv_heads", "num_global_kv_heads", "head_dim", "global_head_dim", "sliding_window",
          "sliding_window_pattern", "k_eq_v", "norm_weight_offset", "reserved", "rope_theta", "rope_local_theta",
          "partial_rotary_factor", "attn_logit_softcapping", "query_pre_attn_scalar", "norm_eps",
          "rope_scaling_factor"]
DEFAULTS = dict(num_heads=8, num_kv_heads=4, num_global_kv_heads=0, head_dim=256, global_head_dim=0,
                sliding_window=0, sliding_window_pattern=1, k_eq_v=0, norm_weight_offset=0, reserved=0,
                rope_theta=1e4, rope_local_theta=0.0, partial_rotary_factor=1.0, attn_logit_softcapping=0.0,
                query_pre_attn_scalar=0.0, norm_eps=1e-6, rope_scaling_factor=0.0)


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("no g++")
    exe = tmp_path_factory.mktemp("san") / "host_logic_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "host_logic.cpp"), os.path.join(ROOT, "tests", "host", "host_logic_check.cpp"),
           "-o", str(exe)]
    subprocess.check_call(cmd)
    return str(exe)


def _cases():
    rng = np.random.default_rng(77)
    cases = []
    page = [   # the pages' tables (Gemma 4, Gemma 2, Gemma 3, Gemma) and the benchmark's shapes
        dict(num_heads=16, num_kv_heads=8, num_global_kv_heads=1, head_dim=256, global_head_dim=512,
             sliding_window=1024, sliding_window_pattern=6, rope_theta=1e6, rope_local_theta=1e4,
             partial_rotary_factor=0.25, k_eq_v=1),
        dict(num_heads=8, num_kv_heads=4, head_dim=256, sliding_window=4096, sliding_window_pattern=2,
             query_pre_attn_scalar=256.0, attn_logit_softcapping=50.0),
        dict(num_heads=4, num_kv_heads=1, head_dim=256, sliding_window=512, sliding_window_pattern=6,
             rope_theta=1e6, rope_local_theta=1e4, norm_weight_offset=1, rope_scaling_factor=8.0),
        dict(num_heads=8, num_kv_heads=1, head_dim=256),
    ]
    sizes = [(64, 65536, 1), (64, 65536, 4), (1, 1, 1), (0, 100, 1), (3, 150, 13), (72, 120, 4),
             (65535, 8192, 1), (2, INT_MAX, 16)]
    for kw in page:
        for layer in (0, 1, 5, 11, INT_MAX - 1, INT_MAX):
            for b, m, ql in sizes:
                cases.append((layer, DEFAULTS | kw, (b, m, ql, 256, 160 * 1024)))
    for _ in range(400):   # random valid-looking configs
        hkv = int(rng.choice([1, 2, 4, 8]))
        kw = dict(num_heads=hkv * int(rng.choice([1, 2, 4, 8, 16])), num_kv_heads=hkv,
                  num_global_kv_heads=int(rng.choice([0, 1])), head_dim=int(rng.choice([64, 96, 256, 512])),
                  global_head_dim=int(rng.choice([0, 512])), sliding_window=int(rng.integers(-3, 5000)),
                  sliding_window_pattern=int(rng.integers(-1, 8)), k_eq_v=int(rng.integers(0, 2)),
                  norm_weight_offset=int(rng.integers(0, 2)), rope_theta=float(rng.choice([1e4, 1e6])),
                  rope_local_theta=float(rng.choice([0.0, 1e4])), partial_rotary_factor=float(rng.random()),
                  attn_logit_softcapping=float(rng.choice([0.0, 30.0, 50.0])),
                  query_pre_attn_scalar=float(rng.choice([0.0, 256.0, 6.0])),
                  rope_scaling_factor=float(rng.choice([0.0, 8.0])))
        size = (int(rng.integers(0, 200)), int(rng.integers(1, 70000)), int(rng.integers(1, 20)),
                int(rng.choice([32, 64, 256, 304])), int(rng.choice([65536, 160 * 1024])))
        cases.append((int(rng.integers(0, 40)), DEFAULTS | kw, size))
    edge = [dict(num_heads=INT_MAX, num_kv_heads=1), dict(num_heads=-8), dict(num_kv_heads=0),
            dict(num_kv_heads=3), dict(head_dim=0), dict(head_dim=-256), dict(head_dim=INT_MAX),
            dict(global_head_dim=-1), dict(num_global_kv_heads=-1), dict(num_global_kv_heads=3),
            dict(reserved=1), dict(k_eq_v=2), dict(norm_weight_offset=-1), dict(rope_theta=float("nan")),
            dict(rope_theta=float("inf")), dict(rope_theta=0.0), dict(rope_theta=-1.0),
            dict(rope_local_theta=float("nan")), dict(partial_rotary_factor=float("nan")),
            dict(partial_rotary_factor=1.5), dict(partial_rotary_factor=-0.1),
            dict(attn_logit_softcapping=float("inf")), dict(query_pre_attn_scalar=float("nan")),
            dict(norm_eps=0.0), dict(norm_eps=float("nan")), dict(rope_scaling_factor=float("-inf")),
            dict(sliding_window=INT_MAX, sliding_window_pattern=INT_MAX),
            dict(sliding_window=INT_MAX, sliding_window_pattern=2, head_dim=512, num_heads=INT_MAX - 3,
                 num_kv_heads=1),
            dict(sliding_window=-INT_MAX - 1, sliding_window_pattern=-INT_MAX - 1)]
    for kw in edge:
        for layer in (-1, 0, 1, INT_MAX):
            for b, m, ql in ((64, INT_MAX, INT_MAX), (INT_MAX, 1, 1), (-1, 0, 0), (1, 1, 1)):
                cases.append((layer, DEFAULTS | kw, (b, m, ql, 0, 0)))
    return cases


def _fmt(v):
    if isinstance(v, float):
        return "nan" if math.isnan(v) else ("inf" if v == math.inf else ("-inf" if v == -math.inf else repr(v)))
    return str(int(v))


def _oracle_layer(kw, layer):
    """The oracle's resolution, or None where the library must refuse the config."""
    ok = (kw["num_heads"] > 0 and kw["num_kv_heads"] > 0 and kw["head_dim"] > 0 and kw["num_global_kv_heads"] >= 0
          and kw["global_head_dim"] >= 0 and kw["reserved"] == 0 and kw["k_eq_v"] in (0, 1)
          and kw["norm_weight_offset"] in (0, 1) and math.isfinite(kw["rope_theta"]) and kw["rope_theta"] > 0
          and math.isfinite(kw["rope_local_theta"]) and 0.0 <= kw["partial_rotary_factor"] <= 1.0
          and math.isfinite(kw["attn_logit_softcapping"]) and math.isfinite(kw["query_pre_attn_scalar"])
          and math.isfinite(kw["norm_eps"]) and kw["norm_eps"] > 0 and math.isfinite(kw["rope_scaling_factor"])
          and layer >= 0)
    if not ok:
        return None
    hg = kw["num_global_kv_heads"] or kw["num_kv_heads"]
    if kw["num_heads"] % kw["num_kv_heads"] or kw["num_heads"] % hg:
        return None
    cfg = R.GemmaAttnConfig(**{f: kw[f] for f in FIELDS if f != "reserved"})
    return R.resolve_layer(cfg, layer)


def test_host_logic_under_sanitizers(driver):
    cases = _cases()
    text = "".join(" ".join(_fmt(x) for x in [layer] + [kw[f] for f in FIELDS] + list(size)) + "\n"
                   for layer, kw, size in cases)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([driver], input=text, capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"exit {r.returncode}\n{r.stderr[-4000:]}"
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    lines = r.stdout.splitlines()
    assert len(lines) == len(cases)
    resolved = 0
    for (layer, kw, size), line in zip(cases, lines):
        got = line.split()
        ref = _oracle_layer(kw, layer)
        if ref is None:
            assert got == ["1"], (layer, kw, got)
            continue
        resolved += 1
        assert got[0] == "0", (layer, kw, got)
        vals = [int(x) for x in got[1:8]] + [float(x) for x in got[8:12]]
        exp = [int(ref["is_global"]), ref["window"], ref["num_kv_heads"], ref["head_dim"], ref["group"],
               ref["rotary_dim"], int(ref["k_eq_v"]), ref["theta"], ref["scale"], ref["softcap"], ref["pos_div"]]
        assert vals == exp, (layer, kw, vals, exp)
        n_wg, span_max, per_seq, tile, total, n_wg8, per_seq8, tile8, total8 = (int(x) for x in got[12:])
        b, m, ql = size[:3]
        if n_wg != -1:
            assert n_wg >= 1 and 1 <= span_max <= m and total > 0
            if per_seq:
                assert n_wg == b
            # int8 plan: never the bf16 tile kernel; one sequence per workgroup when per_seq
            assert n_wg8 >= 1 and total8 > 0 and tile8 == 0
            if per_seq8:
                assert n_wg8 == b
    assert resolved > 300
    assert sum(1 for line in lines if len(line.split()) > 1 and line.split()[12] != "-1") > 300
