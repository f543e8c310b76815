"""The GPU parity suites on the LDS-poisoning debug build.

libgemma_attn_ldsnan.so is the library compiled with GA_LDS_POISON=1: every
kernel fills all of its LDS arrays with all-ones bytes (NaN in bf16, fp16, fp32
and fp64) before its first copy or write.  A kernel that reads an LDS location
it did not write in that launch -- a tile row a copy skipped, a partial score
read before its partner stored it, a staged output slot not yet filled --
then turns an output NaN, which every parity test rejects.  (int8 code tiles
are the exception: the byte 0xFF is the valid code -1; their fp32 scales,
copied with them, carry the check.)

The suites run in one child process with the debug build selected through
GEMMA_ATTN_LIBRARY; the child first checks that the library it loaded is that
build.  They include the full-size tests, so every launch shape the benchmark
times also runs poisoned, and the allocation-free decode entry point's test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(1500)]

SUITES = ["tests/test_gpu_parity.py", "tests/test_gpu_decode_matrix.py", "tests/test_gpu_multi.py",
          "tests/test_gpu_int8.py", "tests/test_gpu_ragged.py", "tests/test_gpu_prefill_qrope.py",
          "tests/test_gpu_kv_sharing.py", "tests/test_gpu_graph.py", "tests/test_gpu_fullsize.py",
          "tests/test_zz_no_alloc.py"]

CHILD = r"""
import os, sys
import pytest
import decoder_attention_amd as ga
lib = ga.load()
want = os.environ["GEMMA_ATTN_LIBRARY"]
if os.path.realpath(lib._name) != os.path.realpath(want):
    sys.exit("loaded %s, not the debug build %s" % (lib._name, want))
print("debug build loaded:", lib._name, flush=True)
sys.exit(pytest.main(sys.argv[1:]))
"""


def test_parity_suites_on_lds_poisoned_build(gpu):
    from decoder_attention_amd import build as b

    assert os.path.exists(b.LIB_LDSNAN), "debug build missing: python -m decoder_attention_amd.build"
    env = dict(os.environ, GEMMA_ATTN_LIBRARY=b.LIB_LDSNAN)
    cmd = [sys.executable, "-u", "-c", CHILD, *SUITES, "-m", "gpu", "-x", "-q", "-p", "no:cacheprovider",
           "--timeout", "300", "--timeout-method", "thread"]
    print("running the parity suites on", b.LIB_LDSNAN, flush=True)
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1400)
    print(r.stdout[-3000:])
    assert r.returncode == 0, r.stdout[-6000:] + r.stderr[-3000:]
    assert "debug build loaded" in r.stdout
    assert " passed" in r.stdout and " failed" not in r.stdout
