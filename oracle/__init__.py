"""fp64 CPU oracle for the Gemma-family decoder attention block.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) may import, call, link or execute anything in this package.
It is used by ``tests/``, by the benchmark's CPU-baseline leg and by the smoke
check, and nowhere else.

``gemma_ref`` is the plain definition of what the block computes (numpy, fp64,
no tiling, no online softmax).  ``brute`` is an independent scalar twin in pure
Python used to pin ``gemma_ref`` on tiny inputs.  The two share no code.

Sources (web pages on the Gemma model family):
  * "Gemma 4" (KerasFormers): sections "What changed from Gemma 3" and the
    ``Gemma4Model`` argument table;
  * "Gemma" (KerasFormers): introduction and the ``GemmaModel`` table;
  * "Gemma 2" (ZeroModels): introduction bullets and the ``Gemma2Model`` table;
  * "Gemma 3" (KerasFormers): "What changed from Gemma 2" and the
    ``Gemma3Model`` table;
  * "google-gemma-4" (atlas architecture summary): summary paragraph and the
    "Training" section.

Every function that follows a reading of an ambiguous passage says so in its
docstring.  Fidelity to released checkpoints is parity unpinned: the pages
print no activations, so the readings below (window boundary, which layer is
global, query scaling, partial-rotary layout, rotary pairing, keys-as-values
source, GQA grouping, decode position) are pinned only against the mathematics
and against the pages' own configuration tables.
"""
from .gemma_ref import (  # noqa: F401
    GemmaAttnConfig,
    resolve_layer,
    rms_norm,
    rotary,
    rotary_zero_pad,
    ROTARY_LAYOUTS,
    rotary_inv_freq,
    round_bf16,
    softcap,
    allowed,
    prologue,
    prefill,
    prefill_rows,
    prefill_ragged,
    decode,
    decode_multi,
    quantize_int8,
    dequantize_int8,
    decode_int8,
    prefill_flops,
    decode_kv_bytes,
)
