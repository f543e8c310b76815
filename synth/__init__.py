"""Seeded synthetic inputs for the Gemma attention block.

This module is shared by the tests, the benchmark and the smoke check.  It only
draws numbers and rounds them to bf16; it holds none of the attention
arithmetic (no norm, no rotary, no softmax), so neither the oracle nor the HIP
path depends on the other through it.

Every tensor is generated on the host with numpy's PCG64 ``default_rng``:
standard normals in float32, rounded to bf16 with round-to-nearest-even, and
handed out as raw bf16 bit patterns (``uint16``).  Large tensors are drawn in
independent per-row streams (one seed per outer index) so that they can be
generated in parallel and so that a single row can be regenerated cheaply.

Seeds follow one rule: ``seed = 1000*config + 10*layer + tensor`` with tensor
ids q 0, k 1, v 2, q-norm weight 3, k-norm weight 4, context lengths 5.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "q_norm_w": 3, "k_norm_w": 4, "ctx": 5}

#: bf16 quiet-NaN bit pattern used to poison cache rows a kernel must not read.
BF16_NAN = np.uint16(0x7FC0)


def seed_for(config: int, layer: int, tensor: str) -> int:
    return 1000 * int(config) + 10 * int(layer) + TENSOR_IDS[tensor]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = BF16_NAN
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return bf16_bits_to_f32(b).astype(np.float64)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16(seed: int, shape, scale: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """N(mean, scale^2) float32 draws rounded to bf16, returned as uint16 bits.

    The leading axis is drawn in independent streams (``SeedSequence([seed, i])``)
    so that row ``i`` can be regenerated on its own by :func:`normal_bf16_row`.
    """
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint16)
    if out.size == 0:
        return out
    lead = shape[0]

    def fill(i: int) -> None:
        out[i] = normal_bf16_row(seed, i, shape[1:], scale, mean)

    if out.size >= (1 << 22) and lead > 1:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(lead)))
    else:
        for i in range(lead):
            fill(i)
    return out


def normal_bf16_row(seed: int, row: int, shape, scale: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """Row ``row`` of :func:`normal_bf16` (same bits), shaped ``shape``."""
    rng = np.random.default_rng(np.random.SeedSequence([int(seed), int(row)]))
    x = rng.standard_normal(tuple(shape), dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    if mean != 0.0:
        x += np.float32(mean)
    return f32_to_bf16_bits(x)


def norm_weight(seed: int, dim: int, mean: float = 1.0, std: float = 0.1) -> np.ndarray:
    """RMSNorm weight vector ~ N(mean, std^2), float32 (not rounded to bf16)."""
    rng = np.random.default_rng(int(seed))
    return (rng.standard_normal(int(dim)) * std + mean).astype(np.float32)


def ctx_lengths(seed: int, batch: int, lo: int = 512, hi: int = 65536) -> np.ndarray:
    """Per-sequence context lengths drawn uniformly from the integers [lo, hi]."""
    rng = np.random.default_rng(int(seed))
    return rng.integers(lo, hi, size=int(batch), endpoint=True).astype(np.int32)
