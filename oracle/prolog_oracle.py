"""CPU oracle of the indexer prolog: key normalisation with the cache update,
and dynamic query quantisation.

TEST INFRASTRUCTURE ONLY, like the rest of this package.  NumPy; shares
nothing with the HIP library.

The pages place these steps before the index computation ("Day0 Inference
Adaptation and Performance Optimization for Kimi K3.1 Pro", section 3;
"Large Language Model Inference Acceleration in Practice", section 3.2;
"... for a New Model", section 3.2): K normalisation together with writing
the new keys into the cache on one stream, Q quantisation on another, the
projections themselves on a third.  They name the steps only; the readings
used here:
  * K normalisation = LayerNorm over the D_I elements of a key row with
    elementwise gain gamma and bias beta (identity when not given) and a
    stabiliser eps: y = (x - mean) / sqrt(var + eps) * gamma + beta, with the
    biased variance.  Evaluated in float64.
  * The normalised key is stored in the cache's format: bf16 (round to
    nearest even), fp8 with one fp32 scale per token, or MXFP8.
  * fp8 with a per-token scale (queries: one scale per query row over all
    heads; keys: one per key row), decided in fp32 as the kernel does:
    scale = fl32(amax / 448) (1 if amax = 0), element = e4m3(fl32(x / scale))
    with round-to-nearest-even and saturation to +-448.
  * MXFP8: the OCP MX conversion (lisfa_oracle.mx_quantize), exact on any
    float32 input.
"""
from __future__ import annotations

import numpy as np

from .lisfa_oracle import encode_e4m3, mx_quantize


def layer_norm(x: np.ndarray, gamma=None, beta=None, eps: float = 1e-6) -> np.ndarray:
    """LayerNorm of each row of x [..., D] in float64."""
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    y = (x - mean) / np.sqrt(var + eps)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)
    if beta is not None:
        y = y + np.asarray(beta, dtype=np.float64)
    return y


def fp8_token_quantize(x: np.ndarray):
    """Per-row fp8: x [n, m] (float32 values) -> (codes uint8 [n, m], scale
    float32 [n]).  scale = fl32(amax / 448), 1 for an all-zero row;
    codes = e4m3(fl32(x / scale)), round to nearest even, saturating."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.abs(x32).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    y32 = (x32 / scale[..., None]).astype(np.float32)
    return encode_e4m3(y32.astype(np.float64)), scale


def quantize_q(q: np.ndarray, fmt: str):
    """Dynamic quantisation of indexer queries q [R, H_I, D_I] (float32
    values, e.g. decoded bf16): fmt "fp8" -> (codes, scale [R]); "mxfp8" ->
    (codes, E8M0 [R, H_I, D_I / 32])."""
    q = np.asarray(q, dtype=np.float32)
    R = q.shape[0]
    if fmt == "fp8":
        codes, scale = fp8_token_quantize(q.reshape(R, -1))
        return codes.reshape(q.shape), scale
    if fmt == "mxfp8":
        return mx_quantize(q.astype(np.float64))
    raise ValueError(fmt)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 (ties to even), as uint16 bit patterns, via the
    float32 value (float64 -> float32 -> bf16 double rounding only matters
    within 2^-24 relative of a bf16 tie, which the tests allow for)."""
    f = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (f >> np.uint64(16)) & np.uint64(1)
    r = (f + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)
