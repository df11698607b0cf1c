"""Residual add + RMSNorm, the step just before the MoE layer, in fp64.
TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (page titles abbreviated):

* [Qwen3] "Qwen3-MoE low-latency inference on Atlas A3 / 950 clusters",
  prefill section "fused-operator optimisation": residual add, RMSNorm and
  dynamic MXFP8 quantisation fused into one pass ("fused RMSNorm + MX
  quant"); and "fused RMSNorm + Cast": the norm before the MoE block returns
  the normalised hidden states both in FP32 (for the gate) and in BF16 (for
  the experts), together with the updated residual.
* [Notes] "LLM inference optimisation study note", section 2 ("Add and
  RMSNorm"): z = x + r, then y_i = z_i / sqrt((1/d) sum_j z_j^2 + eps) * w_i.

Readings where the pages are silent (also listed in the design notes):

* the updated residual is z itself, stored in the hidden-state dtype (bf16);
  the normalisation works on the unrounded sum z;
* without a residual (first layer) z = x;
* outputs: y in fp32 (gate), y rounded to bf16 (experts), or y quantised to
  MXFP8 by the block rule of ``mx.mxfp8_quantize``.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

F64 = np.float64


def add_rmsnorm(x, residual: Optional[np.ndarray], weight, eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """z = x + residual (x alone when residual is None); per row,
    y = z / sqrt(mean(z^2) + eps) * weight.  x, residual: [T, H]; weight: [H].
    Returns (z, y), both fp64."""
    z = np.asarray(x, dtype=F64)
    if residual is not None:
        z = z + np.asarray(residual, dtype=F64)
    w = np.asarray(weight, dtype=F64)
    d = z.shape[-1]
    mean_sq = np.sum(z * z, axis=-1) / d
    y = z / np.sqrt(mean_sq + float(eps))[..., None] * w
    return z, y
