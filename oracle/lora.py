"""The gated low-rank delta of Residual ISD (R-ISD), in float64.

[hotdry] "Token 生成的核心参数与验收机制" and the [project] R-ISD card: a
rank-128 LoRA adapter is active at the MASK positions only, while the
verifying (CLEAN) positions use the base weights.  For one adapted projection
with base output Y:

    Y'[m, :] = Y[m, :] + scale * (X[m, :] @ A) @ B   if row m is a MASK row
    Y'[m, :] = Y[m, :]                                otherwise

The pages state neither alpha nor the scale; scale = 1 is the reading used.
"""

from __future__ import annotations

import numpy as np


def gated_lora_delta(x, a, b, y, mask_rows, scale: float = 1.0) -> np.ndarray:
    """Return Y' [rows, d_out] float64; x: [rows, d_in], a: [d_in, r], b: [r, d_out]."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(y, dtype=np.float64, copy=True)
    gate = np.zeros(x.shape[0], dtype=np.float64)
    gate[np.asarray(mask_rows, dtype=np.int64)] = 1.0
    delta = (x @ np.asarray(a, dtype=np.float64)) @ np.asarray(b, dtype=np.float64)
    return out + scale * gate[:, None] * delta
