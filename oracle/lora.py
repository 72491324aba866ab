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


def gated_projection(x, w, a, b, mask_rows, scale: float = 1.0) -> np.ndarray:
    """One projection of an R-ISD layer, in float64: base weights on every row, the
    adapter added on the MASK rows only ([hotdry] "Token 生成的核心参数与验收机制";
    [project] R-ISD card):

        out[m, :] = x[m, :] @ w + gate[m] * scale * (x[m, :] @ a) @ b

    x: [rows, d_in], w: [d_in, d_out], a: [d_in, r], b: [r, d_out].  With a and b
    None the projection is the base one.  A CLEAN row (gate 0) gets exactly x @ w.
    """
    x = np.asarray(x, dtype=np.float64)
    base = x @ np.asarray(w, dtype=np.float64)
    if a is None:
        return base
    return gated_lora_delta(x, a, b, base, mask_rows, scale)
