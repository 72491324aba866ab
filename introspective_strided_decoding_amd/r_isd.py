"""The projections of one R-ISD transformer layer, each one isd_gated_linear call.

R-ISD ("自省扩散语言模型的 token 生成机制与工程实践", section "Token 生成的核心参数与验收
机制"; I-DLM project page, R-ISD card) keeps the base weights on the verifying
(CLEAN) rows and adds a rank-128 adapter on the MASK rows of every stride.  A
layer of an 8B-class model has seven projections: q, k, v and o around
attention, gate, up and down in the MLP.  This module holds random-init weights
and adapters of those shapes and issues the seven calls on one stream; the
operations between them (norms, rotary embedding, attention, the SiLU product,
residual adds) are not part of it, so every projection reads an input of its own.
Argument marshalling only: the arithmetic runs in libisd.so.
"""

from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import torch

from . import _lib

RANK = 128


def layer_shapes(hidden: int, kv: int, mlp: int) -> List[Tuple[str, int, int]]:
    """(name, d_in, d_out) of the seven projections of one layer."""
    return [("q", hidden, hidden), ("k", hidden, kv), ("v", hidden, kv), ("o", hidden, hidden),
            ("gate", hidden, mlp), ("up", hidden, mlp), ("down", mlp, hidden)]


def stride_mask_rows(batch: int, stride_n: int) -> List[int]:
    """Row indices of the MASK rows when every request contributes its Q = 2N - 1 stride rows
    in order (rows N-1 .. 2N-2 of each request are MASK rows)."""
    q = 2 * stride_n - 1
    return [r * q + i for r in range(batch) for i in range(stride_n - 1, q)]


class RIsdProjections:
    def __init__(self, rows: int, mask_rows: Sequence[int], hidden: int = 4096, kv: int = 1024,
                 mlp: int = 12288, seed: int = 0, device="cuda", weight_std: float = 0.02):
        self.rows = rows
        self.shapes = layer_shapes(hidden, kv, mlp)
        g = torch.Generator(device=device)
        g.manual_seed(seed)

        def rnd(shape, std):
            return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)

        self.mask = torch.tensor(list(mask_rows), dtype=torch.int32, device=device)
        self.p: Dict[str, dict] = {}
        for name, d_in, d_out in self.shapes:
            n = max(_lib.isd_gated_linear_workspace_bytes(rows, d_in, d_out, RANK, self.mask.numel()),
                    _lib.isd_gated_linear_workspace_bytes(rows, d_in, d_out, 0, 0))
            if n == 0:
                raise ValueError(f"projection {name} ({d_in} -> {d_out}) at {rows} rows is not supported")
            self.p[name] = dict(X=rnd((rows, d_in), 1.0), W_t=rnd((d_out, d_in), weight_std),
                                A_t=rnd((RANK, d_in), weight_std), B_t=rnd((d_out, RANK), weight_std),
                                Y=torch.empty((rows, d_out), dtype=torch.bfloat16, device=device),
                                ws=torch.zeros(n, dtype=torch.uint8, device=device))

    def run(self, gated: bool = True, stream=None) -> None:
        """Enqueue the seven projections; gated=False runs the base weights alone."""
        for name, _, _ in self.shapes:
            t = self.p[name]
            if gated:
                _lib.isd_gated_linear(t["X"], t["W_t"], t["Y"], t["ws"], A_t=t["A_t"], B_t=t["B_t"],
                                      mask_rows=self.mask, stream=stream)
            else:
                _lib.isd_gated_linear(t["X"], t["W_t"], t["Y"], t["ws"], stream=stream)

    def flops(self, gated: bool = True) -> int:
        """Algorithmic flops: the base product on every row, the adapter's two products on the
        gated rows."""
        f = sum(2 * self.rows * d_in * d_out for _, d_in, d_out in self.shapes)
        if gated:
            f += sum(2 * self.mask.numel() * RANK * (d_in + d_out) for _, d_in, d_out in self.shapes)
        return f

    def bytes(self, gated: bool = True) -> int:
        """Algorithmic HBM bytes: weights, inputs and outputs once (+ adapter weights)."""
        b = sum(2 * (d_in * d_out + self.rows * (d_in + d_out)) for _, d_in, d_out in self.shapes)
        if gated:
            b += sum(2 * RANK * (d_in + d_out) for _, d_in, d_out in self.shapes)
        return b
