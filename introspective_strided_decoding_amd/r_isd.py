"""The projections of one R-ISD transformer layer: one isd_gated_linear_group call per
group of projections that share an input, or one isd_gated_linear call per projection.

R-ISD ("自省扩散语言模型的 token 生成机制与工程实践", section "Token 生成的核心参数与验收
机制"; I-DLM project page, R-ISD card) keeps the base weights on the verifying
(CLEAN) rows and adds a rank-128 adapter on the MASK rows of every stride.  A
layer of an 8B-class model has seven projections: q, k, v and o around
attention, gate, up and down in the MLP.  This module holds random-init weights
and adapters of those shapes and issues the seven calls; the operations between
them (norms, rotary embedding, attention, the SiLU product, residual adds) are
not part of it, so each group of projections that shares an input in a real
layer (q/k/v, gate/up) reads a synthetic input of its own, and so do o and down.
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


# Projections that read the same input (the normed hidden state for q, k and v; the normed
# attention-block output for gate and up) and so may run side by side; o and down each
# read the output of the step before them.
GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))


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
        dims = {name: (d_in, d_out) for name, d_in, d_out in self.shapes}
        self.p: Dict[str, dict] = {}
        for group in GROUPS:
            X = rnd((rows, dims[group[0]][0]), 1.0)          # one input per group
            for name in group:
                d_in, d_out = dims[name]
                n = max(_lib.isd_gated_linear_workspace_bytes(rows, d_in, d_out, RANK, self.mask.numel()),
                        _lib.isd_gated_linear_workspace_bytes(rows, d_in, d_out, 0, 0))
                if n == 0:
                    raise ValueError(f"projection {name} ({d_in} -> {d_out}) at {rows} rows is not supported")
                self.p[name] = dict(X=X, W_t=rnd((d_out, d_in), weight_std),
                                    A_t=rnd((RANK, d_in), weight_std), B_t=rnd((d_out, RANK), weight_std),
                                    Y=torch.empty((rows, d_out), dtype=torch.bfloat16, device=device),
                                    ws=torch.zeros(n, dtype=torch.uint8, device=device))
        self.group_ws: Dict[Tuple[str, ...], torch.Tensor] = {}
        for group in GROUPS:
            d_in, d_outs = dims[group[0]][0], [dims[name][1] for name in group]
            n = max(_lib.isd_gated_linear_group_workspace_bytes(rows, d_in, d_outs, RANK, self.mask.numel()),
                    _lib.isd_gated_linear_group_workspace_bytes(rows, d_in, d_outs, 0, 0))
            if n == 0:
                raise ValueError(f"group {group} at {rows} rows is not supported")
            self.group_ws[group] = torch.zeros(n, dtype=torch.uint8, device=device)
        self._side = torch.cuda.Stream(device=device)      # default priority

    def _one(self, name: str, gated: bool, stream) -> None:
        t = self.p[name]
        if gated:
            _lib.isd_gated_linear(t["X"], t["W_t"], t["Y"], t["ws"], A_t=t["A_t"], B_t=t["B_t"],
                                  mask_rows=self.mask, stream=stream)
        else:
            _lib.isd_gated_linear(t["X"], t["W_t"], t["Y"], t["ws"], stream=stream)

    def _group(self, group: Tuple[str, ...], gated: bool, stream) -> None:
        ts = [self.p[name] for name in group]
        X = ts[0]["X"]
        Ws, Ys = [t["W_t"] for t in ts], [t["Y"] for t in ts]
        if gated:
            _lib.isd_gated_linear_group(X, Ws, Ys, self.group_ws[group], A_ts=[t["A_t"] for t in ts],
                                        B_ts=[t["B_t"] for t in ts], mask_rows=self.mask, stream=stream)
        else:
            _lib.isd_gated_linear_group(X, Ws, Ys, self.group_ws[group], stream=stream)

    def run(self, gated: bool = True, mode: str = "group") -> None:
        """Enqueue the seven projections on the current stream; gated=False runs the base
        weights alone.  mode "group": one group call per set of projections sharing an
        input (q/k/v, o, gate/up, down).  mode "overlap": one call per projection, the
        second projection of a group on a side stream (forked from and joined back into the
        current stream by events), so one projection's latency-bound adapter kernels run
        under its sibling's product.  mode "sequential": one call per projection, in order.
        Every projection has its own output and every call its own workspace, so calls in
        flight together share no buffer they write."""
        if mode not in ("group", "overlap", "sequential"):
            raise ValueError(f"unknown mode {mode!r}")
        main = torch.cuda.current_stream()
        for group in GROUPS:
            if mode == "group":
                self._group(group, gated, main)
                continue
            if mode == "sequential" or len(group) == 1:
                for name in group:
                    self._one(name, gated, main)
                continue
            fork = torch.cuda.Event()
            fork.record(main)
            self._side.wait_event(fork)
            for i, name in enumerate(group):
                self._one(name, gated, self._side if i % 2 else main)
            join = torch.cuda.Event()
            join.record(self._side)
            main.wait_event(join)

    def flops(self, gated: bool = True) -> int:
        """Algorithmic flops: the base product on every row, the adapter's two products on the
        gated rows."""
        f = sum(2 * self.rows * d_in * d_out for _, d_in, d_out in self.shapes)
        if gated:
            f += sum(2 * self.mask.numel() * RANK * (d_in + d_out) for _, d_in, d_out in self.shapes)
        return f

    def bytes(self, gated: bool = True) -> int:
        """Algorithmic HBM bytes: every weight, each group's input and every output once
        (+ adapter weights)."""
        b = sum(2 * (d_in * d_out + self.rows * d_out) for _, d_in, d_out in self.shapes)
        dims = {name: d_in for name, d_in, _ in self.shapes}
        b += sum(2 * self.rows * dims[group[0]] for group in GROUPS)
        if gated:
            b += sum(2 * RANK * (d_in + d_out) for _, d_in, d_out in self.shapes)
        return b
