"""Strictly causal stride attention over a paged KV cache, in float64.

What it computes ([hypho] "三项关键训练创新", item 1: one causal mask over
MASK and clean tokens, each position sees only its left context; [project],
ISD card: one forward both verifies earlier proposals and proposes new ones;
[hotdry] "Token 生成的核心参数与验收机制": 2N-1 query positions per forward):

For request r with L_r cached positions, stride row i (0 <= i < Q = 2N-1) sits
at absolute position L_r + i.  Query head h reads KV head h // G
(G = Hq / Hkv, grouped-query attention).  Row i attends to

* every cached position 0 .. L_r-1, read from the page pool through the
  request's page table (position t lives in page ``table[r, t // page_size]``,
  slot ``t % page_size``), and
* the stride's own rows 0 .. i (their keys and values come from this pass,
  ``k_new`` / ``v_new``), never to rows after i.

out[r, i, h] = sum_t softmax_t(q . k_t * scale) v_t, with scale = 1/sqrt(D)
(the pages name no scale; this is the usual one).

Plain pool layout used by the oracle: ``pool[page, slot, kv_head, dim]``.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional

import numpy as np


def gather_context(pool: np.ndarray, table_row: np.ndarray, length: int, page_size: int) -> np.ndarray:
    """Logical context [length, Hkv, D] of one request, read page by page."""
    out = np.empty((length,) + pool.shape[2:], dtype=np.float64)
    for t in range(0, length, page_size):
        n = min(page_size, length - t)
        page = int(table_row[t // page_size])
        if page < 0 or page >= pool.shape[0]:
            raise IndexError(f"page table entry {page} out of range for position {t}")
        out[t:t + n] = pool[page, :n]
    return out


def stride_attention(q, k_new, v_new, k_pool, v_pool, page_table, ctx_lens, page_size: int,
                     scale: Optional[float] = None, requests: Optional[Iterable[int]] = None) -> np.ndarray:
    """Attention output [len(requests), Q, Hq, D] in float64.

    q: [B, Q, Hq, D]; k_new, v_new: [B, Q, Hkv, D]; pools: [P, page_size, Hkv, D];
    page_table: [B, max_pages]; ctx_lens: [B].
    """
    B, Q, Hq, D = q.shape
    Hkv = k_new.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    reqs = list(range(B)) if requests is None else list(requests)
    out = np.empty((len(reqs), Q, Hq, D), dtype=np.float64)
    for n, r in enumerate(reqs):
        L = int(ctx_lens[r])
        keys = np.concatenate([gather_context(k_pool, page_table[r], L, page_size),
                               k_new[r].astype(np.float64)], axis=0)        # [L+Q, Hkv, D]
        vals = np.concatenate([gather_context(v_pool, page_table[r], L, page_size),
                               v_new[r].astype(np.float64)], axis=0)
        T = L + Q
        # row i may see keys t <= L + i
        visible = np.arange(T)[None, :] <= (L + np.arange(Q))[:, None]      # [Q, T]
        for h in range(Hq):
            kv = h // G
            s = (q[r, :, h, :].astype(np.float64) @ keys[:, kv, :].T) * scale  # [Q, T]
            s = np.where(visible, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            w = np.exp(s)
            w /= w.sum(axis=1, keepdims=True)
            out[n, :, h, :] = w @ vals[:, kv, :]
    return out
