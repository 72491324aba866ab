"""Committing the accepted prefix of a stride to the KV pages.

TEST INFRASTRUCTURE ONLY (see the package header).

The KV cache is paged as in the AR serving stack I-DLM reuses ([hypho]
"推理：复用 AR 推理栈"; [hotdry] "服务部署与 SGLang 集成").  Stride row i of
request r holds a token at absolute position L_r + i; a row's key/value is
valid exactly when its token and every token before it were accepted, so
after the accept test the rows holding the accepted prefix x_1..x_A are
appended (n_commit = A, ``oracle.accept``).  In general n rows starting at
stride row f are appended: row f + i goes to absolute position L_r + i, i.e.
page ``table[r, (L_r + i) // page_size]``, slot ``(L_r + i) % page_size``,
and the context length grows by n.  f = 0 for a verifying forward; the
decoding loop's re-proposing forward commits the one row that carries the
token resampled the forward before (``oracle.loop``).
"""

from __future__ import annotations

import numpy as np


def kv_commit(k_pool, v_pool, page_table, ctx_lens, k_new, v_new, n_commit, page_size: int,
              first_row=None):
    """Return (k_pool', v_pool', ctx_lens') after appending the committed rows (inputs untouched).

    first_row: [B] stride row of each request's first committed row (None: 0 for all).
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    lens = np.array(ctx_lens, copy=True)
    for r in range(len(ctx_lens)):
        L = int(ctx_lens[r])
        f = 0 if first_row is None else int(first_row[r])
        for i in range(int(n_commit[r])):
            pos = L + i
            page = int(page_table[r, pos // page_size])
            if page < 0 or page >= k_out.shape[0]:
                raise IndexError(f"request {r}: no page mapped for position {pos}")
            k_out[page, pos % page_size] = k_new[r, f + i]
            v_out[page, pos % page_size] = v_new[r, f + i]
        lens[r] = L + int(n_commit[r])
    return k_out, v_out, lens
