"""Committing the accepted prefix of a stride to the KV pages.

The KV cache is paged as in the AR serving stack I-DLM reuses ([hypho]
"推理：复用 AR 推理栈"; [hotdry] "服务部署与 SGLang 集成").  A CLEAN row's
key/value is valid exactly when the token it holds is accepted, so after the
accept test the first n_commit = min(A, N-1) CLEAN rows of the stride are
appended: row i goes to absolute position L_r + i, i.e. page
``table[r, (L_r + i) // page_size]``, slot ``(L_r + i) % page_size``, and the
context length grows by n_commit.
"""

from __future__ import annotations

import numpy as np


def kv_commit(k_pool, v_pool, page_table, ctx_lens, k_new, v_new, n_commit, page_size: int):
    """Return (k_pool', v_pool', ctx_lens') after appending the committed rows (inputs untouched)."""
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    lens = np.array(ctx_lens, copy=True)
    for r in range(len(ctx_lens)):
        L = int(ctx_lens[r])
        for i in range(int(n_commit[r])):
            pos = L + i
            page = int(page_table[r, pos // page_size])
            if page < 0 or page >= k_out.shape[0]:
                raise IndexError(f"request {r}: no page mapped for position {pos}")
            k_out[page, pos % page_size] = k_new[r, i]
            v_out[page, pos % page_size] = v_new[r, i]
        lens[r] = L + int(n_commit[r])
    return k_out, v_out, lens
