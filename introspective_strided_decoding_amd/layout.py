"""KV page-pool layouts of libisd (data movement only, torch ops on any device).

Plain layout (what a caller naturally holds): ``pool[page, slot, kv_head, dim]``.
Library layouts (declared in include/isd.h):

* keys:   ``k_pages[page, kv_head, dim // 8, slot, dim % 8]``
* values: ``v_pages[page, kv_head, dim, sigma(slot)]`` with sigma swapping bits
  2 and 3 of the slot index.

The ISD step itself writes new rows with kv_commit; these helpers load or
inspect a whole pool (prefill, tests, benchmarks).
"""

from __future__ import annotations

import torch

PAGE = 16
# sigma: slot -> storage index (swap bits 2 and 3); it is an involution.
SIGMA = [(s & 3) | ((s & 4) << 1) | ((s & 8) >> 1) for s in range(PAGE)]


def pack_k_pages(k_plain: torch.Tensor) -> torch.Tensor:
    P, S, H, D = k_plain.shape
    assert S == PAGE and D % 8 == 0
    return k_plain.reshape(P, S, H, D // 8, 8).permute(0, 2, 3, 1, 4).contiguous()


def unpack_k_pages(k_pages: torch.Tensor) -> torch.Tensor:
    P, H, C, S, E = k_pages.shape
    return k_pages.permute(0, 3, 1, 2, 4).reshape(P, S, H, C * E).contiguous()


def pack_v_pages(v_plain: torch.Tensor) -> torch.Tensor:
    P, S, H, D = v_plain.shape
    assert S == PAGE
    t = v_plain.permute(0, 2, 3, 1)                       # [P, H, D, slot]
    idx = torch.tensor(SIGMA, device=v_plain.device)      # storage i holds slot SIGMA[i]
    return t.index_select(3, idx).contiguous()


def unpack_v_pages(v_pages: torch.Tensor) -> torch.Tensor:
    P, H, D, S = v_pages.shape
    idx = torch.tensor(SIGMA, device=v_pages.device)
    return v_pages.index_select(3, idx).permute(0, 3, 1, 2).contiguous()
