"""Proposing the next N tokens at the MASK rows of one ISD stride, in float64.

TEST INFRASTRUCTURE ONLY (see the package header).

What the pages state: every forward pass draws N new tokens at the MASK
positions from the proposal distribution q while the CLEAN positions verify
([hypho] "Introspective Strided Decoding（ISD）", first step of the core loop;
[hotdry] "从质量差距到自省机制": MASK positions propose by q).  [hotdry]
"服务部署与 SGLang 集成" lists an argmax proposal policy among the serving
optimisations.

The steps, for MASK row k = 0..N-1 of request r:

1. q_k = softmax of the row's logits, float64: q(y) = exp(l_y - lse) with
   lse = max + log(sum exp(l - max)) (the same normaliser as the accept test).
2. Sampling policy: C = the running sum of q_k in vocabulary order and
   x'_k = the first y with C(y) > u_k * C(V-1) (inverse-CDF sampling; the
   uniform is scaled by the float64 total so rounding of the normaliser cannot
   move u_k past the end).
   Argmax policy: x'_k = the smallest index of the largest logit.

Readings (the pages do not print these):

* Positions: x_1 sits at ``position``, so the stride's proposals end at
  ``position + N - 1``; under the logit shift MASK row k predicts the token at
  absolute position ``position + N + k``.
* Uniforms: word 0 of the Philox4x64-10 block with counter
  ``(request id, position + N + k, step, 1)``.  Counter word 3 = 1 keeps the
  proposal stream apart from the decision stream (word 3 = 0), which uses the
  same (request, position, step) triples in a later step.
"""

from __future__ import annotations

from typing import List, Sequence

import numpy as np

from . import philox

SAMPLE = 0
ARGMAX = 1


def proposal_counter(req_id: int, position: int, step: int):
    """Counter block of the proposal drawn for absolute ``position`` of ``req_id``."""
    if req_id < 0 or position < 0 or step < 0:
        raise ValueError("request id, position and step must be non-negative")
    return (req_id, position, step, 1)


def proposal_uniform(seed, req_id: int, position: int, step: int) -> float:
    """u for the proposal at absolute ``position`` (word 0 of its block)."""
    return philox.unit_double(philox.philox4x64(proposal_counter(req_id, position, step), seed)[0])


def stride_proposal_uniforms(seed, req_id: int, position: int, step: int, n: int) -> List[float]:
    """u_0..u_{N-1} for the MASK rows of one request (x_1 at ``position``)."""
    return [proposal_uniform(seed, req_id, position + n + k, step) for k in range(n)]


def sample_row(logits, u: float):
    """Step 2, sampling policy, for one row.

    Returns (y, margin): margin is the distance from u * total to the nearer
    edge of y's CDF interval, divided by the total.
    """
    l = np.asarray(logits, dtype=np.float64)
    m = float(np.max(l))
    q = np.exp(l - (m + float(np.log(np.sum(np.exp(l - m))))))
    c = np.cumsum(q)
    total = c[-1]
    t = u * total
    y = int(np.searchsorted(c, t, side="right"))    # first y with C(y) > t
    y = min(y, len(c) - 1)
    lo = c[y - 1] if y > 0 else 0.0
    return y, min(t - lo, c[y] - t) / total


def argmax_row(logits) -> int:
    """Step 2, argmax policy: the smallest index holding the largest logit."""
    l = np.asarray(logits, dtype=np.float64)
    return int(np.flatnonzero(l == np.max(l))[0])


def propose_stride(mask_rows, uniforms: Sequence[float], mode: int = SAMPLE):
    """Proposals x'_1..x'_N of one request from its N MASK-row logit rows.

    Returns (tokens, margins); margins are +inf under the argmax policy.
    """
    rows = np.asarray(mask_rows, dtype=np.float64)
    tokens, margins = [], []
    for k in range(rows.shape[0]):
        if mode == ARGMAX:
            tokens.append(argmax_row(rows[k]))
            margins.append(float("inf"))
        else:
            y, mg = sample_row(rows[k], uniforms[k])
            tokens.append(y)
            margins.append(mg)
    return tokens, np.array(margins)


def isd_propose(mask_logits, req_ids, positions, seed, step, mode: int = SAMPLE, requests=None):
    """``propose_stride`` for every request of a [B, N, V] batch with Philox draws.

    Returns (tokens [B', N] int, margins [B', N]) for the requests listed
    (all by default).
    """
    mask_logits = np.asarray(mask_logits)
    B, n, _ = mask_logits.shape
    reqs = range(B) if requests is None else requests
    toks, mgs = [], []
    for r in reqs:
        u = stride_proposal_uniforms(seed, int(req_ids[r]), int(positions[r]), int(step), n)
        t, mg = propose_stride(mask_logits[r], u, mode)
        toks.append(t)
        mgs.append(mg)
    return np.array(toks, dtype=np.int64), np.array(mgs)
