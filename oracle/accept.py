"""The p/q acceptance test and residual resampling of one ISD stride, in float64.

The steps, in the order the pages give them ([hypho] "Introspective Strided
Decoding（ISD）": MASK rows propose from q, clean rows verify with the anchor p,
accept or reject by min(1, p(x)/q(x)); [hotdry] "从质量差距到自省机制": MASK
positions propose with q, CLEAN positions verify with p, acceptance
min(1, p(x)/q(x)); [project] caption on geometric acceptance: position 1 is
always accepted because of the logit shift):

1. Row layout (logit shift, [hypho] "三项关键训练创新", item 2: the hidden
   state at i predicts token i+1).  The stride carries proposals x_1..x_N at
   consecutive positions.  CLEAN row j (0 <= j <= N-2) holds x_{j+1}; its
   logits are the anchor p for x_{j+2}.  Row N-1, the first of the N rows
   that propose, holds x_N; under the logit shift its logits predict the
   token after x_N from an all-clean prefix, i.e. the anchor distribution
   itself, so the next stride's first proposal is drawn from p and needs no
   test ([project] caption on geometric acceptance: position 1 is always
   accepted because of the logit shift).  x_1 was drawn that way by the
   previous pass.  Rows N..2N-2 hold MASK and give q for the next stride's
   positions 2..N; the q logits for x_{j+2} are those the previous pass's
   MASK rows produced, kept by the caller.
2. Normalise every row: lse = max + log(sum exp(l - max)); the log-probability
   of a token is l[x] - lse.
3. For k = 2..N in order: rho_k = p_k(x_k) / q_k(x_k), computed as
   exp(log p - log q); accept iff u_k < rho_k with u_k uniform in [0, 1), so
   rho >= 1 always accepts.  Stop at the first rejection.
   A = 1 + the number of leading accepts (x_1 counts as accepted).
   (One page inverts the two cases in prose; the min(1, p/q) rule that the
   same page and the others state is the one used.)
4. On a rejection at k: draw the committed token from the residual
   r(y) = max(0, p_k(y) - q_k(y)), normalised: S = sum_y r(y), C = the running
   sum of r in vocabulary order, y* = the first y with C(y) > u'_k * S.  The
   pages do not print this step; it is what makes every committed token
   distributed as p (the lossless claim in [project] and [hotdry]).  If S is
   0 in float64 (p and q equal up to rounding) y* is drawn the same way from
   p itself.
5. Committed tokens: x_1..x_A, then y* if A < N.  A row's key and value are
   valid exactly when the token it holds and every token before it are
   accepted, so the KV rows to commit are rows 0..A-1, the accepted prefix
   x_1..x_A: n_commit = A.  y* has no row in this pass; the decoding loop
   (``oracle.loop``) commits it from the row that carries it in the next
   forward.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

from . import philox


def log_normalizer(logits) -> float:
    """lse = m + log(sum(exp(l - m))) of one logit row, float64."""
    l = np.asarray(logits, dtype=np.float64)
    m = float(np.max(l))
    return m + float(np.log(np.sum(np.exp(l - m))))


def residual_cdf(p_row, q_row, lse_p: float, lse_q: float):
    """Running sum of r(y) = max(0, p(y) - q(y)) in vocabulary order; falls back to p if S == 0.

    Returns (C, used_p_fallback).
    """
    p = np.exp(np.asarray(p_row, dtype=np.float64) - lse_p)
    q = np.exp(np.asarray(q_row, dtype=np.float64) - lse_q)
    r = np.maximum(0.0, p - q)
    c = np.cumsum(r)
    if not c[-1] > 0.0:
        return np.cumsum(p), True
    return c, False


def residual_sample(p_row, q_row, u: float, lse_p: Optional[float] = None,
                    lse_q: Optional[float] = None):
    """Inverse-CDF draw from normalize(max(0, p - q)).

    Returns (y, margin, used_p_fallback): margin is the distance from u*S to the
    nearer edge of y's CDF interval, divided by S.
    """
    if lse_p is None:
        lse_p = log_normalizer(p_row)
    if lse_q is None:
        lse_q = log_normalizer(q_row)
    c, fallback = residual_cdf(p_row, q_row, lse_p, lse_q)
    total = c[-1]
    t = u * total
    y = int(np.searchsorted(c, t, side="right"))   # first index with C(y) > t
    y = min(y, len(c) - 1)
    lo = c[y - 1] if y > 0 else 0.0
    margin = min(t - lo, c[y] - t) / total
    return y, margin, fallback


@dataclass
class StrideResult:
    accept_len: int                    # A in [1, N]
    out_tokens: List[int]              # committed tokens (length n_out)
    n_out: int
    n_commit: int                      # stride rows whose KV is committed (= A)
    logp_sel: np.ndarray               # [N-1] log p at the proposals
    logq_sel: np.ndarray               # [N-1] log q at the proposals
    rho: np.ndarray                    # [N-1] p/q at the proposals
    u_accept: np.ndarray               # [N-1] accept uniforms
    decided: int                       # number of accept tests taken (A, or A-1 if all accepted)
    reject_row: int                    # j of the rejected row, or -1
    resample_margin: float = float("inf")
    resample_fallback: bool = False
    accept_margins: np.ndarray = field(default_factory=lambda: np.zeros(0))


def row_normalizers(rows) -> np.ndarray:
    """Step 2 for every row of a [R, V] array."""
    return np.array([log_normalizer(r) for r in np.asarray(rows, dtype=np.float64)])


def verify_stride(p_rows, q_rows, proposals: Sequence[int], uniforms, lse_p=None,
                  lse_q=None) -> StrideResult:
    """Steps 2-5 for one request.

    p_rows, q_rows: [N-1, V] logits; proposals: x_1..x_N; uniforms: list of
    (u_accept, u_resample) for k = 2..N (entry k-2).  lse_p / lse_q may carry
    this module's own ``row_normalizers`` of the rows when they were computed
    before (a large vocabulary decided under many draws).
    """
    p_rows = np.asarray(p_rows, dtype=np.float64)
    q_rows = np.asarray(q_rows, dtype=np.float64)
    n = len(proposals)
    rows = n - 1
    lse_p = row_normalizers(p_rows) if lse_p is None else np.asarray(lse_p, dtype=np.float64)
    lse_q = row_normalizers(q_rows) if lse_q is None else np.asarray(lse_q, dtype=np.float64)
    x = [int(t) for t in proposals]
    logp = np.array([p_rows[j, x[j + 1]] - lse_p[j] for j in range(rows)])
    logq = np.array([q_rows[j, x[j + 1]] - lse_q[j] for j in range(rows)])
    rho = np.exp(logp - logq)
    u_acc = np.array([uniforms[j][0] for j in range(rows)], dtype=np.float64)

    accept_len = 1
    reject_row = -1
    decided = 0
    for k in range(2, n + 1):
        j = k - 2
        decided += 1
        if u_acc[j] < rho[j]:
            accept_len = k
        else:
            reject_row = j
            break

    tokens = x[:accept_len]
    margin, fallback = float("inf"), False
    if reject_row >= 0:
        y, margin, fallback = residual_sample(p_rows[reject_row], q_rows[reject_row],
                                              uniforms[reject_row][1],
                                              lse_p[reject_row], lse_q[reject_row])
        tokens = tokens + [y]
    margins = np.abs(u_acc[:decided] - rho[:decided])
    return StrideResult(accept_len=accept_len, out_tokens=tokens, n_out=len(tokens),
                        n_commit=accept_len, logp_sel=logp, logq_sel=logq,
                        rho=rho, u_accept=u_acc, decided=decided, reject_row=reject_row,
                        resample_margin=margin, resample_fallback=fallback,
                        accept_margins=margins)


def stride_uniforms(seed, req_id: int, position: int, step: int, n: int):
    """Uniforms for k = 2..n of one request; x_k sits at absolute position ``position + k - 1``."""
    return [philox.decision_uniforms(seed, req_id, position + k - 1, step) for k in range(2, n + 1)]


def isd_accept(p_logits, q_logits, proposals, req_ids, positions, seed, step,
               requests: Optional[Sequence[int]] = None, lse_p=None, lse_q=None) -> List[StrideResult]:
    """Run ``verify_stride`` for every request of a batch with Philox draws.

    lse_p / lse_q: optional [B, N-1] row normalisers from ``row_normalizers``.
    """
    B, n = proposals.shape
    reqs = range(B) if requests is None else requests
    out = []
    for r in reqs:
        u = stride_uniforms(seed, int(req_ids[r]), int(positions[r]), int(step), n)
        out.append(verify_stride(p_logits[r], q_logits[r], proposals[r], u,
                                 None if lse_p is None else lse_p[r],
                                 None if lse_q is None else lse_q[r]))
    return out
