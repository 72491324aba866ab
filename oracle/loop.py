"""The multi-step ISD decoding loop on a stationary batch, in plain Python.

TEST INFRASTRUCTURE ONLY (see the package header).

What the pages fix: every forward verifies the previous proposals and proposes
N new ones ([hypho] "Introspective Strided Decoding（ISD）"); each request
advances on its own, with no batch synchronisation ([project], caption on SDAR
synchronisation); the TPF column of [hotdry] "Token 生成的核心参数与验收机制"
is reproduced by a cycle that keeps A + [A < N] tokens and spends 1 + [A < N]
forwards (``oracle.tpf``): after a rejection one more forward proposes again
from the corrected prefix.

The loop, per request (the reading taken where the pages are silent):

* state: mode (VERIFY or REPROPOSE), the stride's proposals x_1..x_N, ``pos``
  (the ``positions`` value the next forward is called with: the absolute
  position of the stride's first row, which is also the context length its
  attention reads), committed tokens and forwards so far;
* one forward of the batch = the accept test on the current proposals, then
  N proposals from the proposing rows (both with Philox draws at this
  forward's step), then ``advance``:

  - VERIFY, A = N: tokens += N; the forward's proposals become the next
    stride; pos += N (x_1 of the next stride is the token after x_N).
  - VERIFY, A < N: tokens += A + 1 (x_1..x_A and the resampled token y*); the
    proposals followed a rejected prefix and are dropped; mode becomes
    REPROPOSE and pos += A + 1 - N, so that the re-proposing forward's row
    N-1 (the first proposing row) sits at y*'s position and carries y*: its
    logit-shifted output is the anchor distribution of the token after y*,
    and its proposing rows k = 0..N-1 propose the tokens at (old pos) + A + 1
    + k under the proposal positions of ``oracle.propose``.
  - REPROPOSE: its accept result is ignored; its proposals become the next
    stride; mode becomes VERIFY and pos += N.
  - forwards += 1 in every case.

* KV rows committed by a forward (``advance`` returns them as a count and the
  stride row of the first one; ``oracle.commit`` writes row f + i at context
  position ctx + i):

  - VERIFY: rows 0..A-1, the accepted prefix x_1..x_A (A rows; when A = N the
    last of them is row N-1, which carries x_N);
  - REPROPOSE: row N-1 only, which carries y* (one row).  Its other rows sit
    at positions already committed and are not written again.

  So every committed token's key and value are written exactly once, at its
  own position, and between forwards the context length ctx satisfies
  ctx = pos in VERIFY mode and ctx = pos + N - 1 in REPROPOSE mode (y* is
  the one committed token whose row is still to come), i.e.
  ctx - ctx_0 = tokens - [mode == REPROPOSE].  A forward's attention reads
  ``pos`` cached positions.  (The loop needs ctx_0 >= N - 1 so that a
  re-proposing stride starts at a position >= 0.)
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import accept, propose

VERIFY = 0
REPROPOSE = 1


@dataclass
class LoopState:
    mode: np.ndarray          # [B] VERIFY / REPROPOSE
    proposals: np.ndarray     # [B, N] the stride's x_1..x_N
    pos: np.ndarray           # [B] positions argument of the next forward
    tokens: np.ndarray        # [B] committed tokens so far
    forwards: np.ndarray      # [B] forwards so far

    @classmethod
    def start(cls, proposals, positions):
        proposals = np.array(proposals, dtype=np.int64)
        B = proposals.shape[0]
        return cls(mode=np.full(B, VERIFY, dtype=np.int64), proposals=proposals,
                   pos=np.array(positions, dtype=np.int64), tokens=np.zeros(B, dtype=np.int64),
                   forwards=np.zeros(B, dtype=np.int64))

    def copy(self):
        return LoopState(self.mode.copy(), self.proposals.copy(), self.pos.copy(), self.tokens.copy(),
                         self.forwards.copy())


def advance(state: LoopState, accept_len, n_out, next_proposals):
    """Apply one forward's results to every request.

    Returns (n_commit [B], first_row [B]): the KV rows this forward commits,
    as a count and the stride row of the first one (``oracle.commit``).
    """
    B, n = state.proposals.shape
    n_commit = np.zeros(B, dtype=np.int64)
    first_row = np.zeros(B, dtype=np.int64)
    for r in range(B):
        state.forwards[r] += 1
        if state.mode[r] == VERIFY:
            a = int(accept_len[r])
            state.tokens[r] += int(n_out[r])
            n_commit[r] = a
            if a == n:
                state.proposals[r] = next_proposals[r]
                state.pos[r] += n
            else:
                state.mode[r] = REPROPOSE
                state.pos[r] += int(n_out[r]) - n
        else:
            n_commit[r] = 1
            first_row[r] = n - 1
            state.proposals[r] = next_proposals[r]
            state.mode[r] = VERIFY
            state.pos[r] += n
    return n_commit, first_row


def forward(state: LoopState, p_logits, q_logits, mask_logits, req_ids, seed, step: int,
            lse_p=None, lse_q=None):
    """One forward of the batch on the oracle: accept, proposals, advance.

    Returns (accept results, proposal margins [B, N], n_commit [B], first_row [B]).
    """
    res = accept.isd_accept(p_logits, q_logits, state.proposals, req_ids, state.pos, seed, step,
                            lse_p=lse_p, lse_q=lse_q)
    nxt, margins = propose.isd_propose(mask_logits, req_ids, state.pos, seed, step)
    n_commit, first_row = advance(state, [o.accept_len for o in res], [o.n_out for o in res], nxt)
    return res, margins, n_commit, first_row
