"""Acceptance and tokens-per-forward (TPF) arithmetic of ISD.

* Geometric acceptance ([project], caption under the stride widget; [hotdry]
  "Token 生成的核心参数与验收机制"): with per-position acceptance rate p,
  position k of a stride survives with probability p^(k-1); position 1 always
  survives (logit shift).  Hence E[accepted] = sum_{k=1..N} p^(k-1).
* TPF ([project], TPF widget: TPF = average tokens per cycle / average
  forwards per cycle).  The pages print TPF for N = 2, 3, 4, 5, 8 at p = 0.9
  ([hotdry] table) but not its formula.  The reading that reproduces every
  printed value: a cycle is one verify forward that keeps A tokens; if a
  proposal is rejected, the resampled token is kept too and one more forward
  is spent proposing again from the corrected prefix.  So
  tokens/cycle = A + [A < N] and forwards/cycle = 1 + [A < N], and
  TPF = (E[A] + 1 - p^(N-1)) / (2 - p^(N-1)).
* Compute-bound identity ([project], derivation steps 1-6): with Q queries per
  forward, total forwards L/TPF, total queries (L/TPF) * Q, overhead
  OH = Q / TPF, and speedup = TPF / OH = TPF^2 / Q.
"""

from __future__ import annotations

from dataclasses import dataclass


def prob_position_kept(k: int, p: float) -> float:
    """Probability that position k (1-based) of a stride is accepted."""
    if k < 1:
        raise ValueError("positions are 1-based")
    return p ** (k - 1)


def expected_accepted(n: int, p: float) -> float:
    """E[A] = sum_{k=1..n} p^(k-1)."""
    return sum(prob_position_kept(k, p) for k in range(1, n + 1))


def tpf_closed_form(n: int, p: float) -> float:
    """Tokens per forward of the ISD loop under the reject-costs-a-forward reading."""
    p_reject = 1.0 - p ** (n - 1)
    return (expected_accepted(n, p) + p_reject) / (1.0 + p_reject)


def queries_per_forward(n: int) -> int:
    """Q = 2N - 1: N-1 CLEAN rows verifying and N MASK rows proposing."""
    return 2 * n - 1


@dataclass
class LoopCounts:
    cycles: int = 0
    forwards: int = 0
    tokens: int = 0
    accepted: int = 0

    def add_cycle(self, accept_len: int, n: int) -> None:
        rejected = accept_len < n
        self.cycles += 1
        self.accepted += accept_len
        self.tokens += accept_len + (1 if rejected else 0)
        self.forwards += 1 + (1 if rejected else 0)

    @property
    def tpf(self) -> float:
        return self.tokens / self.forwards


def total_forwards(tokens: float, tpf: float) -> float:
    """Step 1 of the derivation: forwards needed for ``tokens`` outputs."""
    return tokens / tpf


def total_queries(tokens: float, tpf: float, q: int) -> float:
    """Step 2: every forward carries Q queries."""
    return total_forwards(tokens, tpf) * q


def overhead(tokens: float, tpf: float, q: int) -> float:
    """Step 4: method queries over AR queries (AR spends one query per token)."""
    return total_queries(tokens, tpf, q) / tokens


def compute_bound_speedup(tpf: float, q: int) -> float:
    """Step 5: speedup = TPF / OH = TPF^2 / Q."""
    return tpf * tpf / q
