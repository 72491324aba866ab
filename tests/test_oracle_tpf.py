"""Pins for oracle.tpf against the values the pages print.

* tests/golden/isd_acceptance_table.json: the E[acc] / TPF table of
  "自省扩散语言模型的 token 生成机制与工程实践", section "Token 生成的核心参数与验收机制".
* The same section: N = 4, p = 0.90 gives about 7 queries and TPF about 2.9;
  N = 8 gives TPF above 4.0.
* The compute-bound identity of the I-DLM project page (derivation steps 1-6):
  speedup = TPF / OH = TPF^2 / Q, checked on a simulated decoding loop driven
  by the oracle's own accept test.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import tpf
from oracle.accept import verify_stride

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "isd_acceptance_table.json")


def _table():
    with open(GOLDEN) as f:
        return json.load(f)


def test_expected_accepted_reproduces_printed_column():
    t = _table()
    p = t["acceptance_rate"]
    for row in t["rows"]:
        assert round(tpf.expected_accepted(row["N"], p), 2) == pytest.approx(row["E_acc"], abs=1e-9)


def test_tpf_reproduces_printed_column():
    t = _table()
    p = t["acceptance_rate"]
    for row in t["rows"]:
        assert round(tpf.tpf_closed_form(row["N"], p), 2) == pytest.approx(row["TPF"], abs=1e-9)


def test_stated_n4_and_n8_facts():
    assert tpf.queries_per_forward(4) == _table()["also_stated"]["queries_per_forward_at_N4"]
    assert abs(tpf.tpf_closed_form(4, 0.9) - 2.9) < 0.05
    assert tpf.tpf_closed_form(8, 0.9) > 4.0


def test_e_acc_exact_values():
    assert tpf.expected_accepted(2, 0.9) == pytest.approx(1.9, abs=1e-15)
    assert tpf.expected_accepted(4, 0.9) == pytest.approx(3.439, abs=1e-15)
    assert tpf.expected_accepted(8, 0.9) == pytest.approx((1 - 0.9 ** 8) / 0.1, abs=1e-13)
    assert tpf.prob_position_kept(1, 0.3) == 1.0


def test_alternative_readings_do_not_reproduce_the_table():
    """E[acc] alone, or E[acc] over one forward, are not the printed TPF column."""
    for row in _table()["rows"]:
        if row["N"] == 2:
            continue
        assert round(tpf.expected_accepted(row["N"], 0.9), 2) != row["TPF"]


def _exact_alpha_rows(rng, V, alpha, rows):
    lp = np.empty((rows, V))
    lq = np.empty((rows, V))
    for j in range(rows):
        p = np.append(rng.dirichlet(np.ones(V - 1)), 0.0)
        q = alpha * p
        q[-1] = 1.0 - alpha
        with np.errstate(divide="ignore"):
            lp[j], lq[j] = np.log(p), np.log(q)
    return lp, lq


@pytest.mark.parametrize("N", [2, 4])
def test_simulated_loop_matches_closed_form_and_identity(N):
    rng = np.random.Generator(np.random.PCG64(40 + N))
    alpha, V = 0.9, 10
    lp, lq = _exact_alpha_rows(rng, V, alpha, N - 1)
    qprob = np.exp(lq)
    counts = tpf.LoopCounts()
    cycles = 20000
    per_cycle_tokens = []
    per_cycle_fwd = []
    for _ in range(cycles):
        x = [int(rng.integers(0, V))] + [int(rng.choice(V, p=qprob[j])) for j in range(N - 1)]
        u = [(float(rng.random()), float(rng.random())) for _ in range(N - 1)]
        a = verify_stride(lp, lq, x, u).accept_len
        before_t, before_f = counts.tokens, counts.forwards
        counts.add_cycle(a, N)
        per_cycle_tokens.append(counts.tokens - before_t)
        per_cycle_fwd.append(counts.forwards - before_f)
    # ratio estimator standard error (delta method)
    t = np.asarray(per_cycle_tokens, float)
    f = np.asarray(per_cycle_fwd, float)
    r = t.sum() / f.sum()
    se = math.sqrt(np.var(t - r * f) / cycles) / f.mean()
    assert abs(counts.tpf - tpf.tpf_closed_form(N, alpha)) < 4 * se
    # compute-bound identity on the measured counts
    Q = tpf.queries_per_forward(N)
    L = counts.tokens
    oh = tpf.overhead(L, counts.tpf, Q)
    assert abs(oh - counts.forwards * Q / counts.tokens) < 1e-12
    assert abs(counts.tpf / oh - tpf.compute_bound_speedup(counts.tpf, Q)) < 1e-12


def test_speedup_equals_tpf_over_overhead_on_a_grid():
    """Step 6 of the derivation, for several (N, p): TPF / OH == TPF^2 / Q."""
    for N in (2, 3, 4, 5, 8):
        for p in (0.5, 0.7, 0.9, 0.95):
            t = tpf.tpf_closed_form(N, p)
            Q = tpf.queries_per_forward(N)
            oh = tpf.overhead(1000.0, t, Q)
            assert abs(oh - Q / t) < 1e-12
            assert abs(t / oh - tpf.compute_bound_speedup(t, Q)) < 1e-12
