"""Pins for oracle.propose.

* Closed form: a row whose probabilities are 0, 1/8, 3/8, 1/2 maps u to the
  token whose CDF interval holds u; u = 0 must skip the zero-mass token (the
  first y with C(y) > u, not >= u).
* Library reference: the measure of the uniforms that select each token,
  found by bisection on u with the oracle as a black box, equals scipy's
  softmax of the row.
* Monte Carlo: proposals drawn with the Philox proposal stream have the
  softmax frequencies (chi-square).
* Argmax policy: brute force over the row, ties to the smallest index; the
  sampling policy collapses onto it when one logit dominates.
"""

import math

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import philox, propose

U_MAX = 1.0 - 2.0 ** -53


def _row(probs):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(probs, dtype=np.float64))


@pytest.mark.parametrize("u,y", [(0.0, 1), (0.05, 1), (0.1249, 1), (0.2, 2), (0.4999, 2),
                                 (0.6, 3), (U_MAX, 3)])
def test_worked_example(u, y):
    assert propose.sample_row(_row([0.0, 0.125, 0.375, 0.5]), u)[0] == y


def test_leading_zero_mass_is_never_drawn():
    row = _row([0.0, 0.0, 0.25, 0.0, 0.75])
    for u in (0.0, 1e-300, 0.1, 0.3, U_MAX):
        y = propose.sample_row(row, u)[0]
        assert row[y] > -math.inf


def _interval_measures(row):
    """Measure of {u : sample_row(row, u) = y} for every y, by bisection on the edges."""
    V = len(row)
    edges = [0.0]
    for y in range(V - 1):
        lo, hi = edges[-1], U_MAX
        if propose.sample_row(row, hi)[0] <= y:
            edges.append(1.0)
            continue
        for _ in range(70):
            mid = 0.5 * (lo + hi)
            if propose.sample_row(row, mid)[0] <= y:
                lo = mid
            else:
                hi = mid
        edges.append(hi)
    edges.append(1.0)
    return np.diff(np.array(edges))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_interval_measures_equal_softmax(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    row = rng.normal(0.0, 3.0, size=12)
    np.testing.assert_allclose(_interval_measures(row), scipy.special.softmax(row), rtol=0, atol=1e-12)


def test_philox_stream_frequencies_chi_square():
    rng = np.random.Generator(np.random.PCG64(11))
    row = rng.normal(0.0, 1.0, size=8)
    q = scipy.special.softmax(row)
    seed = (0x1234, 0x5678)
    draws = [propose.sample_row(row, propose.proposal_uniform(seed, r, 100 + r % 7, 3))[0]
             for r in range(20000)]
    counts = np.bincount(draws, minlength=8)
    chi2, pval = scipy.stats.chisquare(counts, q * len(draws))
    assert pval > 1e-4, (counts, q * len(draws))


def test_argmax_ties_go_to_the_smallest_index():
    assert propose.argmax_row([1.0, 3.0, 3.0, 2.0]) == 1
    assert propose.argmax_row([-math.inf, -1.0, -1.0]) == 1
    rng = np.random.Generator(np.random.PCG64(5))
    for _ in range(50):
        row = rng.integers(-3, 4, size=40).astype(np.float64)
        best = 0
        for i in range(len(row)):
            if row[i] > row[best]:
                best = i
        assert propose.argmax_row(row) == best


def test_sampling_collapses_onto_a_dominant_logit():
    row = np.zeros(64)
    row[37] = 200.0
    # the 37 tokens before it hold about 5e-86 of the mass, so only u below that reaches them
    assert propose.sample_row(row, 0.0)[0] == 0
    for u in (1e-80, 0.3, 0.7, U_MAX):
        assert propose.sample_row(row, u)[0] == 37 == propose.argmax_row(row)


def test_proposal_stream_is_its_own_philox_block():
    """Counter word 3 = 1 separates proposals from the decision stream of the same position."""
    seed = (3, 4)
    blk = philox.philox4x64((9, 20, 5, 1), seed)
    assert propose.proposal_uniform(seed, 9, 20, 5) == philox.unit_double(blk[0])
    assert propose.proposal_uniform(seed, 9, 20, 5) != philox.decision_uniforms(seed, 9, 20, 5)[0]
    u = propose.stride_proposal_uniforms(seed, 9, 16, 5, 4)
    assert u == [propose.proposal_uniform(seed, 9, 16 + 4 + k, 5) for k in range(4)]
    assert len(set(u)) == 4


def test_isd_propose_batch_shapes_and_modes():
    rng = np.random.Generator(np.random.PCG64(2))
    logits = rng.normal(0.0, 3.0, size=(3, 4, 50))
    toks, mg = propose.isd_propose(logits, [0, 1, 2], [10, 20, 30], (1, 2), 7)
    assert toks.shape == (3, 4) and mg.shape == (3, 4)
    assert ((toks >= 0) & (toks < 50)).all() and (mg >= 0).all()
    am, _ = propose.isd_propose(logits, [0, 1, 2], [10, 20, 30], (1, 2), 7, mode=propose.ARGMAX)
    assert (am == logits.argmax(axis=-1)).all()
    sub, _ = propose.isd_propose(logits, [0, 1, 2], [10, 20, 30], (1, 2), 7, requests=[2])
    assert (sub[0] == toks[2]).all()
