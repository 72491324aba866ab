"""Pins for oracle.accept.

* scipy's logsumexp / log_softmax are the library references for normalisers
  and selected log-probabilities; constant logits give lse = c + log V.
* Speculative-sampling exactness (Leviathan, Kalman, Matias 2023; Chen et al.
  2023): accept-with-min(1, p/q) plus the residual on rejection commits a
  token distributed exactly as p.  The oracle is treated as a black box and
  its accept region and residual CDF intervals are measured by bisection on
  the uniforms, then summed over all proposals.
* Geometric acceptance: with per-position acceptance exactly alpha,
  P(A >= k) = alpha^(k-1) and E[A] = sum alpha^(k-1) (Monte Carlo, 4 SE).
* Position 1 is always accepted; the test is strict (u = rho rejects).
* Planted mistakes in the oracle (a sign flip in the residual, an inverted
  ratio) make these pins fail.
"""

import math

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import accept, philox
from oracle.accept import log_normalizer, residual_sample, verify_stride

U_MAX = 1.0 - 2.0 ** -53


def _accept_boundary(p_row, q_row, x, verify=verify_stride):
    """sup{u : oracle accepts x} by bisection, for a single-decision stride (N=2)."""
    def accepted(u):
        res = verify(p_row[None], q_row[None], [0, x], [(u, 0.5)])
        return res.accept_len == 2
    if accepted(U_MAX):
        return 1.0
    if not accepted(0.0):
        return 0.0
    lo, hi = 0.0, U_MAX
    for _ in range(64):
        mid = 0.5 * (lo + hi)
        if accepted(mid):
            lo = mid
        else:
            hi = mid
    return hi


def _residual_masses(p_row, q_row, vocab):
    """Measure of {u' : residual draw = y} for every y, by bisection on the CDF edges."""
    def draw(u):
        return residual_sample(p_row, q_row, u)[0]
    edges = [0.0]
    for y in range(1, vocab):
        if draw(U_MAX) < y:           # y and above are never drawn
            edges.append(1.0)
            continue
        if draw(0.0) >= y:
            edges.append(0.0)
            continue
        lo, hi = 0.0, U_MAX
        for _ in range(64):
            mid = 0.5 * (lo + hi)
            if draw(mid) >= y:
                hi = mid
            else:
                lo = mid
        edges.append(hi)
    edges.append(1.0)
    return np.diff(np.asarray(edges))


def _enumerated_commit_distribution(lp, lq, verify=verify_stride):
    V = len(lp)
    q = scipy.special.softmax(lq.astype(np.float64))
    acc = np.array([_accept_boundary(lp, lq, x, verify) for x in range(V)])
    reject_mass = float(np.sum(q * (1.0 - acc)))
    res = _residual_masses(lp, lq, V)
    return q * acc + reject_mass * res


@pytest.mark.parametrize("V,seed", [(8, 0), (8, 1), (64, 2)])
def test_accept_plus_residual_reproduces_p(V, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    lp = rng.normal(0, 2.0, V)
    lq = lp + rng.normal(0, 0.8, V)
    got = _enumerated_commit_distribution(lp, lq)
    want = scipy.special.softmax(lp)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_exactness_on_tiny_config_vocab():
    """The same theorem at V = 1024 with the tiny config's logit law (p ~ N(0, 9), q = p + noise)."""
    rng = np.random.Generator(np.random.PCG64(11))
    V = 1024
    lp = rng.normal(0, 3.0, V).astype(np.float32).astype(np.float64)
    lq = (lp + 0.28 * rng.normal(0, 1.0, V)).astype(np.float32).astype(np.float64)
    got = _enumerated_commit_distribution(lp, lq)
    np.testing.assert_allclose(got, scipy.special.softmax(lp), rtol=0, atol=1e-12)


def test_planted_residual_sign_flip_is_caught(monkeypatch):
    rng = np.random.Generator(np.random.PCG64(3))
    lp = rng.normal(0, 2.0, 8)
    lq = lp + rng.normal(0, 0.8, 8)

    def flipped(p_row, q_row, lse_p, lse_q):
        p = np.exp(np.asarray(p_row, np.float64) - lse_p)
        q = np.exp(np.asarray(q_row, np.float64) - lse_q)
        return np.cumsum(np.maximum(0.0, q - p)), False

    monkeypatch.setattr(accept, "residual_cdf", flipped)
    got = _enumerated_commit_distribution(lp, lq)
    assert np.max(np.abs(got - scipy.special.softmax(lp))) > 1e-3


def test_planted_inverted_ratio_is_caught():
    rng = np.random.Generator(np.random.PCG64(4))
    lp = rng.normal(0, 2.0, 8)
    lq = lp + rng.normal(0, 0.8, 8)

    def swapped(p_rows, q_rows, proposals, uniforms):
        # accept test run with the ratio q/p instead of p/q
        res = verify_stride(p_rows, q_rows, proposals, [(0.0, 0.0)] * (len(proposals) - 1))
        u = uniforms[0][0]
        return accept.StrideResult(accept_len=2 if u < 1.0 / res.rho[0] else 1, out_tokens=[],
                                   n_out=0, n_commit=0, logp_sel=res.logp_sel,
                                   logq_sel=res.logq_sel, rho=1.0 / res.rho, u_accept=np.zeros(1),
                                   decided=1, reject_row=-1)

    got = _enumerated_commit_distribution(lp, lq, verify=swapped)
    assert np.max(np.abs(got - scipy.special.softmax(lp))) > 1e-3


def test_log_normalizer_closed_form_and_scipy():
    assert abs(log_normalizer(np.full(151936, 2.5)) - (2.5 + math.log(151936))) < 1e-12
    rng = np.random.Generator(np.random.PCG64(5))
    for V in (1, 7, 1024, 151936):
        l = rng.normal(0, 3, V)
        assert abs(log_normalizer(l) - scipy.special.logsumexp(l)) < 1e-11
    assert log_normalizer(np.array([-np.inf, 0.0])) == 0.0


def test_selected_log_probs_match_scipy_log_softmax():
    rng = np.random.Generator(np.random.PCG64(6))
    N, V = 5, 300
    lp = rng.normal(0, 3, (N - 1, V))
    lq = lp + rng.normal(0, 0.3, (N - 1, V))
    x = rng.integers(0, V, N)
    res = verify_stride(lp, lq, x, [(0.0, 0.0)] * (N - 1))
    for j in range(N - 1):
        assert abs(res.logp_sel[j] - scipy.special.log_softmax(lp[j])[x[j + 1]]) < 1e-12
        assert abs(res.logq_sel[j] - scipy.special.log_softmax(lq[j])[x[j + 1]]) < 1e-12
        assert abs(res.rho[j] - math.exp(res.logp_sel[j] - res.logq_sel[j])) < 1e-15


def test_position_one_always_accepted():
    rng = np.random.Generator(np.random.PCG64(7))
    N, V = 4, 50
    for trial in range(300):
        lp = rng.normal(0, 3, (N - 1, V))
        lq = rng.normal(0, 3, (N - 1, V))          # unrelated q: many rejections
        x = rng.integers(0, V, N)
        u = [(float(rng.random()), float(rng.random())) for _ in range(N - 1)]
        res = verify_stride(lp, lq, x, u)
        assert 1 <= res.accept_len <= N
        assert res.out_tokens[0] == x[0]
        assert res.out_tokens[: res.accept_len] == [int(t) for t in x[: res.accept_len]]
        assert res.n_out == res.accept_len + (1 if res.accept_len < N else 0)
        assert res.n_commit == res.accept_len           # rows 0..A-1: the accepted prefix


def test_strict_boundary_and_ratio_at_least_one():
    rng = np.random.Generator(np.random.PCG64(8))
    lp = rng.normal(0, 3, (1, 40))
    lq = lp + rng.normal(0, 1, (1, 40))
    x = [0, int(np.argmin(lp[0] - lq[0]))]       # a token with p < q
    rho = verify_stride(lp, lq, x, [(0.0, 0.0)]).rho[0]
    assert rho < 1.0
    assert verify_stride(lp, lq, x, [(rho, 0.3)]).accept_len == 1                    # u == rho rejects
    assert verify_stride(lp, lq, x, [(np.nextafter(rho, 0), 0.3)]).accept_len == 2
    same = verify_stride(lp, lp, x, [(U_MAX, 0.3)])                                  # rho == 1
    assert same.accept_len == 2


def test_residual_zero_mass_falls_back_to_p():
    lp = np.log(np.array([0.1, 0.2, 0.3, 0.4]))
    y, margin, fallback = residual_sample(lp, lp, 0.35)
    assert fallback and y == 2                                                       # CDF 0.1, 0.3, 0.6, 1.0


def _exact_alpha_rows(rng, V, alpha, rows):
    """Rows with sum_x min(p, q) == alpha exactly: q = alpha p + (1 - alpha) delta_{V-1}, p(V-1) = 0."""
    lp = np.empty((rows, V))
    lq = np.empty((rows, V))
    for j in range(rows):
        base = rng.dirichlet(np.ones(V - 1))
        p = np.append(base, 0.0)
        q = alpha * p
        q[-1] = 1.0 - alpha
        with np.errstate(divide="ignore"):
            lp[j] = np.log(p)
            lq[j] = np.log(q)
    return lp, lq


@pytest.mark.parametrize("N,alpha", [(4, 0.9), (2, 0.9), (8, 0.7)])
def test_geometric_acceptance_monte_carlo(N, alpha):
    rng = np.random.Generator(np.random.PCG64(100 + N))
    V = 12
    lp, lq = _exact_alpha_rows(rng, V, alpha, N - 1)
    qprob = np.exp(lq)
    trials = 20000
    counts = np.zeros(N + 1)
    total = 0.0
    for _ in range(trials):
        x = [int(rng.integers(0, V))] + [int(rng.choice(V, p=qprob[j])) for j in range(N - 1)]
        u = [(float(rng.random()), float(rng.random())) for _ in range(N - 1)]
        a = verify_stride(lp, lq, x, u).accept_len
        counts[a] += 1
        total += a
    pk = np.array([alpha ** (k - 1) for k in range(1, N + 1)])           # P(A >= k)
    probs = np.append(pk[:-1] - pk[1:], pk[-1])                           # P(A == k)
    mean = float(np.dot(np.arange(1, N + 1), probs))
    var = float(np.dot(np.arange(1, N + 1) ** 2, probs)) - mean ** 2
    assert abs(mean - sum(pk)) < 1e-12
    assert abs(total / trials - mean) < 4 * math.sqrt(var / trials)
    for k in range(1, N + 1):
        frac = counts[k:].sum() / trials
        se = math.sqrt(pk[k - 1] * (1 - pk[k - 1]) / trials) + 1e-12
        assert abs(frac - pk[k - 1]) < 4 * se + 1e-12


def test_philox_driven_commit_frequencies_follow_p():
    """Chi-square: the token committed at position 2, driven by the Philox uniforms, is ~ p."""
    rng = np.random.Generator(np.random.PCG64(21))
    V = 8
    lp = rng.normal(0, 1.5, (1, V))
    lq = lp + rng.normal(0, 1.0, (1, V))
    qprob = scipy.special.softmax(lq[0])
    seed = (0x1234, 0x5678)
    draws = 12000
    counts = np.zeros(V)
    for step in range(draws):
        x = [3, int(rng.choice(V, p=qprob))]
        u = accept.stride_uniforms(seed, 7, 1000, step, 2)
        res = verify_stride(lp, lq, x, u)
        counts[res.out_tokens[1]] += 1
    expect = scipy.special.softmax(lp[0]) * draws
    stat, pval = scipy.stats.chisquare(counts, expect)
    assert pval > 1e-4, (counts, expect)


def test_stride_uniforms_key_by_absolute_position():
    seed = (5, 6)
    u = accept.stride_uniforms(seed, 9, 4096, 3, 4)
    assert u[0] == philox.decision_uniforms(seed, 9, 4097, 3)
    assert u[2] == philox.decision_uniforms(seed, 9, 4099, 3)
