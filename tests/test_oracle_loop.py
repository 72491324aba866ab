"""Pins for oracle.loop (the multi-step decoding loop).

* The printed TPF column ([hotdry] "Token 生成的核心参数与验收机制", stored in
  tests/golden/isd_acceptance_table.json): ``advance`` driven by accept
  lengths drawn with per-position acceptance 0.9 gives tokens / forwards
  within 4 standard errors of each printed TPF (plus its rounding), for
  N = 2, 3, 4, 5, 8.
* Bookkeeping invariants: every request spends one forward per call;
  committed tokens are the n_out of its VERIFY forwards; every REPROPOSE
  forward follows a rejecting VERIFY forward; a VERIFY forward commits its
  rows 0..A-1 and a REPROPOSE forward its row N-1 (the resampled token); the
  positions move by the committed tokens, less N when the last forward was a
  rejecting VERIFY; the context grows by the committed tokens, one behind
  while a resampled token waits for its row (ctx = pos in VERIFY mode,
  pos + N - 1 in REPROPOSE mode).
* Every committed token's key and value land exactly once, at its own
  position: with each stride row's key encoding the token the row carries,
  the pool after many forwards of the oracle loop (accept test, proposals,
  bookkeeping, commit) spells out the committed token stream, position by
  position, with nothing missing or written twice.
* The compute-bound identity on measured counts: TPF / OH = TPF^2 / Q.
* End to end on small logits with per-row acceptance 0.9: the oracle's own
  accept test and proposals inside the loop give the closed-form TPF.
"""

import json
import os

import numpy as np
import pytest

from oracle import loop, propose, tpf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "isd_acceptance_table.json")


def _table():
    return {row["N"]: row for row in json.load(open(GOLDEN))["rows"]}


def _geometric_accepts(rng, n, alpha, size):
    """A = 1 + number of leading successes among N-1 Bernoulli(alpha) tests."""
    tests = rng.random((size, n - 1)) < alpha
    lead = np.where(tests.all(axis=1), n - 1, np.argmin(tests, axis=1))
    return 1 + lead


@pytest.mark.parametrize("n", [2, 3, 4, 5, 8])
def test_advance_reproduces_printed_tpf(n):
    rng = np.random.Generator(np.random.PCG64(100 + n))
    B, T = 512, 400
    st = loop.LoopState.start(np.zeros((B, n), dtype=np.int64), np.full(B, 1000))
    nxt = np.zeros((B, n), dtype=np.int64)
    for _ in range(T):
        a = _geometric_accepts(rng, n, 0.9, B)
        loop.advance(st, a, a + (a < n), nxt)
    per_req = st.tokens / st.forwards
    tpf_hat = st.tokens.sum() / st.forwards.sum()
    se = per_req.std(ddof=1) / np.sqrt(B)
    printed = _table()[n]["TPF"]
    assert abs(tpf_hat - printed) < 4 * se + 0.005 + 1.0 / T, (n, tpf_hat, printed, se)
    assert abs(tpf_hat - tpf.tpf_closed_form(n, 0.9)) < 4 * se + 1.0 / T


def test_bookkeeping_invariants():
    n, B = 4, 200
    rng = np.random.Generator(np.random.PCG64(7))
    st = loop.LoopState.start(rng.integers(0, 50, size=(B, n)), np.full(B, 500))
    pos0 = st.pos.copy()
    ctx0 = st.pos.copy()                   # the loop starts verifying with ctx = pos
    ctx = ctx0.copy()
    n_out_verify = np.zeros(B, dtype=np.int64)
    last_rejecting_verify = np.zeros(B, dtype=bool)
    for t in range(60):
        mode_before = st.mode.copy()
        a = _geometric_accepts(rng, n, 0.8, B)
        n_out = a + (a < n)
        nxt = rng.integers(0, 50, size=(B, n))
        n_commit, first_row = loop.advance(st, a, n_out, nxt)
        ctx += n_commit
        was_verify = mode_before == loop.VERIFY
        n_out_verify += np.where(was_verify, n_out, 0)
        assert (n_commit[~was_verify] == 1).all() and (first_row[~was_verify] == n - 1).all()
        assert (n_commit[was_verify] == a[was_verify]).all() and (first_row[was_verify] == 0).all()
        pending = st.mode == loop.REPROPOSE
        assert (ctx - ctx0 == st.tokens - pending).all()
        assert (ctx == st.pos + np.where(pending, n - 1, 0)).all()
        # a REPROPOSE forward only ever follows a rejecting VERIFY forward
        assert (st.mode[was_verify & (a < n)] == loop.REPROPOSE).all()
        assert (st.mode[~was_verify] == loop.VERIFY).all()
        # the next stride is the MASK proposals unless the forward rejected
        keep = was_verify & (a < n)
        assert (st.proposals[~keep] == nxt[~keep]).all()
        last_rejecting_verify = was_verify & (a < n)
    assert (st.forwards == 60).all()
    assert (st.tokens == n_out_verify).all()
    assert (st.pos - pos0 == st.tokens - n * last_rejecting_verify).all()


def test_identity_on_measured_counts():
    n = 4
    q = tpf.queries_per_forward(n)
    rng = np.random.Generator(np.random.PCG64(3))
    st = loop.LoopState.start(np.zeros((64, n), dtype=np.int64), np.full(64, 100))
    for _ in range(100):
        a = _geometric_accepts(rng, n, 0.9, 64)
        loop.advance(st, a, a + (a < n), np.zeros((64, n), dtype=np.int64))
    tokens, forwards = int(st.tokens.sum()), int(st.forwards.sum())
    t = tokens / forwards
    oh = forwards * q / tokens
    assert abs(t / oh - t * t / q) < 1e-12


def test_end_to_end_oracle_loop_matches_closed_form():
    """Oracle accept test and proposals inside the loop, logits with per-row acceptance 0.9."""
    from workloads import get_config, make_workload
    n, B, T = 4, 48, 40
    cfg = get_config("tiny_fp32", batch=B, stride_n=n, vocab=256, ctx=16, n_q_heads=1, n_kv_heads=1)
    pool = []
    for k in range(4):
        wl = make_workload(cfg, seed=500 + k, tau_mode="row")
        extra = np.random.Generator(np.random.PCG64(900 + k)).normal(0.0, 3.0, size=(B, 1, 256))
        mask = np.concatenate([extra, wl.q_logits.astype(np.float64)], axis=1)
        pool.append((wl.p_logits, wl.q_logits, mask))
    req_ids = np.arange(B) + 7
    seed = (11, 22)
    st = loop.LoopState.start(np.zeros((B, n), dtype=np.int64), np.full(B, 64))
    # the first stride comes from the forward before the loop (pool entry 3's MASK rows)
    st.proposals, _ = propose.isd_propose(pool[3][2], req_ids, st.pos - n, seed, 10**6)
    for t in range(T):
        p, q, _ = pool[(t - 1) % 4]
        loop.forward(st, p, q, pool[t % 4][2], req_ids, seed, t)
    per_req = st.tokens / st.forwards
    tpf_hat = st.tokens.sum() / st.forwards.sum()
    se = per_req.std(ddof=1) / np.sqrt(B)
    assert abs(tpf_hat - tpf.tpf_closed_form(n, 0.9)) < 4 * se + 1.0 / T, (tpf_hat, se)


@pytest.mark.parametrize("n", [2, 4, 8])
def test_every_committed_token_lands_once_at_its_position(n):
    """Oracle loop forwards with the commit of ``advance``'s rows: stride row i's key holds
    the token the row carries (x_{i+1} in a VERIFY forward; in a REPROPOSE forward the
    committed tokens before the resampled one and, in row N-1, the resampled token), so
    the pool must spell out the committed token stream at positions ctx_0 .. ctx - 1."""
    from oracle.commit import kv_commit
    from workloads import get_config, make_workload
    B, T, V, ps = 24, 30, 64, 16
    cfg = get_config("tiny_fp32", batch=B, stride_n=n, vocab=V, ctx=20, n_q_heads=1, n_kv_heads=1)
    wl = make_workload(cfg, seed=40 + n, tau_mode="row", with_mask_logits=True,
                       extra_tokens=(T + 2) * n)
    req_ids = np.arange(B) + 3
    seed = (5, 6)
    st = loop.LoopState.start(wl.proposals, wl.ctx_lens)
    ctx0 = wl.ctx_lens.astype(np.int64).copy()
    ctx = ctx0.copy()
    k_pool = np.zeros_like(wl.k_pool)
    v_pool = np.zeros_like(wl.v_pool)
    stream = [[] for _ in range(B)]          # committed tokens, in order
    Q, D = cfg.q_rows, cfg.head_dim
    rng = np.random.Generator(np.random.PCG64(9))
    for t in range(T):
        mode = st.mode.copy()
        # the token each stride row carries, written into its key (dim 0) and value
        k_new = np.full((B, Q, 1, D), -1.0, dtype=np.float32)
        for r in range(B):
            if mode[r] == loop.VERIFY:
                carried = list(st.proposals[r])
            else:
                # positions pos .. pos + N - 1: the last N - 1 committed tokens (or context
                # tokens from before the loop, -1 here), then y*
                carried = ([-1] * n + stream[r])[-n:]
            k_new[r, :n, 0, 0] = carried
        v_new = k_new.copy()
        p = rng.normal(0.0, 3.0, size=(B, n - 1, V))
        q = p + rng.normal(0.0, 0.6, size=p.shape)
        mask = rng.normal(0.0, 3.0, size=(B, n, V))
        res, _, n_commit, first_row = loop.forward(st, p, q, mask, req_ids, seed, t)
        for r in range(B):
            if mode[r] == loop.VERIFY:
                stream[r].extend(res[r].out_tokens)
        k_pool, v_pool, ctx = kv_commit(k_pool, v_pool, wl.page_table, ctx, k_new, v_new, n_commit, ps,
                                        first_row=first_row)
        pending = st.mode == loop.REPROPOSE
        assert (ctx - ctx0 == st.tokens - pending).all(), t
    for r in range(B):
        pos = np.arange(ctx0[r], ctx[r])
        keys = k_pool[wl.page_table[r, pos // ps], pos % ps, 0, 0]
        want = stream[r][: len(pos)]
        assert len(stream[r]) == len(pos) + int(st.mode[r] == loop.REPROPOSE)
        assert keys.tolist() == [float(x) for x in want], r
    assert (st.mode == loop.REPROPOSE).any() and (st.mode == loop.VERIFY).any()
