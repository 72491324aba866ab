"""The multi-step decoding loop on the GPU.

* Transition parity: a full loop (attention, accept with the commit,
  proposals, bookkeeping) runs for a number of forwards; before each forward
  the GPU's loop state is read back and the oracle applies the same forward to
  it (accept test, proposals, bookkeeping, commit of the forward's rows).
  Accept lengths, committed tokens, proposals, the new state and the commit
  counts must be identical, except for requests with a near-tie decision; the
  lengths must keep the loop's invariant (committed length = positions, or
  positions + N - 1 while a resampled token waits for its row); the KV pools
  and lengths are compared bit for bit, and a last attention call is checked
  on the grown contexts.  The same check runs on every replay of a recorded
  loop forward.
* TPF: the loop's measured tokens per forward (accept + proposals +
  bookkeeping, logits with per-row acceptance 0.9) reproduce the closed form
  and the printed TPF column for N = 2, 3, 4, 5, 8.
"""

import json
import os

import numpy as np
import pytest
import torch

from parity import ACCEPT_NEAR_TIE, PROPOSE_NEAR_TIE, RESAMPLE_NEAR_TIE, check_attention, device_step, needs_gpu
from workloads import get_config, make_workload

pytestmark = [pytest.mark.gpu, needs_gpu]

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "isd_acceptance_table.json")


def _round(x, dtype):
    t = torch.from_numpy(np.asarray(x, dtype=np.float32))
    return (t.to(torch.bfloat16).float() if dtype == "bf16" else t).numpy()


def _pool(cfg, entries, seed0, tau_mode):
    """Logit sets for successive forwards: (p rows, q rows, MASK rows = [free row | q rows])."""
    out = []
    for k in range(entries):
        wl = make_workload(cfg, seed=seed0 + k, tau_mode=tau_mode)
        row0 = np.random.Generator(np.random.PCG64(seed0 + 77 + k)).normal(
            0.0, cfg.logit_std, size=(cfg.batch, 1, cfg.vocab))
        mask = np.concatenate([_round(row0, cfg.dtype), wl.q_logits], axis=1)
        out.append((wl.p_logits, wl.q_logits, mask))
    return out


def _dev(x, like):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=like.device, dtype=like.dtype)


class OracleLoop:
    """The oracle's copy of a GPU loop: applies each forward the GPU ran to the GPU's own
    state before it, checks every transition, and keeps the oracle's pools and lengths."""

    def __init__(self, wl):
        self.wl = wl
        self.k_pool, self.v_pool, self.ctx = wl.k_pool.copy(), wl.v_pool.copy(), wl.ctx_lens.copy()
        self.near = 0
        self.decisions = 0

    @staticmethod
    def state(st):
        from oracle import loop as oloop
        return oloop.LoopState(st.extra["mode"].cpu().numpy().astype(np.int64),
                               st.proposals.cpu().numpy().astype(np.int64),
                               st.positions.cpu().numpy().astype(np.int64),
                               st.extra["tokens"].cpu().numpy(), st.extra["forwards"].cpu().numpy())

    def check(self, st, pre, p, q, mask, t, step):
        """``pre``: the GPU state before forward t (Philox step ``step``), read by ``state``."""
        from oracle import accept as oaccept
        from oracle import loop as oloop
        from oracle import propose as oprop
        from oracle.commit import kv_commit as ocommit
        wl, cfg = self.wl, self.wl.cfg
        n = cfg.stride_n
        res = oaccept.isd_accept(p, q, pre.proposals, wl.req_ids, pre.pos, wl.philox_seed, step)
        nxt, margins = oprop.isd_propose(mask, wl.req_ids, pre.pos, wl.philox_seed, step)
        post = pre.copy()
        n_commit, first_row = oloop.advance(post, [o.accept_len for o in res], [o.n_out for o in res], nxt)
        verifying = pre.mode == oloop.VERIFY
        tie = np.zeros(cfg.batch, dtype=bool)
        for r, o in enumerate(res):
            tie[r] = verifying[r] and (bool((o.accept_margins < ACCEPT_NEAR_TIE).any())
                                       or o.resample_margin < RESAMPLE_NEAR_TIE)
            tie[r] |= bool((margins[r] < PROPOSE_NEAR_TIE).any())
            self.decisions += o.decided if verifying[r] else 0
        self.near += int(tie.sum())
        ok = ~tie
        got = {k: v.cpu().numpy() for k, v in (("accept_len", st.accept_len), ("n_out", st.n_out),
                                                ("next", st.next_proposals), ("n_commit", st.n_commit),
                                                ("mode", st.extra["mode"]), ("proposals", st.proposals),
                                                ("positions", st.positions), ("tokens", st.extra["tokens"]),
                                                ("forwards", st.extra["forwards"]))}
        assert (got["accept_len"][ok & verifying] == np.array([o.accept_len for o in res])[ok & verifying]).all(), t
        assert (got["n_out"][ok & verifying] == np.array([o.n_out for o in res])[ok & verifying]).all(), t
        assert (got["next"][ok] == nxt[ok]).all(), t
        assert (got["n_commit"][ok] == n_commit[ok]).all(), t
        assert (got["mode"][ok] == post.mode[ok]).all(), t
        assert (got["proposals"][ok] == post.proposals[ok]).all(), t
        assert (got["positions"][ok] == post.pos[ok]).all(), t
        assert (got["tokens"][ok] == post.tokens[ok]).all(), t
        assert (got["forwards"] == pre.forwards + 1).all()
        # the oracle's commit of the GPU's rows (equal to its own outside near-ties)
        first = np.where(pre.mode == oloop.REPROPOSE, n - 1, 0)
        self.k_pool, self.v_pool, self.ctx = ocommit(self.k_pool, self.v_pool, wl.page_table, self.ctx,
                                                     wl.k_new, wl.v_new, got["n_commit"], cfg.page_size,
                                                     first_row=first)
        lens = st.ctx_lens.cpu().numpy()
        assert (lens == self.ctx).all(), t
        pending = got["mode"] == oloop.REPROPOSE
        assert (lens == got["positions"] + np.where(pending, n - 1, 0)).all(), t

    def check_pools(self, st):
        from introspective_strided_decoding_amd.layout import unpack_k_pages, unpack_v_pages
        assert np.array_equal(unpack_k_pages(st.k_pages).float().cpu().numpy(), self.k_pool)
        assert np.array_equal(unpack_v_pages(st.v_pages).float().cpu().numpy(), self.v_pool)

    def check_budget(self):
        assert self.near == 0 or self.near / max(1, self.decisions) < 1e-4


def test_loop_transitions_match_oracle():
    T, K = 12, 3
    cfg = get_config("b8_ctx2k", batch=12, ctx=40, vocab=1000, stride_n=4)
    wl = make_workload(cfg, seed=61, with_mask_logits=True, extra_tokens=T * cfg.stride_n)
    pool = _pool(cfg, K, 300, "batch")
    st = device_step(wl, commit_in_place=True)
    st.loop_start()
    orc = OracleLoop(wl)
    reproposed = 0
    for t in range(T):
        p, q = (wl.p_logits, wl.q_logits) if t == 0 else pool[(t - 1) % K][:2]
        mask = pool[t % K][2]
        st.p_logits.copy_(_dev(p, st.p_logits))
        st.q_logits.copy_(_dev(q, st.q_logits))
        st.mask_logits.copy_(_dev(mask, st.mask_logits))
        pre = orc.state(st)
        reproposed += int((pre.mode == 1).sum())
        st.loop_forward(step=t)
        torch.cuda.synchronize()
        orc.check(st, pre, p, q, mask, t, t)
    orc.check_budget()
    orc.check_pools(st)
    assert reproposed > 0                     # re-proposing forwards committed their row N-1
    # attention over the grown (committed) contexts
    st.attention()
    torch.cuda.synchronize()
    wl.k_pool, wl.v_pool, wl.ctx_lens = orc.k_pool, orc.v_pool, orc.ctx
    check_attention(wl, st.out)
    from introspective_strided_decoding_amd import isd_read_flags
    assert isd_read_flags(st.workspace) == 0


@pytest.mark.parametrize("n", [2, 3, 4, 5, 8])
def test_loop_reproduces_tpf_column(n):
    from oracle import tpf
    table = {row["N"]: row["TPF"] for row in json.load(open(GOLDEN))["rows"]}
    T, K = 60, 3
    cfg = get_config("tiny_fp32", batch=256, stride_n=n, vocab=512, ctx=16, n_q_heads=1, n_kv_heads=1)
    wl = make_workload(cfg, seed=700 + n, tau_mode="row", with_mask_logits=True)
    pool = _pool(cfg, K, 800 + 10 * n, "row")
    st = device_step(wl)
    st.loop_start()
    for t in range(T):
        p, q = (wl.p_logits, wl.q_logits) if t == 0 else pool[(t - 1) % K][:2]
        st.p_logits.copy_(_dev(p, st.p_logits))
        st.q_logits.copy_(_dev(q, st.q_logits))
        st.mask_logits.copy_(_dev(pool[t % K][2], st.mask_logits))
        st.loop_forward(step=t, attention=False)
    torch.cuda.synchronize()
    tokens = st.extra["tokens"].cpu().numpy().astype(np.float64)
    forwards = st.extra["forwards"].cpu().numpy().astype(np.float64)
    assert (forwards == T).all()
    tpf_hat = tokens.sum() / forwards.sum()
    se = (tokens / forwards).std(ddof=1) / np.sqrt(cfg.batch)
    closed = tpf.tpf_closed_form(n, 0.9)
    # the loop ends mid-cycle for some requests: allow 1/T of bias
    assert abs(tpf_hat - closed) < 4 * se + 1.0 / T, (n, tpf_hat, closed, se)
    assert abs(tpf_hat - table[n]) < 4 * se + 1.0 / T + 0.005, (n, tpf_hat, table[n], se)


def test_loop_with_proposals_beside_accept_matches_sequential():
    """Proposals on a second stream beside the accept chain give the same forwards,
    bit for bit, as the calls issued one after another."""
    T, K = 6, 3
    cfg = get_config("b8_ctx2k", batch=10, ctx=40, vocab=3000, stride_n=4)
    wl = make_workload(cfg, seed=62, with_mask_logits=True, extra_tokens=T * cfg.stride_n)
    pool = _pool(cfg, K, 310, "batch")
    a = device_step(wl, commit_in_place=True)
    b = device_step(wl, commit_in_place=True)
    for st in (a, b):
        st.loop_start()
    names = ("accept_len", "n_out", "next_proposals", "n_commit", "proposals", "positions", "ctx_lens",
             "out_tokens", "k_pages", "v_pages")
    for t in range(T):
        p, q = (wl.p_logits, wl.q_logits) if t == 0 else pool[(t - 1) % K][:2]
        for st in (a, b):
            st.p_logits.copy_(_dev(p, st.p_logits))
            st.q_logits.copy_(_dev(q, st.q_logits))
            st.mask_logits.copy_(_dev(pool[t % K][2], st.mask_logits))
        a.loop_forward(step=t, overlap=True)
        b.loop_forward(step=t, overlap=False)
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(getattr(a, n).view(torch.uint8), getattr(b, n).view(torch.uint8)), (t, n)
        for n in ("mode", "tokens", "forwards"):
            assert torch.equal(a.extra[n], b.extra[n]), (t, n)


def _feed(st, pool, wl, t, K):
    p, q = (wl.p_logits, wl.q_logits) if t == 0 else pool[(t - 1) % K][:2]
    st.p_logits.copy_(_dev(p, st.p_logits))
    st.q_logits.copy_(_dev(q, st.q_logits))
    st.mask_logits.copy_(_dev(pool[t % K][2], st.mask_logits))


_STATE = ("accept_len", "n_out", "next_proposals", "n_commit", "proposals", "positions", "ctx_lens",
          "out_tokens", "k_pages", "v_pages")


def _same_state(a, b, t):
    for n in _STATE:
        assert torch.equal(getattr(a, n).view(torch.uint8), getattr(b, n).view(torch.uint8)), (t, n)
    for n in ("mode", "tokens", "forwards"):
        assert torch.equal(a.extra[n], b.extra[n]), (t, n)


def test_loop_device_step_matches_step_argument():
    """Philox steps read from the device forward counts draw what the step argument t
    draws when every request started together (forwards = t)."""
    T, K = 5, 3
    cfg = get_config("b8_ctx2k", batch=9, ctx=40, vocab=3000, stride_n=4)
    wl = make_workload(cfg, seed=63, with_mask_logits=True, extra_tokens=T * cfg.stride_n)
    pool = _pool(cfg, K, 320, "batch")
    a = device_step(wl, commit_in_place=True)
    b = device_step(wl, commit_in_place=True)
    for st in (a, b):
        st.loop_start()
    for t in range(T):
        for st in (a, b):
            _feed(st, pool, wl, t, K)
        a.loop_forward(step=t)
        b.loop_forward(device_step=True)
        torch.cuda.synchronize()
        _same_state(a, b, t)


@pytest.mark.parametrize("overlap", [True, False])
def test_loop_forward_graph_replays_match_eager(overlap):
    """One loop forward recorded into a HIP graph and replayed forward after forward
    (logits refreshed in place in between) leaves the same state, pools and lengths as
    the same forwards issued eagerly, and every replay's transition, commit and lengths
    match the oracle's forward on the state before it."""
    T, K, warm = 6, 3, 2      # the second eager forward is the first with carried q normalisers
    cfg = get_config("b8_ctx2k", batch=8, ctx=40, vocab=3000, stride_n=4)
    wl = make_workload(cfg, seed=64, with_mask_logits=True, extra_tokens=(T + warm) * cfg.stride_n)
    pool = _pool(cfg, K, 330, "batch")
    a = device_step(wl, commit_in_place=True)
    b = device_step(wl, commit_in_place=True)
    for st in (a, b):
        st.loop_start()
    orc = OracleLoop(wl)
    for t in range(warm):
        for st in (a, b):
            _feed(st, pool, wl, t, K)
        pre = orc.state(b)
        for st in (a, b):
            st.loop_forward(device_step=True, overlap=overlap)
        torch.cuda.synchronize()
        p, q = (wl.p_logits, wl.q_logits) if t == 0 else pool[(t - 1) % K][:2]
        orc.check(b, pre, p, q, pool[t % K][2], t, t)
    graph = b.capture_loop_forward(overlap=overlap)
    for t in range(warm, warm + T):
        for st in (a, b):
            _feed(st, pool, wl, t, K)
        a.loop_forward(device_step=True, overlap=overlap)
        torch.cuda.synchronize()
        pre = orc.state(b)
        graph.replay()
        torch.cuda.synchronize()
        _same_state(a, b, t)
        p, q = pool[(t - 1) % K][:2]
        orc.check(b, pre, p, q, pool[t % K][2], t, t)       # Philox step = forward count = t
    orc.check_budget()
    orc.check_pools(b)
    assert int(b.extra["forwards"][0]) == warm + T
