"""Shared helpers of the GPU parity tests: compare libisd against the oracle.

Tolerances (written here once, used by every GPU test):
* attention output and log-probabilities: 2e-2 absolute in bf16, 1e-5 in fp32;
* accept lengths and token ids: exact, except requests with a near-tie
  decision (|u - rho| < 1e-5 for an accept test, or u' * S within 1e-12 * S
  of an edge of the chosen residual interval); near-ties must stay under
  0.01 % of the decisions taken.  Proposals drawn at the MASK rows follow the
  residual's rule (u * total within 1e-12 * total of an edge).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import accept as oaccept
from oracle.attention import stride_attention

ATOL = {"bf16": 2e-2, "f32": 1e-5}
ACCEPT_NEAR_TIE = 1e-5
RESAMPLE_NEAR_TIE = 1e-12
PROPOSE_NEAR_TIE = 1e-12        # u * total within 1e-12 * total of an edge of the drawn token
NEAR_TIE_BUDGET = 1e-4


def gpu_available() -> bool:
    return torch.cuda.is_available()


needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def device_step(wl, **kw):
    from introspective_strided_decoding_amd.step import DeviceStep
    return DeviceStep.from_arrays(wl, **kw)


def oracle_attention(wl, requests=None):
    return stride_attention(wl.q, wl.k_new, wl.v_new, wl.k_pool, wl.v_pool, wl.page_table,
                            wl.ctx_lens, wl.cfg.page_size, requests=requests)


def check_attention(wl, out_gpu: torch.Tensor, requests=None):
    """Element-wise |gpu - oracle| <= tolerance on the requested requests."""
    ref = oracle_attention(wl, requests)
    got = out_gpu.float().cpu().numpy().astype(np.float64)
    if requests is not None:
        got = got[list(requests)]
    err = np.abs(got - ref)
    tol = ATOL[wl.cfg.dtype]
    assert np.isfinite(got).all(), "non-finite attention output"
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"max |err| {worst:.3e} > {tol} ({wl.cfg.name})"
    return worst


def oracle_normalizers(wl):
    """Row log-normalisers of p and q, [B, N-1] each (oracle, computed once per workload)."""
    cache = getattr(wl, "_lse_cache", None)
    if cache is None:
        B, R, V = wl.p_logits.shape
        lp = oaccept.row_normalizers(wl.p_logits.reshape(B * R, V)).reshape(B, R)
        lq = oaccept.row_normalizers(wl.q_logits.reshape(B * R, V)).reshape(B, R)
        cache = (lp, lq)
        wl._lse_cache = cache
    return cache


class AcceptTally:
    def __init__(self):
        self.decisions = 0
        self.near_ties = 0
        self.requests = 0
        self.exact = 0
        self.resamples = 0
        self.accept_total = 0
        self.logp_err = 0.0

    def near_tie_rate(self):
        return self.near_ties / max(1, self.decisions)


def check_accept_step(wl, gpu, seed, step, tally: AcceptTally, requests=None):
    """Compare one accept call (gpu: dict of host numpy arrays) with the oracle."""
    lse_p, lse_q = oracle_normalizers(wl)
    B, N = wl.proposals.shape
    reqs = range(B) if requests is None else requests
    res = oaccept.isd_accept(wl.p_logits, wl.q_logits, wl.proposals, wl.req_ids, wl.positions,
                             seed, step, requests=reqs, lse_p=lse_p, lse_q=lse_q)
    tol = ATOL[wl.cfg.dtype]
    for r, o in zip(reqs, res):
        tally.requests += 1
        tally.decisions += o.decided
        tally.accept_total += o.accept_len
        lp_err = max(np.abs(gpu["logp_sel"][r] - o.logp_sel).max(), np.abs(gpu["logq_sel"][r] - o.logq_sel).max())
        tally.logp_err = max(tally.logp_err, float(lp_err))
        assert lp_err <= tol, f"request {r}: log-prob error {lp_err:.3e}"
        near = bool((o.accept_margins < ACCEPT_NEAR_TIE).any()) or (o.resample_margin < RESAMPLE_NEAR_TIE)
        if near:
            tally.near_ties += 1
            continue
        tally.exact += 1
        if o.reject_row >= 0:
            tally.resamples += 1
        toks = list(gpu["out_tokens"][r][: o.n_out])
        assert int(gpu["accept_len"][r]) == o.accept_len, (r, step, int(gpu["accept_len"][r]), o.accept_len)
        assert int(gpu["n_out"][r]) == o.n_out, (r, step)
        assert int(gpu["n_commit"][r]) == o.n_commit, (r, step)
        assert toks == o.out_tokens, (r, step, toks, o.out_tokens)
        assert all(int(t) == -1 for t in gpu["out_tokens"][r][o.n_out:]), (r, step)


def fetch_accept(st):
    return {"accept_len": st.accept_len.cpu().numpy(), "out_tokens": st.out_tokens.cpu().numpy(),
            "n_out": st.n_out.cpu().numpy(), "n_commit": st.n_commit.cpu().numpy(),
            "logp_sel": st.logp_sel.cpu().numpy().astype(np.float64),
            "logq_sel": st.logq_sel.cpu().numpy().astype(np.float64)}


def check_step_against_oracle(wl, st, tally: AcceptTally = None):
    """Every output of one whole step (st.run(): attention, accept + commit, and the next
    proposals when the workload carries MASK-row logits) against the oracle on the same
    inputs: attention element-wise, accept results outside near-ties, both pools bit for bit
    after the oracle's commit of the GPU's counts, the new lengths, and the proposals."""
    from oracle.commit import kv_commit as oracle_commit
    from oracle.propose import isd_propose as oracle_propose
    from introspective_strided_decoding_amd.layout import unpack_k_pages, unpack_v_pages
    tally = tally if tally is not None else AcceptTally()
    check_attention(wl, st.out)
    got = fetch_accept(st)
    check_accept_step(wl, got, wl.philox_seed, wl.step, tally)
    assert tally.near_ties <= max(0, NEAR_TIE_BUDGET * tally.decisions), tally.near_ties
    k_ref, v_ref, lens_ref = oracle_commit(wl.k_pool, wl.v_pool, wl.page_table, wl.ctx_lens,
                                           wl.k_new, wl.v_new, got["n_commit"], wl.cfg.page_size)
    assert np.array_equal(st.ctx_lens_out.cpu().numpy(), lens_ref)
    assert np.array_equal(unpack_k_pages(st.k_pages).float().cpu().numpy(), k_ref)
    assert np.array_equal(unpack_v_pages(st.v_pages).float().cpu().numpy(), v_ref)
    if getattr(wl, "mask_logits", None) is not None and st.next_proposals is not None:
        nxt, margins = oracle_propose(wl.mask_logits, wl.req_ids, wl.positions, wl.philox_seed, wl.step)
        prop = st.next_proposals.cpu().numpy()
        assert ((prop == nxt) | (margins < PROPOSE_NEAR_TIE)).all()
    return tally
