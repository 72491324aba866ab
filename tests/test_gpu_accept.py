"""isd_accept on the GPU vs the float64 oracle.

Accept lengths, committed tokens, n_out and n_commit must be identical to the
oracle's under the same Philox draws, except for requests with a near-tie
decision, which are counted and must stay under 0.01 % of decisions.  The
selected log-probabilities must match within the dtype tolerance.  Many
draws per input set come from varying the Philox step counter (and key),
so one large logit set is decided under thousands of independent uniforms.
"""

import numpy as np
import pytest
import torch

from parity import (NEAR_TIE_BUDGET, AcceptTally, check_accept_step, device_step, fetch_accept,
                    needs_gpu)
from workloads import get_config, make_workload

pytestmark = [pytest.mark.gpu, needs_gpu]


def _run(wl, steps, seeds=None, requests=None):
    st = device_step(wl)
    tally = AcceptTally()
    for k in range(steps):
        step = wl.step + k
        seed = wl.philox_seed if seeds is None else seeds[k % len(seeds)]
        st.accept(step=step, seed=seed)
        torch.cuda.synchronize()
        check_accept_step(wl, fetch_accept(st), seed, step, tally, requests)
    from introspective_strided_decoding_amd import isd_read_flags
    assert isd_read_flags(st.workspace) == 0
    assert tally.near_tie_rate() < NEAR_TIE_BUDGET, vars(tally)
    return tally


def test_accept_tiny_fp32_many_draws():
    wl = make_workload(get_config("tiny_fp32"))
    seeds = [wl.philox_seed, (1, 2), (0xFFFFFFFFFFFFFFFF, 0x8000000000000000)]
    t = _run(wl, 3000, seeds)
    assert t.resamples > 100
    # one fixed proposal: P(accept) = min(1, rho(x_2)), so E[A] = 1 + min(1, rho)
    from oracle.accept import verify_stride
    rho = verify_stride(wl.p_logits[0], wl.q_logits[0], wl.proposals[0], [(0.0, 0.0)]).rho[0]
    p = min(1.0, rho)
    se = (p * (1 - p) / t.requests) ** 0.5
    assert abs(t.accept_total / t.requests - (1 + p)) < 4 * se + 1e-9


@pytest.mark.parametrize("over", [
    dict(batch=4, ctx=16, vocab=1000, stride_n=4),          # V not a multiple of 8
    dict(batch=3, ctx=16, vocab=8, stride_n=8),             # tiny vocabulary, N=8
    dict(batch=2, ctx=16, vocab=4099, stride_n=5),          # odd V, several shards
    dict(batch=3, ctx=16, vocab=151936, stride_n=2),        # full vocab, single decision
    dict(batch=300, ctx=16, vocab=4099, stride_n=4),        # many requests, one normaliser shard per row
])
def test_accept_small_shapes_bf16(over):
    wl = make_workload(get_config("b8_ctx2k", **over))
    _run(wl, 40)


def test_accept_fp32_large_vocab():
    wl = make_workload(get_config("tiny_fp32", batch=4, vocab=50257, stride_n=4))
    _run(wl, 30)


@pytest.mark.parametrize("off", [650.0, -900.0])
def test_accept_logits_far_outside_exp_range(off):
    """exp(l) of every logit would overflow (or underflow to 0) in float64; the residual
    works relative to each row's max, so the draws still match the oracle."""
    import torch as _t
    wl = make_workload(get_config("b8_ctx2k", batch=4, ctx=16, vocab=3000))
    for name in ("p_logits", "q_logits"):
        x = _t.from_numpy(getattr(wl, name)) + off
        setattr(wl, name, x.to(_t.bfloat16).to(_t.float32).numpy())
    t = _run(wl, 60)
    assert t.resamples > 0


@pytest.mark.parametrize("kind", ["one_difference", "many_differences"])
def test_accept_residual_with_many_boundary_entries(kind):
    """Many entries sit on the boundary of the residual's support.

    The second half of the vocabulary differs (with equal mass in each half), so
    rejections happen.  one_difference: p and q agree on the first half, so half
    of every row shares one logit difference and the one-pass summaries keep
    that group exactly.  many_differences: on the first half q is p plus tiny
    offsets, so those entries are near the boundary with thousands of distinct
    differences and the selection recomputes their shards from the logits."""
    wl = make_workload(get_config("tiny_fp32", batch=4, vocab=8192, stride_n=4, ctx=16))
    B, R, V = wl.p_logits.shape
    rng = np.random.Generator(np.random.PCG64(41))
    p = rng.normal(0.0, 3.0, size=(B, R, V))
    lse = lambda x: x.max(-1, keepdims=True) + np.log(np.exp(x - x.max(-1, keepdims=True)).sum(-1, keepdims=True))
    h = V // 2
    q = p.copy()
    if kind == "many_differences":
        q[:, :, :h] += rng.uniform(-3e-5, 3e-5, size=(B, R, h))
    q[:, :, h:] = rng.normal(0.0, 3.0, size=(B, R, V - h))
    q[:, :, h:] += lse(p[:, :, h:]) - lse(q[:, :, h:])
    wl.p_logits = p.astype(np.float32)
    wl.q_logits = q.astype(np.float32)
    for r in range(B):
        for j in range(R):
            prob = np.exp(wl.q_logits[r, j].astype(np.float64) - lse(wl.q_logits[r, j].astype(np.float64)))
            wl.proposals[r, j + 1] = min(V - 1, int(np.searchsorted(np.cumsum(prob), rng.random() * prob.sum(), "right")))
    wl._lse_cache = None
    t = _run(wl, 40)
    assert t.resamples > 10


def test_accept_identical_rows_always_accept():
    wl = make_workload(get_config("b8_ctx2k", batch=4, ctx=16, vocab=2048))
    wl.q_logits = wl.p_logits.copy()
    st = device_step(wl)
    st.accept()
    torch.cuda.synchronize()
    g = fetch_accept(st)
    assert (g["accept_len"] == wl.cfg.stride_n).all()
    assert (g["n_commit"] == wl.cfg.stride_n).all()       # rows 0..N-1 hold x_1..x_N
    assert np.array_equal(g["out_tokens"], wl.proposals)


def test_accept_out_of_range_token_flags_and_rejects():
    from introspective_strided_decoding_amd import isd_read_flags
    wl = make_workload(get_config("b8_ctx2k", batch=2, ctx=16, vocab=512))
    wl.proposals[1, 2] = 512
    st = device_step(wl)
    st.accept()
    torch.cuda.synchronize()
    assert isd_read_flags(st.workspace) & 4
    g = fetch_accept(st)
    assert g["accept_len"][1] <= 2


@pytest.mark.parametrize("name,steps", [("b8_ctx2k", 100), ("c32_ctx4k", 150), ("c128_lora", 20),
                                        ("c64_ragged", 20)])
def test_accept_full_size(name, steps):
    wl = make_workload(get_config(name))
    t = _run(wl, steps)
    print(f"{name}: {t.decisions} decisions, {t.near_ties} near-ties, {t.resamples} resamples, "
          f"max log-prob err {t.logp_err:.2e}")
    assert t.resamples > 0


@pytest.mark.parametrize("vocab", [2048 * 1024, 2048 * 1024 - 5])
def test_accept_largest_vocabulary(vocab):
    """The largest vocabulary the library takes (1024 residual shards of 2048 entries per
    row), exactly full and with a ragged last shard."""
    wl = make_workload(get_config("b8_ctx2k", batch=2, ctx=16, vocab=vocab, stride_n=3))
    t = _run(wl, 12)
    assert t.requests == 24


@pytest.mark.parametrize("cfg", [dict(name="b8_ctx2k", batch=6, ctx=16, vocab=5000, stride_n=4),
                                 dict(name="tiny_fp32", batch=5, vocab=3001, stride_n=3)])
def test_accept_with_carried_q_normalisers(cfg):
    """The q rows of a verify are the MASK rows of the forward before: the normalisers
    isd_propose writes for them (row max exact, log-normaliser to fp32 rounding) stand in
    for the accept test's own pass over the q rows, with the same decisions (bf16 and fp32
    logits)."""
    from oracle.accept import row_normalizers
    cfg = dict(cfg)
    wl = make_workload(get_config(cfg.pop("name"), **cfg), with_mask_logits=True)
    st = device_step(wl)
    B, N = wl.proposals.shape
    st.mask_logits.copy_(torch.cat([st.mask_logits[:, :1], st.q_logits], dim=1))
    norms = torch.zeros(B, N, 2, dtype=torch.float32, device="cuda")
    st.propose(row_norms=norms)
    torch.cuda.synchronize()
    got = norms.cpu().numpy()[:, 1:].reshape(-1, 2)
    q = np.asarray(wl.q_logits, dtype=np.float64).reshape(-1, wl.q_logits.shape[-1])
    assert np.array_equal(got[:, 0], q.max(axis=1).astype(np.float32))
    lse = got[:, 0].astype(np.float64) + np.log(got[:, 1].astype(np.float64))
    np.testing.assert_allclose(lse, row_normalizers(q), rtol=2e-7, atol=2e-6)
    tally = AcceptTally()
    for k in range(40):
        step = wl.step + k
        st.accept(step=step, q_norms=norms)
        torch.cuda.synchronize()
        check_accept_step(wl, fetch_accept(st), wl.philox_seed, step, tally)
    assert tally.near_tie_rate() < NEAR_TIE_BUDGET, vars(tally)
    assert tally.resamples > 5
