"""isd_propose on the GPU vs the float64 oracle.

Sampled proposals must equal the oracle's inverse-CDF draws under the same
Philox uniforms, except draws within 1e-12 of an edge of the drawn token's
CDF interval (near-ties, counted, under 0.01 %).  Argmax proposals are
integer results and must be identical.  Many draws per logit set come from
varying the step counter.
"""

import numpy as np
import pytest
import torch

from parity import NEAR_TIE_BUDGET, PROPOSE_NEAR_TIE, device_step, needs_gpu
from workloads import get_config, make_workload

pytestmark = [pytest.mark.gpu, needs_gpu]


def _check(wl, steps, argmax=True, seeds=None):
    from introspective_strided_decoding_amd import _lib
    from oracle import propose as oprop
    st = device_step(wl)
    B, N, V = wl.mask_logits.shape
    rows = np.asarray(wl.mask_logits, dtype=np.float64)
    draws = near = 0
    for k in range(steps):
        step = wl.step + k
        seed = wl.philox_seed if seeds is None else seeds[k % len(seeds)]
        st.propose(step=step, seed=seed)
        got = st.next_proposals.cpu().numpy()
        for r in range(B):
            u = oprop.stride_proposal_uniforms(seed, int(wl.req_ids[r]), int(wl.positions[r]), step, N)
            for j in range(N):
                y, margin = oprop.sample_row(rows[r, j], u[j])
                draws += 1
                if margin < PROPOSE_NEAR_TIE:
                    near += 1
                    continue
                assert got[r, j] == y, (wl.cfg.name, step, r, j, got[r, j], y, margin)
    assert near / max(1, draws) < NEAR_TIE_BUDGET, (near, draws)
    if argmax:
        st.propose(mode=_lib.PROPOSE_ARGMAX)
        got = st.next_proposals.cpu().numpy()
        want = np.array([[oprop.argmax_row(rows[r, j]) for j in range(N)] for r in range(B)])
        assert (got == want).all()
    from introspective_strided_decoding_amd import isd_read_flags
    assert isd_read_flags(st.workspace) == 0
    return draws


def test_propose_tiny_fp32_many_draws():
    wl = make_workload(get_config("tiny_fp32"), with_logits=False, with_mask_logits=True)
    assert _check(wl, 500, seeds=[wl.philox_seed, (1, 2)]) == 1000


def test_propose_headline_shape_bf16():
    wl = make_workload(get_config("c32_ctx4k"), with_logits=False, with_mask_logits=True)
    _check(wl, 12)


@pytest.mark.parametrize("over", [
    dict(batch=3, ctx=16, vocab=1003, stride_n=4),          # rows not 16-byte aligned, one shard
    dict(batch=2, ctx=16, vocab=4096, stride_n=3),          # exactly one full shard
    dict(batch=2, ctx=16, vocab=4097, stride_n=3),          # one entry in the last shard
    dict(batch=2, ctx=16, vocab=1, stride_n=2),             # a single token
    dict(batch=4, ctx=16, vocab=50000, stride_n=8),         # ragged last shard, N = 8
])
def test_propose_small_shapes_bf16(over):
    wl = make_workload(get_config("b8_ctx2k", **over), with_logits=False, with_mask_logits=True)
    _check(wl, 30)


def test_propose_extreme_and_tied_logits():
    """Huge and tiny logits, -inf entries, constant rows and exact argmax ties."""
    wl = make_workload(get_config("b8_ctx2k", batch=4, ctx=16, vocab=9000, stride_n=4),
                       with_logits=False, with_mask_logits=True)
    m = wl.mask_logits
    m[0, 0, :] = 0.0                       # uniform row: argmax 0
    m[0, 1, 123] = 900.0                   # one dominant logit far past exp's range
    m[0, 2, :] -= 2000.0                   # every logit far below it
    m[0, 3, 5000:] = -np.inf               # a masked tail
    m[1, 0, ::7] = 8.0                     # many exact maxima
    m[1, 1, :4500] = -np.inf               # a masked head
    m[2, 2, 8999] = 50.0                   # maximum in the last entry
    wl.mask_logits = torch.from_numpy(m).to(torch.bfloat16).float().numpy()
    _check(wl, 30)


@pytest.mark.parametrize("vocab", [2048 * 1024, 2048 * 1024 - 5])
def test_propose_largest_vocabulary(vocab):
    """The largest vocabulary the accept path takes, exactly full and ragged."""
    wl = make_workload(get_config("b8_ctx2k", batch=1, ctx=16, vocab=vocab, stride_n=3), with_logits=False,
                       with_mask_logits=True)
    assert _check(wl, 6) == 18
