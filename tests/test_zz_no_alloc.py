"""isd_accept_commit_noalloc: the accept + commit call without a caller workspace.

Two calls in a row through the C ABI, the second on a smaller input (fewer
requests, shorter vocabulary), each against isd_accept_commit on the same
inputs: every output, both pools and the lengths bit for bit, the flag word
clear; the first call's accept results also against the oracle.  The calls
share the library's per-device scratch, so the second call also shows that
the first left its counters rewound.
"""

import pytest
import torch

from parity import AcceptTally, check_accept_step, device_step, fetch_accept, needs_gpu
from workloads import get_config, make_workload

pytestmark = [pytest.mark.gpu, needs_gpu]

OUTPUTS = ("accept_len", "out_tokens", "n_out", "n_commit", "logp_sel", "logq_sel", "ctx_lens_out",
           "k_pages", "v_pages")


def _bits(t):
    return t.contiguous().view(torch.uint8).cpu()


def _noalloc(st, flags):
    from introspective_strided_decoding_amd import _lib
    _lib.isd_accept_commit_noalloc(
        st.shape, st.p_logits, st.q_logits, st.proposals, st.req_ids, st.positions, st.seed, st.step,
        st.accept_len, st.out_tokens, st.n_out, st.n_commit, st.logp_sel, st.logq_sel, st.k_new, st.v_new,
        st.k_pages, st.v_pages, st.page_table, st.ctx_lens, st.ctx_lens_out, flags=flags)


@pytest.mark.parametrize("name", ["b8_ctx2k", "c64_ragged"])
def test_noalloc_matches_accept_commit_twice(name):
    from introspective_strided_decoding_amd import isd_read_flags
    big = dict(batch=24, vocab=151936) if name == "b8_ctx2k" else dict(batch=20, vocab=151936)
    small = dict(batch=5, vocab=40003) if name == "b8_ctx2k" else dict(batch=3, vocab=9000)
    for k, over in enumerate((big, small)):
        if name == "b8_ctx2k":
            over = dict(over, ctx=300 if k == 0 else 70)
        else:
            over = dict(over, ctx_range=(20, 400))
        wl = make_workload(get_config(name, **over), seed=90 + k)
        ref = device_step(wl)
        got = device_step(wl)
        flags = torch.zeros(1, dtype=torch.int32, device=got.q.device)
        ref.accept_commit()
        _noalloc(got, flags)
        torch.cuda.synchronize()
        for f in OUTPUTS:
            assert torch.equal(_bits(getattr(ref, f)), _bits(getattr(got, f))), (name, k, f)
        assert int(flags.item()) == 0 and isd_read_flags(ref.workspace) == 0
        if k == 0:
            tally = AcceptTally()
            check_accept_step(wl, fetch_accept(got), wl.philox_seed, wl.step, tally)
            assert tally.requests == wl.cfg.batch
