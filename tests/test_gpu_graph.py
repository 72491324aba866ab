"""The step recorded into a HIP graph and replayed.

A graph of one whole step (attention -> accept -> commit -> proposals) must
reproduce the eager step bit for bit on every replay, and the replayed outputs
must match the oracle on the same inputs (attention element-wise, accept
results, both pools, lengths and proposals).  Between replays the outputs are
cleared and unrelated eager work runs on the same device, so a replay that
skipped a kernel, or a counter that was not rewound, shows up as a difference.
"""

import pytest
import torch

from parity import check_step_against_oracle, device_step, needs_gpu
from workloads import get_config, make_workload

pytestmark = [pytest.mark.gpu, needs_gpu]

OUTPUTS = ("out", "accept_len", "out_tokens", "n_out", "n_commit", "logp_sel", "logq_sel",
           "ctx_lens_out", "next_proposals", "k_pages", "v_pages")


def _snapshot(st):
    return {k: getattr(st, k).clone() for k in OUTPUTS}


def _clear(st):
    for k in OUTPUTS:
        if k not in ("k_pages", "v_pages"):
            getattr(st, k).zero_()


@pytest.mark.parametrize("name,over", [
    ("b8_ctx2k", dict(batch=8, ctx=600, vocab=20000)),
    ("c64_ragged", dict(batch=6, vocab=30000)),           # several KV splits, N = 8
    ("tiny_fp32", {}),
])
def test_graph_replays_match_eager(name, over):
    wl = make_workload(get_config(name, **over), with_mask_logits=True)
    st = device_step(wl, max_ctx=int(wl.ctx_lens.max()))
    other = device_step(make_workload(get_config(name, **over), seed=99, with_mask_logits=True))
    st.run()
    torch.cuda.synchronize()
    ref = _snapshot(st)
    graph = st.capture()
    for rep in range(4):
        _clear(st)
        other.run()                                  # eager work of another step in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        if rep == 0:
            check_step_against_oracle(wl, st)           # the replay against the oracle
        for k in OUTPUTS:
            assert torch.equal(getattr(st, k), ref[k]), (name, rep, k)
    from introspective_strided_decoding_amd import isd_read_flags
    assert isd_read_flags(st.workspace) == 0
