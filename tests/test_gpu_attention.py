"""isd_attention on the GPU vs the float64 oracle, element by element.

Small cases span several 32-token tiles, ragged tails (context not a multiple
of the tile or the page), empty contexts, GQA groups of 1, 2 and 4, stride
sizes N = 2..8 and 16 (one and two 32-column row blocks; Q = 31 fills the
stride tile), head dims 64 and 128, fp32
and bf16, and NaN in every pool slot no request owns.  Full-size cases use
the five named workloads at their real shapes (launch configuration as in
the benchmark) and check every request.
"""

import numpy as np
import pytest
import torch

from parity import check_attention, device_step, needs_gpu
from workloads import get_config, make_workload

pytestmark = [pytest.mark.gpu, needs_gpu]

SMALL = [
    ("tiny_fp32", {}),
    ("tiny_fp32", dict(ctx=0)),
    ("tiny_fp32", dict(ctx=37, stride_n=4, n_q_heads=4, n_kv_heads=2, batch=3)),
    ("tiny_fp32", dict(ctx=200, head_dim=128, n_q_heads=8, n_kv_heads=2, stride_n=3)),
    ("b8_ctx2k", dict(batch=3, ctx=1, vocab=64)),
    ("b8_ctx2k", dict(batch=3, ctx=15, vocab=64)),
    ("b8_ctx2k", dict(batch=3, ctx=16, vocab=64)),
    ("b8_ctx2k", dict(batch=3, ctx=17, vocab=64)),
    ("b8_ctx2k", dict(batch=3, ctx=33, vocab=64)),
    ("b8_ctx2k", dict(batch=2, ctx=0, vocab=64)),
    ("b8_ctx2k", dict(batch=2, ctx=777, vocab=64)),
    ("b8_ctx2k", dict(batch=2, ctx=300, vocab=64, head_dim=64)),
    ("b8_ctx2k", dict(batch=2, ctx=129, vocab=64, n_q_heads=16, n_kv_heads=8, stride_n=2)),
    ("c64_ragged", dict(batch=5, ctx_range=(1, 700), vocab=64)),          # N=8: 60 rows, two blocks
    ("c64_ragged", dict(batch=3, ctx_range=(30, 90), vocab=64, head_dim=64)),
    ("b8_ctx2k", dict(batch=2, ctx=70, vocab=64, n_q_heads=16, n_kv_heads=8, stride_n=16)),  # Q = 31, two blocks
    ("tiny_fp32", dict(ctx=45, stride_n=16, n_q_heads=2, n_kv_heads=2, batch=2)),            # Q = 31, fp32
]


@pytest.mark.parametrize("name,over", SMALL, ids=[f"{n}-{i}" for i, (n, _) in enumerate(SMALL)])
def test_attention_small(name, over):
    wl = make_workload(get_config(name, **over), seed=11, with_logits=False)
    st = device_step(wl)
    st.attention()
    torch.cuda.synchronize()
    check_attention(wl, st.out)
    from introspective_strided_decoding_amd import isd_read_flags
    assert isd_read_flags(st.workspace) == 0


@pytest.mark.parametrize("name", ["b8_ctx2k", "c64_ragged"])
def test_attention_never_reads_unowned_slots(name):
    over = dict(batch=3, vocab=64)
    over.update(dict(ctx=45) if name == "b8_ctx2k" else dict(ctx_range=(5, 80)))
    wl = make_workload(get_config(name, **over), seed=12, with_logits=False, junk="nan")
    st = device_step(wl)
    st.attention()
    torch.cuda.synchronize()
    check_attention(wl, st.out)


def test_attention_split_boundaries():
    """max_ctx hints that force many splits (and one split) give the same result."""
    wl = make_workload(get_config("b8_ctx2k", batch=2, ctx=1000, vocab=64), seed=13, with_logits=False)
    outs = []
    for hint in (0, 64, 256, 1000, 5000):
        st = device_step(wl, max_ctx=hint)
        st.attention()
        torch.cuda.synchronize()
        check_attention(wl, st.out)
        outs.append(st.out.float().cpu())
    for o in outs[1:]:
        assert torch.allclose(o, outs[0], atol=2e-2, rtol=0)


def test_attention_deterministic():
    wl = make_workload(get_config("b8_ctx2k", batch=4, ctx=500, vocab=64), seed=14, with_logits=False)
    st = device_step(wl)
    st.attention()
    a = st.out.clone()
    st.attention()
    torch.cuda.synchronize()
    assert torch.equal(a, st.out)


@pytest.mark.parametrize("name", ["tiny_fp32", "b8_ctx2k", "c32_ctx4k", "c64_ragged", "c128_lora"])
def test_attention_full_size(name):
    """Every request of every named workload at its real shape, in the launch
    configuration the benchmark times (one workgroup set per call, the plan's own
    splits), element by element against the oracle."""
    cfg = get_config(name)
    wl = make_workload(cfg, with_logits=False)
    st = device_step(wl, max_ctx=int(wl.ctx_lens.max()))
    st.attention()
    torch.cuda.synchronize()
    check_attention(wl, st.out)
    from introspective_strided_decoding_amd import isd_read_flags
    assert isd_read_flags(st.workspace) == 0


@pytest.mark.parametrize("batch", [300, 520])
def test_attention_many_requests_past_ranking_limit(batch):
    """More requests than the in-kernel longest-first ranking handles (256) and a grid of
    several rounds: the workgroups fall back to index order; every sampled request is
    exact, including the first and last ones."""
    cfg = get_config("b8_ctx2k", batch=batch, ctx_range=(1, 300), ctx=None, vocab=64)
    wl = make_workload(cfg, seed=15, with_logits=False)
    st = device_step(wl)
    st.attention()
    torch.cuda.synchronize()
    order = np.argsort(wl.ctx_lens)
    check_attention(wl, st.out, requests=[0, batch - 1, int(order[0]), int(order[-1]), batch // 2])
    from introspective_strided_decoding_amd import isd_read_flags
    assert isd_read_flags(st.workspace) == 0
