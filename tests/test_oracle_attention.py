"""Pins for oracle.attention.

* torch's scaled_dot_product_attention (float64, CPU, its own GQA head mapping)
  on a dense copy of the context is the library reference;
* closed forms: an empty context makes row 0 copy its own value, constant keys
  make every row the mean of the values it can see;
* invariants: relabelling physical pages changes nothing; later stride rows
  never influence earlier ones.
"""

import math

import numpy as np
import pytest
import torch

from oracle.attention import stride_attention
from workloads import get_config, make_workload


def _dense_context(pool, table, L, ps):
    """Logical context by an independent vectorised gather."""
    pos = np.arange(L)
    return pool[table[pos // ps], pos % ps].astype(np.float64)   # [L, Hkv, D]


def _sdpa_reference(wl, r):
    cfg = wl.cfg
    L = int(wl.ctx_lens[r])
    Q = cfg.q_rows
    k = np.concatenate([_dense_context(wl.k_pool, wl.page_table[r], L, cfg.page_size), wl.k_new[r]], 0)
    v = np.concatenate([_dense_context(wl.v_pool, wl.page_table[r], L, cfg.page_size), wl.v_new[r]], 0)
    qt = torch.from_numpy(wl.q[r].astype(np.float64)).permute(1, 0, 2).unsqueeze(0)   # [1, Hq, Q, D]
    kt = torch.from_numpy(k).permute(1, 0, 2).unsqueeze(0).contiguous()            # [1, Hkv, T, D]
    vt = torch.from_numpy(v).permute(1, 0, 2).unsqueeze(0).contiguous()
    T = L + Q
    mask = torch.arange(T)[None, :] <= (L + torch.arange(Q))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()                                            # [Q, Hq, D]


@pytest.mark.parametrize("overrides", [
    dict(),                                                    # tiny fp32 config as given
    dict(ctx=37, n_q_heads=4, n_kv_heads=2, stride_n=3),       # ragged last page, G=2
    dict(ctx=16, n_q_heads=6, n_kv_heads=3, stride_n=4, head_dim=32),
    dict(ctx=1, stride_n=5),
])
def test_matches_sdpa(overrides):
    cfg = get_config("tiny_fp32", **overrides)
    wl = make_workload(cfg, seed=5, with_logits=False)
    out = stride_attention(wl.q, wl.k_new, wl.v_new, wl.k_pool, wl.v_pool, wl.page_table,
                           wl.ctx_lens, cfg.page_size)
    for r in range(cfg.batch):
        np.testing.assert_allclose(out[r], _sdpa_reference(wl, r), rtol=0, atol=1e-12)


def test_bf16_batch_matches_sdpa_on_sample():
    cfg = get_config("b8_ctx2k", batch=3, ctx=300, vocab=64)
    wl = make_workload(cfg, seed=9, with_logits=False)
    out = stride_attention(wl.q, wl.k_new, wl.v_new, wl.k_pool, wl.v_pool, wl.page_table,
                           wl.ctx_lens, cfg.page_size, requests=[2])
    np.testing.assert_allclose(out[0], _sdpa_reference(wl, 2), rtol=0, atol=1e-11)


def test_empty_context_row0_copies_its_value():
    cfg = get_config("tiny_fp32", ctx=0, n_q_heads=4, n_kv_heads=2)
    wl = make_workload(cfg, seed=1, with_logits=False)
    out = stride_attention(wl.q, wl.k_new, wl.v_new, wl.k_pool, wl.v_pool, wl.page_table,
                           wl.ctx_lens, cfg.page_size)
    G = cfg.group
    for h in range(cfg.n_q_heads):
        np.testing.assert_allclose(out[0, 0, h], wl.v_new[0, 0, h // G], rtol=0, atol=1e-15)


def test_constant_keys_give_mean_of_visible_values():
    cfg = get_config("tiny_fp32", ctx=45, stride_n=3)
    wl = make_workload(cfg, seed=2, with_logits=False)
    wl.k_pool[:] = 0.25
    wl.k_new[:] = 0.25
    out = stride_attention(wl.q, wl.k_new, wl.v_new, wl.k_pool, wl.v_pool, wl.page_table,
                           wl.ctx_lens, cfg.page_size)
    L = int(wl.ctx_lens[0])
    ctx_v = _dense_context(wl.v_pool, wl.page_table[0], L, cfg.page_size)
    for i in range(cfg.q_rows):
        vis = np.concatenate([ctx_v, wl.v_new[0, : i + 1].astype(np.float64)], 0)
        for h in range(cfg.n_q_heads):
            np.testing.assert_allclose(out[0, i, h], vis[:, h // cfg.group].mean(0), rtol=0, atol=1e-13)


def test_page_relabelling_invariance():
    cfg = get_config("tiny_fp32", batch=3, ctx=70, n_q_heads=4, n_kv_heads=2)
    wl = make_workload(cfg, seed=3, with_logits=False)
    out1 = stride_attention(wl.q, wl.k_new, wl.v_new, wl.k_pool, wl.v_pool, wl.page_table,
                            wl.ctx_lens, cfg.page_size)
    perm = np.random.Generator(np.random.PCG64(0)).permutation(wl.num_pages)
    k2 = np.empty_like(wl.k_pool)
    v2 = np.empty_like(wl.v_pool)
    k2[perm] = wl.k_pool
    v2[perm] = wl.v_pool
    table2 = np.where(wl.page_table >= 0, perm[np.maximum(wl.page_table, 0)], -1)
    out2 = stride_attention(wl.q, wl.k_new, wl.v_new, k2, v2, table2, wl.ctx_lens, cfg.page_size)
    assert np.array_equal(out1, out2)


def test_later_rows_do_not_leak_backwards():
    """Changing stride row j's key/value leaves rows i < j unchanged (strict causality)."""
    cfg = get_config("tiny_fp32", ctx=20, stride_n=3)
    wl = make_workload(cfg, seed=4, with_logits=False)
    base = stride_attention(wl.q, wl.k_new, wl.v_new, wl.k_pool, wl.v_pool, wl.page_table,
                            wl.ctx_lens, cfg.page_size)
    j = 2
    wl.k_new[0, j] += 3.0
    wl.v_new[0, j] -= 5.0
    moved = stride_attention(wl.q, wl.k_new, wl.v_new, wl.k_pool, wl.v_pool, wl.page_table,
                             wl.ctx_lens, cfg.page_size)
    assert np.array_equal(base[0, :j], moved[0, :j])
    assert not np.allclose(base[0, j:], moved[0, j:])


def test_nan_junk_outside_context_is_never_read():
    cfg = get_config("tiny_fp32", ctx=37, stride_n=3)
    wl = make_workload(cfg, seed=6, with_logits=False, junk="nan")
    out = stride_attention(wl.q, wl.k_new, wl.v_new, wl.k_pool, wl.v_pool, wl.page_table,
                           wl.ctx_lens, cfg.page_size)
    assert np.isfinite(out).all()


def test_scale_is_inverse_sqrt_head_dim():
    """Doubling q with scale halved reproduces the default result."""
    cfg = get_config("tiny_fp32", ctx=30)
    wl = make_workload(cfg, seed=8, with_logits=False)
    a = stride_attention(wl.q, wl.k_new, wl.v_new, wl.k_pool, wl.v_pool, wl.page_table,
                         wl.ctx_lens, cfg.page_size)
    b = stride_attention(2 * wl.q, wl.k_new, wl.v_new, wl.k_pool, wl.v_pool, wl.page_table,
                         wl.ctx_lens, cfg.page_size, scale=0.5 / math.sqrt(cfg.head_dim))
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)
