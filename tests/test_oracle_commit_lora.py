"""Pins for oracle.commit and oracle.lora.

commit: after appending the committed rows, attention for the next stride
(torch SDPA on the explicit dense sequence) equals the oracle's paged
attention with the grown context; only the named slots change.

lora: brute-force triple loop on a tiny case; A = 0 and an empty gate leave
Y unchanged; CLEAN rows never change; the delta is linear in the scale.

gated projection: explicit loops on a tiny case; identity weights return the
input; zero weights reduce to the delta alone; CLEAN rows equal the base
projection bit for bit; the adapter is a rank-r update.
"""

import numpy as np
import torch

from oracle.attention import stride_attention
from oracle.commit import kv_commit
from oracle.lora import gated_lora_delta, gated_projection
from workloads import get_config, make_workload


def _dense(pool, table, L, ps):
    pos = np.arange(L)
    return pool[table[pos // ps], pos % ps].astype(np.float64)


def test_commit_then_attend_equals_dense_extended_sequence():
    cfg = get_config("tiny_fp32", batch=3, ctx=29, stride_n=4, n_q_heads=4, n_kv_heads=2)
    wl = make_workload(cfg, seed=12, with_logits=False)
    n_commit = np.array([3, 0, 2])
    k2, v2, lens2 = kv_commit(wl.k_pool, wl.v_pool, wl.page_table, wl.ctx_lens, wl.k_new,
                              wl.v_new, n_commit, cfg.page_size)
    assert list(lens2) == list(wl.ctx_lens + n_commit)
    # a fresh stride on top of the grown context
    nxt = make_workload(cfg, seed=13, with_logits=False)
    out = stride_attention(nxt.q, nxt.k_new, nxt.v_new, k2, v2, wl.page_table, lens2, cfg.page_size)
    for r in range(cfg.batch):
        L = int(wl.ctx_lens[r])
        n = int(n_commit[r])
        k = np.concatenate([_dense(wl.k_pool, wl.page_table[r], L, 16), wl.k_new[r, :n], nxt.k_new[r]], 0)
        v = np.concatenate([_dense(wl.v_pool, wl.page_table[r], L, 16), wl.v_new[r, :n], nxt.v_new[r]], 0)
        T, Q = k.shape[0], cfg.q_rows
        mask = torch.arange(T)[None, :] <= (L + n + torch.arange(Q))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(nxt.q[r].astype(np.float64)).permute(1, 0, 2)[None],
            torch.from_numpy(k).permute(1, 0, 2)[None].contiguous(),
            torch.from_numpy(v).permute(1, 0, 2)[None].contiguous(),
            attn_mask=mask, enable_gqa=True)[0].permute(1, 0, 2).numpy()
        np.testing.assert_allclose(out[r], ref, rtol=0, atol=1e-12)


def test_commit_touches_only_named_slots():
    cfg = get_config("tiny_fp32", batch=2, ctx=31, stride_n=4)
    wl = make_workload(cfg, seed=14, with_logits=False)
    n_commit = np.array([3, 1])
    k2, v2, _ = kv_commit(wl.k_pool, wl.v_pool, wl.page_table, wl.ctx_lens, wl.k_new, wl.v_new,
                          n_commit, 16)
    changed = set(zip(*np.nonzero((k2 != wl.k_pool).any(axis=(2, 3)))))
    expect = set()
    for r in range(2):
        for i in range(n_commit[r]):
            pos = wl.ctx_lens[r] + i
            expect.add((int(wl.page_table[r, pos // 16]), int(pos % 16)))
            assert np.array_equal(k2[wl.page_table[r, pos // 16], pos % 16], wl.k_new[r, i])
            assert np.array_equal(v2[wl.page_table[r, pos // 16], pos % 16], wl.v_new[r, i])
    assert changed == expect


def test_commit_nothing_is_identity():
    cfg = get_config("tiny_fp32", ctx=10)
    wl = make_workload(cfg, seed=15, with_logits=False)
    k2, v2, lens = kv_commit(wl.k_pool, wl.v_pool, wl.page_table, wl.ctx_lens, wl.k_new, wl.v_new,
                             np.zeros(1, int), 16)
    assert np.array_equal(k2, wl.k_pool) and np.array_equal(v2, wl.v_pool)
    assert list(lens) == list(wl.ctx_lens)


def test_lora_brute_force():
    rng = np.random.Generator(np.random.PCG64(16))
    rows, d_in, rank, d_out = 5, 6, 3, 4
    x, a = rng.normal(size=(rows, d_in)), rng.normal(size=(d_in, rank))
    b, y = rng.normal(size=(rank, d_out)), rng.normal(size=(rows, d_out))
    mask = [1, 4]
    got = gated_lora_delta(x, a, b, y, mask, scale=0.5)
    want = y.copy()
    for m in mask:
        for o in range(d_out):
            acc = 0.0
            for k in range(rank):
                t = 0.0
                for i in range(d_in):
                    t += x[m, i] * a[i, k]
                acc += t * b[k, o]
            want[m, o] += 0.5 * acc
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_lora_special_cases():
    rng = np.random.Generator(np.random.PCG64(17))
    x, a = rng.normal(size=(7, 8)), rng.normal(size=(8, 2))
    b, y = rng.normal(size=(2, 8)), rng.normal(size=(7, 8))
    assert np.array_equal(gated_lora_delta(x, np.zeros_like(a), b, y, [0, 3]), y)
    assert np.array_equal(gated_lora_delta(x, a, b, y, []), y)
    out = gated_lora_delta(x, a, b, y, [2, 5])
    keep = [0, 1, 3, 4, 6]
    assert np.array_equal(out[keep], y[keep])
    d1 = gated_lora_delta(x, a, b, y, [2, 5], scale=1.0) - y
    d2 = gated_lora_delta(x, a, b, y, [2, 5], scale=2.0) - y
    np.testing.assert_allclose(d2, 2 * d1, rtol=1e-14, atol=1e-14)


def test_gated_projection_brute_force():
    """Every output element by explicit loops: base product on all rows, the adapter's
    two products added on the gated rows only."""
    rng = np.random.Generator(np.random.PCG64(18))
    rows, d_in, rank, d_out = 6, 5, 2, 3
    x, w = rng.normal(size=(rows, d_in)), rng.normal(size=(d_in, d_out))
    a, b = rng.normal(size=(d_in, rank)), rng.normal(size=(rank, d_out))
    mask = [0, 3, 4]
    got = gated_projection(x, w, a, b, mask, scale=0.75)
    for m in range(rows):
        for o in range(d_out):
            want = sum(x[m, i] * w[i, o] for i in range(d_in))
            if m in mask:
                want += 0.75 * sum(sum(x[m, i] * a[i, k] for i in range(d_in)) * b[k, o] for k in range(rank))
            assert abs(got[m, o] - want) <= 1e-12 * (1 + abs(want)), (m, o)


def test_gated_projection_special_cases():
    rng = np.random.Generator(np.random.PCG64(19))
    x, w = rng.normal(size=(7, 8)), rng.normal(size=(8, 8))
    a, b = rng.normal(size=(8, 2)), rng.normal(size=(2, 8))
    mask = [1, 2, 6]
    out = gated_projection(x, w, a, b, mask)
    # identity weights: the base product is the input itself
    np.testing.assert_array_equal(gated_projection(x, np.eye(8), None, None, []), x)
    # zero base weights: only the gated delta is left, as the delta alone computes it
    np.testing.assert_allclose(gated_projection(x, np.zeros((8, 8)), a, b, mask),
                               gated_lora_delta(x, a, b, np.zeros((7, 8)), mask), rtol=0, atol=1e-13)
    # CLEAN rows are bit for bit the base projection; no adapter = empty gate
    base = gated_projection(x, w, None, None, [])
    clean = [0, 3, 4, 5]
    assert np.array_equal(out[clean], base[clean])
    assert np.array_equal(gated_projection(x, w, a, b, []), base)
    # the adapter is a rank-2 update of the gated rows
    assert np.linalg.matrix_rank(out[mask] - base[mask]) <= 2
