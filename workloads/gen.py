"""Seeded input generator for one ISD step.

Recipe (one reading of the workload text, applied to every config):

* Attention operands ``q``, ``k_new``, ``v_new`` and every slot of the KV page
  pool are i.i.d. N(0, 1), rounded to the config dtype.  The pool is filled in
  physical order, so slots that no request owns, and slots past a request's
  context in its last page, hold random values too (or NaN with
  ``junk="nan"``, to prove the kernels never read them).
* Each request owns ``ceil((L_r + Q) / page_size)`` pages: its context plus
  room for the stride it may commit.  Physical page ids come from a seeded
  permutation, so logically adjacent pages are scattered in the pool.  Unused
  page-table entries are -1.
* Anchor logits ``p ~ N(0, logit_std^2)`` rounded to the dtype; proposal logits
  ``q = round(p + tau * z)`` with ``z ~ N(0, 1)``.  ``tau`` is found by
  bisection on the *rounded* logits so that the mean over rows of
  ``sum_x min(softmax(p)(x), softmax(q)(x))`` hits the acceptance target
  (one tau for the batch, one per request, or one per row).
* Proposals: ``x_1`` uniform over the vocabulary (it is decided before this
  step and always kept); ``x_k`` for ``k >= 2`` is drawn from ``softmax(q)`` of
  the row that proposed it.
* LoRA operands (R-ISD configs): ``X, Y ~ N(0, 1)``, ``A, B ~ N(0, lora_std^2)``,
  all rounded to bf16; the gated rows are the N MASK rows of every stride.
* MASK-row logits (``with_mask_logits``), from which the next N proposals are
  drawn: ``N(0, logit_std^2)`` rounded to the dtype, drawn after everything
  above so the other fields do not depend on the flag.

Bulk normals come from ``torch.randn`` with a seeded CPU generator (fast and
deterministic for a given torch build); small integer draws come from numpy's
PCG64.  The softmax used here only shapes the workload (it sets tau and draws
proposals); it is not the oracle's and not the kernels'.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .configs import WorkloadConfig


def _round(x: torch.Tensor, dtype: str) -> torch.Tensor:
    """Round a float32 tensor to the workload dtype, returned as float32."""
    if dtype == "bf16":
        return x.to(torch.bfloat16).to(torch.float32)
    if dtype == "f32":
        return x.to(torch.float32)
    raise ValueError(dtype)


def stride_rows(cfg: WorkloadConfig):
    """(clean_rows, mask_rows) of one stride: rows 0..N-2 are CLEAN, N-1..2N-2 MASK."""
    n = cfg.stride_n
    return list(range(0, n - 1)), list(range(n - 1, 2 * n - 1))


@dataclass
class Workload:
    cfg: WorkloadConfig
    seed: int
    ctx_lens: np.ndarray        # [B] int32
    page_table: np.ndarray      # [B, max_pages] int32, -1 = unmapped
    k_pool: np.ndarray          # [P, page_size, Hkv, D] float32 (dtype-rounded values)
    v_pool: np.ndarray          # [P, page_size, Hkv, D]
    q: np.ndarray               # [B, Q, Hq, D]
    k_new: np.ndarray           # [B, Q, Hkv, D]
    v_new: np.ndarray           # [B, Q, Hkv, D]
    p_logits: np.ndarray        # [B, N-1, V] anchor logits of the CLEAN rows
    q_logits: np.ndarray        # [B, N-1, V] proposal logits saved from the previous pass
    proposals: np.ndarray       # [B, N] int32: x_1..x_N
    req_ids: np.ndarray         # [B] int32
    positions: np.ndarray       # [B] int32: absolute position of x_1
    step: int
    philox_seed: tuple          # (lo, hi) 64-bit key
    tau: np.ndarray             # [B] noise scale used per request
    lora_x: Optional[np.ndarray] = None   # [B*Q, d]
    lora_a: Optional[np.ndarray] = None   # [d, r]
    lora_b: Optional[np.ndarray] = None   # [r, d]
    lora_y: Optional[np.ndarray] = None   # [B*Q, d]
    mask_rows: Optional[np.ndarray] = None  # [B*N] int32
    mask_logits: Optional[np.ndarray] = None  # [B, N, V] logits of the MASK rows

    @property
    def num_pages(self) -> int:
        return self.k_pool.shape[0]

    @property
    def max_pages(self) -> int:
        return self.page_table.shape[1]


def _acceptance_by_row(lp: torch.Tensor, lq: torch.Tensor) -> torch.Tensor:
    """sum_x min(p, q) per row, float64, for shaping the workload only."""
    p = torch.softmax(lp.to(torch.float64), dim=-1)
    q = torch.softmax(lq.to(torch.float64), dim=-1)
    return torch.minimum(p, q).sum(dim=-1)


def _fit_tau(p: torch.Tensor, z: torch.Tensor, dtype: str, groups: torch.Tensor,
             targets: torch.Tensor, iters: int = 40, tol: float = 2e-5) -> torch.Tensor:
    """Bisect one tau per group so that the mean acceptance over the group's rows hits its target.

    p, z: [R, V] float32; groups: [R] int64 group id per row; targets: [G] float64.
    Returns tau per group [G] float64.
    """
    g = targets.shape[0]
    lo = torch.zeros(g, dtype=torch.float64)
    hi = torch.full((g,), 2.0, dtype=torch.float64)
    counts = torch.bincount(groups, minlength=g).to(torch.float64)

    p_prob = torch.softmax(p.to(torch.float64), dim=-1)

    def mean_acc(tau_g):
        tau_rows = tau_g[groups].to(torch.float32).unsqueeze(1)
        lq = _round(p + tau_rows * z, dtype)
        q_prob = torch.softmax(lq.to(torch.float64), dim=-1)
        acc = torch.minimum(p_prob, q_prob).sum(dim=-1)
        return torch.zeros(g, dtype=torch.float64).index_add_(0, groups, acc) / counts

    # grow hi until the acceptance there is below target
    for _ in range(20):
        a = mean_acc(hi)
        need = a > targets
        if not bool(need.any()):
            break
        hi = torch.where(need, hi * 2.0, hi)
    tau = (lo + hi) / 2
    for _ in range(iters):
        tau = (lo + hi) / 2
        a = mean_acc(tau)
        if bool(((a - targets).abs() < tol).all()):
            break
        too_high = a > targets          # acceptance too high -> more noise
        lo = torch.where(too_high, tau, lo)
        hi = torch.where(too_high, hi, tau)
    return tau


def make_workload(cfg: WorkloadConfig, seed: Optional[int] = None, *, junk: str = "random",
                  tau_mode: Optional[str] = None, with_logits: bool = True,
                  with_mask_logits: bool = False, extra_tokens: int = 0) -> Workload:
    """Build one seeded ISD step input for ``cfg``.

    tau_mode: "batch" (one tau for the whole batch), "request" or "row".  Default: "request"
    when the config draws a target per request, else "batch".
    extra_tokens: page room for that many more tokens per request (a decoding loop commits
    into it); 0 keeps the recipe's allocation.
    """
    if seed is None:
        seed = cfg.seed_base
    rng = np.random.Generator(np.random.PCG64(seed))
    tg = torch.Generator().manual_seed(int(seed) * 7919 + 17)

    B, N, Q = cfg.batch, cfg.stride_n, cfg.q_rows
    Hq, Hkv, D, V, ps = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.vocab, cfg.page_size
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")

    # context lengths
    if cfg.ctx is not None:
        ctx = np.full(B, cfg.ctx, dtype=np.int32)
    else:
        lo, hi = cfg.ctx_range
        ctx = rng.integers(lo, hi + 1, size=B).astype(np.int32)

    # shuffled page allocation
    pages_per = (ctx.astype(np.int64) + Q + int(extra_tokens) + ps - 1) // ps
    n_pages = int(pages_per.sum())
    perm = rng.permutation(n_pages).astype(np.int32)
    max_pages = int(pages_per.max())
    table = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for r in range(B):
        table[r, : pages_per[r]] = perm[off: off + pages_per[r]]
        off += int(pages_per[r])

    def normals(*shape, std=1.0):
        x = torch.randn(*shape, generator=tg, dtype=torch.float32)
        if std != 1.0:
            x = x * std
        return x

    k_pool = _round(normals(n_pages, ps, Hkv, D), cfg.dtype)
    v_pool = _round(normals(n_pages, ps, Hkv, D), cfg.dtype)
    if junk == "nan":
        owned = np.zeros((n_pages, ps), dtype=bool)
        for r in range(B):
            for pos in range(int(ctx[r])):
                owned[table[r, pos // ps], pos % ps] = True
        mask = torch.from_numpy(~owned)
        k_pool[mask] = float("nan")
        v_pool[mask] = float("nan")
    elif junk != "random":
        raise ValueError(junk)

    q = _round(normals(B, Q, Hq, D), cfg.dtype)
    k_new = _round(normals(B, Q, Hkv, D), cfg.dtype)
    v_new = _round(normals(B, Q, Hkv, D), cfg.dtype)

    # logits and proposals
    R = B * (N - 1)
    targets_req = np.asarray(cfg.accept_targets, dtype=np.float64)
    if len(targets_req) == 1:
        req_target = np.full(B, targets_req[0])
    else:
        req_target = rng.choice(targets_req, size=B)
    if tau_mode is None:
        tau_mode = "request" if len(cfg.accept_targets) > 1 else "batch"
    proposals = np.zeros((B, N), dtype=np.int32)
    proposals[:, 0] = rng.integers(0, V, size=B)
    tau_req = np.zeros(B)
    if with_logits and R > 0:
        p = _round(normals(R, V, std=cfg.logit_std), cfg.dtype)
        z = normals(R, V)
        row_req = torch.arange(R) // (N - 1)
        if tau_mode == "batch":
            groups = torch.zeros(R, dtype=torch.int64)
            tgt = torch.tensor([float(req_target.mean())], dtype=torch.float64)
        elif tau_mode == "request":
            groups = row_req
            tgt = torch.from_numpy(req_target)
        elif tau_mode == "row":
            groups = torch.arange(R)
            tgt = torch.from_numpy(np.repeat(req_target, N - 1))
        else:
            raise ValueError(tau_mode)
        tau_g = _fit_tau(p, z, cfg.dtype, groups, tgt)
        tau_rows = tau_g[groups]
        lq = _round(p + tau_rows.to(torch.float32).unsqueeze(1) * z, cfg.dtype)
        tau_req = tau_rows.view(B, N - 1)[:, 0].numpy().copy()
        # proposals x_2..x_N ~ softmax(q) by inverse CDF
        qprob = torch.softmax(lq.to(torch.float64), dim=-1)
        cdf = torch.cumsum(qprob, dim=-1)
        u = torch.from_numpy(rng.random(R)).unsqueeze(1) * cdf[:, -1:]
        idx = torch.searchsorted(cdf, u, right=True).clamp_(max=V - 1).squeeze(1)
        proposals[:, 1:] = idx.view(B, N - 1).numpy().astype(np.int32)
        p_logits = p.view(B, N - 1, V).numpy()
        q_logits = lq.view(B, N - 1, V).numpy()
        del qprob, cdf
    else:
        p_logits = np.zeros((B, max(N - 1, 0), V), dtype=np.float32)
        q_logits = np.zeros((B, max(N - 1, 0), V), dtype=np.float32)

    req_ids = (rng.permutation(max(4 * B, 16))[:B] + 1000 * (seed % 1000)).astype(np.int32)
    positions = ctx.copy()
    step = int(rng.integers(0, 1 << 20))
    key = rng.integers(0, np.iinfo(np.int64).max, size=2, dtype=np.int64).astype(np.uint64)
    philox_seed = (int(key[0]), int(key[1]))

    wl = Workload(cfg=cfg, seed=seed, ctx_lens=ctx, page_table=table,
                  k_pool=k_pool.numpy(), v_pool=v_pool.numpy(), q=q.numpy(),
                  k_new=k_new.numpy(), v_new=v_new.numpy(), p_logits=p_logits,
                  q_logits=q_logits, proposals=proposals, req_ids=req_ids,
                  positions=positions, step=step, philox_seed=philox_seed, tau=tau_req)

    if cfg.lora:
        d, rk = cfg.lora_dim, cfg.lora_rank
        rows = B * Q
        wl.lora_x = _round(normals(rows, d), "bf16").numpy()
        wl.lora_a = _round(normals(d, rk, std=cfg.lora_std), "bf16").numpy()
        wl.lora_b = _round(normals(rk, d, std=cfg.lora_std), "bf16").numpy()
        wl.lora_y = _round(normals(rows, d), "bf16").numpy()
        _, mrows = stride_rows(cfg)
        wl.mask_rows = (np.arange(B)[:, None] * Q + np.asarray(mrows)[None, :]).reshape(-1).astype(np.int32)
    if with_mask_logits:
        wl.mask_logits = _round(normals(B, N, V, std=cfg.logit_std), cfg.dtype).numpy()
    return wl
