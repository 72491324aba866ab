"""Device buffers for one ISD step and the three calls in stream order.

``DeviceStep.from_arrays`` takes host arrays by name (numpy or torch: q,
k_new, v_new, plain page pools, page_table, ctx_lens, p/q logits, proposals,
req_ids, positions, step, philox_seed, and optionally the LoRA operands and
the MASK-row logits), moves them to the device in the library layouts,
allocates the outputs and the workspace, and ``run()`` enqueues
isd_attention -> isd_accept -> kv_commit (+ isd_lora_delta when LoRA
operands are present, + isd_propose when MASK-row logits are present).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

from . import _lib
from .layout import pack_k_pages, pack_v_pages


def _t(x, dtype, device):
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(np.ascontiguousarray(x))
    return x.to(device=device, dtype=dtype).contiguous()


@dataclass
class DeviceStep:
    shape: _lib.Shape
    q: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    k_pages: torch.Tensor
    v_pages: torch.Tensor
    page_table: torch.Tensor
    ctx_lens: torch.Tensor
    p_logits: torch.Tensor
    q_logits: torch.Tensor
    proposals: torch.Tensor
    req_ids: torch.Tensor
    positions: torch.Tensor
    step: int
    seed: tuple
    workspace: torch.Tensor
    out: torch.Tensor
    accept_len: torch.Tensor
    out_tokens: torch.Tensor
    n_out: torch.Tensor
    n_commit: torch.Tensor
    logp_sel: torch.Tensor
    logq_sel: torch.Tensor
    ctx_lens_out: torch.Tensor
    lora: Optional[dict] = None
    mask_logits: Optional[torch.Tensor] = None
    next_proposals: Optional[torch.Tensor] = None
    extra: dict = field(default_factory=dict)

    @classmethod
    def from_arrays(cls, a, device="cuda", max_ctx: int = 0, commit_in_place: bool = False):
        dt_name = a.cfg.dtype if hasattr(a, "cfg") else a.dtype
        kv = torch.bfloat16 if dt_name == "bf16" else torch.float32
        code = _lib.ISD_BF16 if dt_name == "bf16" else _lib.ISD_F32
        B, Q, Hq, D = a.q.shape
        Hkv = a.k_new.shape[2]
        N = (Q + 1) // 2
        P = a.k_pool.shape[0]
        V = a.p_logits.shape[-1]
        shape = _lib.Shape(batch=B, stride_n=N, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D,
                           max_pages=a.page_table.shape[1], num_pages=P, vocab=V, kv_dtype=code,
                           logit_dtype=code, max_ctx=max_ctx)
        i32 = torch.int32
        k_plain = _t(a.k_pool, kv, device)
        v_plain = _t(a.v_pool, kv, device)
        ctx = _t(a.ctx_lens, i32, device)
        st = cls(
            shape=shape, q=_t(a.q, kv, device), k_new=_t(a.k_new, kv, device), v_new=_t(a.v_new, kv, device),
            k_pages=pack_k_pages(k_plain), v_pages=pack_v_pages(v_plain),
            page_table=_t(a.page_table, i32, device), ctx_lens=ctx,
            p_logits=_t(a.p_logits, kv, device), q_logits=_t(a.q_logits, kv, device),
            proposals=_t(a.proposals, i32, device), req_ids=_t(a.req_ids, i32, device),
            positions=_t(a.positions, i32, device), step=int(a.step), seed=tuple(a.philox_seed),
            workspace=_lib.new_workspace(shape, device),
            out=torch.empty(B, Q, Hq, D, dtype=kv, device=device),
            accept_len=torch.empty(B, dtype=i32, device=device),
            out_tokens=torch.empty(B, N, dtype=i32, device=device),
            n_out=torch.empty(B, dtype=i32, device=device),
            n_commit=torch.empty(B, dtype=i32, device=device),
            logp_sel=torch.empty(B, N - 1, dtype=torch.float32, device=device),
            logq_sel=torch.empty(B, N - 1, dtype=torch.float32, device=device),
            ctx_lens_out=ctx if commit_in_place else torch.empty(B, dtype=i32, device=device),
        )
        del k_plain, v_plain
        if getattr(a, "mask_logits", None) is not None:
            st.mask_logits = _t(a.mask_logits, kv, device)
            st.next_proposals = torch.empty(B, N, dtype=i32, device=device)
        if getattr(a, "lora_x", None) is not None:
            bf = torch.bfloat16
            # linear-layer layouts: down weight [rank, d_in], up weight [d_out, rank]
            st.lora = dict(X=_t(a.lora_x, bf, device), A_t=_t(np.ascontiguousarray(a.lora_a.T), bf, device),
                           B_t=_t(np.ascontiguousarray(a.lora_b.T), bf, device), Y=_t(a.lora_y, bf, device),
                           mask_rows=_t(a.mask_rows, i32, device))
            n_mask = st.lora["mask_rows"].numel()
            nbytes = _lib.isd_lora_workspace_bytes(n_mask, st.lora["X"].shape[1], st.lora["A_t"].shape[0])
            st.lora["ws"] = torch.zeros(max(256, nbytes), dtype=torch.uint8, device=device)
        return st

    def __setattr__(self, name, value):
        # a buffer replaced by another drops the calls marshalled with the old one
        object.__setattr__(self, name, value)
        self.__dict__.pop("_calls", None)

    def _call(self, key, build):
        """The library call ``key``, checked and marshalled on first use (``build``)."""
        calls = self.__dict__.setdefault("_calls", {})
        c = calls.get(key)
        if c is None or c.lib is not _lib.LIB:
            c = calls[key] = build()
        return c

    def attention(self, stream=None, loop: bool = False):
        """``loop``: the decoding loop's forward, whose context length is the positions
        argument (the stride's first row sits there; while a resampled token waits for
        its row the committed length runs N - 1 ahead of it)."""
        self._call(("attention", loop), lambda: _lib.prepare(
            _lib.isd_attention, self.shape, self.q, self.k_new, self.v_new, self.k_pages, self.v_pages,
            self.page_table, self.positions if loop else self.ctx_lens, self.out, self.workspace))(stream)

    def _step_dev(self, device_step: bool):
        return self.extra["forwards"] if device_step else None

    def accept(self, stream=None, step: Optional[int] = None, seed=None, device_step: bool = False,
               q_norms=None):
        """``device_step``: each request's Philox step is its forward count on the device.
        ``q_norms``: the q rows' normalisers as the previous forward's proposals wrote them."""
        self._call(("accept", device_step, q_norms is not None), lambda: _lib.prepare(
            _lib.isd_accept, self.shape, self.p_logits, self.q_logits, self.proposals, self.req_ids,
            self.positions, self.seed, self.step, self.accept_len, self.out_tokens, self.n_out, self.n_commit,
            self.logp_sel, self.logq_sel, self.workspace, step_dev=self._step_dev(device_step),
            q_norms=q_norms))(
            stream, self.step if step is None else step, self.seed if seed is None else seed)

    def commit(self, stream=None):
        self._call("commit", lambda: _lib.prepare(
            _lib.kv_commit, self.shape, self.k_new, self.v_new, self.k_pages, self.v_pages, self.page_table,
            self.ctx_lens, self.n_commit, self.ctx_lens_out, self.workspace))(stream)

    def accept_commit(self, stream=None, step: Optional[int] = None, seed=None, device_step: bool = False,
                      q_norms=None, loop: bool = False):
        """accept, then commit of the accepted prefix, in one library call; ``loop``: by the
        decoding loop's mode, a re-proposing request commits its row N-1 instead (the token
        the forward before resampled)."""
        self._call(("accept_commit", device_step, q_norms is not None, loop), lambda: _lib.prepare(
            _lib.isd_accept_commit, self.shape, self.p_logits, self.q_logits, self.proposals, self.req_ids,
            self.positions, self.seed, self.step, self.accept_len, self.out_tokens, self.n_out, self.n_commit,
            self.logp_sel, self.logq_sel, self.k_new, self.v_new, self.k_pages, self.v_pages, self.page_table,
            self.ctx_lens, self.ctx_lens_out, self.workspace, step_dev=self._step_dev(device_step),
            q_norms=q_norms, loop_mode=self.extra["mode"] if loop else None))(
            stream, self.step if step is None else step, self.seed if seed is None else seed)

    def propose(self, stream=None, mode: int = _lib.PROPOSE_SAMPLE, step: Optional[int] = None, seed=None,
                device_step: bool = False, row_norms=None):
        """``row_norms``: written with the MASK rows' normalisers (sampling policy)."""
        self._call(("propose", mode, device_step, row_norms is not None), lambda: _lib.prepare(
            _lib.isd_propose, self.shape, self.mask_logits, self.req_ids, self.positions, self.seed,
            self.step, mode, self.next_proposals, self.workspace, step_dev=self._step_dev(device_step),
            row_norms=row_norms))(
            stream, self.step if step is None else step, self.seed if seed is None else seed)

    def loop_start(self):
        """Device state of the multi-step loop: every request starts verifying its proposals."""
        B = self.shape.batch
        dev = self.proposals.device
        self.__dict__.pop("_calls", None)    # calls marshalled with the old loop state
        self.extra["mode"] = torch.zeros(B, dtype=torch.int32, device=dev)
        self.extra["tokens"] = torch.zeros(B, dtype=torch.int64, device=dev)
        self.extra["forwards"] = torch.zeros(B, dtype=torch.int64, device=dev)
        # MASK-row normalisers: written by a forward's proposals, handed on by the bookkeeping,
        # read by the next forward's accept test (two buffers, since accept and proposals run
        # side by side)
        N = self.shape.stride_n
        self.extra["norms_new"] = torch.zeros(B, N, 2, dtype=torch.float32, device=dev)
        self.extra["norms"] = torch.zeros(B, N, 2, dtype=torch.float32, device=dev)
        self.extra["norms_valid"] = False

    def loop_advance(self, stream=None, carry: bool = False):
        """The loop's bookkeeping; with ``carry`` it also hands the proposals' row
        normalisers on to the next forward's accept test."""
        e = self.extra
        self._call(("loop_advance", carry), lambda: _lib.prepare(
            _lib.isd_loop_advance, self.shape, self.accept_len, self.n_out, self.next_proposals, self.n_commit,
            e["mode"], self.proposals, self.positions, e["tokens"], e["forwards"],
            norms_in=e["norms_new"] if carry else None, norms_out=e["norms"] if carry else None))(stream)

    def _side_stream(self):
        """A second stream (default priority) and the two events of a fork and a join."""
        s = self.extra.get("side_stream")
        if s is None:
            dev = self.proposals.device
            s = self.extra["side_stream"] = (torch.cuda.Stream(device=dev), torch.cuda.Event(), torch.cuda.Event())
        return s

    def side_by_side(self) -> bool:
        """Whether the proposals run beside the accept chain on a second stream by default.

        Issued eagerly, the fork and the join cost the queues 5-7 us of idle time per
        forward (measured on MI355X), which only proposals over many logits repay: side by
        side from 16 M MASK-row logits on (c32_ctx4k, 128 rows of 151 936: 6990 against 6665
        forwards/s), one after the other below (b8_ctx2k 17.0 k against 12.2 k, tiny_fp32
        20.8 k against 11.3 k forwards/s)."""
        return self.shape.batch * self.shape.stride_n * self.shape.vocab >= 16 * 2**20

    def _accept_and_propose(self, accept_fn, stream, step: Optional[int], overlap: Optional[bool],
                            device_step: bool = False, row_norms=None):
        """The accept chain on ``stream`` and the proposals on a second stream, joined after
        (``overlap``; None: ``side_by_side()``), or both on ``stream``.

        Both read this forward's logits and neither writes what the other reads
        (their workspace regions are disjoint), so they may run side by side; the
        proposals still start only after everything enqueued before on ``stream``.
        """
        if overlap is None:
            overlap = self.side_by_side()
        if overlap and (stream is None or isinstance(stream, torch.cuda.Stream)):
            main = torch.cuda.current_stream() if stream is None else stream
            side, fork, join = self._side_stream()
            fork.record(main)
            side.wait_event(fork)
            accept_fn(main, step)
            self.propose(side, step=step, device_step=device_step, row_norms=row_norms)
            join.record(side)
            main.wait_event(join)
        else:
            accept_fn(stream, step)
            self.propose(stream, step=step, device_step=device_step, row_norms=row_norms)

    def loop_forward(self, step: int = 0, attention: bool = True, stream=None, overlap: Optional[bool] = None,
                     device_step: bool = False, carry: bool = True):
        """One forward of the decoding loop: attention over ``positions`` cached tokens,
        accept with the commit of the forward's rows, and proposals (side by side with
        ``overlap``, after the accept chain without it; None: ``side_by_side()``), bookkeeping.  Lengths are updated in place, so build the
        step with ``commit_in_place=True``.  With ``device_step`` the Philox
        step of every request is its forward count on the device (``step`` unused), so the
        forward can be recorded once and replayed.  With ``carry`` the proposals also write
        their rows' normalisers, and the next forward's accept test takes its q-row
        normalisers from them instead of a pass over the q rows (the q rows of a verify are
        the MASK rows of the forward before)."""
        e = self.extra
        q_norms = e["norms"] if carry and e.get("norms_valid") else None
        if attention:
            # the forward's rows are committed inside the accept launches, by the loop's mode:
            # a verifying request its accepted prefix, a re-proposing one its row N-1
            self.attention(stream, loop=True)
            accept = lambda s, t: self.accept_commit(s, step=t, device_step=device_step, q_norms=q_norms,
                                                     loop=True)
        else:
            accept = lambda s, t: self.accept(s, step=t, device_step=device_step, q_norms=q_norms)
        self._accept_and_propose(accept, stream, step, overlap, device_step, e["norms_new"] if carry else None)
        self.loop_advance(stream, carry=carry)
        if carry:
            e["norms_valid"] = True

    def capture_loop_forward(self, overlap: Optional[bool] = None):
        """Record one ``loop_forward(device_step=True)`` into a HIP graph and return it.

        Every replay is the next forward: the loop state (proposals, positions, mode,
        forward counts, KV pages and lengths) lives on the device and the Philox step
        comes from the forward counts.  The logits are read from the same buffers on
        every replay, so the caller refreshes them in place between replays.  Recording
        runs nothing; call ``loop_forward(device_step=True, overlap=...)`` eagerly at
        least twice before (the second forward is the first with carried q normalisers),
        so every call is marshalled and the second stream exists."""
        if overlap is None:
            overlap = self.side_by_side()
        if ("accept_commit", True, True, True) not in self.__dict__.get("_calls", {}) or (
                overlap and "side_stream" not in self.extra):
            raise RuntimeError("run loop_forward(device_step=True) eagerly before recording it")
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.loop_forward(overlap=overlap, device_step=True)
        return graph

    def lora_delta(self, stream=None):
        L = self.lora
        _lib.isd_lora_delta(L["X"], L["A_t"], L["B_t"], L["mask_rows"], L["Y"], L["ws"], stream=stream)

    def capture(self):
        """Record one ``run()`` into a HIP graph (``torch.cuda.CUDAGraph``) and return it.

        Every call of the step enqueues kernels only (no allocation, no memset, no
        host synchronisation), and the workspace counters the kernels use are
        rewound by the kernels themselves, so the graph can be replayed any number
        of times; each replay recomputes the step from the buffers' current contents.
        """
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.run()                      # first launches outside the capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.run()
        return graph

    def run(self, stream=None, overlap: Optional[bool] = None):
        """One ISD step: attention -> accept + commit (-> LoRA delta); with MASK logits the
        next proposals run beside the accept chain (``overlap``) or after it (None:
        ``side_by_side()``)."""
        self.attention(stream)
        if self.mask_logits is not None:
            self._accept_and_propose(lambda s, t: self.accept_commit(s, step=t), stream, None, overlap)
        else:
            self.accept_commit(stream)
        if self.lora is not None:
            self.lora_delta(stream)
