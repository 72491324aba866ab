"""ctypes binding of libisd.so (argument marshalling only).

Every function here converts torch tensors to device pointers, checks dtype,
device and contiguity, and calls the C entry point of the same name; all
computation runs in the library's HIP kernels.  A non-OK status raises
IsdError.  Importing this module fails loudly if libisd.so is missing: there
is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# ISD_LIBRARY may name another build of the library (the host-sanitizer build the ABI
# tests run against); the default is the in-tree libisd.so.
LIB_PATH = os.environ.get("ISD_LIBRARY") or os.path.join(_PKG, "libisd.so")

ISD_F32, ISD_BF16 = 0, 1
FLAG_CTX_RANGE, FLAG_PAGE_RANGE, FLAG_TOKEN_RANGE, FLAG_COMMIT_RANGE, FLAG_ROW_RANGE = 1, 2, 4, 8, 16
STATUS = {0: "ISD_OK", 1: "ISD_ERR_NULL", 2: "ISD_ERR_SHAPE", 3: "ISD_ERR_DTYPE",
          4: "ISD_ERR_WORKSPACE", 5: "ISD_ERR_UNSUPPORTED", 6: "ISD_ERR_HIP", 7: "ISD_ERR_ALIGNMENT"}

# Every symbol include/isd.h declares.
EXPORTS = ("isd_workspace_bytes", "isd_workspace_init", "isd_read_flags", "isd_attention",
           "isd_accept", "kv_commit", "isd_accept_commit", "isd_accept_commit_noalloc", "isd_propose", "isd_loop_advance", "isd_lora_workspace_bytes",
           "isd_lora_delta", "isd_gated_linear_workspace_bytes", "isd_gated_linear",
           "isd_gated_linear_group_workspace_bytes", "isd_gated_linear_group",
           "isd_status_string", "isd_last_error", "isd_abi_version")
PROPOSE_SAMPLE, PROPOSE_ARGMAX = 0, 1
LOOP_VERIFY, LOOP_REPROPOSE = 0, 1


class IsdError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        self.status = status
        super().__init__(f"{fn} returned {STATUS.get(status, status)}"
                         + (f": {detail}" if detail else ""))


class CShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("batch", "stride_n", "n_q_heads", "n_kv_heads",
                                              "head_dim", "page_size", "max_pages", "num_pages",
                                              "vocab", "max_ctx", "kv_dtype", "logit_dtype")]


@dataclass(frozen=True)
class Shape:
    batch: int
    stride_n: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    max_pages: int
    num_pages: int
    vocab: int
    kv_dtype: int = ISD_BF16
    logit_dtype: int = ISD_BF16
    page_size: int = 16
    max_ctx: int = 0

    @property
    def q_rows(self) -> int:
        return 2 * self.stride_n - 1

    def c(self) -> CShape:
        return CShape(self.batch, self.stride_n, self.n_q_heads, self.n_kv_heads, self.head_dim,
                      self.page_size, self.max_pages, self.num_pages, self.vocab, self.max_ctx,
                      self.kv_dtype, self.logit_dtype)


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m introspective_strided_decoding_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    P, I32, U32, U64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_size_t
    SP = ctypes.POINTER(CShape)
    sig = {
        "isd_workspace_bytes": (SZ, [SP]),
        "isd_workspace_init": (I32, [SP, P, SZ, P]),
        "isd_read_flags": (I32, [P, ctypes.POINTER(U32), P]),
        "isd_attention": (I32, [SP, P, P, P, P, P, P, P, ctypes.c_float, P, P, SZ, P]),
        "isd_accept": (I32, [SP, P, P, P, P, P, U64, U64, U32, P, P, P, P, P, P, P, P, P, SZ, P]),
        "kv_commit": (I32, [SP, P, P, P, P, P, P, P, P, P, SZ, P]),
        "isd_accept_commit": (I32, [SP, P, P, P, P, P, U64, U64, U32, P, P, P, P, P, P, P, P,
                                    P, P, P, P, P, P, P, P, P, SZ, P]),
        "isd_accept_commit_noalloc": (I32, [SP, P, P, P, P, P, U64, U64, U32, P, P, P, P, P, P, P, P,
                                            P, P, P, P, P, P, P, P, P, P]),
        "isd_propose": (I32, [SP, P, P, P, U64, U64, U32, P, I32, P, P, P, SZ, P]),
        "isd_loop_advance": (I32, [SP, P, P, P, P, P, P, P, P, P, P, P, P]),
        "isd_lora_workspace_bytes": (SZ, [I32, I32, I32]),
        "isd_lora_delta": (I32, [I32, I32, I32, I32, P, P, P, P, I32, ctypes.c_float, P, P, SZ, P]),
        "isd_gated_linear_workspace_bytes": (SZ, [I32, I32, I32, I32, I32]),
        "isd_gated_linear": (I32, [I32, I32, I32, I32, P, P, P, P, P, I32, ctypes.c_float, P, P, SZ, P]),
        "isd_gated_linear_group_workspace_bytes": (SZ, [I32, I32, I32, P, I32, I32]),
        "isd_gated_linear_group": (I32, [I32, I32, I32, P, I32, P, P, P, P, P, I32, ctypes.c_float, P, P, SZ, P]),
        "isd_status_string": (ctypes.c_char_p, [I32]),
        "isd_last_error": (ctypes.c_char_p, []),
        "isd_abi_version": (I32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t: torch.Tensor, name: str, dtype=None, numel: Optional[int] = None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def _tdtype(code: int):
    return torch.bfloat16 if code == ISD_BF16 else torch.float32


class _Captured(Exception):
    def __init__(self, name, args):
        super().__init__(name)
        self.name, self.args = name, args


_capturing = False


def _call(name: str, *args) -> None:
    if _capturing:
        raise _Captured(name, args)
    _check(name, getattr(LIB, name)(*args))


# argument index of seed_lo (seed_hi and step follow) in the calls that draw
_DRAW_POS = {"isd_accept": 6, "isd_accept_commit": 6, "isd_accept_commit_noalloc": 6, "isd_propose": 4}
_M64 = 2**64 - 1


class Prepared:
    """A library call checked and marshalled once: launching it again re-reads only
    the stream and, for the calls that draw, the step counter and the seed."""

    __slots__ = ("name", "lib", "fn", "args", "draw")

    def __init__(self, name: str, args):
        self.name, self.lib, self.fn = name, LIB, getattr(LIB, name)
        self.args = list(args)
        self.draw = _DRAW_POS.get(name)

    def __call__(self, stream=None, step: Optional[int] = None, seed=None) -> None:
        a = self.args
        a[-1] = _stream(stream)
        d = self.draw
        if d is not None:
            if seed is not None:
                a[d], a[d + 1] = int(seed[0]) & _M64, int(seed[1]) & _M64
            if step is not None:
                a[d + 2] = int(step) & 0xFFFFFFFF
        status = self.fn(*a)
        if status != 0:
            _check(self.name, status)


def prepare(wrapper, *args, **kw) -> Prepared:
    """Validate and marshal ``wrapper(*args, **kw)`` (one of the call wrappers of this
    module) without launching it; the result launches it."""
    global _capturing
    _capturing = True
    try:
        wrapper(*args, **kw)
    except _Captured as c:
        return Prepared(c.name, c.args)
    finally:
        _capturing = False
    raise RuntimeError(f"{getattr(wrapper, '__name__', wrapper)} is not a library call wrapper")


def _check(fn: str, status: int):
    if status != 0:
        detail = LIB.isd_last_error().decode() if status == 6 else LIB.isd_status_string(status).decode()
        raise IsdError(fn, status, detail)


def isd_workspace_bytes(shape: Shape) -> int:
    n = LIB.isd_workspace_bytes(ctypes.byref(shape.c()))
    if n == 0:
        raise IsdError("isd_workspace_bytes", 2, "shape rejected")
    return int(n)


def new_workspace(shape: Shape, device="cuda", stream=None) -> torch.Tensor:
    """Allocate (torch) and initialise a workspace for ``shape``."""
    ws = torch.empty(isd_workspace_bytes(shape), dtype=torch.uint8, device=device)
    isd_workspace_init(shape, ws, stream)
    return ws


def isd_workspace_init(shape: Shape, workspace: torch.Tensor, stream=None) -> None:
    _call("isd_workspace_init",
        ctypes.byref(shape.c()), _ptr(workspace, "workspace", torch.uint8), workspace.numel(),
        _stream(stream))


def isd_read_flags(workspace: torch.Tensor, stream=None) -> int:
    out = ctypes.c_uint32(0)
    _call("isd_read_flags", _ptr(workspace, "workspace", torch.uint8), ctypes.byref(out), _stream(stream))
    return int(out.value)


def isd_attention(shape: Shape, q, k_new, v_new, k_pages, v_pages, page_table, ctx_lens, out,
                  workspace, scale: float = 0.0, stream=None) -> None:
    B, Q, Hq, Hkv, D = shape.batch, shape.q_rows, shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    dt = _tdtype(shape.kv_dtype)
    pool = shape.num_pages * Hkv * shape.page_size * D
    _call("isd_attention",
        ctypes.byref(shape.c()), _ptr(q, "q", dt, B * Q * Hq * D), _ptr(k_new, "k_new", dt, B * Q * Hkv * D),
        _ptr(v_new, "v_new", dt, B * Q * Hkv * D), _ptr(k_pages, "k_pages", dt, pool),
        _ptr(v_pages, "v_pages", dt, pool),
        _ptr(page_table, "page_table", torch.int32, B * shape.max_pages),
        _ptr(ctx_lens, "ctx_lens", torch.int32, B), float(scale), _ptr(out, "out", dt, B * Q * Hq * D),
        _ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream))


def _norms(t, name, B, N):
    return None if t is None else _ptr(t, name, torch.float32, B * N * 2)


def isd_accept(shape: Shape, p_logits, q_logits, proposals, req_ids, positions, seed, step: int,
               accept_len, out_tokens, n_out, n_commit, logp_sel, logq_sel, workspace,
               stream=None, step_dev=None, q_norms=None) -> None:
    """q_norms: [B][N][2] float32 as isd_propose wrote them for the MASK rows that proposed
    this stride (see include/isd.h), or None."""
    B, N, V = shape.batch, shape.stride_n, shape.vocab
    dt = _tdtype(shape.logit_dtype)
    i32 = torch.int32
    _call("isd_accept",
        ctypes.byref(shape.c()), _ptr(p_logits, "p_logits", dt, B * (N - 1) * V),
        _ptr(q_logits, "q_logits", dt, B * (N - 1) * V), _ptr(proposals, "proposals", i32, B * N),
        _ptr(req_ids, "req_ids", i32, B), _ptr(positions, "positions", i32, B),
        int(seed[0]) & (2**64 - 1), int(seed[1]) & (2**64 - 1), int(step) & 0xFFFFFFFF,
        None if step_dev is None else _ptr(step_dev, "step_dev", torch.int64, B),
        _norms(q_norms, "q_norms", B, N),
        _ptr(accept_len, "accept_len", i32, B), _ptr(out_tokens, "out_tokens", i32, B * N),
        _ptr(n_out, "n_out", i32, B), _ptr(n_commit, "n_commit", i32, B),
        _ptr(logp_sel, "logp_sel", torch.float32, B * (N - 1)),
        _ptr(logq_sel, "logq_sel", torch.float32, B * (N - 1)),
        _ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream))


def kv_commit(shape: Shape, k_new, v_new, k_pages, v_pages, page_table, ctx_lens_in, n_commit,
              ctx_lens_out, workspace, stream=None) -> None:
    B, Q, Hkv, D = shape.batch, shape.q_rows, shape.n_kv_heads, shape.head_dim
    dt = _tdtype(shape.kv_dtype)
    pool = shape.num_pages * Hkv * shape.page_size * D
    _call("kv_commit",
        ctypes.byref(shape.c()), _ptr(k_new, "k_new", dt, B * Q * Hkv * D),
        _ptr(v_new, "v_new", dt, B * Q * Hkv * D), _ptr(k_pages, "k_pages", dt, pool),
        _ptr(v_pages, "v_pages", dt, pool),
        _ptr(page_table, "page_table", torch.int32, B * shape.max_pages),
        _ptr(ctx_lens_in, "ctx_lens_in", torch.int32, B), _ptr(n_commit, "n_commit", torch.int32, B),
        _ptr(ctx_lens_out, "ctx_lens_out", torch.int32, B),
        _ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream))


def isd_accept_commit(shape: Shape, p_logits, q_logits, proposals, req_ids, positions, seed, step: int,
                      accept_len, out_tokens, n_out, n_commit, logp_sel, logq_sel, k_new, v_new, k_pages,
                      v_pages, page_table, ctx_lens_in, ctx_lens_out, workspace, stream=None,
                      step_dev=None, q_norms=None, loop_mode=None) -> None:
    """isd_accept followed by kv_commit of the accepted prefix, in one call (loop_mode: a
    re-proposing request of the decoding loop commits its row N-1 instead)."""
    _call("isd_accept_commit", *_accept_commit_args(
        shape, p_logits, q_logits, proposals, req_ids, positions, seed, step, accept_len, out_tokens, n_out,
        n_commit, logp_sel, logq_sel, k_new, v_new, k_pages, v_pages, page_table, ctx_lens_in, ctx_lens_out,
        step_dev, q_norms, loop_mode),
        _ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream))


def isd_accept_commit_noalloc(shape: Shape, p_logits, q_logits, proposals, req_ids, positions, seed,
                              step: int, accept_len, out_tokens, n_out, n_commit, logp_sel, logq_sel, k_new,
                              v_new, k_pages, v_pages, page_table, ctx_lens_in, ctx_lens_out, flags=None,
                              stream=None, step_dev=None, q_norms=None, loop_mode=None) -> None:
    """isd_accept_commit with the library's own per-device scratch instead of a workspace;
    ``flags``: one uint32 device word the kernels OR their flag bits into (or None)."""
    _call("isd_accept_commit_noalloc", *_accept_commit_args(
        shape, p_logits, q_logits, proposals, req_ids, positions, seed, step, accept_len, out_tokens, n_out,
        n_commit, logp_sel, logq_sel, k_new, v_new, k_pages, v_pages, page_table, ctx_lens_in, ctx_lens_out,
        step_dev, q_norms, loop_mode),
        None if flags is None else _ptr(flags, "flags", torch.int32, 1), _stream(stream))


def _accept_commit_args(shape, p_logits, q_logits, proposals, req_ids, positions, seed, step, accept_len,
                        out_tokens, n_out, n_commit, logp_sel, logq_sel, k_new, v_new, k_pages, v_pages,
                        page_table, ctx_lens_in, ctx_lens_out, step_dev, q_norms, loop_mode):
    """The arguments isd_accept_commit and its no-allocation variant share, marshalled."""
    B, N, V = shape.batch, shape.stride_n, shape.vocab
    Q, Hkv, D = shape.q_rows, shape.n_kv_heads, shape.head_dim
    dt, kt = _tdtype(shape.logit_dtype), _tdtype(shape.kv_dtype)
    pool = shape.num_pages * Hkv * shape.page_size * D
    i32 = torch.int32
    return (
        ctypes.byref(shape.c()), _ptr(p_logits, "p_logits", dt, B * (N - 1) * V),
        _ptr(q_logits, "q_logits", dt, B * (N - 1) * V), _ptr(proposals, "proposals", i32, B * N),
        _ptr(req_ids, "req_ids", i32, B), _ptr(positions, "positions", i32, B),
        int(seed[0]) & (2**64 - 1), int(seed[1]) & (2**64 - 1), int(step) & 0xFFFFFFFF,
        None if step_dev is None else _ptr(step_dev, "step_dev", torch.int64, B),
        _norms(q_norms, "q_norms", B, N),
        _ptr(accept_len, "accept_len", i32, B), _ptr(out_tokens, "out_tokens", i32, B * N),
        _ptr(n_out, "n_out", i32, B), _ptr(n_commit, "n_commit", i32, B),
        _ptr(logp_sel, "logp_sel", torch.float32, B * (N - 1)),
        _ptr(logq_sel, "logq_sel", torch.float32, B * (N - 1)),
        _ptr(k_new, "k_new", kt, B * Q * Hkv * D), _ptr(v_new, "v_new", kt, B * Q * Hkv * D),
        _ptr(k_pages, "k_pages", kt, pool), _ptr(v_pages, "v_pages", kt, pool),
        _ptr(page_table, "page_table", i32, B * shape.max_pages),
        _ptr(ctx_lens_in, "ctx_lens_in", i32, B), _ptr(ctx_lens_out, "ctx_lens_out", i32, B),
        None if loop_mode is None else _ptr(loop_mode, "loop_mode", i32, B))


def isd_propose(shape: Shape, mask_logits, req_ids, positions, seed, step: int, mode: int,
                proposals, workspace, stream=None, step_dev=None, row_norms=None) -> None:
    """row_norms: [B][N][2] float32 written with each MASK row's (max, sum exp(l - max))
    (sampling policy only), or None."""
    B, N, V = shape.batch, shape.stride_n, shape.vocab
    i32 = torch.int32
    sample = mode == PROPOSE_SAMPLE
    _call("isd_propose",
        ctypes.byref(shape.c()), _ptr(mask_logits, "mask_logits", _tdtype(shape.logit_dtype), B * N * V),
        _ptr(req_ids, "req_ids", i32, B) if sample or req_ids is not None else None,
        _ptr(positions, "positions", i32, B) if sample or positions is not None else None,
        int(seed[0]) & (2**64 - 1), int(seed[1]) & (2**64 - 1), int(step) & 0xFFFFFFFF,
        None if step_dev is None else _ptr(step_dev, "step_dev", torch.int64, B), int(mode),
        _ptr(proposals, "proposals", i32, B * N), _norms(row_norms, "row_norms", B, N),
        _ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream))


def isd_loop_advance(shape: Shape, accept_len, n_out, next_proposals, n_commit, mode, proposals,
                     positions, tokens, forwards, stream=None, norms_in=None, norms_out=None) -> None:
    """norms_in -> norms_out ([B][N][2] float32 each, or both None): the proposals' row
    normalisers handed to the next forward's accept test."""
    B, N = shape.batch, shape.stride_n
    i32, i64 = torch.int32, torch.int64
    _call("isd_loop_advance",
        ctypes.byref(shape.c()), _ptr(accept_len, "accept_len", i32, B), _ptr(n_out, "n_out", i32, B),
        _ptr(next_proposals, "next_proposals", i32, B * N), _ptr(n_commit, "n_commit", i32, B),
        _ptr(mode, "mode", i32, B), _ptr(proposals, "proposals", i32, B * N),
        _ptr(positions, "positions", i32, B), _ptr(tokens, "tokens", i64, B),
        _ptr(forwards, "forwards", i64, B), _norms(norms_in, "norms_in", B, N),
        _norms(norms_out, "norms_out", B, N), _stream(stream))


def isd_lora_workspace_bytes(n_mask: int, d_in: int, rank: int) -> int:
    return int(LIB.isd_lora_workspace_bytes(n_mask, d_in, rank))


def isd_lora_delta(X, A_t, B_t, mask_rows, Y, workspace, scale: float = 1.0, stream=None) -> None:
    """Y[m] += scale * (X[m] @ A_t.T) @ B_t.T for the gated rows m (see include/isd.h)."""
    rows, d_in = X.shape
    rank = A_t.shape[0]
    d_out = B_t.shape[0]
    bf = torch.bfloat16
    _call("isd_lora_delta",
        rows, d_in, d_out, rank, _ptr(X, "X", bf), _ptr(A_t, "A_t", bf, rank * d_in),
        _ptr(B_t, "B_t", bf, d_out * rank), _ptr(mask_rows, "mask_rows", torch.int32), mask_rows.numel(),
        float(scale), _ptr(Y, "Y", bf, rows * d_out), _ptr(workspace, "workspace", torch.uint8),
        workspace.numel(), _stream(stream))


def isd_gated_linear_workspace_bytes(rows: int, d_in: int, d_out: int, rank: int, n_mask: int) -> int:
    return int(LIB.isd_gated_linear_workspace_bytes(rows, d_in, d_out, rank, n_mask))


def isd_gated_linear(X, W_t, Y, workspace, A_t=None, B_t=None, mask_rows=None, scale: float = 1.0,
                     stream=None) -> None:
    """Y = X @ W_t.T, plus scale * (X[m] @ A_t.T) @ B_t.T on the gated rows m when an
    adapter is given (see include/isd.h)."""
    rows, d_in = X.shape
    d_out = W_t.shape[0]
    bf = torch.bfloat16
    if A_t is None:
        rank, a, b, m, n_mask = 0, None, None, None, 0
    else:
        rank = A_t.shape[0]
        a = _ptr(A_t, "A_t", bf, rank * d_in)
        b = _ptr(B_t, "B_t", bf, d_out * rank)
        n_mask = mask_rows.numel()
        m = _ptr(mask_rows, "mask_rows", torch.int32)
    _call("isd_gated_linear",
          rows, d_in, d_out, rank, _ptr(X, "X", bf), _ptr(W_t, "W_t", bf, d_out * d_in), a, b, m, n_mask,
          float(scale), _ptr(Y, "Y", bf, rows * d_out), _ptr(workspace, "workspace", torch.uint8),
          workspace.numel(), _stream(stream))


def _host_array(ctype, values):
    """A host array of ctype (the group call's per-projection sizes and pointers)."""
    return (ctype * len(values))(*values)


def isd_gated_linear_group_workspace_bytes(rows: int, d_in: int, d_outs, rank: int, n_mask: int) -> int:
    d = _host_array(ctypes.c_int32, [int(v) for v in d_outs])
    return int(LIB.isd_gated_linear_group_workspace_bytes(len(d_outs), rows, d_in, d, rank, n_mask))


def isd_gated_linear_group(X, W_ts, Ys, workspace, A_ts=None, B_ts=None, mask_rows=None, scale: float = 1.0,
                           stream=None) -> None:
    """Ys[p] = X @ W_ts[p].T, plus scale * (X[m] @ A_ts[p].T) @ B_ts[p].T on the gated rows m
    when adapters are given: up to four projections of one input in one set of launches
    (see include/isd.h)."""
    rows, d_in = X.shape
    n = len(W_ts)
    if len(Ys) != n or (A_ts is not None and (len(A_ts) != n or len(B_ts) != n)):
        raise ValueError("W_ts, Ys, A_ts and B_ts need one entry per projection")
    bf = torch.bfloat16
    d_outs = [int(w.shape[0]) for w in W_ts]
    d = _host_array(ctypes.c_int32, d_outs)
    w = _host_array(ctypes.c_void_p, [_ptr(t, f"W_ts[{i}]", bf, d_outs[i] * d_in) for i, t in enumerate(W_ts)])
    y = _host_array(ctypes.c_void_p, [_ptr(t, f"Ys[{i}]", bf, rows * d_outs[i]) for i, t in enumerate(Ys)])
    if A_ts is None:
        rank, a, b, m, n_mask = 0, None, None, None, 0
    else:
        rank = A_ts[0].shape[0]
        a = _host_array(ctypes.c_void_p, [_ptr(t, f"A_ts[{i}]", bf, rank * d_in) for i, t in enumerate(A_ts)])
        b = _host_array(ctypes.c_void_p, [_ptr(t, f"B_ts[{i}]", bf, d_outs[i] * rank) for i, t in enumerate(B_ts)])
        n_mask = mask_rows.numel()
        m = _ptr(mask_rows, "mask_rows", torch.int32)
    # the host arrays themselves go into the call, so a recorded argument list keeps them alive
    _call("isd_gated_linear_group",
          n, rows, d_in, d, rank, _ptr(X, "X", bf), w, a, b, m, n_mask, float(scale),
          y, _ptr(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream))
