"""The C ABI without a GPU: libisd.so loads, exports every symbol include/isd.h
declares, and host-side validation returns the documented status codes before
any launch (all calls below fail validation, so nothing reaches the device)."""

import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "isd.h")

lib_mod = pytest.importorskip("introspective_strided_decoding_amd._lib",
                              reason="libisd.so not built")
LIB = lib_mod.LIB
Shape = lib_mod.Shape


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(isd_\w+|kv_commit)\s*\(", text))


def test_header_and_library_agree():
    names = _declared()
    assert names == set(lib_mod.EXPORTS)
    for n in names:
        assert hasattr(LIB, n)


def test_abi_version_and_status_strings():
    assert LIB.isd_abi_version() == 10
    for code in range(8):
        assert LIB.isd_status_string(code)
    assert LIB.isd_status_string(99) == b"unknown status"


def _shape(**kw):
    base = dict(batch=32, stride_n=4, n_q_heads=32, n_kv_heads=8, head_dim=128, max_pages=257,
                num_pages=8224, vocab=151936)
    base.update(kw)
    return Shape(**base)


def _ws(shape):
    return LIB.isd_workspace_bytes(ctypes.byref(shape.c()))


def test_workspace_bytes_rejects_bad_shapes():
    assert _ws(_shape()) > 0
    for bad in (dict(n_q_heads=30), dict(head_dim=96), dict(stride_n=1), dict(batch=0),
                dict(page_size=8), dict(stride_n=33, n_q_heads=8, n_kv_heads=8), dict(stride_n=9),
                dict(stride_n=17, n_q_heads=8, n_kv_heads=8),
                dict(kv_dtype=7), dict(vocab=0), dict(max_ctx=-1)):
        assert _ws(_shape(**bad)) == 0, bad
    assert _ws(_shape(stride_n=16, n_q_heads=8, n_kv_heads=8)) > 0     # Q = 31: one stride tile


def test_workspace_grows_with_splits():
    assert _ws(_shape(max_ctx=8192)) >= _ws(_shape(max_ctx=512))


FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10008)


def _attention(shape, q=FAKE, ws=FAKE, ws_bytes=None, scale=0.0):
    if ws_bytes is None:
        ws_bytes = _ws(shape) if _ws(shape) else 1 << 30
    return LIB.isd_attention(ctypes.byref(shape.c()), q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             scale, FAKE, ws, ws_bytes, None)


def test_attention_validation():
    s = _shape()
    assert _attention(s, q=None) == 1
    assert _attention(s, q=MISALIGNED) == 7
    assert _attention(s, ws_bytes=16) == 4
    assert _attention(s, ws=None) == 1
    assert _attention(s, scale=-1.0) == 2
    assert _attention(_shape(head_dim=80)) == 5
    assert _attention(_shape(n_q_heads=33)) == 2
    assert _attention(_shape(kv_dtype=3)) == 3
    assert LIB.isd_attention(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.0, FAKE, FAKE, 1, None) == 1


def test_accept_and_commit_validation():
    s = _shape()
    n = _ws(s)
    # the accept arguments: 5 tensors, seed_lo, seed_hi, step, step_per_request and q_norms
    # (both may be NULL), 6 outputs, workspace, its size, stream
    args = [FAKE] * 5 + [1, 2, 3, None, None] + [FAKE] * 6 + [FAKE, n, None]
    bad = list(args)
    bad[2] = None
    assert LIB.isd_accept(ctypes.byref(s.c()), *bad) == 1
    bad = list(args)
    bad[0] = MISALIGNED
    assert LIB.isd_accept(ctypes.byref(s.c()), *bad) == 7
    bad = list(args)
    bad[-2] = 8
    assert LIB.isd_accept(ctypes.byref(s.c()), *bad) == 4
    bad = list(args)
    bad[9] = ctypes.c_void_p(0x10004)      # q_norms: pairs of floats, 8-byte aligned
    assert LIB.isd_accept(ctypes.byref(s.c()), *bad) == 7
    bad[9] = MISALIGNED
    bad[-2] = 8
    assert LIB.isd_accept(ctypes.byref(s.c()), *bad) == 4
    cargs = [FAKE] * 8 + [FAKE, n, None]
    bad = list(cargs)
    bad[6] = None
    assert LIB.kv_commit(ctypes.byref(s.c()), *bad) == 1
    bad = list(cargs)
    bad[-2] = 0
    assert LIB.kv_commit(ctypes.byref(s.c()), *bad) == 4
    # isd_accept_commit: the accept arguments, then k_new .. ctx_lens_out, workspace, stream
    # (then loop_mode, which may be NULL)
    fargs = [FAKE] * 5 + [1, 2, 3, None, None] + [FAKE] * 6 + [FAKE] * 7 + [None] + [FAKE, n, None]
    assert len(fargs) == 27
    for i in (2, 16, 20, 22):       # proposals, k_new, page_table, ctx_lens_out
        bad = list(fargs)
        bad[i] = None
        assert LIB.isd_accept_commit(ctypes.byref(s.c()), *bad) == 1, i
    for i in (0, 16, 17, 18, 9):    # p_logits, k_new, v_new, k_pages, q_norms
        bad = list(fargs)
        bad[i] = ctypes.c_void_p(0x10004)
        assert LIB.isd_accept_commit(ctypes.byref(s.c()), *bad) == 7, i
    bad = list(fargs)
    bad[-2] = 8
    assert LIB.isd_accept_commit(ctypes.byref(s.c()), *bad) == 4
    assert LIB.isd_accept_commit(None, *fargs) == 1
    # vocabularies past 1024 residual shards of 2048 entries are refused; the limit itself is not
    for v, want in ((2048 * 1024 + 1, 5), (2048 * 1024, 4)):
        big = _shape(vocab=v)
        bad = list(args)
        bad[-2] = 8
        assert LIB.isd_accept(ctypes.byref(big.c()), *bad) == want, v
        bad = list(fargs)
        bad[-2] = 8
        assert LIB.isd_accept_commit(ctypes.byref(big.c()), *bad) == want, v


def test_accept_commit_noalloc_validation():
    """The no-allocation variant takes isd_accept_commit's arguments without the workspace,
    plus a flag word (NULL allowed), and refuses before any launch what does not fit the
    library's 16 MiB scratch."""
    s = _shape()
    # the accept arguments, then k_new .. ctx_lens_out, loop_mode, flags, stream
    gargs = [FAKE] * 5 + [1, 2, 3, None, None] + [FAKE] * 6 + [FAKE] * 7 + [None, None, None]
    assert len(gargs) == 26
    for i in (2, 16, 20, 22):       # proposals, k_new, page_table, ctx_lens_out
        bad = list(gargs)
        bad[i] = None
        assert LIB.isd_accept_commit_noalloc(ctypes.byref(s.c()), *bad) == 1, i
    for i in (0, 16, 17, 18, 9):    # p_logits, k_new, v_new, k_pages, q_norms
        bad = list(gargs)
        bad[i] = ctypes.c_void_p(0x10004)
        assert LIB.isd_accept_commit_noalloc(ctypes.byref(s.c()), *bad) == 7, i
    assert LIB.isd_accept_commit_noalloc(None, *gargs) == 1
    assert LIB.isd_accept_commit_noalloc(ctypes.byref(_shape(stride_n=1).c()), *gargs) == 2
    # residual partials: batch * ceil(V / 2048) * 176 bytes must fit beside the counters
    too_big = _shape(batch=2048, vocab=151936, max_pages=16, num_pages=32768)     # 27 MB of partials
    assert LIB.isd_accept_commit_noalloc(ctypes.byref(too_big.c()), *gargs) == 4
    assert b"scratch" in LIB.isd_last_error()
    assert LIB.isd_accept_commit_noalloc(ctypes.byref(_shape(vocab=2048 * 1024 + 1).c()), *gargs) == 5


def test_propose_validation():
    s = _shape()
    n = _ws(s)

    def call(logits=FAKE, req=FAKE, pos=FAKE, mode=0, out=FAKE, ws=FAKE, ws_bytes=n, shape=s, norms=None):
        return LIB.isd_propose(ctypes.byref(shape.c()), logits, req, pos, 1, 2, 3, None, mode, out, norms, ws,
                               ws_bytes, None)

    assert call(ws_bytes=8) == 4                      # every check passes up to the workspace size
    assert call(mode=2) == 5
    assert call(mode=-1) == 5
    assert call(logits=None) == 1
    assert call(out=None) == 1
    assert call(req=None) == 1                        # the sampling policy needs the Philox counter
    assert call(req=None, pos=None, mode=1, ws_bytes=8) == 4   # argmax does not
    assert call(logits=MISALIGNED) == 7
    assert call(ws=None) == 1
    assert call(shape=_shape(batch=20000, stride_n=4), ws_bytes=8) == 5   # B * N rows > 65535
    assert call(shape=_shape(logit_dtype=5)) == 3
    assert call(norms=FAKE, ws_bytes=8) == 4               # sampling may write the row normalisers
    assert call(norms=FAKE, mode=1) == 5                   # argmax sums nothing
    assert call(norms=ctypes.c_void_p(0x10004)) == 7


def test_loop_advance_validation():
    s = _shape()
    args = [FAKE] * 9 + [None, None]        # the two normaliser buffers may both be NULL
    assert LIB.isd_loop_advance(None, *args, None) == 1
    for i in range(9):
        bad = list(args)
        bad[i] = None
        assert LIB.isd_loop_advance(ctypes.byref(s.c()), *bad, None) == 1, i
    assert LIB.isd_loop_advance(ctypes.byref(s.c()), *([FAKE] * 9 + [FAKE, None]), None) == 1   # one of two
    assert LIB.isd_loop_advance(ctypes.byref(s.c()), *([FAKE] * 9 + [None, FAKE]), None) == 1
    assert LIB.isd_loop_advance(ctypes.byref(s.c()), *([FAKE] * 9 + [FAKE, ctypes.c_void_p(0x10004)]),
                                None) == 7
    assert LIB.isd_loop_advance(ctypes.byref(_shape(stride_n=1).c()), *args, None) == 2


def test_workspace_init_and_flags_validation():
    s = _shape()
    n = _ws(s)
    assert LIB.isd_workspace_init(ctypes.byref(s.c()), None, n, None) == 1
    assert LIB.isd_workspace_init(ctypes.byref(s.c()), MISALIGNED, n, None) == 7
    assert LIB.isd_workspace_init(ctypes.byref(s.c()), FAKE, 16, None) == 4
    assert LIB.isd_workspace_init(None, FAKE, n, None) == 1
    assert LIB.isd_read_flags(None, None, None) == 1


def test_layout_round_trip_cpu():
    from introspective_strided_decoding_amd.layout import (SIGMA, pack_k_pages, pack_v_pages,
                                                           unpack_k_pages, unpack_v_pages)
    assert sorted(SIGMA) == list(range(16)) and all(SIGMA[SIGMA[s]] == s for s in range(16))
    k = torch.randn(5, 16, 3, 64)
    v = torch.randn(5, 16, 3, 64)
    kp, vp = pack_k_pages(k), pack_v_pages(v)
    assert kp.shape == (5, 3, 8, 16, 8) and vp.shape == (5, 3, 64, 16)
    assert torch.equal(unpack_k_pages(kp), k) and torch.equal(unpack_v_pages(vp), v)
    # element addresses as the header states them
    page, h, slot, d = 3, 2, 11, 45
    assert kp[page, h, d // 8, slot, d % 8] == k[page, slot, h, d]
    sig = (slot & 3) | ((slot & 4) << 1) | ((slot & 8) >> 1)
    assert vp[page, h, d, sig] == v[page, slot, h, d]


def test_lora_validation():
    assert LIB.isd_lora_workspace_bytes(512, 4096, 128) > 0
    assert LIB.isd_lora_workspace_bytes(512, 4000, 128) == 0
    assert LIB.isd_lora_workspace_bytes(512, 4096, 64) == 0
    n = LIB.isd_lora_workspace_bytes(512, 4096, 128)
    ok = dict(rows=896, d_in=4096, d_out=4096, rank=128, X=FAKE, A=FAKE, B=FAKE, m=FAKE, n_mask=512,
              scale=1.0, Y=FAKE, ws=FAKE, wsb=n)

    def call(**kw):
        a = {**ok, **kw}
        return LIB.isd_lora_delta(a["rows"], a["d_in"], a["d_out"], a["rank"], a["X"], a["A"], a["B"], a["m"],
                                  a["n_mask"], a["scale"], a["Y"], a["ws"], a["wsb"], None)
    assert call(rank=64) == 5
    assert call(d_in=4000) == 5
    assert call(d_out=4000) == 5
    assert call(n_mask=900) == 2
    assert call(X=None) == 1
    assert call(Y=MISALIGNED) == 7
    assert call(wsb=100) == 4
    assert call(scale=float("nan")) == 2


def test_gated_linear_validation():
    ws = LIB.isd_gated_linear_workspace_bytes
    assert ws(896, 4096, 4096, 128, 512) > ws(896, 4096, 4096, 0, 0) > 0
    for bad in ((0, 4096, 4096, 0, 0), (70000, 4096, 4096, 0, 0), (8, 4000, 4096, 0, 0), (8, 4096, 4000, 0, 0),
                (8, 4096, 4096, 64, 4), (8, 4096, 4096, 128, 9), (8, 4096, 4096, 128, -1)):
        assert ws(*bad) == 0, bad
    n = ws(224, 4096, 1024, 128, 128)
    ok = dict(rows=224, d_in=4096, d_out=1024, rank=128, X=FAKE, W=FAKE, A=FAKE, B=FAKE, m=FAKE, n_mask=128,
              scale=1.0, Y=FAKE, ws=FAKE, wsb=n)

    def call(**kw):
        a = {**ok, **kw}
        return LIB.isd_gated_linear(a["rows"], a["d_in"], a["d_out"], a["rank"], a["X"], a["W"], a["A"], a["B"],
                                    a["m"], a["n_mask"], a["scale"], a["Y"], a["ws"], a["wsb"], None)
    assert call(wsb=n - 1) == 4                      # everything else valid
    assert call(rows=0) == 2
    assert call(n_mask=225) == 2
    assert call(scale=float("nan")) == 2
    assert call(scale=float("inf")) == 2
    assert call(rank=64) == 5
    assert call(d_in=4000) == 5
    assert call(d_out=1000) == 5
    assert call(rows=70000, n_mask=0) == 5
    for k in ("X", "W", "Y", "ws", "A", "B", "m"):
        assert call(**{k: None}) == 1, k
    assert call(rank=0, A=None, B=None, m=None, n_mask=0, wsb=8) == 4   # base only: no adapter pointers needed
    assert call(m=None, n_mask=0, wsb=8) == 4                          # an empty gate needs no row list
    for k in ("X", "W", "A", "B", "Y", "ws"):
        assert call(**{k: MISALIGNED}) == 7, k
    assert call(d_in=1 << 17) == 5                                     # past the largest input width
    assert call(rows=65536, d_out=1 << 15, n_mask=0) == 5              # rows x width past 2^30


def _i32s(*v):
    return (ctypes.c_int32 * len(v))(*v)


def _ptrs(*v):
    return (ctypes.c_void_p * len(v))(*v)


def test_gated_linear_group_validation():
    gws = LIB.isd_gated_linear_group_workspace_bytes
    ws = LIB.isd_gated_linear_workspace_bytes
    # a group of one is the single-projection call
    for shape in ((224, 4096, 1024, 128, 128), (896, 4096, 12288, 128, 512), (40, 2048, 128, 0, 0)):
        rows, d_in, d_out, rank, n_mask = shape
        assert gws(1, rows, d_in, _i32s(d_out), rank, n_mask) == ws(*shape) > 0
    qkv = _i32s(4096, 1024, 1024)
    assert gws(3, 224, 4096, qkv, 128, 128) > gws(3, 224, 4096, qkv, 0, 0) > 0
    for bad in ((0, 224, 4096, qkv, 0, 0), (5, 224, 4096, _i32s(128, 128, 128, 128, 128), 0, 0),
                (3, 224, 4096, _i32s(4096, 1000, 1024), 0, 0), (2, 224, 4096, _i32s(4096, 0), 0, 0),
                (3, 224, 4096, None, 0, 0), (2, 65536, 4096, _i32s(1 << 14, 1 << 14), 0, 0),
                (3, 224, 4000, qkv, 0, 0), (3, 224, 4096, qkv, 64, 4)):
        assert gws(*bad) == 0, bad
    n = gws(3, 224, 4096, qkv, 128, 128)
    three = _ptrs(FAKE.value, FAKE.value, FAKE.value)
    ok = dict(n=3, rows=224, d_in=4096, d_out=qkv, rank=128, X=FAKE, W=three, A=three, B=three, m=FAKE,
              n_mask=128, scale=1.0, Y=three, ws=FAKE, wsb=n)

    def call(**kw):
        a = {**ok, **kw}
        return LIB.isd_gated_linear_group(a["n"], a["rows"], a["d_in"], a["d_out"], a["rank"], a["X"], a["W"],
                                          a["A"], a["B"], a["m"], a["n_mask"], a["scale"], a["Y"], a["ws"], a["wsb"],
                                          None)
    assert call(wsb=n - 1) == 4                      # everything else valid
    assert call(n=0) == 2
    assert call(n=5) == 5
    assert call(d_out=_i32s(4096, 1000, 1024)) == 5
    assert call(d_out=None) == 1
    assert call(scale=float("nan")) == 2
    for k in ("X", "W", "Y", "ws", "A", "B", "m"):
        assert call(**{k: None}) == 1, k
    for k in ("W", "A", "B", "Y"):
        assert call(**{k: _ptrs(FAKE.value, None, FAKE.value)}) == 1, k        # one member missing
        assert call(**{k: _ptrs(FAKE.value, FAKE.value, MISALIGNED.value)}) == 7, k
    assert call(rank=0, A=None, B=None, m=None, n_mask=0, wsb=8) == 4
