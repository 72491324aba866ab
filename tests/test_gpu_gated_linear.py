"""isd_gated_linear on the GPU vs the float64 oracle (one whole R-ISD projection).

Bar, per element, from the arithmetic the header states (bf16 operands, fp32 sums,
the adapter's rank-128 intermediate rounded once to bf16, one final bf16 rounding):

  |y - y_exact| <= ub |y_exact| + (d_in + r) u (|X||W| + |T||B|)
                   + (ub |T| + d_in u |scale| |X||A|) |B|

with u = 2^-24 (fp32), ub = 2^-8 (bf16) and T = scale X A on the gated rows.  The
relative RMS error must also stay at the level of one bf16 rounding.  Rows outside
the gate must equal the base-only call (rank 0) bit for bit: the property that lets
the CLEAN rows verify with the base model's own numbers.
"""

import numpy as np
import pytest
import torch

from oracle.lora import gated_projection
from parity import needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]

U32, UB = 2.0 ** -24, 2.0 ** -8      # unit roundoff of fp32 (24-bit significand) and bf16 (8-bit)


def _bf16(rng, shape, std=1.0):
    return torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32)).to(torch.bfloat16)


def _inputs(rows, d_in, d_out, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    X = _bf16(rng, (rows, d_in))
    Wt = _bf16(rng, (d_out, d_in), 0.02)
    At = _bf16(rng, (128, d_in), 0.02)
    Bt = _bf16(rng, (d_out, 128), 0.02)
    return X, Wt, At, Bt


def _run(X, Wt, At, Bt, mask, scale=1.0, guard=64):
    """Returns (Y, flags); Y is written into a buffer with a guard tail that must stay untouched."""
    from introspective_strided_decoding_amd import _lib
    rows, d_in = X.shape
    d_out = Wt.shape[0]
    rank = 0 if At is None else 128
    n_mask = 0 if mask is None else len(mask)
    n = _lib.isd_gated_linear_workspace_bytes(rows, d_in, d_out, rank, n_mask)
    assert n > 0
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    buf = torch.full((rows * d_out + guard,), 7.0, dtype=torch.bfloat16, device="cuda")
    Y = buf[:rows * d_out].view(rows, d_out)
    kw = {}
    if rank:
        kw = dict(A_t=At.cuda(), B_t=Bt.cuda(), mask_rows=torch.tensor(mask, dtype=torch.int32, device="cuda"),
                  scale=scale)
    _lib.isd_gated_linear(X.cuda(), Wt.cuda(), Y, ws, **kw)
    torch.cuda.synchronize()
    assert torch.all(buf[rows * d_out:] == 7.0), "write past the output"
    flags = int(ws[:4].view(torch.int32).item())
    return Y.cpu(), flags


def _check(Y, X, Wt, At, Bt, mask, scale, sample=None):
    """Compare rows `sample` (all rows if None) of Y against the oracle, with the bound above."""
    rows = X.shape[0]
    idx = np.arange(rows) if sample is None else np.asarray(sample)
    gate = set(int(m) for m in (mask or []) if 0 <= m < rows)
    sub_mask = [i for i, r in enumerate(idx) if int(r) in gate]
    x = X[idx].double().numpy()
    w = Wt.double().numpy().T
    a = None if At is None else At.double().numpy().T
    b = None if Bt is None else Bt.double().numpy().T
    want = gated_projection(x, w, a, b, sub_mask, scale)
    got = Y[idx].double().numpy()
    d_in = x.shape[1]
    ax, aw = np.abs(x), np.abs(w)
    bound = UB * np.abs(want) + (d_in + 128) * U32 * (ax @ aw)
    if At is not None:
        g = np.zeros((len(idx), 1))
        g[sub_mask] = 1.0
        t = g * scale * (x @ a)
        ab = np.abs(b)
        bound = bound + (d_in + 128) * U32 * (np.abs(t) @ ab) \
            + (UB * np.abs(t) + g * d_in * U32 * abs(scale) * (ax @ np.abs(a))) @ ab
    bound = bound * 1.01
    err = np.abs(got - want)
    assert np.all(err <= bound), (float((err / bound).max()), np.unravel_index(np.argmax(err / bound), err.shape))
    rel_rms = np.sqrt(np.mean((got - want) ** 2) / np.mean(want ** 2))
    assert rel_rms < 4e-3, rel_rms
    return rel_rms


# (rows, d_in, d_out, gated rows), with the tiling the library picks for each: 64 x 64
# tiles, one k range; 64 x 64 tiles again; 64 x 64 tiles with the k range split in 4;
# 128 x 128 tiles with k split in 2 over a ragged last row tile; 128 x 128 tiles of 8 waves,
# ragged; 64 x 64 tiles with every row gated; one row gated; 128 x 128 tiles with a
# two-stage ring (two workgroups per CU); 256 x 256 tiles of 8 waves over a ragged last row
# tile of 8 rows; 256 x 192 tiles of 8 waves over a ragged last row tile of 88 rows; a
# 16640-deep input, whose adapter down-projection leaves 65 chunk partials (summed in two
# batches of 48, the second mostly clamped).
CASES = [
    (20, 256, 128, [1, 3, 4, 17]),
    (70, 512, 384, list(range(0, 70, 2))),
    (40, 2048, 128, list(range(3, 40, 3))),
    (300, 1024, 5376, [r for r in range(300) if r % 7 >= 3]),
    (333, 512, 8192, [r for r in range(333) if r % 5 == 1]),
    (33, 256, 256, list(range(33))),
    (64, 768, 640, [63]),
    (300, 256, 16384, list(range(1, 300, 3))),
    (520, 256, 20480, [r for r in range(520) if r % 7 >= 3]),
    (600, 512, 12288, list(range(2, 600, 4))),
    (48, 16640, 256, [r for r in range(48) if r % 3 != 1]),
]


@pytest.mark.parametrize("rows,d_in,d_out,mask", CASES)
def test_gated_projection_small(rows, d_in, d_out, mask):
    X, Wt, At, Bt = _inputs(rows, d_in, d_out, seed=rows + d_out)
    Y, flags = _run(X, Wt, At, Bt, mask, scale=0.5)
    assert flags == 0
    _check(Y, X, Wt, At, Bt, mask, 0.5)
    base, _ = _run(X, Wt, None, None, None)
    _check(base, X, Wt, None, None, None, 1.0)
    clean = [r for r in range(rows) if r not in set(mask)]
    assert torch.equal(Y[clean].view(torch.int16), base[clean].view(torch.int16))


def test_gated_projection_repeatable_and_duplicate_rows():
    rows, d_in, d_out = 96, 512, 256
    X, Wt, At, Bt = _inputs(rows, d_in, d_out, seed=41)
    mask = [5, 9, 9, 50, 5]
    Y1, _ = _run(X, Wt, At, Bt, mask)
    Y2, _ = _run(X, Wt, At, Bt, mask)
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    Y3, _ = _run(X, Wt, At, Bt, [5, 9, 50])
    assert torch.equal(Y1.view(torch.int16), Y3.view(torch.int16))
    _check(Y1, X, Wt, At, Bt, mask, 1.0)


def test_gated_projection_rows_out_of_range_are_flagged():
    from introspective_strided_decoding_amd import _lib
    rows, d_in, d_out = 50, 256, 128
    X, Wt, At, Bt = _inputs(rows, d_in, d_out, seed=42)
    Y, flags = _run(X, Wt, At, Bt, [2, 50, -1, 7])
    assert flags & _lib.FLAG_ROW_RANGE
    _check(Y, X, Wt, At, Bt, [2, 7], 1.0)


def test_gated_projection_empty_gate_is_base():
    rows, d_in, d_out = 70, 512, 256
    X, Wt, At, Bt = _inputs(rows, d_in, d_out, seed=43)
    Y, _ = _run(X, Wt, At, Bt, [])
    base, _ = _run(X, Wt, None, None, None)
    assert torch.equal(Y.view(torch.int16), base.view(torch.int16))


# The projections of an 8B-class layer (hidden 4096, 32 query and 8 KV heads of 128,
# MLP 12288) at the stride rows of 32 requests (224 rows, 128 gated) and of 128 requests
# (896 rows, 512 gated), N = 4: the MASK rows are 3..6 of every request's 7.
LAYER = {"q": (4096, 4096), "k": (4096, 1024), "gate": (4096, 12288), "down": (12288, 4096)}


@pytest.mark.parametrize("batch", [32, 128])
@pytest.mark.parametrize("proj", list(LAYER))
def test_gated_projection_r_isd_layer_shapes(batch, proj):
    d_in, d_out = LAYER[proj]
    Q, N = 7, 4
    rows = batch * Q
    mask = [r * Q + i for r in range(batch) for i in range(N - 1, Q)]
    X, Wt, At, Bt = _inputs(rows, d_in, d_out, seed=batch + d_in + d_out)
    Y, flags = _run(X, Wt, At, Bt, mask)
    assert flags == 0
    sample = list(range(0, 14)) + list(range(rows - 14, rows)) + list(range(100, rows, 97))
    _check(Y, X, Wt, At, Bt, mask, 1.0, sample=sample)
    base, _ = _run(X, Wt, None, None, None)
    clean = [r * Q + i for r in range(batch) for i in range(N - 1)]
    assert torch.equal(Y[clean].view(torch.int16), base[clean].view(torch.int16))


def test_layer_projections_overlap_group_and_graph_replays():
    """The seven projections of a layer: siblings (q/k/v, gate/up) on two streams give every
    output bit for bit as the one-stream sequence does; the group calls give every output as
    their own eager run does when replayed from a HIP graph (three replays with eager work in
    between), and equal the sequence wherever the two plans sum in the same order (o and down
    are groups of one)."""
    from introspective_strided_decoding_amd.r_isd import RIsdProjections, stride_mask_rows
    batch, n = 32, 4
    proj = RIsdProjections(batch * (2 * n - 1), stride_mask_rows(batch, n), hidden=1024, kv=256, mlp=3072,
                           seed=3, device="cuda")
    names = [nm for nm, _, _ in proj.shapes]

    def outputs():
        return {nm: proj.p[nm]["Y"].clone() for nm in names}

    def clear():
        for nm in names:
            proj.p[nm]["Y"].fill_(0)

    for gated in (True, False):
        proj.run(gated, "sequential")
        torch.cuda.synchronize()
        seq = outputs()
        for mode in ("overlap", "group"):
            clear()
            proj.run(gated, mode)
            torch.cuda.synchronize()
            want = outputs()
            for nm in (names if mode == "overlap" else ["o", "down"]):
                assert torch.equal(want[nm].view(torch.int16), seq[nm].view(torch.int16)), (mode, nm)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                proj.run(gated, mode)
            for rep in range(3):
                clear()
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                for nm in names:
                    assert torch.equal(proj.p[nm]["Y"].view(torch.int16), want[nm].view(torch.int16)), (mode, rep, nm)
            del g


def test_gated_projection_largest_row_count():
    """65536 rows, the most one call takes (64 x 64 tiles, 1024 row tiles), every third gated;
    sampled rows against the oracle, CLEAN rows bit-identical to the base-only call."""
    rows, d_in, d_out = 65536, 256, 128
    X, Wt, At, Bt = _inputs(rows, d_in, d_out, seed=44)
    mask = list(range(0, rows, 3))
    Y, flags = _run(X, Wt, At, Bt, mask)
    assert flags == 0
    sample = list(range(0, 64)) + list(range(rows - 64, rows)) + list(range(1000, rows, 4099))
    _check(Y, X, Wt, At, Bt, mask, 1.0, sample=sample)
    base, _ = _run(X, Wt, None, None, None)
    clean = torch.tensor([r for r in range(rows) if r % 3])
    assert torch.equal(Y[clean].view(torch.int16), base[clean].view(torch.int16))


def _run_group(X, Wts, Ats, Bts, mask, scale=1.0, guard=64):
    """isd_gated_linear_group; returns ([Y_p], flags).  Every output sits in a buffer with a
    guard tail that must stay untouched."""
    from introspective_strided_decoding_amd import _lib
    rows, d_in = X.shape
    d_outs = [w.shape[0] for w in Wts]
    rank = 0 if Ats is None else 128
    n_mask = 0 if mask is None else len(mask)
    n = _lib.isd_gated_linear_group_workspace_bytes(rows, d_in, d_outs, rank, n_mask)
    assert n > 0
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    bufs = [torch.full((rows * d + guard,), 7.0, dtype=torch.bfloat16, device="cuda") for d in d_outs]
    Ys = [b[:rows * d].view(rows, d) for b, d in zip(bufs, d_outs)]
    kw = {}
    if rank:
        kw = dict(A_ts=[a.cuda() for a in Ats], B_ts=[b.cuda() for b in Bts],
                  mask_rows=torch.tensor(mask, dtype=torch.int32, device="cuda"), scale=scale)
    _lib.isd_gated_linear_group(X.cuda(), [w.cuda() for w in Wts], Ys, ws, **kw)
    torch.cuda.synchronize()
    for b, d in zip(bufs, d_outs):
        assert torch.all(b[rows * d:] == 7.0), "write past an output"
    return [y.cpu() for y in Ys], int(ws[:4].view(torch.int32).item())


def _group_inputs(rows, d_in, d_outs, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    X = _bf16(rng, (rows, d_in))
    Wts = [_bf16(rng, (d, d_in), 0.02) for d in d_outs]
    Ats = [_bf16(rng, (128, d_in), 0.02) for _ in d_outs]
    Bts = [_bf16(rng, (d, 128), 0.02) for d in d_outs]
    return X, Wts, Ats, Bts


# (rows, d_in, output widths, gated rows), with the tiling the library picks for the summed
# width: 64 x 64 tiles with k split; four members of 64 x 64 tiles; 128 x 128 tiles with k
# split over a ragged row tile (a q/k/v-like group); 128 x 128 tiles of 8 waves; 128 x 128
# tiles with a two-stage ring (one member's width not a multiple of 256, so no 256 tiles);
# 256 x 256 tiles over a ragged last row tile; 256 x 192 tiles over a ragged last row tile;
# 128 x 192 tiles (one round where 128 x 128 would take two) over a ragged row tile; 128 x
# 256 tiles (the same, with widths that 192 does not divide).
GROUP_CASES = [
    (20, 2048, [128, 256, 128], [1, 3, 4, 17]),
    (64, 768, [128, 256, 384, 128], [63, 0, 31]),
    (300, 1024, [2048, 512, 512], [r for r in range(300) if r % 7 >= 3]),
    (333, 512, [4096, 4096], [r for r in range(333) if r % 5 == 1]),
    (520, 256, [8192, 8064], list(range(1, 520, 3))),
    (520, 256, [8192, 8192], [r for r in range(520) if r % 7 >= 3]),
    (520, 768, [6144, 6144], [r for r in range(520) if r % 3 == 0]),
    (330, 512, [6144, 3072, 3072], [r for r in range(330) if r % 4 == 2]),
    (330, 512, [8192, 2048, 2048], list(range(0, 330, 5))),
]


@pytest.mark.parametrize("rows,d_in,d_outs,mask", GROUP_CASES)
def test_gated_group_small(rows, d_in, d_outs, mask):
    X, Wts, Ats, Bts = _group_inputs(rows, d_in, d_outs, seed=rows + sum(d_outs))
    Ys, flags = _run_group(X, Wts, Ats, Bts, mask, scale=0.5)
    assert flags == 0
    base, _ = _run_group(X, Wts, None, None, None)
    clean = [r for r in range(rows) if r not in set(mask)]
    for p in range(len(d_outs)):
        _check(Ys[p], X, Wts[p], Ats[p], Bts[p], mask, 0.5)
        _check(base[p], X, Wts[p], None, None, None, 1.0)
        assert torch.equal(Ys[p][clean].view(torch.int16), base[p][clean].view(torch.int16)), p


def test_gated_group_of_one_is_the_single_call():
    rows, d_in, d_out = 300, 1024, 5376
    X, Wts, Ats, Bts = _group_inputs(rows, d_in, [d_out], seed=45)
    mask = [r for r in range(rows) if r % 7 >= 3]
    Ys, _ = _run_group(X, Wts, Ats, Bts, mask, scale=0.5)
    Y, _ = _run(X, Wts[0], Ats[0], Bts[0], mask, scale=0.5)
    assert torch.equal(Ys[0].view(torch.int16), Y.view(torch.int16))


def test_gated_group_flags_rows_out_of_range():
    from introspective_strided_decoding_amd import _lib
    rows = 50
    X, Wts, Ats, Bts = _group_inputs(rows, 256, [128, 256], seed=46)
    Ys, flags = _run_group(X, Wts, Ats, Bts, [2, 50, -1, 7])
    assert flags & _lib.FLAG_ROW_RANGE
    for p in range(2):
        _check(Ys[p], X, Wts[p], Ats[p], Bts[p], [2, 7], 1.0)


# The two groups of an 8B-class layer that share an input: q, k, v (hidden 4096 -> 4096,
# 1024, 1024) and gate, up (4096 -> 12288 each), at 224 rows (32 requests x 7, 128 gated)
# and 896 rows (128 x 7, 512 gated); sampled rows against the oracle.
@pytest.mark.parametrize("batch", [32, 128])
@pytest.mark.parametrize("group", [[4096, 1024, 1024], [12288, 12288]])
def test_gated_group_r_isd_layer_shapes(batch, group):
    Q, N = 7, 4
    rows = batch * Q
    mask = [r * Q + i for r in range(batch) for i in range(N - 1, Q)]
    X, Wts, Ats, Bts = _group_inputs(rows, 4096, group, seed=batch + sum(group))
    Ys, flags = _run_group(X, Wts, Ats, Bts, mask)
    assert flags == 0
    base, _ = _run_group(X, Wts, None, None, None)
    sample = list(range(0, 14)) + list(range(rows - 14, rows)) + list(range(100, rows, 97))
    clean = [r * Q + i for r in range(batch) for i in range(N - 1)]
    for p in range(len(group)):
        _check(Ys[p], X, Wts[p], Ats[p], Bts[p], mask, 1.0, sample=sample)
        assert torch.equal(Ys[p][clean].view(torch.int16), base[p][clean].view(torch.int16)), p


def test_gated_group_empty_gate_and_duplicate_rows():
    """An empty gate gives the base-only group call bit for bit; a row listed twice is adapted
    once (same bits as the list without the repeat); results repeat call to call."""
    rows, d_in, d_outs = 96, 512, [256, 128, 384]
    X, Wts, Ats, Bts = _group_inputs(rows, d_in, d_outs, seed=47)
    empty, _ = _run_group(X, Wts, Ats, Bts, [])
    base, _ = _run_group(X, Wts, None, None, None)
    dup, _ = _run_group(X, Wts, Ats, Bts, [5, 9, 9, 50, 5])
    dup2, _ = _run_group(X, Wts, Ats, Bts, [5, 9, 9, 50, 5])
    once, _ = _run_group(X, Wts, Ats, Bts, [5, 9, 50])
    for p in range(len(d_outs)):
        assert torch.equal(empty[p].view(torch.int16), base[p].view(torch.int16)), p
        assert torch.equal(dup[p].view(torch.int16), once[p].view(torch.int16)), p
        assert torch.equal(dup[p].view(torch.int16), dup2[p].view(torch.int16)), p
        _check(dup[p], X, Wts[p], Ats[p], Bts[p], [5, 9, 50], 1.0)
