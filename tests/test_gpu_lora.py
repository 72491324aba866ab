"""isd_lora_delta on the GPU vs the float64 oracle (gated rank-128 delta of R-ISD).

Tolerance 2e-2 absolute on bf16 outputs (the class of the attention output);
rows outside the gate must come back bit for bit unchanged.
"""

import numpy as np
import pytest
import torch

from oracle.lora import gated_lora_delta
from parity import needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]


def _bf16(rng, shape, std=1.0):
    return torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32)).to(torch.bfloat16)


def _run(rows, d_in, d_out, mask, scale=1.0, seed=0, std=0.02):
    from introspective_strided_decoding_amd import _lib
    rng = np.random.Generator(np.random.PCG64(seed))
    X, Y = _bf16(rng, (rows, d_in)), _bf16(rng, (rows, d_out))
    A, B = _bf16(rng, (d_in, 128), std), _bf16(rng, (128, d_out), std)
    dev = "cuda"
    Xd, Yd = X.to(dev), Y.to(dev).clone()
    At, Bt = A.t().contiguous().to(dev), B.t().contiguous().to(dev)
    m = torch.tensor(mask, dtype=torch.int32, device=dev)
    ws = torch.zeros(max(256, _lib.isd_lora_workspace_bytes(len(mask), d_in, 128)), dtype=torch.uint8, device=dev)
    _lib.isd_lora_delta(Xd, At, Bt, m, Yd, ws, scale=scale)
    torch.cuda.synchronize()
    ref = gated_lora_delta(X.double().numpy(), A.double().numpy(), B.double().numpy(), Y.double().numpy(),
                           [r for r in mask if 0 <= r < rows], scale)
    got = Yd.float().cpu()
    return got, ref, Y, ws


@pytest.mark.parametrize("rows,d_in,d_out,mask", [
    (20, 256, 128, [1, 3, 4, 17]),
    (70, 512, 384, list(range(0, 70, 2))),            # 35 gated rows: a ragged 32-row block
    (33, 256, 256, list(range(33))),                  # every row gated
])
def test_lora_small(rows, d_in, d_out, mask):
    got, ref, Y0, _ = _run(rows, d_in, d_out, mask)
    err = np.abs(got.double().numpy() - ref).max()
    assert err <= 2e-2, err
    keep = [r for r in range(rows) if r not in set(mask)]
    assert torch.equal(got[keep], Y0[keep].float())


def test_lora_full_size_r_isd():
    """The R-ISD workload: 128 requests x 7 stride rows, the 4 MASK rows of each gated,
    rank 128 on a 4096 -> 4096 projection, adapter entries ~ N(0, 0.02^2)."""
    B, Q, N = 128, 7, 4
    mask = [r * Q + i for r in range(B) for i in range(N - 1, 2 * N - 1)]
    got, ref, Y0, _ = _run(B * Q, 4096, 4096, mask, seed=5)
    err = np.abs(got.double().numpy() - ref).max()
    assert err <= 2e-2, err
    clean = [r * Q + i for r in range(B) for i in range(N - 1)]
    assert torch.equal(got[clean], Y0[clean].float())


def test_lora_scale_and_empty_gate():
    got, ref, Y0, _ = _run(16, 256, 128, [2, 5], scale=0.5)
    assert np.abs(got.double().numpy() - ref).max() <= 2e-2
    got, ref, Y0, _ = _run(16, 256, 128, [])
    assert torch.equal(got, Y0.float())


def test_lora_out_of_range_row_is_flagged_and_skipped():
    from introspective_strided_decoding_amd import isd_read_flags
    got, ref, Y0, ws = _run(16, 256, 128, [2, 99, 5])
    assert isd_read_flags(ws) & 16
    assert np.abs(got.double().numpy() - ref).max() <= 2e-2
