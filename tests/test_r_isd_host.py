"""Host logic of the R-ISD layer projections, without a GPU: which rows are gated, the
layer's projection shapes, and the workspace the library asks for."""

import pytest

lib_mod = pytest.importorskip("introspective_strided_decoding_amd._lib", reason="libisd.so not built")


def test_stride_mask_rows_are_the_mask_positions():
    from introspective_strided_decoding_amd.r_isd import stride_mask_rows
    # N = 4: Q = 7 rows per request, rows 3..6 are MASK rows
    assert stride_mask_rows(2, 4) == [3, 4, 5, 6, 10, 11, 12, 13]
    # N = 2: Q = 3, row 1 and 2 of every request
    assert stride_mask_rows(3, 2) == [1, 2, 4, 5, 7, 8]
    rows = stride_mask_rows(128, 4)
    assert len(rows) == 512 and len(set(rows)) == 512 and max(rows) == 128 * 7 - 1


def test_layer_shapes_and_groups():
    from introspective_strided_decoding_amd.r_isd import GROUPS, layer_shapes
    shapes = layer_shapes(4096, 1024, 12288)
    assert [s[0] for s in shapes] == ["q", "k", "v", "o", "gate", "up", "down"]
    dims = {n: (i, o) for n, i, o in shapes}
    assert dims["down"] == (12288, 4096) and dims["k"] == (4096, 1024)
    # projections grouped together read the same input width
    for g in GROUPS:
        assert len({dims[n][0] for n in g}) == 1
    assert sorted(n for g in GROUPS for n in g) == sorted(dims)


def test_gated_linear_workspace_sizes():
    ws = lib_mod.LIB.isd_gated_linear_workspace_bytes
    for rows in (1, 7, 224, 896, 65536):
        base = ws(rows, 4096, 4096, 0, 0)
        gated = ws(rows, 4096, 4096, 128, rows)
        assert base > 0 and gated > base
        # the adapter's intermediate alone: rows x 128 bf16, plus the down-projection partials
        assert gated - base >= rows * 128 * 2
    # more gated rows never need less
    assert ws(896, 4096, 4096, 128, 512) <= ws(896, 4096, 4096, 128, 896)
