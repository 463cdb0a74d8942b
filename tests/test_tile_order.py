"""The workgroup -> output-tile order of every launch (XCD renumbering plus grouped
rows), checked on the CPU through the same function the kernels run: for every grid
up to 64 x 64 tiles and every group size the launches use, each workgroup gets a
distinct tile inside the grid, so every output tile is computed exactly once."""
import numpy as np
import pytest

import linear_algebra_sgemm_amd as lib

# group sizes the launches pass (4 and 8), the forced values of the swizzle hook's
# sweeps (1, 2, 16) and the dispatcher's own order (remap off)
GROUPS = (1, 2, 4, 8, 16)


@pytest.mark.parametrize("group_m", GROUPS)
@pytest.mark.parametrize("xcd_remap", [True, False])
def test_every_workgroup_gets_a_distinct_tile(group_m, xcd_remap):
    for tm_count in range(1, 65):
        for tn_count in range(1, 65):
            tm, tn = lib.gemm_debug_tile_map(tm_count, tn_count, group_m, xcd_remap)
            assert tm.min() >= 0 and tm.max() < tm_count, (tm_count, tn_count)
            assert tn.min() >= 0 and tn.max() < tn_count, (tm_count, tn_count)
            flat = tm.astype(np.int64) * tn_count + tn
            assert np.unique(flat).size == tm_count * tn_count, (tm_count, tn_count, group_m)


def test_xcd_runs_are_contiguous_in_the_grouped_order():
    """With the renumbering, the workgroups one XCD receives (ids congruent mod 8)
    walk one contiguous run of the grouped order: at 16 x 16 tiles and group 4 the
    32 tiles of XCD 0 are the first two groups' first half (rows 0-3, columns 0-7)."""
    tm, tn = lib.gemm_debug_tile_map(16, 16, 4, True)
    x0 = set(zip(tm[0::8].tolist(), tn[0::8].tolist()))
    assert x0 == {(r, c) for r in range(4) for c in range(8)}
    tm, tn = lib.gemm_debug_tile_map(16, 16, 4, False)
    # without it, workgroup ids walk the grouped order directly: id 0..3 = rows 0-3 of column 0
    assert list(zip(tm[:4].tolist(), tn[:4].tolist())) == [(0, 0), (1, 0), (2, 0), (3, 0)]


def test_swizzle_hook_validates():
    assert lib.gemm_debug_force_swizzle(0, True) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_force_swizzle(-1, True) == lib.STATUS_INVALID_VALUE
    assert lib.gemm_debug_force_swizzle(65, True) == lib.STATUS_INVALID_VALUE
    assert lib.gemm_debug_force_swizzle(8, False) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_force_swizzle(0, True) == lib.STATUS_SUCCESS
    with pytest.raises(lib.GemmError):
        lib.gemm_debug_tile_map(0, 4, 4)
