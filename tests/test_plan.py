"""What xattn_decode enqueues, from the host-only plan query (no GPU needed).

The plan is what the dispatch follows (api.hip builds its launches from
it), so these checks cover the launch geometry itself: every workgroup's
LDS fits the 160 KiB of a gfx950 compute unit, the beams a workgroup's
query rows belong to are bounded as the kernel's ancestor-slot buffer
assumes (checked against brute-force enumeration of the row blocks), and
the kernel sequence per call matches the ancestor-walk and split rules.
"""
import ctypes
import itertools

import pytest

from generative_recommendation_beam_xattn_amd import binding as B

LDS_LIMIT = 160 * 1024


def shape(**kw):
    base = dict(num_requests=2, beam_width=4, num_q_heads=8, num_kv_heads=2, head_dim=128,
                max_prompt_len=2048, max_steps=16, dtype=B.XATTN_BF16, scale=0.0)
    base.update(kw)
    return B.Shape(**base)


def brute_beams_per_block(BW, G, rows):
    """Most distinct beams the rows of one row block belong to (rows are
    ordered (beam, head in group); block i holds rows [i * rows, (i+1) * rows))."""
    M = BW * G
    return max(len({row // G for row in range(lo, min(lo + rows, M))})
               for lo in range(0, M, rows))


GROUPS = (1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 24, 33, 64)
WIDTHS = (1, 2, 3, 5, 9, 16, 31, 32, 33, 63, 64, 65, 127, 128, 129, 133, 136, 137, 255, 256,
          300, 512, 777)


@pytest.mark.parametrize("D", [64, 128])
def test_lds_fits_and_beam_bound_holds_over_the_shape_space(D):
    checked = 0
    for G, BW, step in itertools.product(GROUPS, WIDTHS, range(16)):
        s = shape(beam_width=BW, num_q_heads=G, num_kv_heads=1, head_dim=D)
        pl = B.plan(s, step)
        if BW * G <= 8:
            assert pl.kernel == B.KERNEL_PER_BEAM_BF16
            continue
        rows = pl.rows_per_block
        assert rows == (32 if BW * G <= 32 else 64 if BW * G <= 64 else 128)
        assert pl.kernels == 1 and pl.ancestor_walk == 0 and pl.workspace_bytes == 0
        exact = brute_beams_per_block(BW, G, rows)
        assert exact <= pl.beams_per_block <= BW
        if rows % G == 0:
            assert pl.beams_per_block == min(rows // G, BW) == exact
        # parent rows are staged whenever they hold at most 2048 ints and fit
        want = 0 < step and step * BW <= 2048
        dyn = pl.beams_per_block * (step + 1) * 4
        par = -(-step * BW // 64) * 64 * 4
        grid = 2 * -(-BW * G // rows)                       # 2 requests x 1 KV head
        assert pl.grid == grid
        # >= 512 workgroups of 128 rows take the paired variant, whose LDS
        # fits twice per CU; otherwise one workgroup per CU
        pstatic = 2 * 4 * 32 * 2 * D
        paired = rows == 128 and grid >= 512 and pstatic + dyn <= LDS_LIMIT // 2
        if paired:
            assert pl.kernel == B.KERNEL_STAGED_BF16_PAIRED, (G, BW, step, D)
            assert pl.threads_per_block == 256
            staged = want and pstatic + dyn + par <= LDS_LIMIT // 2
            assert pl.parents_in_lds == int(staged)
            assert pl.lds_bytes == pstatic + dyn + (par if staged else 0) <= LDS_LIMIT // 2
        else:
            assert pl.kernel == B.KERNEL_STAGED_BF16, (G, BW, step, D)
            assert pl.threads_per_block == rows // 32 * 2 * 64
            static = 2 * 4 * 64 * 2 * D + 2 * 32 * 2 * D
            staged = want and static + dyn + par <= LDS_LIMIT
            assert pl.parents_in_lds == int(staged)
            assert pl.lds_bytes == static + dyn + (par if staged else 0) <= LDS_LIMIT
        checked += 1
    assert checked > 3000


def test_widest_single_head_groups_fill_lds_exactly():
    # 128 one-head beams per workgroup, 16 levels of slots and 15 parent
    # rows of 136 slots: 147456 + 8192 + 8192 bytes, the whole 160 KiB
    pl = B.plan(shape(beam_width=136, num_q_heads=2, num_kv_heads=2), 15)
    assert pl.rows_per_block == 128 and pl.beams_per_block == 128
    assert pl.parents_in_lds == 1
    assert pl.lds_bytes == LDS_LIMIT
    # the paired variant: 65536 + 8192 + 8192 bytes, exactly half
    pl = B.plan(shape(num_requests=32, beam_width=136, num_q_heads=8, num_kv_heads=8), 15)
    assert pl.kernel == B.KERNEL_STAGED_BF16_PAIRED and pl.grid == 512
    assert pl.parents_in_lds == 1
    assert pl.lds_bytes == LDS_LIMIT // 2


def test_workload_plans():
    # the serving, large-batch and wide-beam shapes: one staged kernel
    for (R, BW, Hq, Hkv, L, S), steps in [((16, 128, 16, 4, 1024, 3), range(3)),
                                         ((64, 256, 32, 8, 2048, 3), range(3)),
                                         ((8, 512, 32, 8, 4096, 4), range(4))]:
        for step in steps:
            pl = B.plan(shape(num_requests=R, beam_width=BW, num_q_heads=Hq, num_kv_heads=Hkv,
                              max_prompt_len=L, max_steps=S), step)
            # serving: 256 workgroups, one per CU with two waves per row group;
            # large batch and wide beam: 4096 and 1024, two per CU (paired)
            paired = R * Hkv * BW * (Hq // Hkv) // 128 >= 512
            assert pl.kernel == (B.KERNEL_STAGED_BF16_PAIRED if paired else B.KERNEL_STAGED_BF16)
            assert (pl.kernels, pl.key_splits, pl.rows_per_block) == (1, 1, 128)
            assert pl.grid == R * Hkv * BW * (Hq // Hkv) // 128
            assert pl.threads_per_block == (256 if paired else 512)
            assert pl.lds_bytes <= (LDS_LIMIT // 2 if paired else LDS_LIMIT)
    # the prefix sweep: 512 levels (segmented walk), the Unshared stage first,
    # key splits where the grid is small; one sequence per group runs per beam
    for G, kernels, splits in [(1, 3, 1), (8, 4, 1), (32, 5, 4), (256, 5, 4)]:
        s = shape(num_requests=256 // G, beam_width=G, num_q_heads=32, num_kv_heads=8,
                  max_prompt_len=3584, max_steps=512)
        pl = B.plan(s, 511)
        assert pl.ancestor_walk == 2
        assert pl.kernels == kernels and pl.key_splits == splits, (G, pl.as_dict())
        assert pl.workspace_bytes == B.workspace_size(s, 511)
        assert pl.kernel == (B.KERNEL_PER_BEAM_BF16 if G == 1 else B.KERNEL_STAGED_BF16)


def test_deep_chain_walks():
    # more than 16 levels: one chunked walk kernel while a segment covers the chain
    pl = B.plan(shape(beam_width=40, max_steps=40, max_prompt_len=64), 39)
    assert (pl.ancestor_walk, pl.unshared_kernel, pl.key_splits, pl.kernels) == (1, 1, 1, 3)
    # 8 workgroups over a 32-tile prompt: split over 4, merged by a last kernel
    pl = B.plan(shape(beam_width=40, max_steps=40), 39)
    assert (pl.ancestor_walk, pl.key_splits, pl.kernels, pl.grid) == (1, 4, 4, 32)
    pl = B.plan(shape(beam_width=40, max_steps=40, dtype=B.XATTN_F32), 39)
    assert (pl.kernel, pl.ancestor_walk, pl.unshared_kernel, pl.kernels) == (1, 1, 0, 2)
    # three segments of 64 levels: two walk kernels
    pl = B.plan(shape(beam_width=40, max_steps=151, max_prompt_len=64), 150)
    assert (pl.ancestor_walk, pl.kernels) == (2, 4)


def test_plan_rejects_what_decode_rejects():
    lib = B.load()
    pl = B.Plan()
    assert lib.xattn_plan_decode(ctypes.byref(shape()), 16, ctypes.byref(pl)) == 1
    assert lib.xattn_plan_decode(ctypes.byref(shape(head_dim=96)), 0, ctypes.byref(pl)) == 2
    assert lib.xattn_plan_decode(ctypes.byref(shape()), 0, None) == 1
    assert lib.xattn_plan_decode(None, 0, ctypes.byref(pl)) == 1
