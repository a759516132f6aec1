"""GPU parity at the edges of the LDS operand ring.

A tile of 32, 64 or 96 rows streams K through a ring of 7, 5 or 5 superstep slots (K = 256
each): the first slots are filled up front, and from then on the slot just consumed is
refilled at the start of every superstep, with a constant load wait in the steady state and a
shrinking one in the last supersteps.  These cases put the number of supersteps below, at and
beyond the slot count (several wraps, up to 256 supersteps), with and without a short last
superstep, for each tile height and both scale layouts (whose load counts per superstep
differ), plus a very wide n (many tiles per workgroup), and check every element against the
oracle (same bar and canaries as the per-group tests).  The planner's
chosen tile height is asserted, so that each case runs the ring it is meant to.
"""
import pytest

import precision_moe_nvfp4_amd as gg
from test_gpu_parity import say
from test_gpu_problems import run_problems

pytestmark = pytest.mark.gpu

# (problems, planned chunk height); rows per tile -> 32-row blocks -> ring slots
CASES = [
    # 20-row tiles (one 32-row block, 7 slots): 6, 7, 8 and 15 supersteps; 8 with a short last
    ([(20, 512, 1536, 0), (20, 256, 1792, 0), (20, 256, 2048, 0), (20, 512, 3840, 0), (20, 256, 1856, 0)], 96),
    # 64-row tiles (5 slots): 6 supersteps, the last one short (64 K values)
    ([(288, 4096, 1344, 0)], 64),
    # 90-row tiles (three 32-row blocks, 5 slots): 6 supersteps, the last one short
    ([(90, 4096, 1344, 0)] * 8, 96),
    # 90-row tiles: 4, 5 and 11 supersteps
    ([(90, 4096, 1024, 0)] * 4 + [(90, 4096, 1280, 0)] * 2 + [(90, 4096, 2816, 0)] * 2, 96),
    # long K: 256 supersteps (36 wraps of a 7-slot ring) and the largest load offsets
    ([(3, 130, 65536, 0), (3, 64, 65536 - 192, 0)], 96),
    # wide n: 1024 column tiles over 256 workgroups (4 tiles each), one and 33 rows
    ([(1, 131072, 256, 0)], 96),
    ([(33, 131072, 512, 0)], 96),
]


@pytest.mark.parametrize("layout", [gg.SCALES_ROW_MAJOR, gg.SCALES_BLOCKED])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_ring_edges(case, layout):
    problems, chunk = CASES[case]
    info = gg.nvfp4_gg_plan_info(gg.nvfp4_gg_plan_problems(problems, device=gg.DEVICE_NONE, scale_layout=layout))
    assert info.tile_m == chunk, f"planned chunk height {info.tile_m}, case expects {chunk}"
    say(f"ring case {case}: {problems} layout {layout}")
    run_problems(problems, layout)
