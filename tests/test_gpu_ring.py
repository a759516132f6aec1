"""GPU parity at the edges of the LDS operand ring, for every compiled unit shape.

A unit of NA x NB blocks streams K through a ring of S superstep slots in LDS (K = 256 each;
S = 3 for units of 3 or more blocks, 4 for 1x1 units): the first S supersteps are issued up
front, and from then on the slot read during the previous superstep is refilled at every
barrier, with a constant load wait in the steady state and shrinking ones in the last
supersteps.  For every shape the kernel is compiled for (the planner's choice is overridden
with NVFP4_GG_FORCE_SHAPE), these cases put the number of supersteps below, at and beyond S
(several ring wraps), with and without a short last superstep, with ragged rows and columns,
and check every element against the oracle (same bar and canaries as the per-group tests).
Units of more than 16 blocks keep their extra accumulators in ordinary VGPRs (a separate code
path): every such shape runs here too.
"""
import os
import re

import pytest

import precision_moe_nvfp4_amd as gg
from conftest import ROOT
from test_gpu_parity import say
from test_gpu_problems import run_problems

pytestmark = pytest.mark.gpu


def compiled_shapes():
    text = open(os.path.join(ROOT, "precision_moe_nvfp4_amd", "csrc", "nvfp4_gg_internal.h")).read()
    body = text[text.index("#define NVFP4GG_UNIT_SHAPES(X)"):].split("\n\n", 1)[0]
    return [(int(a), int(b)) for a, b in re.findall(r"X\((\d+), (\d+)\)", body)]


def ring_slots(na, nb):
    """Slots of the ring for a unit shape (the kernel's geometry: 4 KiB of codes per block and
    superstep, four scale regions of 128 B per even-rounded block plus 4 B, 160 KiB of LDS; at
    most 3 slots for units of 3 or more blocks, else at most 4)."""
    nbp, nap = (nb + 1) & ~1, (na + 1) & ~1
    slot = ((na + nb) * 4096 + 4 * (128 * (nbp + nap) + 4) + 15) & ~15
    return min(3 if na + nb >= 3 else 4, (160 * 1024) // slot)


SHAPES = compiled_shapes()


@pytest.mark.parametrize("na,nb", SHAPES)
def test_ring_edges_every_shape(na, nb, monkeypatch):
    S = ring_slots(na, nb)
    monkeypatch.setenv("NVFP4_GG_FORCE_SHAPE", f"{na},{nb}")
    # ragged rows (two row chunks, the second short) and columns (last tile short)
    m1, m2 = 32 * na, max(1, 32 * na - 7)
    n = 32 * nb + 40
    cases = [
        [(m1, n, 256 * (S - 1), 0)],                                   # fewer supersteps than slots
        [(m2, n, 256 * S + 64, 0)],                                    # S + 1, the last one short
        [(m1 + m2, n, 256 * (2 * S + 1), 0), (m2, n, 256 * S - 192, 0)],  # wraps; a 64-K tail
    ]
    for probs in cases:
        plan = gg.nvfp4_gg_plan_problems(probs, device=gg.DEVICE_NONE)
        info = gg.nvfp4_gg_plan_info(plan)
        assert (info.unit_rows[0], info.unit_cols[0]) == (32 * na, 32 * nb)
        say(f"ring shape {na}x{nb} (S={S}): {probs}")
        run_problems(probs, gg.SCALES_ROW_MAJOR)


@pytest.mark.parametrize("na,nb", [(4, 4), (4, 5), (2, 9), (2, 4), (2, 3), (1, 2), (1, 1)])
def test_ring_edges_blocked_scales(na, nb, monkeypatch):
    S = ring_slots(na, nb)
    monkeypatch.setenv("NVFP4_GG_FORCE_SHAPE", f"{na},{nb}")
    probs = [(32 * na + 33, 32 * nb + 40, 256 * (S + 1) + 128, 0), (5, 64, 256 * (S - 1), 0)]
    say(f"ring shape {na}x{nb} blocked scales: {probs}")
    run_problems(probs, gg.SCALES_BLOCKED)


def test_long_k_and_wide_n():
    # long K: 256 supersteps (many ring wraps) and the largest load offsets; wide n: many
    # column tiles per workgroup range
    for probs in ([(3, 130, 65536, 0), (3, 64, 65536 - 192, 0)], [(1, 131072, 256, 0)], [(33, 131072, 512, 0)]):
        say(f"ring long/wide: {probs}")
        run_problems(probs, gg.SCALES_ROW_MAJOR)
