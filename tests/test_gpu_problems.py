"""GPU parity of plans with per-group sizes (nvfp4_gg_plan_problems): each group has its own
m, n, k and C row stride ldc.  Every group is checked against the oracle (run per group) with
the same per-element bar as the shared-size path; the columns n .. ldc-1 of each C row and the
halves around each C_i are canaries that must stay untouched.  Both scale layouts.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_moe_nvfp4_amd as gg
from synthetic import make_inputs
from test_gpu_parity import CANARY, PAD, check, say

pytestmark = pytest.mark.gpu

CASES = [
    [(100, 256, 512, 0), (0, 1000, 256, 0), (300, 130, 1024, 136), (7, 64, 256, 64)],
    [(129, 4096, 256, 4100), (33, 200, 768, 201), (64, 128, 1536, 0)],
    [(1, 16, 256, 17), (96, 520, 2048, 0), (255, 300, 256, 303), (40, 7168, 512, 0)],
]


def run_problems(problems, layout, repeats=1, expect=None):
    """Plan once, run `repeats` times (C canary-filled before each run) and check every run
    against the oracle; `expect(info)` may assert properties of the plan first."""
    dev = torch.device("cuda", 0)
    inps = [make_inputs([m], n, k, seed=1000 + 7 * i + m) for i, (m, n, k, _) in enumerate(problems)]
    conv = (lambda s, k: oracle.scales_to_blocked(s, k, pad=0x7F)) if layout == gg.SCALES_BLOCKED else \
        (lambda s, k: s)
    A = [torch.from_numpy(x.A[0]).to(dev) for x in inps]
    B = [torch.from_numpy(x.B[0]).to(dev) for x in inps]
    SFA = [torch.from_numpy(np.ascontiguousarray(conv(x.SFA[0], x.k))).to(dev) for x in inps]
    SFB = [torch.from_numpy(np.ascontiguousarray(conv(x.SFB[0], x.k))).to(dev) for x in inps]
    bufs, views = [], []
    for m, n, k, ldc in problems:
        ld = ldc or n
        buf = torch.full((PAD + m * ld + PAD,), CANARY, dtype=torch.int16, device=dev)
        bufs.append(buf)
        views.append(buf[PAD:PAD + m * ld])
    plan = gg.nvfp4_gg_plan_problems(problems, scale_layout=layout)
    if expect is not None:
        expect(gg.nvfp4_gg_plan_info(plan))
    first = None
    for rep in range(repeats):
        for buf in bufs:
            buf.fill_(CANARY)
        gg.nvfp4_gg_run(plan, A, B, SFA, SFB, views)
        torch.cuda.synchronize()
        if first is None:
            check_outputs(problems, bufs, inps, f"run {rep}")
            first = [buf.cpu().numpy().copy() for buf in bufs]
        else:
            # later runs of the same plan: bit-identical to the first (a fixed summation order)
            for i, buf in enumerate(bufs):
                assert np.array_equal(buf.cpu().numpy(), first[i]), f"run {rep}: group {i} differs from run 0"


def check_outputs(problems, bufs, inps, what):
    for i, ((m, n, k, ldc), buf, inp) in enumerate(zip(problems, bufs, inps)):
        ld = ldc or n
        h = buf.cpu().numpy().view(np.uint16)
        assert np.all(h[:PAD] == CANARY) and np.all(h[PAD + m * ld:] == CANARY), f"group {i}: write outside C_i"
        c = h[PAD:PAD + m * ld].reshape(m, ld)
        assert np.all(c[:, n:] == CANARY), f"group {i}: write beyond column n"
        if m:
            check(inp, [np.ascontiguousarray(c[:, :n])], f"{what}: group {i} (m={m} n={n} k={k} ldc={ldc})", exact=True)


@pytest.mark.parametrize("layout", [gg.SCALES_ROW_MAJOR, gg.SCALES_BLOCKED])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_per_group_sizes_and_strides(case, layout):
    say(f"problems {CASES[case]} layout {layout}")
    run_problems(CASES[case], layout)


# K not a multiple of 256: the last K step is short (64, 128 or 192 K values)
KTAIL_CASES = [
    [(17, 200, 64, 0)],
    [(100, 130, 192, 0), (64, 130, 320, 136)],
    [(300, 256, 1088, 0), (5, 256, 448, 0), (96, 256, 512, 0)],
    [(129, 1000, 704, 1001), (0, 64, 128, 0), (64, 128, 2112, 0)],
]


@pytest.mark.parametrize("layout", [gg.SCALES_ROW_MAJOR, gg.SCALES_BLOCKED])
@pytest.mark.parametrize("case", range(len(KTAIL_CASES)))
def test_k_tails(case, layout):
    say(f"k tails {KTAIL_CASES[case]} layout {layout}")
    run_problems(KTAIL_CASES[case], layout)
