"""GPU: a call captured into a HIP graph replays correctly, and plans can be destroyed while a
stream is capturing and after the capture (a plan holds host memory only, so a graph keeps
everything it needs in its kernel arguments).  Each replay is preceded by eager work on the
default stream (C refilled with canaries) and checked bit for bit against the eager result."""
import numpy as np
import pytest
import torch

import precision_moe_nvfp4_amd as gg
from synthetic import make_inputs
from test_gpu_parity import CANARY, check, say

pytestmark = pytest.mark.gpu


def test_graph_replay_after_plan_destroyed():
    say("graph capture / destroy")
    dev = torch.device("cuda", 0)
    inp = make_inputs([200, 72], 640, 1024, seed=90)
    A, B, SFA, SFB = gg.device_operands(inp.A, inp.B, inp.SFA, inp.SFB, dev)
    C = [torch.full((mi, inp.n), CANARY, dtype=torch.int16, device=dev) for mi in inp.m]
    plan = gg.nvfp4_gg_plan(inp.m, inp.n, inp.k)
    other = gg.nvfp4_gg_plan([64], 128, 512)
    gg.nvfp4_gg_run(plan, A, B, SFA, SFB, C)
    torch.cuda.synchronize()
    eager = [c.cpu().numpy().view(np.uint16).copy() for c in C]
    check(inp, eager, "graph: eager", exact=True)

    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    for c in C:
        c.fill_(CANARY)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        gg.nvfp4_gg_run(plan, A, B, SFA, SFB, C, stream=s)
        gg.nvfp4_gg_destroy(other)     # legal while the stream captures: no device work
    gg.nvfp4_gg_destroy(plan)          # the graph does not depend on the plan
    for rep in range(3):
        for c in C:
            c.fill_(CANARY)            # eager work between replays (outside the graph)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        got = [c.cpu().numpy().view(np.uint16) for c in C]
        for a, b in zip(got, eager):
            assert np.array_equal(a, b), f"replay {rep} differs from the eager call"
    say("graph capture / destroy: 3 replays equal to the eager call")
