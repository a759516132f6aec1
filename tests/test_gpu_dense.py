"""Dense single-group workload (g = 1, large m): the whole GEMM runs on the GPU at full size in
the launch configuration the bench times.  For 3000 x 1000 x 2048 the oracle recomputes every
element; for 8192 x 4096 x 4096 (about 137 G multiply-adds, too slow for the CPU oracle here) it
recomputes a sample of rows: one full 128-row unit and its neighbours, the last rows and random
rows.  Compared element by element with the usual bar, and with no fp16 bit mismatch: with the
workload recipe's inputs the fp32 sums round to the same fp16 as the exact ones.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_moe_nvfp4_amd as gg
from synthetic import make_inputs
from test_gpu_parity import CANARY, PAD, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m,n,k", [(8192, 4096, 4096), (3000, 1000, 2048)])
def test_dense_single_group_sampled_rows(m, n, k):
    say(f"dense m={m} n={n} k={k}")
    inp = make_inputs([m], n, k, seed=4242)
    dev = torch.device("cuda", 0)
    A, B, SFA, SFB = gg.device_operands(inp.A, inp.B, inp.SFA, inp.SFB, dev)
    buf = torch.full((PAD + m * n + PAD,), CANARY, dtype=torch.int16, device=dev)
    plan = gg.nvfp4_gg_plan([m], n, k)
    gg.nvfp4_gg_run(plan, A, B, SFA, SFB, [buf[PAD:PAD + m * n]])
    torch.cuda.synchronize()
    h = buf.cpu().numpy().view(np.uint16)
    assert np.all(h[:PAD] == CANARY) and np.all(h[PAD + m * n:] == CANARY)
    C = h[PAD:PAD + m * n].reshape(m, n)
    assert not np.any(C == CANARY), "unwritten elements"
    rng = np.random.default_rng(m + n + k)
    if m * n * k <= 8_000_000_000:
        rows = np.arange(m)
    else:
        rows = sorted(set(range(128, 256)) | {0, 1, 127, 256, m - 2, m - 1} |
                      set(int(x) for x in rng.integers(0, m, 40)))
        rows = np.array([r for r in rows if r < m])
    ref = oracle.grouped([len(rows)], n, k, [np.ascontiguousarray(inp.A[0][rows])], [inp.B[0]],
                         [np.ascontiguousarray(inp.SFA[0][rows])], [inp.SFB[0]], want_abs=True)
    got = C[rows]
    r16 = ref.C[0]
    gv = got.view(np.float16).astype(np.float64)
    rv = r16.view(np.float16).astype(np.float64)
    tol = oracle.tolerance(r16, ref.abssum[0])
    bad = np.abs(gv - rv) > tol
    mism = int(np.sum((got != r16) & ((got | r16) & 0x7FFF != 0)))
    say(f"dense: {got.size} checked elements ({len(rows)} of {m} rows), {int(bad.sum())} beyond tolerance, {mism} fp16 bit mismatches")
    assert not bad.any()
    assert mism == 0
