"""GPU parity of the 128x4 blocked scale layout, through the C ABI.

* nvfp4_gg_scales_to_blocked (device converter) against the oracle's permutation, byte for
  byte, including the zeroed padding rows, with a canary tail that must stay untouched.
* nvfp4_gg_run on a plan for blocked scales: the scales are rearranged by the oracle, with
  every padding byte set to an E4M3FN NaN code (0x7F) so that a read of padding would show
  up as NaN in the output; the result must pass the same per-element bar as the row-major
  path against the oracle (which reads the row-major scales) and equal the row-major
  run's output bit for bit (same kernel arithmetic on the same scale values).
"""
import numpy as np
import pytest
import torch

import oracle
import precision_moe_nvfp4_amd as gg
from synthetic import CONFIGS, make_inputs
from test_gpu_parity import CANARY, PAD, check, run_gpu, say

pytestmark = pytest.mark.gpu

NAN_E4M3 = 0x7F


def run_gpu_blocked(inp):
    dev = torch.device("cuda", 0)
    A = [torch.from_numpy(a).to(dev) for a in inp.A]
    B = [torch.from_numpy(b).to(dev) for b in inp.B]
    SFA = [torch.from_numpy(oracle.scales_to_blocked(s, inp.k, pad=NAN_E4M3)).to(dev) for s in inp.SFA]
    SFB = [torch.from_numpy(oracle.scales_to_blocked(s, inp.k, pad=NAN_E4M3)).to(dev) for s in inp.SFB]
    for t, rows in zip(SFA, inp.m):
        assert t.numel() == gg.nvfp4_gg_blocked_scale_bytes(rows, inp.k)
    bufs, views = [], []
    for mi in inp.m:
        buf = torch.full((PAD + mi * inp.n + PAD,), CANARY, dtype=torch.int16, device=dev)
        bufs.append(buf)
        views.append(buf[PAD:PAD + mi * inp.n])
    plan = gg.nvfp4_gg_plan(inp.m, inp.n, inp.k, scale_layout=gg.SCALES_BLOCKED)
    assert gg.nvfp4_gg_plan_info(plan).scale_layout == gg.SCALES_BLOCKED
    gg.nvfp4_gg_run(plan, A, B, SFA, SFB, views)
    torch.cuda.synchronize()
    out = []
    for mi, buf in zip(inp.m, bufs):
        h = buf.cpu().numpy().view(np.uint16)
        assert np.all(h[:PAD] == CANARY) and np.all(h[PAD + mi * inp.n:] == CANARY), "write outside C_i"
        out.append(h[PAD:PAD + mi * inp.n].reshape(mi, inp.n))
    return out


@pytest.mark.parametrize("rows,k", [(1, 256), (100, 512), (128, 256), (257, 1536), (1000, 2048), (4096, 7168)])
def test_converter_matches_the_oracle(rows, k):
    say(f"scales_to_blocked rows={rows} k={k}")
    rng = np.random.default_rng(rows + 31 * k)
    src = rng.integers(0, 256, size=(rows, k // 16), dtype=np.uint8)
    nbytes = gg.nvfp4_gg_blocked_scale_bytes(rows, k)
    dev = torch.device("cuda", 0)
    d_src = torch.from_numpy(src).to(dev)
    d_dst = torch.full((nbytes + 256,), 0xEE, dtype=torch.uint8, device=dev)
    gg.nvfp4_gg_scales_to_blocked(d_dst[:nbytes], d_src, rows, k)
    torch.cuda.synchronize()
    got = d_dst.cpu().numpy()
    assert np.all(got[nbytes:] == 0xEE), "write beyond the blocked tensor"
    assert np.array_equal(got[:nbytes], oracle.scales_to_blocked(src, k, pad=0))


@pytest.mark.parametrize("m,n,k", [
    ([1], 16, 256), ([17, 1, 129], 200, 256), ([255, 0, 3], 130, 512), ([300], 1, 768),
    ([33, 65, 97, 129, 161], 384, 1024), ([384, 500], 136, 256), ([96, 200], 1000, 1536),
])
def test_blocked_gemm_matches_oracle_and_row_major(m, n, k):
    say(f"blocked gemm m={m} n={n} k={k}")
    inp = make_inputs(m, n, k, seed=sum(m) + n + k)
    got = run_gpu_blocked(inp)
    check(inp, got, f"blocked {m} {n} {k}", exact=True)
    ref = run_gpu(inp)
    for i in range(inp.g):
        assert np.array_equal(got[i], ref[i]), f"group {i}: blocked and row-major runs differ"


@pytest.mark.parametrize("name", ["c1", "c3"])
def test_blocked_gemm_full_size(name):
    cfg = CONFIGS[name]
    say(f"blocked gemm {name}: {cfg}")
    inp = make_inputs(cfg.m, cfg.n, cfg.k, cfg.seed)
    check(inp, run_gpu_blocked(inp), f"blocked {name}", exact=True)
