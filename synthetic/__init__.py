"""Seeded synthetic inputs for the NVFP4 grouped GEMM (shared by tests, bench and smoke).

This module only draws random bytes and integers; it holds none of the method's
arithmetic (no decoding, no products, no rounding), so both the CPU oracle and the
HIP path can consume the very same bytes.

Workload shapes.  The four timed shapes are the ones the leaderboard page
"kernelindex submission 498317" prints in its timing docstring (g, k, m, n, seed 1111);
the tiny shape is a parity-only case.  Distribution (a reading, since the leaderboard's
own generator is not on the pages):
  * FP4 E2M1 codes i.i.d. uniform over all 16 codes.  Two codes are packed per byte
    along K with the low nibble holding the even K index, so a uniform random byte is
    exactly two independent uniform codes.
  * FP8 E4M3FN scale codes i.i.d. uniform over 0x08..0x20, i.e. the finite positive
    values in [2^-6, 2^-3].
Per group, in group order, the draws are: A bytes, B bytes, SFA codes, SFB codes,
from numpy's PCG64 seeded with the config seed.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np

SCALE_CODE_LO = 0x08  # E4M3FN code of 2^-6
SCALE_CODE_HI = 0x20  # E4M3FN code of 2^-3


@dataclass(frozen=True)
class GroupedShape:
    name: str
    m: tuple
    n: int
    k: int
    seed: int = 1111
    note: str = ""

    @property
    def g(self) -> int:
        return len(self.m)


# Shapes: "tiny" is the parity-only case; c1..c4 are the page's four timed workloads.
CONFIGS = {
    "c0": GroupedShape("c0", (64, 128), 256, 512, note="tiny parity case"),
    "c1": GroupedShape("c1", (128, 384), 4096, 1536),
    "c2": GroupedShape("c2", (192, 320), 3072, 4096),
    "c3": GroupedShape("c3", (40, 76, 168, 72, 164, 148, 196, 160), 7168, 2048,
                       note="MoE down-projection-like"),
    "c4": GroupedShape("c4", (80, 176, 128, 72, 64, 248, 96, 160), 4096, 7168,
                       note="MoE up-projection-like, ~117 MB of FP4 weights"),
}


@dataclass
class GroupedInputs:
    """Host buffers for one grouped call.  All arrays are C-contiguous uint8.

    A[i]:   [m_i, k/2]   packed E2M1 codes (low nibble = even k)
    B[i]:   [n,   k/2]   packed E2M1 codes
    SFA[i]: [m_i, k/16]  E4M3FN codes, one per 16 consecutive K of a row
    SFB[i]: [n,   k/16]  E4M3FN codes
    """
    m: List[int]
    n: int
    k: int
    A: List[np.ndarray] = field(default_factory=list)
    B: List[np.ndarray] = field(default_factory=list)
    SFA: List[np.ndarray] = field(default_factory=list)
    SFB: List[np.ndarray] = field(default_factory=list)

    @property
    def g(self) -> int:
        return len(self.m)


def make_inputs(m, n: int, k: int, seed: int = 1111,
                scale_lo: int = SCALE_CODE_LO, scale_hi: int = SCALE_CODE_HI) -> GroupedInputs:
    """Draw one grouped call's inputs (see module docstring for the recipe)."""
    if k % 32:
        raise ValueError("k must be a multiple of 32 to pack codes and scales")
    rng = np.random.Generator(np.random.PCG64(seed))
    out = GroupedInputs(m=[int(x) for x in m], n=int(n), k=int(k))
    for mi in out.m:
        out.A.append(rng.integers(0, 256, size=(mi, k // 2), dtype=np.uint8))
        out.B.append(rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8))
        out.SFA.append(rng.integers(scale_lo, scale_hi + 1, size=(mi, k // 16), dtype=np.uint8))
        out.SFB.append(rng.integers(scale_lo, scale_hi + 1, size=(n, k // 16), dtype=np.uint8))
    return out


def make_config(name: str, seed: int | None = None) -> GroupedInputs:
    cfg = CONFIGS[name]
    return make_inputs(cfg.m, cfg.n, cfg.k, cfg.seed if seed is None else seed)
