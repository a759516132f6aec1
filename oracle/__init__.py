"""CPU oracle for the NVFP4 grouped GEMM -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this
package.  The product package (precision_moe_nvfp4_amd) never imports it, and the two
share no code: this side decodes through its own C routines (nvfp4_oracle.c), sums in
fp64 and rounds once to fp16.

What is computed, per group i, row r < m_i, column c < n (see nvfp4_oracle.c for the
citations of the pages):

    C_i[r, c] = RNE_fp16( sum_k e2m1(A_i[r, k]) * e4m3fn(SFA_i[r, k // 16])
                               * e2m1(B_i[c, k]) * e4m3fn(SFB_i[c, k // 16]) )

Every function here is pinned by the CPU tests (tests/test_oracle_*.py) to things other
than itself: the OCP format tables, torch's float8_e4m3fn conversion, numpy's float16
rounding and matmul, closed forms and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB = os.path.join(_HERE, "libnvfp4_oracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the C oracle with gcc (plain C, -O3 without fast-math, OpenMP).  Returns the .so path."""
    cmd = ["gcc", "-O3", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        L.nvfp4_oracle_e2m1.restype = ctypes.c_double
        L.nvfp4_oracle_e2m1.argtypes = [ctypes.c_uint]
        L.nvfp4_oracle_e4m3fn.restype = ctypes.c_double
        L.nvfp4_oracle_e4m3fn.argtypes = [ctypes.c_uint]
        L.nvfp4_oracle_f16_rne.restype = ctypes.c_uint16
        L.nvfp4_oracle_f16_rne.argtypes = [ctypes.c_double]
        L.nvfp4_oracle_max_threads.restype = ctypes.c_int
        L.nvfp4_oracle_grouped.restype = ctypes.c_int
        L.nvfp4_oracle_blocked_offset.restype = ctypes.c_long
        L.nvfp4_oracle_blocked_offset.argtypes = [ctypes.c_long, ctypes.c_long, ctypes.c_int]
        L.nvfp4_oracle_blocked_bytes.restype = ctypes.c_long
        L.nvfp4_oracle_blocked_bytes.argtypes = [ctypes.c_long, ctypes.c_int]
        L.nvfp4_oracle_scales_to_blocked.restype = ctypes.c_int
        L.nvfp4_oracle_scales_to_blocked.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long, ctypes.c_int,
                                                     ctypes.c_int]
        _lib = L
    return _lib


def e2m1(code: int) -> float:
    return lib().nvfp4_oracle_e2m1(code)


def e4m3fn(code: int) -> float:
    return lib().nvfp4_oracle_e4m3fn(code)


def f16_rne(x: float) -> int:
    return int(lib().nvfp4_oracle_f16_rne(float(x)))


def max_threads() -> int:
    return int(lib().nvfp4_oracle_max_threads())


@dataclass
class OracleResult:
    C: List[np.ndarray]                  # uint16 fp16 bits, [m_i, n]
    exact: Optional[List[np.ndarray]]    # float64 sums before rounding
    abssum: Optional[List[np.ndarray]]   # float64 sum_k |a*sa*b*sb|

    def C_f16(self) -> List[np.ndarray]:
        return [c.view(np.float16) for c in self.C]


def _ptrs(arrs, ctype):
    return (ctypes.c_void_p * len(arrs))(*[a.ctypes.data_as(ctypes.c_void_p).value
                                           if a is not None and a.size else None for a in arrs])


def grouped(m, n: int, k: int, A, B, SFA, SFB, want_exact: bool = False,
            want_abs: bool = True, nthreads: int = 0) -> OracleResult:
    """Run the grouped oracle on host uint8 buffers (layouts as in synthetic.GroupedInputs)."""
    g = len(m)
    m = [int(x) for x in m]
    for i in range(g):
        for arr, rows, cols in ((A[i], m[i], k // 2), (B[i], n, k // 2),
                                (SFA[i], m[i], k // 16), (SFB[i], n, k // 16)):
            if arr.dtype != np.uint8 or arr.shape != (rows, cols) or not arr.flags.c_contiguous:
                raise ValueError("oracle input has the wrong dtype, shape or layout")
    C = [np.zeros((mi, n), dtype=np.uint16) for mi in m]
    ex = [np.zeros((mi, n), dtype=np.float64) for mi in m] if want_exact else None
    ab = [np.zeros((mi, n), dtype=np.float64) for mi in m] if want_abs else None
    marr = (ctypes.c_int * max(g, 1))(*m)
    rc = lib().nvfp4_oracle_grouped(
        ctypes.c_int(g), marr, ctypes.c_int(n), ctypes.c_int(k),
        _ptrs(A, None), _ptrs(B, None), _ptrs(SFA, None), _ptrs(SFB, None),
        _ptrs(C, None), _ptrs(ex, None) if ex else None, _ptrs(ab, None) if ab else None,
        ctypes.c_int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle failed")
    return OracleResult(C, ex, ab)


def grouped_inputs(inp, **kw) -> OracleResult:
    """grouped() on a synthetic.GroupedInputs."""
    return grouped(inp.m, inp.n, inp.k, inp.A, inp.B, inp.SFA, inp.SFB, **kw)


def blocked_offset(r: int, c: int, k: int) -> int:
    """Byte offset of scale (row r, K block c) in the 128x4 blocked scale layout."""
    return int(lib().nvfp4_oracle_blocked_offset(int(r), int(c), int(k)))


def blocked_bytes(rows: int, k: int) -> int:
    return int(lib().nvfp4_oracle_blocked_bytes(int(rows), int(k)))


def scales_to_blocked(src: np.ndarray, k: int, pad: int = 0) -> np.ndarray:
    """Row-major scales uint8 [rows, k/16] -> the blocked layout (1-D uint8); bytes of the
    padding rows are set to `pad`."""
    src = np.ascontiguousarray(src, dtype=np.uint8)
    rows = src.shape[0]
    if src.shape != (rows, k // 16):
        raise ValueError("scale matrix must be [rows, k/16]")
    dst = np.empty(blocked_bytes(rows, k), dtype=np.uint8)
    rc = lib().nvfp4_oracle_scales_to_blocked(dst.ctypes.data if dst.size else None,
                                              src.ctypes.data if src.size else None, rows, k, pad)
    if rc != 0:
        raise RuntimeError("oracle blocked conversion failed")
    return dst


def ulp16(ref_bits: np.ndarray) -> np.ndarray:
    """Spacing of fp16 at the oracle's fp16 value: 2^(max(floor(log2|x|), -14) - 10);
    the spacing at 0 and in the subnormal range is 2^-24."""
    x = np.abs(ref_bits.view(np.float16).astype(np.float64))
    x = np.where(np.isfinite(x), x, 65504.0)   # Inf/NaN: spacing of the top binade
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(x > 0, x, 1.0)))
    e = np.where(x > 0, np.maximum(e, -14.0), -14.0)
    return np.ldexp(1.0, (e - 10).astype(np.int64))


def tolerance(ref_bits: np.ndarray, abssum: np.ndarray) -> np.ndarray:
    """Per-element bound |gpu - ref| <= 2 ulp16(ref) + 1e-5 * sum_k |a*b| (dequantised)."""
    return 2.0 * ulp16(ref_bits) + 1e-5 * abssum
