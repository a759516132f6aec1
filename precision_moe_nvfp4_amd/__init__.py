"""Python binding of the MI355X NVFP4 grouped GEMM C ABI (include/nvfp4_gg.h).

Argument marshalling only: every step of the computation runs in the gfx950 kernels of
libnvfp4gg.so.  There is no fallback: if the library is missing, importing the binding
raises.  PyTorch is used for device memory and streams only.

Names mirror the C ABI:
    plan = nvfp4_gg_plan(m, n, k, device=-1, scale_layout=SCALES_ROW_MAJOR)
    plan = nvfp4_gg_plan_problems([(m_i, n_i, k_i, ldc_i), ...], device=-1, scale_layout=...)
    nvfp4_gg_blocked_scale_bytes(rows, k)
    nvfp4_gg_scales_to_blocked(dst, src, rows, k, stream=None)
    nvfp4_gg_run(plan, A, B, SFA, SFB, C, stream=None)
    info = nvfp4_gg_plan_info(plan)
    nvfp4_gg_destroy(plan)
    nvfp4_gg_status_string(status)
A, B, SFA, SFB and C are sequences (caller group order) of device tensors or raw device
addresses: A_i uint8 [m_i, k/2], B_i uint8 [n, k/2], SFA_i uint8 [m_i, k/16],
SFB_i uint8 [n, k/16], C_i float16 [m_i, n], all contiguous.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4gg.so")

MAX_GROUPS = 64
DEVICE_NONE = -2

OK, EINVAL, EALIGN, ENOMEM, EHIP, EUNSUPPORTED = range(6)
SCALES_ROW_MAJOR, SCALES_BLOCKED = 0, 1


class Nvfp4GGError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {nvfp4_gg_status_string(status)} (status {status})")


class Problem(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int), ("n", ctypes.c_int), ("k", ctypes.c_int), ("ldc", ctypes.c_int)]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("g", ctypes.c_int), ("n", ctypes.c_int), ("k", ctypes.c_int),
        ("device", ctypes.c_int), ("num_cus", ctypes.c_int),
        ("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int),
        ("total_tiles", ctypes.c_int), ("grid", ctypes.c_int), ("block", ctypes.c_int),
        ("lds_bytes", ctypes.c_int), ("variant", ctypes.c_int),
        ("order", ctypes.c_int * MAX_GROUPS),
        ("tile_begin", ctypes.c_int * (MAX_GROUPS + 1)),
        ("scale_layout", ctypes.c_int),
        ("unit_rows", ctypes.c_int * MAX_GROUPS),
        ("unit_cols", ctypes.c_int * MAX_GROUPS),
        ("est_us", ctypes.c_double),
    ]


def _hip_runtimes_mapped():
    """Distinct libamdhip64 files mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({os.path.realpath(ln.split()[-1]) for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


def _load():
    # PyTorch ships its own HIP runtime (soname libamdhip64.so.7).  Importing torch first
    # makes the dynamic loader bind this library's libamdhip64.so.7 dependency to that same
    # copy, so tensors, streams and our kernels share one HIP runtime in the process.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python precision_moe_nvfp4_amd/build.py` "
            "(there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError(f"two HIP runtimes are mapped into this process: {runtimes}")
    vp = ctypes.c_void_p
    L.nvfp4_gg_plan.restype = ctypes.c_int
    L.nvfp4_gg_plan.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.nvfp4_gg_plan_layout.restype = ctypes.c_int
    L.nvfp4_gg_plan_layout.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.nvfp4_gg_plan_problems.restype = ctypes.c_int
    L.nvfp4_gg_plan_problems.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.POINTER(Problem), ctypes.c_int,
                                         ctypes.c_int]
    L.nvfp4_gg_blocked_scale_bytes.restype = ctypes.c_size_t
    L.nvfp4_gg_blocked_scale_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
    L.nvfp4_gg_scales_to_blocked.restype = ctypes.c_int
    L.nvfp4_gg_scales_to_blocked.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, vp]
    L.nvfp4_gg_run.restype = ctypes.c_int
    L.nvfp4_gg_run.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    L.nvfp4_gg_plan_info.restype = ctypes.c_int
    L.nvfp4_gg_plan_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    L.nvfp4_gg_destroy.restype = None
    L.nvfp4_gg_destroy.argtypes = [vp]
    L.nvfp4_gg_status_string.restype = ctypes.c_char_p
    L.nvfp4_gg_status_string.argtypes = [ctypes.c_int]
    return L


_lib = _load()


def library():
    """The loaded ctypes handle of libnvfp4gg.so."""
    return _lib


class Plan:
    """Owns one nvfp4_gg_plan_t; released by nvfp4_gg_destroy (or when collected)."""

    def __init__(self, handle: int, m, n: int, k: int):
        self.handle = handle
        self.m = list(m)
        self.n = n
        self.k = k

    @property
    def g(self) -> int:
        return len(self.m)

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.nvfp4_gg_destroy(ctypes.c_void_p(self.handle))
            self.handle = None


class RunArgs:
    """Five host arrays of device pointers, prepared once and reusable across calls."""

    def __init__(self, g: int, A, B, SFA, SFB, C):
        arr = ctypes.c_void_p * g
        self.keep = (A, B, SFA, SFB, C)  # keep tensors alive while the arrays exist
        self.arrays = tuple(arr(*[_addr(x) for x in seq]) for seq in (A, B, SFA, SFB, C))
        for seq in (A, B, SFA, SFB, C):
            if len(seq) != g:
                raise ValueError("every pointer list must have one entry per group")


def _addr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if not x.is_contiguous():
            raise ValueError("operand tensors must be contiguous")
        return x.data_ptr() if x.numel() else None
    raise TypeError("expected a device tensor or an integer device address")


def _stream_handle(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def nvfp4_gg_status_string(status: int) -> str:
    return _lib.nvfp4_gg_status_string(int(status)).decode()


def nvfp4_gg_plan(m: Sequence[int], n: int, k: int, device: int = -1,
                  scale_layout: int = SCALES_ROW_MAJOR) -> Plan:
    g = len(m)
    out = ctypes.c_void_p()
    marr = (ctypes.c_int * max(g, 1))(*[int(x) for x in m])
    st = _lib.nvfp4_gg_plan_layout(ctypes.byref(out), g, marr if g else None, int(n), int(k), int(device),
                                   int(scale_layout))
    if st != OK:
        raise Nvfp4GGError(st, "nvfp4_gg_plan_layout")
    return Plan(out.value, m, int(n), int(k))


def nvfp4_gg_plan_problems(problems, device: int = -1, scale_layout: int = SCALES_ROW_MAJOR) -> Plan:
    """problems: sequence of (m, n, k) or (m, n, k, ldc) per group (ldc 0 = n)."""
    g = len(problems)
    arr = (Problem * max(g, 1))()
    for i, pr in enumerate(problems):
        m_, n_, k_ = (int(x) for x in pr[:3])
        arr[i] = Problem(m_, n_, k_, int(pr[3]) if len(pr) > 3 else 0)
    out = ctypes.c_void_p()
    st = _lib.nvfp4_gg_plan_problems(ctypes.byref(out), g, arr if g else None, int(device), int(scale_layout))
    if st != OK:
        raise Nvfp4GGError(st, "nvfp4_gg_plan_problems")
    plan = Plan(out.value, [int(pr[0]) for pr in problems], 0, 0)
    plan.problems = [tuple(int(x) for x in pr) for pr in problems]
    return plan


def nvfp4_gg_blocked_scale_bytes(rows: int, k: int) -> int:
    return int(_lib.nvfp4_gg_blocked_scale_bytes(int(rows), int(k)))


def nvfp4_gg_scales_to_blocked(dst, src, rows: int, k: int, stream=None) -> None:
    """Enqueue the row-major -> 128x4 blocked conversion of one scale tensor (device
    tensors or addresses; dst holds nvfp4_gg_blocked_scale_bytes(rows, k) bytes)."""
    st = _lib.nvfp4_gg_scales_to_blocked(ctypes.c_void_p(_addr(dst)), ctypes.c_void_p(_addr(src)), int(rows),
                                         int(k), ctypes.c_void_p(_stream_handle(stream)))
    if st != OK:
        raise Nvfp4GGError(st, "nvfp4_gg_scales_to_blocked")


def nvfp4_gg_run(plan: Plan, A=None, B=None, SFA=None, SFB=None, C=None, stream=None,
                 args: RunArgs | None = None) -> None:
    if args is None:
        args = RunArgs(plan.g, A, B, SFA, SFB, C)
    st = _lib.nvfp4_gg_run(ctypes.c_void_p(plan.handle), *[ctypes.cast(a, ctypes.c_void_p) for a in args.arrays],
                           ctypes.c_void_p(_stream_handle(stream)))
    if st != OK:
        raise Nvfp4GGError(st, "nvfp4_gg_run")


def nvfp4_gg_plan_info(plan: Plan) -> PlanInfo:
    info = PlanInfo()
    st = _lib.nvfp4_gg_plan_info(ctypes.c_void_p(plan.handle), ctypes.byref(info))
    if st != OK:
        raise Nvfp4GGError(st, "nvfp4_gg_plan_info")
    return info


def nvfp4_gg_destroy(plan: Plan) -> None:
    if plan.handle:
        _lib.nvfp4_gg_destroy(ctypes.c_void_p(plan.handle))
        plan.handle = None


def device_operands(A, B, SFA, SFB, device="cuda"):
    """Copy host uint8 operand arrays (numpy, caller group order) to device tensors."""
    import torch
    up = lambda arrs: [torch.from_numpy(a).to(device) for a in arrs]
    return up(A), up(B), up(SFA), up(SFB)
