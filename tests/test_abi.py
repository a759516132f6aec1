"""C-ABI checks that need no GPU: the library loads, exports every declared symbol, and
its host-side validation and planning behave as include/nvfp4_gg.h documents."""
import ctypes
import os
import re
import subprocess

import pytest

import precision_moe_nvfp4_amd as gg
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "nvfp4_gg.h")


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^\s*(?:nvfp4_gg_status_t|void|size_t|const char\s*\*)\s*(nvfp4_gg_\w+)\s*\(", text, re.M)


def test_header_declares_the_entry_points():
    assert set(declared_functions()) == {
        "nvfp4_gg_plan", "nvfp4_gg_plan_layout", "nvfp4_gg_plan_problems", "nvfp4_gg_run", "nvfp4_gg_plan_info", "nvfp4_gg_destroy",
        "nvfp4_gg_status_string", "nvfp4_gg_blocked_scale_bytes", "nvfp4_gg_scales_to_blocked"}


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", gg.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, re.M))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(gg.library(), name) is not None


def test_status_strings():
    for st in range(6):
        s = gg.nvfp4_gg_status_string(st)
        assert s and s != "unknown status"
    assert gg.nvfp4_gg_status_string(99) == "unknown status"


def raw_plan(g, m, n, k, device=gg.DEVICE_NONE):
    out = ctypes.c_void_p(1234)
    marr = (ctypes.c_int * max(len(m), 1))(*m) if m is not None else None
    st = gg.library().nvfp4_gg_plan(ctypes.byref(out), g, marr, n, k, device)
    return st, out.value


@pytest.mark.parametrize("g,m,n,k", [
    (0, [], 64, 256), (1, [4], 0, 256), (1, [4], 64, 96), (1, [4], 64, 300), (1, [4], 64, 0), (1, [4], 64, 32),
    (1, [-1], 64, 256), (1, None, 64, 256), (2, [1, (1 << 20) + 1], 64, 256),
])
def test_plan_rejects_bad_arguments(g, m, n, k):
    st, handle = raw_plan(g, m, n, k)
    assert st == gg.EINVAL and handle is None


def test_plan_limits():
    st, handle = raw_plan(65, [1] * 65, 64, 256)
    assert st == gg.EUNSUPPORTED and handle is None
    st, handle = raw_plan(1, [1], 64, 256, device=-3)
    assert st == gg.EINVAL
    st = gg.library().nvfp4_gg_plan(None, 1, (ctypes.c_int * 1)(1), 64, 256, gg.DEVICE_NONE)
    assert st == gg.EINVAL


def ceil_div(a, b):
    return -(-a // b)


@pytest.mark.parametrize("m,n,k", [
    ([80, 176, 128, 72, 64, 248, 96, 160], 4096, 7168),
    ([40, 76, 168, 72, 164, 148, 196, 160], 7168, 2048),
    ([128, 384], 4096, 1536), ([0, 5, 0, 300], 200, 256), ([64] * 64, 256, 512), ([8192], 4096, 4096)])
def test_host_plan_order_and_unit_prefix(m, n, k):
    plan = gg.nvfp4_gg_plan(m, n, k, device=gg.DEVICE_NONE)
    info = gg.nvfp4_gg_plan_info(plan)
    g = len(m)
    assert (info.g, info.n, info.k, info.device, info.num_cus) == (g, n, k, gg.DEVICE_NONE, 256)
    order = list(info.order)[:g]
    assert sorted(order) == list(range(g))
    # largest group first, ties keep the caller order
    assert order == sorted(range(g), key=lambda i: (-m[i], i))
    # each group's units: row chunks of unit_rows times column tiles of unit_cols
    units = []
    for s in range(g):
        mi, ur, uc = m[order[s]], info.unit_rows[s], info.unit_cols[s]
        if mi == 0:
            assert ur == 0 and uc == 0
            units.append(0)
            continue
        assert ur % 32 == 0 and uc % 32 == 0 and (ur // 32) * (uc // 32) <= 20
        units.append(ceil_div(mi, ur) * ceil_div(n, uc))
    prefix = [0]
    for t in units:
        prefix.append(prefix[-1] + t)
    assert list(info.tile_begin)[:g + 1] == prefix
    assert info.total_tiles == prefix[-1]
    # grid: 8 XCDs x virtual workgroups per XCD, one unit range per workgroup
    assert info.grid % 8 == 0 and info.grid <= 256
    assert info.grid >= min(prefix[-1], 256) and info.grid < min(prefix[-1], 256) + 8
    assert (info.block, info.lds_bytes) == (256, 160 * 1024)
    assert info.tile_m == max(info.unit_rows[s] for s in range(g))
    assert info.est_us > 0


def test_page_shapes_plan_to_one_unit_range_per_workgroup():
    # c4 needs 17 accumulator blocks per CU on average; units of up to 20 blocks give every
    # workgroup at most one unit, and c1/c2 fill every workgroup they use with one unit
    for m, n, k, most in (([80, 176, 128, 72, 64, 248, 96, 160], 4096, 7168, 1), ([128, 384], 4096, 1536, 1),
                          ([192, 320], 3072, 4096, 1)):
        info = gg.nvfp4_gg_plan_info(gg.nvfp4_gg_plan(m, n, k, device=gg.DEVICE_NONE))
        assert ceil_div(info.total_tiles, info.grid) <= most, (m, info.total_tiles, info.grid)


def test_run_validates_pointers_before_touching_the_device():
    m, n, k = [4, 0], 64, 256
    plan = gg.nvfp4_gg_plan(m, n, k, device=gg.DEVICE_NONE)
    ok = [0x10000, 0]            # group 1 has m = 0: its pointers are ignored
    # every pointer valid -> validation passes, then the host-only plan is refused
    with pytest.raises(gg.Nvfp4GGError) as e:
        gg.nvfp4_gg_run(plan, ok, ok, ok, ok, ok, stream=0)
    assert e.value.status == gg.EUNSUPPORTED
    with pytest.raises(gg.Nvfp4GGError) as e:
        gg.nvfp4_gg_run(plan, [0, 0], ok, ok, ok, ok, stream=0)
    assert e.value.status == gg.EINVAL
    with pytest.raises(gg.Nvfp4GGError) as e:
        gg.nvfp4_gg_run(plan, ok, [0x10008, 0], ok, ok, ok, stream=0)
    assert e.value.status == gg.EALIGN
    with pytest.raises(gg.Nvfp4GGError) as e:
        gg.nvfp4_gg_run(plan, ok, ok, ok, ok, [0x10002, 0], stream=0)
    assert e.value.status == gg.EALIGN
    L = gg.library()
    assert L.nvfp4_gg_run(ctypes.c_void_p(plan.handle), None, None, None, None, None, None) == gg.EINVAL
    assert L.nvfp4_gg_run(None, None, None, None, None, None, None) == gg.EINVAL
    gg.nvfp4_gg_destroy(plan)
    gg.nvfp4_gg_destroy(plan)    # second destroy is a no-op on the Python side
    L.nvfp4_gg_destroy(None)


def test_plan_info_rejects_null():
    L = gg.library()
    assert L.nvfp4_gg_plan_info(None, None) == gg.EINVAL


def test_plan_layout_validation_and_info():
    L = gg.library()
    out = ctypes.c_void_p(1234)
    marr = (ctypes.c_int * 2)(100, 3)
    assert L.nvfp4_gg_plan_layout(ctypes.byref(out), 2, marr, 64, 256, gg.DEVICE_NONE, 2) == gg.EINVAL
    assert out.value is None
    assert L.nvfp4_gg_plan_layout(ctypes.byref(out), 2, marr, 64, 256, gg.DEVICE_NONE, -1) == gg.EINVAL
    for layout in (gg.SCALES_ROW_MAJOR, gg.SCALES_BLOCKED):
        plan = gg.nvfp4_gg_plan([100, 3], 64, 256, device=gg.DEVICE_NONE, scale_layout=layout)
        info = gg.nvfp4_gg_plan_info(plan)
        assert info.scale_layout == layout
        assert info.variant == (6 if layout == gg.SCALES_BLOCKED else 5)
        assert info.total_tiles > 0


@pytest.mark.parametrize("rows,k,expect", [
    (1, 256, 2048), (128, 256, 2048), (129, 256, 4096), (300, 1536, 3 * 24 * 512), (0, 256, 0), (-1, 256, 0),
    (10, 128, 1024), (200, 192, 2 * 3 * 512), (10, 96, 0), (10, 300, 0), (10, 32, 0),
])
def test_blocked_scale_bytes(rows, k, expect):
    assert gg.nvfp4_gg_blocked_scale_bytes(rows, k) == expect


def test_scales_to_blocked_validates_before_touching_the_device():
    L = gg.library()
    vp = ctypes.c_void_p
    assert L.nvfp4_gg_scales_to_blocked(vp(16), vp(32), 10, 300, None) == gg.EINVAL
    assert L.nvfp4_gg_scales_to_blocked(vp(16), vp(32), -1, 256, None) == gg.EINVAL
    assert L.nvfp4_gg_scales_to_blocked(None, vp(32), 10, 256, None) == gg.EINVAL
    assert L.nvfp4_gg_scales_to_blocked(vp(16), vp(36), 10, 256, None) == gg.EALIGN
    assert L.nvfp4_gg_scales_to_blocked(None, None, 0, 256, None) == gg.OK


@pytest.mark.parametrize("problems", [
    [(4, 0, 256, 0)], [(4, 64, 96, 0)], [(4, 64, 300, 0)], [(4, 64, 32, 0)], [(-1, 64, 256, 0)], [(4, 64, 256, 63)],
    [(4, 64, 256, -1)], [(4, (1 << 20) + 1, 256, 0)], [(1, 64, 256, 0), (1, 64, (1 << 20) + 256, 0)],
])
def test_plan_problems_rejects_bad_sizes(problems):
    with pytest.raises(gg.Nvfp4GGError) as e:
        gg.nvfp4_gg_plan_problems(problems, device=gg.DEVICE_NONE)
    assert e.value.status == gg.EINVAL


def test_plan_problems_mixed_sizes():
    probs = [(100, 256, 512, 0), (0, 1000, 256, 0), (300, 130, 1024, 136), (7, 64, 256, 64)]
    plan = gg.nvfp4_gg_plan_problems(probs, device=gg.DEVICE_NONE)
    info = gg.nvfp4_gg_plan_info(plan)
    assert info.g == 4 and info.n == 0 and info.k == 0        # sizes differ between groups
    # largest work first: m * n * k
    work = [m * n * k for m, n, k, _ in probs]
    order = [info.order[s] for s in range(4)]
    assert order == sorted(range(4), key=lambda i: -work[i])
    units = [ceil_div(probs[order[s]][0], info.unit_rows[s]) * ceil_div(probs[order[s]][1], info.unit_cols[s])
             if probs[order[s]][0] else 0 for s in range(4)]
    assert [info.tile_begin[s + 1] - info.tile_begin[s] for s in range(4)] == units
    # uniform sizes report n and k
    plan2 = gg.nvfp4_gg_plan_problems([(10, 256, 512), (20, 256, 512)], device=gg.DEVICE_NONE)
    info2 = gg.nvfp4_gg_plan_info(plan2)
    assert (info2.n, info2.k) == (256, 512)


@pytest.mark.parametrize("k", [256, 64, 192, 1088, 7168])
def test_k_granularity_and_variant(k):
    # every multiple of 64 plans (a short last K step); the kernel variant follows the scale
    # layout only
    plan = gg.nvfp4_gg_plan([100, 7], 96, k, device=gg.DEVICE_NONE)
    assert gg.nvfp4_gg_plan_info(plan).variant == 5
    blocked = gg.nvfp4_gg_plan([100, 7], 96, k, device=gg.DEVICE_NONE, scale_layout=gg.SCALES_BLOCKED)
    assert gg.nvfp4_gg_plan_info(blocked).variant == 6
    mixed = gg.nvfp4_gg_plan_problems([(10, 64, 512), (10, 64, k)], device=gg.DEVICE_NONE)
    assert gg.nvfp4_gg_plan_info(mixed).total_tiles >= 2


def test_build_script_loads_without_the_package():
    """build() must work on a tree where the library is not built yet: the build script is
    loaded by path and must not import the package (whose __init__ loads the library)."""
    import subprocess
    import sys
    code = ("import sys, __graft_entry__ as g; m = g._hip_build_module(); "
            "assert callable(m.build); "
            "assert 'precision_moe_nvfp4_amd' not in sys.modules, 'package imported'")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    subprocess.run([sys.executable, "-c", code], cwd=root, check=True)


def test_library_imports_no_allocation_copy_or_device_sync():
    # the plan is host memory and a call is one launch: the library does not even link the HIP
    # entry points that allocate, copy, free or synchronise the device
    out = subprocess.run(["nm", "-D", "--undefined-only", gg.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    imported = {line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()}
    for forbidden in ("hipMalloc", "hipFree", "hipMemcpy", "hipMemcpyAsync", "hipMemset", "hipMemsetAsync",
                      "hipDeviceSynchronize", "hipStreamSynchronize", "hipHostMalloc", "hipExtMallocWithFlags"):
        assert forbidden not in imported, forbidden
    assert "hipLaunchKernel" in imported


def _kernel_metadata():
    """The unit kernel's code-object metadata (registers, LDS, scratch) read from the built
    library's gfx950 code object with the ROCm LLVM tools; None when they are missing."""
    import os
    import shutil
    import tempfile
    llvm = "/opt/rocm/llvm/bin"
    tools = [os.path.join(llvm, t) for t in ("clang-offload-bundler", "llvm-readelf")]
    if not all(os.path.exists(t) for t in tools) or shutil.which("objcopy") is None:
        return None
    with tempfile.TemporaryDirectory() as d:
        fat, co = os.path.join(d, "fat.bin"), os.path.join(d, "k.co")
        subprocess.run(["objcopy", "--dump-section", f".hip_fatbin={fat}", gg.LIB_PATH], check=True,
                       capture_output=True)
        subprocess.run([tools[0], "--unbundle", "--type=o", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                        f"--input={fat}", f"--output={co}"], check=True, capture_output=True)
        notes = subprocess.run([tools[1], "--notes", co], check=True, capture_output=True, text=True).stdout
    meta, cur = {}, None
    for line in notes.splitlines():
        line = line.strip().lstrip("- ")
        if ":" not in line:
            continue
        key, val = (s.strip() for s in line.split(":", 1))
        if key == ".agpr_count":
            cur = {key: val}
        elif cur is not None:
            cur[key] = val
            if key == ".name":
                meta[val] = cur
    return meta


def test_unit_kernel_uses_no_scratch():
    # the unit kernel keeps everything in registers and LDS: no scratch (a kernel with a larger
    # scratch allocation launches its waves markedly slower), one workgroup's 160 KiB of LDS
    meta = _kernel_metadata()
    if meta is None:
        pytest.skip("ROCm LLVM tools not available")
    k = [v for name, v in meta.items() if "nvfp4_gg_units" in name]
    assert len(k) == 1
    assert int(k[0][".private_segment_fixed_size"]) == 0
    assert int(k[0][".group_segment_fixed_size"]) == 160 * 1024
    assert int(k[0][".vgpr_count"]) <= 512
