"""The C ABI on the host: the library loads, exports what include/xp.h declares, and
validates arguments synchronously. No kernel is launched here (no GPU needed)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

from fp4_routed_expert_xp_amd import xp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "xp.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(xp_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(xp.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = xp.lib()
    for name in _declared():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", xp.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (xp_\w+)", out))
    assert exported == set(_declared())


def test_library_links_no_oracle_or_torch():
    out = subprocess.run(["readelf", "-d", xp.LIB_PATH], capture_output=True, text=True).stdout
    needed = re.findall(r"NEEDED.*\[(.*)\]", out)
    assert not any("oracle" in n or "torch" in n or "c10" in n for n in needed), needed


def test_status_strings():
    for s in range(-6, 1):
        assert xp.xp_status_string(s).startswith("XP_")
    assert "unknown" in xp.xp_status_string(99)


def test_workspace_layout_is_ordered_and_fits():
    d = xp.dims(4096, 2048, 256, 8)
    for rows in (1, 4, 16, 64, 65, 4096):
        off = xp.xp_workspace_layout(d, rows)
        assert off == sorted(off) and all(o % 256 == 0 for o in off)
        total = xp.xp_workspace_bytes(d, rows)
        assert total >= off[-1] + rows * 8 * 16
    assert xp.xp_workspace_bytes(xp.dims(100, 2048, 256, 8), 4) == 0   # hidden not a multiple of 64


@pytest.mark.parametrize("dims,status", [
    ((4096, 2048, 256, 0), xp.XP_ERR_TOPK),
    ((4096, 2048, 256, 17), xp.XP_ERR_TOPK),
    ((4096, 2048, 4, 8), xp.XP_ERR_TOPK),
    ((4000, 2048, 256, 8), xp.XP_ERR_SHAPE),
    ((4096, 2000, 256, 8), xp.XP_ERR_SHAPE),
    ((4096, 2048, 2048, 8), xp.XP_ERR_SHAPE),
])
def test_bad_dims_rejected_before_any_launch(dims, status):
    L = xp.lib()
    d = xp.dims(*dims)
    P = ctypes.c_void_p(0x1000)
    assert L.xp_route_bucket(ctypes.byref(d), 4, P, P, P, P, 1 << 30, None) == status
    assert L.xp_gateup_rows(ctypes.byref(d), 4, P, P, P, 1 << 30, P, None) == status
    assert L.xp_down_rows(ctypes.byref(d), 4, P, P, P, 1 << 30, P, None) == status
    assert L.xp_combine(ctypes.byref(d), 4, P, P, P, None) == status
    assert L.xp_prefill_gateup(ctypes.byref(d), 4, P, P, P, 1 << 30, P, None) == status
    assert L.xp_prefill_down(ctypes.byref(d), 4, P, P, P, 1 << 30, P, None) == status
    assert L.xp_gateup_rows_act16(ctypes.byref(d), 4, P, P, P, 1 << 30, P, None) == status
    assert L.xp_down_rows_act16(ctypes.byref(d), 4, P, P, P, 1 << 30, P, None) == status
    assert L.xp_combine_y16(ctypes.byref(d), 4, P, P, P, None) == status


def test_null_rows_and_workspace_checks():
    L = xp.lib()
    d = xp.dims(256, 128, 8, 2)
    P = ctypes.c_void_p(0x1000)
    assert L.xp_route_bucket(None, 4, P, P, P, P, 1 << 20, None) == xp.XP_ERR_NULL
    assert L.xp_route_bucket(ctypes.byref(d), -1, P, P, P, P, 1 << 20, None) == xp.XP_ERR_SHAPE
    assert L.xp_route_bucket(ctypes.byref(d), 0, None, None, None, None, 0, None) == xp.XP_OK  # empty batch
    assert L.xp_gateup_rows(ctypes.byref(d), 0, None, None, None, 0, None, None) == xp.XP_OK
    assert L.xp_down_rows(ctypes.byref(d), 0, None, None, None, 0, None, None) == xp.XP_OK
    assert L.xp_combine(ctypes.byref(d), 0, None, None, None, None) == xp.XP_OK
    assert L.xp_route_bucket(ctypes.byref(d), 4, None, P, P, P, 1 << 20, None) == xp.XP_ERR_NULL
    need = xp.xp_workspace_bytes(d, 4)
    assert L.xp_route_bucket(ctypes.byref(d), 4, P, P, P, P, need - 1, None) == xp.XP_ERR_WORKSPACE
    assert L.xp_gateup_rows(ctypes.byref(d), 4, P, P, P, need - 1, P, None) == xp.XP_ERR_WORKSPACE
    assert L.xp_down_rows(ctypes.byref(d), 4, P, P, P, need - 1, P, None) == xp.XP_ERR_WORKSPACE
    assert L.xp_gateup_rows_split(ctypes.byref(d), 4, P, P, P, need, P, None, None) == xp.XP_ERR_NULL
    assert L.xp_route_gateup(ctypes.byref(d), 4, P, P, P, P, None, P, need, P, None) == xp.XP_ERR_NULL
    assert L.xp_route_gateup(ctypes.byref(d), 4, P, P, P, P, P, P, need - 1, P, None) == xp.XP_ERR_WORKSPACE
    assert L.xp_down_combine(ctypes.byref(d), 4, P, P, None, P, need, P, P, None) == xp.XP_ERR_NULL
    assert L.xp_down_combine(ctypes.byref(d), 0, None, None, None, None, 0, None, None, None) == xp.XP_OK
    assert L.xp_prefill_gateup(ctypes.byref(d), 0, None, None, None, 0, None, None) == xp.XP_OK
    assert L.xp_prefill_down(ctypes.byref(d), 0, None, None, None, 0, None, None) == xp.XP_OK
    assert L.xp_prefill_gateup(ctypes.byref(d), -1, P, P, P, need, P, None) == xp.XP_ERR_SHAPE
    assert L.xp_prefill_gateup(ctypes.byref(d), 4, None, P, P, need, P, None) == xp.XP_ERR_NULL
    assert L.xp_prefill_down(ctypes.byref(d), 4, P, P, P, need, None, None) == xp.XP_ERR_NULL
    assert L.xp_prefill_gateup(ctypes.byref(d), 4, P, P, P, need - 1, P, None) == xp.XP_ERR_WORKSPACE
    # x of 4 GiB or more is refused (its loads use 32-bit offsets), before any launch
    big = (1 << 32) // (2 * d.hidden)
    assert L.xp_prefill_gateup(ctypes.byref(d), big, P, P, P, xp.xp_workspace_bytes(d, big), P,
                               None) == xp.XP_ERR_SHAPE
    assert L.xp_prefill_down(ctypes.byref(d), 4, P, P, P, need - 1, P, None) == xp.XP_ERR_WORKSPACE
    assert L.xp_pack_matrix(100, 64, P, P, P, P, None) == xp.XP_ERR_SHAPE
    assert L.xp_pack_matrix(64, 48, P, P, P, P, None) == xp.XP_ERR_SHAPE
    assert L.xp_pack_matrix(64, 64, None, P, P, P, None) == xp.XP_ERR_NULL


def test_tiers_set_get_and_refusals():
    assert xp.xp_get_tiers() == ([2, 4, 6, 8], [2, 4])
    try:
        xp.xp_set_tiers([4], [4])
        assert xp.xp_get_tiers() == ([4], [4])
        xp.xp_set_tiers([2, 4, 8], None)
        assert xp.xp_get_tiers() == ([2, 4, 8], [2, 4])
        for bad in ([1, 2], [2, 2], [4, 2], [2, 9], [0], list(range(2, 10))):
            with pytest.raises(xp.XPError) as ei:
                xp.xp_set_tiers(bad, [2])
            assert ei.value.status == xp.XP_ERR_TIERS
        assert xp.xp_get_tiers() == ([2, 4, 8], [2, 4])    # refused lists change nothing
    finally:
        xp.xp_set_tiers(None, None)
    assert xp.xp_get_tiers() == ([2, 4, 6, 8], [2, 4])


def test_fp8_argument_checks():
    L = xp.lib()
    P = ctypes.c_void_p(16)
    assert xp.xp_fp8_packed_bytes(576, 4096) == 576 * 4096
    for n, k in ((100, 4096), (576, 4000), (0, 128), (16, 0), (16, 128 * 65)):
        assert xp.xp_fp8_packed_bytes(n, k) == 0, (n, k)
        assert L.xp_fp8_pack(n, k, P, P, None) == xp.XP_ERR_SHAPE
        assert L.xp_fp8_rows(1, n, k, P, P, P, P, 0, None) == xp.XP_ERR_SHAPE
    assert L.xp_fp8_pack(16, 128, None, P, None) == xp.XP_ERR_NULL
    assert L.xp_fp8_rows(1, 16, 128, P, None, P, P, 0, None) == xp.XP_ERR_NULL
    assert L.xp_fp8_rows(-1, 16, 128, P, P, P, P, 0, None) == xp.XP_ERR_SHAPE
    assert L.xp_fp8_rows(0, 16, 128, None, None, None, None, 0, None) == xp.XP_OK
    # forms: a power of two up to 16, at most P = next power of two of k/128, P/slices <= 4
    for slices in (3, 32, -1, 8):
        assert L.xp_fp8_rows(1, 16, 512, P, P, P, P, slices, None) == xp.XP_ERR_SHAPE, slices
    assert L.xp_fp8_rows(1, 16, 128 * 40, P, P, P, P, 4, None) == xp.XP_ERR_SHAPE  # P = 64: 16 blocks a slice
    assert L.xp_fp8_rows_f32(1, 100, 4096, P, P, P, P, 0, None) == xp.XP_ERR_SHAPE
    assert L.xp_fp8_rows_f32(1, 16, 128, None, P, P, P, 0, None) == xp.XP_ERR_NULL
    assert L.xp_fp8_rows_f32(0, 16, 128, None, None, None, None, 0, None) == xp.XP_OK
    # misaligned pointers are refused before any launch
    odd = ctypes.c_void_p(0x1008)
    assert L.xp_fp8_rows(1, 16, 128, odd, P, P, P, 0, None) == xp.XP_ERR_SHAPE
    assert L.xp_fp8_rows_f32(1, 16, 128, P, odd, P, P, 0, None) == xp.XP_ERR_SHAPE
    assert L.xp_fp8_pack(16, 128, ctypes.c_void_p(0x1004), P, None) == xp.XP_ERR_SHAPE


def test_bf16_storage_argument_checks():
    L = xp.lib()
    d = xp.dims(256, 128, 8, 2)
    P = ctypes.c_void_p(0x1000)
    need = xp.xp_workspace_bytes(d, 4)
    assert L.xp_gateup_rows_act16(ctypes.byref(d), 0, None, None, None, 0, None, None) == xp.XP_OK
    assert L.xp_down_rows_act16(ctypes.byref(d), 0, None, None, None, 0, None, None) == xp.XP_OK
    assert L.xp_combine_y16(ctypes.byref(d), 0, None, None, None, None) == xp.XP_OK
    assert L.xp_gateup_rows_act16(ctypes.byref(d), 4, P, P, P, need, None, None) == xp.XP_ERR_NULL
    assert L.xp_down_rows_act16(ctypes.byref(d), 4, None, P, P, need, P, None) == xp.XP_ERR_NULL
    assert L.xp_combine_y16(ctypes.byref(d), 4, P, P, None, None) == xp.XP_ERR_NULL
    assert L.xp_gateup_rows_act16(ctypes.byref(d), 4, P, P, P, need - 1, P, None) == xp.XP_ERR_WORKSPACE
    assert L.xp_down_rows_act16(ctypes.byref(d), 4, P, P, P, need - 1, P, None) == xp.XP_ERR_WORKSPACE
    assert L.xp_combine_y16(ctypes.byref(d), -1, P, P, P, None) == xp.XP_ERR_SHAPE


def _tiers_in_child(env):
    code = ("from fp4_routed_expert_xp_amd import xp\n"
            "xp.lib()\n"
            "print(xp.xp_get_tiers())\n")
    full = dict(os.environ, **env)
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=full, cwd=ROOT)


def test_tiers_from_environment():
    r = _tiers_in_child({"XP_TIERS_GU": "4", "XP_TIERS_DN": " "})
    assert r.returncode == 0, r.stderr
    assert "[4]" in r.stdout and "[2, 4]" in r.stdout          # blank keeps the default for down
    r = _tiers_in_child({"XP_TIERS_GU": "2,x", "XP_TIERS_DN": ""})
    assert r.returncode != 0 and "XP_TIERS_GU" in r.stderr
    r = _tiers_in_child({"XP_TIERS_GU": "", "XP_TIERS_DN": "4,2"})
    assert r.returncode != 0 and "XP_TIERS_DN" in r.stderr


def test_stream_probe_argument_checks():
    L = xp.lib()
    d = xp.dims(256, 128, 8, 2)
    P = ctypes.c_void_p(0x1000)
    assert L.xp_stream_weights(ctypes.byref(d), None, None, 0, 7, None, None) == xp.XP_OK   # nothing to read
    assert L.xp_stream_weights(ctypes.byref(d), P, P, -1, 7, P, None) == xp.XP_ERR_SHAPE
    assert L.xp_stream_weights(ctypes.byref(d), P, P, 9, 7, P, None) == xp.XP_ERR_SHAPE    # more ids than experts
    for parts in (0, 8, -1):
        assert L.xp_stream_weights(ctypes.byref(d), P, P, 2, parts, P, None) == xp.XP_ERR_SHAPE
    assert L.xp_stream_weights(ctypes.byref(d), None, P, 2, 7, P, None) == xp.XP_ERR_NULL
    assert L.xp_stream_weights(ctypes.byref(d), P, P, 2, 3, None, None) == xp.XP_ERR_NULL
    bad = xp.dims(100, 128, 8, 2)
    assert L.xp_stream_weights(ctypes.byref(bad), P, P, 2, 7, P, None) == xp.XP_ERR_SHAPE


def test_coded_argument_checks():
    L = xp.lib()
    d = xp.dims(256, 128, 8, 2)
    P = ctypes.c_void_p(0x1000)
    need = xp.xp_workspace_bytes(d, 4)
    assert L.xp_gateup_rows_coded(ctypes.byref(d), 0, None, None, None, None, 0, None, None) == xp.XP_OK
    assert L.xp_gateup_rows_coded(ctypes.byref(d), 4, P, None, P, P, need, P, None) == xp.XP_ERR_NULL
    assert L.xp_gateup_rows_coded(ctypes.byref(d), 4, None, P, P, P, need, P, None) == xp.XP_ERR_NULL
    assert L.xp_gateup_rows_coded(ctypes.byref(d), 4, P, P, P, P, need - 1, P, None) == xp.XP_ERR_WORKSPACE
    assert L.xp_gateup_rows_coded(ctypes.byref(d), -1, P, P, P, P, need, P, None) == xp.XP_ERR_SHAPE
    bad = xp.dims(4000, 128, 8, 2)
    assert L.xp_gateup_rows_coded(ctypes.byref(bad), 4, P, P, P, P, need, P, None) == xp.XP_ERR_SHAPE


def test_fp8_multi_argument_checks():
    L = xp.lib()
    P = ctypes.c_void_p(16)
    arr = (xp.xp_fp8_matrix * 2)(xp.xp_fp8_matrix(16, 16, 16, 16), xp.xp_fp8_matrix(48, 16, 16, 16))
    assert L.xp_fp8_rows_multi(0, 128, None, arr, 2, 0, None) == xp.XP_OK
    assert L.xp_fp8_rows_multi(1, 128, P, arr, 0, 0, None) == xp.XP_ERR_SHAPE
    assert L.xp_fp8_rows_multi(1, 128, P, arr, 9, 0, None) == xp.XP_ERR_SHAPE
    assert L.xp_fp8_rows_multi(1, 128, P, None, 2, 0, None) == xp.XP_ERR_NULL
    assert L.xp_fp8_rows_multi(1, 100, P, arr, 2, 0, None) == xp.XP_ERR_SHAPE     # k not a multiple of 128
    bad = (xp.xp_fp8_matrix * 1)(xp.xp_fp8_matrix(20, 16, 16, 16))                 # n not a multiple of 16
    assert L.xp_fp8_rows_multi(1, 128, P, bad, 1, 0, None) == xp.XP_ERR_SHAPE
    nul = (xp.xp_fp8_matrix * 1)(xp.xp_fp8_matrix(16, None, 16, 16))
    assert L.xp_fp8_rows_multi(1, 128, P, nul, 1, 0, None) == xp.XP_ERR_NULL
    odd = (xp.xp_fp8_matrix * 1)(xp.xp_fp8_matrix(16, 0x1008, 16, 16))
    assert L.xp_fp8_rows_multi(1, 128, P, odd, 1, 0, None) == xp.XP_ERR_SHAPE
    assert L.xp_fp8_rows_multi(1, 128, ctypes.c_void_p(0x1008), arr, 2, 0, None) == xp.XP_ERR_SHAPE
