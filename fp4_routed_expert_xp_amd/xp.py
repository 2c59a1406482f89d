"""Thin Python binding of libxp.so: the same entry points, argument marshalling only.

PyTorch supplies device memory and streams; every step of the path runs in
the library's HIP kernels. ``torch`` is imported before the library is loaded
so that libxp binds to the HIP runtime torch already uses. There is no CPU
fallback: if ``libxp.so`` is missing this module raises when it is first used.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libxp.so")

XP_OK, XP_ERR_NULL, XP_ERR_SHAPE, XP_ERR_TOPK, XP_ERR_WORKSPACE, XP_ERR_TIERS, XP_ERR_HIP = 0, -1, -2, -3, -4, -5, -6

# every symbol include/xp.h declares
EXPORTS = (
    "xp_pack_matrix", "xp_workspace_bytes", "xp_workspace_layout", "xp_route_bucket",
    "xp_gateup_rows", "xp_gateup_rows_split", "xp_down_rows", "xp_combine",
    "xp_set_tiers", "xp_get_tiers", "xp_status_string", "xp_route_gateup", "xp_down_combine",
    "xp_prefill_gateup", "xp_prefill_down", "xp_fp8_packed_bytes", "xp_fp8_pack", "xp_fp8_rows",
    "xp_gateup_rows_act16", "xp_down_rows_act16", "xp_combine_y16", "xp_fp8_rows_f32", "xp_stream_weights",
    "xp_decode_static", "xp_gateup_rows_coded", "xp_fp8_rows_multi",
)


class xp_fp8_matrix(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("y", ctypes.c_void_p)]


class XPError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s: %s" % (where, xp_status_string(status)))
        self.status = status


class xp_dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32)]

    def __repr__(self):
        return "xp_dims(hidden=%d, inter=%d, n_experts=%d, top_k=%d)" % (
            self.hidden, self.inter, self.n_experts, self.top_k)


def dims(hidden: int, inter: int, n_experts: int, top_k: int) -> xp_dims:
    return xp_dims(hidden, inter, n_experts, top_k)


_lib = None


def lib():
    """Load libxp.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libxp.so is not built (%s); run `python -m fp4_routed_expert_xp_amd.build`"
                               % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        D = ctypes.POINTER(xp_dims)
        L.xp_pack_matrix.argtypes = [i32, i32, P, P, P, P, P]
        L.xp_workspace_bytes.argtypes = [D, i32]
        L.xp_workspace_bytes.restype = sz
        L.xp_workspace_layout.argtypes = [D, i32, ctypes.POINTER(sz)]
        L.xp_route_bucket.argtypes = [D, i32, P, P, P, P, sz, P]
        L.xp_gateup_rows.argtypes = [D, i32, P, P, P, sz, P, P]
        L.xp_gateup_rows_split.argtypes = [D, i32, P, P, P, sz, P, P, P]
        L.xp_down_rows.argtypes = [D, i32, P, P, P, sz, P, P]
        L.xp_combine.argtypes = [D, i32, P, P, P, P]
        L.xp_route_gateup.argtypes = [D, i32, P, P, P, P, P, P, sz, P, P]
        L.xp_down_combine.argtypes = [D, i32, P, P, P, P, sz, P, P, P]
        L.xp_prefill_gateup.argtypes = [D, i32, P, P, P, sz, P, P]
        L.xp_prefill_down.argtypes = [D, i32, P, P, P, sz, P, P]
        L.xp_gateup_rows_act16.argtypes = [D, i32, P, P, P, sz, P, P]
        L.xp_down_rows_act16.argtypes = [D, i32, P, P, P, sz, P, P]
        L.xp_combine_y16.argtypes = [D, i32, P, P, P, P]
        L.xp_fp8_packed_bytes.argtypes = [i32, i32]
        L.xp_fp8_packed_bytes.restype = sz
        L.xp_fp8_pack.argtypes = [i32, i32, P, P, P]
        L.xp_fp8_rows.argtypes = [i32, i32, i32, P, P, P, P, i32, P]
        L.xp_fp8_rows_f32.argtypes = [i32, i32, i32, P, P, P, P, i32, P]
        L.xp_stream_weights.argtypes = [D, P, P, i32, i32, P, P]
        L.xp_decode_static.argtypes = [D, i32, P, P, P, P, P, P, P, P, P]
        L.xp_gateup_rows_coded.argtypes = [D, i32, P, P, P, P, sz, P, P]
        L.xp_fp8_rows_multi.argtypes = [i32, i32, P, ctypes.POINTER(xp_fp8_matrix), i32, i32, P]
        L.xp_set_tiers.argtypes = [P, i32, P, i32]
        L.xp_get_tiers.argtypes = [P, P, P, P]
        L.xp_status_string.argtypes = [ctypes.c_int]
        L.xp_status_string.restype = ctypes.c_char_p
        for name in ("xp_pack_matrix", "xp_workspace_layout", "xp_route_bucket", "xp_gateup_rows",
                     "xp_gateup_rows_split", "xp_down_rows", "xp_combine", "xp_set_tiers", "xp_get_tiers",
                     "xp_route_gateup", "xp_down_combine", "xp_prefill_gateup", "xp_prefill_down",
                     "xp_fp8_pack", "xp_fp8_rows", "xp_gateup_rows_act16", "xp_down_rows_act16",
                     "xp_combine_y16", "xp_fp8_rows_f32", "xp_stream_weights", "xp_decode_static",
                     "xp_gateup_rows_coded", "xp_fp8_rows_multi"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
        try:
            _tiers_from_env()
        except ValueError:
            _lib = None
            raise
    return _lib


TIER_ENV = ("XP_TIERS_GU", "XP_TIERS_DN")


def _tiers_from_env() -> None:
    """Pass sizes from XP_TIERS_GU / XP_TIERS_DN ("2,4,6,8" style; unset or blank
    keeps the library's default). A malformed value is refused by name."""
    vals = []
    for name in TIER_ENV:
        v = os.environ.get(name, "").strip()
        if not v:
            vals.append(None)
            continue
        try:
            vals.append([int(t) for t in v.split(",")])
        except ValueError:
            raise ValueError("%s=%r: expected a comma-separated list of pass sizes" % (name, v)) from None
    if vals == [None, None]:
        return
    try:
        xp_set_tiers(*vals)
    except XPError:
        raise ValueError("%s=%r, %s=%r: pass sizes must be strictly increasing, each in 2..8"
                         % (TIER_ENV[0], os.environ.get(TIER_ENV[0], ""), TIER_ENV[1],
                            os.environ.get(TIER_ENV[1], ""))) from None


def xp_status_string(status: int) -> str:
    return lib().xp_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != XP_OK:
        raise XPError(status, where)


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, dtype, name: str, numel: int | None = None) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if numel is not None and t.numel() < numel:
        raise ValueError("%s holds %d elements, needs %d" % (name, t.numel(), numel))


def _dev_bf16(t: torch.Tensor, name: str, numel: int) -> None:
    """bf16 activations: a bfloat16 tensor or its 16-bit patterns (int16/uint16)."""
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError("%s must hold bf16 (bfloat16, or int16/uint16 bit patterns), got %s" % (name, t.dtype))
    _dev(t, t.dtype, name, numel)


# ----------------------------------------------------------------- host calls
def xp_workspace_bytes(d: xp_dims, max_rows: int) -> int:
    return int(lib().xp_workspace_bytes(ctypes.byref(d), int(max_rows)))


def xp_workspace_layout(d: xp_dims, max_rows: int) -> list:
    off = (ctypes.c_size_t * 6)()
    _check(lib().xp_workspace_layout(ctypes.byref(d), int(max_rows), off), "xp_workspace_layout")
    return list(off)


def xp_set_tiers(gu=None, dn=None) -> None:
    def arr(t):
        if not t:
            return None, 0
        a = (ctypes.c_int32 * len(t))(*[int(v) for v in t])
        return a, len(t)
    ga, gn = arr(gu)
    da, dn_ = arr(dn)
    _check(lib().xp_set_tiers(ga, gn, da, dn_), "xp_set_tiers")


def xp_get_tiers():
    g = (ctypes.c_int32 * 8)()
    d = (ctypes.c_int32 * 8)()
    ng, nd = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().xp_get_tiers(g, ctypes.byref(ng), d, ctypes.byref(nd)), "xp_get_tiers")
    return list(g)[:ng.value], list(d)[:nd.value]


# --------------------------------------------------------------- device calls
def xp_pack_matrix(codes: torch.Tensor, scales: torch.Tensor, packed_codes: torch.Tensor,
                   packed_scales: torch.Tensor, stream=None) -> None:
    N, half = codes.shape
    K = 2 * half
    _dev(codes, torch.uint8, "codes")
    _dev(scales, torch.uint8, "scales", N * (K // 32))
    _dev(packed_codes, torch.uint8, "packed_codes", N * half)
    _dev(packed_scales, torch.uint8, "packed_scales", N * (K // 32))
    _check(lib().xp_pack_matrix(N, K, _ptr(codes), _ptr(scales), _ptr(packed_codes), _ptr(packed_scales),
                                _stream(stream)), "xp_pack_matrix")


def xp_route_bucket(d: xp_dims, rows: int, logits, topk_id, topk_w, workspace, stream=None) -> None:
    if rows > 0:
        _dev(logits, torch.float32, "logits", rows * d.n_experts)
        _dev(topk_id, torch.int32, "topk_id", rows * d.top_k)
        _dev(topk_w, torch.float32, "topk_w", rows * d.top_k)
        _dev(workspace, torch.uint8, "workspace")
    nbytes = workspace.numel() if workspace is not None else 0
    _check(lib().xp_route_bucket(ctypes.byref(d), int(rows), _ptr(logits), _ptr(topk_id), _ptr(topk_w),
                                 _ptr(workspace), nbytes, _stream(stream)), "xp_route_bucket")


def xp_gateup_rows(d: xp_dims, rows: int, x, experts, workspace, act, stream=None) -> None:
    if rows > 0:
        _dev_bf16(x, "x", rows * d.hidden)
        _dev(experts, torch.int64, "experts", d.n_experts * 6)
        _dev(act, torch.float32, "act", rows * d.top_k * d.inter)
    nbytes = workspace.numel() if workspace is not None else 0
    _check(lib().xp_gateup_rows(ctypes.byref(d), int(rows), _ptr(x), _ptr(experts), _ptr(workspace), nbytes,
                                _ptr(act), _stream(stream)), "xp_gateup_rows")


def xp_gateup_rows_split(d: xp_dims, rows: int, x, experts, workspace, g, u, stream=None) -> None:
    if rows > 0:
        _dev_bf16(x, "x", rows * d.hidden)
        _dev(experts, torch.int64, "experts", d.n_experts * 6)
        _dev(g, torch.float32, "g", rows * d.top_k * d.inter)
        _dev(u, torch.float32, "u", rows * d.top_k * d.inter)
    nbytes = workspace.numel() if workspace is not None else 0
    _check(lib().xp_gateup_rows_split(ctypes.byref(d), int(rows), _ptr(x), _ptr(experts), _ptr(workspace),
                                      nbytes, _ptr(g), _ptr(u), _stream(stream)), "xp_gateup_rows_split")


def xp_down_rows(d: xp_dims, rows: int, act, experts, workspace, out, stream=None) -> None:
    if rows > 0:
        _dev(act, torch.float32, "act", rows * d.top_k * d.inter)
        _dev(experts, torch.int64, "experts", d.n_experts * 6)
        _dev(out, torch.float32, "out", rows * d.top_k * d.hidden)
    nbytes = workspace.numel() if workspace is not None else 0
    _check(lib().xp_down_rows(ctypes.byref(d), int(rows), _ptr(act), _ptr(experts), _ptr(workspace), nbytes,
                              _ptr(out), _stream(stream)), "xp_down_rows")


def xp_combine(d: xp_dims, rows: int, out, topk_w, y, stream=None) -> None:
    if rows > 0:
        _dev(out, torch.float32, "out", rows * d.top_k * d.hidden)
        _dev(topk_w, torch.float32, "topk_w", rows * d.top_k)
        _dev(y, torch.float32, "y", rows * d.hidden)
    _check(lib().xp_combine(ctypes.byref(d), int(rows), _ptr(out), _ptr(topk_w), _ptr(y), _stream(stream)),
           "xp_combine")


def xp_route_gateup(d: xp_dims, rows: int, logits, x, experts, topk_id, topk_w, workspace, act,
                    stream=None) -> None:
    if rows > 0:
        _dev(logits, torch.float32, "logits", rows * d.n_experts)
        _dev_bf16(x, "x", rows * d.hidden)
        _dev(experts, torch.int64, "experts", d.n_experts * 6)
        _dev(topk_id, torch.int32, "topk_id", rows * d.top_k)
        _dev(topk_w, torch.float32, "topk_w", rows * d.top_k)
        _dev(workspace, torch.uint8, "workspace")
        _dev(act, torch.float32, "act", rows * d.top_k * d.inter)
    nbytes = workspace.numel() if workspace is not None else 0
    _check(lib().xp_route_gateup(ctypes.byref(d), int(rows), _ptr(logits), _ptr(x), _ptr(experts), _ptr(topk_id),
                                 _ptr(topk_w), _ptr(workspace), nbytes, _ptr(act), _stream(stream)),
           "xp_route_gateup")


def xp_down_combine(d: xp_dims, rows: int, act, experts, topk_w, workspace, out, y, stream=None) -> None:
    if rows > 0:
        _dev(act, torch.float32, "act", rows * d.top_k * d.inter)
        _dev(experts, torch.int64, "experts", d.n_experts * 6)
        _dev(topk_w, torch.float32, "topk_w", rows * d.top_k)
        _dev(workspace, torch.uint8, "workspace")
        _dev(out, torch.float32, "out", rows * d.top_k * d.hidden)
        _dev(y, torch.float32, "y", rows * d.hidden)
    nbytes = workspace.numel() if workspace is not None else 0
    _check(lib().xp_down_combine(ctypes.byref(d), int(rows), _ptr(act), _ptr(experts), _ptr(topk_w),
                                 _ptr(workspace), nbytes, _ptr(out), _ptr(y), _stream(stream)), "xp_down_combine")


def xp_decode_static(d: xp_dims, rows: int, logits, x, experts, topk_id, topk_w, act, out, y,
                     stream=None) -> None:
    """xp_route_gateup + xp_down_combine with the plan in the library's own device array (no workspace)."""
    if rows > 0:
        _dev(logits, torch.float32, "logits", rows * d.n_experts)
        _dev_bf16(x, "x", rows * d.hidden)
        _dev(experts, torch.int64, "experts", d.n_experts * 6)
        _dev(topk_id, torch.int32, "topk_id", rows * d.top_k)
        _dev(topk_w, torch.float32, "topk_w", rows * d.top_k)
        _dev(act, torch.float32, "act", rows * d.top_k * d.inter)
        _dev(out, torch.float32, "out", rows * d.top_k * d.hidden)
        _dev(y, torch.float32, "y", rows * d.hidden)
    _check(lib().xp_decode_static(ctypes.byref(d), int(rows), _ptr(logits), _ptr(x), _ptr(experts),
                                  _ptr(topk_id), _ptr(topk_w), _ptr(act), _ptr(out), _ptr(y), _stream(stream)),
           "xp_decode_static")


def xp_prefill_gateup(d: xp_dims, rows: int, x, experts, workspace, act, stream=None) -> None:
    if rows > 0:
        _dev_bf16(x, "x", rows * d.hidden)
        _dev(experts, torch.int64, "experts", d.n_experts * 6)
        _dev(act, torch.float32, "act", rows * d.top_k * d.inter)
    nbytes = workspace.numel() if workspace is not None else 0
    _check(lib().xp_prefill_gateup(ctypes.byref(d), int(rows), _ptr(x), _ptr(experts), _ptr(workspace), nbytes,
                                   _ptr(act), _stream(stream)), "xp_prefill_gateup")


def xp_prefill_down(d: xp_dims, rows: int, act, experts, workspace, out, stream=None) -> None:
    if rows > 0:
        _dev(act, torch.float32, "act", rows * d.top_k * d.inter)
        _dev(experts, torch.int64, "experts", d.n_experts * 6)
        _dev(out, torch.float32, "out", rows * d.top_k * d.hidden)
    nbytes = workspace.numel() if workspace is not None else 0
    _check(lib().xp_prefill_down(ctypes.byref(d), int(rows), _ptr(act), _ptr(experts), _ptr(workspace), nbytes,
                                 _ptr(out), _stream(stream)), "xp_prefill_down")


def xp_gateup_rows_coded(d: xp_dims, rows: int, x_codes, x_scales, experts, workspace, act, stream=None) -> None:
    """Gate/up over E4M3FN-coded activations with one E8M0 scale per 32 (see xp.h)."""
    if rows > 0:
        _dev(x_codes, torch.uint8, "x_codes", rows * d.hidden)
        _dev(x_scales, torch.uint8, "x_scales", rows * (d.hidden // 32))
        _dev(experts, torch.int64, "experts", d.n_experts * 6)
        _dev(act, torch.float32, "act", rows * d.top_k * d.inter)
    nbytes = workspace.numel() if workspace is not None else 0
    _check(lib().xp_gateup_rows_coded(ctypes.byref(d), int(rows), _ptr(x_codes), _ptr(x_scales), _ptr(experts),
                                      _ptr(workspace), nbytes, _ptr(act), _stream(stream)), "xp_gateup_rows_coded")


def _dev_u16(t: torch.Tensor, name: str, numel: int) -> None:
    """bf16 storage: 16-bit patterns (int16/uint16) or a bfloat16 tensor."""
    if not isinstance(t, torch.Tensor) or t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError("%s must hold bf16 (bfloat16, or int16/uint16 bit patterns)" % name)
    _dev(t, t.dtype, name, numel)


def xp_gateup_rows_act16(d: xp_dims, rows: int, x, experts, workspace, act16, stream=None) -> None:
    if rows > 0:
        _dev_bf16(x, "x", rows * d.hidden)
        _dev(experts, torch.int64, "experts", d.n_experts * 6)
        _dev_u16(act16, "act16", rows * d.top_k * d.inter)
    nbytes = workspace.numel() if workspace is not None else 0
    _check(lib().xp_gateup_rows_act16(ctypes.byref(d), int(rows), _ptr(x), _ptr(experts), _ptr(workspace),
                                      nbytes, _ptr(act16), _stream(stream)), "xp_gateup_rows_act16")


def xp_down_rows_act16(d: xp_dims, rows: int, act16, experts, workspace, out, stream=None) -> None:
    if rows > 0:
        _dev_u16(act16, "act16", rows * d.top_k * d.inter)
        _dev(experts, torch.int64, "experts", d.n_experts * 6)
        _dev(out, torch.float32, "out", rows * d.top_k * d.hidden)
    nbytes = workspace.numel() if workspace is not None else 0
    _check(lib().xp_down_rows_act16(ctypes.byref(d), int(rows), _ptr(act16), _ptr(experts), _ptr(workspace),
                                    nbytes, _ptr(out), _stream(stream)), "xp_down_rows_act16")


def xp_combine_y16(d: xp_dims, rows: int, out, topk_w, y16, stream=None) -> None:
    if rows > 0:
        _dev(out, torch.float32, "out", rows * d.top_k * d.hidden)
        _dev(topk_w, torch.float32, "topk_w", rows * d.top_k)
        _dev_u16(y16, "y16", rows * d.hidden)
    _check(lib().xp_combine_y16(ctypes.byref(d), int(rows), _ptr(out), _ptr(topk_w), _ptr(y16),
                                _stream(stream)), "xp_combine_y16")


def xp_fp8_packed_bytes(n: int, k: int) -> int:
    return int(lib().xp_fp8_packed_bytes(int(n), int(k)))


def xp_fp8_pack(w, packed, stream=None) -> None:
    """Repack a [n][k] E4M3FN byte matrix (uint8 device tensor) into ``packed``."""
    n, k = (w.shape[0], w.shape[1]) if isinstance(w, torch.Tensor) and w.dim() == 2 else (0, 0)
    _dev(w, torch.uint8, "w")
    _dev(packed, torch.uint8, "packed", n * k)
    _check(lib().xp_fp8_pack(int(n), int(k), _ptr(w), _ptr(packed), _stream(stream)), "xp_fp8_pack")


def xp_fp8_rows(rows: int, n: int, k: int, x, packed, scales, y, slices: int = 0, stream=None) -> None:
    """y[rows][n] fp32 = x[rows][k] (bf16) times the packed FP8 matrix (see xp_fp8_rows in xp.h)."""
    if rows > 0:
        _dev_bf16(x, "x", rows * k)
        _dev(packed, torch.uint8, "packed", n * k)
        _dev(scales, torch.float32, "scales", ((n + 127) // 128) * (k // 128))
        _dev(y, torch.float32, "y", rows * n)
    _check(lib().xp_fp8_rows(int(rows), int(n), int(k), _ptr(x), _ptr(packed), _ptr(scales), _ptr(y),
                             int(slices), _stream(stream)), "xp_fp8_rows")


def xp_fp8_rows_f32(rows: int, n: int, k: int, x, packed, scales, y, slices: int = 0, stream=None) -> None:
    """y[rows][n] fp32 = x[rows][k] (fp32) times the packed FP8 matrix (see xp_fp8_rows_f32 in xp.h)."""
    if rows > 0:
        _dev(x, torch.float32, "x", rows * k)
        _dev(packed, torch.uint8, "packed", n * k)
        _dev(scales, torch.float32, "scales", ((n + 127) // 128) * (k // 128))
        _dev(y, torch.float32, "y", rows * n)
    _check(lib().xp_fp8_rows_f32(int(rows), int(n), int(k), _ptr(x), _ptr(packed), _ptr(scales), _ptr(y),
                                 int(slices), _stream(stream)), "xp_fp8_rows_f32")


def xp_stream_weights(d: xp_dims, experts, ids, sink, parts: int = 7, stream=None) -> None:
    """Bandwidth probe: read the packed weights of the matrices in ``parts`` (bit 0
    gate, 1 up, 2 down) of the experts in ``ids`` once (see xp.h)."""
    n = 0 if ids is None else ids.numel()
    if n > 0:
        _dev(experts, torch.int64, "experts", d.n_experts * 6)
        _dev(ids, torch.int32, "ids")
        _dev(sink, torch.int32 if sink.dtype == torch.int32 else torch.uint32, "sink", 1)
    _check(lib().xp_stream_weights(ctypes.byref(d), _ptr(experts), _ptr(ids), int(n), int(parts), _ptr(sink),
                                   _stream(stream)), "xp_stream_weights")


def xp_fp8_rows_multi(rows: int, k: int, x, mats, slices: int = 0, stream=None) -> None:
    """One launch for several FP8 projections of the same rows: mats is a list of
    (packed, scales, y) device tensors, y [rows][n] (see xp_fp8_rows_multi in xp.h)."""
    arr = (xp_fp8_matrix * max(len(mats), 1))()
    for i, (packed, scales, y) in enumerate(mats):
        n = packed.numel() // k if k > 0 else 0
        if rows > 0:
            _dev(packed, torch.uint8, "packed", n * k)
            _dev(scales, torch.float32, "scales", ((n + 127) // 128) * (k // 128))
            _dev(y, torch.float32, "y", rows * n)
        arr[i] = xp_fp8_matrix(n, _ptr(packed), _ptr(scales), _ptr(y))
    if rows > 0:
        _dev_bf16(x, "x", rows * k)
    _check(lib().xp_fp8_rows_multi(int(rows), int(k), _ptr(x), arr, len(mats), int(slices), _stream(stream)),
           "xp_fp8_rows_multi")


# -------------------------------------------------------------- conveniences
MATRICES = ("gate", "up", "down")


def pack_expert(plain: dict, stream=None) -> dict:
    """Pack one expert's plain-layout device tensors (gate/up/down codes and scales)."""
    out = {}
    for m in MATRICES:
        c, s = plain[m + "_codes"], plain[m + "_scales"]
        pc = torch.empty_like(c)
        ps = torch.empty_like(s)
        xp_pack_matrix(c, s, pc, ps, stream)
        out[m + "_codes"], out[m + "_scales"] = pc, ps
    return out


def expert_table(n_experts: int, packed: dict, device="cuda") -> torch.Tensor:
    """Device array of xp_expert structs ([E][6] int64 pointers); absent experts are NULL."""
    tab = torch.zeros((n_experts, 6), dtype=torch.int64)
    for e, p in packed.items():
        tab[e] = torch.tensor([p["gate_codes"].data_ptr(), p["gate_scales"].data_ptr(),
                               p["up_codes"].data_ptr(), p["up_scales"].data_ptr(),
                               p["down_codes"].data_ptr(), p["down_scales"].data_ptr()], dtype=torch.int64)
    return tab.to(device)
