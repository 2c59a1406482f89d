"""Plain CPU oracle for the fp4 routed-expert decode path.

TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the bench's
``cpu_baseline`` leg are the only callers. The product package never imports
this module, and this module imports nothing from the product package.

The arithmetic lives in ``oracle.c`` (float64 definition, plus an fp32 replay
of the per-row chains); this file only builds that C file with gcc and
marshals numpy arrays to it. Function-level citations are in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_HDR = os.path.join(_HERE, "oracle.h")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (no fast-math, no contraction) into liboracle.so."""
    stale = (not os.path.exists(_LIB)) or any(
        os.path.getmtime(p) > os.path.getmtime(_LIB) for p in (_SRC, _HDR))
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-fopenmp", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        i32, f64, u = ctypes.c_int, ctypes.c_double, ctypes.c_uint
        P = ctypes.c_void_p
        L.or_e2m1.argtypes = [u]
        L.or_e2m1.restype = f64
        L.or_e4m3fn.argtypes = [u]
        L.or_e4m3fn.restype = f64
        L.or_bf16.argtypes = [ctypes.c_uint16]
        L.or_bf16.restype = f64
        L.or_e8m0.argtypes = [u]
        L.or_e8m0.restype = f64
        L.or_dequant_coded.argtypes = [i32, P, P, P]
        L.or_dequant_coded.restype = None
        L.or_layer_coded.argtypes = [i32] * 5 + [P] * 14
        L.or_layer_coded.restype = i32
        L.or_round_bf16.argtypes = [f64]
        L.or_round_bf16.restype = f64
        L.or_route.argtypes = [i32, i32, i32, P, P, P]
        L.or_route.restype = None
        L.or_fp8_proj.argtypes = [i32, i32, i32, P, P, P, P]
        L.or_fp8_proj.restype = None
        L.or_fp8_proj_f32.argtypes = [i32, i32, i32, P, P, P, P]
        L.or_fp8_proj_f32.restype = None
        L.or_bucket.argtypes = [i32, i32, i32, P, P, P, P]
        L.or_bucket.restype = None
        L.or_passes.argtypes = [i32, P, i32, P, P, i32]
        L.or_passes.restype = i32
        L.or_plan.argtypes = [i32, P, P, P, i32, P, i32]
        L.or_plan.restype = i32
        L.or_matvec.argtypes = [i32, i32, P, P, P, P]
        L.or_matvec.restype = None
        L.or_swiglu.argtypes = [i32, P, P, P]
        L.or_swiglu.restype = None
        L.or_combine.argtypes = [i32, i32, P, P, P]
        L.or_combine.restype = None
        L.or_layer.argtypes = [i32] * 5 + [P] * 13 + [i32]
        L.or_layer.restype = i32
        L.or_chain32.argtypes = [i32, i32, P, P, P, P]
        L.or_chain32.restype = None
        L.or_combine32.argtypes = [i32, i32, P, P, P]
        L.or_combine32.restype = None
        L.or_omp_threads.argtypes = []
        L.or_omp_threads.restype = i32
        L.or_set_threads.argtypes = [i32]
        L.or_set_threads.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ codecs
def e2m1(code: int) -> float:
    return lib().or_e2m1(int(code))


def e4m3fn(byte: int) -> float:
    return lib().or_e4m3fn(int(byte))


def bf16(bits: int) -> float:
    return lib().or_bf16(int(bits))


def e8m0(byte: int) -> float:
    return lib().or_e8m0(int(byte))


def dequant_coded(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 activations from E4M3FN codes [..][H] and E8M0 scales [..][H/32] (one per 32)."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    H = codes.shape[-1]
    rows = codes.reshape(-1, H)
    sc = scales.reshape(-1, H // 32)
    assert sc.shape[0] == rows.shape[0]
    out = np.zeros(rows.shape, dtype=np.float64)
    for r in range(rows.shape[0]):
        lib().or_dequant_coded(H, _p(rows[r]), _p(sc[r]), _p(out[r]))
    return out.reshape(codes.shape)


def decode_matrix(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 W[N][K] from the plain layout (tables built from the oracle's codecs)."""
    t4 = np.array([e2m1(c) for c in range(16)], dtype=np.float64)
    t8 = np.array([e4m3fn(b) for b in range(256)], dtype=np.float64)
    codes = np.asarray(codes, dtype=np.uint8)
    N, half = codes.shape
    K = half * 2
    w = np.empty((N, K), dtype=np.float64)
    w[:, 0::2] = t4[codes & 15]
    w[:, 1::2] = t4[codes >> 4]
    s = t8[np.asarray(scales, dtype=np.uint8)]
    return w * np.repeat(s, 32, axis=1)


# ----------------------------------------------------------------- routing
def route(logits: np.ndarray, k: int):
    logits = _c(logits, np.float32)
    R, E = logits.shape
    ids = np.zeros((R, k), dtype=np.int32)
    w = np.zeros((R, k), dtype=np.float64)
    lib().or_route(R, E, k, _p(logits), _p(ids), _p(w))
    return ids, w


def bucket(topk_id: np.ndarray, E: int):
    topk_id = _c(topk_id, np.int32)
    R, k = topk_id.shape
    count = np.zeros(E, dtype=np.int32)
    offset = np.zeros(E + 1, dtype=np.int32)
    entry = np.zeros(R * k, dtype=np.int32)
    lib().or_bucket(R, E, k, _p(topk_id), _p(count), _p(offset), _p(entry))
    return count, offset, entry


def passes(n: int, tiers):
    t = _c(list(tiers), np.int32)
    cap = max(int(n), 1)               # at most one pass per row
    size = np.zeros(cap, dtype=np.int32)
    real = np.zeros(cap, dtype=np.int32)
    m = lib().or_passes(int(n), _p(t), len(t), _p(size), _p(real), cap)
    return [(int(size[i]), int(real[i])) for i in range(m)]


def plan(count: np.ndarray, offset: np.ndarray, tiers):
    count = _c(count, np.int32)
    offset = _c(offset, np.int32)
    t = _c(list(tiers), np.int32)
    cap = int(count.sum()) + 1
    out = np.zeros((cap, 4), dtype=np.int32)
    m = lib().or_plan(len(count), _p(count), _p(offset), _p(t), len(t), _p(out), cap)
    assert m <= cap
    return out[:m].copy()


# -------------------------------------------------------- float64 layer math
def matvec(codes, scales, x) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    x = _c(x, np.float64)
    N = codes.shape[0]
    K = codes.shape[1] * 2
    assert scales.shape == (N, K // 32) and x.shape == (K,)
    y = np.zeros(N, dtype=np.float64)
    lib().or_matvec(N, K, _p(codes), _p(scales), _p(x), _p(y))
    return y


def swiglu(g, u) -> np.ndarray:
    g = _c(g, np.float64)
    u = _c(u, np.float64)
    a = np.zeros_like(g)
    lib().or_swiglu(g.size, _p(g), _p(u), _p(a))
    return a


def combine(w, out) -> np.ndarray:
    w = _c(w, np.float64)
    out = _c(out, np.float64)
    k, H = out.shape
    y = np.zeros(H, dtype=np.float64)
    lib().or_combine(k, H, _p(w), _p(out), _p(y))
    return y


def round_bf16(v) -> np.ndarray:
    """Each float64 value rounded once to the nearest bf16 value (ties to even)."""
    a = np.asarray(v, dtype=np.float64)
    f = lib().or_round_bf16
    return np.array([f(float(t)) for t in a.reshape(-1)], dtype=np.float64).reshape(a.shape)


def bf16_to_f64(x_bits: np.ndarray) -> np.ndarray:
    b = _c(x_bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def layer(x_bf16: np.ndarray, logits: np.ndarray, experts: dict, H: int, I: int, E: int, k: int,
          act_bf16: bool = False):
    """float64 layer over R rows.

    ``experts`` maps expert id -> dict with the six plain-layout arrays
    (gate_codes, gate_scales, up_codes, up_scales, down_codes, down_scales).
    act_bf16: act is rounded to bf16 (round_bf16) before down, as in the
    bf16-storage variant; the returned act holds the rounded values.
    Returns dict(topk_id, topk_w, act[R][k][I], out[R][k][H], y[R][H], threads).
    """
    x_bf16 = _c(x_bf16, np.uint16)
    logits = _c(logits, np.float32)
    R = x_bf16.shape[0]
    assert x_bf16.shape == (R, H) and logits.shape == (R, E)
    names = ("gate_codes", "gate_scales", "up_codes", "up_scales", "down_codes", "down_scales")
    keep = []
    tables = []
    for nm in names:
        arr = (ctypes.c_void_p * E)()
        for e, ex in experts.items():
            a = _c(ex[nm], np.uint8)
            keep.append(a)
            arr[e] = a.ctypes.data
        tables.append(arr)
    topk_id = np.zeros((R, k), dtype=np.int32)
    topk_w = np.zeros((R, k), dtype=np.float64)
    act = np.zeros((R, k, I), dtype=np.float64)
    out = np.zeros((R, k, H), dtype=np.float64)
    y = np.zeros((R, H), dtype=np.float64)
    # every selected expert must be present
    ids_chk, _ = route(logits, k)
    missing = set(int(e) for e in np.unique(ids_chk)) - set(experts)
    if missing:
        raise KeyError("oracle.layer: experts %s are routed but not given" % sorted(missing))
    threads = lib().or_layer(H, I, E, k, R, _p(x_bf16), _p(logits), *tables,
                             _p(topk_id), _p(topk_w), _p(act), _p(out), _p(y), 1 if act_bf16 else 0)
    return dict(topk_id=topk_id, topk_w=topk_w, act=act, out=out, y=y, threads=threads)


def layer_coded(x_codes: np.ndarray, x_scales: np.ndarray, logits: np.ndarray, experts: dict, H: int, I: int,
                E: int, k: int):
    """float64 layer over R rows whose activations are coded: x_codes [R][H] E4M3FN,
    x_scales [R][H/32] E8M0 (x = e4m3fn(code) * 2^(scale - 127)); otherwise as layer()."""
    x_codes = _c(x_codes, np.uint8)
    x_scales = _c(x_scales, np.uint8)
    logits = _c(logits, np.float32)
    R = x_codes.shape[0]
    assert x_codes.shape == (R, H) and x_scales.shape == (R, H // 32) and logits.shape == (R, E)
    names = ("gate_codes", "gate_scales", "up_codes", "up_scales", "down_codes", "down_scales")
    keep, tables = [], []
    for nm in names:
        arr = (ctypes.c_void_p * E)()
        for e, ex in experts.items():
            a = _c(ex[nm], np.uint8)
            keep.append(a)
            arr[e] = a.ctypes.data
        tables.append(arr)
    ids_chk, _ = route(logits, k)
    missing = set(int(e) for e in np.unique(ids_chk)) - set(experts)
    if missing:
        raise KeyError("oracle.layer_coded: experts %s are routed but not given" % sorted(missing))
    topk_id = np.zeros((R, k), dtype=np.int32)
    topk_w = np.zeros((R, k), dtype=np.float64)
    act = np.zeros((R, k, I), dtype=np.float64)
    out = np.zeros((R, k, H), dtype=np.float64)
    y = np.zeros((R, H), dtype=np.float64)
    threads = lib().or_layer_coded(H, I, E, k, R, _p(x_codes), _p(x_scales), _p(logits), *tables,
                                   _p(topk_id), _p(topk_w), _p(act), _p(out), _p(y))
    return dict(topk_id=topk_id, topk_w=topk_w, act=act, out=out, y=y, threads=threads)


# ------------------------------------------------------ fp32 chain replay
def chain32(codes, scales, x_f32) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    x = _c(x_f32, np.float32)
    N = codes.shape[0]
    K = codes.shape[1] * 2
    assert x.shape == (K,)
    y = np.zeros(N, dtype=np.float32)
    lib().or_chain32(N, K, _p(codes), _p(scales), _p(x), _p(y))
    return y


def combine32(w_f32, out_f32) -> np.ndarray:
    w = _c(w_f32, np.float32)
    out = _c(out_f32, np.float32)
    k, H = out.shape
    y = np.zeros(H, dtype=np.float32)
    lib().or_combine32(k, H, _p(w), _p(out), _p(y))
    return y


def omp_threads() -> int:
    return lib().or_omp_threads()


def set_threads(n: int) -> None:
    """Threads the oracle's parallel loops use from now on (timing only)."""
    lib().or_set_threads(int(n))


def fp8_proj(x_bits: np.ndarray, w: np.ndarray, s: np.ndarray) -> np.ndarray:
    """float64 y [R][N] of the dense FP8 projection (see or_fp8_proj)."""
    x_bits = _c(x_bits, np.uint16)
    w = _c(w, np.uint8)
    s = _c(s, np.float32)
    R, K = x_bits.shape
    N = w.shape[0]
    assert w.shape == (N, K) and K % 128 == 0
    assert s.shape == ((N + 127) // 128, K // 128)
    y = np.zeros((R, N), dtype=np.float64)
    lib().or_fp8_proj(R, N, K, _p(x_bits), _p(w), _p(s), _p(y))
    return y


def fp8_proj_f32(x: np.ndarray, w: np.ndarray, s: np.ndarray) -> np.ndarray:
    """float64 y [R][N] of the dense FP8 projection of fp32 rows (see or_fp8_proj_f32)."""
    x = _c(x, np.float32)
    w = _c(w, np.uint8)
    s = _c(s, np.float32)
    R, K = x.shape
    N = w.shape[0]
    assert w.shape == (N, K) and K % 128 == 0
    assert s.shape == ((N + 127) // 128, K // 128)
    y = np.zeros((R, N), dtype=np.float64)
    lib().or_fp8_proj_f32(R, N, K, _p(x), _p(w), _p(s), _p(y))
    return y
