"""Seeded synthetic inputs for the fp4 routed-expert decode path.

This module only draws inputs (fp4 codes, E4M3 scale bytes, bf16 activations,
fp32 router logits, planted NaN/Inf); it holds none of the method's arithmetic
and imports neither the product package nor the oracle. Both sides' inputs come
from here. A device twin of the weight-byte streams (``synth.hip``, integer
SplitMix64 only) writes the same bytes straight into GPU memory for workloads
too large to draw on the host.

Every value is a pure function of (seed, layer, tensor id, expert, element
index): element i of a stream is the (i+1)-th output of SplitMix64 (Steele,
Lea and Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014)
started from the stream key. Weight-code byte b is byte (b mod 8) of output
b // 8 (little-endian); a scale byte comes from the high 32 bits of its own
output; a normal value is Box-Muller on the two 32-bit halves of one output.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

MASK = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB

# stream (tensor) ids
GATE_CODES, GATE_SCALES, UP_CODES, UP_SCALES, DOWN_CODES, DOWN_SCALES = 1, 2, 3, 4, 5, 6
X, LOGITS, BIAS, PLANT = 7, 8, 9, 10
FP8_WEIGHTS, FP8_SCALES = 11, 12
X_CODES, X_SCALES = 13, 14
MATRICES = {
    "gate": (GATE_CODES, GATE_SCALES),
    "up": (UP_CODES, UP_SCALES),
    "down": (DOWN_CODES, DOWN_SCALES),
}


def _mix(z: int) -> int:
    z &= MASK
    z = ((z ^ (z >> 30)) * M1) & MASK
    z = ((z ^ (z >> 27)) * M2) & MASK
    return z ^ (z >> 31)


def _sm(x: int) -> int:
    """First SplitMix64 output from state x."""
    return _mix((x + GOLDEN) & MASK)


def stream_key(seed: int, layer: int, tensor: int, expert: int = 0) -> int:
    k = _sm(seed & MASK)
    k = _sm(k ^ (layer & MASK))
    k = _sm(k ^ (tensor & MASK))
    return _sm(k ^ (expert & MASK))


def stream(key: int, start: int, count: int) -> np.ndarray:
    """Outputs start .. start+count-1 of SplitMix64 from state ``key`` (uint64)."""
    i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    z = np.uint64(key) + i * np.uint64(GOLDEN)
    z = (z ^ (z >> np.uint64(30))) * np.uint64(M1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(M2)
    return z ^ (z >> np.uint64(31))


# ------------------------------------------------------------ weight bytes
def codes(seed: int, layer: int, expert: int, tensor: int, N: int, K: int) -> np.ndarray:
    """fp4 codes uniform over all 16 values, plain layout [N][K/2] uint8."""
    nbytes = N * K // 2
    assert nbytes % 8 == 0
    w = stream(stream_key(seed, layer, tensor, expert), 0, nbytes // 8)
    return w.astype("<u8").view(np.uint8).reshape(N, K // 2)


def scales(seed: int, layer: int, expert: int, tensor: int, N: int, K: int,
           emin: int, emax: int) -> np.ndarray:
    """E4M3 bytes 2^e with e uniform on {emin..emax}; plain layout [N][K/32] uint8."""
    n = np.uint64(emax - emin + 1)
    w = stream(stream_key(seed, layer, tensor, expert), 0, N * (K // 32))
    e = (((w >> np.uint64(32)) * n) >> np.uint64(32)).astype(np.int64) + emin
    return ((e + 7) << 3).astype(np.uint8).reshape(N, K // 32)


def any_scales(seed: int, layer: int, expert: int, tensor: int, N: int, K: int) -> np.ndarray:
    """E4M3FN bytes uniform over the 254 non-NaN codes (both signs, zero, subnormals,
    every mantissa; 0x7F and 0xFF skipped); plain layout [N][K/32] uint8. Drawn from
    the stream of ``tensor`` + 100, so they differ from the power-of-two scales."""
    w = stream(stream_key(seed, layer, tensor + 100, expert), 0, N * (K // 32))
    b = ((w >> np.uint64(32)) * np.uint64(254)) >> np.uint64(32)
    b = np.where(b >= np.uint64(0x7F), b + np.uint64(1), b)
    return b.astype(np.uint8).reshape(N, K // 32)


def mixed_scales(seed: int, layer: int, expert: int, tensor: int, N: int, K: int,
                 emin: int, emax: int) -> np.ndarray:
    """Scale bytes that mix both kinds by 32-group column: groups g = 0 mod 3 take
    any_scales in every row, groups g = 1 mod 3 take them in rows n = 0 mod 5, and
    the rest keep the power-of-two draw of ``scales``."""
    s = scales(seed, layer, expert, tensor, N, K, emin, emax)
    a = any_scales(seed, layer, expert, tensor, N, K)
    g = np.arange(K // 32)[None, :]
    n = np.arange(N)[:, None]
    pick = (g % 3 == 0) | ((g % 3 == 1) & (n % 5 == 0))
    return np.where(pick, a, s)


def expert_mixed(seed: int, layer: int, e: int, H: int, I: int, emin: int, emax: int) -> dict:
    """``expert`` with every matrix's scales from ``mixed_scales``."""
    out = expert(seed, layer, e, H, I, emin, emax)
    shapes = {"gate": (I, H), "up": (I, H), "down": (H, I)}
    for m, (_, ts) in MATRICES.items():
        N, K = shapes[m]
        out[m + "_scales"] = mixed_scales(seed, layer, e, ts, N, K, emin, emax)
    return out


def expert(seed: int, layer: int, e: int, H: int, I: int, emin: int, emax: int) -> dict:
    """The six plain-layout arrays of one expert: gate/up are [I][H], down is [H][I]."""
    return dict(
        gate_codes=codes(seed, layer, e, GATE_CODES, I, H),
        gate_scales=scales(seed, layer, e, GATE_SCALES, I, H, emin, emax),
        up_codes=codes(seed, layer, e, UP_CODES, I, H),
        up_scales=scales(seed, layer, e, UP_SCALES, I, H, emin, emax),
        down_codes=codes(seed, layer, e, DOWN_CODES, H, I),
        down_scales=scales(seed, layer, e, DOWN_SCALES, H, I, emin, emax),
    )


# ------------------------------------------------ dense FP8 projections
def fp8_weights(seed: int, layer: int, N: int, K: int) -> np.ndarray:
    """E4M3FN bytes [N][K], uniform over the 254 non-NaN codes (0x7F and 0xFF
    are skipped): output i of the stream gives byte i from its high 32 bits."""
    w = stream(stream_key(seed, layer, FP8_WEIGHTS), 0, N * K)
    b = ((w >> np.uint64(32)) * np.uint64(254)) >> np.uint64(32)
    b = np.where(b >= np.uint64(0x7F), b + np.uint64(1), b)
    return b.astype(np.uint8).reshape(N, K)


def fp8_scales(seed: int, layer: int, N: int, K: int, emin: int = -10, emax: int = -6) -> np.ndarray:
    """fp32 scales 2^e, e uniform on {emin..emax}, one per 128 x 128 block:
    [ceil(N/128)][K/128]."""
    nb, kb = (N + 127) // 128, K // 128
    n = np.uint64(emax - emin + 1)
    w = stream(stream_key(seed, layer, FP8_SCALES), 0, nb * kb)
    e = (((w >> np.uint64(32)) * n) >> np.uint64(32)).astype(np.int64) + emin
    return np.ldexp(np.ones(nb * kb, dtype=np.float32), e.astype(np.int32)).reshape(nb, kb)


# --------------------------------------------------------- float streams
def normals(key: int, start: int, count: int) -> np.ndarray:
    """float64 N(0,1) by Box-Muller (cosine branch) on one output per value."""
    w = stream(key, start, count)
    u1 = ((w >> np.uint64(32)).astype(np.float64) + 0.5) * (1.0 / 4294967296.0)
    u2 = (w & np.uint64(0xFFFFFFFF)).astype(np.float64) * (1.0 / 4294967296.0)
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


def f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16 bit patterns (NaN kept quiet)."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16))
    nan = np.isnan(np.asarray(f, dtype=np.float32))
    r = np.where(nan, (u >> np.uint64(16)) | np.uint64(0x40), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def activations(seed: int, layer: int, R: int, H: int) -> np.ndarray:
    """bf16 N(0,1) activations [R][H] as uint16 bit patterns."""
    z = normals(stream_key(seed, layer, X), 0, R * H).astype(np.float32)
    return f32_to_bf16_bits(z).reshape(R, H)


def coded_activations(seed: int, layer: int, R: int, H: int, emin: int = -6, emax: int = -2):
    """Coded activations: E4M3FN codes [R][H] uniform over the 254 non-NaN bytes
    (0x7F and 0xFF skipped) and one E8M0 scale byte per 32, 127 + e with e
    uniform on {emin..emax}: [R][H/32]. Returns (codes, scales), uint8."""
    w = stream(stream_key(seed, layer, X_CODES), 0, R * H)
    b = ((w >> np.uint64(32)) * np.uint64(254)) >> np.uint64(32)
    b = np.where(b >= np.uint64(0x7F), b + np.uint64(1), b)
    n = np.uint64(emax - emin + 1)
    ws = stream(stream_key(seed, layer, X_SCALES), 0, R * (H // 32))
    e = (((ws >> np.uint64(32)) * n) >> np.uint64(32)).astype(np.int64) + emin
    return b.astype(np.uint8).reshape(R, H), (e + 127).astype(np.uint8).reshape(R, H // 32)


def logits(seed: int, layer: int, R: int, E: int, bias_sigma: float = 0.0) -> np.ndarray:
    """fp32 router logits [R][E]: N(0,1), plus a per-expert N(0, sigma^2) bias if asked."""
    z = normals(stream_key(seed, layer, LOGITS), 0, R * E).reshape(R, E)
    if bias_sigma:
        z = z + bias_sigma * normals(stream_key(seed, layer, BIAS), 0, E)[None, :]
    return z.astype(np.float32)


def plant_nan_inf(seed: int, layer: int, x_bits: np.ndarray, nan_bits: int = 0x7FE5):
    """Plant a NaN in one seeded (row, col) and +Inf in another row's seeded col.

    Returns (x_bits_copy, (nan_row, nan_col), (inf_row, inf_col)). Needs >= 2 rows.
    """
    R, H = x_bits.shape
    assert R >= 2
    w = stream(stream_key(seed, layer, PLANT), 0, 4)
    nan_row = int(w[0] % np.uint64(R))
    inf_row = (nan_row + 1 + int(w[1] % np.uint64(R - 1))) % R
    nan_col = int(w[2] % np.uint64(H))
    inf_col = int(w[3] % np.uint64(H))
    x = x_bits.copy()
    x[nan_row, nan_col] = nan_bits
    x[inf_row, inf_col] = 0x7F80
    return x, (nan_row, nan_col), (inf_row, inf_col)


# --------------------------------------------------------- routing shapes
def logits_same(seed: int, layer: int, R: int, E: int) -> np.ndarray:
    """Every row carries the first row's logits, so all rows pick the same experts."""
    one = logits(seed, layer, 1, E)
    return np.repeat(one, R, axis=0)


def logits_disjoint(R: int, E: int, k: int) -> np.ndarray:
    """Row r picks experts (r*k + j) mod E, j = 0..k-1, in that slot order."""
    lg = np.full((R, E), -8.0, dtype=np.float32)
    for r in range(R):
        for j in range(k):
            lg[r, (r * k + j) % E] = 8.0 - 0.5 * j
    return lg


# ----------------------------------------------------------------- configs
@dataclass(frozen=True)
class Config:
    name: str
    H: int
    I: int
    E: int
    k: int
    R: int
    emin: int
    emax: int
    seed: int          # seeds activations, logits and plants
    weight_seed: int   # seeds the layer weights
    routing: str = "random"   # random | same
    bias_sigma: float = 0.0
    plant: bool = False
    layers: int = 1
    notes: str = field(default="", compare=False)

    @property
    def expert_bytes(self) -> int:
        return 3 * self.H * self.I // 2 + 3 * self.H * self.I // 32


# One synthetic release-width model (weights seeded by 1000) is shared by the
# release-width configs; each config seeds its own activations and logits.
CONFIGS = {
    "tiny": Config("tiny", 256, 128, 8, 2, 4, -4, 2, 1001, 1001,
                   notes="hidden 256, intermediate 128, 8 experts, top-2, 4 rows"),
    "one_row": Config("one_row", 4096, 2048, 256, 8, 1, -6, 0, 1002, 1000, layers=40,
                      notes="one decode row, release widths, top-8 of 256"),
    "four_same": Config("four_same", 4096, 2048, 256, 8, 4, -6, 0, 1003, 1000,
                        routing="same", layers=40,
                        notes="4 rows on the same 8 experts, differing activations"),
    "sixteen_random": Config("sixteen_random", 4096, 2048, 256, 8, 16, -6, 0, 1004, 1000,
                             plant=True, layers=40,
                             notes="16 rows, random top-8, NaN and +Inf planted"),
    "prefill": Config("prefill", 4096, 2048, 256, 8, 4096, -6, 0, 1005, 1000,
                      bias_sigma=0.5, notes="4096-row prompt chunk, skewed routing"),
}


def layer_inputs(cfg: Config, layer: int = 0, plant: bool | None = None):
    """(x_bits [R][H] uint16, logits [R][E] float32) for one layer of a config."""
    x = activations(cfg.seed, layer, cfg.R, cfg.H)
    if cfg.routing == "same":
        lg = logits_same(cfg.seed, layer, cfg.R, cfg.E)
    else:
        lg = logits(cfg.seed, layer, cfg.R, cfg.E, cfg.bias_sigma)
    if (cfg.plant if plant is None else plant) and cfg.R >= 2:
        x, _, _ = plant_nan_inf(cfg.seed, layer, x)
    return x, lg


def layer_expert(cfg: Config, layer: int, e: int) -> dict:
    return expert(cfg.weight_seed, layer, e, cfg.H, cfg.I, cfg.emin, cfg.emax)


# ------------------------------------------------------------ device twin
_dev_lib = None


def _device_lib():
    """libxpsynth.so: the integer weight-byte streams written straight into GPU memory."""
    global _dev_lib
    if _dev_lib is None:
        import ctypes
        import os
        import torch  # noqa: F401  (bind to torch's HIP runtime before loading)
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libxpsynth.so")
        if not os.path.exists(path):
            raise RuntimeError("synth/libxpsynth.so is not built; run `python -m fp4_routed_expert_xp_amd.build`")
        L = ctypes.CDLL(path)
        u64, i64, P = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        L.xps_codes.argtypes = [u64, u64, u64, u64, i64, i64, P, P]
        L.xps_codes.restype = ctypes.c_int
        L.xps_scales.argtypes = [u64, u64, u64, u64, i64, i64, ctypes.c_int, ctypes.c_int, P, P]
        L.xps_scales.restype = ctypes.c_int
        L.xps_stream_key.argtypes = [u64, u64, u64, u64]
        L.xps_stream_key.restype = u64
        L.xps_codes_batch.argtypes = [P, ctypes.c_int, i64, i64, P, i64, P]
        L.xps_codes_batch.restype = ctypes.c_int
        L.xps_scales_batch.argtypes = [P, ctypes.c_int, i64, i64, ctypes.c_int, ctypes.c_int, P, i64, P]
        L.xps_scales_batch.restype = ctypes.c_int
        _dev_lib = L
    return _dev_lib


def device_codes(seed, layer, expert, tensor, N, K, out, stream=0):
    """Fill the uint8 device tensor ``out`` ([N][K/2]) with the same bytes as :func:`codes`."""
    assert out.dtype.itemsize == 1 and out.numel() >= N * K // 2 and out.is_contiguous()
    rc = _device_lib().xps_codes(seed, layer, expert, tensor, N, K, out.data_ptr(), stream)
    if rc != 0:
        raise RuntimeError("xps_codes failed: %d" % rc)


def device_scales(seed, layer, expert, tensor, N, K, emin, emax, out, stream=0):
    """Fill the uint8 device tensor ``out`` ([N][K/32]) with the same bytes as :func:`scales`."""
    assert out.dtype.itemsize == 1 and out.numel() >= N * (K // 32) and out.is_contiguous()
    rc = _device_lib().xps_scales(seed, layer, expert, tensor, N, K, emin, emax, out.data_ptr(), stream)
    if rc != 0:
        raise RuntimeError("xps_scales failed: %d" % rc)


def device_expert(seed, layer, e, H, I, emin, emax, device="cuda", stream=0) -> dict:
    """The six plain-layout arrays of one expert, generated on the GPU."""
    import torch
    shapes = {"gate": (I, H), "up": (I, H), "down": (H, I)}
    out = {}
    for m, (tc, ts) in MATRICES.items():
        N, K = shapes[m]
        c = torch.empty((N, K // 2), dtype=torch.uint8, device=device)
        s = torch.empty((N, K // 32), dtype=torch.uint8, device=device)
        device_codes(seed, layer, e, tc, N, K, c, stream)
        device_scales(seed, layer, e, ts, N, K, emin, emax, s, stream)
        out[m + "_codes"], out[m + "_scales"] = c, s
    return out


def device_layer_plain(seed, layer, H, I, E, emin, emax, out, stream=0) -> dict:
    """All E experts of one layer in the plain layout, written into the uint8 device
    tensor ``out`` (E * expert_bytes). Expert e's arrays sit at e * expert_bytes plus
    the offsets returned here: {name: (offset, nbytes)} in the order gate_codes,
    gate_scales, up_codes, up_scales, down_codes, down_scales."""
    import torch
    L = _device_lib()
    shapes = {"gate": (I, H), "up": (I, H), "down": (H, I)}
    offs = {}
    o = 0
    for m in ("gate", "up", "down"):
        N, K = shapes[m]
        offs[m + "_codes"] = (o, N * K // 2)
        o += N * K // 2
        offs[m + "_scales"] = (o, N * K // 32)
        o += N * K // 32
    stride = o
    assert out.numel() >= E * stride and out.dtype == torch.uint8
    base = out.data_ptr()
    for m, (tc, ts) in MATRICES.items():
        N, K = shapes[m]
        for t, name in ((tc, m + "_codes"), (ts, m + "_scales")):
            keys = torch.from_numpy(np.array([stream_key(seed, layer, t, e) for e in range(E)], dtype=np.uint64))
            keys_dev = keys.to(out.device)
            if name.endswith("codes"):
                rc = L.xps_codes_batch(keys_dev.data_ptr(), E, N, K, base + offs[name][0], stride, stream)
            else:
                rc = L.xps_scales_batch(keys_dev.data_ptr(), E, N, K, emin, emax, base + offs[name][0], stride,
                                        stream)
            if rc != 0:
                raise RuntimeError("device generator failed: %d" % rc)
    return dict(stride=stride, offsets=offs)
