"""Build the native libraries in-tree.

- ``fp4_routed_expert_xp_amd/libxp.so``: the product (HIP kernels for gfx950 + the C ABI).
- ``synth/libxpsynth.so``: device twin of the seeded weight-byte generator (test/bench input).
- ``oracle/liboracle.so``: the CPU oracle (gcc), built by ``oracle.build``.

Run ``python -m fp4_routed_expert_xp_amd.build``.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "fp4_routed_expert_xp_amd")
CSRC = os.path.join(PKG, "csrc")
LIBXP = os.path.join(PKG, "libxp.so")
SYNTH_SRC = os.path.join(ROOT, "synth", "synth.hip")
LIBSYNTH = os.path.join(ROOT, "synth", "libxpsynth.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fvisibility=hidden",
    # never let the compiler form packed fp32 math
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc(out: str, srcs: list, extra: list | None = None) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + HIP_FLAGS + (extra or []) + ["-o", tmp] + srcs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed for %s" % out)
    os.replace(tmp, out)


def build_libxp() -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    _hipcc(LIBXP, srcs, ["-I" + os.path.join(ROOT, "include"), "-I" + CSRC])
    return LIBXP


def build_synth() -> str:
    _hipcc(LIBSYNTH, [SYNTH_SRC])
    return LIBSYNTH


def build_oracle() -> str:
    sys.path.insert(0, ROOT) if ROOT not in sys.path else None
    import oracle
    return oracle.build(force=True)


def build_all() -> None:
    build_libxp()
    build_synth()
    build_oracle()


if __name__ == "__main__":
    build_all()
    print("built", LIBXP, LIBSYNTH)
