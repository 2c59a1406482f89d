#!/usr/bin/env python3
"""Generate xp_prefill_asm.h: one 32-wide group of the prefill contraction's matrix work.

Run: python3 gen_prefill_asm.py > xp_prefill_asm.h   (the header is committed; the build does not run this)

Each helper runs one group (K = 32) for NS 16-row slabs of one wave's tile, reading
the activation fragments from LDS itself so that the reads of the next two slabs
are in flight while the current two slabs' matrix instructions issue:

  read slabs 0, 1;  wait
  for each pair of slabs p:
      read the fragments of pair p + 1 (into the other register set)
      the matrix instructions of pair p
      wait for pair p + 1's reads

so only the first pair's read latency is exposed per group, and the fragments take
two register sets of a pair instead of one per slab. Every read the block issues has
landed when it ends (the last pair issues no reads, the others end on their wait),
so no output register is written after the block.

gateup: fragment of slab s at x + 1024 s (16 rows x 32 bf16, the swizzled LDS tile),
        four products per slab: acc[s][c][m] += frag * b[2m + c] (c = 16-column
        tile, m = 0 gate / 1 up), i.e. b = {gate 0, gate 1, up 0, up 1}.
down:   act as bf16 hi and lo halves at hi + 1024 s and lo + 1024 s; per slab and
        16-column tile c (four: one 64-column packed tile) acc[s][c] += hi * b[c],
        then acc[s][c] += lo * b[c], in that order for each accumulator (hi
        products of both slabs of a pair first, so the two products into one
        accumulator are eight instructions apart).

Every accumulator gets exactly the products, in exactly the order, of the plain
per-slab loop this replaces, so results are bit-for-bit the same.

Hazards: a fragment register set is overwritten only by reads issued after the
matrix instructions that read it (a read's data returns long after those have
taken their A operands). The first matrix instruction of a block follows at least
three instructions (two reads and a wait), more than the two wait states a
matrix instruction needs after a VALU write of its B operand or accumulator.
The compiler does not see the matrix instructions inside the blocks, so the
callers run `drain` (20 wait states, with the accumulators as operands) before
any other instruction reads the accumulators.
"""
import sys

MFMA = "v_mfma_f32_16x16x32_bf16"


def gateup(NS: int) -> str:
    P = NS // 2
    L = []

    def rd(buf: int, p: int) -> None:
        for j in range(2):
            off = (2 * p + j) * 1024
            L.append("ds_read_b128 %%[f%d], %%[x]%s" % (2 * buf + j, " offset:%d" % off if off else ""))

    rd(0, 0)
    L.append("s_waitcnt lgkmcnt(0)")
    for p in range(P):
        if p + 1 < P:
            rd((p + 1) % 2, p + 1)
        for j in range(2):
            s, f = 2 * p + j, 2 * (p % 2) + j
            for c, m in ((0, 0), (1, 0), (0, 1), (1, 1)):
                L.append("%s %%[c%d_%d_%d], %%[f%d], %%[b%d], %%[c%d_%d_%d]" % (MFMA, s, c, m, f, 2 * m + c, s, c, m))
        if p + 1 < P:
            L.append("s_waitcnt lgkmcnt(0)")
    outs = ['[c%d_%d_%d] "+v"(c[%d][%d][%d])' % (s, cc, m, s, cc, m)
            for s in range(NS) for cc in range(2) for m in range(2)]
    outs += ['[f%d] "=&v"(f[%d])' % (i, i) for i in range(4)]
    ins = ['[b%d] "v"(b[%d])' % (i, i) for i in range(4)] + ['[x] "v"(x)']
    return ("    static __device__ __forceinline__ void gateup(f32x4 (&c)[%d][2][2], const bf16x8 (&b)[4], uint32_t x) {\n"
            "        u32x4v f[4];\n"
            "        asm volatile(\"%s\"\n            : %s\n            : %s\n            : \"memory\");\n    }\n"
            % (NS, "\\n\\t".join(L), ", ".join(outs), ", ".join(ins)))


def down(NS: int, C: int = 4) -> str:
    P = NS // 2
    L = []

    def rd(buf: int, p: int) -> None:
        for j in range(2):
            off = (2 * p + j) * 1024
            o = " offset:%d" % off if off else ""
            L.append("ds_read_b128 %%[f%d], %%[hi]%s" % (4 * buf + 2 * j, o))
            L.append("ds_read_b128 %%[f%d], %%[lo]%s" % (4 * buf + 2 * j + 1, o))

    rd(0, 0)
    L.append("s_waitcnt lgkmcnt(0)")
    for p in range(P):
        if p + 1 < P:
            rd((p + 1) % 2, p + 1)
        base = 4 * (p % 2)
        for half in (0, 1):  # hi products of both slabs, then lo
            for j in range(2):
                s = 2 * p + j
                for c in range(C):
                    L.append("%s %%[c%d_%d], %%[f%d], %%[b%d], %%[c%d_%d]" % (MFMA, s, c, base + 2 * j + half, c, s, c))
        if p + 1 < P:
            L.append("s_waitcnt lgkmcnt(0)")
    outs = ['[c%d_%d] "+v"(c[%d][%d])' % (s, cc, s, cc) for s in range(NS) for cc in range(C)]
    outs += ['[f%d] "=&v"(f[%d])' % (i, i) for i in range(8)]
    ins = ['[b%d] "v"(b[%d])' % (i, i) for i in range(C)] + ['[hi] "v"(hi)', '[lo] "v"(lo)']
    return ("    static __device__ __forceinline__ void down(f32x4 (&c)[%d][%d], const bf16x8 (&b)[%d], uint32_t hi, "
            "uint32_t lo) {\n"
            "        u32x4v f[8];\n"
            "        asm volatile(\"%s\"\n            : %s\n            : %s\n            : \"memory\");\n    }\n"
            % (NS, C, C, "\\n\\t".join(L), ", ".join(outs), ", ".join(ins)))


def drain(NS: int, dims: str, idx: list) -> str:
    outs = ['"+v"(c%s)' % i for i in idx]
    return ("    static __device__ __forceinline__ void drain(f32x4 (&c)[%d]%s) {\n"
            "        asm volatile(\"s_nop 7\\n\\ts_nop 7\\n\\ts_nop 3\" : %s);\n    }\n"
            % (NS, dims, ", ".join(outs)))


def main() -> None:
    out = [
        "// xp_prefill_asm.h -- generated by gen_prefill_asm.py; do not edit.",
        "// One 32-wide group of the prefill contraction's matrix work per call, with the",
        "// activation fragment reads pipelined two slabs ahead (see the generator's notes).",
        "// Included by xp_prefill.hip after its f32x4, bf16x8 and u32x4v vector types.",
        "#pragma once",
        "",
        "namespace xp {",
        "",
        "template <int NS> struct PfGroup;",
        "",
    ]
    for NS in (2, 4, 6, 8):
        out.append("template <> struct PfGroup<%d> {" % NS)
        out.append(gateup(NS))
        out.append(down(NS))
        out.append(drain(NS, "[2][2]", ["[%d][%d][%d]" % (s, c, m) for s in range(NS) for c in range(2) for m in range(2)]))
        out.append(drain(NS, "[4]", ["[%d][%d]" % (s, c) for s in range(NS) for c in range(4)]))
        out.append("};")
        out.append("")
    out.append("}  // namespace xp")
    sys.stdout.write("\n".join(out) + "\n")


if __name__ == "__main__":
    main()
