#!/usr/bin/env python3
"""Generate xp_prefill_asm.h: one 32-wide group of the prefill contraction's matrix work.

Run: python3 gen_prefill_asm.py > xp_prefill_asm.h   (the header is committed; the build does not run this)

Each helper runs one group (K = 32) for NS 16-row slabs of one wave's tile (NS = 1..10
for gate/up, 1..8 for down; slabs go in pairs, the last alone when NS is odd), reading
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

gate/up: fragment of slab s at x + 1024 s (16 rows x 32 bf16, the swizzled LDS tile),
        four products per slab: acc[s][c][m] += frag * b[2m + c] (c = 16-column
        tile, m = 0 gate / 1 up), i.e. b = {gate 0, gate 1, up 0, up 1}. A group
        is two asm statements: gateup_dec reads the four code words and the first
        two fragments and, once the words are in, decodes them into n with their
        power-of-two scales (frags only issues the fragment reads, for groups the
        caller decodes itself); gateup_tail waits for the fragments and runs the
        matrix instructions with the reads of the later pairs.
down:   act as bf16 hi and lo halves at hi + 1024 s and lo + 1024 s; per slab and
        16-column tile c (four: one 64-column packed tile) acc[s][c] += hi * b[c],
        then acc[s][c] += lo * b[c], in that order for each accumulator (hi
        products of both slabs of a pair first, so the two products into one
        accumulator are eight instructions apart). down_dec also decodes the next
        group's weights into n while the first pair's reads are in flight.

The converts apply only the exponent of their fp32 scale operand, which is exact
for power-of-two scales; for a group with another scale the caller decodes the
words itself (gate/up before the body, down again after it). Every accumulator
gets exactly the products, in exactly the order, of a plain per-slab loop.

Hazards: a fragment register set is overwritten only by reads issued after the
matrix instructions that read it (a read's data returns long after those have
taken their A operands). The first matrix instruction of down_dec follows at least
three instructions (reads and a wait), and gateup_tail opens with two wait states
and a wait: more than the two wait states a matrix instruction needs after a VALU
write of its B operand or accumulator. The fragment registers gateup_dec and
frags leave in flight must not be touched before gateup_tail; the assembly is
checked for that.
The compiler does not see the matrix instructions inside the blocks, so the
callers run `drain` (20 wait states, with the accumulators as operands) before
any other instruction reads the accumulators.
"""
import sys

MFMA = "v_mfma_f32_16x16x32_bf16"


def gateup_dec() -> str:
    """First half of a gate/up group whose weights are decoded in the group body:
    the four code words (gate 0, gate 1, up 0, up 1 of the wave's columns) and
    the first two activation fragments are read, and once the words are in (the
    fragments still in flight) they are decoded into n with their power-of-two
    scales. gateup_tail waits for the fragments and runs the group."""
    L = []
    for q, off in enumerate((0, 256, 2048, 2304)):
        L.append("ds_read_b32 %%[w%d], %%[wa]%s" % (q, " offset:%d" % off if off else ""))
    L.append("ds_read_b128 %[f0], %[x]")
    L.append("ds_read_b128 %[f1], %[x] offset:1024")
    L.append("s_waitcnt lgkmcnt(2)")
    for q in range(4):
        L.append("v_cvt_f32_fp8_e32 %%[n%d], %%[s%d]" % (4 * q + 3, q))
        for b in range(4):
            L.append("v_cvt_scalef32_pk_bf16_fp4 %%[n%d], %%[w%d], %%[n%d]%s"
                     % (4 * q + b, q, 4 * q + 3, "" if b == 0 else " op_sel:[%d,%d,0]" % (b & 1, b >> 1)))
    outs = ['[n%d] "=&v"(n[%d][%d])' % (4 * q + b, q, b) for q in range(4) for b in range(4)]
    outs += ['[w%d] "=&v"(w[%d])' % (q, q) for q in range(4)]
    outs += ['[f0] "=&v"(f[0])', '[f1] "=&v"(f[1])']
    ins = ['[x] "v"(x)', '[wa] "v"(wa)'] + ['[s%d] "v"(sb[%d])' % (q, q) for q in range(4)]
    return ("    static __device__ __forceinline__ void gateup_dec(uint32_t x, uint32_t wa, const uint32_t (&sb)[4], "
            "uint32_t (&n)[4][4], u32x4v (&f)[2]) {\n"
            "        uint32_t w[4];\n"
            "        asm volatile(\"%s\"\n            : %s\n            : %s\n            : \"memory\");\n    }\n"
            % ("\\n\\t".join(L), ", ".join(outs), ", ".join(ins)))


def frags() -> str:
    """The first two activation fragment reads of a gate/up group body, left in
    flight for gateup_tail (the path that decodes its weights outside the body)."""
    return ("    static __device__ __forceinline__ void frags(uint32_t x, u32x4v (&f)[2]) {\n"
            "        asm volatile(\"ds_read_b128 %[f0], %[x]\\n\\tds_read_b128 %[f1], %[x] offset:1024\"\n"
            "            : [f0] \"=&v\"(f[0]), [f1] \"=&v\"(f[1])\n            : [x] \"v\"(x)\n"
            "            : \"memory\");\n    }\n")


def gateup_tail(NS: int) -> str:
    """The rest of a gate/up group after gateup_dec: the group body with its
    first two fragments already requested (in f)."""
    P = (NS + 1) // 2
    # two wait states for a VALU write of an accumulator or B register the
    # compiler may place between the two halves
    L = ["s_nop 1", "s_waitcnt lgkmcnt(0)"]

    def rd(buf: int, p: int) -> None:
        for j in range(min(2, NS - 2 * p)):
            off = (2 * p + j) * 1024
            L.append("ds_read_b128 %%[f%d], %%[x]%s" % (2 * buf + j, " offset:%d" % off if off else ""))

    for p in range(P):
        if p + 1 < P:
            rd((p + 1) % 2, p + 1)
        for j in range(min(2, NS - 2 * p)):
            s, f = 2 * p + j, 2 * (p % 2) + j
            for c, m in ((0, 0), (1, 0), (0, 1), (1, 1)):
                L.append("%s %%[c%d_%d_%d], %%[f%d], %%[b%d], %%[c%d_%d_%d]" % (MFMA, s, c, m, f, 2 * m + c, s, c, m))
        if p + 1 < P:
            L.append("s_waitcnt lgkmcnt(0)")
    outs = ['[c%d_%d_%d] "+v"(c[%d][%d][%d])' % (s, cc, m, s, cc, m)
            for s in range(NS) for cc in range(2) for m in range(2)]
    outs += ['[f0] "+v"(f[0])', '[f1] "+v"(f[1])', '[f2] "=&v"(g[0])', '[f3] "=&v"(g[1])']
    ins = ['[b%d] "v"(b[%d])' % (i, i) for i in range(4)] + ['[x] "v"(x)']
    return ("    static __device__ __forceinline__ void gateup_tail(f32x4 (&c)[%d][2][2], const bf16x8 (&b)[4], "
            "u32x4v (&f)[2], uint32_t x) {\n"
            "        u32x4v g[2];\n"
            "        asm volatile(\"%s\"\n            : %s\n            : %s\n            : \"memory\");\n    }\n"
            % (NS, "\\n\\t".join(L), ", ".join(outs), ", ".join(ins)))


def down(NS: int, C: int = 4, dec: bool = False) -> str:
    P = (NS + 1) // 2
    L = []

    def rd(buf: int, p: int) -> None:
        for j in range(min(2, NS - 2 * p)):
            off = (2 * p + j) * 1024
            o = " offset:%d" % off if off else ""
            L.append("ds_read_b128 %%[f%d], %%[hi]%s" % (4 * buf + 2 * j, o))
            L.append("ds_read_b128 %%[f%d], %%[lo]%s" % (4 * buf + 2 * j + 1, o))

    rd(0, 0)
    if dec:
        # the next group's weights, decoded while the first pair's reads are in
        # flight: word q's E4M3 scale byte to fp32 into n[q][3], which then serves
        # as the scale operand of the four converts (the last one overwrites it)
        for q in range(C):
            L.append("v_cvt_f32_fp8_e32 %%[n%d], %%[s%d]" % (4 * q + 3, q))
            for b in range(4):
                L.append("v_cvt_scalef32_pk_bf16_fp4 %%[n%d], %%[w%d], %%[n%d]%s"
                         % (4 * q + b, q, 4 * q + 3, "" if b == 0 else " op_sel:[%d,%d,0]" % (b & 1, b >> 1)))
    L.append("s_waitcnt lgkmcnt(0)")
    for p in range(P):
        if p + 1 < P:
            rd((p + 1) % 2, p + 1)
        base = 4 * (p % 2)
        for half in (0, 1):  # hi products of both slabs, then lo
            for j in range(min(2, NS - 2 * p)):
                s = 2 * p + j
                for c in range(C):
                    L.append("%s %%[c%d_%d], %%[f%d], %%[b%d], %%[c%d_%d]" % (MFMA, s, c, base + 2 * j + half, c, s, c))
        if p + 1 < P:
            L.append("s_waitcnt lgkmcnt(0)")
    outs = ['[c%d_%d] "+v"(c[%d][%d])' % (s, cc, s, cc) for s in range(NS) for cc in range(C)]
    outs += ['[f%d] "=&v"(f[%d])' % (i, i) for i in range(8)]
    ins = ['[b%d] "v"(b[%d])' % (i, i) for i in range(C)] + ['[hi] "v"(hi)', '[lo] "v"(lo)']
    if dec:
        outs += ['[n%d] "=&v"(n[%d][%d])' % (4 * q + b, q, b) for q in range(C) for b in range(4)]
        ins += ['[w%d] "v"(w[%d])' % (q, q) for q in range(C)] + ['[s%d] "v"(sb[%d])' % (q, q) for q in range(C)]
        head = ("    static __device__ __forceinline__ void down_dec(f32x4 (&c)[%d][%d], const bf16x8 (&b)[%d], "
                "uint32_t hi, uint32_t lo, const uint32_t (&w)[%d], const uint32_t (&sb)[%d], uint32_t (&n)[%d][4]) {\n"
                % (NS, C, C, C, C, C))
    else:
        head = ("    static __device__ __forceinline__ void down(f32x4 (&c)[%d][%d], const bf16x8 (&b)[%d], uint32_t hi, "
                "uint32_t lo) {\n" % (NS, C, C))
    return (head + "        u32x4v f[8];\n"
            "        asm volatile(\"%s\"\n            : %s\n            : %s\n            : \"memory\");\n    }\n"
            % ("\\n\\t".join(L), ", ".join(outs), ", ".join(ins)))


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
    out.append("struct PfDec {")
    out.append(gateup_dec())
    out.append(frags())
    out.append("};")
    out.append("")
    for NS in range(1, 11):   # gate/up up to 10 slabs (a block with a short last block merged), down up to 8
        out.append("template <> struct PfGroup<%d> {" % NS)
        out.append(gateup_tail(NS))
        out.append(drain(NS, "[2][2]", ["[%d][%d][%d]" % (s, c, m) for s in range(NS) for c in range(2) for m in range(2)]))
        if NS <= 8:
            out.append(down(NS, dec=True))
            out.append(drain(NS, "[4]", ["[%d][%d]" % (s, c) for s in range(NS) for c in range(4)]))
        out.append("};")
        out.append("")
    out.append("}  // namespace xp")
    sys.stdout.write("\n".join(out) + "\n")


if __name__ == "__main__":
    main()
