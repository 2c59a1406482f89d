// xp_pass_dev.h — device pieces of a decode pass used by the pass kernels
// (xp_rows.hip): weight decode, the eight-leaf tree, the gate/up leaf walks
// and one gate/up work item.
#pragma once

#include "xp_chain_asm.h"
#include "xp_common.h"

namespace xp {

// Two fp4 codes of byte `B` of `v` -> exact fp32 (low nibble first).
template <int B>
__device__ __forceinline__ f32x2 fp4x2(uint32_t v) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, B);
}

__device__ __forceinline__ float e4m3(uint32_t byte) { return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0); }

// One dword of codes (k ascending from the low nibble) -> its eight weights,
// exact fp32. A group is decoded one dword at a time, just before the quarter
// of the chain that uses it, so only eight decoded weights are live at once.
__device__ __forceinline__ void decode8(uint32_t c, float (&w)[8]) {
    f32x2 a;
    a = fp4x2<0>(c); w[0] = a.x; w[1] = a.y;
    a = fp4x2<1>(c); w[2] = a.x; w[3] = a.y;
    a = fp4x2<2>(c); w[4] = a.x; w[5] = a.y;
    a = fp4x2<3>(c); w[6] = a.x; w[7] = a.y;
}

// Leaves l0..l7 at a[0], a[stride], ..., a[7*stride].
__device__ __forceinline__ float tree8(const float* a, int stride) {
    float s01 = a[0] + a[stride];
    float s23 = a[2 * stride] + a[3 * stride];
    float s45 = a[4 * stride] + a[5 * stride];
    float s67 = a[6 * stride] + a[7 * stride];
    float lo = s01 + s23;
    float hi = s45 + s67;
    return lo + hi;
}

typedef const u32x4 __attribute__((address_space(1)))* gcodes_t;
typedef const uint8_t __attribute__((address_space(1)))* gbytes_t;

// Weight codes are read once: non-temporal loads keep them out of the caches' way.
#ifndef XP_NT_CODES
#define XP_NT_CODES 1
#endif
__device__ __forceinline__ u32x4 load_codes(gcodes_t p) {
#if XP_NT_CODES
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}

// Groups kept in flight per wave: deep for small passes, shallower as rows add
// registers (gate/up keeps within 128 VGPRs for 16-wave workgroups; down within
// 128 so that two 8-wave workgroups share a CU).
#ifndef XP_GU_DEPTH_1
#define XP_GU_DEPTH_1 2
#endif
#ifndef XP_DN_DEPTH_1
#define XP_DN_DEPTH_1 2
#endif
#ifndef XP_GU_DEPTH_4
#define XP_GU_DEPTH_4 2  // passes of 3-4 rows (5-8 rows: one group in flight)
#endif
#ifndef XP_DN_DEPTH_4
#define XP_DN_DEPTH_4 2
#endif
template <int P>
struct GuDepth {
    static constexpr int value = P <= 2 ? XP_GU_DEPTH_1 : (P <= 4 ? XP_GU_DEPTH_4 : 1);
};
template <int P>
struct DnDepth {
    static constexpr int value = P == 1 ? XP_DN_DEPTH_1 : (P <= 4 ? XP_DN_DEPTH_4 : 1);
};

// ------------------------------------------------------------------ gate/up

// An E8M0 byte (an OCP MX scale) as fp32: 2^(b - 127), exact; 0 is 2^-127 (a
// subnormal), 0xFF NaN.
__device__ __forceinline__ float e8m0(uint32_t b) {
    if (b == 255u) return __builtin_nanf("");
    return b == 0u ? __uint_as_float(0x00400000u) : __uint_as_float(b << 23);
}

// One leaf of one matrix (gate or up) for one (pass, tile): returns the P leaf
// values of this lane's column. The leaf's groups are g = leaf, leaf+8, ...;
// every leaf walks ceil(G/8) of them, rounded up to whole loop trips of 2*D
// groups, so the loop body has no branches (the ring's wait counts then follow
// it exactly): a group past the end re-reads group G-1 and its product is
// discarded by a select. EXACT = the walks end on the last group (G a
// multiple of 8 whose leaves' group counts are multiples of 2*D), so no group
// is past the end and the select is left out.
// Activations: bf16 rows (xr[r] = the row's 16-bit pairs), or, when CODED,
// E4M3FN codes (xr[r] = the row's code bytes, read as pairs) with one E8M0
// scale per group (sr[r] = the row's scale bytes); a coded value enters the
// chain as e4m3(code) * 2^(scale - 127), computed exactly in fp32, so the chain
// is the bf16 path's on those values.
// True when every leaf's walk (ceil(G/8) groups rounded up to trips of 2*D)
// ends exactly on its last group.
template <int P>
__device__ __forceinline__ bool exact_walk(int G) {
    constexpr int D = GuDepth<P>::value;
    return (G & 7) == 0 && ((G >> 3) % (2 * D)) == 0;
}

template <int P, bool CODED, bool EXACT>
__device__ __forceinline__ void gu_leaf(gcodes_t cc, gbytes_t ss, const uint32_t* const (&xr)[P],
                                        const uint8_t* const (&sr)[P], int leaf, int G, int lane, float (&acc)[P]) {
    constexpr int D = GuDepth<P>::value;
    const int xl = lane & 15;
    const int ng = (G + 7) >> 3;
#pragma unroll
    for (int r = 0; r < P; ++r) acc[r] = 0.0f;
    // Two register sets of D groups (see gu_leaf2).
    u32x4 bc[2][D];
    uint32_t bs[2][D];
    uint32_t bx[2][D][P];
    uint32_t bsx[2][D][P];
    auto load = [&](int set, int s, int i) {
        const int g = min(leaf + 8 * i, G - 1);
        bc[set][s] = load_codes(cc + (size_t)g * kTile);
        bs[set][s] = ss[(size_t)g * kTile];
#pragma unroll
        for (int r = 0; r < P; ++r) {
            if constexpr (CODED) {
                bx[set][s][r] = ((const uint16_t*)xr[r])[16 * g + xl];
                bsx[set][s][r] = sr[r][g];
            } else {
                bx[set][s][r] = xr[r][16 * g + xl];
            }
        }
    };
    auto half = [&](int set, int i0) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
            const int i = i0 + s;
            const float sc = e4m3(bs[set][s]);
            float p[P], xa[P], xb[P];
            const u32x4 cw = bc[set][s];
            if constexpr (CODED) {
#pragma unroll
                for (int r = 0; r < P; ++r) {
                    const f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8((int)bx[set][s][r], false);
                    const float sx = e8m0(bsx[set][s][r]);
                    xa[r] = v.x * sx;
                    xb[r] = v.y * sx;
                }
                load(set ^ 1, s, i + D);
                { float w[8]; decode8(cw[0], w); Chain<P>::head_f32(w, xa, xb, p); }
            } else {
                uint32_t xc[P];
#pragma unroll
                for (int r = 0; r < P; ++r) xc[r] = bx[set][s][r];
                load(set ^ 1, s, i + D);
                { float w[8]; decode8(cw[0], w); Chain<P>::head_bf16(w, xc, xa, xb, p); }
            }
            { float w[8]; decode8(cw[1], w); Chain<P>::tail1(w, xa, xb, p); }
            { float w[8]; decode8(cw[2], w); Chain<P>::tail2(w, xa, xb, p); }
            { float w[8]; decode8(cw[3], w); Chain<P>::tail3(w, xa, xb, p); }
            const bool valid = EXACT || leaf + 8 * i < G;
#pragma unroll
            for (int r = 0; r < P; ++r) {
                const float v = __builtin_fmaf(p[r], sc, acc[r]);
                acc[r] = valid ? v : acc[r];
            }
        }
    };
#pragma unroll
    for (int s = 0; s < D; ++s) load(0, s, s);
    for (int i0 = 0; i0 < ng; i0 += 2 * D) {
        half(0, i0);
        half(1, i0 + D);
    }
}

// Both matrices of one leaf for one (pass, tile), in one wave: for each of the
// leaf's groups the gate and up codes and scales are loaded together, the rows'
// activations once, and the gate chain then the up chain run over the same
// converted activations. Per matrix and row this is gu_leaf's arithmetic
// exactly (the same chain, scaled fma and leaf), so the bits are gu_leaf's.
template <int P, bool CODED, bool EXACT>
__device__ __forceinline__ void gu_leaf2(gcodes_t cg, gbytes_t sg, gcodes_t cu, gbytes_t su,
                                         const uint32_t* const (&xr)[P], const uint8_t* const (&sr)[P], int leaf,
                                         int G, int lane, float (&accg)[P], float (&accu)[P]) {
    constexpr int D = GuDepth<P>::value;
    const int xl = lane & 15;
    const int ng = (G + 7) >> 3;
#pragma unroll
    for (int r = 0; r < P; ++r) accg[r] = accu[r] = 0.0f;
    // Two register sets of D groups: while the groups of one set are consumed,
    // the loads of the next D groups fill the other, so a load never targets a
    // register still in use and nothing is copied (or waited for) at the loop's
    // back edge; D groups stay in flight throughout.
    u32x4 bg[2][D], bu[2][D];
    uint32_t bsg[2][D], bsu[2][D];
    uint32_t bx[2][D][P];
    uint32_t bsx[2][D][P];
    auto load = [&](int set, int s, int i) {
        const int g = min(leaf + 8 * i, G - 1);
        bg[set][s] = load_codes(cg + (size_t)g * kTile);
        bu[set][s] = load_codes(cu + (size_t)g * kTile);
        bsg[set][s] = sg[(size_t)g * kTile];
        bsu[set][s] = su[(size_t)g * kTile];
#pragma unroll
        for (int r = 0; r < P; ++r) {
            if constexpr (CODED) {
                bx[set][s][r] = ((const uint16_t*)xr[r])[16 * g + xl];
                bsx[set][s][r] = sr[r][g];
            } else {
                bx[set][s][r] = xr[r][16 * g + xl];
            }
        }
    };
    // Consume set `set` (groups i0 .. i0+D-1), loading groups i0+D .. into the other.
    auto half = [&](int set, int i0) {
#pragma unroll
        for (int s = 0; s < D; ++s) {
            const int i = i0 + s;
            const float scg = e4m3(bsg[set][s]), scu = e4m3(bsu[set][s]);
            const u32x4 cwg = bg[set][s], cwu = bu[set][s];
            float p[P], xa[P], xb[P];
            if constexpr (CODED) {
#pragma unroll
                for (int r = 0; r < P; ++r) {
                    const f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8((int)bx[set][s][r], false);
                    const float sx = e8m0(bsx[set][s][r]);
                    xa[r] = v.x * sx;
                    xb[r] = v.y * sx;
                }
                load(set ^ 1, s, i + D);
                { float w[8]; decode8(cwg[0], w); Chain<P>::head_f32(w, xa, xb, p); }
            } else {
                uint32_t xc[P];
#pragma unroll
                for (int r = 0; r < P; ++r) xc[r] = bx[set][s][r];
                load(set ^ 1, s, i + D);
                { float w[8]; decode8(cwg[0], w); Chain<P>::head_bf16(w, xc, xa, xb, p); }
            }
            { float w[8]; decode8(cwg[1], w); Chain<P>::tail1(w, xa, xb, p); }
            { float w[8]; decode8(cwg[2], w); Chain<P>::tail2(w, xa, xb, p); }
            { float w[8]; decode8(cwg[3], w); Chain<P>::tail3(w, xa, xb, p); }
            const bool valid = EXACT || leaf + 8 * i < G;
#pragma unroll
            for (int r = 0; r < P; ++r) {
                const float v = __builtin_fmaf(p[r], scg, accg[r]);
                accg[r] = valid ? v : accg[r];
            }
            { float w[8]; decode8(cwu[0], w); Chain<P>::head_f32(w, xa, xb, p); }
            { float w[8]; decode8(cwu[1], w); Chain<P>::tail1(w, xa, xb, p); }
            { float w[8]; decode8(cwu[2], w); Chain<P>::tail2(w, xa, xb, p); }
            { float w[8]; decode8(cwu[3], w); Chain<P>::tail3(w, xa, xb, p); }
#pragma unroll
            for (int r = 0; r < P; ++r) {
                const float v = __builtin_fmaf(p[r], scu, accu[r]);
                accu[r] = valid ? v : accu[r];
            }
        }
    };
#pragma unroll
    for (int s = 0; s < D; ++s) load(0, s, s);
    for (int i0 = 0; i0 < ng; i0 += 2 * D) {
        half(0, i0);
        half(1, i0 + D);
    }
}

// Gate/up outputs: act in fp32, g and u in fp32 (split), or act stored as bf16.
enum GuOut { kActF32 = 0, kSplit = 1, kActBf16 = 2 };

// x: bf16 rows [R][H], or, when CODED, E4M3FN code rows [R][H] with E8M0 scales xs [R][H/32].
// WAVES = 16: waves 0-7 walk the gate leaves, 8-15 the up leaves (gu_leaf);
// WAVES = 8: wave j walks leaf j of both matrices (gu_leaf2). The leaves land in
// the same LDS slots either way, so the tree and epilogue are shared.
template <int P, int OUT, bool CODED = false, int WAVES = 16>
__device__ __forceinline__ void gu_item(const xp_expert* __restrict__ experts, const void* __restrict__ x,
                        const uint8_t* __restrict__ xs, const int32_t* __restrict__ entry, int4 ps, int tile,
                        int H, int I, int k, float* __restrict__ out0, float* __restrict__ out1, float* red) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int leaf = wave & 7, up = wave >> 3;
    const int e = ps.x, first = ps.y, real = ps.z;
    const int G = H >> 5;

    const xp_expert ex = experts[e];
    const size_t tile_chunks = (size_t)tile * G * kTile;

    const uint32_t* xr[P];
    const uint8_t* sr[P];
#pragma unroll
    for (int r = 0; r < P; ++r) {
        const size_t row = (size_t)(entry[first + (r < real ? r : real - 1)] / k);
        if constexpr (CODED) {
            xr[r] = (const uint32_t*)((const uint8_t*)x + row * H);
            sr[r] = xs + row * (H >> 5);
        } else {
            xr[r] = (const uint32_t*)((const uint16_t*)x + row * H);
            sr[r] = nullptr;
        }
    }
    // leaves -> LDS: red[slot][row][lane], gate leaves in slots 0-7, up in 8-15
    if constexpr (WAVES == 16) {
        const gcodes_t cc = (gcodes_t)(up ? ex.up_codes : ex.gate_codes) + tile_chunks + lane;
        const gbytes_t ss = (gbytes_t)(up ? ex.up_scales : ex.gate_scales) + tile_chunks + lane;
        float acc[P];
        if (exact_walk<P>(G))
            gu_leaf<P, CODED, true>(cc, ss, xr, sr, leaf, G, lane, acc);
        else
            gu_leaf<P, CODED, false>(cc, ss, xr, sr, leaf, G, lane, acc);
#pragma unroll
        for (int r = 0; r < P; ++r) red[(wave * P + r) * kTile + lane] = acc[r];
    } else {
        float accg[P], accu[P];
        const gcodes_t cg = (gcodes_t)ex.gate_codes + tile_chunks + lane, cu = (gcodes_t)ex.up_codes + tile_chunks + lane;
        const gbytes_t sg = (gbytes_t)ex.gate_scales + tile_chunks + lane, su = (gbytes_t)ex.up_scales + tile_chunks + lane;
        if (exact_walk<P>(G))
            gu_leaf2<P, CODED, true>(cg, sg, cu, su, xr, sr, leaf, G, lane, accg, accu);
        else
            gu_leaf2<P, CODED, false>(cg, sg, cu, su, xr, sr, leaf, G, lane, accg, accu);
#pragma unroll
        for (int r = 0; r < P; ++r) {
            red[(leaf * P + r) * kTile + lane] = accg[r];
            red[((8 + leaf) * P + r) * kTile + lane] = accu[r];
        }
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < P * kTile) {
        const int r = t >> 6, c = t & 63;
        if (r < real) {
            const int stride = P * kTile;
            const float g = tree8(red + r * kTile + c, stride);
            const float u = tree8(red + 8 * stride + r * kTile + c, stride);
            const size_t o = (size_t)entry[first + r] * I + (size_t)tile * kTile + c;
            if (OUT == kSplit) {
                out0[o] = g;
                out1[o] = u;
            } else {
                const float a = (g / (1.0f + expf(-g))) * u;
                if (OUT == kActBf16)
                    ((uint16_t*)out0)[o] = bf16_rne(a);
                else
                    out0[o] = a;
            }
        }
    }
    __syncthreads();
}

// Narrow slices: 16 output columns (a quarter of a tile) per workgroup.
constexpr int kNarrow = 16;

// Column slice of workgroup b: the four 16-column slices of a 64-column tile
// go to workgroups on one XCD (workgroup b runs on XCD b mod 8), so the tile's
// lines are fetched into that XCD's L2 once; n_slices = hidden / 16.
__device__ __forceinline__ int narrow_col0(int b, int n_slices) {
    const int n_tiles = n_slices >> 2;
    const int tile = (n_tiles & 7) == 0 ? (b >> 5) * 8 + (b & 7) : b >> 2;
    return tile * kTile + ((n_tiles & 7) == 0 ? (b >> 3) & 3 : b & 3) * kNarrow;
}

}  // namespace xp
